// Mixed attention O = Attn([T_t, T'_{t+1}], C' U C_kappa): split-K online
// softmax over the low-bit positions (those in kappa masked out), the 16-bit
// rows fetched for kappa, and an optional 16-bit tail; then a merge of the
// per-split partials.
//
// SpeCache summary, quick read (third mechanism) and §3 "decoding": the
// 16-bit pairs C_kappa replace their low-bit counterparts; §7 Algorithm 3:
// K = [K' U K_kappa, K_t], A = MaskedSoftmax(Q_t K^T), O = A V.  The split-K /
// online-softmax organisation is the IO-aware exact-attention idea the SemKV
// page cites in §2.4; the result is exact softmax attention up to float32
// accumulation and the float16 rounding of the probabilities fed to the
// matrix cores.
//
// Work decomposition: one workgroup (4 waves) per (split of L positions, KV
// head); each wave owns every 4th 32-position block of the split and all the
// G*T query rows of the KV head, so every low-bit byte is read once.  Per
// block a wave issues, on the matrix cores:
//   scores  S[token][row] = sum_c Khat[token][c] q[row][c]: the key codes
//           expanded to +-s (mfma_frag.h) against the float16 queries; the
//           per-block constant sum_c q_c (z_c + h s_c) comes from a small
//           MFMA prepass over 16 blocks at a time.  With at most 8 rows, the
//           two 16-token tiles of a block share one accumulator: tile 0's
//           rows sit in columns 0-7 and tile 1's in columns 8-15.
//   values  O[row][c] += P[row][token] * Vhat[token][c]: the value codes
//           expanded the same way against the float16 probabilities, plus one
//           MFMA whose columns are the per-token zero-points and scales.
// Softmax maxima are kept per accumulator row and only rescaled when a new
// logit exceeds the running maximum by more than 2^8 (probabilities up to 256
// stay exact enough in float16 and cannot overflow).
#include "mfma_frag.h"

namespace specache {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kEmpty = -1.0e30f;   // running max of a row that has seen nothing
constexpr float kRescale = 8.0f;     // lazy-rescale threshold (log2 units)
constexpr int kMaxBlocksPerSplit = 128;

template <int D, int PACK>
struct AttnSmem {
  static constexpr int W = D / 32;
  static constexpr int RS = 36;  // row stride (halves, a multiple of 4 for 8-byte reads) of the transposed tile
  uint32_t kmask[kMaxBlocksPerSplit];
  float cst[4][16][16];          // per wave: [block of the 16-block group][row]
  int sel_range[2];
  union {
    _Float16 vt[4][D][RS];       // per wave: 16-bit value rows, transposed
    struct {
      float o[4][16][D];
      float zs[4][16][2 * W];
      float m[4][16];
      float l[4][16];
    } comb;
  } u;
};

__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int D, int BITS, int PACK>
__global__ __launch_bounds__(256, 2) void attn_split_kernel(AttnArgs a, int Hkv, int G, int64_t N, int64_t L,
                                                            int S) {
  constexpr int W = D / 32;
  constexpr int CPL = D / 16;       // channels per lane in the value product (= channel tiles)
  constexpr float hK = BITS == 1 ? 0.5f : 1.5f;
  constexpr float hV = BITS == 1 ? 0.5f : 1.5f;
  __shared__ AttnSmem<D, PACK> sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n16 = lane & 15, g = lane >> 4;
  const int split = blockIdx.x;
  const int64_t slice = blockIdx.y;
  const int64_t b = slice / Hkv, h = slice % Hkv;
  const int T = a.T;
  const int R = G * T;
  const int Hq = Hkv * G;
  const int64_t nblk = N / 32;
  const int64_t row0 = b * Hq * T + h * G * T;
  const float qscale = a.sm_scale * kLog2e;
  const int64_t p0 = (int64_t)split * L;
  const int64_t p1 = p0 + L < N ? p0 + L : N;
  const int nb = (int)((p1 - p0) / 32);
  const int64_t blk0 = p0 / 32;

  // ---- kappa positions of this split: a bitmask over its blocks and the range [i0, i1) of
  // fetched rows whose positions fall in it (idx is ascending), found by one parallel pass.
  for (int i = tid; i < kMaxBlocksPerSplit; i += 256) sm.kmask[i] = 0u;
  if (tid < 2) sm.sel_range[tid] = 0;
  __syncthreads();
  {
    const int32_t* ix = a.idx + slice * a.k;
    int below0 = 0, below1 = 0;
    for (int i = tid; i < a.k; i += 256) {
      const int64_t p = ix[i];
      below0 += p < p0 ? 1 : 0;
      below1 += p < p1 ? 1 : 0;
      if (p >= p0 && p < p1) atomicOr(&sm.kmask[(p - p0) >> 5], 1u << ((p - p0) & 31));
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      below0 += __shfl_xor(below0, off);
      below1 += __shfl_xor(below1, off);
    }
    if (lane == 0 && (below0 | below1)) {
      atomicAdd(&sm.sel_range[0], below0);
      atomicAdd(&sm.sel_range[1], below1);
    }
  }
  __syncthreads();
  const int i0 = sm.sel_range[0], i1 = sm.sel_range[1];

  // ---- query fragments: B[k-slot (g, j)][column] = q[row][32w + 8g + j]
  Frag B0[W], B1[W];
  {
    const int r0 = PACK == 2 ? (n16 < 8 ? n16 : -1) : n16;
    const int r1 = PACK == 2 ? (n16 >= 8 ? n16 - 8 : -1) : -1;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      B0[w].v = (r0 >= 0 && r0 < R) ? load_u4(a.q16 + (row0 + r0) * D + 32 * w + 8 * g) : make_uint4(0, 0, 0, 0);
      B1[w].v = (r1 >= 0 && r1 < R) ? load_u4(a.q16 + (row0 + r1) * D + 32 * w + 8 * g) : make_uint4(0, 0, 0, 0);
    }
  }

  float m_used = kEmpty;   // running max (log2 units) of accumulator row n16
  float l_part = 0.0f;     // this lane's share of that row's sum of exponentials
  f32x4 Oacc[CPL];
#pragma unroll
  for (int ct = 0; ct < CPL; ++ct) Oacc[ct] = zero4();
  f32x4 Ozs = zero4();

  const int wv_grp = (CPL * n16) / 32;  // value group of this lane's channels
  // token (within a block) of A/B k-slot j for k-group g: j < 4 -> 4g + j, else 16 + 4g + j - 4
  // bit position of an even token t inside a value word: t / 2
  const int shv[4] = {15 - 2 * g, 14 - 2 * g, 7 - 2 * g, 6 - 2 * g};

  auto online_update = [&](float (&x)[PACK == 2 ? 4 : 8]) {
    constexpr int NX = PACK == 2 ? 4 : 8;
    float bm = x[0];
#pragma unroll
    for (int i = 1; i < NX; ++i) bm = fmaxf(bm, x[i]);
    bm = max_over_groups(bm);
    if (__any(bm > m_used + kRescale)) {
      const float mn = fmaxf(m_used, bm);
      const float alpha = __builtin_amdgcn_exp2f(m_used - mn);
      m_used = mn;
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * g + i);
#pragma unroll
        for (int ct = 0; ct < CPL; ++ct) Oacc[ct][i] *= ai;
        Ozs[i] *= ai;
      }
    }
  };

  // P (float32) -> float16 A fragment; slots j < 4 hold tile-0 tokens, j >= 4 tile-1 tokens.
  auto make_p = [&](const float (&p)[PACK == 2 ? 4 : 8], float mul) {
    Frag A;
    if constexpr (PACK == 2) {
      const uint32_t lo = pack_half2(p[0] * mul, p[1] * mul), hi = pack_half2(p[2] * mul, p[3] * mul);
      const bool t1 = n16 >= 8;
      A.u[0] = t1 ? 0u : lo;
      A.u[1] = t1 ? 0u : hi;
      A.u[2] = t1 ? lo : 0u;
      A.u[3] = t1 ? hi : 0u;
    } else {
#pragma unroll
      for (int d = 0; d < 4; ++d) A.u[d] = pack_half2(p[2 * d] * mul, p[2 * d + 1] * mul);
    }
    return A;
  };

  // ================= low-bit blocks =================
  struct BlockData {
    Words<W> kw[2][BITS];
    uint4 ks[W];
    Words<CPL> vw[BITS];
    uint2 vs_lo, vs_hi, zs_lo, zs_hi;
  };
  // All loads are unconditional (clamped to valid addresses) so that they issue back to back.
  auto load_block = [&](int jj) {
    BlockData bd;
    const int64_t blk = blk0 + jj;
    const uint32_t* kc = a.k_codes + (slice * N + blk * 32) * BITS * W;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int pl = 0; pl < BITS; ++pl) bd.kw[tau][pl] = load_words<W>(kc + ((16 * tau + n16) * BITS + pl) * W);
    const _Float16* kms = a.k_meta + ((slice * nblk + blk) * 2 + 1) * D;
#pragma unroll
    for (int w = 0; w < W; ++w) bd.ks[w] = load_u4(kms + 32 * w + 8 * g);
    const uint32_t* vc = a.v_codes + (slice * nblk + blk) * BITS * D;
#pragma unroll
    for (int pl = 0; pl < BITS; ++pl) bd.vw[pl] = load_words<CPL>(vc + pl * D + CPL * n16);
    const _Float16* vm = a.v_meta + (slice * nblk + blk) * 2 * W * 32;
    bd.vs_lo = load_u2(vm + W * 32 + wv_grp * 32 + 4 * g);
    bd.vs_hi = load_u2(vm + W * 32 + wv_grp * 32 + 16 + 4 * g);
    // rows 0..W-1 of the value metadata are the zero-points of groups 0..W-1, rows W..2W-1 the scales
    const _Float16* zr = vm + (n16 < 2 * W ? n16 : 0) * 32;
    bd.zs_lo = load_u2(zr + 4 * g);
    bd.zs_hi = load_u2(zr + 16 + 4 * g);
    return bd;
  };
  const bool zs_lane = n16 < 2 * W;

  BlockData cur;
  if (wave < nb) cur = load_block(wave);
  for (int jj = wave; jj < nb; jj += 4) {
    const int step = (jj - wave) >> 2;  // index among this wave's blocks
    const bool prepass = (step & 15) == 0;
    Frag az[W], as[W];
    if (prepass) {
      // constant term of the next 16 blocks of this wave (rows x blocks, via MFMA below)
      const int bi = jj + 4 * n16;
      const _Float16* km = a.k_meta + (slice * nblk + blk0 + (bi < nb ? bi : jj)) * 2 * D;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        az[w].v = load_u4(km + 32 * w + 8 * g);
        as[w].v = load_u4(km + D + 32 * w + 8 * g);
      }
    }
    const BlockData nxt = load_block(jj + 4 < nb ? jj + 4 : jj);
    if (prepass) {
      f32x4 accZ = zero4(), accS = zero4();
#pragma unroll
      for (int w = 0; w < W; ++w) {
        accZ = mma(az[w], B0[w], accZ);
        accS = mma(as[w], B0[w], accS);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sm.cst[wave][4 * g + i][n16] = (accZ[i] + hK * accS[i]) * qscale;
      lds_fence();
    }
    const Words<W>(&kw)[2][BITS] = cur.kw;
    const uint4* ks = cur.ks;
    const Words<CPL>* vw = cur.vw;
    const uint2 vs_lo = cur.vs_lo, vs_hi = cur.vs_hi;
    const uint2 zs_lo = zs_lane ? cur.zs_lo : make_uint2(0, 0);
    const uint2 zs_hi = zs_lane ? cur.zs_hi : make_uint2(0, 0);

    // scores
    f32x4 acc[2][BITS];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int pl = 0; pl < BITS; ++pl) acc[tau][pl] = zero4();
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const uint32_t* mag = reinterpret_cast<const uint32_t*>(&ks[w]);
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
        for (int pl = 0; pl < BITS; ++pl) {
          Frag A;
#pragma unroll
          for (int d = 0; d < 4; ++d) A.u[d] = signed_pair(kw[tau][pl].w[w], 15 - 4 * g - d, mag[d]);
          if constexpr (PACK == 2)
            acc[0][pl] = mma(A, tau == 0 ? B0[w] : B1[w], acc[0][pl]);
          else
            acc[tau][pl] = mma(A, B0[w], acc[tau][pl]);
        }
      }
    }
    constexpr int NX = PACK == 2 ? 4 : 8;
    float x[NX];
    const float c0 = sm.cst[wave][step & 15][PACK == 2 ? (n16 & 7) : n16];
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int tau = PACK == 2 ? 0 : i / 4;
      // the expanded operand is -(2b - 1) s: a set bit becomes a negative sign
      const float s = BITS == 1 ? -0.5f * acc[tau][0][i & 3] : -0.5f * acc[tau][0][i & 3] - acc[tau][BITS - 1][i & 3];
      x[i] = fmaf(s, qscale, c0);
    }
    const uint32_t kmw = sm.kmask[jj];
    if (kmw) {
#pragma unroll
      for (int i = 0; i < NX; ++i) {
        const int tok = PACK == 2 ? (16 * (n16 >> 3) + 4 * g + i) : (16 * (i >> 2) + 4 * g + (i & 3));
        if ((kmw >> tok) & 1u) x[i] = -INFINITY;
      }
    }
    online_update(x);
    float p[NX];
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      p[i] = __builtin_amdgcn_exp2f(x[i] - m_used);
      l_part += p[i];
    }
    const Frag Ap = make_p(p, 1.0f);
    Frag Ap2;
    if constexpr (BITS == 2) Ap2 = make_p(p, 2.0f);

    // values
    const uint32_t vmag[4] = {vs_lo.x, vs_lo.y, vs_hi.x, vs_hi.y};
#pragma unroll
    for (int ct = 0; ct < CPL; ++ct) {
#pragma unroll
      for (int pl = 0; pl < BITS; ++pl) {
        Frag Bv;
#pragma unroll
        for (int d = 0; d < 4; ++d) Bv.u[d] = signed_pair(vw[pl].w[ct], shv[d], vmag[d]);
        Oacc[ct] = mma(pl == 0 ? Ap : Ap2, Bv, Oacc[ct]);
      }
    }
    Frag Bzs;
    Bzs.u[0] = zs_lo.x;
    Bzs.u[1] = zs_lo.y;
    Bzs.u[2] = zs_hi.x;
    Bzs.u[3] = zs_hi.y;
    Ozs = mma(Ap, Bzs, Ozs);
    cur = nxt;
  }

  // ================= 16-bit rows: fetched kappa rows of this split, then the tail =================
  const int n_sel = i1 - i0;
  const bool has_tail = (split == S - 1) && a.tail > 0;
  const int n_sel_blk = (n_sel + 31) / 32;
  const int n_tail_blk = has_tail ? (a.tail + 31) / 32 : 0;
  for (int q = wave; q < n_sel_blk + n_tail_blk; q += 4) {
    const bool tail = q >= n_sel_blk;
    const int base = tail ? 32 * (q - n_sel_blk) : i0 + 32 * q;
    const int lim = tail ? a.tail : i1;
    const _Float16* ksrc = tail ? a.k_tail + slice * a.tail * D : a.k_sel + slice * a.k * D;
    const _Float16* vsrc = tail ? a.v_tail + slice * a.tail * D : a.v_sel + slice * a.k * D;
    // transpose the 32 value rows into this wave's LDS tile
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int tok = 16 * tau + n16;
      const bool ok = base + tok < lim;
      const int64_t src_row = ok ? base + tok : lim - 1;
      Frag vv[W];
#pragma unroll
      for (int w = 0; w < W; ++w) vv[w].v = load_u4(vsrc + src_row * D + 32 * w + 8 * g);
#pragma unroll
      for (int w = 0; w < W; ++w) {
        Frag v;
        v.v = ok ? vv[w].v : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 8; ++j) sm.u.vt[wave][32 * w + 8 * g + j][tok] = v.h[j];
      }
    }
    f32x4 acc[2];
    acc[0] = zero4();
    acc[1] = zero4();
    Frag kk[2][W];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int tok = 16 * tau + n16;
      const int64_t src_row = base + tok < lim ? base + tok : lim - 1;
#pragma unroll
      for (int w = 0; w < W; ++w) kk[tau][w].v = load_u4(ksrc + src_row * D + 32 * w + 8 * g);
    }
#pragma unroll
    for (int w = 0; w < W; ++w) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const int tok = 16 * tau + n16;
        Frag A;
        A.v = (base + tok < lim) ? kk[tau][w].v : make_uint4(0, 0, 0, 0);
        if constexpr (PACK == 2)
          acc[0] = mma(A, tau == 0 ? B0[w] : B1[w], acc[0]);
        else
          acc[tau] = mma(A, B0[w], acc[tau]);
      }
    }
    constexpr int NX = PACK == 2 ? 4 : 8;
    float x[NX];
    const int row = PACK == 2 ? (n16 & 7) : n16;
    const int tq = row % T;
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int tok = PACK == 2 ? (16 * (n16 >> 3) + 4 * g + i) : (16 * (i >> 2) + 4 * g + (i & 3));
      const int tau = PACK == 2 ? 0 : i >> 2;
      float v = acc[tau][i & 3] * qscale;
      bool ok = base + tok < lim;
      if (tail) ok = ok && (base + tok <= a.tail - T + tq);
      x[i] = ok ? v : -INFINITY;
    }
    online_update(x);
    float p[NX];
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      p[i] = __builtin_amdgcn_exp2f(x[i] - m_used);
      l_part += p[i];
    }
    const Frag Ap2 = make_p(p, -2.0f);  // the value accumulator is scaled by -1/2 at the end
    lds_fence();
#pragma unroll
    for (int ct = 0; ct < CPL; ++ct) {
      const int c = CPL * n16 + ct;
      const uint2 lo = load_u2(&sm.u.vt[wave][c][4 * g]);
      const uint2 hi = load_u2(&sm.u.vt[wave][c][16 + 4 * g]);
      Frag Bv;
      Bv.u[0] = lo.x;
      Bv.u[1] = lo.y;
      Bv.u[2] = hi.x;
      Bv.u[3] = hi.y;
      Oacc[ct] = mma(Ap2, Bv, Oacc[ct]);
    }
    lds_fence();
  }

  // ================= wave epilogue =================
  const float l_row = sum_over_groups(l_part);  // row n16
  float fin_m = m_used, fin_l = l_row;          // final (m, l) of row (n16 & 7) or n16
  float f_self = 1.0f, f_other = 0.0f;          // weights of rows n16 and n16 ^ 8
  if constexpr (PACK == 2) {
    const float m2 = __shfl_xor(m_used, 8);
    const float l2 = __shfl_xor(l_row, 8);
    const float mm = fmaxf(m_used, m2);
    f_self = __builtin_amdgcn_exp2f(m_used - mm);
    f_other = __builtin_amdgcn_exp2f(m2 - mm);
    fin_m = mm;
    fin_l = f_self * l_row + f_other * l2;
  }
  __syncthreads();  // all waves are done with their value tiles; the LDS union becomes the combine buffer
  if (g == 0 && n16 < (PACK == 2 ? 8 : 16)) {
    sm.u.comb.m[wave][n16] = fin_m;
    sm.u.comb.l[wave][n16] = fin_l;
  }
  // accumulator rows 4g' + i; with PACK == 2 rows r and r + 8 fold into r (lanes g' < 2)
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * g + i;
    float ws = 1.0f, wo = 0.0f;
    if constexpr (PACK == 2) {
      ws = __shfl(f_self, r & 7);
      wo = __shfl(f_other, r & 7);
    }
    float zsv = Ozs[i];
    if constexpr (PACK == 2) zsv = ws * zsv + wo * __shfl_xor(Ozs[i], 32);
    float ov[CPL];
#pragma unroll
    for (int ct = 0; ct < CPL; ++ct) {
      ov[ct] = Oacc[ct][i];
      if constexpr (PACK == 2) ov[ct] = ws * ov[ct] + wo * __shfl_xor(Oacc[ct][i], 32);
    }
    const bool keep = PACK == 2 ? (g < 2) : true;
    if (keep) {
      if (n16 < 2 * W) sm.u.comb.zs[wave][r][n16] = zsv;
#pragma unroll
      for (int ct = 0; ct < CPL; ++ct) sm.u.comb.o[wave][r][CPL * n16 + ct] = ov[ct];
    }
  }
  __syncthreads();

  // ================= combine the four waves and write this split's partials =================
  for (int e = tid; e < R * D; e += 256) {
    const int r = e / D, c = e % D;
    float M = kEmpty;
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) M = fmaxf(M, sm.u.comb.m[w4][r]);
    float lsum = 0.0f, o = 0.0f;
    const int gv = c / 32;
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
      const float e4 = __builtin_amdgcn_exp2f(sm.u.comb.m[w4][r] - M);
      lsum += e4 * sm.u.comb.l[w4][r];
      o += e4 * (-0.5f * sm.u.comb.o[w4][r][c] + sm.u.comb.zs[w4][r][gv] + hV * sm.u.comb.zs[w4][r][W + gv]);
    }
    const int64_t row = row0 + r;
    a.part_acc[(row * S + split) * D + c] = o;
    if (c == 0) {
      a.part_ml[(row * S + split) * 2] = M;
      a.part_ml[(row * S + split) * 2 + 1] = lsum;
    }
  }
}

// One workgroup per query row: weights 2^(m_s - M) of the S split partials in
// LDS, then each thread sums its channel over the splits with all loads in flight.
template <int D>
__global__ __launch_bounds__(D) void attn_merge_kernel(const float* __restrict__ part_ml,
                                                       const float* __restrict__ part_acc, int S,
                                                       _Float16* __restrict__ out) {
  constexpr int kMaxS = 1024;
  __shared__ float wts[kMaxS];
  __shared__ float red[D / 64];
  __shared__ float Mrow, Lrow;
  const int64_t row = blockIdx.x;
  const int c = threadIdx.x;
  const float* ml = part_ml + row * S * 2;
  float M = kEmpty;
  for (int s = c; s < S; s += D) M = fmaxf(M, ml[2 * s]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if ((c & 63) == 0) red[c >> 6] = M;
  __syncthreads();
  if (c == 0) {
    float m = red[0];
#pragma unroll
    for (int i = 1; i < D / 64; ++i) m = fmaxf(m, red[i]);
    Mrow = m;
  }
  __syncthreads();
  M = Mrow;
  float l = 0.0f;
  for (int s = c; s < S; s += D) {
    const float w = __builtin_amdgcn_exp2f(ml[2 * s] - M);
    wts[s] = w;
    l = fmaf(ml[2 * s + 1], w, l);
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
  __syncthreads();
  if ((c & 63) == 0) red[c >> 6] = l;
  __syncthreads();
  if (c == 0) {
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) t += red[i];
    Lrow = t;
  }
  __syncthreads();
  const float* acc = part_acc + row * S * D + c;
  float o = 0.0f;
  int s = 0;
  for (; s + 8 <= S; s += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = acc[(int64_t)(s + u) * D];
#pragma unroll
    for (int u = 0; u < 8; ++u) o = fmaf(v[u], wts[s + u], o);
  }
  for (; s < S; ++s) o = fmaf(acc[(int64_t)s * D], wts[s], o);
  out[row * D + c] = (_Float16)(o / Lrow);
}

template <int D, int BITS>
void launch_split(const Dims& d, const AttnPlan& plan, const AttnArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)plan.S, (unsigned)d.slices());
  if (d.G * a.T <= 8)
    attn_split_kernel<D, BITS, 2><<<grid, 256, 0, s>>>(a, d.Hkv, d.G, d.N, plan.L, plan.S);
  else
    attn_split_kernel<D, BITS, 1><<<grid, 256, 0, s>>>(a, d.Hkv, d.G, d.N, plan.L, plan.S);
}

}  // namespace

hipError_t launch_decode_attn(const Dims& d, const AttnPlan& plan, const AttnArgs& a, hipStream_t s) {
  const unsigned rows = (unsigned)((int64_t)d.B * d.Hq * a.T);
  if (d.D == 128) {
    if (d.bits == 1) launch_split<128, 1>(d, plan, a, s); else launch_split<128, 2>(d, plan, a, s);
    attn_merge_kernel<128><<<rows, 128, 0, s>>>(a.part_ml, a.part_acc, plan.S, a.out16);
  } else {
    if (d.bits == 1) launch_split<64, 1>(d, plan, a, s); else launch_split<64, 2>(d, plan, a, s);
    attn_merge_kernel<64><<<rows, 64, 0, s>>>(a.part_ml, a.part_acc, plan.S, a.out16);
  }
  return hipGetLastError();
}

}  // namespace specache
