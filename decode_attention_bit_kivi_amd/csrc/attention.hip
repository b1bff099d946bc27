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
#include "merge.h"
#include "mfma_frag.h"

namespace specache {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kEmpty = kMergeEmpty;  // running max of a row that has seen nothing
constexpr float kRescale = 8.0f;     // lazy-rescale threshold (log2 units)
constexpr int kMaxBlocksPerSplit = kAttnMaxBlocks;

template <int D, int PACK>
struct AttnSmem {
  static constexpr int W = D / 32;
  static constexpr int RS = 36;  // row stride (halves, a multiple of 4 for 8-byte reads) of the transposed tile
  uint32_t kmask[kMaxBlocksPerSplit];
  float rank_m[4][16], rank_l[4][16];  // per wave: ranking statistics of each query row
  float cst[4][16][16];          // per wave: [block of the 16-block group][row]
  uint4 kscale[4][16][4][W];     // per wave: key scales [block of the group][k-group][chunk]
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

// F16: the 16-bit comparator -- no low-bit cache; every position of the split is a 16-bit row
// of a.k_sel / a.v_sel (the whole 16-bit cache, a.k = its positions per slice).
template <int D, int KB, int VB, int PACK, bool RANK, bool F16 = false>
__global__ __launch_bounds__(256, 2) void attn_split_kernel(AttnArgs a, int Hkv, int G, int64_t N, int64_t L,
                                                            int S) {
  constexpr int W = D / 32;
  constexpr int CPL = D / 16;       // channels per lane in the value product (= channel tiles)
  constexpr float hK = KB == 1 ? 0.5f : 1.5f;  // KB, VB: bits of the key and value codes
  constexpr float hV = VB == 1 ? 0.5f : 1.5f;
  __shared__ AttnSmem<D, PACK> sm;

  const int tid = threadIdx.x;
  // the wave index as a wave-uniform (scalar) value: block indices and the address arithmetic
  // derived from it then run on the scalar unit, beside the VALU
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g = lane >> 4;
  const int split = blockIdx.x;
  const int64_t slice = blockIdx.y;
  const int64_t b = slice / Hkv, h = slice % Hkv;
  const int T = a.T;
  const int R = G * T;
  const int Hq = Hkv * G;
  const int64_t row0 = b * Hq * T + h * G * T;
  const float qscale = a.sm_scale * kLog2e;
  const int64_t p0 = (int64_t)split * L;
  const int64_t p1 = p0 + L < N ? p0 + L : N;
  const int nb = (int)((p1 - p0) / 32);
  const int64_t blk0 = p0 / 32;

  if (RANK && split == 0)  // the rank kernels accumulate a per-slice histogram here
    for (int i = tid; i < 2048; i += 256) a.rank_hist[slice * 2048 + i] = 0u;

  // ---- kappa positions of this split: a bitmask over its blocks and the range [i0, i1) of
  // fetched rows whose positions fall in it (idx is ascending), found by one parallel pass.
  int i0 = (int)p0, i1 = (int)p1;
  if constexpr (!F16) {
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
  i0 = sm.sel_range[0];
  i1 = sm.sel_range[1];
  }

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
  float l_part = 0.0f;     // this lane's share of that row's sum of exponentials (low-bit positions)
  float l16 = 0.0f;        // the same over the 16-bit rows (fetched and tail), kept apart for the ranking
  // ranking: the C' terms of kappa positions (masked out of the attention), kept relative to
  // their own running max m_corr (per lane) so that the attention's arithmetic is untouched
  float m_corr = kEmpty, l_corr = 0.0f;
  f32x4 Oacc[CPL];
#pragma unroll
  for (int ct = 0; ct < CPL; ++ct) Oacc[ct] = zero4();
  f32x4 Ozs = zero4();

  const int gshift = a.group == 64 ? 1 : 0;  // groups of 64 (keys: tokens, values: channels)
  const int Wg = W >> gshift;                 // value groups per token
  const int wv_grp = (CPL * n16) >> (5 + gshift);  // value group of this lane's channels
  const int arow = PACK == 2 ? (n16 & 7) : n16;  // query row of this lane's logits
  const bool rank_lane = RANK && arow < R && (arow % T) == a.rank_row;
  // token (within a block) of A/B k-slot j for k-group g: j < 4 -> 4g + j, else 16 + 4g + j - 4
  // bit position of an even token t inside a value word: t / 2
  const int shv[4] = {15 - 2 * g, 14 - 2 * g, 7 - 2 * g, 6 - 2 * g};

  constexpr int NX = PACK == 2 ? 4 : 8;
  const float k1 = -0.5f * qscale;  // the expanded key operand is -(2b - 1) s

  // Rescale the accumulators of this lane's rows when a block raises a row maximum by more
  // than 2^kRescale.  xr holds logits relative to the current maximum; on a rescale they are
  // recomputed from the absolute values xa.
  auto online_update = [&](float (&xr)[NX], const float (&xa)[NX]) {
    // the wave-wide vote needs no per-row maximum: some row's maximum exceeds the threshold
    // exactly when some lane's does
    float bm = xr[0];
#pragma unroll
    for (int i = 1; i < NX; ++i) bm = fmaxf(bm, xr[i]);
    if (__any(bm > kRescale)) {
      float ba = xa[0];
#pragma unroll
      for (int i = 1; i < NX; ++i) ba = fmaxf(ba, xa[i]);
      ba = max_over_groups(ba);
      const float mn = fmaxf(m_used, ba);
      const float alpha = __builtin_amdgcn_exp2f(m_used - mn);
      m_used = mn;
      l_part *= alpha;
      l16 *= alpha;
#pragma unroll
      for (int i = 0; i < NX; ++i) xr[i] = xa[i] - mn;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ai = __shfl(alpha, 4 * g + i);
#pragma unroll
        for (int ct = 0; ct < CPL; ++ct) Oacc[ct][i] *= ai;
        Ozs[i] *= ai;
      }
    }
  };

  // round to nearest even (one v_cvt_pk_f16_f32): the sums l_part / l16 hold the unrounded p, so
  // the rounding of the value product's operand must not lean one way
  auto pack2 = [](float a, float b) { return pack_half2(a, b); };
  // P (float32) -> float16 A fragment; slots j < 4 hold tile-0 tokens, j >= 4 tile-1 tokens.
  auto make_p = [&](const float (&p)[NX], float mul) {
    Frag A;
    if constexpr (PACK == 2) {
      const uint32_t lo = pack2(p[0] * mul, p[1] * mul), hi = pack2(p[2] * mul, p[3] * mul);
      const bool t1 = n16 >= 8;
      A.u[0] = t1 ? 0u : lo;
      A.u[1] = t1 ? 0u : hi;
      A.u[2] = t1 ? lo : 0u;
      A.u[3] = t1 ? hi : 0u;
    } else {
#pragma unroll
      for (int d = 0; d < 4; ++d) A.u[d] = pack2(p[2 * d] * mul, p[2 * d + 1] * mul);
    }
    return A;
  };

  // ================= low-bit blocks =================
  // A block's key codes and value data load on separate schedules (each one block ahead of its use).
  struct KData {
    Words<W> kw[2][KB];
  };
  struct VData {
    Words<CPL> vw[VB];
    uint2 vs_lo, vs_hi, zs_lo, zs_hi;
  };
  const int64_t Ns = a.seq_stride, nblk_s = a.seq_stride / 32;  // the cache's layout stride
  const uint32_t* kc_slice = a.k_codes + slice * Ns * KB * W;
  const uint32_t* vc_slice = a.v_codes + slice * nblk_s * VB * D;
  const _Float16* vm_slice = a.v_meta + slice * nblk_s * 2 * Wg * 32;
  const _Float16* km_slice = a.k_meta + slice * (nblk_s >> gshift) * 2 * D;
  const int zrow = n16 < 2 * Wg ? n16 : 0;  // value-metadata row of the zero-point / scale column
  // All loads are unconditional (clamped to valid blocks) so that they issue back to back.
  // the rank row's logits of this slice ([G][N] floats): lane offset of the lane's head row
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const __amdgpu_buffer_rsrc_t rl_buf =
      make_rsrc(RANK && a.rank_logits ? static_cast<const void*>(a.rank_logits + slice * G * N)
                                      : static_cast<const void*>(a.q16),
                RANK && a.rank_logits ? (uint32_t)(G * N * 4) : 0u);
  const uint32_t rl_lane = (uint32_t)((arow / T) * N * 4);
  // A block's base addresses are wave-uniform (scalar); each lane adds a loop-invariant unsigned
  // 32-bit offset.  The codes are read through raw buffers over the slice (scalar block offset,
  // per-lane offset), the value metadata through the scalar base of the block.
  const __amdgpu_buffer_rsrc_t kc_buf = make_rsrc(kc_slice, (uint32_t)(Ns * KB * W * 4));
  const __amdgpu_buffer_rsrc_t vc_buf = make_rsrc(vc_slice, (uint32_t)(nblk_s * VB * D * 4));
  const uint32_t off_k = (uint32_t)(n16 * KB * W * 4), off_v = (uint32_t)(CPL * n16 * 4);
  const uint32_t off_vs = (uint32_t)(Wg * 32 + wv_grp * 32 + 4 * g), off_zs = (uint32_t)(zrow * 32 + 4 * g);
  auto load_k = [&](int jj) {
    KData kd;
    const int64_t blk = blk0 + jj;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int pl = 0; pl < KB; ++pl)
        kd.kw[tau][pl] = buffer_words<W>(kc_buf, off_k + (uint32_t)((16 * tau * KB + pl) * W * 4),
                                         (uint32_t)(blk * 32 * KB * W * 4));
    return kd;
  };
  auto load_v = [&](int jj) {
    VData bd;
    const int64_t blk = blk0 + jj;
#pragma unroll
    for (int pl = 0; pl < VB; ++pl)
      bd.vw[pl] = buffer_words<CPL>(vc_buf, off_v + (uint32_t)(pl * D * 4), (uint32_t)(blk * VB * D * 4));
    const _Float16* vm = vm_slice + blk * 2 * Wg * 32;
    bd.vs_lo = load_u2(vm + off_vs);
    bd.vs_hi = load_u2(vm + 16 + off_vs);
    // rows 0..W-1 of the value metadata are the zero-points of groups 0..W-1, rows W..2W-1 the scales
    bd.zs_lo = load_u2(vm + off_zs);
    bd.zs_hi = load_u2(vm + 16 + off_zs);
    return bd;
  };
  // Prepass over the wave's next 16 blocks: zero-points and scales of the keys against the
  // queries give the per-block constant; the scales also go to LDS for the expansion.
  Frag pz[W], ps[W];
  auto prepass_load = [&](int jj) {
    const int bi = jj + 4 * n16;
    const _Float16* km = km_slice + ((blk0 + (bi < nb ? bi : jj)) >> gshift) * 2 * D;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      pz[w].v = load_u4(km + 32 * w + 8 * g);
      ps[w].v = load_u4(km + D + 32 * w + 8 * g);
    }
  };
  auto prepass_finish = [&]() {
    f32x4 accZ = zero4(), accS = zero4();
#pragma unroll
    for (int w = 0; w < W; ++w) {
      accZ = mma(pz[w], B0[w], accZ);
      accS = mma(ps[w], B0[w], accS);
      sm.kscale[wave][n16][g][w] = ps[w].v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) sm.cst[wave][4 * g + i][n16] = (accZ[i] + hK * accS[i]) * qscale;
    lds_fence();
  };

  // scores of a block: the key codes expanded against the queries on the matrix cores
  auto score_block = [&](const KData& kd, int step, f32x4 (&acc)[2][KB]) {
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int pl = 0; pl < KB; ++pl) acc[tau][pl] = zero4();
    // chunks w and w + 1 expand together (one 64-bit shift per pair of words); the products
    // accumulate in the order w, tau as for one chunk at a time
#pragma unroll
    for (int w = 0; w < W; w += 2) {
      const uint4 ka = sm.kscale[wave][step & 15][g][w], kb = sm.kscale[wave][step & 15][g][w + 1];
      const uint32_t ma[4] = {ka.x, ka.y, ka.z, ka.w}, mb[4] = {kb.x, kb.y, kb.z, kb.w};
#pragma unroll
      for (int pl = 0; pl < KB; ++pl) {
        Frag A0[2], A1[2];  // [tau]: chunk w, chunk w + 1
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
          for (int d = 0; d < 4; ++d)
            signed_pairs2(kd.kw[tau][pl].w[w], kd.kw[tau][pl].w[w + 1], 15 - 4 * g - d, ma[d], mb[d], A0[tau].u[d],
                          A1[tau].u[d]);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int tau = 0; tau < 2; ++tau) {
            const Frag& A = h2 == 0 ? A0[tau] : A1[tau];
            if constexpr (PACK == 2)
              acc[0][pl] = mma(A, tau == 0 ? B0[w + h2] : B1[w + h2], acc[0][pl]);
            else
              acc[tau][pl] = mma(A, B0[w + h2], acc[tau][pl]);
          }
      }
    }
  };
  auto block_const = [&](int step) { return sm.cst[wave][step & 15][PACK == 2 ? (n16 & 7) : n16]; };
  // the rest of a block: logits, softmax, ranking outputs, values.  c0: the block's constant.
  auto finish_block = [&](const VData& bd, const f32x4 (&acc)[2][KB], float c0, int jj) {
    const float c0m = c0 - m_used;
    float xr[NX], xa[NX];
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int tau = PACK == 2 ? 0 : i / 4;
      const float sacc = KB == 1 ? acc[tau][0][i & 3] : acc[tau][0][i & 3] + 2.0f * acc[tau][KB - 1][i & 3];
      xr[i] = fmaf(sacc, k1, c0m);
      xa[i] = fmaf(sacc, k1, c0);
    }
    const uint32_t kmw = sm.kmask[jj];
    if constexpr (RANK) {
      // the rank row's logits against C' (before any kappa masking), log2 units; when ranking
      // by the mixed cache the kappa positions are written by the 16-bit pass instead
      if (rank_lane && a.rank_mixed && kmw) {
        float* dst = a.rank_logits + (slice * G + arow / T) * N + (blk0 + jj) * 32;
#pragma unroll
        for (int i = 0; i < NX; ++i) {
          const int tok = PACK == 2 ? (16 * (n16 >> 3) + 4 * g + i) : (16 * (i >> 2) + 4 * g + (i & 3));
          if (!((kmw >> tok) & 1u)) dst[tok] = xa[i];
        }
      } else if (rank_lane) {
        // through the raw buffer over the slice's logits: the block offset is scalar (read from
        // the first lane, so that the compiler keeps it in a scalar register)
        const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)((blk0 + jj) * 32 * 4));
        typedef float f4_t __attribute__((ext_vector_type(4)));
        if constexpr (PACK == 2) {
          const f4_t v = {xa[0], xa[1], xa[2], xa[3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rl_buf,
                                                 (int)(rl_lane + 4 * (16 * (n16 >> 3) + 4 * g)), (int)soff, 0);
        } else {
          const f4_t v0 = {xa[0], xa[1], xa[2], xa[3]};
          const f4_t v1 = {xa[4], xa[5], xa[6], xa[7]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v0), rl_buf, (int)(rl_lane + 16 * g),
                                                 (int)soff, 0);
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v1), rl_buf,
                                                 (int)(rl_lane + 4 * (16 + 4 * g)), (int)soff, 0);
        }
      }
    }
    if constexpr (RANK && PACK == 2) {
      // the bound of each 8-position group for the pruned selection: this lane's four logits
      // are tokens 4g .. 4g + 3 of tile n16 >> 3 for row arow, lanes g and g ^ 1 of n16 a group
      if (a.rank_gmax) {
        const float gm = max_over_group_pairs(fmaxf(fmaxf(xa[0], xa[1]), fmaxf(xa[2], xa[3])));
        if (rank_lane && (g & 1) == 0)
          a.rank_gmax[(slice * G + arow / T) * (N / kBoundGroup) + (blk0 + jj) * 4 + 2 * (n16 >> 3) + (g >> 1)] = gm;
      }
    }
    float xc[NX];  // C' logits of masked positions, for the ranking statistics
    if (kmw) {
#pragma unroll
      for (int i = 0; i < NX; ++i) {
        const int tok = PACK == 2 ? (16 * (n16 >> 3) + 4 * g + i) : (16 * (i >> 2) + 4 * g + (i & 3));
        xc[i] = -INFINITY;
        if ((kmw >> tok) & 1u) {
          xc[i] = xa[i];
          xr[i] = -INFINITY;
          xa[i] = -INFINITY;
        }
      }
    }
    online_update(xr, xa);
    float p[NX];
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      p[i] = __builtin_amdgcn_exp2f(xr[i]);
      l_part += p[i];
    }
    if constexpr (RANK) {
      if (kmw) {
        float cm = xc[0];
#pragma unroll
        for (int i = 1; i < NX; ++i) cm = fmaxf(cm, xc[i]);
        const float mn = fmaxf(m_corr, cm);
        l_corr *= __builtin_amdgcn_exp2f(m_corr - mn);
        m_corr = mn;
#pragma unroll
        for (int i = 0; i < NX; ++i) l_corr += __builtin_amdgcn_exp2f(xc[i] - mn);
      }
    }
    const Frag Ap = make_p(p, 1.0f);
    Frag Ap2;
    if constexpr (VB == 2) Ap2 = make_p(p, 2.0f);

    // values
    const uint32_t vmag[4] = {bd.vs_lo.x, bd.vs_lo.y, bd.vs_hi.x, bd.vs_hi.y};
#pragma unroll
    for (int ct = 0; ct < CPL; ct += 2) {
#pragma unroll
      for (int pl = 0; pl < VB; ++pl) {
        Frag Bv0, Bv1;  // channel tiles ct and ct + 1, one 64-bit shift per pair of words
#pragma unroll
        for (int d = 0; d < 4; ++d)
          signed_pairs2(bd.vw[pl].w[ct], bd.vw[pl].w[ct + 1], shv[d], vmag[d], vmag[d], Bv0.u[d], Bv1.u[d]);
        Oacc[ct] = mma(pl == 0 ? Ap : Ap2, Bv0, Oacc[ct]);
        Oacc[ct + 1] = mma(pl == 0 ? Ap : Ap2, Bv1, Oacc[ct + 1]);
      }
    }
    // columns n16 >= 2 Wg carry another row's (finite) metadata: their outputs are never read
    Frag Bzs;
    Bzs.u[0] = bd.zs_lo.x;
    Bzs.u[1] = bd.zs_lo.y;
    Bzs.u[2] = bd.zs_hi.x;
    Bzs.u[3] = bd.zs_hi.y;
    Ozs = mma(Ap, Bzs, Ozs);
  };

  // ================= 16-bit rows: the fetched kappa rows of this split, then the tail =================
  // Block q of a wave's share (q = wave, wave + 4, ...): the fetched rows' blocks run before the
  // low-bit blocks, so that their loads and transposes overlap the other waves' low-bit work (the
  // wave then has more low-bit blocks left than the others and takes the issue priority until it
  // has caught up); the tail's blocks run after them.  Their exponentials go to l16, so the
  // low-bit sums l_part stay the ranking statistics over C'.
  const int n_sel = i1 - i0;
  const bool has_tail = (split == S - 1) && a.tail > 0;
  const int n_sel_blk = (n_sel + 31) / 32;
  const int n_tail_blk = has_tail ? (a.tail + 31) / 32 : 0;
  const int first_tail_q = n_sel_blk + ((wave - n_sel_blk) % 4 + 4) % 4;  // first q >= n_sel_blk of this wave
  auto f16_block = [&](int q) {
    const bool tail = q >= n_sel_blk;
    const int base = tail ? 32 * (q - n_sel_blk) : i0 + 32 * q;
    const int lim = tail ? a.tail : i1;
    const _Float16* ksrc = tail ? a.k_tail + slice * a.tail * D : a.k_sel + slice * a.k * D;
    const _Float16* vsrc = tail ? a.v_tail + slice * a.tail * D : a.v_sel + slice * a.k * D;
    // all 32 value and key rows in flight together, then the values transposed into this
    // wave's LDS tile
    Frag vv[2][W], kk[2][W];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int tok = 16 * tau + n16;
      const int64_t src_row = base + tok < lim ? base + tok : lim - 1;
#pragma unroll
      for (int w = 0; w < W; ++w) vv[tau][w].v = load_u4(vsrc + src_row * D + 32 * w + 8 * g);
#pragma unroll
      for (int w = 0; w < W; ++w) kk[tau][w].v = load_u4(ksrc + src_row * D + 32 * w + 8 * g);
    }
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int tok = 16 * tau + n16;
      const bool ok = base + tok < lim;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        Frag v;
        v.v = ok ? vv[tau][w].v : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int j = 0; j < 8; ++j) sm.u.vt[wave][32 * w + 8 * g + j][tok] = v.h[j];
      }
    }
    f32x4 acc[2];
    acc[0] = zero4();
    acc[1] = zero4();
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
    float xr[NX], xa[NX];
    const int row = PACK == 2 ? (n16 & 7) : n16;
    const int tq = row % T;
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int tok = PACK == 2 ? (16 * (n16 >> 3) + 4 * g + i) : (16 * (i >> 2) + 4 * g + (i & 3));
      const int tau = PACK == 2 ? 0 : i >> 2;
      const float v = acc[tau][i & 3] * qscale;
      bool ok = base + tok < lim;
      if constexpr (RANK) {
        // ranking by the mixed cache: a fetched row's logit replaces its low-bit one
        if (a.rank_mixed && rank_lane && !tail && ok) {
          const int64_t pos = a.idx[slice * a.k + base + tok];
          a.rank_logits[(slice * G + arow / T) * N + pos] = v;
        }
      }
      if (tail) ok = ok && (base + tok <= a.tail - T + tq);
      xa[i] = ok ? v : -INFINITY;
      xr[i] = xa[i] - m_used;
    }
    online_update(xr, xa);
    float p[NX];
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      p[i] = __builtin_amdgcn_exp2f(xr[i]);
      l16 += p[i];
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
  };
  __builtin_amdgcn_s_setprio(3);  // a chain of latencies: issue it ahead of the other waves' loops
  for (int q = wave; q < n_sel_blk; q += 4) f16_block(q);

  // Software pipeline over this wave's blocks (jj = vw + 4 i, i = 0 .. nw - 1): iteration i
  // issues block i + 1's score MFMAs before finishing block i (softmax, values), so the matrix
  // cores work on one block while the VALU finishes the other; key codes load two blocks ahead,
  // value data one.  A block's constant is read right after the prepass that covers it (the next
  // prepass rewrites the LDS slots).
  if constexpr (!F16) {
    // low-bit blocks jj = vw + 4 i: the waves that took one 16-bit block more than the others
    // take the last places of the rotation, which get one low-bit block fewer when the split's
    // block count is not a multiple of 4
    const int vw = (wave - n_sel_blk) & 3;
    const int nw = vw < nb ? (nb - vw + 3) / 4 : 0;
    auto blk = [&](int i) { return vw + 4 * (i < nw ? i : nw - 1); };  // clamped to the last block
    if (nw > 0) {
      KData k0 = load_k(blk(0)), k1 = load_k(blk(1));
      VData v0 = load_v(blk(0)), v1;
      f32x4 acc0[2][KB], acc1[2][KB];
      prepass_load(blk(0));
      prepass_finish();
      score_block(k0, 0, acc0);
      float c0_0 = block_const(0), c0_1 = 0.0f;
      // Issue priority by the blocks this wave has left: two workgroups share each compute
      // unit, and the SIMD arbiter otherwise favours the older one, which then finishes long
      // before the younger and leaves one wave per SIMD for the rest.  A wave that has got
      // ahead drops below the waves behind it, so the waves of a SIMD finish together.
      const int pr1 = nw / 16 + 1, pr2 = nw / 6 + 1, pr3 = nw / 3 + 1;
      for (int i = 0; i < nw; i += 2) {
        const int rem = nw - i;
        if (rem > pr3) __builtin_amdgcn_s_setprio(3);
        else if (rem > pr2) __builtin_amdgcn_s_setprio(2);
        else if (rem > pr1) __builtin_amdgcn_s_setprio(1);
        else __builtin_amdgcn_s_setprio(0);
        k0 = load_k(blk(i + 2));
        v1 = load_v(blk(i + 1));
        if (i + 1 < nw) {
          if (((i + 1) & 15) == 0) {
            prepass_load(blk(i + 1));
            prepass_finish();
          }
          score_block(k1, i + 1, acc1);
          c0_1 = block_const(i + 1);
        }
        finish_block(v0, acc0, c0_0, blk(i));
        if (i + 1 >= nw) break;
        k1 = load_k(blk(i + 3));
        v0 = load_v(blk(i + 2));
        if (i + 2 < nw) {
          if (((i + 2) & 15) == 0) {
            prepass_load(blk(i + 2));
            prepass_finish();
          }
          score_block(k0, i + 2, acc0);
          c0_0 = block_const(i + 2);
        }
        finish_block(v1, acc1, c0_1, blk(i + 1));
      }
    }
  }

  __builtin_amdgcn_s_setprio(3);  // the rest of the workgroup is a chain of latencies: let it through

  // ranking statistics over C' = the low-bit positions processed so far, kappa positions included
  float rank_m_lane = m_used, rank_l_lane = l_part;
  if constexpr (RANK) {
    rank_m_lane = max_over_groups(fmaxf(m_used, m_corr));  // the same for the four lanes of a row
    rank_l_lane = l_part * __builtin_amdgcn_exp2f(m_used - rank_m_lane) +
                  l_corr * __builtin_amdgcn_exp2f(m_corr - rank_m_lane);
  }

  // ================= 16-bit rows of the tail (the fetched rows went first) =================
  for (int q = first_tail_q; q < n_sel_blk + n_tail_blk; q += 4) f16_block(q);

  // ================= wave epilogue =================
  const float l_row = sum_over_groups(l_part + l16);  // row n16
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
  if constexpr (RANK) {
    // per query row: sum over the k-groups (same max), then (PACK == 2) fold the two tiles' rows
    float rl = sum_over_groups(rank_l_lane), rm = rank_m_lane;
    if constexpr (PACK == 2) {
      const float m2 = __shfl_xor(rm, 8), l2 = __shfl_xor(rl, 8);
      const float mm = fmaxf(rm, m2);
      rl = rl * __builtin_amdgcn_exp2f(rm - mm) + l2 * __builtin_amdgcn_exp2f(m2 - mm);
      rm = mm;
    }
    if (g == 0 && n16 < 16) {
      sm.rank_m[wave][n16] = rm;
      sm.rank_l[wave][n16] = rl;
    }
  }
  __syncthreads();  // all waves are done with their value tiles; the LDS union becomes the combine buffer
  if constexpr (RANK) {
    // one thread per head: combine the four waves and write this split's statistics over C'
    if (!a.rank_mixed && tid < G) {
      const int r = tid * T + a.rank_row;
      float M = kEmpty;
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) M = fmaxf(M, sm.rank_m[w4][r]);
      float Ls = 0.0f;
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) Ls += sm.rank_l[w4][r] * __builtin_amdgcn_exp2f(sm.rank_m[w4][r] - M);
      a.rank_m[(slice * G + tid) * S + split] = M;
      a.rank_l[(slice * G + tid) * S + split] = Ls;
    }
  }
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
      if (n16 < 2 * Wg) sm.u.comb.zs[wave][r][n16] = zsv;
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
    const int gv = c >> (5 + gshift);
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
      const float e4 = __builtin_amdgcn_exp2f(sm.u.comb.m[w4][r] - M);
      lsum += e4 * sm.u.comb.l[w4][r];
      o += e4 * (-0.5f * sm.u.comb.o[w4][r][c] + sm.u.comb.zs[w4][r][gv] + hV * sm.u.comb.zs[w4][r][Wg + gv]);
    }
    const int64_t row = row0 + r;
    a.part_acc[(row * S + split) * D + c] = o;
    if (c == 0) {
      a.part_ml[(row * S + split) * 2] = M;
      a.part_ml[(row * S + split) * 2 + 1] = lsum;
      if constexpr (RANK) {
        // ranking by the mixed cache: the rank row's own softmax statistics of this split
        if (a.rank_mixed && r % T == a.rank_row) {
          a.rank_m[(slice * G + r / T) * S + split] = M;
          a.rank_l[(slice * G + r / T) * S + split] = lsum;
        }
      }
    }
  }
}

// Four query rows per workgroup, one wave each.
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(const float* __restrict__ part_ml,
                                                         const float* __restrict__ part_acc, int S, int64_t rows,
                                                         _Float16* __restrict__ out) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row < rows) merge_row_wave<D>(part_ml, part_acc, S, out, row);
}

template <int D, int KB, int VB, bool RANK>
void launch_split(const Dims& d, const AttnPlan& plan, const AttnArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)plan.S, (unsigned)d.slices());
  if (d.G * a.T <= 8)
    attn_split_kernel<D, KB, VB, 2, RANK><<<grid, 256, 0, s>>>(a, d.Hkv, d.G, d.N, plan.L, plan.S);
  else
    attn_split_kernel<D, KB, VB, 1, RANK><<<grid, 256, 0, s>>>(a, d.Hkv, d.G, d.N, plan.L, plan.S);
}

template <int D, bool RANK>
void launch_split_d(const Dims& d, const AttnPlan& plan, const AttnArgs& a, hipStream_t s) {
  if (d.bits == 1) {
    if (d.vbits == 1) launch_split<D, 1, 1, RANK>(d, plan, a, s); else launch_split<D, 1, 2, RANK>(d, plan, a, s);
  } else {
    if (d.vbits == 1) launch_split<D, 2, 1, RANK>(d, plan, a, s); else launch_split<D, 2, 2, RANK>(d, plan, a, s);
  }
}

template <bool RANK>
void launch_split_r(const Dims& d, const AttnPlan& plan, const AttnArgs& a, hipStream_t s) {
  if (d.D == 128) launch_split_d<128, RANK>(d, plan, a, s); else launch_split_d<64, RANK>(d, plan, a, s);
}

}  // namespace

hipError_t launch_attn_split(const Dims& d, const AttnPlan& plan, const AttnArgs& a, hipStream_t s) {
  if (attn_stream_serves(d, a)) return launch_attn_stream(d, plan, a, s);
  if (a.rank_logits) launch_split_r<true>(d, plan, a, s); else launch_split_r<false>(d, plan, a, s);
  return hipGetLastError();
}

hipError_t launch_attn16_split(const Dims& d, const AttnPlan& plan, const AttnArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)plan.S, (unsigned)d.slices());
  const bool pack2 = d.G * a.T <= 8;
  if (d.D == 128) {
    if (pack2) attn_split_kernel<128, 1, 1, 2, false, true><<<grid, 256, 0, s>>>(a, d.Hkv, d.G, d.N, plan.L, plan.S);
    else attn_split_kernel<128, 1, 1, 1, false, true><<<grid, 256, 0, s>>>(a, d.Hkv, d.G, d.N, plan.L, plan.S);
  } else {
    if (pack2) attn_split_kernel<64, 1, 1, 2, false, true><<<grid, 256, 0, s>>>(a, d.Hkv, d.G, d.N, plan.L, plan.S);
    else attn_split_kernel<64, 1, 1, 1, false, true><<<grid, 256, 0, s>>>(a, d.Hkv, d.G, d.N, plan.L, plan.S);
  }
  return hipGetLastError();
}

hipError_t launch_attn_merge(const Dims& d, const AttnPlan& plan, const AttnArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)d.B * d.Hq * a.T;
  const unsigned blocks = (unsigned)ceil_div(rows, 4);
  if (d.D == 128)
    attn_merge_kernel<128><<<blocks, 256, 0, s>>>(a.part_ml, a.part_acc, plan.S, rows, a.out16);
  else
    attn_merge_kernel<64><<<blocks, 256, 0, s>>>(a.part_ml, a.part_acc, plan.S, rows, a.out16);
  return hipGetLastError();
}

}  // namespace specache
