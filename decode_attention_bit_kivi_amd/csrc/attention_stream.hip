// Split kernel of the mixed attention for its common decode shape -- head_dim 128, 1-bit key and
// value codes, at most 8 query rows per KV head (G * T <= 8) -- with the low-bit cache streamed
// through LDS.
//
// It computes what attn_split_kernel (attention.hip) computes for this shape, with the same
// operands and the same order of products (SpeCache summary, quick read (third mechanism) and
// §3 "decoding": the 16-bit pairs C_kappa replace their low-bit counterparts; §7 Algorithm 3:
// K = [K' U K_kappa, K_t], A = MaskedSoftmax(Q_t K^T), O = A V), and the same work decomposition:
// one workgroup of four waves per (split, KV head), wave w taking the split's 32-position blocks
// w, w + 4, ...; its outputs are the split partials and, in the RANK form, the rank row's logits
// and statistics (over C', or those of the attention itself when ranking by the mixed cache) and
// the maxima of every 8 positions.  One difference in the softmax: the running maximum of a row here also
// covers the low-bit logits of the kappa positions, whose exponentials, dropped from the
// attention, are the kappa terms of the ranking statistics over C' (attn_split_kernel keeps
// those terms apart, with a maximum of their own).  The results agree to rounding; both forms of
// this kernel (with and without the ranking outputs) compute the same attention bit for bit.
//
// What differs is how a block's bytes reach the matrix-core operands.  The operand layout holds
// each code word and value-metadata entry in 4 lanes and each key scale in 16, so loading it
// directly keeps 4 to 16 register bytes per byte in flight, and the bytes a wave can have in
// flight bound the bandwidth (Little's law at HBM latency).  Here each lane loads 8 bytes of each
// of a block's four arrays (key codes, key zero-points and scales, value codes, value metadata:
// 2 KB, every byte once) kStreamAhead blocks before the block's turn; when the turn comes the
// wave writes them to an LDS slot of its own and reads its operands back from there (LDS
// accesses of one wave complete in order, so no barrier is involved).  A block's constant
// sum_c q_c (z_c + h s_c) comes from four MFMAs on the staged zero-points and scales, so there is
// no separate pass over the key metadata that would wait for its loads.
//
// The kernel is held to 168 registers so that three workgroups share a compute unit (three waves
// per SIMD): the VALU work of expanding the codes, not the bytes, bounds a wave, and a third wave
// keeps the SIMD issuing while the other two wait on LDS and the matrix cores.  Each wave then
// streams two blocks ahead.
#include "merge.h"
#include "mfma_frag.h"

#include <type_traits>

namespace specache {

namespace {

constexpr int kStD = 128;
constexpr int kStW = kStD / 32;    // 32-channel chunks
constexpr int kStCPL = kStD / 16;  // value channel tiles (channels per lane)
constexpr int kStRS = 36;          // row stride (halves) of the transposed 16-bit value tile
constexpr int kStreamAhead = 2;    // blocks whose bytes each wave has in flight (three waves per SIMD)
// A staged block in LDS: key codes (512 bytes), key zero-points then scales (256 bytes each, 16
// bytes apart), value codes (16 bytes after every 64 channels' words), value metadata (64-byte rows,
// 8 bytes apart).  The gaps put the addresses that one operand read sends to the same bank row on
// different banks: rows 0 and 1 mod 4 of the constant's operand (zero-points, scales), lanes n16 and
// n16 + 8 of the value codes, the 8 rows of zero-points and scales of the value metadata.
constexpr int kStKC = 0, kStKM = 512, kStKS = kStKM + 272, kStVC = kStKM + 528, kStVM = kStVC + 528;
constexpr int kStSlot = kStVM + 8 * 72;  // 2144 bytes, a multiple of 16
static_assert(kStSlot % 16 == 0 && kStKS % 16 == 0 && kStVC % 16 == 0 && kStVM % 8 == 0, "LDS read alignment");
constexpr float kStLog2e = 1.4426950408889634f;
constexpr float kStRescale = 8.0f;  // lazy-rescale threshold (log2 units)
constexpr uint32_t kStDropped = 0x80000000u;  // a buffer offset past every buffer here: the store is dropped

struct StreamSmem {
  uint32_t kmask[kAttnMaxBlocks];
  float rank_m[4][16], rank_l[4][16];  // per wave: ranking statistics of each query row
  int sel_range[2];
  uint4 bq[kStW][64];  // the query fragments (identical in every wave), lane l's at [w][l]
  // 16-byte aligned: the operands are read back with 16-byte LDS reads
  union alignas(16) {
    union {  // per wave: the 16-bit value tile, or (during the low-bit blocks) two staged blocks
      _Float16 vt[kStD][kStRS];
      unsigned char stage[2][kStSlot];
    } w[4];
    struct {
      float o[4][8][kStD];  // per wave: final-form output rows (16-byte aligned for float4 access)
      float m[4][8];
      float l[4][8];
    } comb;
  } u;
};

// Ranking by the mixed cache with at most kStashFloats fetched-row logits per slice (rows x G):
// the fetched rows' 16-bit logits wait in LDS until the low-bit loop has stored every position's
// logit, then overwrite those of their positions.
constexpr int kStashFloats = 2048;
struct StreamSmemStash : StreamSmem {
  float kst[kStashFloats];  // [fetched row of the split][head]
};

__device__ __forceinline__ void st_lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int R>
using IC = std::integral_constant<int, R>;

// MODE 0: attention only; 1: with the rank row's logits, bounds and statistics against C';
// 2: with the ranking by the mixed-cache attention row; 3: the same with the fetched rows' logits
// held in LDS until the end (the loop then stores like form 1); 4: the rank row's logits and
// statistics against C' alone (score_topk: no values, no fetched rows, no tail, no output).
template <int MODE>
__global__ __launch_bounds__(256, 3) void attn_stream_kernel(AttnArgs a, int Hkv, int G, int64_t N, int64_t L, int S) {
  // Only the explicit fmaf calls fuse: the compiler may not contract a product and a sum on its own,
  // which it could do differently in the two instantiations and so make the attention of the fused
  // step differ from decode_attn's in the last bit.
#pragma clang fp contract(off)
  constexpr bool RANK = MODE != 0, MIXED = MODE == 2 || MODE == 3, STASH = MODE == 3, SCORE = MODE == 4;
  constexpr int D = kStD, W = kStW, CPL = kStCPL, P = kStreamAhead;
  constexpr int U = P % 2 == 0 ? P : 2 * P;  // unroll: the stage buffers and the two score sets
  constexpr float hK = 0.5f, hV = 0.5f;    // 1-bit codes: the operand is the sign of s around z + s/2
  static_assert(U == 2 || U == 4, "the remainder steps below are written out for U <= 4");
  __shared__ std::conditional_t<STASH, StreamSmemStash, StreamSmem> sm;

  const int tid = threadIdx.x;
  // the wave index as a wave-uniform (scalar) value: block indices and LDS bases derived from it
  // stay on the scalar unit
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g = lane >> 4;
  const int split = blockIdx.x;
  const int64_t slice = blockIdx.y;
  const int64_t b = slice / Hkv, h = slice % Hkv;
  const int T = a.T;
  const int R = G * T;
  const int Hq = Hkv * G;
  const int64_t row0 = b * Hq * T + h * G * T;
  const float qscale = a.sm_scale * kStLog2e;
  const int64_t p0 = (int64_t)split * L;
  const int64_t p1 = p0 + L < N ? p0 + L : N;
  const int nb = (int)((p1 - p0) / 32);
  const int64_t blk0 = p0 / 32;

  // ---- the kappa indices are loaded before anything else: the scan below then waits for them
  // alone, with the query and staged loads issued after them still in flight
  constexpr int kIdxPre = 2;  // indices per thread loaded up front (the rest, when k > 512, in the scan)
  const int32_t* ix = a.idx + slice * a.k;
  int32_t ixv[kIdxPre];
#pragma unroll
  for (int j = 0; j < kIdxPre; ++j) ixv[j] = tid + 256 * j < a.k ? ix[tid + 256 * j] : 0;

  // ---- query fragments: B[k-slot (g, j)][column n] = q[row n & 7][32w + 8g + j], every row in both
  // halves of the columns.  A 16-token tile's products go to an accumulator of its own, and lane
  // n16 keeps tile n16 >> 3's (columns 0-7: tile 0, 8-15: tile 1): the values attn_split_kernel
  // accumulates for these columns, product for product.  They are the same in every wave and are
  // read back from LDS at each use: three workgroups share a compute unit, and 16 registers held
  // through the loop would not leave room for the third.
  const int arow = n16 & 7;  // query row of this lane's logits
  const bool tile1 = n16 >= 8;
  uint4 bq_ld[W];
#pragma unroll
  for (int w = 0; w < W; ++w)
    bq_ld[w] = arow < R ? load_u4(a.q16 + (row0 + arow) * D + 32 * w + 8 * g) : make_uint4(0, 0, 0, 0);
  auto Bq = [&](int w) {
    Frag f;
    f.v = sm.bq[w][lane];
    return f;
  };

  float m_used = kMergeEmpty;  // running max (log2 units) of accumulator row n16
  float l_part = 0.0f;         // this lane's share of that row's sum of exponentials (low-bit positions)
  float l16 = 0.0f;            // the same over the 16-bit rows (fetched and tail)
  // the C' exponentials of the kappa positions, relative to m_used (ranking statistics over C')
  float l_kappa = 0.0f;
  f32x4 Oacc[CPL];
#pragma unroll
  for (int ct = 0; ct < CPL; ++ct) Oacc[ct] = zero4();
  f32x4 Ozs = zero4();

  const int gshift = a.group == 64 ? 1 : 0;  // groups of 64 (keys: tokens, values: channels)
  const int Wg = W >> gshift;                 // value groups per token
  const int wv_grp = (CPL * n16) >> (5 + gshift);  // value group of this lane's channels
  const bool rank_lane = RANK && arow < R && (arow % T) == a.rank_row;
  const int shv[4] = {15 - 2 * g, 14 - 2 * g, 7 - 2 * g, 6 - 2 * g};
  const float k1 = -0.5f * qscale;  // the expanded key operand is -(2b - 1) s

  // Rescale the accumulators of this lane's rows when a block raises a row maximum by more than
  // 2^kStRescale; xr holds logits relative to the current maximum, recomputed from the absolute
  // values xa on a rescale.
  auto online_update = [&](float (&xr)[4], const float (&xa)[4]) {
    float bm = fmaxf(fmaxf(xr[0], xr[1]), fmaxf(xr[2], xr[3]));
    if (__any(bm > kStRescale)) {
      float ba = fmaxf(fmaxf(xa[0], xa[1]), fmaxf(xa[2], xa[3]));
      ba = max_over_groups(ba);
      const float mn = fmaxf(m_used, ba);
      const float alpha = __builtin_amdgcn_exp2f(m_used - mn);
      m_used = mn;
      l_part *= alpha;
      l16 *= alpha;
      l_kappa *= alpha;
#pragma unroll
      for (int i = 0; i < 4; ++i) xr[i] = xa[i] - mn;
      // whole-accumulator products: the accumulators then keep their registers through this
      // (rarely taken) branch, where per-element products left register copies on the common path
      const f32x4 av = {__shfl(alpha, 4 * g), __shfl(alpha, 4 * g + 1), __shfl(alpha, 4 * g + 2),
                        __shfl(alpha, 4 * g + 3)};
#pragma unroll
      for (int ct = 0; ct < CPL; ++ct) Oacc[ct] = Oacc[ct] * av;
      Ozs = Ozs * av;
    }
  };
  // P (float32, four values of the score layout) -> the value product's A fragment: slots 0-3 hold
  // tile 0's tokens, slots 4-7 tile 1's; each value rounded to nearest even.
  auto make_p = [&](const float (&p)[4], float mul) {
    const uint32_t lo = pack_half2(p[0] * mul, p[1] * mul), hi = pack_half2(p[2] * mul, p[3] * mul);
    Frag A;
    A.u[0] = tile1 ? 0u : lo;
    A.u[1] = tile1 ? 0u : hi;
    A.u[2] = tile1 ? lo : 0u;
    A.u[3] = tile1 ? hi : 0u;
    return A;
  };

  // ================= low-bit blocks, streamed =================
  const int64_t Ns = a.seq_stride, nblk_s = a.seq_stride / 32;  // the cache's layout stride
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const __amdgpu_buffer_rsrc_t kc_buf = make_rsrc(a.k_codes + slice * Ns * W, (uint32_t)(Ns * W * 4));
  const __amdgpu_buffer_rsrc_t km_buf =
      make_rsrc(a.k_meta + slice * (nblk_s >> gshift) * 2 * D, (uint32_t)((nblk_s >> gshift) * 2 * D * 2));
  const __amdgpu_buffer_rsrc_t vc_buf = make_rsrc(a.v_codes + slice * nblk_s * D, (uint32_t)(nblk_s * D * 4));
  const __amdgpu_buffer_rsrc_t vm_buf =
      make_rsrc(a.v_meta + slice * nblk_s * 2 * Wg * 32, (uint32_t)(nblk_s * 2 * Wg * 32 * 2));
  const uint32_t vm_bytes = (uint32_t)(2 * Wg * 32 * 2);  // value metadata of a block: 512 or 256 bytes
  // lane offsets of the staged block: 8 bytes per lane and array (the value metadata of groups of 64
  // is 256 bytes; the upper lanes repeat it)
  const uint32_t off_stage = (uint32_t)(8 * lane), off_stage_vm = off_stage & (vm_bytes - 1);
  // LDS offsets of this lane's 8 bytes of each array in a staged block
  const uint32_t s_kc = (uint32_t)(kStKC + 8 * lane);
  const uint32_t s_km = (uint32_t)(lane < 32 ? kStKM + 8 * lane : kStKS + 8 * (lane - 32));
  const uint32_t s_vc = (uint32_t)(kStVC + 8 * lane + 16 * (lane >> 5));
  const uint32_t s_vm = (uint32_t)(kStVM + 72 * (lane >> 3) + 8 * (lane & 7));
  const __amdgpu_buffer_rsrc_t rl_buf =
      make_rsrc(RANK && a.rank_logits ? static_cast<const void*>(a.rank_logits + slice * G * N)
                                      : static_cast<const void*>(a.q16),
                RANK && a.rank_logits ? (uint32_t)(G * N * 4) : 0u);
  const uint32_t rl_lane = (uint32_t)((arow / T) * N * 4);
  const __amdgpu_buffer_rsrc_t gm_buf =
      make_rsrc(RANK && a.rank_gmax ? static_cast<const void*>(a.rank_gmax + slice * G * (N / kBoundGroup))
                                    : static_cast<const void*>(a.q16),
                RANK && a.rank_gmax ? (uint32_t)(G * (N / kBoundGroup) * 4) : 0u);
  // LDS byte offsets of this lane's operands in a staged block
  const int zrow = n16 < 2 * Wg ? n16 : 0;  // value-metadata row of the zero-point / scale column
  const uint32_t l_kc = (uint32_t)(kStKC + 16 * n16);                         // + 256: tile 1
  const uint32_t l_ks = (uint32_t)(kStKS + 16 * g);                                 // scales, + 64 w
  const uint32_t l_kzs = (uint32_t)(((n16 & 3) == 1 ? kStKS : kStKM) + 16 * g);      // + 64 w
  const uint32_t l_vc = (uint32_t)(kStVC + 4 * CPL * n16 + 16 * (n16 >> 3));         // + 16: channels 4..7
  const uint32_t l_vs = (uint32_t)(kStVM + 72 * (Wg + wv_grp) + 8 * g);             // + 32: tokens 16..
  const uint32_t l_zs = (uint32_t)(kStVM + 72 * zrow + 8 * g);                       // + 32: tokens 16..

  struct Staged {
    u32x4_t kc_km, vc_vm;  // 8 bytes of each array
  };
  auto stage_load = [&](int jj) {
    const uint32_t blk = (uint32_t)(blk0 + jj);
    const auto kc = __builtin_amdgcn_raw_buffer_load_b64(kc_buf, (int)off_stage, (int)(blk * 512u), 0);
    const auto km = __builtin_amdgcn_raw_buffer_load_b64(km_buf, (int)off_stage, (int)((blk >> gshift) * 512u), 0);
    Staged st;
    st.kc_km = u32x4_t{kc[0], kc[1], km[0], km[1]};
    if constexpr (SCORE) {  // keys only
      st.vc_vm = u32x4_t{0u, 0u, 0u, 0u};
    } else {
      const auto vc = __builtin_amdgcn_raw_buffer_load_b64(vc_buf, (int)off_stage, (int)(blk * 512u), 0);
      const auto vm = __builtin_amdgcn_raw_buffer_load_b64(vm_buf, (int)off_stage_vm, (int)(blk * vm_bytes), 0);
      st.vc_vm = u32x4_t{vc[0], vc[1], vm[0], vm[1]};
    }
    return st;
  };
  auto stage_ptr = [&](int slot) { return sm.u.w[wave].stage[slot]; };
  auto stage_store = [&](const Staged& st, int slot) {
    unsigned char* p = stage_ptr(slot);
    *reinterpret_cast<uint2*>(p + s_kc) = make_uint2(st.kc_km[0], st.kc_km[1]);
    *reinterpret_cast<uint2*>(p + s_km) = make_uint2(st.kc_km[2], st.kc_km[3]);
    if constexpr (!SCORE) {
      *reinterpret_cast<uint2*>(p + s_vc) = make_uint2(st.vc_vm[0], st.vc_vm[1]);
      *reinterpret_cast<uint2*>(p + s_vm) = make_uint2(st.vc_vm[2], st.vc_vm[3]);
    }
  };

  // Scores of the staged block in `slot`: the key codes expanded against the queries (chunks w and
  // w + 1 together, one 64-bit shift per pair of words) and the block's constant from four MFMAs
  // whose A rows 4g' and 4g' + 1 are the zero-points and the scales (accumulator registers 0 and 1
  // of every lane then hold sum_c q_c z_c and sum_c q_c s_c of its column's row).
  struct Scores {
    f32x4 x;   // this lane's logits before scaling (its tile)
    float c0;  // the block's constant for the lane's row
  };
  struct KOps {
    uint4 kt[2];   // key codes of tokens n16 and 16 + n16
    uint4 ks[W];   // key scales of the lane's channels, chunk w
    uint4 kzs[W];  // zero-points or scales (by row) for the constant's MFMAs
  };
  auto read_k = [&](int slot) {
    const unsigned char* p = stage_ptr(slot);
    KOps ko;
    ko.kt[0] = *reinterpret_cast<const uint4*>(p + l_kc);
    ko.kt[1] = *reinterpret_cast<const uint4*>(p + l_kc + 256);
#pragma unroll
    for (int w = 0; w < W; ++w) ko.ks[w] = *reinterpret_cast<const uint4*>(p + l_ks + 64 * w);
#pragma unroll
    for (int w = 0; w < W; ++w) ko.kzs[w] = *reinterpret_cast<const uint4*>(p + l_kzs + 64 * w);
    return ko;
  };
  auto score = [&](const KOps& ko) {
    const uint32_t kw[2][4] = {{ko.kt[0].x, ko.kt[0].y, ko.kt[0].z, ko.kt[0].w},
                               {ko.kt[1].x, ko.kt[1].y, ko.kt[1].z, ko.kt[1].w}};
    f32x4 acct[2] = {zero4(), zero4()};
#pragma unroll
    for (int w = 0; w < W; w += 2) {
      const uint4 ka = ko.ks[w], kb = ko.ks[w + 1];
      const uint32_t ma[4] = {ka.x, ka.y, ka.z, ka.w}, mb[4] = {kb.x, kb.y, kb.z, kb.w};
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        Frag A0, A1;  // chunks w, w + 1 of tile tau
#pragma unroll
        for (int d = 0; d < 4; ++d)
          signed_pairs2(kw[tau][w], kw[tau][w + 1], 15 - 4 * g - d, ma[d], mb[d], A0.u[d], A1.u[d]);
        acct[tau] = mma(A0, Bq(w), acct[tau]);
        acct[tau] = mma(A1, Bq(w + 1), acct[tau]);
      }
    }
    f32x4 accc = zero4();
#pragma unroll
    for (int w = 0; w < W; ++w) {
      Frag Z;
      Z.v = ko.kzs[w];
      accc = mma(Z, Bq(w), accc);
    }
    Scores sc;
#pragma unroll
    for (int i = 0; i < 4; ++i) sc.x[i] = tile1 ? acct[1][i] : acct[0][i];
    sc.c0 = fmaf(hK, accc[1], accc[0]) * qscale;
    return sc;
  };

  // The rest of block jj (staged in `slot`, scored into sc): logits, ranking outputs, softmax,
  // values.
  struct VOps {
    uint4 va, vb;                        // value code words of the lane's channels
    uint2 vs_lo, vs_hi, zs_lo, zs_hi;    // value scales, zero-point / scale columns
    uint32_t kmw;                        // kappa positions of the block
  };
  auto read_v = [&](int slot, int jj) {
    const unsigned char* q = stage_ptr(slot);
    VOps vo;
    vo.va = *reinterpret_cast<const uint4*>(q + l_vc);
    vo.vb = *reinterpret_cast<const uint4*>(q + l_vc + 16);
    vo.vs_lo = *reinterpret_cast<const uint2*>(q + l_vs);
    vo.vs_hi = *reinterpret_cast<const uint2*>(q + l_vs + 32);
    vo.zs_lo = *reinterpret_cast<const uint2*>(q + l_zs);
    vo.zs_hi = *reinterpret_cast<const uint2*>(q + l_zs + 32);
    vo.kmw = sm.kmask[jj];
    return vo;
  };
  auto finish = [&](const VOps& vo, const Scores& sc, int jj) {
    const float c0 = sc.c0, c0m = c0 - m_used;
    float xr[4], xa[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xr[i] = fmaf(sc.x[i], k1, c0m);
      xa[i] = fmaf(sc.x[i], k1, c0);
    }
    const uint32_t kmw = vo.kmw;
    if constexpr (RANK) {
      // the rank row's logits against C' (before any kappa masking), log2 units, through the raw
      // buffer over the slice's logits (the block offset is scalar)
      typedef float f4_t __attribute__((ext_vector_type(4)));
      const f4_t v = {xa[0], xa[1], xa[2], xa[3]};
      const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)((blk0 + jj) * 32 * 4));
      const uint32_t voff = rl_lane + 4 * (16 * (n16 >> 3) + 4 * g);
      if constexpr (MIXED && !STASH) {
        // the kappa positions are written by the 16-bit blocks instead
        if (rank_lane && kmw) {
          float* dst = a.rank_logits + (slice * G + arow / T) * N + (blk0 + jj) * 32;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tok = 16 * (n16 >> 3) + 4 * g + i;
            if (!((kmw >> tok) & 1u)) dst[tok] = xa[i];
          }
        } else if (rank_lane) {
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rl_buf, (int)voff, (int)soff, 0);
        }
      } else {
        // issued by every lane, the lanes without a rank row addressing past the buffer (such a
        // store is dropped): with no branch around it the compiler counts it, and the waits for
        // the staged loads stay exact.  An ordinary (cached) store: the selection that follows
        // reads the candidate groups' logits back sooner than with non-temporal stores.  (Form 3
        // stores the kappa positions' low-bit logits too; the end of the kernel writes their
        // 16-bit ones over them.)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), rl_buf,
                                               (int)(rank_lane ? voff : kStDropped), (int)soff, 0);
      }
      // the bound of each 8-position group for the pruned selection (a buffer of size 0 when it
      // is not wanted): lanes g and g ^ 1 of n16 hold the eight logits of row arow at positions
      // 16 (n16 >> 3) + 8 (g >> 1) .. of the block
      const float gm = max_over_group_pairs(fmaxf(fmaxf(xa[0], xa[1]), fmaxf(xa[2], xa[3])));
      const uint32_t goff =
          4u * (uint32_t)((arow / T) * (N / kBoundGroup) + (blk0 + jj) * 4 + 2 * (n16 >> 3) + (g >> 1));
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, gm), gm_buf,
                                            (int)(rank_lane && (g & 1) == 0 ? goff : kStDropped), 0, 0);
    }
    // The running maximum covers every C' logit, kappa positions included: their exponentials
    // are then the ranking statistics' terms over C' as they stand, and the attention drops them
    // (their 16-bit rows take their place).
    online_update(xr, xa);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(xr[i]);
    if (kmw) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = 16 * (n16 >> 3) + 4 * g + i;
        if ((kmw >> tok) & 1u) {
          if constexpr (RANK && !MIXED) l_kappa += p[i];
          p[i] = 0.0f;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) l_part += p[i];
    if constexpr (SCORE) return;  // the statistics are all a score pass keeps
    const Frag Ap = make_p(p, 1.0f);

    // values: the value codes expanded against P, plus one MFMA whose columns are the per-token
    // zero-points and scales
    const uint32_t vw[CPL] = {vo.va.x, vo.va.y, vo.va.z, vo.va.w, vo.vb.x, vo.vb.y, vo.vb.z, vo.vb.w};
    const uint2 vs_lo = vo.vs_lo, vs_hi = vo.vs_hi, zs_lo = vo.zs_lo, zs_hi = vo.zs_hi;
    const uint32_t vmag[4] = {vs_lo.x, vs_lo.y, vs_hi.x, vs_hi.y};
#pragma unroll
    for (int ct = 0; ct < CPL; ct += 2) {
      Frag Bv0, Bv1;  // channel tiles ct and ct + 1, one 64-bit shift per pair of words
#pragma unroll
      for (int d = 0; d < 4; ++d) signed_pairs2(vw[ct], vw[ct + 1], shv[d], vmag[d], vmag[d], Bv0.u[d], Bv1.u[d]);
      Oacc[ct] = mma(Ap, Bv0, Oacc[ct]);
      Oacc[ct + 1] = mma(Ap, Bv1, Oacc[ct + 1]);
    }
    // columns n16 >= 2 Wg carry another row's (finite) metadata: their outputs are never read
    Frag Bzs;
    Bzs.u[0] = zs_lo.x;
    Bzs.u[1] = zs_lo.y;
    Bzs.u[2] = zs_hi.x;
    Bzs.u[3] = zs_hi.y;
    Ozs = mma(Ap, Bzs, Ozs);
  };

  // low-bit blocks jj = wave + 4 i of this wave; their first P blocks' loads are issued before
  // anything else, so that they are in flight through the kappa scan and the fetched 16-bit blocks
  const int vw = wave;
  const int nw = vw < nb ? (nb - vw + 3) / 4 : 0;
  // clamped to the last block (block 0 for a wave with none, whose loads are then unused): the
  // loads are issued unconditionally, so that the waits for the ones before them stay exact
  auto blk = [&](int i) { return nw > 0 ? vw + 4 * (i < nw ? i : nw - 1) : 0; };
  Staged stg[P];
#pragma unroll
  for (int j = 0; j < P; ++j) stg[j] = stage_load(blk(j));

  if (RANK && split == 0)  // the rank kernels accumulate a per-slice histogram here
    for (int i = tid; i < 2048; i += 256) a.rank_hist[slice * 2048 + i] = 0u;

  // ---- kappa positions of this split: a bitmask over its blocks and the range [i0, i1) of the
  // fetched rows whose positions fall in it (idx is ascending)
  for (int i = tid; i < kAttnMaxBlocks; i += 256) sm.kmask[i] = 0u;
  if (tid < 2) sm.sel_range[tid] = 0;
  __syncthreads();
  {
    int below0 = 0, below1 = 0;
    auto take = [&](int64_t p) {
      below0 += p < p0 ? 1 : 0;
      below1 += p < p1 ? 1 : 0;
      if (p >= p0 && p < p1) atomicOr(&sm.kmask[(p - p0) >> 5], 1u << ((p - p0) & 31));
    };
#pragma unroll
    for (int j = 0; j < kIdxPre; ++j)
      if (tid + 256 * j < a.k) take(ixv[j]);
    for (int i = tid + 256 * kIdxPre; i < a.k; i += 256) take(ix[i]);
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
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < W; ++w) sm.bq[w][lane] = bq_ld[w];
  }
  __syncthreads();
  const int i0 = sm.sel_range[0], i1 = sm.sel_range[1];

  // ================= 16-bit rows: the fetched kappa rows of this split, then the tail =================
  // 16-bit block q (the fetched rows' blocks, then the tail's) goes to wave 3 - q mod 4: the waves
  // with the fewest low-bit blocks take them first.  The fetched rows' blocks run before the
  // low-bit blocks and the tail's after them; their exponentials go to l16, so the low-bit sums
  // l_part stay the ranking statistics over C'.
  const int n_sel = i1 - i0;
  const bool has_tail = (split == S - 1) && a.tail > 0;
  const int n_sel_blk = (n_sel + 31) / 32;
  const int n_tail_blk = has_tail ? (a.tail + 31) / 32 : 0;
  const int first_tail_q = n_sel_blk + ((3 - wave - n_sel_blk) % 4 + 4) % 4;  // first q >= n_sel_blk of this wave
  auto f16_block = [&](int q) {
    const bool tail = q >= n_sel_blk;
    const int base = tail ? 32 * (q - n_sel_blk) : i0 + 32 * q;
    const int lim = tail ? a.tail : i1;
    const _Float16* ksrc = tail ? a.k_tail + slice * a.tail * D : a.k_sel + slice * a.k * D;
    const _Float16* vsrc = tail ? a.v_tail + slice * a.tail * D : a.v_sel + slice * a.k * D;
    _Float16(*vt)[kStRS] = sm.u.w[wave].vt;
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
        for (int j = 0; j < 8; ++j) vt[32 * w + 8 * g + j][tok] = v.h[j];
      }
    }
    f32x4 acct[2] = {zero4(), zero4()};
#pragma unroll
    for (int w = 0; w < W; ++w) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        Frag A;
        A.v = (base + 16 * tau + n16 < lim) ? kk[tau][w].v : make_uint4(0, 0, 0, 0);
        acct[tau] = mma(A, Bq(w), acct[tau]);
      }
    }
    float xr[4], xa[4];
    const int tq = arow % T;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 16 * (n16 >> 3) + 4 * g + i;
      const float v = (tile1 ? acct[1][i] : acct[0][i]) * qscale;
      bool ok = base + tok < lim;
      if constexpr (RANK) {
        // ranking by the mixed cache: a fetched row's logit replaces its low-bit one
        if (MIXED && rank_lane && !tail && ok) {
          if constexpr (STASH) {
            sm.kst[(base - i0 + tok) * G + arow / T] = v;  // the split's fetched row base - i0 + tok
          } else {
            const int64_t pos = a.idx[slice * a.k + base + tok];
            a.rank_logits[(slice * G + arow / T) * N + pos] = v;
          }
        }
      }
      if (tail) ok = ok && (base + tok <= a.tail - T + tq);
      xa[i] = ok ? v : -INFINITY;
      xr[i] = xa[i] - m_used;
    }
    online_update(xr, xa);
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = __builtin_amdgcn_exp2f(xr[i]);
      l16 += p[i];
    }
    const Frag Ap2 = make_p(p, -2.0f);  // the value accumulator is scaled by -1/2 at the end
    st_lds_fence();
#pragma unroll
    for (int ct = 0; ct < CPL; ++ct) {
      const int c = CPL * n16 + ct;
      const uint2 lo = load_u2(&vt[c][4 * g]);
      const uint2 hi = load_u2(&vt[c][16 + 4 * g]);
      Frag Bv;
      Bv.u[0] = lo.x;
      Bv.u[1] = lo.y;
      Bv.u[2] = hi.x;
      Bv.u[3] = hi.y;
      Oacc[ct] = mma(Ap2, Bv, Oacc[ct]);
    }
    st_lds_fence();
  };

  __builtin_amdgcn_s_setprio(3);  // a chain of latencies: issue it ahead of the other waves' loops
  for (int q = 3 - wave; q < n_sel_blk; q += 4) f16_block(q);

  if (nw > 0) {
    // Step i (r = i mod U): block i + 1's bytes go to its slot and its buffer takes block
    // i + 1 + P's loads; block i + 1 is scored while block i is finished, so the matrix cores work
    // on one block while the VALU finishes the other.  Buffers, slots and score sets are indexed
    // by r, so that the unrolled steps address fixed registers.
    Scores sc[2];
    auto step = [&](int i, auto rc) {
      constexpr int r = decltype(rc)::value;
      constexpr int b1 = (r + 1) % P, s1 = (r + 1) & 1, s0 = r & 1;
      // each block's LDS reads sit next to its arithmetic: at three waves per SIMD there is no
      // room to hold both blocks' operands at once
      stage_store(stg[b1], s1);
      stg[b1] = stage_load(blk(i + 1 + P));
      if (i + 1 < nw) sc[s1] = score(read_k(s1));
      finish(read_v(s0, blk(i)), sc[s0], blk(i));
    };
    stage_store(stg[0], 0);
    stg[0] = stage_load(blk(P));
    sc[0] = score(read_k(0));
    // Issue priority by the blocks this wave has left: three workgroups share each compute unit, and
    // the SIMD arbiter otherwise favours the oldest, which then finishes long before the others and
    // leaves fewer waves per SIMD for the rest.
    const int pr1 = nw / 16 + 1, pr2 = nw / 6 + 1, pr3 = nw / 3 + 1;
    int i = 0;
    for (; i + U <= nw; i += U) {
      const int rem = nw - i;
      if (rem > pr3) __builtin_amdgcn_s_setprio(3);
      else if (rem > pr2) __builtin_amdgcn_s_setprio(2);
      else if (rem > pr1) __builtin_amdgcn_s_setprio(1);
      else __builtin_amdgcn_s_setprio(0);
      step(i, IC<0>{});
      step(i + 1, IC<1>{});
      if constexpr (U == 4) {
        step(i + 2, IC<2>{});
        step(i + 3, IC<3>{});
      }
    }
    // the last nw mod U blocks, each step on the path of the one before it
    __builtin_amdgcn_s_setprio(0);
    if (i < nw) {
      step(i, IC<0>{});
      if constexpr (U == 4) {
        if (i + 1 < nw) {
          step(i + 1, IC<1>{});
          if (i + 2 < nw) step(i + 2, IC<2>{});
        }
      }
    }
  }

  __builtin_amdgcn_s_setprio(3);  // the rest of the workgroup is a chain of latencies: let it through

  // ranking statistics over C' = the low-bit positions, kappa positions included (the same
  // maximum in the four lanes of a row)
  const float rank_m_lane = m_used, rank_l_lane = l_part + l_kappa;

  // ================= 16-bit rows of the tail (the fetched rows went first) =================
  for (int q = first_tail_q; q < n_sel_blk + n_tail_blk; q += 4) f16_block(q);

  // ================= wave epilogue =================
  // per accumulator row: the final (max, sum); with tile 0's rows in n16 < 8 and tile 1's in
  // n16 >= 8, fold the two tiles of a query row
  const float l_row = sum_over_groups(l_part + l16);
  const float m2 = __shfl_xor(m_used, 8);
  const float l2 = __shfl_xor(l_row, 8);
  const float mm = fmaxf(m_used, m2);
  const float f_self = __builtin_amdgcn_exp2f(m_used - mm);
  const float f_other = __builtin_amdgcn_exp2f(m2 - mm);
  if constexpr (RANK && !MIXED) {  // (the mixed ranking takes the attention's own statistics)
    float rl = sum_over_groups(rank_l_lane), rm = rank_m_lane;
    const float rm2 = __shfl_xor(rm, 8), rl2 = __shfl_xor(rl, 8);
    const float rmm = fmaxf(rm, rm2);
    rl = rl * __builtin_amdgcn_exp2f(rm - rmm) + rl2 * __builtin_amdgcn_exp2f(rm2 - rmm);
    if (g == 0) {
      sm.rank_m[wave][n16] = rmm;
      sm.rank_l[wave][n16] = rl;
    }
  }
  __syncthreads();  // all waves are done with their tiles and slots; the LDS union becomes the combine buffer
  if constexpr (STASH) {
    // the fetched rows' 16-bit logits over the low-bit ones the loop stored at their positions
    const int n_kst = (i1 - i0) * G;
    for (int e = tid; e < n_kst; e += 256) {
      const int r = e / G, hh = e - r * G;
      a.rank_logits[(slice * G + hh) * N + ix[i0 + r]] = sm.kst[e];
    }
  }
  if constexpr (RANK) {
    // one thread per head: combine the four waves and write this split's statistics over C'
    if (!MIXED && tid < G) {
      const int r = tid * T + a.rank_row;
      float M = kMergeEmpty;
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) M = fmaxf(M, sm.rank_m[w4][r]);
      float Ls = 0.0f;
#pragma unroll
      for (int w4 = 0; w4 < 4; ++w4) Ls += sm.rank_l[w4][r] * __builtin_amdgcn_exp2f(sm.rank_m[w4][r] - M);
      a.rank_m[(slice * G + tid) * S + split] = M;
      a.rank_l[(slice * G + tid) * S + split] = Ls;
    }
  }
  if constexpr (SCORE) return;  // a score pass writes no attention output (every thread leaves here)
  if (g == 0 && n16 < 8) {
    sm.u.comb.m[wave][n16] = mm;
    sm.u.comb.l[wave][n16] = f_self * l_row + f_other * l2;
  }
  // accumulator rows 4g' + i of the lane's channels in final form, -O/2 + Z + h S with Z and S the
  // zero-point and scale columns of the channels' value group in the metadata product (held by
  // lanes wv_grp and Wg + wv_grp of the same k-group); then rows r and r + 8 (the two tiles of a
  // query row, lanes g' and g' ^ 2) fold into r (lanes g' < 2) with their weights
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * g + i;
    const float zl = __shfl(Ozs[i], 16 * g + wv_grp);
    const float sl = __shfl(Ozs[i], 16 * g + Wg + wv_grp);
    const float base = zl + hV * sl;
    const float ws = __shfl(f_self, r & 7);
    const float wo = __shfl(f_other, r & 7);
    float ov[CPL];
#pragma unroll
    for (int ct = 0; ct < CPL; ++ct) ov[ct] = -0.5f * Oacc[ct][i] + base;
#pragma unroll
    for (int ct = 0; ct < CPL; ++ct) ov[ct] = ws * ov[ct] + wo * __shfl_xor(ov[ct], 32);
    if (g < 2) {
      float4* dst = reinterpret_cast<float4*>(&sm.u.comb.o[wave][r][CPL * n16]);
      dst[0] = make_float4(ov[0], ov[1], ov[2], ov[3]);
      dst[1] = make_float4(ov[4], ov[5], ov[6], ov[7]);
    }
  }
  __syncthreads();

  // ================= combine the four waves and write this split's partials =================
  // row r = tid / 32, channels 4 (tid mod 32) .. + 3
  const int r = tid >> 5, c = 4 * (tid & 31);
  if (r < R) {
    float mw[4], M = kMergeEmpty;
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
      mw[w4] = sm.u.comb.m[w4][r];
      M = fmaxf(M, mw[w4]);
    }
    float lsum = 0.0f;
    float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll
    for (int w4 = 0; w4 < 4; ++w4) {
      const float e4 = __builtin_amdgcn_exp2f(mw[w4] - M);
      lsum += e4 * sm.u.comb.l[w4][r];
      const float4 ow = *reinterpret_cast<const float4*>(&sm.u.comb.o[w4][r][c]);
      o.x += e4 * ow.x;
      o.y += e4 * ow.y;
      o.z += e4 * ow.z;
      o.w += e4 * ow.w;
    }
    const int64_t row = row0 + r;
    *reinterpret_cast<float4*>(&a.part_acc[(row * S + split) * D + c]) = o;
    if (c == 0) {
      a.part_ml[(row * S + split) * 2] = M;
      a.part_ml[(row * S + split) * 2 + 1] = lsum;
      if constexpr (RANK) {
        // ranking by the mixed cache: the rank row's own softmax statistics of this split
        if (MIXED && r % T == a.rank_row) {
          a.rank_m[(slice * G + r / T) * S + split] = M;
          a.rank_l[(slice * G + r / T) * S + split] = lsum;
        }
      }
    }
  }
}

}  // namespace

bool attn_stream_serves(const Dims& d, const AttnArgs& a) {
  return d.D == kStD && d.bits == 1 && d.vbits == 1 && d.G * a.T <= 8;
}

hipError_t launch_score_stream(const Dims& d, const AttnPlan& plan, const AttnArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)plan.S, (unsigned)d.slices());
  attn_stream_kernel<4><<<grid, 256, 0, s>>>(a, d.Hkv, d.G, d.N, plan.L, plan.S);
  return hipGetLastError();
}

hipError_t launch_attn_stream(const Dims& d, const AttnPlan& plan, const AttnArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)plan.S, (unsigned)d.slices());
  if (!a.rank_logits)
    attn_stream_kernel<0><<<grid, 256, 0, s>>>(a, d.Hkv, d.G, d.N, plan.L, plan.S);
  else if (!a.rank_mixed)
    attn_stream_kernel<1><<<grid, 256, 0, s>>>(a, d.Hkv, d.G, d.N, plan.L, plan.S);
  else if ((int64_t)a.k * d.G <= kStashFloats)
    attn_stream_kernel<3><<<grid, 256, 0, s>>>(a, d.Hkv, d.G, d.N, plan.L, plan.S);
  else
    attn_stream_kernel<2><<<grid, 256, 0, s>>>(a, d.Hkv, d.G, d.N, plan.L, plan.S);
  return hipGetLastError();
}

}  // namespace specache
