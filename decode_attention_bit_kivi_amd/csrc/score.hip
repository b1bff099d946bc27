// Low-bit scoring for the speculative ranking: the logits of the rank row's G
// query heads against the dequantized keys of C', plus per-split softmax
// statistics per head.
//
// SpeCache summary, quick read (second mechanism) and §3 "prefetch and offload
// during decoding": the speculative token's attention over the low-bit copy
// decides which 16-bit pairs to fetch.
//
// Within a 32-token key block the zero-point z and scale s are per channel:
//   q . Khat(p) = sum_c q_c (z_c + h s_c) - (1/2) sum_c q_c (-(2b - 1) s_c)   (1 bit, h = 1/2)
// The first sum is one number per (block, head) and comes from a small MFMA
// prepass (zero-points and scales of 16 blocks against the queries); the
// second is a matrix product of the expanded codes (mfma_frag.h) with the
// float16 queries on the matrix cores.  Every product is exact, so the
// logits carry only float32 accumulation error (the ranking tie band is 1e-5).
// Two bits: h = 3/2 and plane 1 enters with weight 1.
//
// Layout: grid (splits, slices), 256 threads = 4 waves; a wave owns every
// 4th 32-position block of its split.  With at most 8 heads the two 16-token
// tiles of a block share one accumulator (heads in columns 0-7 for tile 0,
// 8-15 for tile 1).  Logits go to [slice][head][position] as float32 in log2
// units (natural-unit logit times log2 e); the
// per-split statistics are (max, sum of 2^(x - max)) in log2 units.
#include "mfma_frag.h"

namespace specache {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int D, int BITS, int PACK>
__global__ __launch_bounds__(256, 2) void score_kernel(const _Float16* __restrict__ q16, int T, int rank_row,
                                                       const uint32_t* __restrict__ k_codes,
                                                       const _Float16* __restrict__ k_meta, int64_t N, int64_t Ns,
                                                       int gshift, int G,
                                                       int Hkv, float sm_scale, int64_t L, int S,
                                                       float* __restrict__ logits, float* __restrict__ part_m,
                                                       float* __restrict__ part_l, uint32_t* __restrict__ hist) {
  constexpr int W = D / 32;
  constexpr float hK = BITS == 1 ? 0.5f : 1.5f;
  const float qscale = sm_scale * kLog2e;  // the logits are written in log2 units
  constexpr int NX = PACK == 2 ? 4 : 8;
  __shared__ float cst[4][16][16];
  __shared__ float red_m[4][16], red_l[4][16];

  const int tid = threadIdx.x;
  // the wave index as a wave-uniform (scalar) value: block indices and base offsets stay scalar
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n16 = lane & 15, g = lane >> 4;
  const int split = blockIdx.x;
  const int64_t slice = blockIdx.y;
  const int64_t b = slice / Hkv, h = slice % Hkv;
  const int Hq = Hkv * G;
  const int64_t ngrp_s = Ns >> (5 + gshift);  // the cache's layout stride in key groups (32 << gshift)
  const int64_t p0 = (int64_t)split * L;
  const int64_t p1 = p0 + L < N ? p0 + L : N;
  const int nb = (int)((p1 - p0) / 32);
  const int64_t blk0 = p0 / 32;
  if (split == 0)  // the rank kernels accumulate a per-slice histogram here
    for (int i = tid; i < 2048; i += 256) hist[slice * 2048 + i] = 0u;

  // query fragments of the rank row: B[k-slot (g, j)][column] = q[head][32w + 8g + j]
  Frag B0[W], B1[W];
  {
    const int r0 = PACK == 2 ? (n16 < 8 ? n16 : -1) : n16;
    const int r1 = PACK == 2 ? (n16 >= 8 ? n16 - 8 : -1) : -1;
    const int ra = r0 >= 0 && r0 < G ? r0 : 0, rb = r1 >= 0 && r1 < G ? r1 : 0;
    const _Float16* qa = q16 + ((b * Hq + h * G + ra) * T + rank_row) * D;
    const _Float16* qb = q16 + ((b * Hq + h * G + rb) * T + rank_row) * D;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const uint4 va = load_u4(qa + 32 * w + 8 * g), vb = load_u4(qb + 32 * w + 8 * g);
      B0[w].v = (r0 >= 0 && r0 < G) ? va : make_uint4(0, 0, 0, 0);
      B1[w].v = (r1 >= 0 && r1 < G) ? vb : make_uint4(0, 0, 0, 0);
    }
  }

  struct BlockData {
    Words<W> kw[2][BITS];
    uint4 ks[W];
  };
  // Raw buffers over the slice's codes and key metadata: a block's offset is scalar, each lane
  // adds a loop-invariant offset.
  const __amdgpu_buffer_rsrc_t kc_buf = make_rsrc(k_codes + slice * Ns * BITS * W, (uint32_t)(Ns * BITS * W * 4));
  const __amdgpu_buffer_rsrc_t km_buf = make_rsrc(k_meta + slice * ngrp_s * 2 * D, (uint32_t)(ngrp_s * 2 * D * 2));
  const uint32_t off_k = (uint32_t)(n16 * BITS * W * 4), off_m = (uint32_t)((D + 8 * g) * 2);
  auto load_block = [&](int jj) {
    BlockData bd;
    const int64_t blk = blk0 + jj;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int pl = 0; pl < BITS; ++pl)
        bd.kw[tau][pl] = buffer_words<W>(kc_buf, off_k + (uint32_t)((16 * tau * BITS + pl) * W * 4),
                                         (uint32_t)(blk * 32 * BITS * W * 4));
    const uint32_t moff = (uint32_t)((blk >> gshift) * 2 * D * 2);  // the group's zero-points; scales follow
#pragma unroll
    for (int w = 0; w < W; ++w) {
      const Words<4> v = buffer_words<4>(km_buf, off_m + (uint32_t)(32 * w * 2), moff);
      bd.ks[w] = make_uint4(v.w[0], v.w[1], v.w[2], v.w[3]);
    }
    return bd;
  };

  float m2 = -INFINITY, l2 = 0.0f;   // this lane's running (max, sum 2^(x - max)) in log2 units
  const int head = PACK == 2 ? (n16 & 7) : n16;
  const bool writer = head < G;
  const __amdgpu_buffer_rsrc_t lg_buf = make_rsrc(logits + slice * G * N, (uint32_t)(G * N * 4));
  const uint32_t lg_lane = (uint32_t)((writer ? head : 0) * N * 4);

  BlockData cur;
  if (wave < nb) cur = load_block(wave);
  for (int jj = wave; jj < nb; jj += 4) {
    const int step = (jj - wave) >> 2;
    const bool prepass = (step & 15) == 0;
    Frag az[W], as[W];
    if (prepass) {
      const int bi = jj + 4 * n16;
      const _Float16* km = k_meta + (slice * ngrp_s + ((blk0 + (bi < nb ? bi : jj)) >> gshift)) * 2 * D;
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
      for (int i = 0; i < 4; ++i) cst[wave][4 * g + i][n16] = accZ[i] + hK * accS[i];
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }

    f32x4 acc[2][BITS];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int pl = 0; pl < BITS; ++pl) acc[tau][pl] = zero4();
    // chunks w and w + 1 expand together (one 64-bit shift per pair of words); the products
    // accumulate in the order w, tau as for one chunk at a time
#pragma unroll
    for (int w = 0; w < W; w += 2) {
      const uint32_t* ma = reinterpret_cast<const uint32_t*>(&cur.ks[w]);
      const uint32_t* mb = reinterpret_cast<const uint32_t*>(&cur.ks[w + 1]);
#pragma unroll
      for (int pl = 0; pl < BITS; ++pl) {
        Frag A0[2], A1[2];  // [tau]: chunk w, chunk w + 1
#pragma unroll
        for (int tau = 0; tau < 2; ++tau)
#pragma unroll
          for (int d = 0; d < 4; ++d)
            signed_pairs2(cur.kw[tau][pl].w[w], cur.kw[tau][pl].w[w + 1], 15 - 4 * g - d, ma[d], mb[d], A0[tau].u[d],
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
    const float c0 = cst[wave][step & 15][head];
    float x[NX];
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int tau = PACK == 2 ? 0 : i / 4;
      const float s = BITS == 1 ? -0.5f * acc[tau][0][i & 3] : -0.5f * acc[tau][0][i & 3] - acc[tau][BITS - 1][i & 3];
      x[i] = qscale * (c0 + s);  // log2 units
    }
    if (writer) {  // through the raw buffer over the slice's logits (block offset scalar)
      const uint32_t soff = (uint32_t)((blk0 + jj) * 32 * 4);
      typedef float f4_t __attribute__((ext_vector_type(4)));
      typedef unsigned int u4_t __attribute__((ext_vector_type(4)));
      if constexpr (PACK == 2) {
        const f4_t v = {x[0], x[1], x[2], x[3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4_t, v), lg_buf,
                                               (int)(lg_lane + 4 * (16 * (n16 >> 3) + 4 * g)), (int)soff, 0);
      } else {
        const f4_t v0 = {x[0], x[1], x[2], x[3]}, v1 = {x[4], x[5], x[6], x[7]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4_t, v0), lg_buf, (int)(lg_lane + 16 * g),
                                               (int)soff, 0);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u4_t, v1), lg_buf, (int)(lg_lane + 4 * (16 + 4 * g)),
                                               (int)soff, 0);
      }
    }
    float bm = x[0];
#pragma unroll
    for (int i = 1; i < NX; ++i) bm = fmaxf(bm, x[i]);
    const float mn = fmaxf(m2, bm);
    float add = 0.0f;
#pragma unroll
    for (int i = 0; i < NX; ++i) add += __builtin_amdgcn_exp2f(x[i] - mn);
    l2 = l2 * __builtin_amdgcn_exp2f(m2 - mn) + add;
    m2 = mn;
    cur = nxt;
  }

  // per head: combine the lanes of the head (k-groups and, with PACK == 2, both tiles), then the waves
  auto combine = [](float& m, float& l, float mo, float lo) {
    const float mn = fmaxf(m, mo);
    l = (mn == -INFINITY) ? 0.0f : l * __builtin_amdgcn_exp2f(m - mn) + lo * __builtin_amdgcn_exp2f(mo - mn);
    m = mn;
  };
  {
    float mo = __shfl_xor(m2, 16), lo = __shfl_xor(l2, 16);
    combine(m2, l2, mo, lo);
    mo = __shfl_xor(m2, 32);
    lo = __shfl_xor(l2, 32);
    combine(m2, l2, mo, lo);
    if constexpr (PACK == 2) {
      mo = __shfl_xor(m2, 8);
      lo = __shfl_xor(l2, 8);
      combine(m2, l2, mo, lo);
    }
  }
  if (lane < 16) {
    red_m[wave][lane] = m2;
    red_l[wave][lane] = l2;
  }
  __syncthreads();
  if (tid < G) {
    float m = red_m[0][tid], l = red_l[0][tid];
#pragma unroll
    for (int w4 = 1; w4 < 4; ++w4) combine(m, l, red_m[w4][tid], red_l[w4][tid]);
    part_m[(slice * G + tid) * S + split] = m;
    part_l[(slice * G + tid) * S + split] = l;
  }
}

template <int D, int BITS>
void launch_score_t(const Dims& d, const ScorePlan& plan, const _Float16* q16, int n_tokens, int rank_row,
                    const uint32_t* k_codes, const _Float16* k_meta, float sm_scale, float* logits, float* part_m,
                    float* part_l, uint32_t* hist, hipStream_t s) {
  const dim3 grid((unsigned)plan.S, (unsigned)d.slices());
  if (d.G <= 8)
    score_kernel<D, BITS, 2><<<grid, 256, 0, s>>>(q16, n_tokens, rank_row, k_codes, k_meta, d.N, d.Ns, d.group == 64 ? 1 : 0, d.G, d.Hkv,
                                                  sm_scale, plan.L, plan.S, logits, part_m, part_l, hist);
  else
    score_kernel<D, BITS, 1><<<grid, 256, 0, s>>>(q16, n_tokens, rank_row, k_codes, k_meta, d.N, d.Ns, d.group == 64 ? 1 : 0, d.G, d.Hkv,
                                                  sm_scale, plan.L, plan.S, logits, part_m, part_l, hist);
}

}  // namespace

hipError_t launch_score(const Dims& d, const ScorePlan& plan, const _Float16* q16, int n_tokens,
                        int rank_row, const uint32_t* k_codes, const _Float16* k_meta, float sm_scale,
                        float* logits, float* part_m, float* part_l, uint32_t* hist, hipStream_t s) {
  if (d.D == 128) {
    if (d.bits == 1)
      launch_score_t<128, 1>(d, plan, q16, n_tokens, rank_row, k_codes, k_meta, sm_scale, logits, part_m, part_l, hist, s);
    else
      launch_score_t<128, 2>(d, plan, q16, n_tokens, rank_row, k_codes, k_meta, sm_scale, logits, part_m, part_l, hist, s);
  } else {
    if (d.bits == 1)
      launch_score_t<64, 1>(d, plan, q16, n_tokens, rank_row, k_codes, k_meta, sm_scale, logits, part_m, part_l, hist, s);
    else
      launch_score_t<64, 2>(d, plan, q16, n_tokens, rank_row, k_codes, k_meta, sm_scale, logits, part_m, part_l, hist, s);
  }
  return hipGetLastError();
}

}  // namespace specache
