// Low-bit scoring for the speculative ranking: logits of the rank row's G
// query heads against the dequantized keys of C', plus per-split softmax
// statistics (running max and sum of exponentials) per head.
//
// SpeCache summary, quick read (second mechanism) and §3 "prefetch and offload
// during decoding": the speculative token's attention over the low-bit copy
// decides which 16-bit pairs to fetch.
//
// Within a 32-token key block the zero-point and scale are per channel, so
//   q . Khat(p) = sum_c q_c z_c + sum_c (q_c s_c) code(p, c):
// the first sum is one number per (block, head) and the second is a dot
// product of a per-block table a_c = q_c s_c with the codes.
//
// Layout: grid (splits, slices), 128 threads; a split is L positions (a
// multiple of 128) walked in rounds of 128 positions = 4 key blocks, one
// position per thread.
#include "common.h"

namespace specache {

namespace {

template <int D>
__global__ __launch_bounds__(128) void score_kernel(const _Float16* __restrict__ q16, int T, int rank_row,
                                                    const uint32_t* __restrict__ k_codes,
                                                    const _Float16* __restrict__ k_meta, int64_t N,
                                                    int bits, int G, int Hkv, float sm_scale, int64_t L,
                                                    int S, float* __restrict__ logits,
                                                    float* __restrict__ part_m, float* __restrict__ part_l) {
  constexpr int W = D / 32;
  __shared__ float qs[kMaxRows][D];
  __shared__ float zs[4][2][D];
  __shared__ float atab[4][D][kMaxRows];
  __shared__ float ctab[4][kMaxRows];
  __shared__ float red_m[2][kMaxRows];
  __shared__ float red_l[2][kMaxRows];

  const int t = threadIdx.x;
  const int split = blockIdx.x;
  const int64_t slice = blockIdx.y;
  const int64_t b = slice / Hkv, h = slice % Hkv;
  const int64_t nblk = N / 32;
  const int Hq = Hkv * G;

  for (int e = t; e < G * D; e += 128) {
    const int g = e / D, c = e % D;
    qs[g][c] = (float)q16[((b * Hq + h * G + g) * T + rank_row) * D + c];
  }

  float m_run[kMaxRows], l_run[kMaxRows];
#pragma unroll
  for (int g = 0; g < kMaxRows; ++g) {
    m_run[g] = -INFINITY;
    l_run[g] = 0.0f;
  }

  const int64_t p_begin = (int64_t)split * L;
  const int64_t p_end = p_begin + L < N ? p_begin + L : N;
  for (int64_t p0 = p_begin; p0 < p_end; p0 += 128) {
    const int nb = (int)((p_end - p0) / 32 < 4 ? (p_end - p0) / 32 : 4);
    const int64_t blk0 = p0 / 32;
    __syncthreads();  // previous round's tables are no longer read
    for (int e = t; e < nb * 2 * D; e += 128)
      zs[e / (2 * D)][(e / D) & 1][e % D] = (float)k_meta[(slice * nblk + blk0) * 2 * D + e];
    __syncthreads();
    for (int e = t; e < nb * D * G; e += 128) {
      const int bb = e / (D * G), r = e % (D * G);
      const int cp = r / G, g = r % G;
      const int c = 32 * (cp / 32) + bit_to_elem(cp % 32);
      atab[bb][cp][g] = qs[g][c] * zs[bb][1][c];
    }
    for (int pr = t; pr < nb * G; pr += 128) {
      const int bb = pr / G, g = pr % G;
      float acc = 0.0f;
      for (int c = 0; c < D; ++c) acc = fmaf(qs[g][c], zs[bb][0][c], acc);
      ctab[bb][g] = acc;
    }
    __syncthreads();

    const int64_t p = p0 + t;
    if (p < p_end) {
      const int bb = t / 32;
      uint32_t wd[2][W];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int w = 0; w < W; ++w) wd[j][w] = (j < bits) ? k_codes[((slice * N + p) * bits + j) * W + w] : 0u;
      float acc[kMaxRows];
#pragma unroll
      for (int g = 0; g < kMaxRows; ++g) acc[g] = 0.0f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        for (int i = 0; i < 32; ++i) {
          const float cf = (float)(((wd[0][w] >> i) & 1u) + 2u * ((wd[1][w] >> i) & 1u));
          const float* a = &atab[bb][32 * w + i][0];
#pragma unroll
          for (int g = 0; g < kMaxRows; ++g)
            if (g < G) acc[g] = fmaf(cf, a[g], acc[g]);
        }
      }
#pragma unroll
      for (int g = 0; g < kMaxRows; ++g) {
        if (g < G) {
          const float x = sm_scale * (ctab[bb][g] + acc[g]);
          logits[(slice * G + g) * N + p] = x;
          const float mn = fmaxf(m_run[g], x);
          l_run[g] = l_run[g] * __expf(m_run[g] - mn) + __expf(x - mn);
          m_run[g] = mn;
        }
      }
    }
  }

  // Reduce (m, l) per head over the 128 threads: within each wave, then across the two waves.
  const int lane = t & 63, wv = t >> 6;
#pragma unroll
  for (int g = 0; g < kMaxRows; ++g) {
    float m = m_run[g], l = l_run[g];
    for (int off = 32; off > 0; off >>= 1) {
      const float mo = __shfl_xor(m, off);
      const float lo = __shfl_xor(l, off);
      const float mn = fmaxf(m, mo);
      l = (mn == -INFINITY) ? 0.0f : l * __expf(m - mn) + lo * __expf(mo - mn);
      m = mn;
    }
    if (lane == 0) {
      red_m[wv][g] = m;
      red_l[wv][g] = l;
    }
  }
  __syncthreads();
  if (t < G) {
    const float m0 = red_m[0][t], m1 = red_m[1][t];
    const float mn = fmaxf(m0, m1);
    const float l = (mn == -INFINITY) ? 0.0f : red_l[0][t] * __expf(m0 - mn) + red_l[1][t] * __expf(m1 - mn);
    part_m[(slice * G + t) * S + split] = mn;
    part_l[(slice * G + t) * S + split] = l;
  }
}

}  // namespace

hipError_t launch_score(const Dims& d, const ScorePlan& plan, const _Float16* q16, int n_tokens,
                        int rank_row, const uint32_t* k_codes, const _Float16* k_meta, float sm_scale,
                        float* logits, float* part_m, float* part_l, hipStream_t s) {
  const dim3 grid((unsigned)plan.S, (unsigned)d.slices());
  if (d.D == 128)
    score_kernel<128><<<grid, 128, 0, s>>>(q16, n_tokens, rank_row, k_codes, k_meta, d.N, d.bits, d.G, d.Hkv,
                                           sm_scale, plan.L, plan.S, logits, part_m, part_l);
  else
    score_kernel<64><<<grid, 128, 0, s>>>(q16, n_tokens, rank_row, k_codes, k_meta, d.N, d.bits, d.G, d.Hkv,
                                          sm_scale, plan.L, plan.S, logits, part_m, part_l);
  return hipGetLastError();
}

}  // namespace specache
