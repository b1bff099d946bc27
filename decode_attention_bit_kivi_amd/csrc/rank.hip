// ArgTopK of the speculative row: merge the split statistics into each head's
// log-sum-exp, form the rank r(p) = log sum_g exp(s_g(p) - LSE_g) (the
// attention mass the G heads put on p), and select the k largest with a
// most-significant-digit radix select, ties to the lower position, emitted in
// ascending order.
//
// SpeCache summary, §7 Algorithms 2 and 3 (ArgTopK of the attention row), and
// §2 "attention sparsity" (a position is worth the attention mass it holds).
//
// One 1024-thread workgroup per slice.  Keys are kept in global memory (they
// fit in L2 for every supported N) and re-read by each of the four 8-bit
// digit passes; histograms live in LDS.
#include "common.h"

namespace specache {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

__device__ __forceinline__ uint32_t order_key(float r) {
  const uint32_t f = __float_as_uint(r);
  return (f & 0x80000000u) ? ~f : (f | 0x80000000u);
}

// Exclusive prefix sum over the workgroup; returns the exclusive value, writes the total.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scratch, uint32_t& total) {
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) scratch[wv] = x;
  __syncthreads();
  if (wv == 0) {
    uint32_t s = lane < kWaves ? scratch[lane] : 0u;
#pragma unroll
    for (int off = 1; off < kWaves; off <<= 1) {
      const uint32_t y = __shfl_up(s, off);
      if (lane >= off) s += y;
    }
    if (lane < kWaves) scratch[kWaves + lane] = s;  // inclusive wave prefix
  }
  __syncthreads();
  const uint32_t before = wv > 0 ? scratch[kWaves + wv - 1] : 0u;
  total = scratch[2 * kWaves - 1];
  __syncthreads();
  return before + x - v;
}

__global__ __launch_bounds__(kThreads) void rank_select_kernel(const float* __restrict__ logits,
                                                               const float* __restrict__ part_m,
                                                               const float* __restrict__ part_l, int G,
                                                               int S, int64_t N, int k,
                                                               float* __restrict__ keys,
                                                               int32_t* __restrict__ idx_out) {
  __shared__ float lse[kMaxRows];
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scan_scratch[2 * kWaves];
  __shared__ uint32_t sel_digit, sel_above;

  const int t = threadIdx.x;
  const int64_t slice = blockIdx.x;
  const float* lg = logits + slice * G * N;
  float* ky = keys + slice * N;

  if (t < G) {
    const float* pm = part_m + (slice * G + t) * S;
    const float* pl = part_l + (slice * G + t) * S;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, pm[s]);
    float Ls = 0.0f;
    for (int s = 0; s < S; ++s)
      if (pm[s] != -INFINITY) Ls += pl[s] * expf(pm[s] - M);
    lse[t] = M + logf(Ls);
  }
  if (t < 256) hist[t] = 0u;
  if (t == 0) {
    sel_digit = 0u;
    sel_above = 0u;
  }
  __syncthreads();

  // r(p) and the first digit histogram.
  for (int64_t p = t; p < N; p += kThreads) {
    float lp[kMaxRows];
    float mx = -INFINITY;
#pragma unroll
    for (int g = 0; g < kMaxRows; ++g) {
      if (g < G) {
        lp[g] = lg[(int64_t)g * N + p] - lse[g];
        mx = fmaxf(mx, lp[g]);
      }
    }
    float sum = 0.0f;
#pragma unroll
    for (int g = 0; g < kMaxRows; ++g)
      if (g < G) sum += expf(lp[g] - mx);
    const float r = mx + logf(sum);
    ky[p] = r;
    atomicAdd(&hist[order_key(r) >> 24], 1u);
  }
  __syncthreads();

  uint32_t prefix = 0u, mask = 0u, krem = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (pass > 0) {
      if (t < 256) hist[t] = 0u;
      __syncthreads();
      for (int64_t p = t; p < N; p += kThreads) {
        const uint32_t u = order_key(ky[p]);
        if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
      }
      __syncthreads();
    }
    // Counts from the top digit down: thread i < 256 looks at digit 255 - i.
    const uint32_t v = t < 256 ? hist[255 - t] : 0u;
    uint32_t tot;
    const uint32_t excl = block_exclusive_scan(v, scan_scratch, tot);
    const uint32_t incl = excl + v;
    if (t < 256 && incl >= krem && excl < krem) {
      sel_digit = 255u - (uint32_t)t;
      sel_above = excl;
    }
    __syncthreads();
    prefix |= sel_digit << shift;
    mask |= 255u << shift;
    krem -= sel_above;
    __syncthreads();
  }
  // prefix is the k-th largest key; take every key above it and the first krem equal to it.
  uint32_t out_base = 0u, eq_seen = 0u;
  for (int64_t p0 = 0; p0 < N; p0 += kThreads) {
    const int64_t p = p0 + t;
    const uint32_t u = p < N ? order_key(ky[p]) : 0u;
    const uint32_t gt = (p < N && u > prefix) ? 1u : 0u;
    const uint32_t eq = (p < N && u == prefix) ? 1u : 0u;
    uint32_t eq_tot, take_tot;
    const uint32_t eq_ex = block_exclusive_scan(eq, scan_scratch, eq_tot);
    const uint32_t take = gt | ((eq && eq_seen + eq_ex < krem) ? 1u : 0u);
    const uint32_t take_ex = block_exclusive_scan(take, scan_scratch, take_tot);
    if (take && out_base + take_ex < (uint32_t)k) idx_out[slice * k + out_base + take_ex] = (int32_t)p;
    out_base += take_tot;
    eq_seen += eq_tot;
  }
}

}  // namespace

hipError_t launch_rank_select(const Dims& d, const ScorePlan& plan, const float* logits,
                              const float* part_m, const float* part_l, int k, float* keys,
                              int32_t* idx_out, hipStream_t s) {
  rank_select_kernel<<<(unsigned)d.slices(), kThreads, 0, s>>>(logits, part_m, part_l, d.G, plan.S, d.N, k,
                                                               keys, idx_out);
  return hipGetLastError();
}

}  // namespace specache
