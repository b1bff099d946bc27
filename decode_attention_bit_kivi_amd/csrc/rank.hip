// ArgTopK of the speculative row: merge the split statistics into each head's
// log-sum-exp, form the rank r(p) = log sum_g exp(s_g(p) - LSE_g) (the
// attention mass the G heads put on p), and select the k largest with a
// most-significant-digit radix select, ties to the lower position, emitted in
// ascending order.
//
// SpeCache summary, §7 Algorithms 2 and 3 (ArgTopK of the attention row), and
// §2 "attention sparsity" (a position is worth the attention mass it holds).
//
// Two kernels:
//   rank_keys    (grid: position chunks x slices) computes r(p) for every
//                position, writes it as an order-preserving 32-bit key, and
//                adds the histogram of the keys' top 11 bits into a per-slice
//                global histogram (zeroed by the score kernel of the same call);
//   rank_select  (one 1024-thread workgroup per slice) picks the digit that
//                holds the k-th largest key, refines it with two more digit
//                passes (11 and 10 bits), and compacts the selected positions
//                in ascending order.  Both passes and the compaction read the
//                keys (L2-resident) as 32 consecutive keys per thread.
#include "common.h"

namespace specache {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kRun = 32;                       // consecutive keys per thread in rank_select
constexpr int kTile = kSelThreads * kRun;      // positions per rank_select sweep
constexpr int kKeyThreads = 256;
constexpr int kKeyChunk = kKeyThreads * 16;    // positions per rank_keys workgroup
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ uint32_t order_key(float r) {
  const uint32_t f = __float_as_uint(r);
  return (f & 0x80000000u) ? ~f : (f | 0x80000000u);
}

// Exclusive prefix sum over the 1024-thread workgroup; returns the exclusive value, writes the total.
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
    uint32_t s = lane < kSelWaves ? scratch[lane] : 0u;
#pragma unroll
    for (int off = 1; off < kSelWaves; off <<= 1) {
      const uint32_t y = __shfl_up(s, off);
      if (lane >= off) s += y;
    }
    if (lane < kSelWaves) scratch[kSelWaves + lane] = s;  // inclusive wave prefix
  }
  __syncthreads();
  const uint32_t before = wv > 0 ? scratch[kSelWaves + wv - 1] : 0u;
  total = scratch[2 * kSelWaves - 1];
  __syncthreads();
  return before + x - v;
}

// ---------------------------------------------------------------- rank_keys

__global__ __launch_bounds__(kKeyThreads) void rank_keys_kernel(const float* __restrict__ logits,
                                                                const float* __restrict__ part_m,
                                                                const float* __restrict__ part_l, int G, int S,
                                                                int64_t N, float* __restrict__ rkey,
                                                                uint32_t* __restrict__ ghist) {
  __shared__ float lse2[kMaxRows];  // log2-sum-exp2 of each head, in log2 units
  __shared__ uint32_t hist[2048];
  const int t = threadIdx.x;
  const int64_t slice = blockIdx.y;
  const int64_t c0 = (int64_t)blockIdx.x * kKeyChunk;
  if (t < G) {  // split statistics are (max, sum 2^(x - max)) in log2 units
    const float* pm = part_m + (slice * G + t) * S;
    const float* pl = part_l + (slice * G + t) * S;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, pm[s]);
    float Ls = 0.0f;
    for (int s = 0; s < S; ++s)
      if (pm[s] != -INFINITY) Ls += pl[s] * exp2f(pm[s] - M);
    lse2[t] = M + log2f(Ls);
  }
  for (int i = t; i < 2048; i += kKeyThreads) hist[i] = 0u;
  __syncthreads();

  // each thread: 4 runs of 4 consecutive positions (float4 per head)
  const float* lg = logits + slice * G * N;
#pragma unroll
  for (int rr = 0; rr < 4; ++rr) {
    const int64_t p = c0 + 4 * (t + rr * kKeyThreads);
    if (p >= N) break;
    float4 x[kMaxRows];
#pragma unroll
    for (int g = 0; g < kMaxRows; ++g)
      if (g < G) x[g] = *reinterpret_cast<const float4*>(lg + (int64_t)g * N + p);
    float r[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float lp[kMaxRows];
      float mx = -INFINITY;
#pragma unroll
      for (int g = 0; g < kMaxRows; ++g)
        if (g < G) {
          const float v = e == 0 ? x[g].x : (e == 1 ? x[g].y : (e == 2 ? x[g].z : x[g].w));
          lp[g] = fmaf(v, kLog2e, -lse2[g]);  // log2 of the head's probability
          mx = fmaxf(mx, lp[g]);
        }
      float sum = 0.0f;
#pragma unroll
      for (int g = 0; g < kMaxRows; ++g)
        if (g < G) sum += __builtin_amdgcn_exp2f(lp[g] - mx);
      r[e] = (mx + __builtin_amdgcn_logf(sum)) * kLn2;  // v_log_f32 is log2
    }
    *reinterpret_cast<float4*>(rkey + slice * N + p) = make_float4(r[0], r[1], r[2], r[3]);
#pragma unroll
    for (int e = 0; e < 4; ++e) atomicAdd(&hist[order_key(r[e]) >> 21], 1u);
  }
  __syncthreads();
  uint32_t* gh = ghist + slice * 2048;
  for (int i = t; i < 2048; i += kKeyThreads)
    if (hist[i]) atomicAdd(&gh[i], hist[i]);
}

// ---------------------------------------------------------------- rank_select

// 32 keys of one thread's run, as order-preserving integers (positions >= N read as 0).
__device__ __forceinline__ void load_run(const float* ky, int64_t N, int64_t p, uint32_t (&u)[kRun]) {
  if (p + kRun <= N) {
#pragma unroll
    for (int v = 0; v < kRun / 4; ++v) {
      const float4 f = *reinterpret_cast<const float4*>(ky + p + 4 * v);
      u[4 * v] = order_key(f.x);
      u[4 * v + 1] = order_key(f.y);
      u[4 * v + 2] = order_key(f.z);
      u[4 * v + 3] = order_key(f.w);
    }
  } else {
#pragma unroll
    for (int e = 0; e < kRun; ++e) u[e] = p + e < N ? order_key(ky[p + e]) : 0u;
  }
}

__global__ __launch_bounds__(kSelThreads) void rank_select_kernel(const float* __restrict__ rkey,
                                                                  const uint32_t* __restrict__ ghist, int64_t N,
                                                                  int k, int32_t* __restrict__ idx_out) {
  __shared__ uint32_t hist[2048];
  __shared__ uint32_t scan_scratch[2 * kSelWaves];
  __shared__ uint32_t sel_digit, sel_above;

  const int t = threadIdx.x;
  const int64_t slice = blockIdx.x;
  const float* ky = rkey + slice * N;
  const uint32_t* gh = ghist + slice * 2048;
  for (int i = t; i < 2048; i += kSelThreads) hist[i] = gh[i];
  if (t == 0) {
    sel_digit = 0u;
    sel_above = 0u;
  }
  __syncthreads();

  // digits: bits 31..21 (11, histogram from rank_keys), 20..10 (11), 9..0 (10)
  uint32_t prefix = 0u, mask = 0u, krem = (uint32_t)k;
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nbins = pass == 2 ? 1024 : 2048;
    if (pass > 0) {
      for (int i = t; i < 2048; i += kSelThreads) hist[i] = 0u;
      __syncthreads();
      for (int64_t p0 = 0; p0 < N; p0 += kTile) {
        const int64_t p = p0 + (int64_t)t * kRun;
        if (p < N) {
          uint32_t u[kRun];
          load_run(ky, N, p, u);
#pragma unroll
          for (int e = 0; e < kRun; ++e)
            if (p + e < N && (u[e] & mask) == prefix) atomicAdd(&hist[(u[e] >> shift) & (uint32_t)(nbins - 1)], 1u);
        }
      }
      __syncthreads();
    }
    // counts from the top digit down: thread t covers digits nbins-1-2t and nbins-2-2t
    const int dhi = nbins - 1 - 2 * t, dlo = dhi - 1;
    const uint32_t hhi = dhi >= 0 ? hist[dhi] : 0u;
    const uint32_t hlo = dlo >= 0 ? hist[dlo] : 0u;
    uint32_t tot;
    const uint32_t excl = block_exclusive_scan(hhi + hlo, scan_scratch, tot);
    if (dhi >= 0 && excl < krem && excl + hhi >= krem) {
      sel_digit = (uint32_t)dhi;
      sel_above = excl;
    } else if (dlo >= 0 && excl + hhi < krem && excl + hhi + hlo >= krem) {
      sel_digit = (uint32_t)dlo;
      sel_above = excl + hhi;
    }
    __syncthreads();
    prefix |= sel_digit << shift;
    mask |= (uint32_t)(nbins - 1) << shift;
    krem -= sel_above;
    __syncthreads();
  }

  // prefix is the k-th largest key: take every key above it and the first krem equal to it
  uint32_t out_base = 0u, eq_seen = 0u;
  for (int64_t p0 = 0; p0 < N; p0 += kTile) {
    const int64_t p = p0 + (int64_t)t * kRun;
    uint32_t u[kRun];
    uint32_t ngt = 0u, neq = 0u;
    if (p < N) {
      load_run(ky, N, p, u);
#pragma unroll
      for (int e = 0; e < kRun; ++e) {
        const bool in = p + e < N;
        ngt += (in && u[e] > prefix) ? 1u : 0u;
        neq += (in && u[e] == prefix) ? 1u : 0u;
      }
    }
    uint32_t eq_tot, take_tot;
    const uint32_t eq_before = eq_seen + block_exclusive_scan(neq, scan_scratch, eq_tot);
    const uint32_t eq_take = eq_before >= krem ? 0u : (krem - eq_before < neq ? krem - eq_before : neq);
    uint32_t out = out_base + block_exclusive_scan(ngt + eq_take, scan_scratch, take_tot);
    if (p < N) {
      uint32_t eq_left = eq_take;
#pragma unroll
      for (int e = 0; e < kRun; ++e) {
        const bool in = p + e < N;
        bool take = in && u[e] > prefix;
        if (in && u[e] == prefix && eq_left > 0u) {
          take = true;
          --eq_left;
        }
        if (take && out < (uint32_t)k) idx_out[slice * k + out++] = (int32_t)(p + e);
      }
    }
    out_base += take_tot;
    eq_seen += eq_tot;
  }
}

}  // namespace

hipError_t launch_rank_select(const Dims& d, int S, const float* logits, const float* part_m,
                              const float* part_l, int k, float* keys, uint32_t* hist, int32_t* idx_out,
                              hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(d.N, kKeyChunk), (unsigned)d.slices());
  rank_keys_kernel<<<grid, kKeyThreads, 0, s>>>(logits, part_m, part_l, d.G, S, d.N, keys, hist);
  rank_select_kernel<<<(unsigned)d.slices(), kSelThreads, 0, s>>>(keys, hist, d.N, k, idx_out);
  return hipGetLastError();
}

}  // namespace specache
