// Pre-fetch(C_kappa): copy the selected 16-bit K/V rows into device buffers.
//
// SpeCache summary, §7 Algorithm 3 (Pre-fetch) and §2: transferring only the
// top-k rows instead of the whole offloaded cache is what makes the host copy
// affordable; the copy runs in the background, overlapped with the following
// layers' compute (quick read, second mechanism).
//
// The source is pinned host memory read directly by the kernel (zero copy
// over the host link) or device memory.  The copy is bound by the host link,
// not by the GPU, so the kernel runs on a small fixed grid (kGatherBlocks
// workgroups) that leaves almost every CU to the compute stream it overlaps
// with; each thread keeps kUnroll 16-byte host reads in flight to cover the
// link's latency.  D*2/16 lanes cover one row, consecutive lanes on
// consecutive bytes.
#include "common.h"

namespace specache {

namespace {

#ifndef SPECACHE_GATHER_BLOCKS
#define SPECACHE_GATHER_BLOCKS 32
#endif
#ifndef SPECACHE_GATHER_UNROLL
#define SPECACHE_GATHER_UNROLL 1
#endif
constexpr int kGatherBlocks = SPECACHE_GATHER_BLOCKS;
constexpr int kUnroll = SPECACHE_GATHER_UNROLL;

template <int D>
__global__ __launch_bounds__(256) void gather_kernel(const int32_t* __restrict__ idx, int k, int64_t N,
                                                     const uint4* __restrict__ k_src,
                                                     const uint4* __restrict__ v_src,
                                                     uint4* __restrict__ k_sel, uint4* __restrict__ v_sel,
                                                     int64_t total_rows) {
  constexpr int kLanesPerRow = D * 2 / 16;
  constexpr int kRowsPerPass = 256 / kLanesPerRow;
  const int part = threadIdx.x % kLanesPerRow;
  const int64_t stride = (int64_t)gridDim.x * kRowsPerPass;
  const uint32_t nan2 = 0x7e007e00u;  // two float16 quiet NaNs
  for (int64_t base = (int64_t)blockIdx.x * kRowsPerPass + threadIdx.x / kLanesPerRow; base < total_rows;
       base += stride * kUnroll) {
    uint4 kv[kUnroll], vv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t row = base + u * stride;
      kv[u] = make_uint4(nan2, nan2, nan2, nan2);
      vv[u] = kv[u];
      if (row < total_rows) {
        const int64_t slice = row / k;
        const int32_t p = idx[row];
        if (p >= 0 && p < N) {
          const int64_t src = (slice * N + p) * kLanesPerRow + part;
#ifdef SPECACHE_GATHER_NT
          typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
          const u32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(k_src + src));
          const u32x4_t c = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(v_src + src));
          kv[u] = make_uint4(a.x, a.y, a.z, a.w);
          vv[u] = make_uint4(c.x, c.y, c.z, c.w);
#else
          kv[u] = k_src[src];
          vv[u] = v_src[src];
#endif
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t row = base + u * stride;
      if (row < total_rows) {
        k_sel[row * kLanesPerRow + part] = kv[u];
        v_sel[row * kLanesPerRow + part] = vv[u];
      }
    }
  }
}

}  // namespace

hipError_t launch_gather(const Dims& d, const int32_t* idx, int k, const _Float16* k_src,
                         const _Float16* v_src, _Float16* k_sel, _Float16* v_sel, hipStream_t s) {
  const int64_t rows = d.slices() * k;
  if (rows == 0) return hipSuccess;
  const int rows_per_pass = 256 / (d.D * 2 / 16);
  const int64_t need = ceil_div(rows, rows_per_pass);
  const unsigned grid = (unsigned)(need < kGatherBlocks ? need : kGatherBlocks);
  if (d.D == 128)
    gather_kernel<128><<<grid, 256, 0, s>>>(idx, k, d.N, reinterpret_cast<const uint4*>(k_src),
                                            reinterpret_cast<const uint4*>(v_src), reinterpret_cast<uint4*>(k_sel),
                                            reinterpret_cast<uint4*>(v_sel), rows);
  else
    gather_kernel<64><<<grid, 256, 0, s>>>(idx, k, d.N, reinterpret_cast<const uint4*>(k_src),
                                           reinterpret_cast<const uint4*>(v_src), reinterpret_cast<uint4*>(k_sel),
                                           reinterpret_cast<uint4*>(v_sel), rows);
  return hipGetLastError();
}

}  // namespace specache
