// Pre-fetch(C_kappa): copy the selected 16-bit K/V rows into device buffers.
//
// SpeCache summary, §7 Algorithm 3 (Pre-fetch) and §2: transferring only the
// top-k rows instead of the whole offloaded cache is what makes the host copy
// affordable; the copy runs in the background, overlapped with the following
// layers' compute (quick read, second mechanism).
//
// The source is pinned host memory read directly by the kernel (zero copy
// over the host link) or device memory.  D*2/16 lanes per row, one 16-byte
// load per lane, consecutive lanes on consecutive bytes of a row; 256
// threads move 256*16 bytes of K and as much of V per round.
#include "common.h"

namespace specache {

namespace {

template <int D>
__global__ __launch_bounds__(256) void gather_kernel(const int32_t* __restrict__ idx, int k, int64_t N,
                                                     const uint4* __restrict__ k_src,
                                                     const uint4* __restrict__ v_src,
                                                     uint4* __restrict__ k_sel, uint4* __restrict__ v_sel,
                                                     int64_t total_rows) {
  constexpr int kLanesPerRow = D * 2 / 16;
  constexpr int kRowsPerBlock = 256 / kLanesPerRow;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  const int part = threadIdx.x % kLanesPerRow;
  if (row >= total_rows) return;
  const int64_t slice = row / k;
  const int32_t p = idx[row];
  uint4 kv, vv;
  if (p >= 0 && p < N) {
    const int64_t src = (slice * N + p) * kLanesPerRow + part;
    kv = k_src[src];
    vv = v_src[src];
  } else {
    const uint32_t nan2 = 0x7e007e00u;  // two float16 quiet NaNs
    kv = make_uint4(nan2, nan2, nan2, nan2);
    vv = kv;
  }
  k_sel[row * kLanesPerRow + part] = kv;
  v_sel[row * kLanesPerRow + part] = vv;
}

}  // namespace

hipError_t launch_gather(const Dims& d, const int32_t* idx, int k, const _Float16* k_src,
                         const _Float16* v_src, _Float16* k_sel, _Float16* v_sel, hipStream_t s) {
  const int64_t rows = d.slices() * k;
  if (rows == 0) return hipSuccess;
  const int lanes = d.D * 2 / 16;
  const int rows_per_block = 256 / lanes;
  const unsigned grid = (unsigned)ceil_div(rows, rows_per_block);
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
