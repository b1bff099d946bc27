// Pre-fetch(C_kappa): copy the selected 16-bit K/V rows into device buffers.
//
// SpeCache summary, §7 Algorithm 3 (Pre-fetch) and §2: transferring only the
// top-k rows instead of the whole offloaded cache is what makes the host copy
// affordable; the copy runs in the background, overlapped with the following
// layers' compute (quick read, second mechanism).
//
// Resident-set reuse (§3 "prefetch and offload during decoding": the used rows
// outside the new top-k are evicted, so rows in both sets stay): reuse_kernel
// copies the rows the previous selection already holds on the device and marks
// the others, and gather_missing_kernel fetches only the marked rows.
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

// An index outside [0, N) gives a NaN row.
template <int D>
__global__ __launch_bounds__(256) void gather_kernel(const int32_t* __restrict__ idx, int k, int64_t N, int64_t Ns,
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
          const int64_t src = (slice * Ns + p) * kLanesPerRow + part;
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

// Resident-set reuse: row i of the new selection whose position is also in the previous
// selection (at row j) is copied from the previous rows (device to device); the others are
// marked for fetching: fetch_idx[i] = position, or -1 for a copied row.  A position outside
// [0, N) is marked with N, so that the fetch writes a NaN row for it.  Grid: (chunks of 256 /
// (D/8) rows, slices); one lane group per row, so each lane's work is one chain: index load,
// search of the previous selection (staged in LDS when it has at most kPrevLds entries), copy.
constexpr int kPrevLds = 4096;

template <int D>
__global__ __launch_bounds__(256) void reuse_kernel(const int32_t* __restrict__ idx, int k,
                                                    const int32_t* __restrict__ idx_prev, int k_prev, int64_t N,
                                                    const uint4* __restrict__ k_prev_rows,
                                                    const uint4* __restrict__ v_prev_rows, uint4* __restrict__ k_sel,
                                                    uint4* __restrict__ v_sel, int32_t* __restrict__ fetch_idx) {
  constexpr int kLanesPerRow = D * 2 / 16;
  constexpr int kRowsPerBlock = 256 / kLanesPerRow;
  __shared__ int32_t prev[kPrevLds];
  const int tid = threadIdx.x;
  const int64_t slice = blockIdx.y;
  const int i = blockIdx.x * kRowsPerBlock + tid / kLanesPerRow;  // this lane group's entry
  const int part = tid % kLanesPerRow;
  const int32_t p = i < k ? idx[slice * k + i] : 0;  // in flight while the previous selection is staged
  const int32_t* ip = idx_prev + slice * k_prev;
  const bool in_lds = k_prev <= kPrevLds;
  if (in_lds)
    for (int j = tid; j < k_prev; j += 256) prev[j] = ip[j];
  __syncthreads();
  if (i >= k) return;
  int lo = 0, hi = k_prev;  // first entry of the previous selection >= p
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    const int32_t v = in_lds ? prev[mid] : ip[mid];
    if (v < p) lo = mid + 1; else hi = mid;
  }
  const bool valid = p >= 0 && p < N;
  const bool found = valid && lo < k_prev && (in_lds ? prev[lo] : ip[lo]) == p;
  if (found) {
    const int64_t src = (slice * k_prev + lo) * kLanesPerRow + part;
    const int64_t dst = (slice * k + i) * kLanesPerRow + part;
    const uint4 kr = k_prev_rows[src], vr = v_prev_rows[src];
    k_sel[dst] = kr;
    v_sel[dst] = vr;
  }
  if (part == 0) fetch_idx[slice * k + i] = found ? -1 : (valid ? p : (int32_t)N);
}

// The fetch of the rows a reuse pass left (index >= 0; negative = resident, untouched): each
// wave takes 64 consecutive rows, ballots the ones to fetch, and copies them kRowsPerWave at
// a time (one per 16-lane group for D = 128), so its lanes stay busy however sparse they are.
template <int D>
__global__ __launch_bounds__(256) void gather_missing_kernel(const int32_t* __restrict__ idx, int k, int64_t N,
                                                             int64_t Ns,
                                                             const uint4* __restrict__ k_src,
                                                             const uint4* __restrict__ v_src,
                                                             uint4* __restrict__ k_sel, uint4* __restrict__ v_sel,
                                                             int64_t total_rows) {
  constexpr int kLanesPerRow = D * 2 / 16;
  constexpr int kRowsPerWave = 64 / kLanesPerRow;
  const int lane = threadIdx.x & 63;
  const int grp = lane / kLanesPerRow, part = lane % kLanesPerRow;
  const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  const uint32_t nan2 = 0x7e007e00u;
  for (int64_t c0 = wave * 64; c0 < total_rows; c0 += nwaves * 64) {
    const int64_t mine = c0 + lane;
    const int32_t pm = mine < total_rows ? idx[mine] : -1;
    uint64_t todo = __ballot(pm >= 0);
    while (todo) {
      // the kRowsPerWave lowest rows still to fetch; group grp takes the grp-th of them
      int pick = -1;
      uint64_t t = todo;
#pragma unroll
      for (int g = 0; g < kRowsPerWave; ++g) {
        const int b = t ? __builtin_ctzll(t) : -1;
        if (g == grp) pick = b;
        if (t) t &= t - 1;
      }
      todo = t;
      const int32_t p = __shfl(pm, pick < 0 ? 0 : pick);
      if (pick >= 0) {
        const int64_t row = c0 + pick;
        const int64_t slice = row / k;
        uint4 kv = make_uint4(nan2, nan2, nan2, nan2), vv = kv;
        if (p < N) {
          const int64_t src = (slice * Ns + p) * kLanesPerRow + part;
          kv = k_src[src];
          vv = v_src[src];
        }
        k_sel[row * kLanesPerRow + part] = kv;
        v_sel[row * kLanesPerRow + part] = vv;
      }
    }
  }
}

template <int D, bool SKIP_NEG>
void launch_gather_t(const Dims& d, const int32_t* idx, int k, const _Float16* k_src, const _Float16* v_src,
                     _Float16* k_sel, _Float16* v_sel, hipStream_t s) {
  const int64_t rows = d.slices() * k;
  if (SKIP_NEG) {
    const int64_t need = ceil_div(rows, 256);  // 64 rows per wave, 4 waves per workgroup
    const unsigned grid = (unsigned)(need < kGatherBlocks ? need : kGatherBlocks);
    gather_missing_kernel<D><<<grid, 256, 0, s>>>(idx, k, d.N, d.Ns, reinterpret_cast<const uint4*>(k_src),
                                                  reinterpret_cast<const uint4*>(v_src),
                                                  reinterpret_cast<uint4*>(k_sel), reinterpret_cast<uint4*>(v_sel),
                                                  rows);
    return;
  }
  const int rows_per_pass = 256 / (D * 2 / 16);
  const int64_t need = ceil_div(rows, rows_per_pass);
  const unsigned grid = (unsigned)(need < kGatherBlocks ? need : kGatherBlocks);
  gather_kernel<D><<<grid, 256, 0, s>>>(idx, k, d.N, d.Ns, reinterpret_cast<const uint4*>(k_src),
                                         reinterpret_cast<const uint4*>(v_src), reinterpret_cast<uint4*>(k_sel),
                                         reinterpret_cast<uint4*>(v_sel), rows);
}

}  // namespace

hipError_t launch_gather(const Dims& d, const int32_t* idx, int k, const _Float16* k_src,
                         const _Float16* v_src, _Float16* k_sel, _Float16* v_sel, bool skip_negative,
                         hipStream_t s) {
  if (d.slices() * k == 0) return hipSuccess;
  if (d.D == 128) {
    if (skip_negative) launch_gather_t<128, true>(d, idx, k, k_src, v_src, k_sel, v_sel, s);
    else launch_gather_t<128, false>(d, idx, k, k_src, v_src, k_sel, v_sel, s);
  } else {
    if (skip_negative) launch_gather_t<64, true>(d, idx, k, k_src, v_src, k_sel, v_sel, s);
    else launch_gather_t<64, false>(d, idx, k, k_src, v_src, k_sel, v_sel, s);
  }
  return hipGetLastError();
}

hipError_t launch_reuse(const Dims& d, const int32_t* idx, int k, const int32_t* idx_prev, int k_prev,
                        const _Float16* k_prev_rows, const _Float16* v_prev_rows, _Float16* k_sel, _Float16* v_sel,
                        int32_t* fetch_idx, hipStream_t s) {
  if (d.slices() * k == 0) return hipSuccess;
  const dim3 grid((unsigned)ceil_div(k, 256 / (d.D * 2 / 16)), (unsigned)d.slices());
  auto u4 = [](const _Float16* p) { return reinterpret_cast<const uint4*>(p); };
  auto w4 = [](_Float16* p) { return reinterpret_cast<uint4*>(p); };
  if (d.D == 128)
    reuse_kernel<128><<<grid, 256, 0, s>>>(idx, k, idx_prev, k_prev, d.N, u4(k_prev_rows), u4(v_prev_rows), w4(k_sel),
                                           w4(v_sel), fetch_idx);
  else
    reuse_kernel<64><<<grid, 256, 0, s>>>(idx, k, idx_prev, k_prev, d.N, u4(k_prev_rows), u4(v_prev_rows), w4(k_sel),
                                          w4(v_sel), fetch_idx);
  return hipGetLastError();
}

}  // namespace specache
