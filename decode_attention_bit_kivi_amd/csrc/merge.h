// Merge of the split-K partials of one query row: the splits' (running max m_s, sum l_s) in
// log2 units and their unnormalised outputs o_s combine into
//   out = sum_s 2^(m_s - M) o_s / sum_s 2^(m_s - M) l_s,   M = max_s m_s,
// the usual rescaling of partial softmax sums (the IO-aware exact-attention idea the SemKV page
// cites in §2.4).  One wave per row: lanes stride over the splits for M and the denominator, and
// each lane sums its D/64 channels over the splits in order.  The standalone merge kernel and the
// fused decode step's selection launch both call it, so their outputs agree bit for bit.
#pragma once

#include "common.h"

namespace specache {

constexpr float kMergeEmpty = -1.0e30f;  // the running max of a split that saw nothing

template <int D>
__device__ __forceinline__ void merge_row_wave(const float* __restrict__ part_ml, const float* __restrict__ part_acc,
                                               int S, _Float16* __restrict__ out, int64_t row) {
  constexpr int CPL = D / 64;  // channels per lane
  const int lane = threadIdx.x & 63;
  const float* ml = part_ml + row * S * 2;
  float M = kMergeEmpty;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, ml[2 * s]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float l = 0.0f;
  for (int s = lane; s < S; s += 64) l = fmaf(ml[2 * s + 1], __builtin_amdgcn_exp2f(ml[2 * s] - M), l);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) l += __shfl_xor(l, off);
  const float* acc = part_acc + row * S * D + CPL * lane;
  float o[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) o[c] = 0.0f;
  int s = 0;
  for (; s + 8 <= S; s += 8) {  // eight splits' loads in flight
    float v[8][CPL], m8[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      m8[u] = ml[2 * (s + u)];
#pragma unroll
      for (int c = 0; c < CPL; ++c) v[u][c] = acc[(int64_t)(s + u) * D + c];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float w = __builtin_amdgcn_exp2f(m8[u] - M);
#pragma unroll
      for (int c = 0; c < CPL; ++c) o[c] = fmaf(v[u][c], w, o[c]);
    }
  }
  for (; s < S; ++s) {
    const float w = __builtin_amdgcn_exp2f(ml[2 * s] - M);
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[c] = fmaf(acc[(int64_t)s * D + c], w, o[c]);
  }
#pragma unroll
  for (int c = 0; c < CPL; ++c) out[row * D + CPL * lane + c] = (_Float16)(o[c] / l);
}

}  // namespace specache
