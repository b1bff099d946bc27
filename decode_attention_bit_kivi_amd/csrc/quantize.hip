// Quant(K), Quant(V): group min/max -> float16 zero-point and scale -> codes
// -> bit planes.
//
// Quantizer of the SpeCache summary, §3: KIVI's z = min, s = (max - min)/(2^B - 1)
// at two bits ("original KIVI quantization"), and at one bit the modified
// z = (3 min + max)/4, s = (max - min)/2 ("improved 1-bit quantization"), with
// round-half-up codes.  Keys are grouped per channel over 32 tokens and
// values per token over 32 channels (KIVI's grouping, SemKV page §2.1).
//
// Bit-exact by construction: min/max are exact, z and s are evaluated in
// float32 in the order the equations are written (no contraction in this
// file), the division is correctly rounded, and the rounding decision
// floor(q + 1/2) is taken as exact comparisons q >= j - 1/2.
//
// One workgroup per (slice, 32-token block); HBM-bound: 2 x 32 x D float16
// in, 2 x (b*D/8 + 4*D/32) x 32 bytes out.
#pragma clang fp contract(off)

#include "common.h"

namespace specache {

namespace {

// z16, s16 of a group, canonical +0.
__device__ __forceinline__ void zero_point_scale(float mn, float mx, int bits, _Float16& z16,
                                                 _Float16& s16) {
  float z, s;
  if (bits == 1) {
    const float t = 3.0f * mn;   // exact
    const float u = t + mx;
    z = u * 0.25f;
    const float d = mx - mn;
    s = d * 0.5f;
  } else {
    z = mn;
    const float d = mx - mn;
    s = __fdiv_rn(d, 3.0f);
  }
  z16 = (_Float16)z;
  s16 = (_Float16)s;
  if (z16 == (_Float16)0.0f) z16 = (_Float16)0.0f;
  if (s16 == (_Float16)0.0f) s16 = (_Float16)0.0f;
}

__device__ __forceinline__ int encode(float x, float zf, float sf, int bits) {
  if (sf == 0.0f) return 0;
  const float q = __fdiv_rn(x - zf, sf);
  int code = q >= 0.5f ? 1 : 0;
  if (bits == 2) code += (q >= 1.5f ? 1 : 0) + (q >= 2.5f ? 1 : 0);
  return code;
}

// Copy a [ROWS][D] float16 tile into LDS rows of stride D + 2 halves (the pad
// spreads a column over distinct banks).
template <int D, int NT, int ROWS = 32>
__device__ __forceinline__ void load_tile(const _Float16* __restrict__ src, _Float16 (*tile)[D + 2]) {
  constexpr int kChunks = ROWS * D / 8;  // 16-byte chunks
  for (int ci = threadIdx.x; ci < kChunks; ci += NT) {
    const uint4 v = reinterpret_cast<const uint4*>(src)[ci];
    const int row = ci / (D / 8);
    const int col = (ci % (D / 8)) * 8;
    uint32_t* dst = reinterpret_cast<uint32_t*>(&tile[row][col]);
    dst[0] = v.x;
    dst[1] = v.y;
    dst[2] = v.z;
    dst[3] = v.w;
  }
}

// Keys: thread t owns channel c = 32*(t/32) + e(t%32); a wave ballot over the
// channels of one token is then directly the packed word of that token.
// Grid: (key groups to write, slices).  Source group b is positions GK*b.. of a slice of src_len
// positions; it becomes the cache's key group grp0 + b (positions GK*(grp0 + b)..) of a slice of
// Ns positions.  GK = 32 or 64 tokens per key group.
template <int D, int GK>
__global__ __launch_bounds__(D) void quant_keys_kernel(const _Float16* __restrict__ k16, int64_t src_len,
                                                       uint32_t* __restrict__ codes,
                                                       _Float16* __restrict__ meta, int64_t Ns, int64_t grp0,
                                                       int bits) {
  constexpr int W = D / 32;
  __shared__ _Float16 tile[GK][D + 2];
  const int64_t grp = grp0 + blockIdx.x;
  const int64_t slice = blockIdx.y;
  const int64_t ngrp = Ns / GK;
  const int t = threadIdx.x;
  load_tile<D, D, GK>(k16 + (slice * src_len + (int64_t)blockIdx.x * GK) * D, tile);
  __syncthreads();

  const int c = 32 * (t >> 5) + bit_to_elem(t & 31);
  float mn = (float)tile[0][c], mx = mn;
#pragma unroll
  for (int p = 1; p < GK; ++p) {
    const float x = (float)tile[p][c];
    mn = fminf(mn, x);
    mx = fmaxf(mx, x);
  }
  _Float16 z16, s16;
  zero_point_scale(mn, mx, bits, z16, s16);
  _Float16* m = meta + (slice * ngrp + grp) * 2 * D;
  m[c] = z16;
  m[D + c] = s16;
  const float zf = (float)z16, sf = (float)s16;

  const int lane = t & 63;
  uint32_t keep[2][2] = {{0u, 0u}, {0u, 0u}};
  for (int p = 0; p < GK; ++p) {
    const int code = encode((float)tile[p][c], zf, sf, bits);
    for (int j = 0; j < bits; ++j) {
      const unsigned long long bal = __ballot((code >> j) & 1);
      if (lane == p) {
        keep[j][0] = (uint32_t)bal;
        keep[j][1] = (uint32_t)(bal >> 32);
      }
    }
  }
  if (lane < GK) {
    const int w0 = 2 * (t >> 6);  // the two words this wave's 64 channels form
    uint32_t* dst = codes + ((slice * Ns + grp * GK + lane) * bits) * W;
    for (int j = 0; j < bits; ++j) {
      dst[j * W + w0] = keep[j][0];
      dst[j * W + w0 + 1] = keep[j][1];
    }
  }
}

// Values: thread t owns (group w = t/32, token e(t%32)); a wave ballot over
// the tokens of one channel is then directly that channel's packed word.
// gshift = 1: value groups of 64 channels (two 32-channel halves, lanes t and t ^ 32).
template <int D>
__global__ __launch_bounds__(D) void quant_values_kernel(const _Float16* __restrict__ v16, int64_t src_len,
                                                         uint32_t* __restrict__ codes,
                                                         _Float16* __restrict__ meta, int64_t Ns, int64_t blk0,
                                                         int bits, int gshift) {
  constexpr int W = D / 32;
  __shared__ _Float16 tile[32][D + 2];
  const int64_t blk = blk0 + blockIdx.x;
  const int64_t slice = blockIdx.y;
  const int64_t nblk = Ns / 32;
  const int t = threadIdx.x;
  load_tile<D, D>(v16 + (slice * src_len + (int64_t)blockIdx.x * 32) * D, tile);
  __syncthreads();

  const int w = t >> 5;
  const int p = bit_to_elem(t & 31);
  float mn = (float)tile[p][32 * w], mx = mn;
#pragma unroll
  for (int cc = 1; cc < 32; ++cc) {
    const float x = (float)tile[p][32 * w + cc];
    mn = fminf(mn, x);
    mx = fmaxf(mx, x);
  }
  if (gshift) {  // the other 32 channels of the 64-channel group, same token
    mn = fminf(mn, __shfl_xor(mn, 32));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
  }
  _Float16 z16, s16;
  zero_point_scale(mn, mx, bits, z16, s16);
  const int Wg = W >> gshift, wg = w >> gshift;  // value groups per token; this thread's group
  _Float16* m = meta + (slice * nblk + blk) * 2 * Wg * 32;
  if ((w & gshift) == 0) {
    m[wg * 32 + p] = z16;
    m[Wg * 32 + wg * 32 + p] = s16;
  }
  const float zf = (float)z16, sf = (float)s16;

  const int lane = t & 63;
  uint32_t keep[2][2] = {{0u, 0u}, {0u, 0u}};
  for (int cc = 0; cc < 32; ++cc) {
    const int code = encode((float)tile[p][32 * w + cc], zf, sf, bits);
    for (int j = 0; j < bits; ++j) {
      const unsigned long long bal = __ballot((code >> j) & 1);
      if (lane == cc) {
        keep[j][0] = (uint32_t)bal;
        keep[j][1] = (uint32_t)(bal >> 32);
      }
    }
  }
  if (lane < 32) {
    const int w0 = 2 * (t >> 6);
    uint32_t* dst = codes + (slice * nblk + blk) * bits * D;
    for (int j = 0; j < bits; ++j) {
      dst[j * D + 32 * w0 + lane] = keep[j][0];
      dst[j * D + 32 * (w0 + 1) + lane] = keep[j][1];
    }
  }
}

}  // namespace

hipError_t launch_quantize(const Dims& d, const _Float16* k16, const _Float16* v16, int64_t src_len, int64_t blk0,
                           int64_t nblocks, uint32_t* k_codes, _Float16* k_meta, uint32_t* v_codes,
                           _Float16* v_meta, hipStream_t s) {
  if (nblocks == 0) return hipSuccess;
  const int gshift = d.group == 64 ? 1 : 0;
  const dim3 vgrid((unsigned)nblocks, (unsigned)d.slices());
  const dim3 kgrid((unsigned)(nblocks >> gshift), (unsigned)d.slices());  // blk0, nblocks: whole key groups
  const int64_t kgrp0 = blk0 >> gshift;
  if (d.D == 128) {
    if (gshift) quant_keys_kernel<128, 64><<<kgrid, 128, 0, s>>>(k16, src_len, k_codes, k_meta, d.Ns, kgrp0, d.bits);
    else quant_keys_kernel<128, 32><<<kgrid, 128, 0, s>>>(k16, src_len, k_codes, k_meta, d.Ns, kgrp0, d.bits);
    quant_values_kernel<128><<<vgrid, 128, 0, s>>>(v16, src_len, v_codes, v_meta, d.Ns, blk0, d.vbits, gshift);
  } else {
    if (gshift) quant_keys_kernel<64, 64><<<kgrid, 64, 0, s>>>(k16, src_len, k_codes, k_meta, d.Ns, kgrp0, d.bits);
    else quant_keys_kernel<64, 32><<<kgrid, 64, 0, s>>>(k16, src_len, k_codes, k_meta, d.Ns, kgrp0, d.bits);
    quant_values_kernel<64><<<vgrid, 64, 0, s>>>(v16, src_len, v_codes, v_meta, d.Ns, blk0, d.vbits, gshift);
  }
  return hipGetLastError();
}

}  // namespace specache
