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
// file), and the rounding decision floor(q + 1/2) on the correctly rounded
// quotient q is taken by exact comparisons that need no division (encode).
//
// One workgroup per (slice, 32-token block); HBM-bound: 2 x 32 x D float16
// in, 2 x (b*D/8 + 4*D/32) x 32 bytes out.
#pragma clang fp contract(off)

#include "common.h"

#include <type_traits>
#include <utility>

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

// code = clamp(floor(q + 1/2)) with q = RN(RN(x - z) / s), decided without the division.  RN(y)
// >= t for t = 1/2, 3/2, 5/2 exactly when y >= t - h, h half the gap below t (2^-26, 2^-24, 2^-23;
// the tie rounds to t, whose last mantissa bit is even), i.e. when d - t s >= -h s for d = RN(x - z)
// and s > 0.  t s and h s are exact, and RN(d - t s) (one fused multiply-add) keeps the comparison:
// near the threshold d is within a factor two of t s, so the difference is exact (Sterbenz), and
// away from it the difference is far larger than h s.  A zero scale gives code 0 (its thresholds are
// +inf); a non-finite one (never for finite float16 input) takes the correctly rounded division.
struct Coder {
  float zf, sf, h0, h1, h2;
  bool slow;
  __device__ __forceinline__ Coder(float z, float s) : zf(z), sf(s) {
    slow = !(s <= 65504.0f);
    h0 = s == 0.0f ? INFINITY : -s * 0x1p-26f;
    h1 = s == 0.0f ? INFINITY : -s * 0x1p-24f;
    h2 = s == 0.0f ? INFINITY : -s * 0x1p-23f;
  }
  // the code of x; MAYBE_SLOW = false when no lane of the wave has a non-finite scale
  template <int BITS, bool MAYBE_SLOW>
  __device__ __forceinline__ int code(float x) const {
    const float d = x - zf;
    if (MAYBE_SLOW && slow) {
      if (sf == 0.0f) return 0;
      const float q = __fdiv_rn(d, sf);
      return BITS == 1 ? (q >= 0.5f ? 1 : 0) : (q >= 0.5f ? 1 : 0) + (q >= 1.5f ? 1 : 0) + (q >= 2.5f ? 1 : 0);
    }
    if constexpr (BITS == 1) return fmaf(-0.5f, sf, d) >= h0 ? 1 : 0;
    return (fmaf(-0.5f, sf, d) >= h0 ? 1 : 0) + (fmaf(-1.5f, sf, d) >= h1 ? 1 : 0) +
           (fmaf(-2.5f, sf, d) >= h2 ? 1 : 0);
  }
};

// f(std::integral_constant<int, i>) for i = 0 .. N-1, unrolled at compile time.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
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
template <int D, int GK, int BITS>
__global__ __launch_bounds__(D) void quant_keys_kernel(const _Float16* __restrict__ k16, int64_t src_len,
                                                       uint32_t* __restrict__ codes,
                                                       _Float16* __restrict__ meta, int64_t Ns, int64_t grp0) {
  constexpr int W = D / 32;
  __shared__ _Float16 tile[GK][D + 2];
  const int64_t grp = grp0 + blockIdx.x;
  const int64_t slice = blockIdx.y;
  const int64_t ngrp = Ns / GK;
  const int t = threadIdx.x;
  load_tile<D, D, GK>(k16 + (slice * src_len + (int64_t)blockIdx.x * GK) * D, tile);
  __syncthreads();

  // the thread's channel over the group's tokens, read once for min/max and codes
  const int c = 32 * (t >> 5) + bit_to_elem(t & 31);
  float x[GK];
#pragma unroll
  for (int p = 0; p < GK; ++p) x[p] = (float)tile[p][c];
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int p = 1; p < GK; ++p) {
    mn = fminf(mn, x[p]);
    mx = fmaxf(mx, x[p]);
  }
  _Float16 z16, s16;
  zero_point_scale(mn, mx, BITS, z16, s16);
  _Float16* m = meta + (slice * ngrp + grp) * 2 * D;
  m[c] = z16;
  m[D + c] = s16;
  const Coder cd((float)z16, (float)s16);

  // token p's word: the wave's ballot over its channels, kept by lane p
  const int lane = t & 63;
  uint32_t keep[BITS][2];
#pragma unroll
  for (int j = 0; j < BITS; ++j) keep[j][0] = keep[j][1] = 0u;
  auto encode_all = [&](auto maybe_slow) {
    static_for<GK>([&](auto ic) {
      constexpr int p = decltype(ic)::value;
      const int code = cd.code<BITS, decltype(maybe_slow)::value>(x[p]);
#pragma unroll
      for (int j = 0; j < BITS; ++j) {
        const unsigned long long bal = __ballot((code >> j) & 1);
        keep[j][0] = lane == p ? (uint32_t)bal : keep[j][0];
        keep[j][1] = lane == p ? (uint32_t)(bal >> 32) : keep[j][1];
      }
    });
  };
  if (__any(cd.slow)) encode_all(std::true_type{});
  else encode_all(std::false_type{});
  if (lane < GK) {
    const int w0 = 2 * (t >> 6);  // the two words this wave's 64 channels form
    uint32_t* dst = codes + ((slice * Ns + grp * GK + lane) * BITS) * W;
#pragma unroll
    for (int j = 0; j < BITS; ++j) {
      dst[j * W + w0] = keep[j][0];
      dst[j * W + w0 + 1] = keep[j][1];
    }
  }
}

// Values: thread t owns (group w = t/32, token e(t%32)); a wave ballot over
// the tokens of one channel is then directly that channel's packed word.
// gshift = 1: value groups of 64 channels (two 32-channel halves, lanes t and t ^ 32).
template <int D, int BITS>
__global__ __launch_bounds__(D) void quant_values_kernel(const _Float16* __restrict__ v16, int64_t src_len,
                                                         uint32_t* __restrict__ codes,
                                                         _Float16* __restrict__ meta, int64_t Ns, int64_t blk0,
                                                         int gshift) {
  constexpr int W = D / 32;
  __shared__ _Float16 tile[32][D + 2];
  const int64_t blk = blk0 + blockIdx.x;
  const int64_t slice = blockIdx.y;
  const int64_t nblk = Ns / 32;
  const int t = threadIdx.x;
  load_tile<D, D>(v16 + (slice * src_len + (int64_t)blockIdx.x * 32) * D, tile);
  __syncthreads();

  // the thread's 32 channels of its token, read once (two per 32-bit LDS read)
  const int w = t >> 5;
  const int p = bit_to_elem(t & 31);
  float x[32];
#pragma unroll
  for (int cc = 0; cc < 32; cc += 2) {
    const uint32_t two = *reinterpret_cast<const uint32_t*>(&tile[p][32 * w + cc]);
    x[cc] = (float)__builtin_bit_cast(_Float16, (uint16_t)(two & 0xffffu));
    x[cc + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(two >> 16));
  }
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int cc = 1; cc < 32; ++cc) {
    mn = fminf(mn, x[cc]);
    mx = fmaxf(mx, x[cc]);
  }
  if (gshift) {  // the other 32 channels of the 64-channel group, same token
    mn = fminf(mn, __shfl_xor(mn, 32));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
  }
  _Float16 z16, s16;
  zero_point_scale(mn, mx, BITS, z16, s16);
  const int Wg = W >> gshift, wg = w >> gshift;  // value groups per token; this thread's group
  _Float16* m = meta + (slice * nblk + blk) * 2 * Wg * 32;
  if ((w & gshift) == 0) {
    m[wg * 32 + p] = z16;
    m[Wg * 32 + wg * 32 + p] = s16;
  }
  const Coder cd((float)z16, (float)s16);

  // channel cc's word: the wave's ballot over its tokens, kept by lane cc
  const int lane = t & 63;
  uint32_t keep[BITS][2];
#pragma unroll
  for (int j = 0; j < BITS; ++j) keep[j][0] = keep[j][1] = 0u;
  auto encode_all = [&](auto maybe_slow) {
    static_for<32>([&](auto ic) {
      constexpr int cc = decltype(ic)::value;
      const int code = cd.code<BITS, decltype(maybe_slow)::value>(x[cc]);
#pragma unroll
      for (int j = 0; j < BITS; ++j) {
        const unsigned long long bal = __ballot((code >> j) & 1);
        keep[j][0] = lane == cc ? (uint32_t)bal : keep[j][0];
        keep[j][1] = lane == cc ? (uint32_t)(bal >> 32) : keep[j][1];
      }
    });
  };
  if (__any(cd.slow)) encode_all(std::true_type{});
  else encode_all(std::false_type{});
  if (lane < 32) {
    const int w0 = 2 * (t >> 6);
    uint32_t* dst = codes + (slice * nblk + blk) * BITS * D;
#pragma unroll
    for (int j = 0; j < BITS; ++j) {
      dst[j * D + 32 * w0 + lane] = keep[j][0];
      dst[j * D + 32 * (w0 + 1) + lane] = keep[j][1];
    }
  }
}

template <int D>
void launch_quant_d(const Dims& d, const _Float16* k16, const _Float16* v16, int64_t src_len, int64_t blk0,
                    int64_t kgrp0, dim3 kgrid, dim3 vgrid, int gshift, uint32_t* k_codes, _Float16* k_meta,
                    uint32_t* v_codes, _Float16* v_meta, hipStream_t s) {
  if (d.bits == 1) {
    if (gshift) quant_keys_kernel<D, 64, 1><<<kgrid, D, 0, s>>>(k16, src_len, k_codes, k_meta, d.Ns, kgrp0);
    else quant_keys_kernel<D, 32, 1><<<kgrid, D, 0, s>>>(k16, src_len, k_codes, k_meta, d.Ns, kgrp0);
  } else {
    if (gshift) quant_keys_kernel<D, 64, 2><<<kgrid, D, 0, s>>>(k16, src_len, k_codes, k_meta, d.Ns, kgrp0);
    else quant_keys_kernel<D, 32, 2><<<kgrid, D, 0, s>>>(k16, src_len, k_codes, k_meta, d.Ns, kgrp0);
  }
  if (d.vbits == 1) quant_values_kernel<D, 1><<<vgrid, D, 0, s>>>(v16, src_len, v_codes, v_meta, d.Ns, blk0, gshift);
  else quant_values_kernel<D, 2><<<vgrid, D, 0, s>>>(v16, src_len, v_codes, v_meta, d.Ns, blk0, gshift);
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
  if (d.D == 128) launch_quant_d<128>(d, k16, v16, src_len, blk0, kgrp0, kgrid, vgrid, gshift, k_codes, k_meta,
                                      v_codes, v_meta, s);
  else launch_quant_d<64>(d, k16, v16, src_len, blk0, kgrp0, kgrid, vgrid, gshift, k_codes, k_meta, v_codes,
                          v_meta, s);
  return hipGetLastError();
}

}  // namespace specache
