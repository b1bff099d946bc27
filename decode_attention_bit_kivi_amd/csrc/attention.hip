// Mixed attention O = Attn([T_t, T'_{t+1}], C' U C_kappa): split-K online
// softmax over (i) the low-bit positions not in kappa, (ii) the k fetched
// 16-bit rows, (iii) an optional 16-bit tail, followed by a merge of the
// per-split partials.
//
// SpeCache summary, quick read (third mechanism) and §3 "decoding": the
// 16-bit pairs C_kappa replace their low-bit counterparts; §7 Algorithm 3:
// K = [K' U K_kappa, K_t], A = MaskedSoftmax(Q_t K^T).  The split-K /
// online-softmax organisation is the IO-aware exact-attention idea the SemKV
// page cites in §2.4 (FlashAttention); the result is exact softmax attention
// up to float32 rounding.
//
// Each workgroup handles every query row of one KV head (G heads x T tokens,
// at most 16 rows) for one split, so each low-bit byte is read once for all
// the rows that share it.  Logits are kept in log2 units (q pre-scaled by
// sm_scale * log2 e); partials are (m, l, acc[D]) with l = sum 2^(x - m).
#include "common.h"

namespace specache {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int D>
__global__ __launch_bounds__(256) void attn_split_kernel(AttnArgs a, int Hkv, int G, int64_t N, int bits,
                                                         int64_t L, int S_lb, int Lsel, int S_sel, int S) {
  constexpr int W = D / 32;
  constexpr int kRowGroups = 256 / D;
  constexpr int kAccRows = kMaxRows / kRowGroups;
  __shared__ float qf[kMaxRows][D];
  __shared__ float kh[32][D + 1];
  __shared__ float vh[32][D + 1];
  __shared__ float P[kMaxRows][32];
  __shared__ float m_s[kMaxRows], l_s[kMaxRows], alpha_s[kMaxRows];
  __shared__ int valid[32];
  __shared__ uint32_t kmask[64];

  const int t = threadIdx.x;
  const int split = blockIdx.x;
  const int64_t slice = blockIdx.y;
  const int64_t b = slice / Hkv, h = slice % Hkv;
  const int T = a.T;
  const int R = G * T;
  const int Hq = Hkv * G;
  const int64_t nblk = N / 32;
  const int64_t row0 = b * Hq * T + h * G * T;  // first query row of this slice
  const float qscale = a.sm_scale * kLog2e;

  for (int e = t; e < R * D; e += 256) qf[e / D][e % D] = (float)a.q16[row0 * D + e] * qscale;
  if (t < kMaxRows) {
    m_s[t] = -INFINITY;
    l_s[t] = 0.0f;
    alpha_s[t] = 1.0f;
  }

  int kind;
  int64_t first, count;
  if (split < S_lb) {
    kind = 0;
    first = (int64_t)split * L;
    count = N - first < L ? N - first : L;
  } else if (split < S_lb + S_sel) {
    kind = 1;
    first = (int64_t)(split - S_lb) * Lsel;
    count = a.k - first < Lsel ? a.k - first : Lsel;
  } else {
    kind = 2;
    first = 0;
    count = a.tail;
  }

  if (kind == 0) {
    if (t < 64) kmask[t] = 0u;
    __syncthreads();
    for (int i = t; i < a.k; i += 256) {
      const int64_t p = a.idx[slice * a.k + i];
      if (p >= first && p < first + count) atomicOr(&kmask[(p - first) >> 5], 1u << ((p - first) & 31));
    }
  }

  const int c_own = t % D, rg = t / D;
  float acc[kAccRows];
#pragma unroll
  for (int j = 0; j < kAccRows; ++j) acc[j] = 0.0f;
  __syncthreads();

  for (int64_t j0 = 0; j0 < count; j0 += 32) {
    const int nvalid = count - j0 < 32 ? (int)(count - j0) : 32;
    if (kind == 0) {
      const int64_t blk = (first + j0) / 32;
      {  // keys: thread -> token t/8, D/8 channels
        const int tau = t >> 3;
        const int c0 = (t & 7) * (D / 8);
        const uint32_t* kw = a.k_codes + ((slice * N + blk * 32 + tau) * bits) * W;
        const _Float16* km = a.k_meta + (slice * nblk + blk) * 2 * D;
        uint32_t w0[W], w1[W];
#pragma unroll
        for (int w = 0; w < W; ++w) {
          w0[w] = kw[w];
          w1[w] = bits == 2 ? kw[W + w] : 0u;
        }
#pragma unroll
        for (int cc = 0; cc < D / 8; ++cc) {
          const int c = c0 + cc;
          const int w = c >> 5, bi = elem_to_bit(c & 31);
          const uint32_t code = ((w0[w] >> bi) & 1u) + 2u * ((w1[w] >> bi) & 1u);
          kh[tau][c] = fmaf((float)code, (float)km[D + c], (float)km[c]);
        }
      }
      {  // values: thread -> channel c_own, tokens rg, rg + kRowGroups, ...
        const uint32_t* vw = a.v_codes + (slice * nblk + blk) * bits * D;
        const _Float16* vm = a.v_meta + (slice * nblk + blk) * 2 * W * 32;
        const uint32_t w0 = vw[c_own], w1 = bits == 2 ? vw[D + c_own] : 0u;
        const int wg = c_own >> 5;
        for (int tau = rg; tau < 32; tau += kRowGroups) {
          const int bi = elem_to_bit(tau);
          const uint32_t code = ((w0 >> bi) & 1u) + 2u * ((w1 >> bi) & 1u);
          vh[tau][c_own] = fmaf((float)code, (float)vm[W * 32 + wg * 32 + tau], (float)vm[wg * 32 + tau]);
        }
      }
      if (t < 32) valid[t] = ((kmask[j0 >> 5] >> t) & 1u) ? 0 : 1;
    } else {
      const _Float16* ks = kind == 1 ? a.k_sel + (slice * a.k + first + j0) * D : a.k_tail + (slice * a.tail + j0) * D;
      const _Float16* vs = kind == 1 ? a.v_sel + (slice * a.k + first + j0) * D : a.v_tail + (slice * a.tail + j0) * D;
      for (int e = t; e < 32 * D; e += 256) {
        const int tau = e / D, c = e % D;
        kh[tau][c] = tau < nvalid ? (float)ks[e] : 0.0f;
        vh[tau][c] = tau < nvalid ? (float)vs[e] : 0.0f;
      }
      if (t < 32) valid[t] = t < nvalid ? 1 : 0;
    }
    __syncthreads();

    for (int r0 = 0; r0 < R; r0 += 8) {
      const int r = r0 + (t >> 5);
      const int tau = t & 31;
      if (r < R) {
        float x = 0.0f;
#pragma unroll 16
        for (int c = 0; c < D; ++c) x = fmaf(qf[r][c], kh[tau][c], x);
        bool ok = valid[tau] != 0;
        if (kind == 2) ok = ok && (j0 + tau <= (int64_t)(a.tail - T + r % T));
        if (!ok) x = -INFINITY;
        float bm = x;
#pragma unroll
        for (int off = 16; off > 0; off >>= 1) bm = fmaxf(bm, __shfl_xor(bm, off));
        const float m_old = m_s[r];
        const float m_new = fmaxf(m_old, bm);
        const float p = (m_new == -INFINITY) ? 0.0f : exp2f(x - m_new);
        const float alpha = (m_new == -INFINITY) ? 1.0f : exp2f(m_old - m_new);
        float ps = p;
#pragma unroll
        for (int off = 16; off > 0; off >>= 1) ps += __shfl_xor(ps, off);
        P[r][tau] = p;
        if (tau == 0) {
          m_s[r] = m_new;
          l_s[r] = l_s[r] * alpha + ps;
          alpha_s[r] = alpha;
        }
      }
    }
    __syncthreads();

#pragma unroll
    for (int j = 0; j < kAccRows; ++j) {
      const int r = rg + j * kRowGroups;
      if (r < R) {
        float s = acc[j] * alpha_s[r];
#pragma unroll 8
        for (int tau = 0; tau < 32; ++tau) s = fmaf(P[r][tau], vh[tau][c_own], s);
        acc[j] = s;
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < kAccRows; ++j) {
    const int r = rg + j * kRowGroups;
    if (r < R) {
      const int64_t row = row0 + r;
      a.part_acc[(row * S + split) * D + c_own] = acc[j];
      if (c_own == 0) {
        a.part_ml[(row * S + split) * 2] = m_s[r];
        a.part_ml[(row * S + split) * 2 + 1] = l_s[r];
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(D) void attn_merge_kernel(const float* __restrict__ part_ml,
                                                       const float* __restrict__ part_acc, int S,
                                                       _Float16* __restrict__ out) {
  const int64_t row = blockIdx.x;
  const int c = threadIdx.x;
  const float* ml = part_ml + row * S * 2;
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, ml[2 * s]);
  float l = 0.0f, o = 0.0f;
  for (int s = 0; s < S; ++s) {
    const float m = ml[2 * s];
    if (m == -INFINITY) continue;
    const float w = exp2f(m - M);
    l = fmaf(ml[2 * s + 1], w, l);
    o = fmaf(part_acc[(row * S + s) * D + c], w, o);
  }
  out[row * D + c] = (_Float16)(o / l);
}

}  // namespace

hipError_t launch_decode_attn(const Dims& d, const AttnPlan& plan, const AttnArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)plan.S, (unsigned)d.slices());
  const unsigned rows = (unsigned)((int64_t)d.B * d.Hq * a.T);
  if (d.D == 128) {
    attn_split_kernel<128><<<grid, 256, 0, s>>>(a, d.Hkv, d.G, d.N, d.bits, plan.L, plan.S_lb, plan.Lsel,
                                                plan.S_sel, plan.S);
    attn_merge_kernel<128><<<rows, 128, 0, s>>>(a.part_ml, a.part_acc, plan.S, a.out16);
  } else {
    attn_split_kernel<64><<<grid, 256, 0, s>>>(a, d.Hkv, d.G, d.N, d.bits, plan.L, plan.S_lb, plan.Lsel,
                                               plan.S_sel, plan.S);
    attn_merge_kernel<64><<<rows, 64, 0, s>>>(a.part_ml, a.part_acc, plan.S, a.out16);
  }
  return hipGetLastError();
}

}  // namespace specache
