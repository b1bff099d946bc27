// ArgTopK of the speculative row: merge the split statistics into each head's
// log-sum-exp, form the rank r(p) = log sum_g exp(s_g(p) - LSE_g) (the
// attention mass the G heads put on p), and select the k largest, ties to the
// lower position, emitted in ascending order.
//
// SpeCache summary, §7 Algorithms 2 and 3 (ArgTopK of the attention row), and
// §2 "attention sparsity" (a position is worth the attention mass it holds).
//
// Kernels:
//   rank_keys    (grid: position chunks x slices) computes r(p) for every
//                position, writes it and its maximum over every 16 positions,
//                and adds a coarse histogram of r into a per-slice global
//                histogram (zeroed by the kernel that wrote the logits).  The
//                coarse bins are linear in r over a window of 32 below log G
//                (r <= log G always): 64 bins per unit of r.
//   rank_select  (one 1024-thread workgroup per slice) finds the coarse bin
//                that holds the k-th largest r, gathers that bin's keys into
//                LDS, finds the exact k-th largest key there (one wave counting
//                for at most 64 keys, else a three-digit radix select), and
//                marks the selected positions for one prefix sum that turns
//                them into the ascending output.  Its forms:
//                - resident: a slice of at most 32768 positions read once into
//                  registers (32 keys a thread), from rank_keys' keys or, with
//                  at most 4 heads per KV head, forming r(p) and the histogram
//                  itself from the logits (r(p) through rank_keys' function,
//                  each head's log-sum-exp merged over 16 lanes as the pruned
//                  form merges it, so the two forms' keys are the same bits; no
//                  key buffer unless the caller asks for r);
//                - pruned (the fused step): bounds of every 8 positions from
//                  the split kernel's per-head logit maxima; only the groups
//                  whose upper bound reaches the k-th lower bound are read;
//                - keys (longer slices): from rank_keys' keys, reading only the
//                  groups whose maximum reaches the threshold bin, or sweeping
//                  every key (bitmaps of 128K positions at a time) when too
//                  many do.
//   The exact selection compares order-preserving 32-bit integer keys of the
//   float r.
#include "merge.h"

#include <type_traits>

namespace specache {

namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kKeyThreads = 256;
constexpr int kKeyChunk = kKeyThreads * 8;     // positions per rank_keys workgroup
constexpr int kBins = 2048;
constexpr float kBinSpan = 32.0f;              // r window of the coarse bins, below log G
constexpr float kBinScale = kBins / kBinSpan;  // bins per unit of r (a power of two: exact)
constexpr int kCand = 16384;                   // keys of the threshold bin held in LDS
constexpr float kLn2 = 0.69314718055994531f;

__device__ __forceinline__ uint32_t order_key(float r) {
  const uint32_t f = __float_as_uint(r);
  return (f & 0x80000000u) ? ~f : (f | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// Coarse bin of r: non-decreasing in r (subtraction and truncation are monotone, the scale is
// exact), so every key of a higher bin is larger than every key of a lower one.
__device__ __forceinline__ uint32_t coarse_bin(float r, float r_lo) {
  const float x = (r - r_lo) * kBinScale;
  if (!(x >= 0.0f)) return 0u;  // below the window (or NaN)
  if (x >= (float)(kBins - 1)) return kBins - 1;
  return (uint32_t)x;
}

// Inclusive prefix sum over a wave with DPP lane moves (no LDS round trips): shifts by 1, 2, 4
// and 8 within each row of 16 lanes, then the last lane of row 0 (of rows 0-1) added to rows 1
// and 3 (2 and 3).  Lanes without a source add 0.
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t x) {
  int v = (int)x;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2, 3
  return (uint32_t)v;
}

// Exclusive prefix sum over the 1024-thread workgroup; returns the exclusive value, writes the
// total.  One barrier: each wave posts its total, then every wave scans the 16 totals itself.
// scratch holds two sets of totals, used in turn (ph, uniform, flips at each call): a wave can only
// come back to a set after the barrier of the call in between, which every wave reaches after
// reading it.  Everything every thread does before the call precedes everything any thread does
// after it.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scratch, uint32_t& total, int& ph) {
  const int t = threadIdx.x, lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  uint32_t* tot_w = scratch + ph * kSelWaves;
  ph ^= 1;
  const uint32_t x = wave_inclusive_scan(v);
  if (lane == 63) tot_w[wv] = x;
  __syncthreads();
  const uint32_t s = wave_inclusive_scan(lane < kSelWaves ? tot_w[lane] : 0u);  // lanes 0-15: inclusive
  const uint32_t before = wv > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)s, wv - 1) : 0u;
  total = (uint32_t)__builtin_amdgcn_readlane((int)s, kSelWaves - 1);
  return before + x - v;
}

// For the key c of this lane, among the first nc (<= 64, wave-uniform) lanes' keys: (number
// above c) | (number equal to c) << 16.  Each key is read from its lane with v_readlane (no LDS
// round trip per key).
__device__ __forceinline__ uint32_t count_above_equal(uint32_t c, uint32_t nc) {
  uint32_t gt = 0u, eq = 0u;
  const int n = __builtin_amdgcn_readfirstlane((int)nc);
  for (int j = 0; j < n; ++j) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)c, j);
    gt += o > c ? 1u : 0u;
    eq += o == c ? 1u : 0u;
  }
  return gt | (eq << 16);
}

// Merge of two (max, sum 2^(x - max)) pairs of one head, log2 units.
__device__ __forceinline__ void merge_stat(float& M, float& L, float m, float l) {
  const float mn = fmaxf(M, m);
  L = (M == -INFINITY ? 0.0f : L * exp2f(M - mn)) + (m == -INFINITY ? 0.0f : l * exp2f(m - mn));
  M = mn;
}

// One head's log2-sum-exp2 from its S split statistics, read by TPH lanes of one wave (lane j
// takes splits j, j + TPH, ...; its first pair, m_first / l_first, already loaded), merged across
// the lanes.  Every lane returns the head's value.
template <int TPH>
__device__ __forceinline__ float head_lse2(const float* pm, const float* pl, int S, int j, float m_first,
                                           float l_first) {
  float M = -INFINITY, L = 0.0f;
  for (int s = j; s < S; s += TPH) merge_stat(M, L, s == j ? m_first : pm[s], s == j ? l_first : pl[s]);
#pragma unroll
  for (int off = 1; off < TPH; off <<= 1) merge_stat(M, L, __shfl_xor(M, off), __shfl_xor(L, off));
  return M + log2f(L);
}

// The same from 16 lanes: lane j of each row of 16 takes splits j, j + 16, ... (its first pair,
// m_first / l_first, already loaded), and the rows merge across their lanes with DPP moves (no
// LDS round trip): swaps of neighbours, then of pairs, then the two halves of each half row and of
// the row (mirrors).  Each merge is symmetric, so every lane ends with the same bits.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float head_lse2_row(const float* pm, const float* pl, int S, int j, float m_first,
                                               float l_first) {
  float M = -INFINITY, L = 0.0f;
  for (int s = j; s < S; s += 16) merge_stat(M, L, s == j ? m_first : pm[s], s == j ? l_first : pl[s]);
  merge_stat(M, L, dpp_move<0xB1>(M), dpp_move<0xB1>(L));    // quad_perm [1, 0, 3, 2]
  merge_stat(M, L, dpp_move<0x4E>(M), dpp_move<0x4E>(L));    // quad_perm [2, 3, 0, 1]
  merge_stat(M, L, dpp_move<0x141>(M), dpp_move<0x141>(L));  // row_half_mirror
  merge_stat(M, L, dpp_move<0x140>(M), dpp_move<0x140>(L));  // row_mirror
  return M + log2f(L);
}

// r of the position held in component e of x[g] (head g's logit, log2 units):
// log sum_g exp(s_g - LSE_g), in natural-log units.
template <int GM>
__device__ __forceinline__ float rank_of(const float4 (&x)[GM], int e, const float* lse2, int G) {
  float lp[GM];
  float mx = -INFINITY;
#pragma unroll
  for (int g = 0; g < GM; ++g)
    if (g < G) {
      const float4 v4 = x[g];
      const float v = e == 0 ? v4.x : (e == 1 ? v4.y : (e == 2 ? v4.z : v4.w));
      lp[g] = v - lse2[g];  // log2 of the head's probability (the logits are in log2 units)
      mx = fmaxf(mx, lp[g]);
    }
  float sum = 0.0f;
#pragma unroll
  for (int g = 0; g < GM; ++g)
    if (g < G) sum += __builtin_amdgcn_exp2f(lp[g] - mx);
  // v_log_f32 is log2; adding +0 turns a -0 into +0, so that comparing the floats and comparing
  // their order-preserving keys agree
  return (mx + __builtin_amdgcn_logf(sum)) * kLn2 + 0.0f;
}

// ---------------------------------------------------------------- rank_keys

// Also the maximum key of every 16 positions into kmax[slice][N / 16] (the four lanes of a group
// hold its four runs of one step), for the selection from the groups that reach the threshold bin.
template <int GM>  // GM >= G: the heads' logits of a run are held in registers
__global__ __launch_bounds__(kKeyThreads) void rank_keys_kernel(const float* logits, const float* part_m,
                                                                const float* part_l, int G, int S,
                                                                int64_t N, float r_lo, float* __restrict__ rkey,
                                                                uint32_t* __restrict__ ghist,
                                                                float* __restrict__ kmax) {
  __shared__ float lse2[GM];  // log2-sum-exp2 of each head, in log2 units
  __shared__ uint32_t hist[kBins];
  const int t = threadIdx.x;
  const int64_t slice = blockIdx.y;
  const int64_t c0 = (int64_t)blockIdx.x * kKeyChunk;

  // Each head's log-sum-exp comes from the split statistics (max, sum 2^(x - max)), log2 units:
  // kKeyThreads / GM threads per head read the splits in parallel and merge across lanes.  Their
  // first split's loads are issued before anything else (clamped, unconditional), so that waiting
  // for them leaves the logits' loads in flight.
  constexpr int TPH = kKeyThreads / GM;  // 64, 32 or 16: within one wave
  const int hg = t / TPH, hj = t % TPH;
  const int64_t st0 = (slice * G + (hg < G ? hg : 0)) * S + (hj < S ? hj : 0);
  const float m_first = part_m[st0], l_first = part_l[st0];
  // keeps these two loads ahead of the logits' loads (the inputs are not restrict-qualified, so
  // that the compiler cannot treat the loads as invariant and move them past such points)
  asm volatile("" ::: "memory");
  // Each thread: kRuns runs of 4 consecutive positions (a float4 per head), NB runs in flight
  // (all of them for up to 4 heads), with clamped addresses.  Small chunks (two runs a thread)
  // keep more workgroups, and so more of the logits' loads, in flight at once.
  constexpr int kRuns = kKeyChunk / (4 * kKeyThreads);
  constexpr int NB = GM <= 4 ? kRuns : (kRuns < 2 ? kRuns : 2);
  const float* lg = logits + slice * G * N;
  float4 x[NB][GM];
  auto load = [&](int rr, float4 (&dst)[GM]) {
    int64_t p = c0 + 4 * (t + rr * kKeyThreads);
    if (p >= N) p = c0;  // past the end: a valid address, the values go unused
#pragma unroll
    for (int g = 0; g < GM; ++g)
      dst[g] = *reinterpret_cast<const float4*>(lg + (int64_t)(g < G ? g : 0) * N + p);
    asm volatile("" ::: "memory");  // runs issue in order, so each run waits only for its own loads
  };
#pragma unroll
  for (int rr = 0; rr < NB; ++rr) load(rr, x[rr]);
  {
    const int g = hg < G ? hg : 0;  // the lanes of heads past G merge head 0 again, unused
    const float l2 = head_lse2<TPH>(part_m + (slice * G + g) * S, part_l + (slice * G + g) * S, S, hj, m_first,
                                    l_first);
    if (hg < G && hj == 0) lse2[hg] = l2;
  }
  for (int i = t; i < kBins; i += kKeyThreads) hist[i] = 0u;
  __syncthreads();
  uint32_t cur_bin = 0u, cur_cnt = 0u;  // this thread's pending histogram increment
#pragma unroll
  for (int rr = 0; rr < kRuns; ++rr) {
    const int64_t p = c0 + 4 * (t + rr * kKeyThreads);
    if (p < N) {  // N is a multiple of 32: the whole float4 is in range
      float r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = rank_of<GM>(x[rr % NB], e, lse2, G);
      *reinterpret_cast<float4*>(rkey + slice * N + p) = make_float4(r[0], r[1], r[2], r[3]);
      // lanes 4j .. 4j + 3 hold positions 16j' .. 16j' + 15 (p is a multiple of 16 at lane 4j;
      // N is a multiple of 32, so the four lanes of a group are all in range together)
      float gm = fmaxf(fmaxf(r[0], r[1]), fmaxf(r[2], r[3]));
      gm = fmaxf(gm, __shfl_xor(gm, 1));
      gm = fmaxf(gm, __shfl_xor(gm, 2));
      if ((t & 3) == 0) kmax[slice * (N / 16) + p / 16] = gm;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t b = coarse_bin(r[e], r_lo);
        if (cur_cnt != 0u && b != cur_bin) atomicAdd(&hist[cur_bin], cur_cnt), cur_cnt = 0u;
        cur_bin = b;
        ++cur_cnt;
      }
    }
    if (rr + NB < kRuns) load(rr + NB, x[rr % NB]);  // the slot just consumed takes a later run
  }
  if (cur_cnt) atomicAdd(&hist[cur_bin], cur_cnt);
  __syncthreads();
  uint32_t* gh = ghist + slice * kBins;
  for (int i = t; i < kBins; i += kKeyThreads)
    if (hist[i]) atomicAdd(&gh[i], hist[i]);
}

// ---------------------------------------------------------------- rank_select

constexpr int kChunk = 131072;        // positions per compaction chunk
constexpr int kWords = kChunk / 32;   // bitmap words of a chunk
constexpr int kWordsPerThread = kWords / kSelThreads;

struct SelectSmem {
  uint32_t hist[kBins];
  uint32_t scan_scratch[2 * kSelWaves];
  uint32_t sel_digit, sel_above, sel_count, n_cand;
  union {
    uint32_t cand[kCand];  // keys of the threshold bin
    struct {
      uint32_t gt[kWords];  // positions of the chunk above the threshold
      uint32_t eq[kWords];  // positions of the chunk equal to it
    } bm;
  } u;
};

// Visit the values of positions [p0, p1) (multiples of 4), coalesced: each float4 load of the
// workgroup reads 4096 consecutive values, and a thread has kSweepU of them in flight before
// it processes any.  fn(base, v) gets this thread's values of one step: v[4u + e] is position
// base + 4 * (threadIdx.x + u * kSelThreads) + e, -inf past p1.
constexpr int kSweepU = 8;
template <typename Fn>
__device__ __forceinline__ void sweep(const float* ky, int64_t p0, int64_t p1, Fn fn) {
  for (int64_t base = p0; base < p1; base += (int64_t)kSweepU * 4 * kSelThreads) {
    float v[4 * kSweepU];
#pragma unroll
    for (int u = 0; u < kSweepU; ++u) {
      const int64_t p = base + 4 * ((int64_t)threadIdx.x + u * kSelThreads);
      const float4 f = p < p1 ? *reinterpret_cast<const float4*>(ky + p)
                              : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      v[4 * u] = f.x;
      v[4 * u + 1] = f.y;
      v[4 * u + 2] = f.z;
      v[4 * u + 3] = f.w;
    }
    fn(base, v);
  }
}

__device__ __forceinline__ int64_t sweep_pos(int64_t base, int i) {
  return base + 4 * ((int64_t)threadIdx.x + (i >> 2) * kSelThreads) + (i & 3);
}

// The digit of hist[0, nbins) holding the krem-th largest element, counted from the top, the
// number of elements in the digits above it and the number in the digit itself (so that no
// thread reads hist after the call: a caller may clear it next without a barrier).
// With krem outside [1, total], digit 0 and 0 above it.  Exactly one thread writes the answer,
// after the scan's barrier: the reads of the previous call's answer precede that barrier.
template <typename Smem>
__device__ __forceinline__ void pick_digit(Smem& sm, int& ph, int nbins, uint32_t krem, uint32_t& digit,
                                           uint32_t& above, uint32_t& count) {
  const int t = threadIdx.x;
  // thread t covers digits nbins-1-2t and nbins-2-2t
  const int dhi = nbins - 1 - 2 * t, dlo = dhi - 1;
  const uint32_t hhi = dhi >= 0 ? sm.hist[dhi] : 0u;
  const uint32_t hlo = dlo >= 0 ? sm.hist[dlo] : 0u;
  uint32_t tot;
  const uint32_t excl = block_exclusive_scan(hhi + hlo, sm.scan_scratch, tot, ph);
  if (krem >= 1u && krem <= tot) {
    if (dhi >= 0 && excl < krem && excl + hhi >= krem) {
      sm.sel_digit = (uint32_t)dhi;
      sm.sel_above = excl;
      sm.sel_count = hhi;
    } else if (dlo >= 0 && excl + hhi < krem && excl + hhi + hlo >= krem) {
      sm.sel_digit = (uint32_t)dlo;
      sm.sel_above = excl + hhi;
      sm.sel_count = hlo;
    }
  } else if (dlo == 0 || (dhi == 0 && dlo < 0)) {
    sm.sel_digit = 0u;
    sm.sel_above = 0u;
    sm.sel_count = dlo == 0 ? hlo : hhi;
  }
  __syncthreads();
  digit = sm.sel_digit;
  above = sm.sel_above;
  count = sm.sel_count;
}

// Exact radix select: the krem-th largest key among those `count` feeds to the histogram, as
// (key thr, number of keys equal to thr to take, number of keys equal to thr).
// count(shift, nbins, prefix, mask) adds every key u with (u & mask) == prefix to
// sm.hist[(u >> shift) & (nbins - 1)].
template <typename Smem, typename Count>
__device__ __forceinline__ void radix_select(Smem& sm, int& ph, uint32_t krem, Count count, uint32_t& thr,
                                             uint32_t& need_eq, uint32_t& n_eq) {
  const int t = threadIdx.x;
  uint32_t prefix = 0u, mask = 0u;
  for (int pass = 0; pass < 3; ++pass) {  // digits: bits 31..21, 20..10, 9..0
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const int nbins = pass == 2 ? 1024 : 2048;
    for (int i = t; i < kBins; i += kSelThreads) sm.hist[i] = 0u;
    __syncthreads();
    count(shift, nbins, prefix, mask);
    __syncthreads();
    uint32_t dg, ab, cnt;
    pick_digit(sm, ph, nbins, krem, dg, ab, cnt);
    prefix |= dg << shift;
    mask |= (uint32_t)(nbins - 1) << shift;
    krem -= ab;
    if (pass == 2) n_eq = cnt;  // the last digit's bin holds exactly the keys equal to thr
  }
  thr = prefix;
  need_eq = krem;
}

// Smallest order key of a non-NaN value whose coarse bin is >= b, for b < kBins, found by one
// wave.  Between the keys of -inf and +inf the bins are non-decreasing in the key, and bin(+inf) =
// kBins - 1 >= b.  Each round probes 64 evenly spaced keys of [lo, hi] (the answer is in it, and
// the condition holds at hi): the answer lies at or below the first probe where it holds and
// above the probe before.
__device__ uint32_t first_key_of_bin_wave(uint32_t b, float r_lo) {
  const int lane = threadIdx.x & 63;
  uint32_t lo = 0x007fffffu, hi = 0xff800000u;
  if (b == 0u) return lo;  // every value is in a bin >= 0
  {
    // the bin starts at about r_lo + b / kBinScale: probe the 64 keys around that value first
    const uint32_t c = order_key(r_lo + (float)b / kBinScale);
    const uint32_t x = c - 32u + (uint32_t)lane;
    const uint64_t m = __ballot(coarse_bin(key_value(x), r_lo) >= b);
    if (m != 0u && !(m & 1u)) return c - 32u + (uint32_t)__builtin_ctzll(m);  // the answer is inside
  }
  while (lo < hi) {
    const uint64_t step = ((uint64_t)(hi - lo) + 63u) / 64u;
    uint64_t x = (uint64_t)lo + (uint64_t)lane * step;
    if (x > hi) x = hi;
    const uint64_t m = __ballot(coarse_bin(key_value((uint32_t)x), r_lo) >= b);
    if (m == 0u) {  // every probe below the answer (the last one is then below hi)
      lo = (uint32_t)(lo + 63u * step) + 1u;
      continue;
    }
    const int j = __builtin_ctzll(m);
    if (j == 0) break;  // the answer is lo
    const uint64_t xj = (uint64_t)lo + (uint64_t)j * step;
    hi = (uint32_t)(xj < hi ? xj : hi);
    lo = (uint32_t)((uint64_t)lo + (uint64_t)(j - 1) * step) + 1u;
  }
  return lo;
}

// The selection of slice `slice` from every key of the slice (rkey) and their coarse histogram
// (ghist), in sweeps over the keys: the threshold bin's keys into LDS, the exact threshold among
// them, then the positions above it (and the first equal ones) in position order, a chunk at a
// time.  bin_vals: two floats of LDS outside sm.
__device__ void select_by_sweeps(SelectSmem& sm, float* bin_vals, const float* __restrict__ rkey,
                                 const uint32_t* __restrict__ ghist, int64_t N, int k, float r_lo,
                                 int32_t* __restrict__ idx_out, int64_t slice) {
  const int t = threadIdx.x, lane = t & 63;
  int ph = 0;  // the block scans' scratch set (the caller's scans ended before its barrier)
  const float* ky = rkey + slice * N;
  const uint32_t* gh = ghist + slice * kBins;
  for (int i = t; i < kBins; i += kSelThreads) sm.hist[i] = gh[i];
  if (t == 0) sm.n_cand = 0u;
  __syncthreads();

  uint32_t bin, above, in_bin;
  pick_digit(sm, ph, kBins, (uint32_t)k, bin, above, in_bin);
  // the threshold bin as an interval of values [lo, hi) (the top bin runs to +inf), found by two
  // binary searches over the keys.  The ranks hold no -0 and no NaN, so comparing the floats
  // orders them as their keys do.
  if (t < 64) {
    const uint32_t key = first_key_of_bin_wave(bin, r_lo);
    if (t == 0) bin_vals[0] = key_value(key);
  } else if (t < 128) {
    const float vb = bin + 1 < (uint32_t)kBins ? key_value(first_key_of_bin_wave(bin + 1, r_lo)) : INFINITY;
    if (t == 64) bin_vals[1] = vb;
  }
  __syncthreads();
  const float va = bin_vals[0], vb = bin_vals[1];
  const bool top_open = bin + 1 >= (uint32_t)kBins;

  uint32_t thr, need_eq, n_thr;
  if (in_bin <= (uint32_t)kCand) {
    // gather the threshold bin's keys into LDS (any order)
    sweep(ky, 0, N, [&](int64_t base, const float (&v)[4 * kSweepU]) {
      uint32_t mine = 0u;
#pragma unroll
      for (int i = 0; i < 4 * kSweepU; ++i)
        mine |= (sweep_pos(base, i) < N && v[i] >= va && (top_open || v[i] < vb)) ? (1u << i) : 0u;
      if (!__any(mine != 0u)) return;
      // slots: one prefix sum over the wave and one LDS atomic per wave
      const uint32_t n = __popc(mine);
      const uint32_t incl = wave_inclusive_scan(n);
      uint32_t base_slot = 0u;
      if (lane == 63) base_slot = atomicAdd(&sm.n_cand, incl);
      base_slot = __shfl(base_slot, 63);
      uint32_t slot = base_slot + incl - n;
#pragma unroll
      for (int i = 0; i < 4 * kSweepU; ++i)
        if ((mine >> i) & 1u) {
          if (slot < (uint32_t)kCand) sm.u.cand[slot] = order_key(v[i]);
          ++slot;
        }
    });
    __syncthreads();
    const uint32_t nc = sm.n_cand < (uint32_t)kCand ? sm.n_cand : (uint32_t)kCand;
    radix_select(sm, ph, (uint32_t)k - above,
                 [&](int shift, int nbins, uint32_t prefix, uint32_t mask) {
                   for (uint32_t i = t; i < nc; i += kSelThreads) {
                     const uint32_t u = sm.u.cand[i];
                     if ((u & mask) == prefix) atomicAdd(&sm.hist[(u >> shift) & (uint32_t)(nbins - 1)], 1u);
                   }
                 },
                 thr, need_eq, n_thr);
  } else {
    radix_select(sm, ph, (uint32_t)k,
                 [&](int shift, int nbins, uint32_t prefix, uint32_t mask) {
                   sweep(ky, 0, N, [&](int64_t base, const float (&v)[4 * kSweepU]) {
#pragma unroll
                     for (int i = 0; i < 4 * kSweepU; ++i) {
                       const uint32_t u = order_key(v[i]);
                       if (sweep_pos(base, i) < N && (u & mask) == prefix)
                         atomicAdd(&sm.hist[(u >> shift) & (uint32_t)(nbins - 1)], 1u);
                     }
                   });
                 },
                 thr, need_eq, n_thr);
  }
  __syncthreads();  // the candidate keys are dead: their LDS becomes the bitmaps

  // Every value above thr and the first need_eq equal to it, in position order: per chunk, mark
  // them in two bitmaps, then compact the bitmaps' set bits with one prefix sum.
  const float vthr = key_value(thr);
  const bool all_eq = need_eq == n_thr;  // every key equal to thr is taken: one bitmap, one prefix sum
  uint32_t out_base = 0u, eq_seen = 0u;
  for (int64_t c0 = 0; c0 < N; c0 += kChunk) {
    const int64_t c1 = c0 + kChunk < N ? c0 + kChunk : N;
    // the previous chunk's bitmap words are read by the threads that own them (kWordsPerThread
    // each) and cleared here by others: every read must come first
    if (c0 > 0) __syncthreads();
    for (int i = t; i < kWords; i += kSelThreads) {
      sm.u.bm.gt[i] = 0u;
      sm.u.bm.eq[i] = 0u;
    }
    __syncthreads();
    sweep(ky, c0, c1, [&](int64_t base, const float (&v)[4 * kSweepU]) {
#pragma unroll
      for (int i = 0; i < 4 * kSweepU; ++i) {
        const int64_t q = sweep_pos(base, i) - c0;
        if (q >= c1 - c0) continue;
        if (v[i] > vthr || (all_eq && v[i] == vthr)) atomicOr(&sm.u.bm.gt[q >> 5], 1u << (q & 31));
        else if (v[i] == vthr) atomicOr(&sm.u.bm.eq[q >> 5], 1u << (q & 31));
      }
    });
    __syncthreads();
    uint32_t ngt = 0u, neq = 0u;
#pragma unroll
    for (int j = 0; j < kWordsPerThread; ++j) {
      ngt += __popc(sm.u.bm.gt[t * kWordsPerThread + j]);
      neq += __popc(sm.u.bm.eq[t * kWordsPerThread + j]);
    }
    uint32_t eq_tot = 0u, take_tot;
    uint32_t eq_take = 0u;
    if (!all_eq) {
      const uint32_t eq_before = eq_seen + block_exclusive_scan(neq, sm.scan_scratch, eq_tot, ph);
      eq_take = eq_before >= need_eq ? 0u : (need_eq - eq_before < neq ? need_eq - eq_before : neq);
    }
    uint32_t out = out_base + block_exclusive_scan(ngt + eq_take, sm.scan_scratch, take_tot, ph);
    uint32_t eq_left = eq_take;
#pragma unroll
    for (int j = 0; j < kWordsPerThread; ++j) {
      const int w = t * kWordsPerThread + j;
      uint32_t m = sm.u.bm.gt[w];
      uint32_t e = sm.u.bm.eq[w];
      while (eq_left > 0u && e != 0u) {  // the lowest equal positions first
        const uint32_t low = e & (0u - e);
        m |= low;
        e ^= low;
        --eq_left;
      }
      while (m != 0u) {
        const int b = __builtin_ctz(m);
        m &= m - 1u;
        if (out < (uint32_t)k) idx_out[slice * k + out] = (int32_t)(c0 + 32 * w + b);
        ++out;
      }
    }
    out_base += take_tot;
    eq_seen += eq_tot;
    __syncthreads();  // the bitmaps are rewritten by the next chunk
  }
}

// ---- rank_select for slices of at most kResidentN positions: the keys stay in registers
// (one coalesced read), the threshold bin's interval comes from two one-wave searches, a bin of
// at most 64 keys is resolved by one wave counting, and the compaction builds one bitmap word
// per thread from mark bytes.
constexpr int64_t kResidentN = (int64_t)kSelThreads * 4 * kSweepU;
constexpr int kResidentWords = (int)(kResidentN / 32);

static_assert(kBins == 2 * kSelThreads, "two histogram bins per thread");
static_assert(kResidentWords == kSelThreads, "one bitmap word per thread");
static_assert(kSweepU == 8, "eight mark bytes per bitmap word");

struct ResidentSmem {
  uint32_t hist[kBins];
  uint32_t scan_scratch[2 * kSelWaves];
  uint32_t sel_digit, sel_above, sel_count, n_cand;
  uint32_t res[4];  // small-bin selection: thr, need_eq, n_eq, found
  float bin_vals[2];
  // marks of positions 4n .. 4n + 3: bit e selected (above the threshold, or equal to it when all
  // equal keys are taken), bit 4 + e equal to the threshold otherwise
  alignas(16) uint8_t marks[kResidentN / 4];
  uint32_t cand[kCand];
};

// Inputs of the resident selection when it forms r(p) itself (FUSED): the rank row's logits and
// the split statistics, as rank_keys takes them, for G <= kFusedG heads.  keys_out, if not null,
// receives r as rank_keys would write it.
struct FusedRank {
  const float* logits;  // [slices][G][N], log2 units
  const float* part_m;  // [slices][G][S]
  const float* part_l;
  int G, S;
  float* keys_out;
};

constexpr int kFusedG = 4;   // heads per slice the fused form holds in registers
constexpr int kFusedNB = 3;  // float4 runs (of every head) a thread has in flight

template <int D, bool FUSED>
__global__ __launch_bounds__(kSelThreads) void rank_select_resident_kernel(const float* __restrict__ rkey,
                                                                           const uint32_t* __restrict__ ghist,
                                                                           int64_t N, int k, float r_lo,
                                                                           int32_t* __restrict__ idx_out,
                                                                           unsigned n_sel, MergeJob mj,
                                                                           FusedRank fr) {
  if (blockIdx.x >= n_sel) {  // a merge workgroup: one query row per wave
    const int64_t row = (int64_t)(blockIdx.x - n_sel) * kSelWaves + (threadIdx.x >> 6);
    if (row < mj.rows) merge_row_wave<D>(mj.part_ml, mj.part_acc, mj.S, mj.out16, row);
    return;
  }
  __shared__ ResidentSmem sm;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  int ph = 0;  // the block scans' scratch set
  const int64_t slice = blockIdx.x;
  // N <= kResidentN: positions fit 32 bits; a float4 is wholly in range or wholly past N
  auto in_range = [&](int u) { return 4 * (t + u * kSelThreads) < (int)N; };
  // v[4u + e]: position 4 * (t + u * kSelThreads) + e, -inf past N (N is a multiple of 32)
  float v[4 * kSweepU];
  if constexpr (FUSED) {
    // r(p) formed here (the arithmetic of rank_keys, shared with it): each head's log-sum-exp
    // from the split statistics by one wave per head, then the float4 runs of the G heads'
    // logits, kFusedNB runs in flight (issued before the statistics, clamped addresses), and the
    // coarse histogram with LDS atomics
    __shared__ float lse2[kFusedG];
    const int G = fr.G, S = fr.S;
    const float* lg = fr.logits + slice * G * N;
    float4 x[kFusedNB][kFusedG];
    // the logits are read once: non-temporal loads (measured ~0.5 µs faster per call)
    typedef float f4v __attribute__((ext_vector_type(4)));
    auto load = [&](int u, float4 (&dst)[kFusedG]) {
      int64_t p = 4 * ((int64_t)t + u * kSelThreads);
      if (p >= N) p = 0;  // past the end: a valid address, the values go unused
#pragma unroll
      for (int g = 0; g < kFusedG; ++g) {
        const f4v w = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(lg + (int64_t)(g < G ? g : 0) * N + p));
        dst[g] = make_float4(w.x, w.y, w.z, w.w);
      }
      asm volatile("" ::: "memory");  // runs issue in order, so each run waits only for its own loads
    };
    const int hw = wave < G ? wave : 0;  // waves past G merge head 0 again, unused
    const int64_t sb = (slice * G + hw) * S;
    const int j0 = (lane & 15) < S ? (lane & 15) : 0;
    const float m_first = fr.part_m[sb + j0], l_first = fr.part_l[sb + j0];
    asm volatile("" ::: "memory");
#pragma unroll
    for (int u = 0; u < kFusedNB; ++u) load(u, x[u]);
    sm.hist[t] = 0u;
    sm.hist[t + kSelThreads] = 0u;
    if (wave < kFusedG) {
      const float l2 = head_lse2_row(fr.part_m + sb, fr.part_l + sb, S, lane & 15, m_first, l_first);
      if (wave < G && lane == 0) lse2[wave] = l2;
    }
    if (t == 0) {
      sm.n_cand = 0u;
      sm.res[3] = 0u;
    }
    __syncthreads();
    uint32_t cur_bin = 0u, cur_cnt = 0u;  // this thread's pending histogram increment
#pragma unroll
    for (int u = 0; u < kSweepU; ++u) {
      if (in_range(u)) {
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = rank_of<kFusedG>(x[u % kFusedNB], e, lse2, G);
        if (fr.keys_out)
          *reinterpret_cast<float4*>(fr.keys_out + slice * N + 4 * (t + u * kSelThreads)) =
              make_float4(r[0], r[1], r[2], r[3]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[4 * u + e] = r[e];
          const uint32_t b = coarse_bin(r[e], r_lo);
          if (cur_cnt != 0u && b != cur_bin) atomicAdd(&sm.hist[cur_bin], cur_cnt), cur_cnt = 0u;
          cur_bin = b;
          ++cur_cnt;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[4 * u + e] = -INFINITY;
      }
      if (u + kFusedNB < kSweepU) load(u + kFusedNB, x[u % kFusedNB]);  // the slot just consumed
    }
    if (cur_cnt) atomicAdd(&sm.hist[cur_bin], cur_cnt);
    __syncthreads();
  } else {
    const float* ky = rkey + slice * N;
    const uint32_t* gh = ghist + slice * kBins;
    // the histogram's loads first and then the keys', all unconditional (clamped addresses), so
    // that waiting for the histogram leaves the keys in flight; the empty statement with a memory
    // clobber keeps every load above the first barrier
    const uint32_t h0 = gh[t], h1 = gh[t + kSelThreads];
    float4 f[kSweepU];
#pragma unroll
    for (int u = 0; u < kSweepU; ++u) {
      const int64_t p = 4 * ((int64_t)t + u * kSelThreads);
      f[u] = *reinterpret_cast<const float4*>(ky + (p < N ? p : 0));
    }
    asm volatile("" ::: "memory");
    sm.hist[t] = h0;
    sm.hist[t + kSelThreads] = h1;
#pragma unroll
    for (int u = 0; u < kSweepU; ++u) {
      const bool in = in_range(u);
      v[4 * u] = in ? f[u].x : -INFINITY;
      v[4 * u + 1] = in ? f[u].y : -INFINITY;
      v[4 * u + 2] = in ? f[u].z : -INFINITY;
      v[4 * u + 3] = in ? f[u].w : -INFINITY;
    }
    if (t == 0) {
      sm.n_cand = 0u;
      sm.res[3] = 0u;
    }
    __syncthreads();
  }

  uint32_t bin, above, in_bin;
  pick_digit(sm, ph, kBins, (uint32_t)k, bin, above, in_bin);
  if (wave == 0) {
    const uint32_t key = first_key_of_bin_wave(bin, r_lo);
    if (lane == 0) sm.bin_vals[0] = key_value(key);
  } else if (wave == 1) {
    const float vb = bin + 1 < (uint32_t)kBins ? key_value(first_key_of_bin_wave(bin + 1, r_lo)) : INFINITY;
    if (lane == 0) sm.bin_vals[1] = vb;
  }
  __syncthreads();
  const float va = sm.bin_vals[0], vb = sm.bin_vals[1];
  const bool top_open = bin + 1 >= (uint32_t)kBins;

  uint32_t thr, need_eq, n_thr;
  if (in_bin <= (uint32_t)kCand) {
    // the threshold bin's keys into LDS (any order): one prefix sum and one LDS atomic per wave
    uint32_t mine = 0u;
#pragma unroll
    for (int u = 0; u < kSweepU; ++u)
      if (in_range(u))
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = v[4 * u + e];
          mine |= (x >= va && (top_open || x < vb)) ? (1u << (4 * u + e)) : 0u;
        }
    if (__any(mine != 0u)) {
      const uint32_t n = __popc(mine);
      const uint32_t incl = wave_inclusive_scan(n);
      uint32_t base_slot = 0u;
      if (lane == 63) base_slot = atomicAdd(&sm.n_cand, incl);
      base_slot = __shfl(base_slot, 63);
      uint32_t slot = base_slot + incl - n;
#pragma unroll
      for (int i = 0; i < 4 * kSweepU; ++i)
        if ((mine >> i) & 1u) {
          if (slot < (uint32_t)kCand) sm.cand[slot] = order_key(v[i]);
          ++slot;
        }
    }
    __syncthreads();
    const uint32_t nc = sm.n_cand < (uint32_t)kCand ? sm.n_cand : (uint32_t)kCand;
    const uint32_t krem = (uint32_t)k - above;
    if (nc <= 64u) {
      if (wave == 0) {
        // lane j: how many of the bin's keys are above / equal to key j; key j is the threshold
        // when the krem-th largest falls among its equals
        const uint32_t c = (uint32_t)lane < nc ? sm.cand[lane] : 0u;
        const uint32_t gt_eq = count_above_equal(c, nc);
        const uint32_t gt = gt_eq & 0xffffu, eq = gt_eq >> 16;
        const uint64_t m = __ballot((uint32_t)lane < nc && gt < krem && krem <= gt + eq);
        if (m != 0u && lane == __builtin_ctzll(m)) {
          sm.res[0] = c;
          sm.res[1] = krem - gt;
          sm.res[2] = eq;
          sm.res[3] = 1u;
        }
      }
      __syncthreads();
    }
    if (sm.res[3]) {
      thr = sm.res[0];
      need_eq = sm.res[1];
      n_thr = sm.res[2];
    } else {
      radix_select(sm, ph, krem,
                   [&](int shift, int nbins, uint32_t prefix, uint32_t mask) {
                     for (uint32_t i = t; i < nc; i += kSelThreads) {
                       const uint32_t u = sm.cand[i];
                       if ((u & mask) == prefix) atomicAdd(&sm.hist[(u >> shift) & (uint32_t)(nbins - 1)], 1u);
                     }
                   },
                   thr, need_eq, n_thr);
    }
  } else {
    radix_select(sm, ph, (uint32_t)k,
                 [&](int shift, int nbins, uint32_t prefix, uint32_t mask) {
#pragma unroll
                   for (int i = 0; i < 4 * kSweepU; ++i) {
                     const uint32_t u = order_key(v[i]);
                     if (in_range(i >> 2) && (u & mask) == prefix)
                       atomicAdd(&sm.hist[(u >> shift) & (uint32_t)(nbins - 1)], 1u);
                   }
                 },
                 thr, need_eq, n_thr);
  }

  // Every key above thr and the first need_eq equal to it, in position order: a mark byte per
  // float4, then thread t gathers the eight bytes of positions 32t .. 32t + 31 into two words
  // (selected, equal) and one prefix sum over the words orders the output.
  const float vthr = key_value(thr);
  const bool all_eq = need_eq == n_thr;  // every key equal to thr is taken
#pragma unroll
  for (int u = 0; u < kSweepU; ++u) {
    uint32_t mk = 0u;
    if (in_range(u))
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = v[4 * u + e];
        mk |= (x > vthr || (all_eq && x == vthr)) ? (1u << e) : 0u;
        mk |= (!all_eq && x == vthr) ? (16u << e) : 0u;
      }
    sm.marks[t + u * kSelThreads] = (uint8_t)mk;
  }
  __syncthreads();
  uint32_t m = 0u, e = 0u;
  {
    const uint2 b8 = *reinterpret_cast<const uint2*>(&sm.marks[8 * t]);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t byte = ((j < 4 ? b8.x : b8.y) >> (8 * (j & 3))) & 0xffu;
      m |= (byte & 15u) << (4 * j);
      e |= (byte >> 4) << (4 * j);
    }
  }
  uint32_t tot;
  if (!all_eq) {
    const uint32_t ne = __popc(e);
    const uint32_t eq_before = block_exclusive_scan(ne, sm.scan_scratch, tot, ph);
    uint32_t eq_take = eq_before >= need_eq ? 0u : (need_eq - eq_before < ne ? need_eq - eq_before : ne);
    while (eq_take > 0u) {  // the lowest equal positions first
      const uint32_t low = e & (0u - e);
      m |= low;
      e ^= low;
      --eq_take;
    }
  }
  uint32_t out = block_exclusive_scan(__popc(m), sm.scan_scratch, tot, ph);
  while (m != 0u) {
    const int b = __builtin_ctz(m);
    m &= m - 1u;
    if (out < (uint32_t)k) idx_out[slice * k + out] = (int32_t)(32 * t + b);
    ++out;
  }
}

// ---- rank_select from per-group bounds (the fused step, slices of at most kResidentN positions,
// at most kFusedG heads).  r(p) is non-decreasing in every head's logit, so with M_g the maximum
// of head g's logits over a group of kBoundGroup (8) positions:
//   U = r(M_1, .., M_G)             bounds r from above over the group, and
//   L = max_g (M_g - LSE_g)         from below at the position holding that maximum (r is at
//                                   least any one head's log-probability);
// at least k positions therefore have r >= the k-th largest L, and only a group whose U reaches
// that value can hold a selected position.  The kernel reads the bounds, the logits of those
// groups only, and selects among their positions exactly as the resident selection does.
// Ranking by the mixed cache, the fetched positions' logits are 16-bit ones written after the
// bounds were taken: the groups that hold them are always read and give no L.  The same kernel,
// in its KEYS form (below), serves slices longer than kResidentN from rank_keys' keys.
constexpr int kMaxBoundGroups = (int)(kResidentN / kBoundGroup);  // 4096: four groups per thread
constexpr float kBoundMargin = 1e-3f;  // slack on U for the rounding of its arithmetic
// The long-slice form's groups: 16 positions, from rank_keys' maxima of r(p).
constexpr int kGrp = 16;
constexpr int kMaxGroups = (int)(kResidentN / kGrp);  // 2048
constexpr int kMaxPasses = 8;  // candidate passes: a group's positions 4 to a lane, 32 keys a thread

static_assert(kMaxBoundGroups == 4 * kSelThreads, "four bound groups per thread");
static_assert(kMaxBoundGroups / (kSelThreads / (kBoundGroup / 4)) == kMaxPasses &&
                  kMaxGroups / (kSelThreads / (kGrp / 4)) == kMaxPasses,
              "32 keys per thread");

struct PrunedSmem {
  uint32_t hist[kBins];
  uint32_t scan_scratch[2 * kSelWaves];
  uint32_t sel_digit, sel_above, sel_count, n_cand;
  uint32_t kgrp[kMaxBoundGroups / 32];  // mixed-cache ranking: the groups holding a fetched position
  float lse2[kFusedG];
  uint32_t n_grp;
  uint16_t grp[kMaxBoundGroups];  // candidate groups, ascending
  uint32_t cand[kCand];
};

struct PrunedRank {
  const float* logits;  // [slices][G][N], log2 units
  const float* part_m;  // [slices][G][S]
  const float* part_l;
  const float* gmax;    // [slices][G][N / kBoundGroup], log2 units
  int G, S;
  // Ranking by the mixed cache: the fetched positions ([slices][n_kappa]), whose logits are the
  // 16-bit ones written after the bounds were taken from the low-bit ones; null otherwise.
  const int32_t* kappa;
  int n_kappa;
};

// The long-slice form (KEYS): slices longer than one selection workgroup holds, from rank_keys'
// keys, their global histogram and their maxima over every 16 positions.  The histogram gives
// the coarse bin of the k-th largest key; a key lies in that bin or a higher one exactly when
// its own bin does (the bins are non-decreasing in the key), so only the groups whose maximum
// reaches the bin are read (about k of them) and the selection among their keys is the same.
// More than kMaxGroups such groups (a crowded threshold bin, or k near kMaxGroups): the sweeps
// over every key instead, in the same workgroup's LDS.
struct GroupedSmem {
  uint32_t hist[kBins];
  uint32_t scan_scratch[2 * kSelWaves];
  uint32_t sel_digit, sel_above, sel_count, n_cand;
  uint32_t grp[kMaxGroups];  // candidate groups, ascending (indices past 65535 at long slices)
  uint32_t cand[kCand];
};
union KeyedSmem {
  GroupedSmem g;
  SelectSmem s;  // the sweeps' layout, once the grouped form has given up
};
constexpr int kKmaxPre = 8;  // group maxima a thread loads before the histogram is read (128K: all)

struct KeyGroups {
  const float* rkey;      // [slices][N]: r(p)
  const float* kmax;      // [slices][N / 16]: their maxima over every 16 positions
  const uint32_t* ghist;  // [slices][kBins]: their coarse histogram
};

template <int D, bool KEYS>
__global__ __launch_bounds__(kSelThreads) void rank_select_pruned_kernel(int64_t N, int k, float r_lo,
                                                                         int32_t* __restrict__ idx_out,
                                                                         unsigned n_sel, MergeJob mj, PrunedRank pr,
                                                                         KeyGroups kg) {
  if (blockIdx.x >= n_sel) {  // a merge workgroup: one query row per wave
    const int64_t row = (int64_t)(blockIdx.x - n_sel) * kSelWaves + (threadIdx.x >> 6);
    if (row < mj.rows) merge_row_wave<D>(mj.part_ml, mj.part_acc, mj.S, mj.out16, row);
    return;
  }
  __shared__ std::conditional_t<KEYS, KeyedSmem, PrunedSmem> smem;
  __shared__ float sweep_vals[2];
  auto& sm = [&]() -> auto& {
    if constexpr (KEYS) return smem.g;
    else return smem;
  }();
  // positions per group: 8 (the split kernels' bounds) or 16 (rank_keys' maxima); a group's
  // positions are read 4 to a lane, LPG lanes a group, PASS groups a pass
  constexpr int GS = KEYS ? kGrp : kBoundGroup, LPG = GS / 4, PASS = kSelThreads / LPG;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6, ql = t % LPG, gj = t / LPG;
  const int64_t slice = blockIdx.x;
  int ph = 0;  // the block scans' scratch set
  // the candidates' keys: pass s (PASS groups; lane ql of a group holds its positions
  // 4 ql .. 4 ql + 3) in v[4s .. 4s + 3] for group grp_of[s] (-1 for none: keys -inf); passes
  // then threads in position order
  float v[4 * kMaxPasses];
  int grp_of[kMaxPasses];
  int n_pass;
  uint32_t bin, above, in_bin;  // the k-th key's coarse bin, the keys above it and in it
  if constexpr (!KEYS) {
    const int G = pr.G, S = pr.S;
    const int ngrp = (int)(N / GS);  // N is a multiple of 32 and at most kResidentN: ngrp % 4 == 0

    // the bounds of groups 4t .. 4t + 3 (a float4 per head) and the first split statistics are
    // loaded before anything waits
    float4 gm[kFusedG];
    {
      const float* gp = pr.gmax + slice * G * ngrp;
      const int i0 = 4 * t < ngrp ? 4 * t : 0;
#pragma unroll
      for (int g = 0; g < kFusedG; ++g) gm[g] = *reinterpret_cast<const float4*>(gp + (g < G ? g : 0) * ngrp + i0);
    }
    const int hw = wave < G ? wave : 0;
    const int64_t sb = (slice * G + hw) * S;
    const int j0 = (lane & 15) < S ? (lane & 15) : 0;
    const float m_first = pr.part_m[sb + j0], l_first = pr.part_l[sb + j0];
    // ranking by the mixed cache: a group that holds a fetched position is a candidate whatever
    // its bounds say (its logit there is a 16-bit one, taken after them), and gives no L
    const bool mixed = pr.kappa != nullptr;  // uniform
    const int32_t* kp = mixed ? pr.kappa + slice * pr.n_kappa : nullptr;
    const int32_t kp0 = mixed && t < pr.n_kappa ? kp[t] : -1;
    asm volatile("" ::: "memory");
    sm.hist[t] = 0u;
    sm.hist[t + kSelThreads] = 0u;
    if (t < kMaxBoundGroups / 32) sm.kgrp[t] = 0u;
    if (wave < kFusedG) {
      const float l2 = head_lse2_row(pr.part_m + sb, pr.part_l + sb, S, lane & 15, m_first, l_first);
      if (wave < G && lane == 0) sm.lse2[wave] = l2;
    }
    if (t == 0) {
      sm.n_cand = 0u;
    }
    __syncthreads();
    if (mixed) {
      auto mark = [&](int32_t p) {
        if (p >= 0 && p < N) atomicOr(&sm.kgrp[p / (32 * GS)], 1u << ((p / GS) & 31));
      };
      mark(kp0);
      for (int i = t + kSelThreads; i < pr.n_kappa; i += kSelThreads) mark(kp[i]);
      __syncthreads();
    }
    float lse2[kFusedG];
#pragma unroll
    for (int g = 0; g < kFusedG; ++g) lse2[g] = g < G ? sm.lse2[g] : 0.0f;

    // head g's log2-probability bound over group s, and L of the four groups (natural-log units)
    auto lp_of = [&](int s, int g) {
      return (s == 0 ? gm[g].x : (s == 1 ? gm[g].y : (s == 2 ? gm[g].z : gm[g].w))) - lse2[g];
    };
    float L[4], mx2[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      mx2[s] = -INFINITY;
#pragma unroll
      for (int g = 0; g < kFusedG; ++g)
        if (g < G) mx2[s] = fmaxf(mx2[s], lp_of(s, g));
      L[s] = mx2[s] * kLn2 + 0.0f;
    }
    const bool gv = 4 * t < ngrp;  // groups 4t .. 4t + 3, all or none
    const uint32_t kw = mixed ? (sm.kgrp[t >> 3] >> ((4 * t) & 31)) & 15u : 0u;  // their fetched-row bits

    // tau_lo: below the k-th largest L (the lower edge of the coarse bin holding it, one bin down);
    // with fewer than k groups giving an L, no bound (bin 0)
    float tau_lo = -INFINITY;
    if (k <= ngrp) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if (gv && !((kw >> s) & 1u)) atomicAdd(&sm.hist[coarse_bin(L[s], r_lo)], 1u);
      __syncthreads();
      uint32_t bin, above, in_lo;
      pick_digit(sm, ph, kBins, (uint32_t)k, bin, above, in_lo);
      if (bin > 0u) tau_lo = r_lo + (float)(bin - 1u) / kBinScale;
      sm.hist[t] = 0u;
      sm.hist[t + kSelThreads] = 0u;
    }
    // candidate groups, compacted in ascending order.  U >= tau_lo is tested as
    // sum_g 2^(lp_g - t2) >= 1 with t2 = tau_lo in log2 units less the margin: the logarithm and
    // the maximum of U's own arithmetic are not needed for the comparison.  A group whose maxima
    // are all -inf is never a candidate (U is not a number there).
    const float t2 = tau_lo / kLn2 - kBoundMargin / kLn2;
    uint32_t cm = 0u;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bool reach = tau_lo == -INFINITY;
      if (!reach) {
        float sum = 0.0f;
#pragma unroll
        for (int g = 0; g < kFusedG; ++g)
          if (g < G) sum += __builtin_amdgcn_exp2f(lp_of(s, g) - t2);
        reach = sum >= 1.0f;
      }
      cm |= (gv && ((reach && mx2[s] > -INFINITY) || ((kw >> s) & 1u))) ? (1u << s) : 0u;
    }
    {
      uint32_t tot;
      uint32_t off = block_exclusive_scan((uint32_t)__popc(cm), sm.scan_scratch, tot, ph);
#pragma unroll
      for (int s = 0; s < 4; ++s)
        if ((cm >> s) & 1u) sm.grp[off++] = (uint16_t)(4 * t + s);
      if (t == 0) sm.n_grp = tot;
    }
    __syncthreads();
    const uint32_t n_grp = sm.n_grp;

    // r of the candidates' positions, two lanes per group (lane ql = t % 2 holds positions
    // 4 ql .. 4 ql + 3 of the group, so that the two lanes read each head's 32 bytes of the group
    // together): pass s covers candidates PASS s .. PASS s + PASS - 1, candidate PASS s + t / 2 in
    // v[4s .. 4s + 3]; -inf where there is none.  Passes then threads then lanes run in position order.
    const float* lg = pr.logits + slice * G * N;
    n_pass = (int)((n_grp + PASS - 1) / PASS);  // <= kMaxPasses
    uint32_t cur_bin = 0u, cur_cnt = 0u;  // this thread's pending histogram increment
#pragma unroll
    for (int s0 = 0; s0 < kMaxPasses; s0 += 2) {
      if (s0 >= n_pass) {  // uniform: no candidates from here on
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          grp_of[s0 + u] = -1;
#pragma unroll
          for (int e = 0; e < 4; ++e) v[4 * (s0 + u) + e] = -INFINITY;
        }
        continue;
      }
      float4 x[2][kFusedG];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const uint32_t j = (uint32_t)((s0 + u) * PASS + gj);
        grp_of[s0 + u] = j < n_grp ? (int)sm.grp[j] : -1;
        const int c = grp_of[s0 + u] >= 0 ? grp_of[s0 + u] : 0;  // a valid address, unused
#pragma unroll
        for (int g = 0; g < kFusedG; ++g)
          x[u][g] = *reinterpret_cast<const float4*>(lg + (int64_t)(g < G ? g : 0) * N + GS * c + 4 * ql);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float r = -INFINITY;
          if (grp_of[s0 + u] >= 0) {
            r = rank_of<kFusedG>(x[u], e, lse2, G);
            const uint32_t b = coarse_bin(r, r_lo);
            if (cur_cnt != 0u && b != cur_bin) atomicAdd(&sm.hist[cur_bin], cur_cnt), cur_cnt = 0u;
            cur_bin = b;
            ++cur_cnt;
          }
          v[4 * (s0 + u) + e] = r;
        }
    }
    if (cur_cnt) atomicAdd(&sm.hist[cur_bin], cur_cnt);
    __syncthreads();

    // the exact threshold among the candidates, as the resident selection finds it
    pick_digit(sm, ph, kBins, (uint32_t)k, bin, above, in_bin);
  } else {
    // thread t looks at groups [g0, g1) = [t per, (t + 1) per); their maxima are loaded together
    // with the histogram when they fit in registers
    const int64_t ngrp = N / GS;
    const float* gx = kg.kmax + slice * ngrp;
    const int64_t per = (ngrp + kSelThreads - 1) / kSelThreads;
    const int64_t g0 = (int64_t)t * per, g1 = g0 + per < ngrp ? g0 + per : ngrp;
    const bool pre = per <= kKmaxPre;  // uniform
    float gk[kKmaxPre];
#pragma unroll
    for (int i = 0; i < kKmaxPre; ++i) gk[i] = pre && g0 + i < g1 ? gx[g0 + i] : 0.0f;
    const uint32_t* gh = kg.ghist + slice * kBins;
    for (int i = t; i < kBins; i += kSelThreads) sm.hist[i] = gh[i];
    if (t == 0) sm.n_cand = 0u;
    __syncthreads();
    pick_digit(sm, ph, kBins, (uint32_t)k, bin, above, in_bin);

    // candidate groups, compacted in ascending order: a key is in the threshold bin or a higher
    // one exactly when its bin is, so a group that holds one has its maximum there too
    auto reaches = [&](float m) { return coarse_bin(m, r_lo) >= bin; };
    uint32_t mine = 0u;
    if (pre) {
#pragma unroll
      for (int i = 0; i < kKmaxPre; ++i) mine += g0 + i < g1 && reaches(gk[i]) ? 1u : 0u;
    } else {
      for (int64_t g = g0; g < g1; ++g) mine += reaches(gx[g]) ? 1u : 0u;
    }
    uint32_t n_grp;
    uint32_t off = block_exclusive_scan(mine, sm.scan_scratch, n_grp, ph);
    if (n_grp <= (uint32_t)kMaxGroups && mine != 0u) {
      if (pre) {
#pragma unroll
        for (int i = 0; i < kKmaxPre; ++i)
          if (g0 + i < g1 && reaches(gk[i])) sm.grp[off++] = (uint32_t)(g0 + i);
      } else {
        for (int64_t g = g0; g < g1; ++g)
          if (reaches(gx[g])) sm.grp[off++] = (uint32_t)g;
      }
    }
    if (n_grp > (uint32_t)kMaxGroups) {  // uniform
      __syncthreads();  // this form's LDS becomes the sweeps'
      select_by_sweeps(smem.s, sweep_vals, kg.rkey, kg.ghist, N, k, r_lo, idx_out, slice);
      return;
    }
    __syncthreads();

    // the candidates' keys, four lanes a group: pass s covers candidates PASS s .. PASS s + 255
    const float* ky = kg.rkey + slice * N;
    n_pass = (int)((n_grp + PASS - 1) / PASS);  // <= kMaxPasses
#pragma unroll
    for (int s = 0; s < kMaxPasses; ++s) {
      const uint32_t j = (uint32_t)(s * PASS + gj);
      grp_of[s] = s < n_pass && j < n_grp ? (int)sm.grp[j] : -1;
      float4 x = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      if (grp_of[s] >= 0) x = *reinterpret_cast<const float4*>(ky + (int64_t)GS * grp_of[s] + 4 * ql);
      v[4 * s] = x.x;
      v[4 * s + 1] = x.y;
      v[4 * s + 2] = x.z;
      v[4 * s + 3] = x.w;
    }
  }
  auto valid = [&](int i) { return grp_of[i >> 2] >= 0; };

  uint32_t thr, need_eq, n_thr;
  if (in_bin <= (uint32_t)kCand) {
    // the passes past n_pass hold no candidates: their keys are skipped by a uniform branch
    uint32_t mine = 0u;
#pragma unroll
    for (int s = 0; s < kMaxPasses; ++s) {
      if (s >= n_pass) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * s + e;
        const float x = v[i];
        mine |= (valid(i) && coarse_bin(x, r_lo) == bin) ? (1u << i) : 0u;
      }
    }
    if (__any(mine != 0u)) {
      const uint32_t n = __popc(mine);
      const uint32_t incl = wave_inclusive_scan(n);
      uint32_t base_slot = 0u;
      if (lane == 63) base_slot = atomicAdd(&sm.n_cand, incl);
      base_slot = __shfl(base_slot, 63);
      uint32_t slot = base_slot + incl - n;
#pragma unroll
      for (int s = 0; s < kMaxPasses; ++s) {
        if (s >= n_pass) continue;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if ((mine >> (4 * s + e)) & 1u) {
            if (slot < (uint32_t)kCand) sm.cand[slot] = order_key(v[4 * s + e]);
            ++slot;
          }
      }
    }
    __syncthreads();
    const uint32_t nc = sm.n_cand < (uint32_t)kCand ? sm.n_cand : (uint32_t)kCand;
    const uint32_t krem = (uint32_t)k - above;
    // at most 64 keys in the bin: every wave finds the exact threshold among them itself (the same
    // keys, so the same answer in every wave), which saves a barrier to publish it
    bool found = false;
    if (nc <= 64u) {
      const uint32_t c = (uint32_t)lane < nc ? sm.cand[lane] : 0u;
      const uint32_t gt_eq = count_above_equal(c, nc);
      const uint32_t gt = gt_eq & 0xffffu, eq = gt_eq >> 16;
      const uint64_t m = __ballot((uint32_t)lane < nc && gt < krem && krem <= gt + eq);
      if (m != 0u) {
        const int src = __builtin_ctzll(m);
        thr = __builtin_amdgcn_readlane(c, src);
        need_eq = krem - __builtin_amdgcn_readlane(gt, src);
        n_thr = __builtin_amdgcn_readlane(eq, src);
        found = true;
      }
    }
    if (!found) {
      radix_select(sm, ph, krem,
                   [&](int shift, int nbins, uint32_t prefix, uint32_t mask) {
                     for (uint32_t i = t; i < nc; i += kSelThreads) {
                       const uint32_t u = sm.cand[i];
                       if ((u & mask) == prefix) atomicAdd(&sm.hist[(u >> shift) & (uint32_t)(nbins - 1)], 1u);
                     }
                   },
                   thr, need_eq, n_thr);
    }
  } else {
    radix_select(sm, ph, (uint32_t)k,
                 [&](int shift, int nbins, uint32_t prefix, uint32_t mask) {
#pragma unroll
                   for (int i = 0; i < 4 * kMaxPasses; ++i) {
                     const uint32_t u = order_key(v[i]);
                     if (valid(i) && (u & mask) == prefix) atomicAdd(&sm.hist[(u >> shift) & (uint32_t)(nbins - 1)], 1u);
                   }
                 },
                 thr, need_eq, n_thr);
  }

  // Every key above thr and the first need_eq equal to it, in position order (pass, then thread,
  // then lane bit).  Per pass a thread has at most 4 such keys; the prefix sums run over two
  // passes at once, one 16-bit field each (a pass holds at most 4096 keys).
  const float vthr = key_value(thr);
  const bool all_eq = need_eq == n_thr;
  uint32_t sel[kMaxPasses], eqm[kMaxPasses];
#pragma unroll
  for (int s = 0; s < kMaxPasses; ++s) {
    sel[s] = 0u;
    eqm[s] = 0u;
    if (s >= n_pass) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (valid(4 * s + e)) {
        const float x = v[4 * s + e];
        sel[s] |= (x > vthr || (all_eq && x == vthr)) ? (1u << e) : 0u;
        eqm[s] |= (!all_eq && x == vthr) ? (1u << e) : 0u;
      }
  }
  // exclusive prefix over (pass, thread) of per-pass counts: cnt(s) -> before(s)
  auto pass_prefix = [&](const uint32_t (&m)[kMaxPasses], uint32_t (&before)[kMaxPasses]) {
    uint32_t carried = 0u;
#pragma unroll
    for (int s = 0; s < kMaxPasses; s += 2) {
      if (s >= n_pass) {  // uniform: nothing from here on
        before[s] = carried;
        before[s + 1] = carried;
        continue;
      }
      uint32_t tot;
      const uint32_t packed = (uint32_t)__popc(m[s]) | ((uint32_t)__popc(m[s + 1]) << 16);
      const uint32_t ex = block_exclusive_scan(packed, sm.scan_scratch, tot, ph);
      before[s] = carried + (ex & 0xffffu);
      before[s + 1] = carried + (tot & 0xffffu) + (ex >> 16);
      carried += (tot & 0xffffu) + (tot >> 16);
    }
  };
  if (!all_eq) {
    uint32_t before[kMaxPasses];
    pass_prefix(eqm, before);
#pragma unroll
    for (int s = 0; s < kMaxPasses; ++s) {
      if (s >= n_pass) continue;
      const uint32_t ne = __popc(eqm[s]);
      uint32_t take = before[s] >= need_eq ? 0u : (need_eq - before[s] < ne ? need_eq - before[s] : ne);
      while (take > 0u) {  // the lowest equal positions first
        const uint32_t low = eqm[s] & (0u - eqm[s]);
        sel[s] |= low;
        eqm[s] ^= low;
        --take;
      }
    }
  }
  uint32_t out0[kMaxPasses];
  pass_prefix(sel, out0);
#pragma unroll
  for (int s = 0; s < kMaxPasses; ++s) {
    if (s >= n_pass) continue;
    uint32_t m = sel[s], out = out0[s];
    while (m != 0u) {
      const int b = __builtin_ctz(m);
      m &= m - 1u;
      if (out < (uint32_t)k) idx_out[slice * k + out] = (int32_t)(GS * grp_of[s] + 4 * ql + b);
      ++out;
    }
  }
}

template <int GM>
void launch_keys(const Dims& d, int S, const float* logits, const float* part_m, const float* part_l, float r_lo,
                 float* keys, uint32_t* hist, float* kmax, hipStream_t s) {
  const dim3 grid((unsigned)ceil_div(d.N, kKeyChunk), (unsigned)d.slices());
  rank_keys_kernel<GM><<<grid, kKeyThreads, 0, s>>>(logits, part_m, part_l, d.G, S, d.N, r_lo, keys, hist, kmax);
}

template <int D>
void launch_select(const Dims& d, int k, float r_lo, const float* keys, const uint32_t* hist, const float* kmax,
                   int32_t* idx_out, const MergeJob& mj, const FusedRank* fr, hipStream_t s) {
  const unsigned n_sel = (unsigned)d.slices();
  const unsigned grid = n_sel + (unsigned)ceil_div(mj.rows, kSelWaves);
  const FusedRank none{nullptr, nullptr, nullptr, 0, 0, nullptr};
  if (fr)
    rank_select_resident_kernel<D, true><<<grid, kSelThreads, 0, s>>>(nullptr, nullptr, d.N, k, r_lo, idx_out,
                                                                      n_sel, mj, *fr);
  else if (d.N <= kResidentN)
    rank_select_resident_kernel<D, false><<<grid, kSelThreads, 0, s>>>(keys, hist, d.N, k, r_lo, idx_out, n_sel,
                                                                       mj, none);
  else
    rank_select_pruned_kernel<D, true><<<grid, kSelThreads, 0, s>>>(d.N, k, r_lo, idx_out, n_sel, mj, PrunedRank{},
                                                                   KeyGroups{keys, kmax, hist});
}

}  // namespace

bool rank_select_prunable(const Dims& d, int k) {
  return d.N <= kResidentN && d.G <= kFusedG && k <= d.N / kBoundGroup;
}

hipError_t launch_rank_select(const Dims& d, int S, const float* logits, const float* part_m,
                              const float* part_l, int k, float* keys, bool keys_wanted, uint32_t* hist,
                              int32_t* idx_out, const MergeJob* merge, hipStream_t s, const float* gmax,
                              const int32_t* kappa, int n_kappa, float* kmax) {
  const float r_lo = logf((float)d.G) - kBinSpan;  // the same value for both kernels
  const MergeJob none{nullptr, nullptr, 0, 0, nullptr};
  const MergeJob& mj = merge ? *merge : none;
  if (gmax && !keys_wanted && rank_select_prunable(d, k)) {
    const PrunedRank pr{logits, part_m, part_l, gmax, d.G, S, n_kappa > 0 ? kappa : nullptr, n_kappa};
    const unsigned n_sel = (unsigned)d.slices();
    const unsigned grid = n_sel + (unsigned)ceil_div(mj.rows, kSelWaves);
    if (d.D == 64)
      rank_select_pruned_kernel<64, false><<<grid, kSelThreads, 0, s>>>(d.N, k, r_lo, idx_out, n_sel, mj, pr, KeyGroups{});
    else
      rank_select_pruned_kernel<128, false><<<grid, kSelThreads, 0, s>>>(d.N, k, r_lo, idx_out, n_sel, mj, pr,
                                                                         KeyGroups{});
    return hipGetLastError();
  }
  if (d.N <= kResidentN && d.G <= kFusedG) {  // one launch: the selection forms r(p) itself
    const FusedRank fr{logits, part_m, part_l, d.G, S, keys_wanted ? keys : nullptr};
    if (d.D == 64)
      launch_select<64>(d, k, r_lo, nullptr, nullptr, nullptr, idx_out, mj, &fr, s);
    else
      launch_select<128>(d, k, r_lo, nullptr, nullptr, nullptr, idx_out, mj, &fr, s);
    return hipGetLastError();
  }
  if (d.G <= 4)
    launch_keys<4>(d, S, logits, part_m, part_l, r_lo, keys, hist, kmax, s);
  else if (d.G <= 8)
    launch_keys<8>(d, S, logits, part_m, part_l, r_lo, keys, hist, kmax, s);
  else
    launch_keys<16>(d, S, logits, part_m, part_l, r_lo, keys, hist, kmax, s);
  if (d.D == 64)
    launch_select<64>(d, k, r_lo, keys, hist, kmax, idx_out, mj, nullptr, s);
  else
    launch_select<128>(d, k, r_lo, keys, hist, kmax, idx_out, mj, nullptr, s);
  return hipGetLastError();
}

}  // namespace specache
