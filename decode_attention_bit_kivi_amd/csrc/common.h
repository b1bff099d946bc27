// Shared definitions of libspecache's HIP sources (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

namespace specache {

constexpr int kGroup = 32;        // code block: 32 tokens (the smaller quantization group)
constexpr int kMaxRows = 16;      // G * T query rows per KV head handled by one workgroup
constexpr int kMaxTail = 64;
// The runtime only accepts a compute-unit mask that leaves at least one unit on
// every accelerator complex die (8 on MI355X); the low mask bits interleave over them.
constexpr int kMinGatherCUs = 8;
constexpr int64_t kMaxAttnSeqLen = int64_t(4096) * 1024;  // 1024 splits of at most 4096 positions

// Problem dimensions after validation.
struct Dims {
  int B, Hq, Hkv, D, bits, G, W;
  int vbits;         // bits of the value codes (bits: of the key codes)
  int group;         // quantization group: 32 or 64 (key tokens, value channels)
  int64_t N, nblk;   // positions and 32-position blocks per slice (the cache's current length)
  int64_t Ns;        // positions per slice the cache buffers are laid out for (>= N)
  int64_t slices() const { return (int64_t)B * Hkv; }
};

// Bit i of a packed word stands for element 2*(i mod 16) + (i div 16):
// even elements in the low half-word, odd elements in the high half-word.
__host__ __device__ __forceinline__ int bit_to_elem(int i) { return 2 * (i & 15) + (i >> 4); }
__host__ __device__ __forceinline__ int elem_to_bit(int e) { return (e >> 1) + ((e & 1) << 4); }

__host__ __device__ __forceinline__ int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
__host__ __device__ __forceinline__ int64_t ceil_div(int64_t x, int64_t m) { return (x + m - 1) / m; }

// ---- split plans (pure functions of the shape; used for workspace sizing and launch) ----

struct ScorePlan {
  int64_t L;       // positions per split (multiple of 128)
  int S;           // splits per slice
};

inline ScorePlan score_plan(const Dims& d) {
  const int64_t target = 2048;  // workgroups to aim for
  int64_t L = ceil_div(d.N * d.slices(), target);
  L = round_up(L, 128);
  if (L < 128) L = 128;
  if (L > 4096) L = 4096;
  ScorePlan p;
  p.L = L;
  p.S = (int)ceil_div(d.N, L);
  return p;
}

struct AttnPlan {
  int64_t L;       // positions per split (a multiple of 32, at most 4096)
  int S;           // splits per slice; a split also handles the fetched rows of its
                   // positions, and the last split handles the tail
};

constexpr int kPlanMaxCUs = 256;     // compute units the attention plans are sized for at most
constexpr int kAttnWGsPerCU = 2;     // resident workgroups per compute unit: general attention kernels
constexpr int kStreamWGsPerCU = 3;   // the same for the streamed split kernel (attention_stream.hip)
constexpr int kAttnMaxBlocks = 256;  // 32-position blocks per split (the kernel's kappa bitmask)
constexpr int kAttnMaxSplits = 1024; // splits per slice (the merge kernel's weight table)

inline int64_t attn_min_splits(const Dims& d) { return ceil_div(d.nblk, kAttnMaxBlocks); }

// Most splits per slice any compute-unit count may get: about four rounds of kAttnWGsPerCU
// workgroups on kPlanMaxCUs units (over two rounds of the streamed kernel's).  The workspace is
// sized for it.
inline int64_t attn_max_splits(const Dims& d) {
  int64_t cap = ceil_div(int64_t(4) * kPlanMaxCUs * kAttnWGsPerCU, d.slices());
  if (cap > d.nblk) cap = d.nblk;
  if (cap < attn_min_splits(d)) cap = attn_min_splits(d);
  if (cap > kAttnMaxSplits) cap = kAttnMaxSplits;
  return cap;
}

inline AttnPlan attn_plan_splits(const Dims& d, int64_t S) {
  AttnPlan p;
  p.L = 32 * ceil_div(d.nblk, S);
  p.S = (int)ceil_div(d.N, p.L);
  return p;
}

// Splits per slice for `cus` compute units holding `wgs_per_cu` workgroups each: the fewest
// splits whose estimated time is within 3% of the best.  The estimate of S splits is (rounds of
// the slices * S workgroups over the resident slots) x (blocks of the busiest of a workgroup's
// four waves).  The workgroups are spread evenly over the 8 dies and the 4 shader engines of
// each, and a stream's units (its CU mask interleaves over the dies) can leave some engines a
// unit short, so the slots are counted at floor(cus / 32) units per engine: 704 workgroups on
// 240 units at three a unit ran in two rounds (11 splits per slice of a 32K layer of 64 slices:
// 64 us, against 51 us for 10 splits).
inline AttnPlan attn_plan(const Dims& d, int cus, int wgs_per_cu) {
  if (cus < 8) cus = 8;
  if (cus > kPlanMaxCUs) cus = kPlanMaxCUs;
  const int64_t usable = cus >= 32 ? 32 * (cus / 32) : cus;
  const int64_t slots = usable * wgs_per_cu;
  const int64_t lo = attn_min_splits(d), hi = attn_max_splits(d);
  int64_t best = INT64_MAX;
  int64_t cost[kAttnMaxSplits + 1];
  for (int64_t S = lo; S <= hi; ++S) {
    const int64_t bps = ceil_div(d.nblk, S);
    const int64_t used = ceil_div(d.nblk, bps);
    cost[S] = ceil_div(d.slices() * used, slots) * ceil_div(bps, 4);
    if (cost[S] < best) best = cost[S];
  }
  int64_t pick = hi;
  for (int64_t S = lo; S <= hi; ++S)
    if (100 * cost[S] <= 103 * best) {
      pick = S;
      break;
    }
#ifdef SPECACHE_TUNING  // experiments only: force the split count
  if (const char* e = getenv("SPECACHE_ATTN_SPLITS")) {
    const int64_t f = atoll(e);
    if (f >= lo && f <= hi) pick = f;
  }
#endif
  return attn_plan_splits(d, pick);
}

// ---- launchers (defined in the .hip files) ----

// Quantizes nblocks 32-position blocks per slice of k16 / v16 ([slices][src_len][D]) into cache
// blocks blk0 .. blk0 + nblocks - 1.
hipError_t launch_quantize(const Dims& d, const _Float16* k16, const _Float16* v16, int64_t src_len, int64_t blk0,
                           int64_t nblocks, uint32_t* k_codes, _Float16* k_meta, uint32_t* v_codes,
                           _Float16* v_meta, hipStream_t s);

// Also zeroes `hist` ([slices][2048]) for the rank kernels that follow on the same stream.
hipError_t launch_score(const Dims& d, const ScorePlan& plan, const _Float16* q16, int n_tokens,
                        int rank_row, const uint32_t* k_codes, const _Float16* k_meta, float sm_scale,
                        float* logits, float* part_m, float* part_l, uint32_t* hist, hipStream_t s);

// The attention's split merge, run by extra workgroups of the selection launch (they use the
// compute units the per-slice selection leaves idle).
struct MergeJob {
  const float* part_ml;   // [rows][S][2]
  const float* part_acc;  // [rows][S][D]
  int S;
  int64_t rows;
  _Float16* out16;        // [rows][D]
};

// part_m / part_l: [slices][G][S] per-split (max, sum 2^(x - max)) of the logits, log2 units.
// merge: null, or the attention merge to run alongside the selection.  keys: where r(p) goes
// (the caller's output when keys_wanted, else workspace a slice too large for one workgroup's
// registers uses between its two kernels).
// gmax: null, or the per-group logit maxima the split kernel wrote (rank_gmax); with them,
// and no keys wanted, a slice of at most 32768 positions is selected from the logits of the
// position groups whose bound reaches the k-th rank only.  kappa / n_kappa: for the ranking by the
// mixed cache, the fetched positions ([slices][n_kappa]) whose 16-bit logits replaced the
// low-bit ones after the maxima were taken (their groups are always read); else null / 0.
// kmax: [slices][N / 16] floats of workspace for the maxima of r(p) over every 16 positions,
// written by the two-launch form (rank_keys) for its selection to read only the groups that
// reach the threshold bin.
hipError_t launch_rank_select(const Dims& d, int S, const float* logits, const float* part_m,
                              const float* part_l, int k, float* keys, bool keys_wanted, uint32_t* hist,
                              int32_t* idx_out, const MergeJob* merge, hipStream_t s, const float* gmax,
                              const int32_t* kappa, int n_kappa, float* kmax);

// Positions per bound group: rank_gmax holds, per head, the maximum of the rank row's logits over
// every kBoundGroup consecutive positions, which the pruned selection reads.
constexpr int kBoundGroup = 8;

// Whether the pruned selection (per-group bounds) serves this problem: slices of at most 32768
// positions, at most 4 heads per KV head, k at most one per group.
bool rank_select_prunable(const Dims& d, int k);

// skip_negative: rows with a negative index are left untouched (resident-set reuse).
hipError_t launch_gather(const Dims& d, const int32_t* idx, int k, const _Float16* k_src,
                         const _Float16* v_src, _Float16* k_sel, _Float16* v_sel, bool skip_negative,
                         hipStream_t s);

hipError_t launch_reuse(const Dims& d, const int32_t* idx, int k, const int32_t* idx_prev, int k_prev,
                        const _Float16* k_prev_rows, const _Float16* v_prev_rows, _Float16* k_sel, _Float16* v_sel,
                        int32_t* fetch_idx, hipStream_t s);

struct AttnArgs {
  const _Float16* q16;
  int T;
  const uint32_t* k_codes;
  const _Float16* k_meta;
  const uint32_t* v_codes;
  const _Float16* v_meta;
  int64_t seq_stride;  // positions per slice the low-bit cache is laid out for
  int group;           // quantization group (32 or 64)
  const int32_t* idx;
  int k;
  const _Float16* k_sel;
  const _Float16* v_sel;
  const _Float16* k_tail;
  const _Float16* v_tail;
  int tail;
  float sm_scale;
  _Float16* out16;
  float* part_ml;    // [B][Hq][T][S][2]  (running max in log2 units, sum of exp2)
  float* part_acc;   // [B][Hq][T][S][D]
  // Ranking outputs of the fused step (all null / unused for plain attention):
  int rank_row;
  int rank_mixed;        // 0: rank against C'; 1: rank by the row of the mixed-cache attention
  float* rank_logits;    // [slices][G][N]: the rank row's logits (log2 units)
  float* rank_m;         // [slices][G][S]: per-split max of its softmax (log2 units)
  float* rank_l;         // [slices][G][S]: per-split sum of 2^(x - max)
  uint32_t* rank_hist;   // [slices][2048]: zeroed by the split kernel for the rank kernels
  // optional (null: not written; only with G * T <= 8): per head, the maximum of the rank row's
  // logits over every kBoundGroup consecutive positions, [slices][G][N / kBoundGroup], log2 units
  // (ranking by the mixed cache: the low-bit logits, before the fetched rows' replace them)
  float* rank_gmax;
};

// Split kernel of the attention; with a.rank_logits set it also emits the ranking logits and
// statistics of the rank row: against C' (rank_mixed = 0), or those of the attention itself
// over C' with the fetched rows substituted and the visible tail (rank_mixed = 1).
hipError_t launch_attn_split(const Dims& d, const AttnPlan& plan, const AttnArgs& a, hipStream_t s);
hipError_t launch_attn_merge(const Dims& d, const AttnPlan& plan, const AttnArgs& a, hipStream_t s);
// The split kernel that streams the low-bit cache through LDS (attention_stream.hip), for head_dim
// 128, 1-bit key and value codes and G * T <= 8; launch_attn_split uses it whenever it serves, with
// the same plan and outputs.
bool attn_stream_serves(const Dims& d, const AttnArgs& a);
// Resident workgroups per compute unit of the split kernel that serves these arguments.
inline int attn_split_wgs_per_cu(const Dims& d, const AttnArgs& a) {
  return attn_stream_serves(d, a) ? kStreamWGsPerCU : kAttnWGsPerCU;
}
hipError_t launch_attn_stream(const Dims& d, const AttnPlan& plan, const AttnArgs& a, hipStream_t s);
// The same kernel as a score pass (score_topk): the rank row's logits against C' into
// a.rank_logits, its per-split statistics into a.rank_m / a.rank_l and the zeroed histogram
// (a.rank_hist); a.k = 0, a.tail = 0, no attention output.  Serves what attn_stream_serves does.
hipError_t launch_score_stream(const Dims& d, const AttnPlan& plan, const AttnArgs& a, hipStream_t s);
// The 16-bit comparator's split kernel: a.k_sel / a.v_sel are the whole 16-bit cache, a.k its
// positions per slice; partials as launch_attn_split's, merged by launch_attn_merge.
hipError_t launch_attn16_split(const Dims& d, const AttnPlan& plan, const AttnArgs& a, hipStream_t s);

}  // namespace specache
