// The C ABI declared in include/specache.h: argument validation on the host,
// workspace carving, and dispatch to the kernel launchers.  Nothing here
// allocates memory; the only state is the per-device address of the
// no-allocation decode step's static scratch array.
#include <algorithm>
#include <cstring>
#include <mutex>

#include "../../include/specache.h"
#include "common.h"

using namespace specache;

namespace {

bool make_dims(const specache_shape* s, Dims* d, int* err) {
  *err = SPECACHE_OK;
  if (!s) {
    *err = SPECACHE_ERR_INVALID;
    return false;
  }
  const int64_t cap = s->seq_capacity ? s->seq_capacity : s->seq_len;
  if (s->batch <= 0 || s->n_q_heads <= 0 || s->n_kv_heads <= 0 || s->head_dim <= 0 || s->seq_len <= 0 ||
      s->n_q_heads % s->n_kv_heads != 0 || s->seq_len % kGroup != 0 || s->batch > 65535 ||
      (int64_t)s->batch * s->n_kv_heads > 65535 || cap < s->seq_len || cap % kGroup != 0 ||
      (s->group == 64 && (s->seq_len % 64 != 0 || cap % 64 != 0)) ||
      cap > (int64_t(1) << 31) - 1) {
    *err = SPECACHE_ERR_INVALID;
    return false;
  }
  const int vbits = s->v_bits ? s->v_bits : s->bits;
  if ((s->bits != 1 && s->bits != 2) || (vbits != 1 && vbits != 2)) {
    *err = SPECACHE_ERR_INVALID;
    return false;
  }
  if ((s->group != 32 && s->group != 64) || (s->head_dim != 64 && s->head_dim != 128) ||
      s->n_q_heads / s->n_kv_heads > kMaxRows) {
    *err = SPECACHE_ERR_UNSUPPORTED;
    return false;
  }
  d->B = s->batch;
  d->Hq = s->n_q_heads;
  d->Hkv = s->n_kv_heads;
  d->D = s->head_dim;
  d->bits = s->bits;
  d->vbits = vbits;
  d->group = s->group;
  d->G = s->n_q_heads / s->n_kv_heads;
  d->W = s->head_dim / 32;
  d->N = s->seq_len;
  d->nblk = s->seq_len / kGroup;
  d->Ns = cap;
  return true;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct ScoreWs {
  size_t logits, part_m, part_l, keys, hist, kmax, gmax, total;
};

// Split statistics sized for the score kernel's plan or the streamed kernel's, whichever has more
// splits (score_topk runs the streamed kernel's score pass where it serves).
ScoreWs score_ws(const Dims& d, const ScorePlan& p) {
  ScoreWs w;
  const size_t S = (size_t)std::max<int64_t>(p.S, attn_max_splits(d));
  w.logits = 0;
  size_t off = align256(sizeof(float) * (size_t)d.slices() * d.G * d.N);
  w.part_m = off;
  off += align256(sizeof(float) * (size_t)d.slices() * d.G * S);
  w.part_l = off;
  off += align256(sizeof(float) * (size_t)d.slices() * d.G * S);
  w.keys = off;
  off += align256(sizeof(float) * (size_t)d.slices() * d.N);
  w.hist = off;
  off += align256(sizeof(uint32_t) * (size_t)d.slices() * 2048);
  w.kmax = off;  // per-16-position maxima of r(p) (the two-launch selection)
  off += align256(sizeof(float) * (size_t)d.slices() * (d.N / 16));
  w.gmax = off;  // per-group logit maxima of each head (the streamed score pass's bounds)
  off += align256(sizeof(float) * (size_t)d.slices() * d.G * (d.N / kBoundGroup));
  w.total = off;
  return w;
}

struct AttnWs {
  size_t ml, acc, total;
  // fused step only:
  size_t logits, rank_m, rank_l, keys, hist, gmax, total_step;
};

// Sized for attn_max_splits, the most splits any launch plan uses.
AttnWs attn_ws(const Dims& d, int T) {
  AttnWs w;
  const size_t rows = (size_t)d.B * d.Hq * T;
  const size_t S = (size_t)attn_max_splits(d);
  w.ml = 0;
  w.acc = align256(sizeof(float) * rows * S * 2);
  w.total = w.acc + align256(sizeof(float) * rows * S * d.D);
  size_t off = w.total;
  w.logits = off;
  off += align256(sizeof(float) * (size_t)d.slices() * d.G * d.N);
  w.rank_m = off;
  off += align256(sizeof(float) * (size_t)d.slices() * d.G * S);
  w.rank_l = off;
  off += align256(sizeof(float) * (size_t)d.slices() * d.G * S);
  w.keys = off;
  off += align256(sizeof(float) * (size_t)d.slices() * d.N);
  w.hist = off;
  off += align256(sizeof(uint32_t) * (size_t)d.slices() * 2048);
  w.gmax = off;  // per-group logit maxima of the pruned selection, or (two-launch form) the
                 // per-16-position maxima of r(p)
  off += align256(sizeof(float) * (size_t)d.slices() * d.G * (d.N / kBoundGroup));
  w.total_step = off;
  return w;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SPECACHE_OK : SPECACHE_ERR_HIP; }

bool lowbit_ok(const specache_lowbit* c) {
  return c && c->k_codes && c->k_meta && c->v_codes && c->v_meta;
}

// A gather source must be device memory or pinned host memory; returns the
// pointer the device uses, or null.
const void* device_view(const void* p) {
  hipPointerAttribute_t attr;
  std::memset(&attr, 0, sizeof(attr));
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of an unregistered pointer
    return nullptr;
  }
  if (attr.type == hipMemoryTypeDevice) return p;
  if (attr.type == hipMemoryTypeHost) {
    void* dp = nullptr;
    if (hipHostGetDevicePointer(&dp, const_cast<void*>(p), 0) != hipSuccess || dp == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    return dp;
  }
  return nullptr;
}

}  // namespace

namespace {
int stream_cus(hipStream_t s);  // the compute units a stream's kernels may use (below)
}  // namespace

extern "C" {

size_t specache_lowbit_bytes(const specache_shape* shape, size_t* k_codes, size_t* k_meta, size_t* v_codes,
                             size_t* v_meta) {
  Dims d;
  int err;
  if (!make_dims(shape, &d, &err)) return 0;
  const size_t pos = (size_t)d.slices() * d.Ns;  // laid out for the capacity
  const size_t nb = (size_t)d.Ns / kGroup;
  const size_t kc = pos * d.bits * d.W * 4;
  const size_t km = (size_t)d.slices() * (d.Ns / d.group) * 2 * d.D * 2;
  const size_t vc = (size_t)d.slices() * nb * d.vbits * d.D * 4;
  const size_t vm = (size_t)d.slices() * nb * 2 * (d.D / d.group) * 32 * 2;
  if (k_codes) *k_codes = kc;
  if (k_meta) *k_meta = km;
  if (v_codes) *v_codes = vc;
  if (v_meta) *v_meta = vm;
  return kc + km + vc + vm;
}

int specache_quantize_pack(const specache_shape* shape, const void* k16, const void* v16,
                           const specache_lowbit* out, void* stream) {
  Dims d;
  int err;
  if (!make_dims(shape, &d, &err)) return err;
  if (!k16 || !v16 || !lowbit_ok(out)) return SPECACHE_ERR_INVALID;
  return hip_status(launch_quantize(d, static_cast<const _Float16*>(k16), static_cast<const _Float16*>(v16), d.Ns, 0,
                                    d.nblk, static_cast<uint32_t*>(out->k_codes), static_cast<_Float16*>(out->k_meta),
                                    static_cast<uint32_t*>(out->v_codes), static_cast<_Float16*>(out->v_meta),
                                    static_cast<hipStream_t>(stream)));
}

int specache_quantize_append(const specache_shape* shape, const void* k16_new, const void* v16_new, int64_t n_new,
                             const specache_lowbit* cache, void* stream) {
  Dims d;
  int err;
  if (!make_dims(shape, &d, &err)) return err;
  if (n_new < 0 || n_new % d.group != 0 || d.N + n_new > d.Ns) return SPECACHE_ERR_INVALID;
  if (n_new == 0) return SPECACHE_OK;
  if (!k16_new || !v16_new || !lowbit_ok(cache)) return SPECACHE_ERR_INVALID;
  return hip_status(launch_quantize(d, static_cast<const _Float16*>(k16_new), static_cast<const _Float16*>(v16_new),
                                    n_new, d.nblk, n_new / kGroup, static_cast<uint32_t*>(cache->k_codes),
                                    static_cast<_Float16*>(cache->k_meta), static_cast<uint32_t*>(cache->v_codes),
                                    static_cast<_Float16*>(cache->v_meta), static_cast<hipStream_t>(stream)));
}

int specache_offload_fp16(const specache_shape* shape, const void* k16_new, const void* v16_new, int64_t n_new,
                          int64_t pos0, void* k16_dst, void* v16_dst, void* stream) {
  Dims d;
  int err;
  if (!make_dims(shape, &d, &err)) return err;
  if (n_new < 0 || pos0 < 0 || pos0 + n_new > d.Ns) return SPECACHE_ERR_INVALID;
  if (n_new == 0) return SPECACHE_OK;
  if (!k16_new || !v16_new || !k16_dst || !v16_dst) return SPECACHE_ERR_INVALID;
  if (!device_view(k16_dst) || !device_view(v16_dst)) return SPECACHE_ERR_NOT_PINNED;
  const size_t row = (size_t)d.D * sizeof(_Float16);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // one strided copy per tensor: slice b*Hkv+h of the new rows -> positions pos0.. of that slice
  const void* srcs[2] = {k16_new, v16_new};
  void* dsts[2] = {k16_dst, v16_dst};
  for (int t = 0; t < 2; ++t) {
    char* dst = static_cast<char*>(dsts[t]) + (size_t)pos0 * row;
    if (hipMemcpy2DAsync(dst, (size_t)d.Ns * row, srcs[t], (size_t)n_new * row, (size_t)n_new * row,
                         (size_t)d.slices(), hipMemcpyDefault, s) != hipSuccess)
      return SPECACHE_ERR_HIP;
  }
  return SPECACHE_OK;
}

size_t specache_score_topk_workspace_size(const specache_shape* shape, int n_tokens, int k) {
  Dims d;
  int err;
  if (!make_dims(shape, &d, &err) || n_tokens < 1 || n_tokens > 2 || k < 1 || k > d.N) return 0;
  return score_ws(d, score_plan(d)).total;
}

int specache_score_topk(const specache_shape* shape, const void* q16, int n_tokens, int rank_row,
                        const specache_lowbit* cache, float sm_scale, int k, int32_t* idx_out, float* rank_key_out,
                        void* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  int err;
  if (!make_dims(shape, &d, &err)) return err;
  if (n_tokens < 1 || n_tokens > 2 || rank_row < 0 || rank_row >= n_tokens || k < 1 || k > d.N || !q16 ||
      !lowbit_ok(cache) || !idx_out || !(sm_scale > 0.0f) || sm_scale == INFINITY)
    return SPECACHE_ERR_INVALID;
  const ScorePlan plan = score_plan(d);
  const ScoreWs ws = score_ws(d, plan);
  if (!workspace || workspace_bytes < ws.total) return SPECACHE_ERR_WORKSPACE;
  char* base = static_cast<char*>(workspace);
  float* logits = reinterpret_cast<float*>(base + ws.logits);
  float* part_m = reinterpret_cast<float*>(base + ws.part_m);
  float* part_l = reinterpret_cast<float*>(base + ws.part_l);
  float* keys = rank_key_out ? rank_key_out : reinterpret_cast<float*>(base + ws.keys);
  uint32_t* hist = reinterpret_cast<uint32_t*>(base + ws.hist);
  hipStream_t s = static_cast<hipStream_t>(stream);
  // the streamed kernel's score pass where it serves (head_dim 128, 1-bit codes, G * T <= 8),
  // else the score kernel
  AttnArgs sa;
  std::memset(&sa, 0, sizeof(sa));
  sa.q16 = static_cast<const _Float16*>(q16);
  sa.T = n_tokens;
  sa.k_codes = static_cast<const uint32_t*>(cache->k_codes);
  sa.k_meta = static_cast<const _Float16*>(cache->k_meta);
  sa.v_codes = static_cast<const uint32_t*>(cache->v_codes);
  sa.v_meta = static_cast<const _Float16*>(cache->v_meta);
  sa.seq_stride = d.Ns;
  sa.group = d.group;
  sa.sm_scale = sm_scale;
  sa.rank_row = rank_row;
  sa.rank_logits = logits;
  sa.rank_m = part_m;
  sa.rank_l = part_l;
  sa.rank_hist = hist;
  int S = plan.S;
  hipError_t e;
  if (attn_stream_serves(d, sa)) {
    const AttnPlan ap = attn_plan(d, stream_cus(s), kStreamWGsPerCU);
    S = ap.S;
    // with no keys asked for, the bounds for the pruned selection (as in the fused step)
    if (!rank_key_out && rank_select_prunable(d, k)) sa.rank_gmax = reinterpret_cast<float*>(base + ws.gmax);
    e = launch_score_stream(d, ap, sa, s);
  } else {
    e = launch_score(d, plan, static_cast<const _Float16*>(q16), n_tokens, rank_row,
                     static_cast<const uint32_t*>(cache->k_codes), static_cast<const _Float16*>(cache->k_meta),
                     sm_scale, logits, part_m, part_l, hist, s);
  }
  if (e != hipSuccess) return SPECACHE_ERR_HIP;
  e = launch_rank_select(d, S, logits, part_m, part_l, k, keys, rank_key_out != nullptr, hist, idx_out,
                         nullptr, s, sa.rank_gmax, nullptr, 0, reinterpret_cast<float*>(base + ws.kmax));
  return hip_status(e);
}

int specache_gather_fp16(const specache_shape* shape, const int32_t* idx, int k, const void* k16_src,
                         const void* v16_src, void* k_sel, void* v_sel, void* stream) {
  Dims d;
  int err;
  if (!make_dims(shape, &d, &err)) return err;
  if (k < 0 || k > d.N) return SPECACHE_ERR_INVALID;
  if (k == 0) return SPECACHE_OK;
  if (!idx || !k16_src || !v16_src || !k_sel || !v_sel) return SPECACHE_ERR_INVALID;
  const void* ks = device_view(k16_src);
  const void* vs = device_view(v16_src);
  if (!ks || !vs) return SPECACHE_ERR_NOT_PINNED;
  return hip_status(launch_gather(d, idx, k, static_cast<const _Float16*>(ks), static_cast<const _Float16*>(vs),
                                  static_cast<_Float16*>(k_sel), static_cast<_Float16*>(v_sel), false,
                                  static_cast<hipStream_t>(stream)));
}

int specache_gather_reuse(const specache_shape* shape, const int32_t* idx, int k, const int32_t* idx_prev,
                          int k_prev, const void* k_sel_prev, const void* v_sel_prev, void* k_sel, void* v_sel,
                          int32_t* fetch_idx, void* stream) {
  Dims d;
  int err;
  if (!make_dims(shape, &d, &err)) return err;
  if (k < 0 || k > d.N || k_prev < 0 || k_prev > d.N) return SPECACHE_ERR_INVALID;
  if (k == 0) return SPECACHE_OK;
  if (!idx || !k_sel || !v_sel || !fetch_idx) return SPECACHE_ERR_INVALID;
  if (k_prev > 0 && (!idx_prev || !k_sel_prev || !v_sel_prev)) return SPECACHE_ERR_INVALID;
  if (k_sel == k_sel_prev || v_sel == v_sel_prev) return SPECACHE_ERR_INVALID;
  return hip_status(launch_reuse(d, idx, k, idx_prev, k_prev, static_cast<const _Float16*>(k_sel_prev),
                                 static_cast<const _Float16*>(v_sel_prev), static_cast<_Float16*>(k_sel),
                                 static_cast<_Float16*>(v_sel), fetch_idx, static_cast<hipStream_t>(stream)));
}

int specache_gather_fp16_missing(const specache_shape* shape, const int32_t* fetch_idx, int k, const void* k16_src,
                                 const void* v16_src, void* k_sel, void* v_sel, void* stream) {
  Dims d;
  int err;
  if (!make_dims(shape, &d, &err)) return err;
  if (k < 0 || k > d.N) return SPECACHE_ERR_INVALID;
  if (k == 0) return SPECACHE_OK;
  if (!fetch_idx || !k16_src || !v16_src || !k_sel || !v_sel) return SPECACHE_ERR_INVALID;
  const void* ks = device_view(k16_src);
  const void* vs = device_view(v16_src);
  if (!ks || !vs) return SPECACHE_ERR_NOT_PINNED;
  return hip_status(launch_gather(d, fetch_idx, k, static_cast<const _Float16*>(ks),
                                  static_cast<const _Float16*>(vs), static_cast<_Float16*>(k_sel),
                                  static_cast<_Float16*>(v_sel), true, static_cast<hipStream_t>(stream)));
}

size_t specache_decode_attn_workspace_size(const specache_shape* shape, int n_tokens, int k, int tail_len) {
  Dims d;
  int err;
  if (!make_dims(shape, &d, &err) || n_tokens < 1 || n_tokens > 2 || k < 0 || k > d.N || tail_len < 0 ||
      tail_len > kMaxTail || d.G * n_tokens > kMaxRows || d.N > kMaxAttnSeqLen)
    return 0;
  return attn_ws(d, n_tokens).total;
}

namespace {

// Compute units a stream's kernels may use: its CU mask (streams made by
// specache_*_stream_create), else the whole device.
int stream_cus(hipStream_t s) {
  int dev = 0, cus = kPlanMaxCUs;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return kPlanMaxCUs;
  uint32_t mask[64] = {0};
  if (s == nullptr || hipExtStreamGetCUMask(s, 64, mask) != hipSuccess) {
    (void)hipGetLastError();
    return cus;
  }
  int n = 0;
  for (int i = 0; i < 64; ++i) n += __builtin_popcount(mask[i]);
  return n > 0 && n < cus ? n : cus;
}

int fill_attn_args(const Dims& d, const void* q16, int n_tokens, const specache_lowbit* cache, const int32_t* idx,
                   int k, const void* k_sel, const void* v_sel, const void* k_tail, const void* v_tail, int tail_len,
                   float sm_scale, void* out16, AttnArgs* a) {
  if (n_tokens < 1 || n_tokens > 2 || k < 0 || k > d.N || tail_len < 0 || tail_len > kMaxTail || !q16 ||
      !lowbit_ok(cache) || !out16 || !(sm_scale > 0.0f) || sm_scale == INFINITY)
    return SPECACHE_ERR_INVALID;
  if (d.G * n_tokens > kMaxRows || d.N > kMaxAttnSeqLen) return SPECACHE_ERR_UNSUPPORTED;
  if (k > 0 && (!idx || !k_sel || !v_sel)) return SPECACHE_ERR_INVALID;
  if (tail_len > 0 && (!k_tail || !v_tail)) return SPECACHE_ERR_INVALID;
  std::memset(a, 0, sizeof(*a));
  a->q16 = static_cast<const _Float16*>(q16);
  a->T = n_tokens;
  a->k_codes = static_cast<const uint32_t*>(cache->k_codes);
  a->k_meta = static_cast<const _Float16*>(cache->k_meta);
  a->v_codes = static_cast<const uint32_t*>(cache->v_codes);
  a->v_meta = static_cast<const _Float16*>(cache->v_meta);
  a->seq_stride = d.Ns;
  a->group = d.group;
  a->idx = idx;
  a->k = k;
  a->k_sel = static_cast<const _Float16*>(k_sel);
  a->v_sel = static_cast<const _Float16*>(v_sel);
  a->k_tail = static_cast<const _Float16*>(k_tail);
  a->v_tail = static_cast<const _Float16*>(v_tail);
  a->tail = tail_len;
  a->sm_scale = sm_scale;
  a->out16 = static_cast<_Float16*>(out16);
  return SPECACHE_OK;
}

}  // namespace

int specache_decode_attn(const specache_shape* shape, const void* q16, int n_tokens, const specache_lowbit* cache,
                         const int32_t* idx, int k, const void* k_sel, const void* v_sel, const void* k_tail,
                         const void* v_tail, int tail_len, float sm_scale, void* out16, void* workspace,
                         size_t workspace_bytes, void* stream) {
  Dims d;
  int err;
  if (!make_dims(shape, &d, &err)) return err;
  AttnArgs a;
  err = fill_attn_args(d, q16, n_tokens, cache, idx, k, k_sel, v_sel, k_tail, v_tail, tail_len, sm_scale, out16, &a);
  if (err != SPECACHE_OK) return err;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const AttnPlan plan = attn_plan(d, stream_cus(s), attn_split_wgs_per_cu(d, a));
  const AttnWs ws = attn_ws(d, n_tokens);
  if (!workspace || workspace_bytes < ws.total) return SPECACHE_ERR_WORKSPACE;
  char* base = static_cast<char*>(workspace);
  a.part_ml = reinterpret_cast<float*>(base + ws.ml);
  a.part_acc = reinterpret_cast<float*>(base + ws.acc);
  if (launch_attn_split(d, plan, a, s) != hipSuccess) return SPECACHE_ERR_HIP;
  return hip_status(launch_attn_merge(d, plan, a, s));
}

size_t specache_decode_attn_fp16_workspace_size(const specache_shape* shape, int n_tokens, int tail_len) {
  Dims d;
  int err;
  if (!make_dims(shape, &d, &err) || n_tokens < 1 || n_tokens > 2 || tail_len < 0 || tail_len > kMaxTail ||
      d.G * n_tokens > kMaxRows || d.N > kMaxAttnSeqLen)
    return 0;
  return attn_ws(d, n_tokens).total;
}

int specache_decode_attn_fp16(const specache_shape* shape, const void* q16, int n_tokens, const void* k16,
                              const void* v16, const void* k_tail, const void* v_tail, int tail_len, float sm_scale,
                              void* out16, void* workspace, size_t workspace_bytes, void* stream) {
  Dims d;
  int err;
  if (!make_dims(shape, &d, &err)) return err;
  if (n_tokens < 1 || n_tokens > 2 || tail_len < 0 || tail_len > kMaxTail || !q16 || !k16 || !v16 || !out16 ||
      !(sm_scale > 0.0f) || sm_scale == INFINITY)
    return SPECACHE_ERR_INVALID;
  if (d.G * n_tokens > kMaxRows || d.N > kMaxAttnSeqLen) return SPECACHE_ERR_UNSUPPORTED;
  if (tail_len > 0 && (!k_tail || !v_tail)) return SPECACHE_ERR_INVALID;
  const void* kd = device_view(k16);
  const void* vd = device_view(v16);
  if (!kd || !vd) return SPECACHE_ERR_NOT_PINNED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const AttnPlan plan = attn_plan(d, stream_cus(s), kAttnWGsPerCU);
  const AttnWs ws = attn_ws(d, n_tokens);
  if (!workspace || workspace_bytes < ws.total) return SPECACHE_ERR_WORKSPACE;
  AttnArgs a;
  std::memset(&a, 0, sizeof(a));
  a.q16 = static_cast<const _Float16*>(q16);
  a.T = n_tokens;
  a.k = (int)d.Ns;  // the whole 16-bit cache is the row array: row p = position p
  a.k_sel = static_cast<const _Float16*>(kd);
  a.v_sel = static_cast<const _Float16*>(vd);
  a.k_tail = static_cast<const _Float16*>(k_tail);
  a.v_tail = static_cast<const _Float16*>(v_tail);
  a.tail = tail_len;
  a.sm_scale = sm_scale;
  a.out16 = static_cast<_Float16*>(out16);
  char* base = static_cast<char*>(workspace);
  a.part_ml = reinterpret_cast<float*>(base + ws.ml);
  a.part_acc = reinterpret_cast<float*>(base + ws.acc);
  if (launch_attn16_split(d, plan, a, s) != hipSuccess) return SPECACHE_ERR_HIP;
  return hip_status(launch_attn_merge(d, plan, a, s));
}

size_t specache_decode_step_workspace_size(const specache_shape* shape, int n_tokens, int k, int tail_len,
                                           int k_next) {
  Dims d;
  int err;
  if (!make_dims(shape, &d, &err) || n_tokens < 1 || n_tokens > 2 || k < 0 || k > d.N || tail_len < 0 ||
      tail_len > kMaxTail || d.G * n_tokens > kMaxRows || d.N > kMaxAttnSeqLen || k_next < 1 || k_next > d.N)
    return 0;
  return attn_ws(d, n_tokens).total_step;
}

}  // extern "C"

namespace {

int decode_step_impl(const specache_shape* shape, const void* q16, int n_tokens, int rank_row, int rank_mixed,
                     const specache_lowbit* cache, const int32_t* idx, int k, const void* k_sel, const void* v_sel,
                     const void* k_tail, const void* v_tail, int tail_len, float sm_scale, void* out16, int k_next,
                     int32_t* idx_next_out, float* rank_key_out, void* workspace, size_t workspace_bytes,
                     void* stream) {
  Dims d;
  int err;
  if (!make_dims(shape, &d, &err)) return err;
  AttnArgs a;
  err = fill_attn_args(d, q16, n_tokens, cache, idx, k, k_sel, v_sel, k_tail, v_tail, tail_len, sm_scale, out16, &a);
  if (err != SPECACHE_OK) return err;
  if (rank_row < 0 || rank_row >= n_tokens || k_next < 1 || k_next > d.N || !idx_next_out ||
      (rank_mixed != 0 && rank_mixed != 1))
    return SPECACHE_ERR_INVALID;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const AttnPlan plan = attn_plan(d, stream_cus(s), attn_split_wgs_per_cu(d, a));
  const AttnWs ws = attn_ws(d, n_tokens);
  if (!workspace || workspace_bytes < ws.total_step) return SPECACHE_ERR_WORKSPACE;
  char* base = static_cast<char*>(workspace);
  a.part_ml = reinterpret_cast<float*>(base + ws.ml);
  a.part_acc = reinterpret_cast<float*>(base + ws.acc);
  a.rank_row = rank_row;
  a.rank_mixed = rank_mixed;
  a.rank_logits = reinterpret_cast<float*>(base + ws.logits);
  a.rank_m = reinterpret_cast<float*>(base + ws.rank_m);
  a.rank_l = reinterpret_cast<float*>(base + ws.rank_l);
  a.rank_hist = reinterpret_cast<uint32_t*>(base + ws.hist);
  float* keys = rank_key_out ? rank_key_out : reinterpret_cast<float*>(base + ws.keys);
  // bounds for the pruned selection: no key output, one bound group per selected position at
  // most (G * T <= 8 follows from G <= 4).  Ranking by the mixed cache replaces the fetched rows'
  // logits after the bounds are taken: the selection then reads their groups whatever the bounds.
  if (!rank_key_out && rank_select_prunable(d, k_next)) a.rank_gmax = reinterpret_cast<float*>(base + ws.gmax);
  // the split merge runs inside the selection's launch, on the compute units it leaves idle
  if (launch_attn_split(d, plan, a, s) != hipSuccess) return SPECACHE_ERR_HIP;
  const MergeJob merge{a.part_ml, a.part_acc, plan.S, (int64_t)d.B * d.Hq * n_tokens, a.out16};
  return hip_status(launch_rank_select(d, plan.S, a.rank_logits, a.rank_m, a.rank_l, k_next, keys,
                                       rank_key_out != nullptr, a.rank_hist, idx_next_out, &merge, s,
                                       a.rank_gmax, rank_mixed ? idx : nullptr, rank_mixed ? k : 0,
                                       reinterpret_cast<float*>(base + ws.gmax)));
}

// The no-allocation decode step's scratch: one array per GPU, in the library's code object, held
// until the process ends.  Host code never uses the array's name as an address (on the host it
// is only a stand-in for the symbol); the device address comes from hipGetSymbolAddress, taken
// once per device with that device current.
static __device__ __align__(256) unsigned char scratch[SPECACHE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
struct ScratchSlot {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// The current device's scratch address, or null (status in *err).
void* scratch_address(int* err) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    *err = SPECACHE_ERR_HIP;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *err = SPECACHE_ERR_UNSUPPORTED;
    return nullptr;
  }
  ScratchSlot& slot = g_scratch[dev];
  std::call_once(slot.once, [&slot] {
    slot.err = hipGetSymbolAddress(&slot.ptr, HIP_SYMBOL(scratch));
    if (slot.err != hipSuccess) slot.ptr = nullptr;
  });
  if (slot.err != hipSuccess || !slot.ptr) {
    *err = SPECACHE_ERR_HIP;
    return nullptr;
  }
  *err = SPECACHE_OK;
  return slot.ptr;
}

}  // namespace

extern "C" {

int specache_decode_step(const specache_shape* shape, const void* q16, int n_tokens, int rank_row,
                         int rank_mixed, const specache_lowbit* cache, const int32_t* idx, int k, const void* k_sel,
                         const void* v_sel, const void* k_tail, const void* v_tail, int tail_len, float sm_scale,
                         void* out16, int k_next, int32_t* idx_next_out, float* rank_key_out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  return decode_step_impl(shape, q16, n_tokens, rank_row, rank_mixed, cache, idx, k, k_sel, v_sel, k_tail, v_tail,
                          tail_len, sm_scale, out16, k_next, idx_next_out, rank_key_out, workspace, workspace_bytes,
                          stream);
}

int specache_decode_step_noalloc(const specache_shape* shape, const void* q16, int n_tokens, int rank_row,
                                 int rank_mixed, const specache_lowbit* cache, const int32_t* idx, int k,
                                 const void* k_sel, const void* v_sel, const void* k_tail, const void* v_tail,
                                 int tail_len, float sm_scale, void* out16, int k_next, int32_t* idx_next_out,
                                 float* rank_key_out, void* stream) {
  const size_t need = specache_decode_step_workspace_size(shape, n_tokens, k, tail_len, k_next);
  if (need > SPECACHE_NOALLOC_SCRATCH_BYTES) return SPECACHE_ERR_TOO_LARGE;
  int err = SPECACHE_OK;
  void* ws = nullptr;
  if (need > 0) {  // else the arguments are invalid: decode_step_impl names the error
    ws = scratch_address(&err);
    if (!ws) return err;
  }
  return decode_step_impl(shape, q16, n_tokens, rank_row, rank_mixed, cache, idx, k, k_sel, v_sel, k_tail, v_tail,
                          tail_len, sm_scale, out16, k_next, idx_next_out, rank_key_out, ws,
                          ws ? (size_t)SPECACHE_NOALLOC_SCRATCH_BYTES : 0, stream);
}

namespace {

// A stream whose kernels run on compute units [first, first + count) of the current device.
int create_cu_stream(int first, int count, bool all_from_first, void** stream_out) {
  if (!stream_out) return SPECACHE_ERR_INVALID;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return SPECACHE_ERR_HIP;
  if (all_from_first) count = cus - first;
  if (first < 0 || count < kMinGatherCUs || first + count > cus) return SPECACHE_ERR_INVALID;
  const int words = (cus + 31) / 32;
  if (words > 64) return SPECACHE_ERR_UNSUPPORTED;
  // The mask is passed with a length of words * 32 entries, all zero past the first `words`, so
  // that it is read in bounds and means the same whether that length counts bits or words.
  uint32_t mask[64 * 32] = {0};
  for (int i = first; i < first + count; ++i) mask[i / 32] |= 1u << (i % 32);
  hipStream_t st = nullptr;
  if (hipExtStreamCreateWithCUMask(&st, (uint32_t)(words * 32), mask) != hipSuccess) return SPECACHE_ERR_HIP;
  *stream_out = st;
  return SPECACHE_OK;
}

}  // namespace

int specache_gather_stream_create(int n_cus, void** stream_out) {
  return create_cu_stream(0, n_cus, false, stream_out);
}

int specache_compute_stream_create(int reserved_cus, void** stream_out) {
  if (reserved_cus < kMinGatherCUs) return SPECACHE_ERR_INVALID;
  return create_cu_stream(reserved_cus, 0, true, stream_out);
}

int specache_stream_destroy(void* stream) {
  if (!stream) return SPECACHE_ERR_INVALID;
  return hip_status(hipStreamDestroy(static_cast<hipStream_t>(stream)));
}

const char* specache_status_string(int status) {
  switch (status) {
    case SPECACHE_OK: return "ok";
    case SPECACHE_ERR_INVALID: return "invalid argument";
    case SPECACHE_ERR_UNSUPPORTED: return "unsupported shape";
    case SPECACHE_ERR_WORKSPACE: return "workspace missing or too small";
    case SPECACHE_ERR_NOT_PINNED: return "gather source is neither device memory nor pinned host memory";
    case SPECACHE_ERR_HIP: return "HIP runtime error";
    case SPECACHE_ERR_TOO_LARGE:
      return "problem needs more scratch than the no-allocation entry point's static buffer holds";
    default: return "unknown status";
  }
}

int specache_abi_version(void) { return SPECACHE_ABI_VERSION; }

}  // extern "C"
