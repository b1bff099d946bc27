// The C ABI declared in include/specache.h: argument validation on the host,
// workspace carving, and dispatch to the kernel launchers.  Nothing here
// allocates memory or keeps state.
#include <cstring>

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
  if (s->batch <= 0 || s->n_q_heads <= 0 || s->n_kv_heads <= 0 || s->head_dim <= 0 || s->seq_len <= 0 ||
      s->n_q_heads % s->n_kv_heads != 0 || s->seq_len % kGroup != 0 || s->batch > 65535 ||
      (int64_t)s->batch * s->n_kv_heads > 65535 || s->seq_len > (int64_t(1) << 31) - 1) {
    *err = SPECACHE_ERR_INVALID;
    return false;
  }
  if (s->bits != 1 && s->bits != 2) {
    *err = SPECACHE_ERR_INVALID;
    return false;
  }
  if (s->group != kGroup || (s->head_dim != 64 && s->head_dim != 128) ||
      s->n_q_heads / s->n_kv_heads > kMaxRows) {
    *err = SPECACHE_ERR_UNSUPPORTED;
    return false;
  }
  d->B = s->batch;
  d->Hq = s->n_q_heads;
  d->Hkv = s->n_kv_heads;
  d->D = s->head_dim;
  d->bits = s->bits;
  d->G = s->n_q_heads / s->n_kv_heads;
  d->W = s->head_dim / 32;
  d->N = s->seq_len;
  d->nblk = s->seq_len / kGroup;
  return true;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct ScoreWs {
  size_t logits, part_m, part_l, keys, hist, total;
};

ScoreWs score_ws(const Dims& d, const ScorePlan& p) {
  ScoreWs w;
  w.logits = 0;
  size_t off = align256(sizeof(float) * (size_t)d.slices() * d.G * d.N);
  w.part_m = off;
  off += align256(sizeof(float) * (size_t)d.slices() * d.G * p.S);
  w.part_l = off;
  off += align256(sizeof(float) * (size_t)d.slices() * d.G * p.S);
  w.keys = off;
  off += align256(sizeof(float) * (size_t)d.slices() * d.N);
  w.hist = off;
  off += align256(sizeof(uint32_t) * (size_t)d.slices() * 2048);
  w.total = off;
  return w;
}

struct AttnWs {
  size_t ml, acc, total;
};

AttnWs attn_ws(const Dims& d, const AttnPlan& p, int T) {
  AttnWs w;
  const size_t rows = (size_t)d.B * d.Hq * T;
  w.ml = 0;
  w.acc = align256(sizeof(float) * rows * p.S * 2);
  w.total = w.acc + align256(sizeof(float) * rows * p.S * d.D);
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

extern "C" {

size_t specache_lowbit_bytes(const specache_shape* shape, size_t* k_codes, size_t* k_meta, size_t* v_codes,
                             size_t* v_meta) {
  Dims d;
  int err;
  if (!make_dims(shape, &d, &err)) return 0;
  const size_t pos = (size_t)d.slices() * d.N;
  const size_t kc = pos * d.bits * d.W * 4;
  const size_t km = (size_t)d.slices() * d.nblk * 2 * d.D * 2;
  const size_t vc = (size_t)d.slices() * d.nblk * d.bits * d.D * 4;
  const size_t vm = (size_t)d.slices() * d.nblk * 2 * d.W * 32 * 2;
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
  return hip_status(launch_quantize(d, static_cast<const _Float16*>(k16), static_cast<const _Float16*>(v16),
                                    static_cast<uint32_t*>(out->k_codes), static_cast<_Float16*>(out->k_meta),
                                    static_cast<uint32_t*>(out->v_codes), static_cast<_Float16*>(out->v_meta),
                                    static_cast<hipStream_t>(stream)));
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
  hipError_t e = launch_score(d, plan, static_cast<const _Float16*>(q16), n_tokens, rank_row,
                              static_cast<const uint32_t*>(cache->k_codes), static_cast<const _Float16*>(cache->k_meta),
                              sm_scale, logits, part_m, part_l, hist, s);
  if (e != hipSuccess) return SPECACHE_ERR_HIP;
  e = launch_rank_select(d, plan, logits, part_m, part_l, k, keys, hist, idx_out, s);
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
                                  static_cast<_Float16*>(k_sel), static_cast<_Float16*>(v_sel),
                                  static_cast<hipStream_t>(stream)));
}

size_t specache_decode_attn_workspace_size(const specache_shape* shape, int n_tokens, int k, int tail_len) {
  Dims d;
  int err;
  if (!make_dims(shape, &d, &err) || n_tokens < 1 || n_tokens > 2 || k < 0 || k > d.N || tail_len < 0 ||
      tail_len > kMaxTail || d.G * n_tokens > kMaxRows || d.N > kMaxAttnSeqLen)
    return 0;
  return attn_ws(d, attn_plan(d, k, tail_len), n_tokens).total;
}

int specache_decode_attn(const specache_shape* shape, const void* q16, int n_tokens, const specache_lowbit* cache,
                         const int32_t* idx, int k, const void* k_sel, const void* v_sel, const void* k_tail,
                         const void* v_tail, int tail_len, float sm_scale, void* out16, void* workspace,
                         size_t workspace_bytes, void* stream) {
  Dims d;
  int err;
  if (!make_dims(shape, &d, &err)) return err;
  if (n_tokens < 1 || n_tokens > 2 || k < 0 || k > d.N || tail_len < 0 || tail_len > kMaxTail || !q16 ||
      !lowbit_ok(cache) || !out16 || !(sm_scale > 0.0f) || sm_scale == INFINITY)
    return SPECACHE_ERR_INVALID;
  if (d.G * n_tokens > kMaxRows || d.N > kMaxAttnSeqLen) return SPECACHE_ERR_UNSUPPORTED;
  if (k > 0 && (!idx || !k_sel || !v_sel)) return SPECACHE_ERR_INVALID;
  if (tail_len > 0 && (!k_tail || !v_tail)) return SPECACHE_ERR_INVALID;
  const AttnPlan plan = attn_plan(d, k, tail_len);
  const AttnWs ws = attn_ws(d, plan, n_tokens);
  if (!workspace || workspace_bytes < ws.total) return SPECACHE_ERR_WORKSPACE;
  char* base = static_cast<char*>(workspace);
  AttnArgs a;
  a.q16 = static_cast<const _Float16*>(q16);
  a.T = n_tokens;
  a.k_codes = static_cast<const uint32_t*>(cache->k_codes);
  a.k_meta = static_cast<const _Float16*>(cache->k_meta);
  a.v_codes = static_cast<const uint32_t*>(cache->v_codes);
  a.v_meta = static_cast<const _Float16*>(cache->v_meta);
  a.idx = idx;
  a.k = k;
  a.k_sel = static_cast<const _Float16*>(k_sel);
  a.v_sel = static_cast<const _Float16*>(v_sel);
  a.k_tail = static_cast<const _Float16*>(k_tail);
  a.v_tail = static_cast<const _Float16*>(v_tail);
  a.tail = tail_len;
  a.sm_scale = sm_scale;
  a.out16 = static_cast<_Float16*>(out16);
  a.part_ml = reinterpret_cast<float*>(base + ws.ml);
  a.part_acc = reinterpret_cast<float*>(base + ws.acc);
  return hip_status(launch_decode_attn(d, plan, a, static_cast<hipStream_t>(stream)));
}

const char* specache_status_string(int status) {
  switch (status) {
    case SPECACHE_OK: return "ok";
    case SPECACHE_ERR_INVALID: return "invalid argument";
    case SPECACHE_ERR_UNSUPPORTED: return "unsupported shape";
    case SPECACHE_ERR_WORKSPACE: return "workspace missing or too small";
    case SPECACHE_ERR_NOT_PINNED: return "gather source is neither device memory nor pinned host memory";
    case SPECACHE_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int specache_abi_version(void) { return SPECACHE_ABI_VERSION; }

}  // extern "C"
