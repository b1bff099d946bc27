/*
 * specache.h -- C ABI of libspecache: decode-step attention over a 1/2-bit
 * KIVI-style KV cache with speculative top-k prefetch of 16-bit rows, for
 * AMD Instinct MI355X (gfx950).
 *
 * The method is SpeCache ("SpeCache: Speculative Key-Value Caching for
 * Efficient Generation of LLMs", papercache.org summary of arXiv:2503.16163):
 * the GPU keeps only a low-bit copy C' of the KV cache, the 16-bit cache C
 * lives in host memory, each decode step runs two query tokens (the real T_t
 * and a speculative T'_{t+1}), ranks positions by the speculative token's
 * attention over C', prefetches the top-k 16-bit rows, and attends over
 * C' with those rows substituted.  The four calls below map onto the
 * operations of the summary's appendix algorithms:
 *
 *   Quant(K), Quant(V)     (Algorithm 1)      -> specache_quantize_pack
 *   ArgTopK(A_{1,:})       (Algorithms 2, 3)  -> specache_score_topk
 *   Pre-fetch(C_kappa)     (Algorithms 2, 3)  -> specache_gather_fp16
 *   Attn(.., C' U C_kappa) (Algorithm 3)      -> specache_decode_attn
 *   Offload(C)             is the caller's own device-to-host copy.
 *
 * specache_decode_step fuses the last two compute steps of one decode step:
 * the attention of Algorithm 3 and the ArgTopK of its speculative row come
 * out of one pass over C' (the speculative row's logits against C' are
 * formed by that attention anyway).
 *
 * ------------------------------------------------------------------------
 * Conventions (every call)
 * ------------------------------------------------------------------------
 *  - Plain pointers.  Unless a parameter says otherwise, a pointer is device
 *    memory of the current HIP device, caller-allocated and caller-owned; the
 *    library never frees or retains it.  Inputs are read only; outputs are
 *    fully overwritten.
 *  - `stream` is a hipStream_t (NULL = the legacy default stream).  Calls
 *    only enqueue work and return; results are ready when the stream reaches
 *    them.  Ordering across streams is the caller's job (HIP events).
 *  - The library keeps no state and allocates nothing: scratch space comes
 *    from a caller-provided workspace whose size the *_workspace_size
 *    functions return.  (One exception: specache_decode_step_noalloc, for
 *    callers that cannot allocate, keeps its scratch in a static array of the
 *    library's device code.)
 *  - The attention calls split the positions of each slice over a number of
 *    workgroups chosen for the compute units `stream` may use (its CU mask,
 *    else the whole device).  Results are deterministic for a given stream
 *    configuration; on streams with different CU counts they may differ in
 *    the last bits (the order of float32 accumulation changes).
 *  - Return value: a specache_status.  Argument errors are detected on the
 *    host before anything is enqueued; SPECACHE_ERR_HIP means a HIP runtime
 *    call or a kernel launch failed (faults inside kernels surface at the
 *    caller's next synchronization, as with any HIP kernel).  No C++
 *    exception crosses this boundary.
 *  - All tensors are dense, row-major (last index fastest), with the shapes
 *    given below.  float16 is IEEE binary16.
 *
 * ------------------------------------------------------------------------
 * Shapes and symbols
 * ------------------------------------------------------------------------
 *  B = batch, Hq = query heads, Hkv = KV heads, G = Hq / Hkv (query head hq
 *  reads KV head hq / G), D = head_dim (64 or 128), N = cached positions
 *  (a positive multiple of 32; specache_shape.seq_len), Nc = positions the
 *  cache buffers are laid out for (specache_shape.seq_capacity, 0 meaning
 *  Nc = N; a multiple of 32, Nc >= N), T = query tokens per step (1 or 2;
 *  row 0 is the real token T_t, row 1 the speculative token T'_{t+1}),
 *  b = bits per code (1 or 2; specache_shape.bits for the keys and
 *  specache_shape.v_bits, default the same, for the values -- the summary's
 *  §5 pairs 1- or 2-bit keys with 1- or 2-bit values), g = quantization
 *  group = 32, W = D / 32.
 *  G * T <= 16.  Every call reads and writes positions [0, N) of the caches;
 *  positions [N, Nc) are room for specache_quantize_append and
 *  specache_offload_fp16 (the decode-time cache update).
 *
 * ------------------------------------------------------------------------
 * Low-bit cache C' (written by specache_quantize_pack)
 * ------------------------------------------------------------------------
 *  Quantizer: the summary's §3.  Keys are grouped per channel over 32
 *  consecutive tokens, values per token over 32 consecutive channels (KIVI's
 *  grouping, as restated in the SemKV page, §2.1).  For a group with minimum
 *  mn and maximum mx (computed in float32 from the float16 inputs):
 *    b = 1 (§3 "improved 1-bit quantization"): z = (3*mn + mx)/4,
 *          s = (mx - mn)/2, evaluated as z = (3*mn + mx) * 0.25 and
 *          s = (mx - mn) * 0.5 in float32;
 *    b = 2 (§3 "original KIVI quantization"): z = mn, s = (mx - mn)/3 with a
 *          correctly rounded float32 division;
 *  z and s are stored as float16 (round to nearest even; -0 stored as +0).
 *  code(x) = clamp(floor(q + 1/2), 0, 2^b - 1) with q = (x - z16) / s16 in
 *  float32 (round half up, the summary's rounding), and code 0 when s16 == 0.
 *  Dequantized value: code * s16 + z16.
 *
 *  Bit planes: a code's bit j (j = 0 least significant) lives in plane j.
 *  Within every 32-bit word, bit i (i = 0..31) stands for element
 *  e(i) = 2*(i mod 16) + (i div 16): even elements in the low half-word, odd
 *  elements in the high half-word (element e is a channel for keys, a token
 *  for values).
 *
 *  k_codes  uint32 [B][Hkv][Nc][bk][W]     (bk, bv: key and value bits)
 *                                          word (p, j, w) holds plane j of the
 *                                          codes of token p, channels 32w+e(i).
 *  k_meta   float16[B][Hkv][Nc/32][2][D]   [blk][0][c] = z, [blk][1][c] = s of the
 *                                          key group (tokens 32blk..32blk+31, channel c).
 *  v_codes  uint32 [B][Hkv][Nc/32][bv][D]  word (blk, j, c) holds plane j of the
 *                                          codes of channel c, tokens 32blk+e(i).
 *  v_meta   float16[B][Hkv][Nc/32][2][W][32] [blk][0][w][t] = z, [blk][1][w][t] = s of
 *                                          the value group (token 32blk+t, channels
 *                                          32w..32w+31).
 *  Bytes per position per KV head: (bk*D/8 + 4*D/32) for keys and
 *  (bv*D/8 + 4*D/32) for values -- 64 B at D = 128 with 1-bit keys and
 *  values (one eighth of float16), 96 B with 2 bits for both.
 *
 * ------------------------------------------------------------------------
 * Other tensors
 * ------------------------------------------------------------------------
 *  q16, out16      float16 [B][Hq][T][D]
 *  k16, v16        float16 [B][Hkv][Nc][D]     the full 16-bit cache C (positions [0, N) used)
 *  idx             int32   [B][Hkv][k]         strictly ascending, each in [0, N)
 *  k_sel, v_sel    float16 [B][Hkv][k][D]      row i = 16-bit row idx[i]
 *  k_tail, v_tail  float16 [B][Hkv][R][D]      optional 16-bit positions after the
 *                                              cache (the step's own new KV)
 *  rank_key        float32 [B][Hkv][N]         r(p), see specache_score_topk
 */
#ifndef SPECACHE_H_
#define SPECACHE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPECACHE_ABI_VERSION 6

typedef enum specache_status {
  SPECACHE_OK = 0,
  SPECACHE_ERR_INVALID = 1,     /* bad argument: null pointer, size out of range, inconsistent shape */
  SPECACHE_ERR_UNSUPPORTED = 2, /* valid but not built: head_dim not 64/128, group != 32, G*T > 16 */
  SPECACHE_ERR_WORKSPACE = 3,   /* workspace null or smaller than the *_workspace_size value */
  SPECACHE_ERR_NOT_PINNED = 4,  /* gather source is neither device memory nor pinned host memory */
  SPECACHE_ERR_HIP = 5,         /* a HIP runtime call or kernel launch failed */
  SPECACHE_ERR_TOO_LARGE = 6    /* specache_decode_step_noalloc: scratch needed beyond its static buffer */
} specache_status;

/* Shape of one layer's cache.  group must be 32. */
typedef struct specache_shape {
  int32_t batch;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int64_t seq_len;       /* N: cached positions in use */
  int32_t bits;
  int32_t group;
  int64_t seq_capacity;  /* Nc: positions the cache buffers hold; 0 = seq_len */
  int32_t v_bits;        /* bits of the value codes; 0 = bits (then bits is both) */
  int32_t reserved;      /* 0 */
} specache_shape;

/* The four device buffers of C' (layouts above). */
typedef struct specache_lowbit {
  void* k_codes;
  void* k_meta;
  void* v_codes;
  void* v_meta;
} specache_lowbit;

/* Byte sizes of the four C' buffers for `shape`, laid out for its capacity Nc (0 for an
 * invalid shape). */
size_t specache_lowbit_bytes(const specache_shape* shape, size_t* k_codes, size_t* k_meta,
                             size_t* v_codes, size_t* v_meta);

/*
 * Quant(K), Quant(V) of the summary's Algorithm 1 (prefill), with the §3
 * quantizer described above: reads positions [0, N) of k16, v16
 * [B][Hkv][Nc][D] (device float16) and writes them into the four buffers of
 * `out`.  Bit-exact by definition (no floating-point freedom).  Inputs must
 * be finite.
 */
int specache_quantize_pack(const specache_shape* shape, const void* k16, const void* v16,
                           const specache_lowbit* out, void* stream);

/*
 * C' = [C', C'_t] of Algorithm 3 (the decode-time cache update): quantizes
 * n_new new positions, k16_new / v16_new [B][Hkv][n_new][D] (device float16),
 * into positions [N, N + n_new) of `cache`, exactly as specache_quantize_pack
 * would have quantized them as part of the whole cache.  A key group spans 32
 * tokens, so positions are appended in whole groups: n_new is a multiple of
 * 32 and the newest tokens wait in the 16-bit tail (the residual window;
 * specache_decode_attn's k_tail / v_tail) until a group is complete.
 * N + n_new <= Nc.  After the call the cache holds N + n_new positions (pass
 * seq_len = N + n_new from then on).
 */
int specache_quantize_append(const specache_shape* shape, const void* k16_new, const void* v16_new,
                             int64_t n_new, const specache_lowbit* cache, void* stream);

/*
 * C = [C, Offload(C_t)] of Algorithm 3: copies k16_new / v16_new
 * [B][Hkv][n_new][D] (device float16) into positions [pos0, pos0 + n_new) of
 * the 16-bit cache k16_dst / v16_dst [B][Hkv][Nc][D] -- pinned host memory (the
 * source of specache_gather_fp16) or device memory; anything else returns
 * SPECACHE_ERR_NOT_PINNED.  One strided DMA copy per tensor on `stream`.
 * 0 <= pos0, pos0 + n_new <= Nc.
 */
int specache_offload_fp16(const specache_shape* shape, const void* k16_new, const void* v16_new,
                          int64_t n_new, int64_t pos0, void* k16_dst, void* v16_dst, void* stream);

/*
 * ArgTopK over the speculative row (the summary's quick read, second
 * mechanism; §3 "prefetch and offload during decoding"; Algorithm 3's
 * ArgTopK(A_{1,:}), Algorithm 2 with n_tokens = 1).
 *
 * For every slice (b, h) and each of its G query heads hq = h*G + gi, the
 * logits of row `rank_row` against C' are s_gi(p) = sm_scale * q . Khat(p)
 * (Khat dequantized; the 16-bit rows play no part).  With LSE_gi the
 * log-sum-exp of s_gi over p, the rank of position p is
 *     r(p) = log sum_gi exp(s_gi(p) - LSE_gi),
 * the log of the attention mass the G heads put on p.  idx_out [B][Hkv][k]
 * receives the k positions of largest r in ascending order (ties -> lower
 * position).  rank_key_out, if not NULL, receives r [B][Hkv][N] (float32).
 *
 * n_tokens in {1, 2}; 0 <= rank_row < n_tokens; 1 <= k <= N.
 * Workspace: specache_score_topk_workspace_size bytes, device memory,
 * 256-byte aligned.
 */
size_t specache_score_topk_workspace_size(const specache_shape* shape, int n_tokens, int k);
int specache_score_topk(const specache_shape* shape, const void* q16, int n_tokens, int rank_row,
                        const specache_lowbit* cache, float sm_scale, int k, int32_t* idx_out,
                        float* rank_key_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Pre-fetch(C_kappa) of Algorithm 3: k_sel[b][h][i][:] = k16_src[b][h][idx[b][h][i]][:]
 * and the same for values -- a byte copy.  k16_src / v16_src may be pinned
 * host memory (hipHostMalloc, or torch pin_memory) read directly by the
 * kernel over the host link, or device memory; anything else returns
 * SPECACHE_ERR_NOT_PINNED.  An idx entry outside [0, N) is not dereferenced:
 * its output row is filled with float16 NaN.  0 <= k <= N (k = 0 is a no-op).
 * Typically enqueued on a side stream after an event recorded behind
 * specache_score_topk.
 */
int specache_gather_fp16(const specache_shape* shape, const int32_t* idx, int k,
                         const void* k16_src, const void* v16_src, void* k_sel, void* v_sel,
                         void* stream);

/*
 * Resident-set reuse (SpeCache summary, §3 "prefetch and offload during
 * decoding": once the attention ends the next top-k rows are prefetched while
 * the used rows outside the new top-k are evicted -- so rows in both sets stay
 * on the device).  Two calls together produce what specache_gather_fp16(idx)
 * would, fetching only the rows that are not resident:
 *
 * specache_gather_reuse: for every slice and row i of the new selection idx
 * [B][Hkv][k] (ascending), if idx[i] is also in the previous selection
 * idx_prev [B][Hkv][k_prev] (ascending) at row j, copy row j of k_sel_prev /
 * v_sel_prev ([B][Hkv][k_prev][D] float16, device) into row i of k_sel / v_sel
 * ([B][Hkv][k][D], device; must not be the previous buffers) and set
 * fetch_idx[i] = -1; otherwise set fetch_idx[i] = idx[i] (N for an entry
 * outside [0, N)) and leave the row.  fetch_idx [B][Hkv][k] int32, device.
 * Device-to-device work: run it on the compute stream.
 *
 * specache_gather_fp16_missing: specache_gather_fp16 over fetch_idx, except
 * that rows with a negative entry are left untouched.  Host-link work: run it
 * on the gather stream after an event behind specache_gather_reuse.
 *
 * 0 <= k, k_prev <= N; k_prev = 0 marks every row for fetching.
 */
int specache_gather_reuse(const specache_shape* shape, const int32_t* idx, int k, const int32_t* idx_prev,
                          int k_prev, const void* k_sel_prev, const void* v_sel_prev, void* k_sel, void* v_sel,
                          int32_t* fetch_idx, void* stream);
int specache_gather_fp16_missing(const specache_shape* shape, const int32_t* fetch_idx, int k,
                                 const void* k16_src, const void* v16_src, void* k_sel, void* v_sel,
                                 void* stream);

/*
 * A stream for specache_gather_fp16 whose kernels run on only `n_cus` compute
 * units of the current device (hipExtStreamCreateWithCUMask, default
 * priority).  The prefetch is meant to run in the background, in parallel
 * with the compute that follows (SpeCache summary, quick read, second
 * mechanism; §3); a zero-copy gather waits on the host link for most of its
 * life, and the compute units that host its waves serve other kernels'
 * memory requests far slower meanwhile, so confining it to a few compute
 * units keeps the overlapped attention and scoring at full speed.  8 units
 * sustain the host link.  8 <= n_cus <= the device's compute-unit count (the
 * runtime needs at least one unit on each of the 8 accelerator complex dies;
 * the low mask bits interleave over them).
 * *stream_out receives a hipStream_t owned by the caller; release it with
 * specache_stream_destroy.  It is a blocking stream (the runtime creates
 * CU-masked streams without hipStreamNonBlocking): work on the legacy default
 * (NULL) stream serializes with it, so run the overlapped compute on a
 * non-default stream.
 */
int specache_gather_stream_create(int n_cus, void** stream_out);

/*
 * The complement of specache_gather_stream_create(reserved_cus): a stream
 * whose kernels run on every compute unit except the `reserved_cus` ones a
 * gather stream of that size uses, so that the overlapped compute never shares
 * a compute unit with the gather's waves.  8 <= reserved_cus, and at least 8
 * units must remain.  Blocking stream, released with
 * specache_stream_destroy, like the gather stream.
 */
int specache_compute_stream_create(int reserved_cus, void** stream_out);
int specache_stream_destroy(void* stream);

/*
 * Ordering between two streams of one GPU through a flag in device memory, for
 * the overlapped loop of §3 "decoding" (the prefetch stream waits for the
 * selection it fetches, then runs beside the other layers' compute) without a
 * queue barrier between the streams.
 *
 * specache_flag_set enqueues on `stream` a kernel that, once every earlier
 * command on that stream has completed, stores `value` into *flag (uint32 in
 * device memory, caller-owned) with release ordering at device scope.
 * specache_flag_wait enqueues on `stream` a one-wave kernel that polls *flag
 * (acquire at device scope) until it has reached `value` (flag - value taken
 * as a signed 32-bit distance, so a sequence number may wrap); work enqueued
 * on `stream` after it sees everything the setter's stream published.  The
 * wait is bounded: after max_wait_us microseconds (1 <= max_wait_us) it stops
 * waiting and adds 1 to *timeouts (uint32 in device memory, caller-owned and
 * zeroed by the caller), so the caller can detect a flag that was never set.
 * The flag only ever needs to grow: use increasing sequence numbers rather
 * than clearing it.  The setter must be able to run while the wait runs: the
 * two streams must not share a hardware queue (the library's gather and
 * compute streams each have their own), and where kernel dispatches are
 * serialised (a profiler collecting per-dispatch counters does this) a wait
 * whose setter comes later ends only at the time limit.
 * Returns SPECACHE_ERR_INVALID for a null pointer or max_wait_us == 0,
 * SPECACHE_ERR_HIP if the launch fails.
 */
int specache_flag_set(uint32_t* flag, uint32_t value, void* stream);
int specache_flag_wait(const uint32_t* flag, uint32_t value, uint32_t max_wait_us, uint32_t* timeouts,
                       void* stream);

/*
 * O = Attn([T_t, T'_{t+1}], C' U C_kappa) (the summary's quick read, third
 * mechanism; §3 "decoding"; Algorithm 3): softmax attention of every query
 * row over the N cached positions, where the k positions listed in idx use
 * the 16-bit rows k_sel / v_sel in place of their dequantized low-bit rows,
 * followed by the tail_len positions of k_tail / v_tail; tail position j is
 * visible to query row t iff j <= tail_len - n_tokens + t (the masked
 * softmax of Algorithm 3: the real token does not see the speculative
 * token's entry).  Logits are sm_scale * q . k.  out16 [B][Hq][T][D] float16.
 *
 * N <= 4194304 (SPECACHE_ERR_UNSUPPORTED above);
 * 0 <= k <= N (k = 0: pure low-bit attention; idx, k_sel, v_sel may be NULL);
 * idx must be strictly ascending within [0, N) per slice (not checked on the
 * device); 0 <= tail_len <= 64 (k_tail / v_tail may be NULL when 0).
 * Workspace: specache_decode_attn_workspace_size bytes, device memory.
 */
size_t specache_decode_attn_workspace_size(const specache_shape* shape, int n_tokens, int k,
                                           int tail_len);
int specache_decode_attn(const specache_shape* shape, const void* q16, int n_tokens,
                         const specache_lowbit* cache, const int32_t* idx, int k,
                         const void* k_sel, const void* v_sel, const void* k_tail,
                         const void* v_tail, int tail_len, float sm_scale, void* out16,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step's compute in one pass over C' (Algorithm 3 of the
 * SpeCache summary: Attn over C' U C_kappa, and ArgTopK(A_{1,:}) of the
 * speculative row for the next step's prefetch; §3 "prefetch and offload
 * during decoding": the indices are recorded during the attention).  With
 * rank_mixed = 0 it is equivalent to
 *     specache_decode_attn(shape, q16, n_tokens, cache, idx, k, k_sel, v_sel,
 *                          k_tail, v_tail, tail_len, sm_scale, out16, ...)
 *     specache_score_topk(shape, q16, n_tokens, rank_row, cache, sm_scale,
 *                         k_next, idx_next_out, rank_key_out, ...)
 * (same out16 bits; the ranking is the one of specache_score_topk, the
 * logits of row rank_row against C' with the 16-bit rows and the tail
 * taking no part) but the low-bit cache is read once.
 *
 * rank_mixed = 1 takes Algorithm 3's A_{1,:} literally: row rank_row's
 * masked softmax over the keys the attention uses -- C' with the fetched
 * 16-bit rows in place of theirs, and the tail entries visible to that row
 * -- so r(p) = log sum_gi A_gi(p) over the N cached positions (the tail
 * shares each head's normalization but is no candidate).  out16 is the same
 * in both modes.
 *
 * Arguments as for the two calls; 0 <= rank_row < n_tokens;
 * rank_mixed in {0, 1}; 1 <= k_next <= N; idx_next_out [B][Hkv][k_next]
 * int32, ascending.
 * idx_next_out may be the same buffer as idx (the attention has consumed idx
 * before the selection writes, in stream order); rank_key_out [B][Hkv][N]
 * float32 or NULL.  Workspace: specache_decode_step_workspace_size bytes,
 * device memory (it holds the speculative row's logits, 4*B*Hq*N bytes, plus
 * the attention partials).
 */
size_t specache_decode_step_workspace_size(const specache_shape* shape, int n_tokens, int k,
                                           int tail_len, int k_next);
int specache_decode_step(const specache_shape* shape, const void* q16, int n_tokens, int rank_row,
                         int rank_mixed, const specache_lowbit* cache, const int32_t* idx, int k,
                         const void* k_sel, const void* v_sel, const void* k_tail,
                         const void* v_tail, int tail_len, float sm_scale, void* out16,
                         int k_next, int32_t* idx_next_out, float* rank_key_out,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * specache_decode_step for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same call and result
 * (same kernels; out16 and idx_next_out identical to specache_decode_step's on the same stream)
 * with its scratch in a static device array of the library instead of a caller workspace.
 * Allocates nothing: no hipMalloc / hipFree on any call.
 *
 * The array holds SPECACHE_NOALLOC_SCRATCH_BYTES per GPU (every GPU the library runs on keeps its
 * own copy until the process ends); a problem whose specache_decode_step_workspace_size exceeds
 * it returns SPECACHE_ERR_TOO_LARGE before anything is enqueued (128 MiB holds, for example, the
 * 32K-context step at batch 16 with 8 KV heads, 32 query heads and k = 328).  Every call on one
 * GPU shares that GPU's array, which keeps the last call's contents (no part of it needs to start
 * at zero: the kernels clear what they accumulate into).  Calls on one stream are ordered; calls
 * that overlap on one GPU (several streams, or several host threads) race on the array and give
 * undefined results.  Other arguments and errors as for specache_decode_step.
 */
#define SPECACHE_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
int specache_decode_step_noalloc(const specache_shape* shape, const void* q16, int n_tokens, int rank_row,
                                 int rank_mixed, const specache_lowbit* cache, const int32_t* idx, int k,
                                 const void* k_sel, const void* v_sel, const void* k_tail, const void* v_tail,
                                 int tail_len, float sm_scale, void* out16, int k_next, int32_t* idx_next_out,
                                 float* rank_key_out, void* stream);

/*
 * The 16-bit comparator: O = Attn(q, C) over the full 16-bit cache held in
 * device memory -- the "16-bit" decoding the SpeCache summary's throughput
 * ratios are taken against (quick read, results; §5 Table 3).  Same kernel
 * organisation and partial merge as specache_decode_attn, with every cached
 * position a 16-bit row: k16 / v16 [B][Hkv][Nc][D] float16 (positions [0, N)
 * used; device memory, or pinned host memory read over the host link), the
 * optional tail and its mask as in specache_decode_attn, out16
 * [B][Hq][T][D].  Workspace: specache_decode_attn_fp16_workspace_size bytes.
 */
size_t specache_decode_attn_fp16_workspace_size(const specache_shape* shape, int n_tokens, int tail_len);
int specache_decode_attn_fp16(const specache_shape* shape, const void* q16, int n_tokens, const void* k16,
                              const void* v16, const void* k_tail, const void* v_tail, int tail_len,
                              float sm_scale, void* out16, void* workspace, size_t workspace_bytes,
                              void* stream);

/* Static description of a status code. */
const char* specache_status_string(int status);

/* SPECACHE_ABI_VERSION of the built library. */
int specache_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPECACHE_H_ */
