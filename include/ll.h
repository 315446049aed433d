/*
 * ll.h -- C ABI of the frame-sink + short-window KV-cache attention library
 * (libll.so, HIP kernels for AMD Instinct MI355X / gfx950).
 *
 * What the library computes comes from the paper "LongLive: Real-time
 * Interactive Long Video Generation":
 *   - frame-level autoregressive generation conditioned on a per-layer KV
 *     cache, causal across chunks of latent frames (Abstract; §3.2);
 *   - short-window attention over the most recent frames plus a frame sink:
 *     the first frame chunk's tokens are kept in the cache for good and are
 *     concatenated to every layer's keys/values; the rest of the cache is a
 *     short rolling window evicted in the usual way (§3.3 "Efficient long
 *     inference"; §4 "Implementation");
 *   - KV-recache at a prompt switch: the cache of the most recent window is
 *     rebuilt (§3.1 "KV recache"; §3.3, last paragraph);
 *   - text cross-attention injecting the prompt (§3.1).
 *
 * Notation.  T tokens per latent frame, C frames per chunk, S sink frames,
 * W window frames (the window counts the chunk being generated), H heads,
 * D head dimension.  C_tok = C*T tokens per chunk, R = (W-C)/C ring slots of
 * one chunk each, n_sc = S/C sink chunks.  Chunk j's frames are [jC, (j+1)C).
 *
 * Conventions for every call.
 *   - Pointers named q, k, v, k_cur, v_cur, k_txt, v_txt, out are DEVICE
 *     pointers to token-major activations [n][H][D] (contiguous, element type
 *     = the activation dtype, base 16-byte aligned).  lse is a nullable device
 *     pointer to float [H][n_q].  Config, handle and query outputs are HOST
 *     pointers.
 *   - The library never allocates device memory and never frees the caller's.
 *     The caller owns the cache's device buffer and every input/output, and
 *     keeps them alive until the work enqueued on the stream has finished.
 *   - All argument and state validation is synchronous and happens before
 *     anything is enqueued.  On any error nothing is enqueued and no host
 *     state changes; the status says why and ll_last_error() gives a
 *     thread-local message.  A launch failure returns LL_ERR_HIP.  Device
 *     faults surface at the caller's next synchronisation.  No C++ exception
 *     crosses this ABI.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream).
 *     All calls on one cache must be ordered on one stream (or otherwise
 *     ordered by the caller): an append or recache overwrites ring slots that
 *     an earlier attention call may still be reading.  Host state advances at
 *     enqueue time.  A handle is not thread-safe.
 */
#ifndef LL_H
#define LL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipStream_t without pulling in the HIP headers (same underlying type). */
typedef struct ihipStream_t* ll_stream_t;

typedef struct ll_cache ll_cache; /* opaque host-side handle */

typedef enum {
  LL_OK = 0,
  LL_ERR_INVALID_ARG = 1,      /* NULL/misaligned pointer, bad size or index */
  LL_ERR_BAD_STATE = 2,        /* call not valid in the cache's current state */
  LL_ERR_UNSUPPORTED = 3,      /* geometry or dtype combination not supported */
  LL_ERR_BUFFER_TOO_SMALL = 4, /* device buffer smaller than required */
  LL_ERR_HIP = 5,              /* a HIP launch/runtime call failed */
  LL_ERR_INTERNAL = 6
} ll_status;

typedef enum { LL_F32 = 0, LL_BF16 = 1, LL_I8 = 2 } ll_dtype;

/* How the attention reads an I8 cache (ll_cache_set_int8_dequant). */
typedef enum { LL_I8_STAGED = 0, LL_I8_IN_KERNEL = 1 } ll_int8_dequant;

/* Which cached tensor ll_cache_layout describes. */
typedef enum { LL_WHICH_K = 0, LL_WHICH_V = 1, LL_WHICH_KSCALE = 2, LL_WHICH_VSCALE = 3 } ll_which;
/* Which cache segment ll_cache_layout describes. */
typedef enum { LL_SEG_SINK = 0, LL_SEG_RING = 1 } ll_segment;

#define LL_MAX_RING_SLOTS 30

/*
 * Cache geometry.  Supported: head_dim in {64, 128}; sink_frames a multiple of
 * frames_per_chunk (0 allowed: no sink); window_frames >= frames_per_chunk and
 * window_frames - frames_per_chunk a multiple of frames_per_chunk with at most
 * LL_MAX_RING_SLOTS ring slots; (act_dtype, kv_dtype) one of (F32, F32),
 * (BF16, BF16), (BF16, I8).  With kv_dtype I8 the cache stores int8 K/V and an
 * fp32 scale per (token, head): s = max|x|/127 (IEEE fp32 division),
 * q = clamp(round_half_even(x/s), -127, 127), s = 0 and q = 0 for an all-zero
 * vector.  (The paper reports INT8 inference without giving a scheme; this
 * per-token, per-head KV scheme is this library's own.)  With kv_dtype BF16 or
 * I8 every sink chunk and ring slot is its own key run: at most 39 of them.
 * One chunk of activations ([C_tok][H][D]) must be smaller than 4 GiB.
 */
typedef struct {
  int32_t num_layers;
  int32_t num_heads;
  int32_t head_dim;
  int32_t tokens_per_frame;
  int32_t frames_per_chunk;
  int32_t sink_frames;
  int32_t window_frames; /* includes the chunk being generated */
  int32_t act_dtype;     /* ll_dtype of q, k, v, k_cur, v_cur, out */
  int32_t kv_dtype;      /* ll_dtype of the cached K/V */
} ll_cache_config;

/* Device bytes the cache needs for `cfg` (all layers), written to *bytes.  An
 * I8 cache also holds one layer's bf16 staging area, which the staged
 * attention mode, the backward and the linear-attention variant rewrite from
 * the layer's codes before reading it. */
ll_status ll_cache_required_bytes(const ll_cache_config* cfg, size_t* bytes);

/*
 * Create a host handle over a caller-owned device buffer `dev_buf` of
 * `dev_bytes` bytes (256-byte aligned, at least ll_cache_required_bytes).
 * The buffer's contents need no initialisation: nothing is read before it is
 * written.  The buffer must outlive the handle and all enqueued work.
 */
ll_status ll_cache_create(const ll_cache_config* cfg, void* dev_buf, size_t dev_bytes,
                          ll_cache** out);

/* The configuration `cache` was created with, written to *cfg (host memory). */
ll_status ll_cache_get_config(const ll_cache* cache, ll_cache_config* cfg);

/* Destroy the host handle (the device buffer is the caller's). NULL is a no-op. */
ll_status ll_cache_destroy(ll_cache* cache);

/*
 * How ll_sink_window_attn and ll_window_reencode_attn read an I8 cache
 * (INT8 KV variant).  Host state only; enqueues nothing.
 *   LL_I8_IN_KERNEL: the attention kernel reads the int8 codes and their
 *     scales and attends over the exact values q * s: codes are converted
 *     exactly to bf16 tiles on chip, the K scale multiplies each score in
 *     fp32 and the V scale is folded into P before its bf16 rounding.
 *   LL_I8_STAGED (default): one extra launch per call first writes a bf16
 *     copy, bf16(q * s), of the layer's resident codes into the cache's
 *     staging area, and the bf16 attention kernel reads that copy (faster on
 *     MI355X; about 3.4x the call's algorithmic HBM bytes against 1.6x in the
 *     kernel, and one more bf16 rounding of q * s).
 * LL_ERR_INVALID_ARG for a mode outside the enum or a cache whose kv_dtype is
 * not I8.  The backward and the linear-attention variant always read the
 * staged copy.
 */
ll_status ll_cache_set_int8_dequant(ll_cache* cache, int32_t mode);

/* Forget every appended chunk in every layer (host-only; enqueues nothing). */
ll_status ll_cache_reset(ll_cache* cache);

/*
 * Append the next chunk's keys/values to layer `layer` (paper §3.3: sink kept,
 * rolling window evicted).  k, v: [C_tok][H][D] of act_dtype.  Appended chunk
 * j goes to sink rows [j*C_tok, (j+1)*C_tok) while j < n_sc, else to ring slot
 * (j - n_sc) mod R, overwriting (evicting) the oldest window chunk.  With
 * R == 0 a non-sink chunk is counted but not stored.  With kv_dtype I8 the
 * chunk is quantised on the way in.
 */
ll_status ll_cache_append_chunk(ll_cache* cache, int32_t layer, const void* k, const void* v,
                                ll_stream_t stream);

/*
 * KV-recache (paper §3.1; §3.3: only the most recent window is rebuilt):
 * rewrite every resident non-sink window chunk of layer `layer` in place,
 * oldest to newest, from k, v: [n_tokens][H][D] of act_dtype, where n_tokens
 * must equal (resident ring chunks) * C_tok.  layer == -1 rewrites all layers
 * in one launch from k, v: [num_layers][n_tokens][H][D]; every layer must then
 * hold the same resident ring slots in the same oldest-to-newest order (as
 * layers that have appended equally many chunks do).  The sink is never
 * rewritten.  LL_ERR_BAD_STATE if no window chunk is resident or the layers'
 * rings differ.
 */
ll_status ll_cache_recache(ll_cache* cache, int32_t layer, const void* k, const void* v,
                           int64_t n_tokens, ll_stream_t stream);

/*
 * Sink + short-window attention for the queries of the next chunk
 * c = (chunks appended to `layer`) (paper §3.3).  Keys/values are, addressed
 * in place without copies: the resident sink tokens, the resident ring chunks,
 * and, when n_cur == C_tok, the caller's k_cur/v_cur [C_tok][H][D] of the
 * current chunk (n_cur == 0: cache only).  One softmax runs over their union;
 * there is no mask inside the set (causal across chunks only).
 *   q, out: [n_q][H][D] act_dtype (n_q >= 0; 0 is a no-op).
 *   scale:  logit scale, finite and > 0 (1/sqrt(D) in a standard DiT).
 *   lse:    nullable float [H][n_q]: natural-log sum of exp(scale * q.k).
 * Accumulation is fp32 (bf16 MFMA products for BF16 activations).  The scale
 * is folded into the queries before their bf16 rounding.  An I8 cache is read
 * as ll_cache_set_int8_dequant selects (in the attention kernel, or through a
 * bf16 staging copy written by one extra launch on the same stream); the
 * current chunk is used as given.
 * LL_ERR_BAD_STATE if the key set is empty.
 */
ll_status ll_sink_window_attn(const ll_cache* cache, int32_t layer, const void* q, int64_t n_q,
                              const void* k_cur, const void* v_cur, int64_t n_cur, float scale,
                              void* out, float* lse, ll_stream_t stream);

/*
 * Backward of ll_sink_window_attn for the training step (paper §3.2: frames
 * generated earlier are detached and gradients flow through the current clip
 * only; §3.3: training keeps the last W frames' K/V without gradient, the
 * current clip's K/V with gradient, and the sink concatenated to every layer).
 * The key set is the one the forward call with the same arguments used: the
 * cached sink and window (detached: they get no gradient) and, when
 * n_cur == C_tok, the current chunk k_cur/v_cur, which does.
 *   q, out, dout: [n_q][H][D] bf16 (out and lse from the forward call);
 *   lse:   float [H][n_q], required;
 *   delta: float [H][n_q] device workspace, overwritten with rowsum(dout*out);
 *   dq:    float [n_q][H][D], written; when dk_cur/dv_cur are asked for, the
 *          call first uses its first n_q*H*D*2 bytes as scratch for a bf16
 *          copy of the scaled queries, so dq must not overlap any input;
 *   dk_cur, dv_cur: float [C_tok][H][D], written when n_cur == C_tok (ignored
 *          when n_cur == 0).  With them, (n_q + 64) * H * D * 2 must be below
 *          4 GiB (else LL_ERR_UNSUPPORTED).
 * Gradients are fp32, accumulated in fp32 from bf16 MFMA products of bf16
 * operands (P and dS rounded to bf16); P is recomputed from the forward's lse.
 * BF16 activations only (else LL_ERR_UNSUPPORTED); with an I8 cache the
 * context is the same bf16(q * s) staging copy the forward attends over.
 * n_q >= 1.  LL_ERR_BAD_STATE if the key set is empty.
 */
ll_status ll_sink_window_attn_bwd(const ll_cache* cache, int32_t layer, const void* q, int64_t n_q,
                                  const void* k_cur, const void* v_cur, int64_t n_cur, float scale,
                                  const void* out, const float* lse, const void* dout, float* delta,
                                  float* dq, float* dk_cur, float* dv_cur, ll_stream_t stream);

/*
 * ll_sink_window_attn_bwd without the delta workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, serving
 * loops, harnesses that forbid allocation).  Same arguments, layouts,
 * numerics and errors otherwise.  delta lives in a static device array of
 * 2^20 floats that the library holds on each GPU until the process ends:
 * num_heads * n_q must be at most 1048576 (else LL_ERR_UNSUPPORTED, nothing
 * enqueued).  Every call on one GPU uses that GPU's array; calls that overlap
 * on one GPU (other streams or threads) race.  Each call rewrites the part it
 * reads, so nothing carries over between calls.  Allocates nothing.
 */
ll_status ll_sink_window_attn_bwd_noalloc(const ll_cache* cache, int32_t layer, const void* q, int64_t n_q,
                                          const void* k_cur, const void* v_cur, int64_t n_cur, float scale,
                                          const void* out, const float* lse, const void* dout, float* dq,
                                          float* dk_cur, float* dv_cur, ll_stream_t stream);

/*
 * Self-attention of the re-encoding pass of a KV-recache (paper §3.1 "KV
 * recache": at a prompt switch the frames already generated are encoded again
 * with the new prompt to rebuild the cache; §3.3: the cache holds the sink and
 * the short window).  Call it after ll_cache_recache has written the new K/V
 * of layer `layer`.  The queries are the resident window chunks', oldest chunk
 * first: q, out [n_q][H][D] of act_dtype with n_q = (resident window chunks)
 * * C_tok.  The queries of window chunk r attend, in one softmax, to the
 * resident sink tokens and the window chunks 0..r (causal across chunks, no
 * mask inside a chunk); frames evicted before the switch take no part.
 *   scale: finite and > 0;  lse: nullable float [H][n_q].
 * Numerics as ll_sink_window_attn.  LL_ERR_BAD_STATE if no window chunk is
 * resident; LL_ERR_INVALID_ARG if n_q differs from the resident token count.
 */
ll_status ll_window_reencode_attn(const ll_cache* cache, int32_t layer, const void* q,
                                  int64_t n_q, float scale, void* out, float* lse,
                                  ll_stream_t stream);

/*
 * Linear-attention variant of ll_sink_window_attn (paper §4 "Implementation":
 * the method was also built on a linear-attention video model for more speed;
 * the paper gives no formulation, so this is the plain reading): the same key
 * set (resident sink, resident window, and the current chunk when
 * n_cur == C_tok) with the weights w_ij = phi(q_i) . phi(k_j),
 * phi(x) = max(x, 0) elementwise, and
 *   out_i = sum_j w_ij v_j / (sum_j w_ij + 1e-6)
 * (no logit scale; a query with no positive weight gets 0).  Computed in the
 * associative form S = sum_j phi(k_j) v_j^T, z = sum_j phi(k_j) per head:
 * fp32 accumulation of bf16 MFMA products, S kept as a bf16 pair (~16
 * significant bits) for the output product.
 *   q, out: [n_q][H][D] bf16 (n_q >= 0; 0 is a no-op after validation).
 *   work:   device workspace of at least ll_linear_attn_workspace_bytes,
 *           256-byte aligned, owned by the caller; overwritten (partial sums).
 * Three launches on the stream (plus the int8 staging launch for an I8
 * cache, as ll_sink_window_attn).  BF16 activations only (else
 * LL_ERR_UNSUPPORTED); LL_ERR_BUFFER_TOO_SMALL if work_bytes is short;
 * LL_ERR_BAD_STATE if the key set is empty.  Calls sharing one workspace
 * must be stream-ordered.
 */
ll_status ll_sink_window_linear_attn(const ll_cache* cache, int32_t layer, const void* q, int64_t n_q,
                                     const void* k_cur, const void* v_cur, int64_t n_cur, void* out,
                                     void* work, size_t work_bytes, ll_stream_t stream);

/* Workspace bytes ll_sink_window_linear_attn needs for this cache's H and D. */
ll_status ll_linear_attn_workspace_bytes(const ll_cache* cache, size_t* bytes);

/*
 * Text cross-attention (paper §3.1: cross-attention injects the prompt):
 * unmasked softmax attention of q [n_q][H][D] to k_txt, v_txt [n_txt][H][D],
 * all of `dtype` (F32 or BF16); out [n_q][H][D]; lse nullable [H][n_q];
 * scale finite and > 0.
 * head_dim in {64, 128}; n_txt >= 1.
 */
ll_status ll_cross_attn(const void* q, int64_t n_q, const void* k_txt, const void* v_txt,
                        int64_t n_txt, int32_t num_heads, int32_t head_dim, int32_t dtype,
                        float scale, void* out, float* lse, ll_stream_t stream);

/*
 * Host state of one layer.  Any output pointer may be NULL.  slot_chunk, if
 * given, receives R entries: the chunk index held by each ring slot, -1 if
 * empty.  ring_next is the slot the next non-sink append writes.
 */
ll_status ll_cache_query(const ll_cache* cache, int32_t layer, int64_t* chunks_appended,
                         int32_t* ring_valid, int32_t* ring_next, int64_t* slot_chunk);

/*
 * Where a cached tensor lives inside the device buffer, for snapshots and
 * tests.  For (which, segment) it returns the byte offset (from dev_buf) of
 * element [0][0][0][0] of a 4-D view, its element strides and its shape
 * (shape may be NULL).
 *   - K, and V of an F32 or I8 cache: [H][rows][cols][1]; rows = S*T (sink)
 *     or R*C_tok (ring; slot s is rows [s*C_tok, (s+1)*C_tok)); cols = D
 *     (element type kv_dtype), or 1 for the fp32 scales (I8 only).
 *   - V of a BF16 cache: [H][tiles][D][64], V transposed in tiles of 64 keys,
 *     C_tok rounded up to whole tiles per chunk slot (the sink's chunks, then
 *     the ring's slots), zeros after a chunk's last key.  Key i of slot s is in
 *     tile s*ceil(C_tok/64) + i/64, column p = i%64 with bits 2 and 3 swapped
 *     (the key order in which the attention kernel's PV operand wants it).
 */
ll_status ll_cache_layout(const ll_cache* cache, int32_t layer, int32_t which, int32_t segment,
                          size_t* byte_offset, int64_t* strides /*[4]*/, int64_t* shape /*[4]*/);

/* Static text for a status code. */
const char* ll_status_str(ll_status status);

/* Thread-local message for the last error on this thread ("" if none). */
const char* ll_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LL_H */
