/*
 * swa.h — C ABI of libswa: causal sliding-window attention (SWA) with
 * grouped-query heads (GQA), a rolling-buffer KV cache, chunked prefill and
 * single-token decode, for AMD Instinct MI355X (gfx950).
 *
 * The method is the one of Mistral 7B as described by the pages
 *   "Mistral 7B — 슬라이딩 윈도우 어텐션 중심 정리"            (digest)
 *   "[arXiv 2310.06825] Mistral 7B: 슬라이딩 윈도우 어텐션과 ..." (essay)
 *   "Mistral 7B: Engineering Extreme Efficiency in LLMs"         (explainer)
 *   "LLM 추론용 SWA는 ... 캐시를 무한히 키우지 않는 기술에 가깝다" (sinks)
 *
 * WINDOW CONVENTION (fixed).  A query at absolute position i attends the key
 * at absolute position j iff
 *       0 <= j <= i   and   ( i - window < j   or   j < n_sink )
 * i.e. `window` keys including itself, plus the first n_sink positions
 * (attention sinks).  With dilation d > 1 the window part keeps only the keys
 * with (i - j) divisible by d: i, i-d, i-2d, ... inside the same span, so the
 * rolling buffer is unchanged (the dilated sliding window the digest lists
 * for Longformer, "Longformer vs Mistral SWA — 구조적 비교"; the pages define
 * none: this is the reading taken).  Digest "핵심 구성요소" / explainer How It Works 2 give
 * the SWA mask; this is its reading that matches a window-slot buffer that is
 * written before it is read (digest "Rolling Buffer KV Cache 동작 설명":
 * the query at p reads p-W+1 .. p).  The sink prefix follows the sinks page,
 * "왜 단순 sliding window만으로는 부족한가".
 *
 * CACHE SLOT of position p (digest "쓰기(write) 단계"; explainer How It
 * Works 3: slot = p mod W):
 *       slot(p) = p < n_sink ? p : n_sink + (p - n_sink) % window
 * A cache holds S = n_sink + window slots per sequence.
 *
 * GQA: query head h uses KV head h / (n_q_heads / n_kv_heads) (explainer
 * How It Works 1: subsets of query heads share one K/V head; contiguous
 * subsets).
 *
 * RoPE (digest "Methods": theta = 10000): element pair (2k, 2k+1) of a head
 * vector at position p is rotated counter-clockwise by p * theta^(-2k/D).
 * Queries are rotated at their position, keys at their original position.
 * rope_theta == 0 disables it.  Angles are formed in double precision and
 * reduced to [-pi, pi] before a float sine/cosine; the rotation is float.
 *
 * LAYOUTS (row-major, contiguous, element type = params.dtype):
 *   q, out   : [batch][n_tok][n_q_heads][head_dim]     (prefill)
 *              [batch][n_q_heads][head_dim]            (decode)
 *   k, v     : [batch][n_tok][n_kv_heads][head_dim]    (raw, un-rotated)
 *   k_cache, v_cache : [batch][n_sink + window][n_kv_heads][head_dim]
 *              k_cache holds rotated keys, v_cache the values verbatim.
 *   lse      : float32 [batch][n_q_heads][n_tok] (prefill), [batch][n_q_heads]
 *              (decode): natural-log sum of exp of the scaled scores.
 *   start_pos / pos : int32 [batch], device memory.
 * All pointers are DEVICE pointers except `params`, which is host memory.
 *
 * OWNERSHIP: the caller allocates and owns every buffer, including the
 * workspaces whose sizes the *_workspace_bytes functions return.  The library
 * keeps no state between calls (beyond each device's compute-unit count,
 * read once) and allocates nothing; calls on different
 * streams with disjoint buffers may run concurrently.
 *
 * ERRORS: arguments are checked on the host before any HIP call; a bad
 * argument returns a negative swa_status and launches nothing.  A failed
 * launch returns SWA_ERR_LAUNCH.  Work is asynchronous on `stream`; kernel
 * faults surface on the stream like any HIP error.  Position values are
 * device data and are trusted: a negative position, or one >= 2^30, is
 * undefined behaviour.
 *
 * PRECISION: bf16 inputs are multiplied on the matrix cores with float32
 * accumulation; softmax statistics are float32; outputs are rounded once to
 * the output type.  The float32 dtype runs float32 arithmetic throughout.
 */
#ifndef SWA_H
#define SWA_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum swa_status {
  SWA_OK = 0,
  SWA_ERR_NULL = -1,        /* a required pointer is NULL                        */
  SWA_ERR_SHAPE = -2,       /* inconsistent or out-of-range sizes                */
  SWA_ERR_DTYPE = -3,       /* unknown dtype                                     */
  SWA_ERR_UNSUPPORTED = -4, /* valid request the library does not implement      */
  SWA_ERR_WORKSPACE = -5,   /* workspace pointer NULL or smaller than required   */
  SWA_ERR_LAUNCH = -6,      /* a kernel launch failed (hipGetLastError)          */
  SWA_ERR_SCRATCH = -7      /* the call needs more than the library's fixed
                               scratch array (swa_decode_step_noalloc)           */
} swa_status;

typedef enum swa_dtype { SWA_BF16 = 0, SWA_F32 = 1 } swa_dtype;

typedef struct swa_params {
  int32_t batch;       /* sequences, >= 1                                       */
  int32_t n_q_heads;   /* query heads, multiple of n_kv_heads                   */
  int32_t n_kv_heads;  /* key/value heads, >= 1                                 */
  int32_t head_dim;    /* 64 or 128                                             */
  int32_t window;      /* W >= 1: rolling slots; keys i-W < j <= i              */
  int32_t n_sink;      /* 0 <= n_sink <= 4096 global prefix positions (sinks)   */
  float scale;         /* softmax scale; 0 means 1/sqrt(head_dim)               */
  float rope_theta;    /* RoPE base; 0 disables RoPE                            */
  int32_t dtype;       /* swa_dtype of q, k, v, out and the caches              */
  int32_t dilation;    /* d >= 1 (0 means 1): the window part keeps only the
                          keys at distances 0, d, 2d, ... (below)              */
} swa_params;

/*
 * swa_cache_write — rotate keys and scatter a run of tokens into the
 * rolling buffer.  Digest "쓰기(write) 단계" (slot = p % W; K_buf[slot] = k_p;
 * V_buf[slot] = v_p), explainer How It Works 3.
 *   k, v      : [batch][n_tok][n_kv_heads][head_dim] raw keys and values.
 *   start_pos : device int32[batch]; token t of sequence b has position
 *               start_pos[b] + t.
 *   n_tok     : >= 1.
 *   k_cache, v_cache : caches, updated in place.
 * Equivalent to writing the tokens one by one in order: when n_tok exceeds
 * the window, only positions that survive (p >= start+n_tok-window, or sinks)
 * are written, so every slot has exactly one writer and the result is
 * deterministic.
 */
int swa_cache_write(const swa_params* params, const void* k, const void* v,
                    const int32_t* start_pos, int32_t n_tok, void* k_cache, void* v_cache,
                    hipStream_t stream);

/* Bytes of workspace swa_prefill_chunk needs for a chunk of `chunk_len`
 * tokens (the chunk's rotated keys).  0 on a bad argument. */
size_t swa_prefill_workspace_bytes(const swa_params* params, int32_t chunk_len);

/*
 * swa_prefill_chunk — attention of one prefill chunk.  Essay §4.1 and
 * Figure 3, explainer How It Works 4: the chunk's queries attend causally to
 * the chunk and, within the window, to what the cache held before the chunk.
 *   q         : [batch][chunk_len][n_q_heads][head_dim] raw queries.
 *   k, v      : [batch][chunk_len][n_kv_heads][head_dim] raw keys, values.
 *   k_cache, v_cache : the caches as they stand before the chunk (positions
 *               < start_pos[b]); both NULL means no position before the
 *               chunk exists (a sequence's first chunk): the queries then
 *               attend only the chunk's keys.
 *   start_pos : device int32[batch], position of the chunk's first token.
 *   out       : [batch][chunk_len][n_q_heads][head_dim].
 *   lse       : float32 [batch][n_q_heads][chunk_len], or NULL.
 *   workspace : >= swa_prefill_workspace_bytes(params, chunk_len) bytes.
 * Does NOT write the cache: call swa_cache_write(k, v, start_pos, chunk_len)
 * afterwards on the same stream (digest "Pre-fill과의 상호작용": after each
 * chunk the buffer holds the last W entries).
 */
int swa_prefill_chunk(const swa_params* params, const void* q, const void* k, const void* v,
                      const void* k_cache, const void* v_cache, const int32_t* start_pos,
                      int32_t chunk_len, void* out, float* lse, void* workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * swa_prefill_chunk_aligned — swa_prefill_chunk for chunks that start at
 * multiples of the window, the pages' own chunking: digest summary
 * "Pre-fill + Chunking" and explainer How It Works 4 cut a prompt into
 * chunks of W tokens, so from position 0 chunk c starts at c*W (essay §4.1:
 * the window size as the chunk size).  The rolling buffer then holds
 * positions start - W .. start - 1 in slot order and the attention reads it
 * as one run of rows.  Arguments, layouts, workspace and results as
 * swa_prefill_chunk, and byte-identical to it.
 *   start_pos : device int32[batch]; every start_pos[b] must be a multiple of
 *               window.  The host cannot see the positions, so the device
 *               checks: a sequence whose start is not a multiple gets NaN in
 *               every out row and lse entry.
 * With sinks, dilation, or a shape off the fast kernel (bf16, head_dim 128,
 * 1, 2, 4 or 8 query heads per KV head) it runs swa_prefill_chunk (any
 * start).
 */
int swa_prefill_chunk_aligned(const swa_params* params, const void* q, const void* k, const void* v,
                              const void* k_cache, const void* v_cache, const int32_t* start_pos,
                              int32_t chunk_len, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/*
 * swa_prefill_chunk_aligned_write_prev — one boundary of a chunked prompt:
 * swa_cache_write of the previous chunk, then swa_prefill_chunk_aligned of
 * the next, on the same stream, with results byte-identical to those two
 * calls (essay §4.1 and explainer How It Works 4: each chunk attends to the
 * cache that the chunks before it filled, then is written into it).  On the
 * fast shape the previous chunk's write and the next chunk's key rotation
 * run as one pass, a launch fewer per boundary.
 *   k_prev, v_prev : [batch][prev_len][n_kv_heads][head_dim] raw keys and
 *               values of the previous chunk, starting at start_prev[b]
 *               (device int32[batch]); prev_len >= 1.
 *   q, k, v, start_pos, chunk_len, out, lse, workspace : the next chunk, as
 *               swa_prefill_chunk_aligned (every start a multiple of window;
 *               NaN rows for a sequence whose start is not).
 *   k_cache, v_cache : the caches, updated in place with the previous chunk
 *               and then read by the next chunk's attention (not NULL).
 * The workspace must not overlap k_prev, v_prev or the caches.  With sinks,
 * dilation, or a shape off the fast kernel it makes the two calls.
 */
int swa_prefill_chunk_aligned_write_prev(const swa_params* params, const void* k_prev,
                                         const void* v_prev, const int32_t* start_prev, int32_t prev_len,
                                         const void* q, const void* k, const void* v, void* k_cache,
                                         void* v_cache, const int32_t* start_pos, int32_t chunk_len,
                                         void* out, float* lse, void* workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/*
 * swa_rope_keys — the key-rotation pass of swa_prefill_chunk on its own:
 * k_rot[b][t] = RoPE(k[b][t], start_pos[b] + t) (digest "Methods": RoPE,
 * theta from the architecture table), same layout as k.  With rope_theta == 0
 * it is a copy.  For callers that keep rotated keys themselves.
 */
int swa_rope_keys(const swa_params* params, const void* k, const int32_t* start_pos,
                  int32_t n_tok, void* k_rot, hipStream_t stream);

/*
 * swa_rope_keys_cache_write — swa_rope_keys and swa_cache_write in one pass
 * over the chunk: every key rotated into k_rot, and the entries that survive
 * the chunk (digest "Rolling Buffer KV Cache 동작 설명", 쓰기(write) 단계)
 * stored into the caches; k_rot, k_cache and v_cache afterwards are
 * byte-identical to those two calls'.  It writes the caches BEFORE the
 * chunk's attention, so it is for chunks whose attention reads no cache: a
 * sequence's first chunk (start_pos 0, or swa_prefill_attention called with
 * NULL caches).  A chunk that reads the cache keeps the order of essay §4.1
 * (swa_rope_keys, swa_prefill_attention, then swa_cache_write).
 *   k, v      : [batch][n_tok][n_kv_heads][head_dim] raw keys, values.
 *   k_rot     : [batch][n_tok][n_kv_heads][head_dim] rotated keys (output).
 *   k_cache, v_cache : [batch][n_sink + window][n_kv_heads][head_dim].
 * Errors as swa_cache_write; nothing is launched on an error.
 */
int swa_rope_keys_cache_write(const swa_params* params, const void* k, const void* v,
                              const int32_t* start_pos, int32_t n_tok, void* k_rot,
                              void* k_cache, void* v_cache, hipStream_t stream);

/*
 * swa_prefill_attention — the attention pass of swa_prefill_chunk on keys
 * that are already rotated (k_rot from swa_rope_keys); queries are rotated on
 * load.  Arguments and semantics otherwise as swa_prefill_chunk; it needs no
 * workspace.  swa_prefill_chunk == swa_rope_keys + swa_prefill_attention.
 */
int swa_prefill_attention(const swa_params* params, const void* q, const void* k_rot,
                          const void* v, const void* k_cache, const void* v_cache,
                          const int32_t* start_pos, int32_t chunk_len, void* out, float* lse,
                          hipStream_t stream);

/*
 * Varlen (ragged) batches: each sequence brings its own chunk length.
 * Essay §4.1 and digest "Pre-fill과의 상호작용": the chunk size is a free
 * choice, so the sequences of one batch may each prefill a different number
 * of tokens, and a sequence that decodes one token is a chunk of length 1.
 *   chunk_lens : HOST int32[batch], chunk_lens[b] in 0 .. 2^24 (0: the
 *                sequence takes no part), at least one token in all;
 *                total = sum of chunk_lens.
 *   q, out     : [total][n_q_heads][head_dim], k, v, k_rot :
 *                [total][n_kv_heads][head_dim]: the sequences packed one
 *                after the other in batch order (sequence b at rows
 *                chunk_lens[0] + .. + chunk_lens[b-1] onwards).
 *   lse        : float32 [n_q_heads][total], or NULL.
 *   start_pos, k_cache, v_cache : as in the calls above, per sequence.
 * Every other rule is that of the fixed-length call of the same name: the
 * result for sequence b is what that call gives with batch 1, chunk_len =
 * chunk_lens[b].  Errors as there, and SWA_ERR_SHAPE for a length out of
 * range or an empty batch; SWA_ERR_NULL when chunk_lens is NULL.  Up to 64
 * sequences go to one launch (more take several, on the same stream).
 */
size_t swa_prefill_varlen_workspace_bytes(const swa_params* params, const int32_t* chunk_lens);
int swa_rope_keys_varlen(const swa_params* params, const void* k, const int32_t* start_pos,
                         const int32_t* chunk_lens, void* k_rot, hipStream_t stream);
int swa_prefill_attention_varlen(const swa_params* params, const void* q, const void* k_rot,
                                 const void* v, const void* k_cache, const void* v_cache,
                                 const int32_t* start_pos, const int32_t* chunk_lens, void* out,
                                 float* lse, hipStream_t stream);
int swa_prefill_chunk_varlen(const swa_params* params, const void* q, const void* k, const void* v,
                             const void* k_cache, const void* v_cache, const int32_t* start_pos,
                             const int32_t* chunk_lens, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);
int swa_cache_write_varlen(const swa_params* params, const void* k, const void* v,
                           const int32_t* start_pos, const int32_t* chunk_lens, void* k_cache,
                           void* v_cache, hipStream_t stream);

/*
 * swa_step_varlen — one whole step of a mixed batch: every sequence's chunk
 * attends (the sequences of one token decode it), then every chunk goes
 * into the rolling buffers.  Same arguments and layouts as above; k_cache
 * and v_cache are read and written.  The result is that of
 * swa_prefill_chunk_varlen followed by swa_cache_write_varlen, up to
 * rounding: with bf16, head_dim 128 and 1, 2, 4 or 8 query heads per KV
 * head (no dilation), the
 * sequences of one token go to the decode kernel after the cache write
 * (the rest to the prefill kernel, before it), so that a decode token costs
 * a decode, not a 64-query prefill tile.
 *   workspace : >= swa_step_varlen_workspace_bytes(params, chunk_lens) bytes.
 */
size_t swa_step_varlen_workspace_bytes(const swa_params* params, const int32_t* chunk_lens);
int swa_step_varlen(const swa_params* params, const void* q, const void* k, const void* v,
                    void* k_cache, void* v_cache, const int32_t* start_pos,
                    const int32_t* chunk_lens, void* out, float* lse, void* workspace,
                    size_t workspace_bytes, hipStream_t stream);

/* Bytes of workspace swa_decode needs (split-K partial results). */
size_t swa_decode_workspace_bytes(const swa_params* params);

/*
 * swa_decode — one decode step per sequence against the rolling buffer.
 * Digest "읽기(read) 단계": the query at p reads the buffer entries of
 * positions p-W+1 .. p (plus sinks); digest "Pre-fill과의 상호작용": same
 * cache convention as prefill.
 *   q         : [batch][n_q_heads][head_dim] raw queries (rotated at pos[b]).
 *   k_cache, v_cache : caches that already hold position pos[b] (call
 *               swa_cache_write with n_tok = 1 first).
 *   pos       : device int32[batch], position of the token being decoded.
 *   out       : [batch][n_q_heads][head_dim];  lse: float32 [batch][n_q_heads]
 *               or NULL.
 *   workspace : >= swa_decode_workspace_bytes(params) bytes.
 * Slots whose implied position is negative (fewer than W tokens so far) are
 * never read.  Deterministic: no atomics.
 */
int swa_decode(const swa_params* params, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* pos, void* out, float* lse, void* workspace, size_t workspace_bytes,
               hipStream_t stream);

/*
 * swa_decode_step — a whole decode step per sequence: store the new token's
 * entry, then attend.  Digest "쓰기(write) 단계" then "읽기(read) 단계": the
 * key/value of position pos[b] go to slot(pos[b]) (the key rotated at
 * pos[b]), and the query at pos[b] reads positions pos[b]-W+1 .. pos[b]
 * (plus sinks), the new entry included.  The result, and the cache contents
 * afterwards, are those of swa_cache_write (n_tok = 1) followed by
 * swa_decode.  With bf16, head_dim 128 and 1, 2, 4 or 8 query heads per KV
 * head (4 with a dilated window) this is one launch (plus the combine when
 * the slots are split over several ranges): the work-group whose slot range
 * holds slot(pos[b]) stores the entry and attends to the new key and value
 * from its own registers rather than to what it reads back from that slot,
 * and every K/V byte it reads serves all query heads of its KV head.  Other
 * shapes run the two calls.
 *   q       : [batch][n_q_heads][head_dim] raw queries.
 *   k, v    : [batch][n_kv_heads][head_dim] raw new key / value of the token
 *             at pos[b] (the key is rotated here, the value stored as is).
 *   k_cache, v_cache : [batch][n_sink + window][n_kv_heads][head_dim],
 *             read and written (slot(pos[b]) of each sequence).
 *   pos, out, lse, workspace : as swa_decode (same workspace size).
 * Errors as swa_decode; nothing is launched when an argument is rejected.
 */
int swa_decode_step(const swa_params* params, const void* q, const void* k, const void* v,
                    void* k_cache, void* v_cache, const int32_t* pos, void* out, float* lse,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * swa_decode_step_noalloc — swa_decode_step without a workspace, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, layouts,
 * result and cache contents as swa_decode_step; the split-K partial results
 * go to a fixed array of the library (swa_noalloc_scratch_bytes() bytes, one
 * copy per device, held until the process ends).  Nothing is allocated.
 * Calls that overlap in time on one GPU share that array and race: issue
 * them one after the other (one stream, or synchronised streams).
 * Errors as swa_decode_step, and SWA_ERR_SCRATCH (nothing launched) when
 * swa_decode_workspace_bytes(params) exceeds the array.
 */
size_t swa_noalloc_scratch_bytes(void);
int swa_decode_step_noalloc(const swa_params* params, const void* q, const void* k, const void* v,
                            void* k_cache, void* v_cache, const int32_t* pos, void* out, float* lse,
                            hipStream_t stream);

/* Human-readable name of a swa_status value. */
const char* swa_status_string(int status);

/* Test hooks: run the same device index functions the kernels use.
 * swa_debug_slots: slots[t] = slot(positions[t]) for t < n (device arrays).
 * swa_debug_mask : mask[t] = 1 iff key position k_pos[t] is in the key set of
 *                  query position q_pos (device arrays). */
int swa_debug_slots(const swa_params* params, const int32_t* positions, int32_t n,
                    int32_t* slots, hipStream_t stream);
int swa_debug_mask(const swa_params* params, int32_t q_pos, const int32_t* k_pos, int32_t n,
                   uint8_t* mask, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SWA_H */
