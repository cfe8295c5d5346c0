/*
 * orthros.h — C ABI of the MI355X (gfx950) Orthros attention hot path (liborthros.so).
 *
 * Method: "Orthros: Phase-Aware Heterogeneous Attention for Efficient Transformers".
 *   - Base stream (§3.1 Eq. 4): every base token t attends, with its base query
 *     q_t = alpha (.) q_raw_t + beta, to the w most recent keys max(0, t-w+1) .. t (0-based,
 *     itself included) and appends its key/value to a full, never-evicted cache.
 *   - Output stream (§3.1 Eq. 5): tokens duplicated at prediction positions attend, with the
 *     output query q'_t = alpha' (.) q'_raw_t + beta', to every key 0 .. t; they never write
 *     keys or values.
 *   - Regimes (§3.2): pre-training duplicates every position (orthros_forward_pt);
 *     supervised fine-tuning duplicates the response positions only (orthros_forward_sft);
 *     prefilling runs the base stream over the prompt and one output row at the last prompt
 *     token (orthros_prefill, or orthros_prefill_chunk for a prompt arriving in chunks);
 *     decoding processes one new token per sequence as a base copy (cache append + window)
 *     and an output copy (full history) (orthros_decode_step, or orthros_decode_step_paged
 *     over a paged cache filled by orthros_paged_write).
 * The key/value and query projections (x W_K, x W_V, x W_Q) and the output projection are the
 * caller's: the library starts from head-split projections (Algorithm 1, the split-heads step)
 * and returns the per-head outputs of the two attention calls, before the heads are merged.
 *
 * Conventions shared by every call
 *   - Pointers are device pointers on the current HIP device unless a parameter says "host".
 *     The caller owns and allocates every buffer, including the workspace; the library never
 *     allocates, frees or keeps device memory between calls.
 *   - Every call only enqueues work on `stream` (0 = the null stream) and returns; none
 *     synchronises except orthros_read_device_status and orthros_timing_end.
 *   - Tensors are dense and row-major with the shapes given. Queries/keys/values/outputs use
 *     the head-split layout [batch, tokens, heads, head_dim]. The cache is head-major:
 *     cache_k/cache_v [batch, kv_heads, capacity, head_dim], so each (sequence, kv head)
 *     history is one contiguous stream. cache_len is int32 [batch].
 *   - Element type: shape.dtype for q/k/v/o/cache (fp32 or bf16). Scale-offset vectors are
 *     always fp32 [num_q_heads * head_dim] (one entry per query head and channel).
 *   - Grouped queries: query head h reads kv head h / (num_q_heads / num_kv_heads).
 *   - Every pointer must be 16-byte aligned. Outputs must not alias inputs.
 *   - bf16 arithmetic: scale-offset in fp32, scores and softmax in fp32, fp32 accumulation,
 *     output rounded once to bf16 (round to nearest even). The query enters the matrix cores
 *     and the probabilities enter the value product as bf16: rounded once for the windowed
 *     and pre-training rows (a few thousand keys), carried as a bf16 pair (value + rounding
 *     residue, two products) for the split-key rows (decode, the output rows of prefill and of
 *     short SFT responses), whose 100K-key rows would otherwise accumulate a relative error of
 *     order 3e-3. fp32 calls compute every step in fp32.
 *   - Return value: ORTHROS_OK (0) or a negative ORTHROS_E_* code. Arguments are validated
 *     before anything is enqueued, so a call that returns an argument error has no effect.
 */
#ifndef ORTHROS_H
#define ORTHROS_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ORTHROS_F32 = 0,
  ORTHROS_BF16 = 1
} orthros_dtype;

enum {
  ORTHROS_OK = 0,
  ORTHROS_E_INVALID = -1,      /* null pointer, non-positive size, misaligned pointer, a prompt
                                  longer than the cache capacity, keys/values overlapping the
                                  cache they are copied into, ... */
  ORTHROS_E_UNSUPPORTED = -2,  /* dtype / head_dim / head-group combination not built */
  ORTHROS_E_WORKSPACE = -3,    /* workspace missing or smaller than orthros_workspace_bytes */
  ORTHROS_E_LAUNCH = -4        /* a HIP launch or runtime call failed */
};

/* Sticky device status bits, read with orthros_read_device_status. */
enum {
  ORTHROS_STATUS_CACHE_FULL = 1, /* a decode step found cache_len == capacity: its token was
                                    not appended (its attention outputs are still exact); or a
                                    paged write found no room for a sequence's tokens */
  ORTHROS_STATUS_BAD_PAGE = 2    /* a block-table entry outside [0, num_pages) was met: page 0
                                    was read in its place (those outputs are meaningless) and
                                    nothing was written through it */
};

/* Problem shape, passed by host pointer. */
typedef struct {
  int32_t batch;          /* sequences, >= 1 */
  int32_t num_q_heads;    /* H_q >= 1 */
  int32_t num_kv_heads;   /* H_kv >= 1, divides H_q */
  int32_t head_dim;       /* d: 64 or 128 */
  int32_t window;         /* w >= 1: keys t-w+1 .. t (Eq. 4); w >= T is plain causal */
  int32_t dtype;          /* orthros_dtype */
  int64_t capacity;       /* cache slots per (sequence, kv head), >= 1 */
  float softmax_scale;    /* score scale; <= 0 selects 1/sqrt(head_dim) */
  int32_t reserved;       /* must be 0 */
} orthros_shape;

/* Scale-offset vectors of §3.1 (device pointers, fp32 [num_q_heads * head_dim] each). */
typedef struct {
  const float* alpha_base;
  const float* beta_base;
  const float* alpha_out;
  const float* beta_out;
} orthros_affine;

/* Bytes of workspace the forward calls on this shape need (0 if the shape is invalid or
 * max_rows_T < 1). max_rows_T is the largest number of output-stream rows per sequence that a
 * call using this workspace computes at once: 1 for prefill, decode and pre-training (whose
 * output rows do not use the workspace), R for orthros_forward_sft with R response rows. The
 * workspace holds the split partials of the few-row kernel and the sticky status word;
 * zero-fill it once when it is allocated (the status word must start at 0), and never share
 * it between calls that may run concurrently. */
size_t orthros_workspace_bytes(const orthros_shape* shape, int64_t max_rows_T);

/* Prefilling regime (§3.2, T_in = P-1, T_out = 1).
 *   q_base  [B, P, H_q, d]   base-stream raw queries (before the scale-offset)
 *   q_out   [B, 1, H_q, d]   raw query of the duplicated last prompt token
 *   k, v    [B, P, H_kv, d]  keys/values of the prompt
 *   cache_k, cache_v         [B, H_kv, capacity, d]: rows 0..P-1 are overwritten with k, v
 *   cache_len [B]            set to P
 *   o_base  [B, P, H_q, d]   Eq. 4 for every prompt position
 *   o_out   [B, 1, H_q, d]   Eq. 5 at position P-1 (keys 0..P-1)
 * Requires 1 <= P <= capacity (ORTHROS_E_INVALID otherwise).
 * Keys and values already in the cache: k and v may be the cache's own rows (k == cache_k and
 * v == cache_v here, cache_k + past_len * d elements for orthros_prefill_chunk), which the
 * two layouts allow only with one kv head and with B == 1 or capacity == P; the copy is then
 * skipped. Any other overlap of k or v with cache_k or cache_v is ORTHROS_E_INVALID. The same
 * holds for orthros_forward_pt / orthros_forward_sft with a cache and orthros_prefill_chunk;
 * the paged calls reject any overlap of k or v with the page pool. */
int orthros_prefill(const orthros_shape* shape, int64_t P,
                    const void* q_base, const void* q_out, const void* k, const void* v,
                    const orthros_affine* affine,
                    void* cache_k, void* cache_v, int32_t* cache_len,
                    void* o_base, void* o_out,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Decoding regime (§3.2, one new token per sequence).
 * For each sequence b with L = cache_len[b] (read on the device):
 *   the base copy attends over keys max(0, L-w+1) .. L and the output copy over 0 .. L,
 *   where key L is this step's (k_new, v_new); then (k_new, v_new) is written to cache row L
 *   and cache_len[b] becomes L+1. If L == capacity the attention outputs are still computed
 *   (over the L cached keys plus the new one) but nothing is appended, cache_len is left as
 *   is, and ORTHROS_STATUS_CACHE_FULL is set in the workspace's status word.
 *   q_base, q_out  [B, H_q, d];  k_new, v_new [B, H_kv, d];  o_base, o_out [B, H_q, d]
 *   max_len_hint   host upper bound on max_b cache_len[b] before the step; it only sizes the
 *                  split grid (any value >= 1 is correct; a close bound is fastest). */
int orthros_decode_step(const orthros_shape* shape,
                        const void* q_base, const void* q_out,
                        const void* k_new, const void* v_new,
                        const orthros_affine* affine,
                        void* cache_k, void* cache_v, int32_t* cache_len,
                        int64_t max_len_hint,
                        void* o_base, void* o_out,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* orthros_decode_step for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. It takes no workspace and
 * calls no allocating routine: the split partials live in a fixed array inside the library,
 * ORTHROS_NOALLOC_SCRATCH_BYTES bytes on each device, held from the moment the library's code
 * is loaded onto that device until the process ends. The sticky status bits (as in the
 * workspace's status word: ORTHROS_STATUS_CACHE_FULL) are OR-ed into *device_status, a
 * caller-owned device int32 that the caller zeroes.
 *   - Same arguments, outputs and rounding as orthros_decode_step, minus the workspace.
 *   - A step needs 2 B H_q nsplit (head_dim + 2) fp32 values (each of the three arrays rounded
 *     up to 256 bytes), where nsplit (1 .. 64) is the split count orthros_decode_step picks for
 *     max_len_hint; a step that needs more than ORTHROS_NOALLOC_SCRATCH_BYTES returns
 *     ORTHROS_E_WORKSPACE and enqueues nothing. The 16-sequence, 32-head, d 128 decode of
 *     131072-token caches needs about 1 MiB. fp32 calls use no partials.
 *   - Every call on one device shares that device's array: calls that may overlap in time on
 *     one device (other streams, other threads) race and give wrong results. Calls on one
 *     stream are ordered and safe.
 *   - The first call with a device current looks up the array's device address
 *     (hipGetSymbolAddress) and keeps it; make that first call before any graph capture.
 *   - The per-stage timing (orthros_timing_begin) does not record this call. */
#define ORTHROS_NOALLOC_SCRATCH_BYTES (8u << 20)
int orthros_decode_step_noalloc(const orthros_shape* shape,
                                const void* q_base, const void* q_out,
                                const void* k_new, const void* v_new,
                                const orthros_affine* affine,
                                void* cache_k, void* cache_v, int32_t* cache_len,
                                int64_t max_len_hint,
                                void* o_base, void* o_out,
                                int32_t* device_status, hipStream_t stream);

/* Pre-training regime (§3.2, T_in = 0, T_out = T): every position duplicated.
 *   q_base, q_out [B, T, H_q, d]; k, v [B, T, H_kv, d]; o_base, o_out [B, T, H_q, d]
 *   o_base[t] is Eq. 4 with q_base[t]; o_out[t] is Eq. 5 with q_out[t].
 *   cache_k/cache_v/cache_len: optional (all NULL, or all set with T <= capacity); when set,
 *   rows 0..T-1 receive k, v and cache_len is set to T. */
int orthros_forward_pt(const orthros_shape* shape, int64_t T,
                       const void* q_base, const void* q_out, const void* k, const void* v,
                       const orthros_affine* affine,
                       void* cache_k, void* cache_v, int32_t* cache_len,
                       void* o_base, void* o_out,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Supervised fine-tuning regime (§3.2, T_in = T - T_out, T_out = R >= 1): base rows at every
 * position, output rows only at the R response positions.
 *   q_base   [B, T, H_q, d]   base-stream raw queries
 *   q_out    [B, R, H_q, d]   raw queries of the duplicated response tokens, row r for position
 *                             out_pos[r]
 *   out_pos  int32 [R]        device array of positions in [0, T) (the same for every
 *                             sequence; any order, sorted is fastest; values outside [0, T)
 *                             are clamped into it)
 *   k, v     [B, T, H_kv, d]
 *   o_base   [B, T, H_q, d]   Eq. 4 at every position
 *   o_out    [B, R, H_q, d]   Eq. 5 at position out_pos[r] (keys 0 .. out_pos[r])
 *   cache_k/cache_v/cache_len: optional, as for orthros_forward_pt.
 *   workspace: at least orthros_workspace_bytes(shape, R) bytes. */
int orthros_forward_sft(const orthros_shape* shape, int64_t T,
                        const void* q_base, const void* q_out,
                        const int32_t* out_pos, int64_t R,
                        const void* k, const void* v,
                        const orthros_affine* affine,
                        void* cache_k, void* cache_v, int32_t* cache_len,
                        void* o_base, void* o_out,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Prefilling regime (§3.2) for a prompt that arrives in chunks: the cache already holds
 * past_len tokens of each sequence (cache_len[b] must equal past_len on entry) and C more are
 * prefilled. The chunk's keys/values go to cache rows past_len .. past_len+C-1 and cache_len
 * becomes past_len + C; the chunk's base rows attend over windows that reach back into the
 * cached tokens, and the output row at the chunk's last token (position past_len + C - 1)
 * attends over the whole cache. With past_len = 0 this is orthros_prefill.
 *   q_base  [B, C, H_q, d]; q_out [B, 1, H_q, d]; k, v [B, C, H_kv, d]
 *   o_base  [B, C, H_q, d]  Eq. 4 at positions past_len .. past_len+C-1
 *   o_out   [B, 1, H_q, d]  Eq. 5 at position past_len + C - 1
 * q_out and o_out may both be NULL: then no output-stream row is computed. The prefilling
 * regime duplicates only the prompt's last token (T_out = 1), so the chunks before the last
 * one need no output row, and skipping it saves a pass over the whole cache per chunk.
 * Exactly one of them NULL is ORTHROS_E_INVALID.
 * Requires past_len >= 0, C >= 1, past_len + C <= capacity. */
int orthros_prefill_chunk(const orthros_shape* shape, int64_t past_len, int64_t C,
                          const void* q_base, const void* q_out, const void* k, const void* v,
                          const orthros_affine* affine,
                          void* cache_k, void* cache_v, int32_t* cache_len,
                          void* o_base, void* o_out,
                          void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Training (§3.2 Pre-Training: the loss is taken at every position, and the scale-offset
 * vectors of §3.1 are learnable). orthros_forward_pt_lse is orthros_forward_pt (without the
 * cache) that also returns, per row of each stream, the natural-log log-sum-exp of the row's
 * scaled scores, lse_t = log sum_j exp(s q_t . k_j) over the row's keys:
 *   lse_base, lse_out  fp32 [B, H_q, T] (head-major, positions contiguous). */
int orthros_forward_pt_lse(const orthros_shape* shape, int64_t T,
                           const void* q_base, const void* q_out, const void* k, const void* v,
                           const orthros_affine* affine,
                           void* o_base, void* o_out, float* lse_base, float* lse_out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Gradients of the scale-offset vectors (device pointers, fp32 [num_q_heads * head_dim]). */
typedef struct {
  float* dalpha_base;
  float* dbeta_base;
  float* dalpha_out;
  float* dbeta_out;
} orthros_affine_grad;

/* Bytes of workspace orthros_backward_pt needs for sequences of T tokens (0 if invalid). Its
 * contents need no initialisation. */
size_t orthros_backward_workspace_bytes(const orthros_shape* shape, int64_t T);

/* Backward of the Pre-Training regime (both streams). Inputs are those of the forward
 * (q_base, q_out, k, v [.., d], affine), its outputs o_base, o_out and lse_base, lse_out (from
 * orthros_forward_pt_lse) and the loss gradients do_base, do_out [B, T, H_q, d]. Outputs:
 *   dq_base, dq_out [B, T, H_q, d]  gradients with respect to the raw queries (before the
 *                                   scale-offset)
 *   dk, dv [B, T, H_kv, d]          both streams' contributions, summed over the query heads of
 *                                   each kv head's group
 *   dgrad                           d alpha, d beta of each stream, summed over sequences and
 *                                   positions (host pointer to a struct of device pointers)
 * With P the softmax weights of a row, dP = dO V^T and D = rowsum(dO (.) O), the score
 * gradient is P (.) (dP - D); the kernels recompute P from the saved lse. bf16 calls take
 * bf16 operands on the matrix cores with fp32 accumulation and return dq, dk, dv in bf16 (the
 * scale-offset gradients are fp32); fp32 calls compute in fp32. Sums over rows run in a fixed
 * order, so results are deterministic. */
int orthros_backward_pt(const orthros_shape* shape, int64_t T,
                        const void* q_base, const void* q_out, const void* k, const void* v,
                        const orthros_affine* affine,
                        const void* o_base, const void* o_out,
                        const float* lse_base, const float* lse_out,
                        const void* do_base, const void* do_out,
                        void* dq_base, void* dq_out, void* dk, void* dv,
                        const orthros_affine_grad* dgrad,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Supervised fine-tuning (§3.2: output rows only at the R response positions) for training:
 * orthros_forward_sft_lse is orthros_forward_sft (without the cache) that also returns the
 * rows' log-sum-exp, lse_base fp32 [B, H_q, T] and lse_out fp32 [B, H_q, R] (response rows in
 * the order of out_pos); orthros_backward_sft is orthros_backward_pt for those rows: q_out,
 * o_out, do_out, dq_out are [B, R, H_q, d] and lse_out is [B, H_q, R]; the base stream is as
 * in pre-training. out_pos: device int32 [R], any order, clamped into [0, T). The workspace
 * holds orthros_backward_sft_workspace_bytes(shape, T, R) bytes. */
int orthros_forward_sft_lse(const orthros_shape* shape, int64_t T,
                            const void* q_base, const void* q_out,
                            const int32_t* out_pos, int64_t R,
                            const void* k, const void* v, const orthros_affine* affine,
                            void* o_base, void* o_out, float* lse_base, float* lse_out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);
size_t orthros_backward_sft_workspace_bytes(const orthros_shape* shape, int64_t T, int64_t R);
int orthros_backward_sft(const orthros_shape* shape, int64_t T,
                         const void* q_base, const void* q_out,
                         const int32_t* out_pos, int64_t R,
                         const void* k, const void* v, const orthros_affine* affine,
                         const void* o_base, const void* o_out,
                         const float* lse_base, const float* lse_out,
                         const void* do_base, const void* do_out,
                         void* dq_base, void* dq_out, void* dk, void* dv,
                         const orthros_affine_grad* dgrad,
                         void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Paged key/value cache: a pool of fixed-size pages shared by the batch, as a serving engine
 * keeps it (the batched decoding that "Orthros: Phase-Aware Heterogeneous Attention for
 * Efficient Transformers" names as future work in §5). Token t of sequence b lives in page
 * block_table[b * max_pages + t / page_size], slot t % page_size. Within a page the layout is
 * head-major like the contiguous cache, so each (page, kv head) is one run of page_size rows:
 *   k_pages, v_pages  [num_pages, H_kv, page_size, d] (shape.dtype)
 *   block_table       int32 [batch, max_pages], device; entries are page indices
 *   page_size         a power of two (1 .. 2^24); pages of 64 or more rows are fastest
 * A sequence's capacity is max_pages * page_size and must equal shape.capacity. The caller
 * owns the pool and the table and assigns pages; a sequence's table entries must name pages
 * for every position it holds or is about to receive. */
typedef struct {
  void* k_pages;
  void* v_pages;
  const int32_t* block_table;
  int64_t num_pages;
  int32_t page_size;
  int32_t max_pages;
} orthros_paged_kv;

/* orthros_decode_step over a paged cache (§3.2 decoding; same outputs, same rounding):
 * sequence b's keys 0 .. L-1 (L = cache_len[b]) are read through its table row, key L is this
 * step's (k_new, v_new), which is then written to position L through the table, and
 * cache_len[b] becomes L+1. A full sequence (L == capacity) sets ORTHROS_STATUS_CACHE_FULL
 * and is not appended; a bad table entry sets ORTHROS_STATUS_BAD_PAGE. Arguments as for
 * orthros_decode_step, with the cache given by `cache` (host pointer). */
int orthros_decode_step_paged(const orthros_shape* shape,
                              const void* q_base, const void* q_out,
                              const void* k_new, const void* v_new,
                              const orthros_affine* affine,
                              const orthros_paged_kv* cache, int32_t* cache_len,
                              int64_t max_len_hint,
                              void* o_base, void* o_out,
                              void* workspace, size_t workspace_bytes, hipStream_t stream);

/* orthros_prefill_chunk over a paged cache (§3.2 prefilling, the prompt arriving in chunks):
 * the chunk's keys/values go to positions past_len .. past_len+C-1 through the table
 * (cache_len[b] must equal past_len on entry and becomes past_len + C), its base rows' windows
 * and the output row read the cached tokens through the table. Same outputs as
 * orthros_prefill_chunk (q_out and o_out may both be NULL, as there). bf16 calls need pages of at least 64 rows (ORTHROS_E_UNSUPPORTED
 * otherwise); a bad table entry sets ORTHROS_STATUS_BAD_PAGE. */
int orthros_prefill_chunk_paged(const orthros_shape* shape, int64_t past_len, int64_t C,
                                const void* q_base, const void* q_out,
                                const void* k, const void* v, const orthros_affine* affine,
                                const orthros_paged_kv* cache, int32_t* cache_len,
                                void* o_base, void* o_out,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Appends T tokens per sequence to a paged cache: k, v [B, T, H_kv, d] go to positions
 * cache_len[b] .. cache_len[b] + T - 1 through the table, then cache_len[b] += T (prefilling a
 * prompt into pages, §3.2: the base tokens write the cache). A sequence without room for all T
 * tokens is left unchanged and ORTHROS_STATUS_CACHE_FULL is set. A sequence whose table
 * entries for those positions include one outside [0, num_pages) sets
 * ORTHROS_STATUS_BAD_PAGE: nothing is written through the bad entry and its cache_len is left
 * unchanged (rows written through its good entries lie past cache_len and count as unused).
 * orthros_prefill_chunk_paged writes the chunk the same way. Requires T >= 1. */
int orthros_paged_write(const orthros_shape* shape, int64_t T, const void* k, const void* v,
                        const orthros_paged_kv* cache, int32_t* cache_len,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Copies the workspace's sticky status word to *host_status (host pointer) after draining
 * `stream`; clears it on the device afterwards when `clear` is non-zero (the bits are sticky,
 * so a caller that has handled them resets them here). workspace_bytes is the workspace's
 * size, checked to hold the status word (ORTHROS_E_INVALID otherwise). Synchronous. */
int orthros_read_device_status(void* workspace, size_t workspace_bytes, int32_t* host_status,
                               int clear, hipStream_t stream);

/* Static, human-readable text for a return code. */
const char* orthros_status_string(int code);

/* Optional kernel timing. After orthros_timing_begin(), every call records a pair of HIP
 * events around each kernel it launches, on the call's stream. orthros_timing_end() waits for
 * them and writes, per stage, the summed milliseconds and the launch count (host arrays of
 * ORTHROS_NUM_STAGES entries), then stops recording. Host-side state; not thread-safe. */
enum {
  ORTHROS_STAGE_CACHE_WRITE = 0,  /* bulk cache write (prefill / pt / paged write) */
  ORTHROS_STAGE_BAND = 1,         /* banded flash kernel (Eq. 4 windows, Eq. 5 causal rows) */
  ORTHROS_STAGE_SPLIT_ROWS = 2,   /* split-key few-row kernel (output rows, decode pair) */
  ORTHROS_STAGE_MERGE = 3,        /* split merge */
  ORTHROS_STAGE_APPEND = 4,       /* decode append + length update */
  ORTHROS_STAGE_ROWS_F32 = 5,     /* fp32 row kernel */
  ORTHROS_STAGE_BWD_Q = 6,        /* backward: query side (and the query preparation) */
  ORTHROS_STAGE_BWD_KV = 7,       /* backward: key / value side */
  ORTHROS_STAGE_BWD_AFFINE = 8,   /* backward: scale-offset gradients */
  ORTHROS_NUM_STAGES = 9
};
int orthros_timing_begin(void);
int orthros_timing_end(double* stage_ms, int64_t* stage_launches);

#ifdef __cplusplus
}
#endif

#endif /* ORTHROS_H */
