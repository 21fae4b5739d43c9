/*
 * gqa.h -- C ABI of the grouped-query attention library for MI355X (gfx950).
 *
 * The library computes, for every sequence b and query head a,
 *
 *     O[b,a] = softmax( scale * Q[b,a] K[b,g(a)]^T + M ) V[b,g(a)],
 *     g(a) = floor(a / r),  r = h_q / h_kv,
 *
 * which covers multi-head (h_kv = h_q), grouped-query (1 < h_kv < h_q) and
 * multi-query (h_kv = 1) attention with one code path.  Sources (web pages):
 *   [EffSeq]    "序列计算与存储", note.the0xka1.cc efficient-sequence-models:
 *               section 分组查询注意力 (formula, group map, shapes, causal or
 *               padding mask), 缓存字节 (cache layout (B, h_kv, T, d_h) read
 *               through the group index, never duplicated), 在线 softmax
 *               (running max, normalizer and unnormalized output).
 *   [AttnVar]   "第三章：MHA 的局限与 MQA、GQA、Flash Attention", sections 3.1
 *               (decode: the new token's K/V are appended, then all visible
 *               K/V are read), 3.3 (is_causal only fits equal Q/K lengths),
 *               3.5 (merging two partial softmax states).
 *   [MhaMqaGqa] zane-jiang mha-mqa-gqa, sections 4 (KV cache), 7 (one K/V
 *               tile serves all r query rows of its group), 9 (split the
 *               history when rows are few).
 *   [Ch09]      "第 09 章 GQA、MLA 与跨层 KV 共享", section 09.2 (absolute
 *               query position in cached decoding; reset clears K, V and the
 *               position together).
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller.  Layouts are
 *     dense row-major: Q and O are (B, h_q, S_q, d_h); K, V and the caches are
 *     (B, h_kv, T, d_h).  Integer arrays are device int32.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t passed as
 *     void*; NULL means the default stream).  Calls return once enqueued.
 *     The stream belongs to the calling thread's current device, the device
 *     every pointer refers to.
 *   - The library allocates no device memory.  Its only state is a per-device
 *     record that its kernels with more than 64 KiB of LDS have been allowed
 *     it (set on the first call on each device, safe under concurrent first
 *     calls); calls on different streams are independent.
 *   - Host-checkable argument errors return a status before any launch and
 *     leave every output untouched.  Launch failures return GQA_ERR_HIP.
 *   - Data conditions that only the device can see have defined results:
 *     lengths are clamped to [0, capacity]; a query row with no visible key
 *     is written as zeros; cache rows a query cannot see are never used, so
 *     they may hold any bits (NaN included).
 *   - `scale` multiplies Q K^T; it must be finite and > 0 (the pages fix it at
 *     1/sqrt(d_h); the Python binding passes that when given none).
 *   - Supported: in_dtype GQA_F32 with out_dtype GQA_F32 for 1 <= d_h <= 256
 *     (reference-precision path); in_dtype GQA_BF16 with out_dtype GQA_F32 or
 *     GQA_BF16 for d_h in {64, 128} (matrix-core path, fp32 accumulation).
 *     On the bf16 path of the prefill calls one (sequence, K/V head) of K or V
 *     must span at most 2^31 - 1 bytes: T_cap * d_h * 2 <= 2147483647
 *     (T_cap <= 8,388,607 at d_h 128), as the kernels address it with 32-bit
 *     buffer offsets.  Anything else returns GQA_ERR_UNSUPPORTED.
 *   - Alignment: bf16 tensors and fp32 outputs of the bf16 path need 16-byte
 *     aligned base pointers; fp32 tensors need 4-byte alignment.
 */
#ifndef GQA_H
#define GQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GQA_OK = 0,
  GQA_ERR_INVALID_ARGUMENT = 1,
  GQA_ERR_UNSUPPORTED = 2,
  GQA_ERR_WORKSPACE_TOO_SMALL = 3,
  GQA_ERR_HIP = 4,
  GQA_ERR_SCRATCH_LIMIT = 5
} gqa_status_t;

/* Size of the library's static device scratch used by gqa_decode_noalloc (per GPU). */
#define GQA_DECODE_SCRATCH_BYTES ((size_t)16 << 20)

typedef enum { GQA_F32 = 0, GQA_BF16 = 1 } gqa_dtype_t;

typedef enum { GQA_MASK_NONE = 0, GQA_MASK_CAUSAL = 1 } gqa_mask_t;

/*
 * Prefill: S_q = T queries at positions 0..T-1 attend to T keys.
 * Key j is visible to query i iff j < len_b and (mask == GQA_MASK_NONE or j <= i),
 * with len_b = kv_lens[b] clamped to [0, T] (kv_lens == NULL: len_b = T).
 * Causal masking is the [EffSeq] / [Ch09] 09.2 mask (-inf for j > i), applied
 * by selection; padding follows the per-sequence-length reading of [EffSeq].
 *
 *   q  (B, h_q, T, d_h)  in_dtype      k, v (B, h_kv, T, d_h) in_dtype
 *   o  (B, h_q, T, d_h)  out_dtype     kv_lens (B,) int32 or NULL
 * Errors: GQA_ERR_INVALID_ARGUMENT for a size < 1, h_q % h_kv != 0, a NULL or
 * misaligned tensor pointer, an unknown mask, a scale that is not finite and
 * positive; GQA_ERR_UNSUPPORTED for an unsupported dtype / d_h combination.
 */
int gqa_prefill(const void* q, const void* k, const void* v, void* o,
                int B, int h_q, int h_kv, int T, int d_h,
                int mask, const int32_t* kv_lens, float scale,
                int in_dtype, int out_dtype, void* stream);

/*
 * Chunked (offset) prefill: S_q queries of sequence b sit at absolute
 * positions q_pos0[b] + i (i = 0..S_q-1) and attend to a cache of capacity
 * T_cap whose first kv_lens[b] rows are valid ([MhaMqaGqa] section 7: every
 * packed row keeps its own causal position; [Ch09] 09.2: absolute positions).
 * Key j is visible to query i iff j < kv_lens[b] and (mask == NONE or
 * j <= q_pos0[b] + i).  With q_pos0 = 0, S_q = T_cap = T and kv_lens = T this
 * is gqa_prefill.  q_pos0 == NULL means kv_lens[b] - S_q (the chunk is the
 * newest S_q positions of the history) when S_q != T_cap, and 0 when S_q ==
 * T_cap: a chunk as long as the cache is a prefill, row i at position i, and
 * kv_lens then masks keys only, exactly as in gqa_prefill.  kv_lens == NULL
 * means T_cap.
 *
 *   q (B, h_q, S_q, d_h)  k_cache, v_cache (B, h_kv, T_cap, d_h)  o (B, h_q, S_q, d_h)
 * Errors: as gqa_prefill.
 */
int gqa_prefill_chunk(const void* q, const void* k_cache, const void* v_cache, void* o,
                      int B, int h_q, int h_kv, int S_q, int T_cap, int d_h,
                      int mask, const int32_t* kv_lens, const int32_t* q_pos0,
                      float scale, int in_dtype, int out_dtype, void* stream);

/*
 * Bytes of device workspace gqa_decode needs for these sizes (any
 * max_seq_len <= T_cap).  Returns 0 for invalid sizes and for the fp32 path,
 * which needs none.  `in_dtype` selects the path.
 */
size_t gqa_decode_workspace_bytes(int B, int h_q, int h_kv, int T_cap, int d_h, int in_dtype);

/*
 * Decode: one query per sequence (S_q = 1) attends to its KV cache in place,
 * every query head a reading cache head g(a) ([EffSeq] 缓存字节; [MhaMqaGqa]
 * section 7).  The query of sequence b sits at absolute position
 * p_b = q_pos[b] (q_pos == NULL: seq_lens[b] - 1) and sees keys
 * j < min(seq_lens[b], p_b + 1, max_seq_len) (clamped to [0, T_cap]).
 * The history is split across workgroups and the partial softmax states are
 * merged ([AttnVar] 3.5; [MhaMqaGqa] section 9).
 *
 *   q (B, h_q, 1, d_h) in_dtype     k_cache, v_cache (B, h_kv, T_cap, d_h) in_dtype
 *   seq_lens (B,) int32 = valid cache rows, the current token included
 *   q_pos (B,) int32 or NULL       o (B, h_q, 1, d_h) out_dtype
 *   max_seq_len: host bound on the visible length used to size the grid;
 *     <= 0 means T_cap; must be <= T_cap.
 *   workspace: device scratch of at least gqa_decode_workspace_bytes(...)
 *     bytes (may be NULL when that is 0); contents need no initialisation.
 * Errors: as gqa_prefill, plus max_seq_len > T_cap (INVALID_ARGUMENT) and
 * GQA_ERR_WORKSPACE_TOO_SMALL.
 */
int gqa_decode(const void* q, const void* k_cache, const void* v_cache,
               const int32_t* seq_lens, const int32_t* q_pos, void* o,
               int B, int h_q, int h_kv, int T_cap, int d_h, int max_seq_len,
               float scale, int in_dtype, int out_dtype,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * Append one new token's key and value to each sequence's cache: row
 * write_pos[b] of every cache head of sequence b receives k_new[b, :, 0, :]
 * and v_new[b, :, 0, :] ([AttnVar] 3.1; [MhaMqaGqa] section 4).  A write_pos
 * outside [0, T_cap) skips that sequence.  Lengths are the caller's: this
 * call never changes seq_lens, so appending the same token twice is the
 * caller's error ([Ch09] 09.4).
 *
 *   k_cache, v_cache (B, h_kv, T_cap, d_h) dtype   k_new, v_new (B, h_kv, 1, d_h) dtype
 *   write_pos (B,) int32
 * Errors: GQA_ERR_INVALID_ARGUMENT for a size < 1, a NULL or misaligned
 * pointer, an unknown dtype.
 */
int gqa_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                  const int32_t* write_pos, int B, int h_kv, int T_cap, int d_h,
                  int dtype, void* stream);

/*
 * Paged KV cache (the deployment form the pages list next to the contiguous
 * cache: [AttnVar] 3.6 names paging fragments, [MhaMqaGqa] §8 page metadata).
 * Page pools k_pages, v_pages are (n_pages, h_kv, page_size, d_h); token j of
 * sequence b is row j % page_size of page block_table[b][j / page_size], with
 * block_table (B, max_pages_per_seq) int32.  The capacity of a sequence is
 * T_cap = max_pages_per_seq * page_size; everything else is gqa_decode's
 * contract (positions, lengths, max_seq_len, workspace: size it with
 * gqa_decode_workspace_bytes(B, h_q, h_kv, T_cap, d_h, in_dtype)).  A page index
 * outside [0, n_pages) backs no key: its keys are not read and count as
 * invisible.  Supported: in_dtype GQA_BF16, d_h in {64, 128}, page_size a
 * multiple of 64; otherwise GQA_ERR_UNSUPPORTED.
 */
int gqa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                     const int32_t* block_table, const int32_t* seq_lens, const int32_t* q_pos, void* o,
                     int B, int h_q, int h_kv, int page_size, int n_pages, int max_pages_per_seq, int d_h,
                     int max_seq_len, float scale, int in_dtype, int out_dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * kv_append into a paged cache: token position write_pos[b] goes to row
 * write_pos[b] % page_size of page block_table[b][write_pos[b] / page_size].
 * A position outside [0, T_cap) or an invalid page index skips the sequence.
 * Rows must be a multiple of 16 bytes (d_h * element size); else UNSUPPORTED.
 */
int gqa_kv_append_paged(void* k_pages, void* v_pages, const void* k_new, const void* v_new,
                        const int32_t* block_table, const int32_t* write_pos, int B, int h_kv,
                        int page_size, int n_pages, int max_pages_per_seq, int d_h, int dtype, void* stream);

/*
 * One decode step in one call: gqa_kv_append(k_cache, v_cache, k_new, v_new,
 * write_pos) followed by gqa_decode(...) on the same caches, with the same
 * results (the pages' decode step appends the new token's K and V, then
 * attends over every visible row: [AttnVar] 3.1; [MhaMqaGqa] section 4).  On
 * the bf16 path with r = h_q / h_kv <= 16 the decode kernel itself writes the
 * new rows and uses them where it reads row write_pos[b], saving the append's
 * launch; otherwise the two run as two launches.  Arguments as gqa_decode and
 * gqa_kv_append (k_new, v_new (B, h_kv, 1, d_h) in_dtype, write_pos (B,)
 * int32; a write_pos outside [0, T_cap) skips that sequence's append).
 * Errors: those of both calls, all checked before anything is launched.
 */
int gqa_append_decode(const void* q, void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                      const int32_t* write_pos, const int32_t* seq_lens, const int32_t* q_pos, void* o,
                      int B, int h_q, int h_kv, int T_cap, int d_h, int max_seq_len,
                      float scale, int in_dtype, int out_dtype,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same step on a paged cache: gqa_kv_append_paged followed by
 * gqa_decode_paged, fused in the same way (an append whose page index is
 * outside the pool is skipped, and its row stays invisible).  Arguments and
 * errors as those two calls.
 */
int gqa_append_decode_paged(const void* q, void* k_pages, void* v_pages, const void* k_new, const void* v_new,
                            const int32_t* block_table, const int32_t* write_pos, const int32_t* seq_lens,
                            const int32_t* q_pos, void* o, int B, int h_q, int h_kv, int page_size, int n_pages,
                            int max_pages_per_seq, int d_h, int max_seq_len, float scale, int in_dtype,
                            int out_dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Rotary position encoding inside the attention kernels.  Every query head and
 * every stored key head is rotated by its position before the scores are formed
 * ([EffSeq] 分组查询注意力; [MhaMqaGqa] note under the parameter table), in the
 * form gqa_rope applies (pair (x[i], x[i + d_h/2]) turned by
 * p * rope_base^(-2 i / d_h)).  These calls rotate Q as the kernels load it, so
 * no rotated copy of Q is written; results are bit-identical to gqa_rope on Q
 * followed by the plain call.  Keys are not rotated here: K (prefill) or the
 * cache (decode) must already hold rotated keys, as gqa_rope on the prompt's K
 * and gqa_kv_append_rope leave them.
 *
 * gqa_prefill_rope: gqa_prefill with query row i rotated at position i.
 * Supported: in_dtype GQA_BF16, d_h in {64, 128}; rope_base finite and > 1
 * (else INVALID_ARGUMENT); GQA_F32 returns UNSUPPORTED.  Otherwise as gqa_prefill.
 */
int gqa_prefill_rope(const void* q, const void* k, const void* v, void* o,
                     int B, int h_q, int h_kv, int T, int d_h,
                     int mask, const int32_t* kv_lens, float scale, float rope_base,
                     int in_dtype, int out_dtype, void* stream);

/*
 * gqa_prefill_chunk with query row i of sequence b rotated at its absolute
 * position q_pos0[b] + i (q_pos0 == NULL: the default positions of
 * gqa_prefill_chunk).
 * Supported and errors as gqa_prefill_rope; otherwise as gqa_prefill_chunk.
 */
int gqa_prefill_chunk_rope(const void* q, const void* k_cache, const void* v_cache, void* o,
                           int B, int h_q, int h_kv, int S_q, int T_cap, int d_h,
                           int mask, const int32_t* kv_lens, const int32_t* q_pos0,
                           float scale, float rope_base, int in_dtype, int out_dtype, void* stream);

/*
 * One decode step with rotary encoding: gqa_kv_append_rope (k_new rotated at
 * write_pos[b]) followed by gqa_decode with each query rotated at its position
 * p_b = q_pos[b] (q_pos == NULL: seq_lens[b] - 1), bit-identical to those two
 * calls with gqa_rope applied to q at p_b.  As gqa_append_decode, the append
 * runs inside the decode kernel when r <= 16.  Arguments as gqa_append_decode
 * plus rope_base; supported and errors as gqa_prefill_rope.
 */
int gqa_append_decode_rope(const void* q, void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                           const int32_t* write_pos, const int32_t* seq_lens, const int32_t* q_pos, void* o,
                           int B, int h_q, int h_kv, int T_cap, int d_h, int max_seq_len,
                           float scale, float rope_base, int in_dtype, int out_dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Paged forms of the rotating calls: gqa_kv_append_paged_rope is
 * gqa_kv_append_paged with the new key rotated at write_pos[b] (supported and
 * errors as gqa_kv_append_rope, plus the paged arguments' errors), and
 * gqa_append_decode_paged_rope is gqa_kv_append_paged_rope followed by
 * gqa_decode_paged with each query rotated at its position, bit-identical to
 * those calls with gqa_rope applied to q, fused as gqa_append_decode_paged is.
 */
int gqa_kv_append_paged_rope(void* k_pages, void* v_pages, const void* k_new, const void* v_new,
                             const int32_t* block_table, const int32_t* write_pos, int B, int h_kv,
                             int page_size, int n_pages, int max_pages_per_seq, int d_h, float base, int dtype,
                             void* stream);
int gqa_append_decode_paged_rope(const void* q, void* k_pages, void* v_pages, const void* k_new,
                                 const void* v_new, const int32_t* block_table, const int32_t* write_pos,
                                 const int32_t* seq_lens, const int32_t* q_pos, void* o, int B, int h_q, int h_kv,
                                 int page_size, int n_pages, int max_pages_per_seq, int d_h, int max_seq_len,
                                 float scale, float rope_base, int in_dtype, int out_dtype, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * gqa_prefill that also writes the row log-sum-exp of the scaled scores,
 * lse[b][a][i] = log sum_j exp(scale q_i . k_j) over the visible keys (natural
 * log; -inf for a row with no visible key), fp32 (B, h_q, T).  These per-row
 * statistics are all the backward pass keeps of the forward ([EffSeq] 在线
 * softmax: the running maximum m and normalizer l; lse = m + log l).  Arguments
 * and errors as gqa_prefill, plus INVALID_ARGUMENT for a NULL or misaligned lse.
 */
int gqa_prefill_lse(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int h_q, int h_kv, int T, int d_h,
                    int mask, const int32_t* kv_lens, float scale,
                    int in_dtype, int out_dtype, void* stream);

/*
 * Bytes of device workspace gqa_prefill_backward needs: one float per query row.
 * Returns 0 for invalid sizes.
 */
size_t gqa_prefill_backward_workspace_bytes(int B, int h_q, int T);

/*
 * Gradients of prefill attention: dq (B, h_q, T, d_h), dk and dv (B, h_kv, T, d_h),
 * all fp32, from q, k, v (in_dtype), the forward output o (o_dtype, fp32 or bf16),
 * its gradient d_o (in_dtype) and the lse gqa_prefill_lse wrote.  Probabilities
 * are recomputed from lse rather than stored ([EffSeq] 在线 softmax; [AttnVar]
 * 3.5); the gradients of K/V head g are the sums over its r query heads, formed
 * inside the library without atomics (results are deterministic).  mask,
 * kv_lens and scale must be the ones the forward used.  dq, dk, dv are fully
 * written (zeros for keys no row can see).
 *   workspace: at least gqa_prefill_backward_workspace_bytes(B, h_q, T) bytes,
 *     4-byte aligned; contents need no initialisation.
 * Supported: in_dtype GQA_BF16 with d_h in {64, 128} and T * d_h * 2 <=
 * 2147483647 (32-bit offsets within one head); otherwise UNSUPPORTED.
 * Errors: as gqa_prefill for sizes, mask and scale; INVALID_ARGUMENT for a NULL
 * pointer or misalignment (bf16 tensors and gradients 16-byte aligned);
 * WORKSPACE_TOO_SMALL.
 */
int gqa_prefill_backward(const void* q, const void* k, const void* v, const void* o, const void* d_o,
                         const float* lse, float* dq, float* dk, float* dv,
                         int B, int h_q, int h_kv, int T, int d_h, int mask, const int32_t* kv_lens,
                         float scale, int in_dtype, int o_dtype,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Rotary position encoding.  Every query head and every stored key head is
 * rotated by its position before scores are formed ([EffSeq] 分组查询注意力:
 * all query heads and each key head actually kept are rotated; [MhaMqaGqa] note
 * under the parameter table: attention uses the position-processed Q and K).
 * The pages print no rotation formula; the one used is the common rotary form:
 * element i of a head row is paired with element i + d_h/2 and the pair at
 * position p is turned by p * theta_i, theta_i = base^(-2 i / d_h):
 *     y[i] = x[i] cos - x[i + d_h/2] sin,   y[i + d_h/2] = x[i + d_h/2] cos + x[i] sin.
 *
 * gqa_rope: x, y (B, H, S, d_h) of `dtype`; row s of sequence b is at position
 * pos0[b] + s (pos0 == NULL: s).  y may be x (in place); any other overlap is
 * undefined.  Use it on Q (H = h_q) before gqa_prefill / gqa_prefill_chunk /
 * gqa_decode, and on the prompt's K (H = h_kv) before it becomes the cache.
 * Angles: theta_i / 2 pi is passed to the kernels as a 64-bit fixed-point
 * fraction of a turn (computed on the host), the integer product with p drops
 * whole turns exactly, and the remaining fraction feeds the hardware sine and
 * cosine; the rotation itself is fp32, and bf16 results are rounded to nearest
 * even.  The calls that rotate inside the attention kernels use the same
 * arithmetic and give bit-identical results.
 * Errors: INVALID_ARGUMENT for a size < 1, a NULL or misaligned pointer, a base
 * that is not finite or not > 1; UNSUPPORTED for an odd d_h, d_h > 256 or an
 * unknown dtype.
 */
int gqa_rope(const void* x, void* y, const int32_t* pos0, int B, int H, int S, int d_h, float base,
             int dtype, void* stream);

/*
 * gqa_rope_qk: gqa_rope of q (B, h_q, S, d_h) into q_out and of k (B, h_kv, S,
 * d_h) into k_out, both at positions pos0[b] + s, in one launch (the rotations
 * named above for the query heads and the kept key heads).  Results are
 * bit-identical to two gqa_rope calls.  q_out may be q and k_out may be k (in
 * place); any other overlap among the four tensors is undefined.
 * Errors: as gqa_rope, for each tensor.
 */
int gqa_rope_qk(const void* q, void* q_out, const void* k, void* k_out, const int32_t* pos0, int B,
                int h_q, int h_kv, int S, int d_h, float base, int dtype, void* stream);

/*
 * gqa_kv_append with the key rotated at its own position write_pos[b] on the way
 * into the cache (values are copied unchanged).  Rows already in the cache are
 * never touched: a cache that other readers share stays read-only to them
 * ([Ch09] 09.4).  Arguments and skip rule as gqa_kv_append; base and errors as
 * gqa_rope.
 */
int gqa_kv_append_rope(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                       const int32_t* write_pos, int B, int h_kv, int T_cap, int d_h, float base,
                       int dtype, void* stream);

/*
 * gqa_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, serving loops that forbid allocation, harnesses without an
 * allocator): the same call, results bit-identical to gqa_decode with a large
 * enough workspace, but the partial softmax states live in a static device
 * array inside the library, GQA_DECODE_SCRATCH_BYTES (16 MiB) per GPU, held
 * from the first call on that GPU until the process ends.  Nothing is
 * allocated or freed by this call.  The caller still passes q, the caches,
 * seq_lens, q_pos and o.  Shapes whose split plan needs more than
 * GQA_DECODE_SCRATCH_BYTES (gqa_decode_workspace_bytes(...) above it) return
 * GQA_ERR_SCRATCH_LIMIT before anything is launched.  The scratch needs no
 * clearing: every partial state a call merges is written earlier in that call.
 * Every call on one GPU shares that GPU's array, so calls that overlap on one
 * GPU (concurrent streams, or threads) race and give undefined results; calls
 * ordered on one stream are safe.  The first call on each GPU must find that GPU
 * current (it records the array's address for it).  Arguments and other errors
 * as gqa_decode.
 */
int gqa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* seq_lens, const int32_t* q_pos, void* o,
                       int B, int h_q, int h_kv, int T_cap, int d_h, int max_seq_len,
                       float scale, int in_dtype, int out_dtype, void* stream);

/* Static, NUL-terminated description of a status code. */
const char* gqa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H */
