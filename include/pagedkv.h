/*
 * pagedkv.h -- C ABI of libpagedkv.so, the PagedAttention hot path for AMD
 * Instinct MI355X (gfx950, CDNA4).
 *
 * The problem these calls solve is stated on the pages this library follows
 * (each call below cites its own passage):
 *   - gaoleia.github.io "PagedAttention 和 Continuous Batching": §1.3 (a
 *     physical block holds block_size tokens of K and of V, each token a
 *     [num_heads, head_dim] row), §1.4 (a per-request block table maps
 *     logical block i to a physical block), §1.5 (slot mapping), §1.6 (paged
 *     attention: gather each sequence's blocks in logical order, keep seq_len
 *     tokens, softmax(q K^T / sqrt(d)) V), §2.4-§2.5 (one step mixes decode
 *     rows with 512-token prefill chunks);
 *   - feifeigd.github.io "vLLM 架构详解", 一 PagedAttention (append_token writes
 *     a new token's K/V at its in-block position).
 *
 * Conventions shared by every call
 *   Memory.   Every pointer argument is a DEVICE pointer owned by the caller
 *             (pkv_swap_blocks also takes pinned host memory);
 *             the library allocates and frees nothing and keeps no state
 *             other than a thread-local error string and process-wide tuning
 *             knobs.  Buffers must stay alive until the enqueued work ends.
 *   Streams.  `stream` is a hipStream_t passed as void* (NULL = the default
 *             stream).  Calls only enqueue kernels, in stream order, and never
 *             synchronise: one or two per call, three for a varlen call
 *             with prefill-chunk rows (decode split, merge -- which also
 *             builds the prefill kernel's item plan -- then prefill).  The
 *             decode rows' split-K parts need their merge after the split
 *             kernel ends, and the prefill rows run in a persistent kernel of
 *             their own; the one-launch form (pkv_set_varlen_single_launch)
 *             is correct but slower on MI355X.
 *   Errors.   Arguments are validated on the host before anything is
 *             enqueued: a call that returns non-zero has enqueued nothing,
 *             except PKV_EHIP (the launch itself failed).  pkv_last_error()
 *             then describes the failure.
 *   Device contents that cannot be checked without a sync (block ids,
 *             seq_lens, positions, slots) are clamped so that no access leaves
 *             the caller's buffers; values outside their documented range give
 *             unspecified (but memory-safe) results.
 *   Layouts.  All arrays are dense and row-major.  KV pools are
 *             [num_blocks, block_size, num_kv_heads, head_dim]: the K (or V)
 *             row of token `off` of physical block `b` for KV head `h` starts
 *             at element ((b*block_size + off)*num_kv_heads + h)*head_dim.
 *             block_tables is int32 [num_seqs, max_blocks_per_seq]; entries past
 *             a sequence's last block are ignored (pad them with -1).
 *   Types.    dtype PKV_BF16 means query/key/value/caches hold bfloat16,
 *             PKV_F32 float32; outputs are always float32; accumulation is
 *             float32.  PKV_FP8_E4M3 pools (the *_fp8 calls) hold one OCP
 *             E4M3 byte per element with one float scale per pool, while
 *             query/key/value stay bfloat16 (key/value may also be float32).
 *             Pointers to data must be 16-byte aligned.
 *   GQA.      Query head hq reads KV head hq / (num_q_heads / num_kv_heads).
 *   Support.  head_dim in {64, 128}; block_size in {16, 32};
 *             num_q_heads % num_kv_heads == 0.  Other values return
 *             PKV_EUNSUPPORTED.
 *   Limits.   A token row (num_kv_heads * head_dim elements; for the E4M3
 *             writes, of the float32 or bfloat16 input) of at most 2^31 - 1
 *             bytes, block tables of at most 2^31 - 1 tokens
 *             (max_blocks_per_seq * block_size), and pools (and block-copy
 *             pools) under 2^62 bytes: the kernels' index arithmetic is exact
 *             inside these bounds, and larger arguments return
 *             PKV_EUNSUPPORTED before anything is enqueued.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2 } pkv_dtype;

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = 1,        /* bad pointer, size or alignment                  */
  PKV_EUNSUPPORTED = 2,  /* valid but not built (head_dim, block_size, ...)  */
  PKV_EWORKSPACE = 3,    /* workspace missing or smaller than required      */
  PKV_EHIP = 4           /* a HIP runtime call failed                       */
} pkv_status;

/* Library version, major*10000 + minor*100 + patch. */
int pkv_version(void);

/* Human-readable name of a status code (static storage). */
const char* pkv_status_string(int status);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* pkv_last_error(void);

/*
 * Slot mapping (gaoleia "PagedAttention 和 Continuous Batching" §1.5).
 *   For every new token t, let s be the sequence with
 *   query_start_loc[s] <= t < query_start_loc[s+1] and p = positions[t]:
 *     slot_mapping[t] = block_tables[s][p / block_size] * block_size
 *                       + p % block_size
 *   p < 0 (padding) gives -1, and so does a token outside every sequence or
 *   a position whose logical block is past max_blocks_per_seq or holds a
 *   negative id.
 *   block_tables    int32 [num_seqs, max_blocks_per_seq]      (device, read)
 *   positions       int32 [num_tokens]                        (device, read)
 *   query_start_loc int32 [num_seqs + 1], non-decreasing, 0 first (device)
 *   slot_mapping    int64 [num_tokens]                        (device, written)
 *   num_tokens may be 0 (nothing is enqueued).
 */
int pkv_compute_slot_mapping(const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                             const int32_t* positions, const int32_t* query_start_loc,
                             int32_t num_tokens, int32_t block_size, int64_t* slot_mapping,
                             void* stream);

/*
 * reshape_and_cache: write each new token's K and V rows into its slot
 * (feifeigd "vLLM 架构详解" 一 PagedAttention, append_token / _write_kv;
 * gaoleia §2.4, the decode step appends K6,V6 before attending).
 *   key, value              [num_tokens, num_kv_heads, head_dim]  (device, read)
 *   key_cache, value_cache  [num_blocks, block_size, num_kv_heads, head_dim]
 *                           (device, rows at the slots overwritten in place)
 *   slot_mapping            int64 [num_tokens]; -1 = skip this token; slots
 *                           >= num_blocks*block_size are skipped too.
 *   A bit copy (no conversion): key/value and the caches share `dtype`.
 *   Duplicate slots are a caller error (the winner is unspecified).
 */
int pkv_reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                          const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                          int32_t head_dim, int64_t num_blocks, int32_t block_size, pkv_dtype dtype,
                          void* stream);

/*
 * pkv_compute_slot_mapping followed by pkv_reshape_and_cache, fused into one
 * kernel launch (same results, bit for bit): each new token's slot is computed
 * as pkv_compute_slot_mapping defines it and its K and V rows are copied
 * there.  Arguments are those of the two calls; slot_mapping may be NULL
 * (slots are then not stored).  Tokens whose slot is -1 or beyond the pool are
 * skipped.
 */
int pkv_write_new_tokens(const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                         const int32_t* positions, const int32_t* query_start_loc, int32_t num_tokens,
                         int32_t block_size, const void* key, const void* value, void* key_cache,
                         void* value_cache, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                         pkv_dtype dtype, int64_t* slot_mapping, void* stream);

/*
 * FP8 KV cache (feifeigd "vLLM 架构详解" 三 生产级部署配置, 关键参数调优:
 * kv-cache-dtype fp8 halves KV-cache memory at a small loss of precision).
 * The pages fix neither format nor scaling; these calls use OCP FP8 E4M3
 * (bias 7, no infinities, largest finite 448) with one float scale per pool.
 * An element x is stored as the E4M3 code nearest to the float32 product
 * x * (1.0f / scale) -- the reciprocal rounded to float32 on the host, ties to
 * the even code, magnitudes beyond 448 saturating to +-448 -- and read back as
 * code value * scale.  key/value must be finite.
 *
 * pkv_reshape_and_cache_fp8 / pkv_write_new_tokens_fp8: as pkv_reshape_and_cache
 * / pkv_write_new_tokens, with key/value of in_dtype (PKV_BF16 or PKV_F32)
 * [num_tokens, num_kv_heads, head_dim] and key_cache/value_cache uint8
 * [num_blocks, block_size, num_kv_heads, head_dim] (E4M3 codes).
 * num_kv_heads * head_dim must be a multiple of 16.  k_scale and v_scale must
 * be positive and finite with finite reciprocals (else PKV_EINVAL).
 */
int pkv_reshape_and_cache_fp8(const void* key, const void* value, void* key_cache, void* value_cache,
                              const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                              int32_t head_dim, int64_t num_blocks, int32_t block_size, pkv_dtype in_dtype,
                              float k_scale, float v_scale, void* stream);
int pkv_write_new_tokens_fp8(const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                             const int32_t* positions, const int32_t* query_start_loc, int32_t num_tokens,
                             int32_t block_size, const void* key, const void* value, void* key_cache,
                             void* value_cache, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                             pkv_dtype in_dtype, float k_scale, float v_scale, int64_t* slot_mapping,
                             void* stream);

/*
 * Bytes of device workspace pkv_paged_attention_decode needs for this shape
 * on the CURRENT device (the split of the work depends on its compute-unit
 * count).  Returns 0 for shapes the library does not support.  dtype is the
 * pool type (PKV_FP8_E4M3 for pkv_paged_attention_decode_fp8).
 */
size_t pkv_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, pkv_dtype dtype);

/*
 * Paged decode attention (gaoleia §1.6): one query row per sequence.
 *   out[s][hq][:] = sum_j softmax_j(scale * q[s][hq] . K_j) V_j over the
 *   first seq_lens[s] tokens j of sequence s, K_j/V_j being the rows of KV head
 *   hq / (num_q_heads / num_kv_heads) found through block_tables[s].
 *   out          float32 [num_seqs, num_q_heads, head_dim]   (device, written)
 *   query        [num_seqs, num_q_heads, head_dim] of dtype  (device, read)
 *   key_cache, value_cache  pools as above (device, read)
 *   block_tables int32 [num_seqs, max_blocks_per_seq]; seq_lens int32 [num_seqs]
 *   seq_lens[s] == 0 gives a zero row.  seq_lens are clamped to
 *   max_blocks_per_seq*block_size; block ids to [0, num_blocks).
 *   max_seq_len  the caller's upper bound of seq_lens (host scalar).  It
 *                must be >= 0 and is otherwise not used: it neither sizes the
 *                workspace nor clamps seq_lens (seq_lens are only clamped to
 *                max_blocks_per_seq*block_size, as above), so a value below
 *                the true lengths changes nothing.
 *   workspace    >= pkv_decode_workspace_size(...) bytes, 256-byte aligned.
 *                Its first 4 bytes must be zero before the first call that
 *                uses it (zero-fill a new workspace once); every call leaves
 *                them zero again, and the rest of it is scratch.  Long
 *                sequences are split over several workers (split-K); the
 *                last part of the work is handed out in units from a counter
 *                in that first word, and a second kernel merges the parts
 *                (and resets the counter).  Calls sharing a workspace must
 *                be ordered (one stream).
 *   num_seqs <= 8192.
 */
int pkv_paged_attention_decode(float* out, const void* query, const void* key_cache,
                               const void* value_cache, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int64_t num_blocks, int32_t block_size, int32_t max_seq_len, float scale,
                               pkv_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode attention over E4M3 pools: pkv_paged_attention_decode with query
 * bfloat16 [num_seqs, num_q_heads, head_dim], key_cache/value_cache uint8
 * E4M3 codes, and every K element read as code value * k_scale, every V
 * element as code value * v_scale (the scales of the write).  Tiles are
 * widened to bfloat16 exactly in registers; k_scale is folded into `scale`
 * and v_scale into the final normalisation.  Workspace as for
 * pkv_decode_workspace_size(..., PKV_FP8_E4M3).
 */
int pkv_paged_attention_decode_fp8(float* out, const void* query, const void* key_cache, const void* value_cache,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                   int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int64_t num_blocks, int32_t block_size, int32_t max_seq_len, float scale,
                                   float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * One decode step in one call (gaoleia §2.4: the step first appends the new
 * token's K and V to the sequence's last block, then attends over every
 * token; §1.5 for the slot).  For each sequence s the new token is position
 * seq_lens[s] - 1:
 *   1. its rows key[s] and value[s] are written to its slot, exactly as
 *      pkv_write_new_tokens with positions[s] = seq_lens[s] - 1 and
 *      query_start_loc = 0, 1, ..., num_seqs would (no write when
 *      seq_lens[s] == 0, when seq_lens[s] > max_blocks_per_seq * block_size,
 *      or when the token's block id is outside [0, num_blocks));
 *   2. out = pkv_paged_attention_decode over the pools as step 1 left them.
 * Results equal those two calls bit for bit.  The write is fused into the
 * attention launch: the wavefront that attends over the sequence's last
 * chunk takes the new token's K/V from key/value and also stores them.
 *   key, value   [num_seqs, num_kv_heads, head_dim] of dtype (device, read)
 *   key_cache, value_cache  written at the new tokens' slots, read elsewhere
 *   Other arguments, the workspace and the limits as for
 *   pkv_paged_attention_decode (workspace from pkv_decode_workspace_size).
 *   No sequence may read a slot that another sequence's new token writes
 *   (such blocks must have been copied on write first).
 */
int pkv_decode_step(float* out, const void* query, const void* key, const void* value, void* key_cache,
                    void* value_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                    int32_t head_dim, int64_t num_blocks, int32_t block_size, int32_t max_seq_len, float scale,
                    pkv_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pkv_decode_step over E4M3 pools: query, key and value bfloat16; the write
 * encodes as pkv_write_new_tokens_fp8 (in_dtype PKV_BF16) and the attention
 * is pkv_paged_attention_decode_fp8, with the same k_scale / v_scale.
 */
int pkv_decode_step_fp8(float* out, const void* query, const void* key, const void* value, void* key_cache,
                        void* value_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int64_t num_blocks, int32_t block_size, int32_t max_seq_len, float scale,
                        float k_scale, float v_scale, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Shared prefixes (feifeigd.github.io "vLLM 架构详解" 一, 共享前缀的 Block
 * 复用: sequences that start with the same tokens -- a system prompt, the
 * prompt of parallel samples -- hold that prefix once, in physical blocks
 * whose reference count exceeds one).  These calls compute exactly what
 * pkv_paged_attention_decode / pkv_decode_step compute (the same results up
 * to float summation order), but read each group's shared blocks once for
 * all its members' query heads instead of once per member.
 *   prefix_groups  int32 [num_groups][3] (device, read): for group g,
 *                  (first_seq, num_seqs, shared_tokens): sequences first_seq
 *                  .. first_seq + num_seqs - 1 share their first
 *                  shared_tokens tokens, i.e. their block tables hold the
 *                  same block ids for those tokens (the prefix is read
 *                  through the table of first_seq).  Values are clamped to
 *                  the batch and shared_tokens is rounded down to a multiple
 *                  of 16 (the members read the rest through their own
 *                  tables, which is still exact).  A member shorter than the
 *                  prefix attends only its own seq_lens tokens.  Groups
 *                  should not overlap (a sequence in two groups is still
 *                  computed exactly, through one of them, with some work
 *                  repeated).  Tables that do not agree on the shared blocks
 *                  give unspecified (memory-safe) results.
 *   num_groups     host scalar, 0 .. 1024 (0: the plain call).
 *   pkv_decode_step_shared: as pkv_decode_step; a member's new token is
 *                  never read from the shared blocks (a decode step does not
 *                  write into a shared block: the host copies it first).
 *   dtype PKV_BF16 (and E4M3 pools through the _fp8 call); num_seqs <= 4096.
 *   workspace >= pkv_decode_shared_workspace_size(..., num_groups) bytes,
 *   256-byte aligned, first 4 bytes zero before its first use (as for
 *   pkv_paged_attention_decode); PKV_EUNSUPPORTED for float32 pools.
 */
size_t pkv_decode_shared_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size, pkv_dtype dtype, int32_t num_groups);
int pkv_paged_attention_decode_shared(float* out, const void* query, const void* key_cache,
                                      const void* value_cache, const int32_t* block_tables,
                                      int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int64_t num_blocks, int32_t block_size, int32_t max_seq_len, float scale,
                                      pkv_dtype dtype, const int32_t* prefix_groups, int32_t num_groups,
                                      void* workspace, size_t workspace_bytes, void* stream);
int pkv_paged_attention_decode_shared_fp8(float* out, const void* query, const void* key_cache,
                                          const void* value_cache, const int32_t* block_tables,
                                          int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                          int64_t num_blocks, int32_t block_size, int32_t max_seq_len, float scale,
                                          float k_scale, float v_scale, const int32_t* prefix_groups,
                                          int32_t num_groups, void* workspace, size_t workspace_bytes,
                                          void* stream);
int pkv_decode_step_shared(float* out, const void* query, const void* key, const void* value, void* key_cache,
                           void* value_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int64_t num_blocks, int32_t block_size, int32_t max_seq_len,
                           float scale, pkv_dtype dtype, const int32_t* prefix_groups, int32_t num_groups,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free decode attention, for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same computation, arguments (less
 * the workspace), layouts and errors as pkv_paged_attention_decode (F32 or
 * BF16 pools), and the same kernels.  The split-K workspace lives in a
 * static device array of the library of pkv_noalloc_scratch_bytes() bytes
 * (16 MiB) that every device running this call holds until the process ends;
 * the call itself allocates nothing.  A call that would need more scratch
 * (pkv_decode_workspace_size(...) above that size, e.g. more than about 3,000
 * sequences x KV heads of 8 heads per group) returns PKV_EUNSUPPORTED
 * before anything is enqueued.  All calls on one device share that array:
 * calls that overlap on one device (other streams, other host threads
 * without ordering) race and give wrong results; calls in one stream are
 * ordered and safe.  The array starts zero-filled and every call leaves its
 * counter word zero, so nothing needs clearing between calls.
 */
int pkv_paged_attention_decode_noalloc(float* out, const void* query, const void* key_cache,
                                       const void* value_cache, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int64_t num_blocks, int32_t block_size, int32_t max_seq_len, float scale,
                                       pkv_dtype dtype, void* stream);
/* Size in bytes of the static scratch of pkv_paged_attention_decode_noalloc. */
size_t pkv_noalloc_scratch_bytes(void);

/*
 * Bytes of device workspace pkv_paged_attention_varlen needs (current device).
 */
size_t pkv_varlen_workspace_size(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t max_query_len,
                                 int32_t block_size, pkv_dtype dtype);

/*
 * Varlen attention for a step that mixes prefill chunks and decode rows
 * (gaoleia §2.4-§2.5; fanquanpp.github.io "vLLM服务内部" 分块预填充).
 *   Sequence s owns query rows query_start_loc[s] .. query_start_loc[s+1]-1
 *   (q_s rows).  Row i of it sits at position seq_lens[s] - q_s + i and
 *   attends keys 0 .. that position (causal mask aligned to the end of the
 *   key range, so a chunk after c cached tokens sees c + i + 1 keys).  The K/V
 *   of the step's own tokens must already be in the cache
 *   (pkv_reshape_and_cache first).
 *   out    float32 [num_tokens, num_q_heads, head_dim]  (device, written)
 *   query  [num_tokens, num_q_heads, head_dim] of dtype (device, read)
 *   query_start_loc int32 [num_seqs + 1] with query_start_loc[num_seqs] ==
 *   num_tokens; max_query_len >= every q_s (host scalar); seq_lens[s] >= q_s.
 *   Rows of a sequence with seq_lens[s] < q_s are unspecified.
 *   workspace >= pkv_varlen_workspace_size(...) bytes, 256-byte aligned.
 *                Its first 8 bytes hold work counters: they must be zero
 *                before the first call that uses it (zero-fill a new
 *                workspace once); every call leaves them zero.  Calls
 *                sharing a workspace must not overlap.
 *   num_seqs <= 8192.
 *   The decode rows run first, through the split and merge kernels, then
 *   the chunks.  After pkv_set_varlen_single_launch(1), calls with bfloat16
 *   or E4M3 pools, head_dim 128, max_query_len > 1 and num_seqs <= 2048 run
 *   both in one launch instead (the decode rows' work queued after the
 *   chunks').
 */
int pkv_paged_attention_varlen(float* out, const void* query, const void* key_cache,
                               const void* value_cache, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* seq_lens,
                               const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens,
                               int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                               int32_t block_size, float scale, pkv_dtype dtype, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * Varlen attention over E4M3 pools: pkv_paged_attention_varlen with the pool
 * conventions of pkv_paged_attention_decode_fp8 (query bfloat16, pools E4M3
 * codes read as code value * k_scale / v_scale).  Workspace as for
 * pkv_varlen_workspace_size(..., PKV_FP8_E4M3).
 */
int pkv_paged_attention_varlen_fp8(float* out, const void* query, const void* key_cache, const void* value_cache,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                   const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens,
                                   int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks, int32_t block_size,
                                   float scale, float k_scale, float v_scale, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * Copy-on-write block copies inside the pools (lakecityint.com/news/209622
 * §3.2: before a sequence writes into a block other tables share, a fresh
 * block receives a copy of it and the writer's table is pointed there).
 *   For every pair i, block block_mapping[i][1] of key_cache becomes a bit
 *   copy of block block_mapping[i][0], and the same in value_cache.
 *   key_cache, value_cache  pools [num_blocks, ...] (device, read and written)
 *   block_mapping  int64 [num_pairs][2] (src, dst)     (device, read)
 *   block_bytes    bytes of one block of one pool (block_size * num_kv_heads
 *                  * head_dim * element size); a multiple of 16.
 *   Pairs with an id outside [0, num_blocks) are skipped.  Destinations must
 *   be distinct and no destination may also be a source of the same call
 *   (otherwise the result is unspecified).  num_pairs may be 0.
 */
int pkv_copy_blocks(void* key_cache, void* value_cache, const int64_t* block_mapping, int32_t num_pairs,
                    int64_t num_blocks, int64_t block_bytes, void* stream);

/*
 * Swap blocks between two pools, typically a GPU pool and a pinned host pool
 * (5688vip.com "vLLM核心机制" §3.3 and lakecityint §2.1: a preempted
 * sequence's blocks are moved to CPU memory and later brought back, possibly
 * into other physical blocks).
 *   For every pair i, block block_mapping[i][1] of dst_key (dst_value) becomes
 *   a bit copy of block block_mapping[i][0] of src_key (src_value).
 *   Each pool pointer is device memory of the current device or pinned host
 *   memory (hipHostMalloc, or a pinned torch tensor); pageable host memory is
 *   rejected with PKV_EINVAL.  src_value and dst_value may both be NULL (one
 *   pool is moved).  block_mapping is device or pinned host memory.
 *   Pairs with a src id outside [0, src_num_blocks) or a dst id outside
 *   [0, dst_num_blocks) are skipped; destinations must be distinct.
 *   One kernel moves every pair (host memory is accessed over PCIe through
 *   the device's mapping of it).
 */
int pkv_swap_blocks(const void* src_key, const void* src_value, void* dst_key, void* dst_value,
                    const int64_t* block_mapping, int32_t num_pairs, int64_t src_num_blocks,
                    int64_t dst_num_blocks, int64_t block_bytes, void* stream);

/*
 * Measurement and test knobs (process-wide; not needed for normal use).
 *
 * pkv_set_profile_events: when both are non-NULL, every later attention call
 * on this thread records `start` (a hipEvent_t) right before its dominant
 * kernel and `stop` right after it, on the call's stream, so a caller can
 * time that kernel alone: the split kernel of pkv_paged_attention_decode,
 * the prefill-chunk kernel of pkv_paged_attention_varlen.  NULL, NULL turns
 * it off.
 *
 * pkv_set_decode_workers: number of workers (wavefronts) the decode split
 * uses; 0 restores the default (compute units x pkv_get_waves_per_cu(),
 * lowered for a call whose block tables hold fewer chunks than that: at most
 * num_seqs x KV heads x ceil(group / 16) x ceil(max_blocks_per_seq x
 * block_size / 32) plus the segment cost per pair).  A forced count is used
 * as given.  The workspace size follows the setting (sized for the full
 * default count).  Used by tests to force many different split points.
 * Returns the previous value.
 *
 * pkv_set_waves_per_cu: default worker density per compute unit (4..16,
 * multiple of 4; default 4).  Returns the previous value.
 *
 * pkv_set_decode_segment_cost: virtual chunks (0..64, default 2) the decode
 * split charges for each (sequence, KV head) range a worker starts, so that
 * workers crossing more ranges get fewer real chunks (a new range costs a
 * dependent block-table load and a first-chunk round trip, two to three
 * chunks of streaming on MI355X).  0 splits by real chunks only.  The
 * shared-prefix calls always split by real chunks.  Results do not depend
 * on it beyond float reordering.  Returns the previous value (-1 for an
 * out-of-range argument).
 *
 * pkv_set_varlen_single_launch: 1 runs the mixed varlen calls described at
 * pkv_paged_attention_varlen in one launch, 0 (default) in the split +
 * merge + prefill launches (same results up to float reordering; the one
 * launch is the slower of the two on MI355X).  Returns the previous value
 * (-1 for an argument other than 0 or 1).
 *
 * pkv_set_decode_dynamic: the share (permille, 0..500) of the decode
 * split's chunks that is handed out in units of at least unit_chunks chunks
 * (1..4096, default 4) from a counter, to the wavefronts that finish their
 * static range first (the rest is split in equal static ranges).  0 gives a
 * fully static split; -1 (the default) chooses per call: 200 for E4M3
 * pools, 120 when the call has at most one (sequence, KV head, head tile)
 * pair per four workers, else 0.  Every unit's range is fixed by the call's
 * arguments, so results do not depend on which wavefront ran it.  Returns
 * the previous share (-2 for an out-of-range argument).
 */
int pkv_set_profile_events(void* start_event, void* stop_event);

/*
 * pkv_stream_read: enqueue a plain streaming read of `bytes` bytes (a multiple
 * of 16) at device pointer `buf` (16-byte aligned): the HBM read rate the part
 * reaches in practice, to quote beside its peak, and a read-only way to push
 * other data out of the caches before a cold timing.  Not part of the paged
 * attention method.  sink: device uint32 [sink_len], sink_len a multiple of 4
 * in [4, 262144]; the read uses sink_len / 4 workgroups and stores the XOR of
 * the words each wavefront read into one sink entry (so the XOR of the whole
 * sink is the XOR of the buffer's 32-bit words).  bytes == 0 enqueues nothing.
 * PKV_EINVAL for null pointers, misalignment or a bad length.
 */
int pkv_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t sink_len, void* stream);

int pkv_set_decode_workers(int32_t workers);
int pkv_set_waves_per_cu(int32_t waves);
int pkv_set_decode_segment_cost(int32_t chunks);
int pkv_set_decode_dynamic(int32_t permille, int32_t unit_chunks);
int pkv_set_varlen_single_launch(int32_t on);
int pkv_get_waves_per_cu(void);

#ifdef __cplusplus
}
#endif
#endif /* PAGEDKV_H */
