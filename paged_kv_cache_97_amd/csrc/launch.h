// Host-side launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Element type of the KV pools (queries are bf16 for BF16 and FP8, fp32 for F32).
enum class KvKind { F32, BF16, FP8 };

// Everything the decode kernels read; built and validated by the API layer.
struct DecodeArgs {
  float* out;                 // [B, Hq, D] (decode) or [T, Hq, D] (varlen rows)
  const void* query;          // [rows, Hq, D]
  const void* key_cache;      // [NB, BS, Hkv, D]
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  // Optional varlen row offsets [B + 1].  NULL: sequence s owns query/out row s.
  // Otherwise only sequences with exactly one row (decode rows) are handled,
  // at row qsl[s]; every other sequence is left untouched.
  const int32_t* qsl;
  int max_blocks;
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int group;                  // Hq / Hkv
  int head_dim;
  int head_tiles;             // ceil(group / 16)
  int tile_cols;              // min(group, 16)
  int64_t num_blocks;
  float scale_log2;           // scale * log2(e) (times k_scale for FP8 pools)
  float v_scale;              // multiplies every output (FP8 pools; 1 otherwise)
  int workers;                // wavefronts sharing the work (split points)
  // Virtual chunks charged at the start of every non-empty pair: the equal
  // split of the work is made over real + virtual chunks, so a wave whose
  // range crosses into a new pair (and pays the new pair's block-table and
  // first-chunk latency) gets that many fewer real chunks.  0: plain split.
  int seg_chunks;
  // Dynamic tail: the last dyn_permille / 1000 of the chunk space is cut into
  // units of at least unit_chunks chunks that wavefronts take from *counter
  // (zero on entry; the merge kernel resets it) after their static range.
  int dyn_permille;
  int unit_chunks;
  // Optional fused cache write (decode only, qsl == NULL): new_k / new_v
  // [B, Hkv, D] are the rows of each sequence's new token, position
  // seq_lens[s] - 1 (query element type: float32 for F32 pools, bfloat16
  // otherwise).  The token's slot is written and the attention takes the
  // token's K/V from these rows.  k_inv / v_inv: float32 reciprocals of the
  // pool scales (FP8 pools).
  const void* new_k;
  const void* new_v;
  float k_inv;
  float v_inv;
  // Optional (varlen calls whose prefill rows use the workgroup-shared
  // kernel): the merge launch carries one more workgroup that builds that
  // kernel's item plan here, for tables of prefill_max_tok tokens.
  int* prefill_plan;
  int prefill_max_tok;
  // Optional shared prefixes (the *_shared calls): groups int32 [num_groups][3]
  // = (first sequence, number of sequences, shared tokens).  The sequences of
  // a group read their first shared tokens through the first member's block
  // table in one pass for all their query heads.
  const int32_t* groups;
  int num_groups;
  int pre_pairs_cap;          // prefix pairs the workspace holds
  // workspace
  int* seq_group;             // [B] each sequence's group or -1 (prefix calls; split kernel writes it)
  int* gchunk;                // [num_groups + 1] chunk prefix sums of the prefix region
  int* gpair;                 // [num_groups + 1] prefix-pair prefix sums
  float* pre_ml;              // [pre slots][prefix_cols][2]  prefix parts: (max, sum) per column
  float* pre_o;               // [pre slots][prefix_cols][D]  prefix parts: unnormalised outputs
  int* cum;                   // [B + 1] chunk prefix sums (written by the split kernel)
  int* counter;               // the units taken so far (the workspace's first word)
  float* part_ml;             // [slots, tile_cols, 2]  (max, sum) in the log2 domain
  float* part_o;              // [slots, tile_cols, D]  unnormalised partial outputs
};

size_t decode_workspace_bytes(int num_seqs, int num_kv_heads, int group, int head_dim, int workers);
// Splits the workspace into the DecodeArgs pointers.
void decode_workspace_carve(DecodeArgs& a, void* ws, int head_dim);
// Shared-prefix calls: the decode workspace followed by the prefix region's
// tables and parts (num_groups groups).
size_t decode_prefix_workspace_bytes(int num_seqs, int num_kv_heads, int group, int head_dim, int workers,
                                     int num_groups);
void decode_prefix_workspace_carve(DecodeArgs& a, void* ws, int head_dim);
// Query columns of one prefix pair: four MFMA column tiles for head_dim 64,
// two for 128 (four would not fit the registers of a double-buffered pass).
constexpr int prefix_cols(int head_dim) { return head_dim == 128 ? 32 : 64; }
constexpr int kMaxPrefixGroups = 1024;
constexpr int kMaxPrefixSeqs = 4096;

hipError_t launch_decode(const DecodeArgs& a, int head_dim, int block_size, KvKind kind,
                         hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop);

hipError_t launch_slot_mapping(const int32_t* bt, int num_seqs, int max_blocks, const int32_t* pos,
                               const int32_t* qsl, int num_tokens, int block_size, int64_t* slots,
                               hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* kc, void* vc,
                                    const int64_t* slots, int num_tokens, int row_bytes,
                                    int64_t num_slots, hipStream_t stream);

hipError_t launch_write_tokens(const int32_t* bt, int num_seqs, int max_blocks, const int32_t* pos,
                               const int32_t* qsl, int num_tokens, int block_size, const void* key,
                               const void* value, void* kc, void* vc, int row_bytes, int64_t num_slots,
                               int64_t* slots, hipStream_t stream);

// Quantising variants: key/value rows of `in_kind` (BF16 or F32) are stored
// as E4M3 bytes of x * k_inv (v_inv); row_elems = num_kv_heads * head_dim
// (a multiple of 16).
hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, void* kc, void* vc,
                                        const int64_t* slots, int num_tokens, int row_elems, int64_t num_slots,
                                        KvKind in_kind, float k_inv, float v_inv, hipStream_t stream);
hipError_t launch_write_tokens_fp8(const int32_t* bt, int num_seqs, int max_blocks, const int32_t* pos,
                                   const int32_t* qsl, int num_tokens, int block_size, const void* key,
                                   const void* value, void* kc, void* vc, int row_elems, int64_t num_slots,
                                   int64_t* slots, KvKind in_kind, float k_inv, float v_inv, hipStream_t stream);


// Prefill-chunk rows of a varlen step (sequences with more than one query row).
struct PrefillArgs {
  float* out;                 // [T, Hq, D]
  const void* query;          // [T, Hq, D]
  const void* key_cache;
  const void* value_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* qsl;         // [B + 1]
  int max_blocks;
  int num_seqs;
  int num_q_heads;
  int num_kv_heads;
  int group;
  int64_t num_blocks;
  float scale_log2;
  float v_scale;              // multiplies every output (FP8 pools; 1 otherwise)
  int waves;                  // wavefronts in the grid
  int* plan;                  // workspace: item plan + work counter (prefill_plan_bytes)
};

// Workspace bytes of the prefill item plan for num_seqs sequences.
size_t prefill_plan_bytes(int num_seqs);

// Dispatches to the workgroup-shared kernel (bf16 or FP8 pools, head_dim 128;
// its plan built beforehand) or the per-wave kernel (other shapes).
hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int block_size, KvKind kind, int cus,
                          hipStream_t stream);
hipError_t launch_prefill_lds(const PrefillArgs& a, int block_size, bool fp8, int cus, hipStream_t stream);
// Whether launch_prefill takes the workgroup-shared kernel, whose item plan
// (PrefillArgs::plan) must have been built beforehand (DecodeArgs::prefill_plan).
bool prefill_uses_plan(int head_dim, KvKind kind);

// Mixed varlen steps whose prefill rows use the workgroup-shared kernel:
// prefill and decode rows in one launch of `grid` workgroups (one per
// compute unit).  The workspace holds the item counter and the count of
// finished workgroups (words 0 and 1, zero on entry and left zero) and
// 8 part slots per workgroup for the decode rows.  num_seqs <= kMixedMaxSeqs.
constexpr int kMixedMaxSeqs = 2048;
size_t mixed_workspace_bytes(int grid, int tile_cols, int head_dim);
hipError_t launch_mixed_varlen(const PrefillArgs& p, DecodeArgs d, void* workspace, int block_size, bool fp8,
                               int grid, hipStream_t stream);

// Whole-block copies for every (src, dst) pair of mapping (int64 [pairs][2]);
// src1/dst1 may be null (one pool).  Pairs with an id outside its pool are
// skipped.  streaming: non-temporal loads and stores (copies inside device
// memory); off for copies to or from pinned host memory.
hipError_t launch_block_copy(const void* src0, void* dst0, const void* src1, void* dst1, const int64_t* mapping,
                             int num_pairs, int64_t src_blocks, int64_t dst_blocks, int64_t block_bytes,
                             bool streaming, hipStream_t stream);

// Streaming read of bytes (a multiple of 16) from buf with `blocks`
// workgroups of 256 threads; sink receives one XOR word per wavefront
// (blocks * 4 words).
hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int blocks, hipStream_t stream);

}  // namespace pkv
