// C ABI of libpagedkv.so: argument validation, sizing and kernel dispatch.
// Every check runs on the host before anything is enqueued.
#include <stdarg.h>
#include <stdio.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <cmath>

#include "../../include/pagedkv.h"
#include "launch.h"

namespace {

thread_local char g_err[512] = "";
thread_local hipEvent_t g_ev_start = nullptr;
thread_local hipEvent_t g_ev_stop = nullptr;
std::atomic<int> g_workers_override{0};
std::atomic<int> g_waves_per_cu{4};
std::atomic<int> g_seg_chunks{2};              // virtual chunks charged per pair started
std::atomic<int> g_dyn_permille{-1};             // -1: chosen per call (dynamic_share)
std::atomic<int> g_unit_chunks{4};
std::atomic<int> g_varlen_single{0};           // mixed varlen steps in one launch (opt-in)

constexpr int kMaxSeqs = 8192;

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = 0;
  return PKV_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(pkv_dtype dt) { return dt == PKV_BF16 ? 2 : 4; }

// Limits that keep the kernels' index arithmetic exact: a token row (all KV
// heads of one token) of at most 2^31 - 1 bytes, since the kernels count row
// vectors in 32 bits, and a pool of blocks x block_bytes well inside int64
// (2^62 bytes), since they form byte and element offsets as block id x block
// size in 64 bits.
bool row_fits(int64_t row_bytes) { return row_bytes <= INT32_MAX; }
bool pool_addressable(int64_t blocks, int64_t block_bytes) {
  return (__int128)blocks * block_bytes < ((__int128)1 << 62);
}

int hip_fail(hipError_t e, const char* what) {
  return fail(PKV_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Compute units of the current device (0 on failure).
int current_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return cus;
}

// Wavefronts sharing a decode split: the forced count if one is set, else
// waves-per-CU times the compute units, but never more than max_chunks, an
// upper bound of the chunks the launch can hold (workers beyond the chunk
// count would only add empty parts for the merge to step over).
int decode_workers(int64_t max_chunks = INT64_MAX) {
  const int forced = g_workers_override.load();
  if (forced > 0) return forced;
  int cus = current_cus();
  if (cus <= 0) cus = 256;
  const int64_t full = (int64_t)cus * g_waves_per_cu.load();
  return (int)std::max<int64_t>(1, std::min(full, max_chunks));
}

// Attention calls: the table width in tokens (max_blocks_per_seq x
// block_size) is a 32-bit count in the kernels, like seq_lens, and the pools
// must be addressable.  Call after check_shape.
int check_attention_bounds(int32_t max_blocks_per_seq, int32_t block_size, int64_t num_blocks,
                           int32_t num_kv_heads, int32_t head_dim, pkv_dtype dtype) {
  if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX)
    return fail(PKV_EUNSUPPORTED, "block tables of %d blocks of %d tokens exceed 2^31 - 1 tokens", max_blocks_per_seq,
                block_size);
  const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * (dtype == PKV_FP8_E4M3 ? 1 : elem_bytes(dtype));
  if (!row_fits(row_bytes) || !pool_addressable(num_blocks, (int64_t)block_size * row_bytes))
    return fail(PKV_EUNSUPPORTED, "pool too large to address (%lld blocks of %d rows of %lld bytes)",
                (long long)num_blocks, block_size, (long long)row_bytes);
  return PKV_OK;
}

int check_shape(int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                pkv_dtype dtype) {
  if (num_q_heads <= 0 || num_kv_heads <= 0)
    return fail(PKV_EINVAL, "head counts must be positive (%d, %d)", num_q_heads, num_kv_heads);
  if (num_q_heads % num_kv_heads)
    return fail(PKV_EINVAL, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads, num_kv_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_EUNSUPPORTED, "head_dim %d (supported: 64, 128)", head_dim);
  if (block_size != 16 && block_size != 32)
    return fail(PKV_EUNSUPPORTED, "block_size %d (supported: 16, 32)", block_size);
  if (dtype != PKV_F32 && dtype != PKV_BF16 && dtype != PKV_FP8_E4M3)
    return fail(PKV_EUNSUPPORTED, "dtype %d", (int)dtype);
  return PKV_OK;
}

// Pool format of an attention call: element kind and, for E4M3 pools, the
// two scales (1 otherwise).
struct KvFormat {
  pkv::KvKind kind;
  float k_scale;
  float v_scale;
};

KvFormat plain_format(pkv_dtype dt) { return {dt == PKV_BF16 ? pkv::KvKind::BF16 : pkv::KvKind::F32, 1.f, 1.f}; }

// A pool scale must be positive and finite with a finite float32 reciprocal.
bool good_scale(float s) { return std::isfinite(s) && s > 0.f && std::isfinite(1.0f / s); }

// Upper bound of the chunks (real and virtual) a decode split can see:
// sequences x (KV head, head tile) pairs x chunks per pair, computed in 128
// bits and saturated so that no argument values overflow it.
int64_t chunk_bound(int64_t num_seqs, int64_t pairs_per_seq, int64_t max_tokens, int seg_chunks) {
  const __int128 n = (__int128)num_seqs * pairs_per_seq * ((max_tokens + 31) / 32 + seg_chunks);
  return n > (__int128)INT64_MAX ? INT64_MAX : (int64_t)n;
}

// The chunk count times the worker count must stay far inside int64 (the
// kernels multiply the two).
bool split_fits(int64_t chunks, int64_t workers) { return chunks < (int64_t(1) << 40) && workers <= 65536; }

// Share (permille) of a decode split's chunks handed out as units to the
// wavefronts that finish first.  Measured on MI355X: E4M3 pools gain 7 % from
// 150-200 (their static split ends with a long tail of late waves), so do
// batches of few long (sequence, KV head) pairs -- at most one pair per four
// workers, each pair spread over many workers -- (6 % on 16 sequences of
// 16k-32k tokens); batches of many short pairs lose 1-2 %, so they keep a
// fully static split.
int dynamic_share(pkv::KvKind kind, int64_t pairs, int workers) {
  const int forced = g_dyn_permille.load();
  if (forced >= 0) return forced;
  if (kind == pkv::KvKind::FP8) return 200;
  return 4 * pairs <= workers ? 120 : 0;
}

}  // namespace

extern "C" {

int pkv_version(void) { return 100; }

const char* pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "PKV_OK";
    case PKV_EINVAL: return "PKV_EINVAL: invalid argument";
    case PKV_EUNSUPPORTED: return "PKV_EUNSUPPORTED: unsupported configuration";
    case PKV_EWORKSPACE: return "PKV_EWORKSPACE: workspace missing or too small";
    case PKV_EHIP: return "PKV_EHIP: HIP runtime error";
    default: return "unknown pkv status";
  }
}

const char* pkv_last_error(void) { return g_err; }

int pkv_set_profile_events(void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(PKV_EINVAL, "profile events must be both set or both NULL");
  g_ev_start = static_cast<hipEvent_t>(start_event);
  g_ev_stop = static_cast<hipEvent_t>(stop_event);
  return ok();
}

int pkv_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t sink_len, void* stream) {
  if (bytes == 0) return ok();
  if (!buf || !sink) return fail(PKV_EINVAL, "null pointer");
  if (!aligned16(buf) || bytes % 16) return fail(PKV_EINVAL, "buffer must be 16-byte aligned and a multiple of 16 bytes");
  if (sink_len < 4 || sink_len > 262144 || sink_len % 4)
    return fail(PKV_EINVAL, "sink_len %d must be a multiple of 4 in [4, 262144]", sink_len);
  const hipError_t e = pkv::launch_stream_read(buf, (int64_t)bytes, sink, sink_len / 4,
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "stream read launch");
}

int pkv_set_decode_segment_cost(int32_t chunks) {
  if (chunks < 0 || chunks > 64) return -1;
  return g_seg_chunks.exchange(chunks);
}

int pkv_set_decode_dynamic(int32_t permille, int32_t unit_chunks) {
  if (permille < -1 || permille > 500 || unit_chunks < 1 || unit_chunks > 4096) return -2;
  g_unit_chunks.store(unit_chunks);
  return g_dyn_permille.exchange(permille);
}

int pkv_set_varlen_single_launch(int32_t on) {
  if (on != 0 && on != 1) return -1;
  return g_varlen_single.exchange(on);
}

int pkv_set_decode_workers(int32_t workers) {
  if (workers < 0 || workers > 65536) return -1;
  return g_workers_override.exchange(workers);
}

int pkv_set_waves_per_cu(int32_t waves) {
  if (waves < 4 || waves > 16 || waves % 4) return -1;
  return g_waves_per_cu.exchange(waves);
}

int pkv_get_waves_per_cu(void) { return g_waves_per_cu.load(); }

int pkv_compute_slot_mapping(const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                             const int32_t* positions, const int32_t* query_start_loc,
                             int32_t num_tokens, int32_t block_size, int64_t* slot_mapping,
                             void* stream) {
  if (num_tokens < 0 || num_seqs < 0 || max_blocks_per_seq < 0)
    return fail(PKV_EINVAL, "negative size (num_tokens %d, num_seqs %d, max_blocks %d)", num_tokens,
                num_seqs, max_blocks_per_seq);
  if (block_size <= 0) return fail(PKV_EINVAL, "block_size %d", block_size);
  if (num_tokens == 0) return ok();
  if (!positions || !query_start_loc || !slot_mapping || (num_seqs > 0 && max_blocks_per_seq > 0 && !block_tables))
    return fail(PKV_EINVAL, "null pointer");
  hipError_t e = pkv::launch_slot_mapping(block_tables, num_seqs, max_blocks_per_seq, positions,
                                          query_start_loc, num_tokens, block_size, slot_mapping,
                                          static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "slot_mapping launch");
}

int pkv_reshape_and_cache(const void* key, const void* value, void* key_cache, void* value_cache,
                          const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                          int32_t head_dim, int64_t num_blocks, int32_t block_size, pkv_dtype dtype,
                          void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks < 0 || block_size <= 0)
    return fail(PKV_EINVAL, "bad size (tokens %d, kv_heads %d, head_dim %d, blocks %lld, block_size %d)",
                num_tokens, num_kv_heads, head_dim, (long long)num_blocks, block_size);
  if (dtype != PKV_F32 && dtype != PKV_BF16) return fail(PKV_EUNSUPPORTED, "dtype %d", (int)dtype);
  const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * elem_bytes(dtype);
  if (row_bytes % 16) return fail(PKV_EUNSUPPORTED, "token row of %lld bytes is not a multiple of 16", (long long)row_bytes);
  if (!row_fits(row_bytes) || !pool_addressable(num_blocks, (int64_t)block_size * row_bytes))
    return fail(PKV_EUNSUPPORTED, "pool too large to address (%lld blocks of %d rows of %lld bytes)",
                (long long)num_blocks, block_size, (long long)row_bytes);
  if (num_tokens == 0) return ok();
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return fail(PKV_EINVAL, "null pointer");
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
    return fail(PKV_EINVAL, "key/value/cache pointers must be 16-byte aligned");
  hipError_t e = pkv::launch_reshape_and_cache(key, value, key_cache, value_cache, slot_mapping, num_tokens,
                                               (int)row_bytes, num_blocks * block_size,
                                               static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "reshape_and_cache launch");
}

int pkv_write_new_tokens(const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                         const int32_t* positions, const int32_t* query_start_loc, int32_t num_tokens,
                         int32_t block_size, const void* key, const void* value, void* key_cache,
                         void* value_cache, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                         pkv_dtype dtype, int64_t* slot_mapping, void* stream) {
  if (num_tokens < 0 || num_seqs < 0 || max_blocks_per_seq < 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      num_blocks < 0 || block_size <= 0)
    return fail(PKV_EINVAL, "bad size (tokens %d, seqs %d, max_blocks %d, kv_heads %d, head_dim %d, blocks %lld, "
                "block_size %d)", num_tokens, num_seqs, max_blocks_per_seq, num_kv_heads, head_dim,
                (long long)num_blocks, block_size);
  if (dtype != PKV_F32 && dtype != PKV_BF16) return fail(PKV_EUNSUPPORTED, "dtype %d", (int)dtype);
  const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * elem_bytes(dtype);
  if (row_bytes % 16) return fail(PKV_EUNSUPPORTED, "token row of %lld bytes is not a multiple of 16", (long long)row_bytes);
  if (!row_fits(row_bytes) || !pool_addressable(num_blocks, (int64_t)block_size * row_bytes))
    return fail(PKV_EUNSUPPORTED, "pool too large to address (%lld blocks of %d rows of %lld bytes)",
                (long long)num_blocks, block_size, (long long)row_bytes);
  if (num_tokens == 0) return ok();
  if (!positions || !query_start_loc || !key || !value || !key_cache || !value_cache ||
      (num_seqs > 0 && max_blocks_per_seq > 0 && !block_tables))
    return fail(PKV_EINVAL, "null pointer");
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
    return fail(PKV_EINVAL, "key/value/cache pointers must be 16-byte aligned");
  hipError_t e = pkv::launch_write_tokens(block_tables, num_seqs, max_blocks_per_seq, positions, query_start_loc,
                                          num_tokens, block_size, key, value, key_cache, value_cache, (int)row_bytes,
                                          num_blocks * block_size, slot_mapping, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "write_new_tokens launch");
}

static int check_fp8_write(int32_t num_tokens, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                           int32_t block_size, pkv_dtype in_dtype, float k_scale, float v_scale) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || num_blocks < 0 || block_size <= 0)
    return fail(PKV_EINVAL, "bad size (tokens %d, kv_heads %d, head_dim %d, blocks %lld, block_size %d)",
                num_tokens, num_kv_heads, head_dim, (long long)num_blocks, block_size);
  if (in_dtype != PKV_F32 && in_dtype != PKV_BF16)
    return fail(PKV_EUNSUPPORTED, "key/value dtype %d (bf16 or f32)", (int)in_dtype);
  const int64_t row_elems = (int64_t)num_kv_heads * head_dim;   // E4M3 rows: one byte per element
  if (row_elems % 16)
    return fail(PKV_EUNSUPPORTED, "token row of %lld elements is not a multiple of 16", (long long)row_elems);
  // the unquantised input rows (up to 4 bytes per element) must fit too
  if (!row_fits(4 * row_elems) || !pool_addressable(num_blocks, (int64_t)block_size * row_elems))
    return fail(PKV_EUNSUPPORTED, "pool too large to address (%lld blocks of %d rows of %lld elements)",
                (long long)num_blocks, block_size, (long long)row_elems);
  if (!good_scale(k_scale) || !good_scale(v_scale))
    return fail(PKV_EINVAL, "k_scale %g / v_scale %g must be positive and finite", k_scale, v_scale);
  return PKV_OK;
}

int pkv_reshape_and_cache_fp8(const void* key, const void* value, void* key_cache, void* value_cache,
                              const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                              int32_t head_dim, int64_t num_blocks, int32_t block_size, pkv_dtype in_dtype,
                              float k_scale, float v_scale, void* stream) {
  int st = check_fp8_write(num_tokens, num_kv_heads, head_dim, num_blocks, block_size, in_dtype, k_scale, v_scale);
  if (st != PKV_OK) return st;
  if (num_tokens == 0) return ok();
  if (!key || !value || !key_cache || !value_cache || !slot_mapping) return fail(PKV_EINVAL, "null pointer");
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
    return fail(PKV_EINVAL, "key/value/cache pointers must be 16-byte aligned");
  hipError_t e = pkv::launch_reshape_and_cache_fp8(
      key, value, key_cache, value_cache, slot_mapping, num_tokens, num_kv_heads * head_dim, num_blocks * block_size,
      in_dtype == PKV_BF16 ? pkv::KvKind::BF16 : pkv::KvKind::F32, 1.0f / k_scale, 1.0f / v_scale,
      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "reshape_and_cache_fp8 launch");
}

int pkv_write_new_tokens_fp8(const int32_t* block_tables, int32_t num_seqs, int32_t max_blocks_per_seq,
                             const int32_t* positions, const int32_t* query_start_loc, int32_t num_tokens,
                             int32_t block_size, const void* key, const void* value, void* key_cache,
                             void* value_cache, int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                             pkv_dtype in_dtype, float k_scale, float v_scale, int64_t* slot_mapping, void* stream) {
  int st = check_fp8_write(num_tokens, num_kv_heads, head_dim, num_blocks, block_size, in_dtype, k_scale, v_scale);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || max_blocks_per_seq < 0)
    return fail(PKV_EINVAL, "negative size (seqs %d, max_blocks %d)", num_seqs, max_blocks_per_seq);
  if (num_tokens == 0) return ok();
  if (!positions || !query_start_loc || !key || !value || !key_cache || !value_cache ||
      (num_seqs > 0 && max_blocks_per_seq > 0 && !block_tables))
    return fail(PKV_EINVAL, "null pointer");
  if (!aligned16(key) || !aligned16(value) || !aligned16(key_cache) || !aligned16(value_cache))
    return fail(PKV_EINVAL, "key/value/cache pointers must be 16-byte aligned");
  hipError_t e = pkv::launch_write_tokens_fp8(
      block_tables, num_seqs, max_blocks_per_seq, positions, query_start_loc, num_tokens, block_size, key, value,
      key_cache, value_cache, num_kv_heads * head_dim, num_blocks * block_size, slot_mapping,
      in_dtype == PKV_BF16 ? pkv::KvKind::BF16 : pkv::KvKind::F32, 1.0f / k_scale, 1.0f / v_scale,
      static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "write_new_tokens_fp8 launch");
}

int pkv_copy_blocks(void* key_cache, void* value_cache, const int64_t* block_mapping, int32_t num_pairs,
                    int64_t num_blocks, int64_t block_bytes, void* stream) {
  if (num_pairs < 0 || num_blocks < 0 || block_bytes <= 0)
    return fail(PKV_EINVAL, "bad size (pairs %d, blocks %lld, block_bytes %lld)", num_pairs,
                (long long)num_blocks, (long long)block_bytes);
  if (block_bytes % 16) return fail(PKV_EINVAL, "block_bytes %lld is not a multiple of 16", (long long)block_bytes);
  if (!pool_addressable(num_blocks, block_bytes))
    return fail(PKV_EUNSUPPORTED, "pool too large to address (%lld blocks of %lld bytes)", (long long)num_blocks,
                (long long)block_bytes);
  if (num_pairs == 0) return ok();
  if (!key_cache || !value_cache || !block_mapping) return fail(PKV_EINVAL, "null pointer");
  if (!aligned16(key_cache) || !aligned16(value_cache)) return fail(PKV_EINVAL, "pools must be 16-byte aligned");
  hipError_t e = pkv::launch_block_copy(key_cache, key_cache, value_cache, value_cache, block_mapping, num_pairs,
                                        num_blocks, num_blocks, block_bytes, true, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "copy_blocks launch");
}

// Device address of `p` for a kernel on the current device: device memory of
// that device, or pinned host memory (through its device mapping).  Returns
// false for pageable host memory or another device's memory.
static bool kernel_address(const void* p, const void** out, const char* name) {
  hipPointerAttribute_t attr;
  memset(&attr, 0, sizeof attr);
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();                  // do not leave the query's error for the next launch check
    fail(PKV_EINVAL, "%s is neither device memory nor pinned host memory", name);
    return false;
  }
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (attr.type == hipMemoryTypeDevice && attr.device == dev) {
    *out = p;
    return true;
  }
  if (attr.type == hipMemoryTypeHost && attr.devicePointer != nullptr) {
    *out = attr.devicePointer;
    return true;
  }
  fail(PKV_EINVAL, "%s is neither memory of the current device nor pinned host memory (type %d, device %d)", name,
       (int)attr.type, attr.device);
  return false;
}

int pkv_swap_blocks(const void* src_key, const void* src_value, void* dst_key, void* dst_value,
                    const int64_t* block_mapping, int32_t num_pairs, int64_t src_num_blocks,
                    int64_t dst_num_blocks, int64_t block_bytes, void* stream) {
  if (num_pairs < 0 || src_num_blocks < 0 || dst_num_blocks < 0 || block_bytes <= 0)
    return fail(PKV_EINVAL, "bad size (pairs %d, blocks %lld/%lld, block_bytes %lld)", num_pairs,
                (long long)src_num_blocks, (long long)dst_num_blocks, (long long)block_bytes);
  if (block_bytes % 16) return fail(PKV_EINVAL, "block_bytes %lld is not a multiple of 16", (long long)block_bytes);
  if (!pool_addressable(src_num_blocks, block_bytes) || !pool_addressable(dst_num_blocks, block_bytes))
    return fail(PKV_EUNSUPPORTED, "pool too large to address (%lld / %lld blocks of %lld bytes)",
                (long long)src_num_blocks, (long long)dst_num_blocks, (long long)block_bytes);
  if (num_pairs == 0) return ok();
  if (!src_key || !dst_key || !block_mapping) return fail(PKV_EINVAL, "null pointer");
  if ((src_value == nullptr) != (dst_value == nullptr))
    return fail(PKV_EINVAL, "src_value and dst_value must be both set or both NULL");
  if (!aligned16(src_key) || !aligned16(dst_key) || !aligned16(src_value) || !aligned16(dst_value))
    return fail(PKV_EINVAL, "pools must be 16-byte aligned");
  const void *sk, *dk, *sv = nullptr, *dv = nullptr, *map;
  if (!kernel_address(src_key, &sk, "src_key") || !kernel_address(dst_key, &dk, "dst_key") ||
      !kernel_address(block_mapping, &map, "block_mapping"))
    return PKV_EINVAL;
  if (src_value && (!kernel_address(src_value, &sv, "src_value") || !kernel_address(dst_value, &dv, "dst_value")))
    return PKV_EINVAL;
  hipError_t e = pkv::launch_block_copy(sk, const_cast<void*>(dk), sv, const_cast<void*>(dv),
                                        static_cast<const int64_t*>(map), num_pairs, src_num_blocks, dst_num_blocks,
                                        block_bytes, false, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ok() : hip_fail(e, "swap_blocks launch");
}

size_t pkv_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, pkv_dtype dtype) {
  if (num_seqs < 0 || num_seqs > kMaxSeqs) return 0;
  if (check_shape(num_q_heads, num_kv_heads, head_dim, block_size, dtype) != PKV_OK) return 0;
  return pkv::decode_workspace_bytes(num_seqs, num_kv_heads, num_q_heads / num_kv_heads, head_dim,
                                     decode_workers());
}

static int run_decode(float* out, const void* query, const void* key_cache, const void* value_cache,
                      const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                      const int32_t* qsl, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int64_t num_blocks, int32_t block_size, int32_t max_seq_len,
                      float scale, KvFormat fmt, void* workspace, size_t workspace_bytes,
                      hipStream_t stream, const void* new_k = nullptr, const void* new_v = nullptr,
                      int* prefill_plan = nullptr, const int32_t* groups = nullptr, int num_groups = 0) {
  const int group = num_q_heads / num_kv_heads;
  const int head_tiles = (group + 15) / 16;
  const int seg_chunks = num_groups > 0 ? 0 : g_seg_chunks.load();
  const int64_t max_chunks = chunk_bound(num_seqs, (int64_t)num_kv_heads * head_tiles,
                                         (int64_t)max_blocks_per_seq * block_size, seg_chunks);
  const int workers = decode_workers(max_chunks);
  if (!split_fits(max_chunks, workers))
    return fail(PKV_EUNSUPPORTED, "problem too large for the split arithmetic");
  const size_t need = num_groups > 0
                          ? pkv::decode_prefix_workspace_bytes(num_seqs, num_kv_heads, group, head_dim, workers,
                                                               num_groups)
                          : pkv::decode_workspace_bytes(num_seqs, num_kv_heads, group, head_dim, workers);
  if (!workspace || workspace_bytes < need)
    return fail(PKV_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(PKV_EINVAL, "workspace must be 256-byte aligned");
  pkv::DecodeArgs a{};
  a.out = out;
  a.query = query;
  a.key_cache = key_cache;
  a.value_cache = value_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.qsl = qsl;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.head_dim = head_dim;
  a.head_tiles = head_tiles;
  a.tile_cols = group < 16 ? group : 16;
  a.num_blocks = num_blocks;
  a.scale_log2 = scale * fmt.k_scale * 1.4426950408889634f;
  a.v_scale = fmt.v_scale;
  a.workers = workers;
  a.seg_chunks = seg_chunks;
  a.dyn_permille = dynamic_share(fmt.kind, (int64_t)num_seqs * num_kv_heads * head_tiles, workers);
  a.unit_chunks = g_unit_chunks.load();
  a.new_k = new_k;
  a.new_v = new_v;
  a.k_inv = fmt.kind == pkv::KvKind::FP8 ? 1.0f / fmt.k_scale : 1.0f;
  a.v_inv = fmt.kind == pkv::KvKind::FP8 ? 1.0f / fmt.v_scale : 1.0f;
  a.prefill_plan = prefill_plan;
  a.prefill_max_tok = max_blocks_per_seq * block_size;
  a.groups = groups;
  a.num_groups = num_groups;
  if (num_groups > 0)
    pkv::decode_prefix_workspace_carve(a, workspace, head_dim);
  else
    pkv::decode_workspace_carve(a, workspace, head_dim);
  (void)max_seq_len;
  hipError_t e = pkv::launch_decode(a, head_dim, block_size, fmt.kind, stream, g_ev_start, g_ev_stop);
  return e == hipSuccess ? ok() : hip_fail(e, "decode launch");
}

static int decode_impl(float* out, const void* query, const void* key_cache, const void* value_cache,
                       const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                       int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int64_t num_blocks, int32_t block_size, int32_t max_seq_len, float scale, pkv_dtype dtype,
                       KvFormat fmt, void* workspace, size_t workspace_bytes, void* stream,
                       const void* new_k = nullptr, const void* new_v = nullptr,
                       const int32_t* groups = nullptr, int32_t num_groups = 0) {
  int st = check_shape(num_q_heads, num_kv_heads, head_dim, block_size, dtype);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || num_seqs > kMaxSeqs) return fail(PKV_EUNSUPPORTED, "num_seqs %d (max %d)", num_seqs, kMaxSeqs);
  if (num_groups < 0) return fail(PKV_EINVAL, "num_groups %d", num_groups);
  if (num_groups > 0) {
    if (dtype == PKV_F32) return fail(PKV_EUNSUPPORTED, "shared prefixes need bf16 or E4M3 pools");
    if (num_groups > pkv::kMaxPrefixGroups)
      return fail(PKV_EUNSUPPORTED, "num_groups %d (max %d)", num_groups, pkv::kMaxPrefixGroups);
    if (num_seqs > pkv::kMaxPrefixSeqs)
      return fail(PKV_EUNSUPPORTED, "num_seqs %d with shared prefixes (max %d)", num_seqs, pkv::kMaxPrefixSeqs);
    if (!groups) return fail(PKV_EINVAL, "null pointer (prefix groups)");
  }
  if (max_blocks_per_seq < 0 || num_blocks < 0 || max_seq_len < 0)
    return fail(PKV_EINVAL, "negative size");
  st = check_attention_bounds(max_blocks_per_seq, block_size, num_blocks, num_kv_heads, head_dim, dtype);
  if (st != PKV_OK) return st;
  if (num_seqs == 0) return ok();
  if (!out || !query || !seq_lens || (max_blocks_per_seq > 0 && (!block_tables || !key_cache || !value_cache)))
    return fail(PKV_EINVAL, "null pointer");
  if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache))
    return fail(PKV_EINVAL, "out/query/cache pointers must be 16-byte aligned");
  if (!std::isfinite(scale)) return fail(PKV_EINVAL, "scale is not finite");
  if (max_blocks_per_seq > 0 && num_blocks == 0) return fail(PKV_EINVAL, "empty pool with a non-empty block table");
  return run_decode(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, seq_lens, nullptr,
                    num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size, max_seq_len,
                    scale, fmt, workspace, workspace_bytes, static_cast<hipStream_t>(stream), new_k, new_v,
                    nullptr, groups, num_groups);
}

int pkv_paged_attention_decode(float* out, const void* query, const void* key_cache,
                               const void* value_cache, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               int64_t num_blocks, int32_t block_size, int32_t max_seq_len, float scale,
                               pkv_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype == PKV_FP8_E4M3)
    return fail(PKV_EINVAL, "E4M3 pools need their scales: use pkv_paged_attention_decode_fp8");
  return decode_impl(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, num_blocks, block_size, max_seq_len, scale, dtype,
                     plain_format(dtype), workspace, workspace_bytes, stream);
}

int pkv_paged_attention_decode_fp8(float* out, const void* query, const void* key_cache, const void* value_cache,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                   int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int64_t num_blocks, int32_t block_size, int32_t max_seq_len, float scale,
                                   float k_scale, float v_scale, void* workspace, size_t workspace_bytes,
                                   void* stream) {
  if (!good_scale(k_scale) || !good_scale(v_scale))
    return fail(PKV_EINVAL, "k_scale %g / v_scale %g must be positive and finite", k_scale, v_scale);
  return decode_impl(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, num_blocks, block_size, max_seq_len, scale,
                     PKV_FP8_E4M3, KvFormat{pkv::KvKind::FP8, k_scale, v_scale}, workspace, workspace_bytes,
                     stream);
}

int pkv_decode_step(float* out, const void* query, const void* key, const void* value, void* key_cache,
                    void* value_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                    const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                    int32_t head_dim, int64_t num_blocks, int32_t block_size, int32_t max_seq_len, float scale,
                    pkv_dtype dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype == PKV_FP8_E4M3) return fail(PKV_EINVAL, "E4M3 pools need their scales: use pkv_decode_step_fp8");
  if (num_seqs > 0 && (!key || !value)) return fail(PKV_EINVAL, "null pointer");
  if (!aligned16(key) || !aligned16(value)) return fail(PKV_EINVAL, "key/value must be 16-byte aligned");
  return decode_impl(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, num_blocks, block_size, max_seq_len, scale, dtype,
                     plain_format(dtype), workspace, workspace_bytes, stream, key, value);
}

int pkv_decode_step_fp8(float* out, const void* query, const void* key, const void* value, void* key_cache,
                        void* value_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                        const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int64_t num_blocks, int32_t block_size, int32_t max_seq_len, float scale,
                        float k_scale, float v_scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (!good_scale(k_scale) || !good_scale(v_scale))
    return fail(PKV_EINVAL, "k_scale %g / v_scale %g must be positive and finite", k_scale, v_scale);
  if (num_seqs > 0 && (!key || !value)) return fail(PKV_EINVAL, "null pointer");
  if (!aligned16(key) || !aligned16(value)) return fail(PKV_EINVAL, "key/value must be 16-byte aligned");
  return decode_impl(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, num_blocks, block_size, max_seq_len, scale,
                     PKV_FP8_E4M3, KvFormat{pkv::KvKind::FP8, k_scale, v_scale}, workspace, workspace_bytes,
                     stream, key, value);
}

// ---------------------------------------------------------------- allocation-free decode
// Device scratch of pkv_paged_attention_decode_noalloc: the split-K workspace
// (chunk prefix sums, part maxima and sums, partial outputs) of one call.
// Each device that runs the entry point holds its own copy until the process
// ends.  In host code `scratch` names a host-side stand-in, not device memory:
// only the per-device address from hipGetSymbolAddress is ever passed on.
constexpr size_t kScratchBytes = size_t(16) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's address of `scratch`, looked up once per device with
// that device current.  Returns nullptr (and sets the error) on failure.
void* device_scratch() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    hip_fail(e, "hipGetDevice");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    fail(PKV_EUNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

size_t pkv_noalloc_scratch_bytes(void) { return kScratchBytes; }

int pkv_paged_attention_decode_noalloc(float* out, const void* query, const void* key_cache,
                                       const void* value_cache, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int64_t num_blocks, int32_t block_size, int32_t max_seq_len, float scale,
                                       pkv_dtype dtype, void* stream) {
  if (dtype == PKV_FP8_E4M3)
    return fail(PKV_EINVAL, "E4M3 pools need their scales: pkv_paged_attention_decode_noalloc takes F32 or BF16");
  int st = check_shape(num_q_heads, num_kv_heads, head_dim, block_size, dtype);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || num_seqs > kMaxSeqs) return fail(PKV_EUNSUPPORTED, "num_seqs %d (max %d)", num_seqs, kMaxSeqs);
  const size_t need = pkv_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, dtype);
  if (need > kScratchBytes)
    return fail(PKV_EUNSUPPORTED,
                "pkv_paged_attention_decode_noalloc: this shape needs up to %zu bytes of scratch, the library's static "
                "scratch holds %zu; use pkv_paged_attention_decode with a workspace",
                need, kScratchBytes);
  void* ws = device_scratch();
  if (ws == nullptr) return PKV_EHIP;
  return decode_impl(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, num_blocks, block_size, max_seq_len, scale, dtype,
                     plain_format(dtype), ws, kScratchBytes, stream);
}

size_t pkv_decode_shared_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size, pkv_dtype dtype, int32_t num_groups) {
  if (num_seqs < 0 || num_seqs > pkv::kMaxPrefixSeqs || num_groups < 0 || num_groups > pkv::kMaxPrefixGroups)
    return 0;
  if (dtype == PKV_F32 || check_shape(num_q_heads, num_kv_heads, head_dim, block_size, dtype) != PKV_OK) return 0;
  return pkv::decode_prefix_workspace_bytes(num_seqs, num_kv_heads, num_q_heads / num_kv_heads, head_dim,
                                            decode_workers(), num_groups);
}

int pkv_paged_attention_decode_shared(float* out, const void* query, const void* key_cache,
                                      const void* value_cache, const int32_t* block_tables,
                                      int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int64_t num_blocks, int32_t block_size, int32_t max_seq_len, float scale,
                                      pkv_dtype dtype, const int32_t* prefix_groups, int32_t num_groups,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype == PKV_FP8_E4M3)
    return fail(PKV_EINVAL, "E4M3 pools need their scales: use pkv_paged_attention_decode_shared_fp8");
  return decode_impl(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, num_blocks, block_size, max_seq_len, scale, dtype,
                     plain_format(dtype), workspace, workspace_bytes, stream, nullptr, nullptr, prefix_groups,
                     num_groups);
}

int pkv_paged_attention_decode_shared_fp8(float* out, const void* query, const void* key_cache,
                                          const void* value_cache, const int32_t* block_tables,
                                          int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t num_seqs,
                                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                          int64_t num_blocks, int32_t block_size, int32_t max_seq_len, float scale,
                                          float k_scale, float v_scale, const int32_t* prefix_groups,
                                          int32_t num_groups, void* workspace, size_t workspace_bytes,
                                          void* stream) {
  if (!good_scale(k_scale) || !good_scale(v_scale))
    return fail(PKV_EINVAL, "k_scale %g / v_scale %g must be positive and finite", k_scale, v_scale);
  return decode_impl(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, num_blocks, block_size, max_seq_len, scale,
                     PKV_FP8_E4M3, KvFormat{pkv::KvKind::FP8, k_scale, v_scale}, workspace, workspace_bytes,
                     stream, nullptr, nullptr, prefix_groups, num_groups);
}

int pkv_decode_step_shared(float* out, const void* query, const void* key, const void* value, void* key_cache,
                           void* value_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                           int32_t head_dim, int64_t num_blocks, int32_t block_size, int32_t max_seq_len,
                           float scale, pkv_dtype dtype, const int32_t* prefix_groups, int32_t num_groups,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (dtype == PKV_FP8_E4M3) return fail(PKV_EINVAL, "E4M3 pools need their scales");
  if (num_seqs > 0 && (!key || !value)) return fail(PKV_EINVAL, "null pointer");
  if (!aligned16(key) || !aligned16(value)) return fail(PKV_EINVAL, "key/value must be 16-byte aligned");
  return decode_impl(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, seq_lens, num_seqs,
                     num_q_heads, num_kv_heads, head_dim, num_blocks, block_size, max_seq_len, scale, dtype,
                     plain_format(dtype), workspace, workspace_bytes, stream, key, value, prefix_groups,
                     num_groups);
}

static size_t varlen_decode_part(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim) {
  const size_t d = pkv::decode_workspace_bytes(num_seqs, num_kv_heads, num_q_heads / num_kv_heads, head_dim,
                                               decode_workers());
  return (d + 255) / 256 * 256;
}

static int mixed_grid() {
  const int cus = current_cus();
  return cus > 0 ? cus : 256;
}

static size_t mixed_part(int group, int head_dim) {
  return pkv::mixed_workspace_bytes(mixed_grid(), group < 16 ? group : 16, head_dim);
}

size_t pkv_varlen_workspace_size(int32_t num_seqs, int32_t num_tokens, int32_t num_q_heads,
                                 int32_t num_kv_heads, int32_t head_dim, int32_t max_query_len,
                                 int32_t block_size, pkv_dtype dtype) {
  (void)num_tokens;
  (void)max_query_len;
  if (num_seqs < 0 || num_seqs > kMaxSeqs) return 0;
  if (check_shape(num_q_heads, num_kv_heads, head_dim, block_size, dtype) != PKV_OK) return 0;
  // either layout: the split + merge + prefill launches, or the one mixed launch
  const size_t three = varlen_decode_part(num_seqs, num_q_heads, num_kv_heads, head_dim) +
                       pkv::prefill_plan_bytes(num_seqs);
  return std::max(three, mixed_part(num_q_heads / num_kv_heads, head_dim));
}

static int varlen_impl(float* out, const void* query, const void* key_cache, const void* value_cache,
                       const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                       const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens, int32_t max_query_len,
                       int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                       int64_t num_blocks, int32_t block_size, float scale, pkv_dtype dtype, KvFormat fmt,
                       void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(num_q_heads, num_kv_heads, head_dim, block_size, dtype);
  if (st != PKV_OK) return st;
  if (num_seqs < 0 || num_seqs > kMaxSeqs) return fail(PKV_EUNSUPPORTED, "num_seqs %d (max %d)", num_seqs, kMaxSeqs);
  if (num_tokens < 0 || max_query_len < 0 || max_blocks_per_seq < 0 || num_blocks < 0 || max_seq_len < 0)
    return fail(PKV_EINVAL, "negative size");
  if (num_tokens > 0 && max_query_len == 0) return fail(PKV_EINVAL, "max_query_len is 0 with %d tokens", num_tokens);
  st = check_attention_bounds(max_blocks_per_seq, block_size, num_blocks, num_kv_heads, head_dim, dtype);
  if (st != PKV_OK) return st;
  if (num_seqs == 0 || num_tokens == 0) return ok();
  if (!out || !query || !seq_lens || !query_start_loc ||
      (max_blocks_per_seq > 0 && (!block_tables || !key_cache || !value_cache)))
    return fail(PKV_EINVAL, "null pointer");
  if (!aligned16(out) || !aligned16(query) || !aligned16(key_cache) || !aligned16(value_cache))
    return fail(PKV_EINVAL, "out/query/cache pointers must be 16-byte aligned");
  if (!std::isfinite(scale)) return fail(PKV_EINVAL, "scale is not finite");
  if (max_blocks_per_seq > 0 && num_blocks == 0) return fail(PKV_EINVAL, "empty pool with a non-empty block table");
  const int group = num_q_heads / num_kv_heads;
  if ((int64_t)max_query_len * group > (int64_t)1 << 30) return fail(PKV_EUNSUPPORTED, "max_query_len too large");
  // prefill items per sequence: KV heads x column blocks of 256 (row, head) columns; the item counters are int
  const int64_t head_tiles = (group + 15) / 16;
  if (((int64_t)num_tokens * group / 256 + num_seqs) * num_kv_heads * head_tiles > ((int64_t)1 << 30))
    return fail(PKV_EUNSUPPORTED, "too many (row, head) columns for one call");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool lds_prefill = max_query_len > 1 && pkv::prefill_uses_plan(head_dim, fmt.kind);
  const bool mixed = lds_prefill && g_varlen_single.load() != 0 && num_seqs <= pkv::kMixedMaxSeqs;
  const size_t dec_bytes = varlen_decode_part(num_seqs, num_q_heads, num_kv_heads, head_dim);
  {
    // check the workspace before enqueueing anything
    const size_t need = mixed ? mixed_part(group, head_dim) : dec_bytes + pkv::prefill_plan_bytes(num_seqs);
    if (!workspace || workspace_bytes < need)
      return fail(PKV_EWORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return fail(PKV_EINVAL, "workspace must be 256-byte aligned");
  }
  pkv::PrefillArgs p{};
  p.out = out;
  p.query = query;
  p.key_cache = key_cache;
  p.value_cache = value_cache;
  p.block_tables = block_tables;
  p.seq_lens = seq_lens;
  p.qsl = query_start_loc;
  p.max_blocks = max_blocks_per_seq;
  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = group;
  p.num_blocks = num_blocks;
  p.scale_log2 = scale * fmt.k_scale * 1.4426950408889634f;
  p.v_scale = fmt.v_scale;
  if (mixed) {
    // Prefill chunks and decode rows in one launch (the decode rows' pairs
    // queued after the prefill items); profile events bracket it.  Opt-in:
    // on the 8 x 512-row + 120-row step it measured 0.725 against 0.681 ms
    // for the three launches (the decode code in the same kernel moves the
    // prefill's LDS reads later, 5 %; a decode item pays its own claim,
    // start-up and merge, 30 %; the prefill leaves little tail to fill).
    pkv::DecodeArgs d{};
    d.out = out;
    d.query = query;
    d.key_cache = key_cache;
    d.value_cache = value_cache;
    d.block_tables = block_tables;
    d.seq_lens = seq_lens;
    d.qsl = query_start_loc;
    d.max_blocks = max_blocks_per_seq;
    d.num_seqs = num_seqs;
    d.num_q_heads = num_q_heads;
    d.num_kv_heads = num_kv_heads;
    d.group = group;
    d.head_dim = head_dim;
    d.head_tiles = (int)head_tiles;
    d.tile_cols = group < 16 ? group : 16;
    d.num_blocks = num_blocks;
    d.scale_log2 = p.scale_log2;
    d.v_scale = fmt.v_scale;
    const int grid = mixed_grid();
    if (g_ev_start) (void)hipEventRecord(g_ev_start, s);
    hipError_t e = pkv::launch_mixed_varlen(p, d, workspace, block_size, fmt.kind == pkv::KvKind::FP8, grid, s);
    if (e != hipSuccess) return hip_fail(e, "mixed varlen launch");
    if (g_ev_stop) (void)hipEventRecord(g_ev_stop, s);
    return ok();
  }
  int* plan = reinterpret_cast<int*>(static_cast<char*>(workspace) + dec_bytes);
  // Decode rows (sequences with exactly one query row) first, through the
  // split and merge kernels; the merge launch also builds the prefill
  // kernel's item plan (one extra workgroup), so no launch of its own.
  hipEvent_t e0 = g_ev_start, e1 = g_ev_stop;
  g_ev_start = nullptr;
  g_ev_stop = nullptr;
  int rc = run_decode(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, seq_lens,
                      query_start_loc, num_seqs, num_q_heads, num_kv_heads, head_dim, num_blocks, block_size,
                      max_seq_len, scale, fmt, workspace, workspace_bytes, s, nullptr, nullptr,
                      lds_prefill ? plan : nullptr);
  g_ev_start = e0;
  g_ev_stop = e1;
  if (rc != PKV_OK) return rc;
  // profile events (if set) bracket the prefill kernel, the step's dominant one
  if (g_ev_start) (void)hipEventRecord(g_ev_start, s);
  if (max_query_len > 1) {
    const int cus = current_cus();
    p.waves = (cus > 0 ? cus : 256) * 4;
    p.plan = plan;
    hipError_t e = pkv::launch_prefill(p, head_dim, block_size, fmt.kind, cus, s);
    if (e != hipSuccess) return hip_fail(e, "prefill launch");
  }
  if (g_ev_stop) (void)hipEventRecord(g_ev_stop, s);
  return ok();
}

int pkv_paged_attention_varlen(float* out, const void* query, const void* key_cache,
                               const void* value_cache, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, const int32_t* seq_lens,
                               const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens,
                               int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks,
                               int32_t block_size, float scale, pkv_dtype dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (dtype == PKV_FP8_E4M3)
    return fail(PKV_EINVAL, "E4M3 pools need their scales: use pkv_paged_attention_varlen_fp8");
  return varlen_impl(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, seq_lens,
                     query_start_loc, num_seqs, num_tokens, max_query_len, max_seq_len, num_q_heads, num_kv_heads,
                     head_dim, num_blocks, block_size, scale, dtype, plain_format(dtype), workspace,
                     workspace_bytes, stream);
}

int pkv_paged_attention_varlen_fp8(float* out, const void* query, const void* key_cache, const void* value_cache,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                   const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens,
                                   int32_t max_query_len, int32_t max_seq_len, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int64_t num_blocks, int32_t block_size,
                                   float scale, float k_scale, float v_scale, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (!good_scale(k_scale) || !good_scale(v_scale))
    return fail(PKV_EINVAL, "k_scale %g / v_scale %g must be positive and finite", k_scale, v_scale);
  return varlen_impl(out, query, key_cache, value_cache, block_tables, max_blocks_per_seq, seq_lens,
                     query_start_loc, num_seqs, num_tokens, max_query_len, max_seq_len, num_q_heads, num_kv_heads,
                     head_dim, num_blocks, block_size, scale, PKV_FP8_E4M3,
                     KvFormat{pkv::KvKind::FP8, k_scale, v_scale}, workspace, workspace_bytes, stream);
}

}  // extern "C"

// Status reporting for the library's host-only parts (the native scheduler).
namespace pkv {
int report(int status, const char* msg) {
  if (status == PKV_OK) return ok();
  return fail(status, "%s", msg);
}
}  // namespace pkv

