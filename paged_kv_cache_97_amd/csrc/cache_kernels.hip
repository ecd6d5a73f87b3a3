// Slot mapping and the cache write (reshape_and_cache).
//
// Slot arithmetic: gaoleia.github.io "PagedAttention 和 Continuous Batching"
// §1.5 (logical block = pos / block_size, offset = pos % block_size,
// slot = table[logical block] * block_size + offset).  Cache write: feifeigd
// "vLLM 架构详解" 一 PagedAttention (a new token's K/V goes to its in-block
// position of its block) and gaoleia §1.3 (block layout [block_size, heads,
// head_dim]), so a slot's K row for all KV heads is one contiguous
// num_kv_heads*head_dim run of the pool.
//
// Both kernels are pure data movement bounded by launch latency at serving
// sizes; the write moves 16 bytes per lane with fully coalesced rows.
//
// FP8 pools (feifeigd "vLLM 架构详解" 三 生产级部署配置: kv-cache-dtype fp8
// halves KV memory): the write stores OCP E4M3 bytes.  Each element is
// multiplied by the host-computed float32 reciprocal of the pool's scale,
// clamped to +-448 (the largest finite E4M3 value, so large inputs saturate),
// and rounded to nearest-even by v_cvt_pk_fp8_f32.  Inputs must be finite.
#include "common.h"
#include "launch.h"

namespace pkv {

// query_start_loc is staged in LDS when it fits (lds_n > 0), so the owner
// search costs one global round trip instead of log2(num_seqs).
__global__ void __launch_bounds__(256)
slot_mapping_kernel(const int32_t* __restrict__ block_tables, int num_seqs, int max_blocks,
                    const int32_t* __restrict__ positions, const int32_t* __restrict__ qsl,
                    int num_tokens, int block_size, int64_t* __restrict__ slots, int lds_n) {
  extern __shared__ int qs[];
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  for (int i = threadIdx.x; i < lds_n; i += blockDim.x) qs[i] = qsl[i];
  if (lds_n > 0) __syncthreads();
  if (t >= num_tokens) return;
  const int p = positions[t];
  const int32_t* q = lds_n > 0 ? qs : qsl;
  // sequence owning row t: the last s with qsl[s] <= t
  int lo = 0, hi = num_seqs;  // invariant: qsl[lo] <= t (qsl[0] == 0), answer in [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (q[mid] <= t) lo = mid; else hi = mid;
  }
  int64_t slot = -1;
  if (num_seqs > 0 && t < q[lo + 1] && p >= 0) {
    const int lb = p / block_size;
    if (lb < max_blocks) {
      const int phys = block_tables[(int64_t)lo * max_blocks + lb];
      if (phys >= 0) slot = (int64_t)phys * block_size + (p - lb * block_size);
    }
  }
  slots[t] = slot;
}

// One lane moves 16 bytes of K and 16 bytes of V; a token row is
// row_vecs*16 bytes (num_kv_heads*head_dim*elem).
__global__ void __launch_bounds__(256)
reshape_and_cache_kernel(const u32x4* __restrict__ key, const u32x4* __restrict__ value,
                         u32x4* __restrict__ key_cache, u32x4* __restrict__ value_cache,
                         const int64_t* __restrict__ slots, int64_t total, int row_vecs,
                         int64_t num_slots) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / row_vecs;
    const int64_t c = i - t * row_vecs;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) continue;
    const u32x4 k = key[i];
    const u32x4 v = value[i];
    key_cache[slot * row_vecs + c] = k;
    value_cache[slot * row_vecs + c] = v;
  }
}

// Slot mapping and cache write of a step's new tokens in one launch: each
// workgroup takes kTokensPerWg tokens, a few lanes compute their slots (owner
// search over query_start_loc staged in LDS), then all lanes copy the rows.
constexpr int kTokensPerWg = 8;
constexpr int kQslLds = 1024;

// The slots of tokens t0 .. t0 + kTokensPerWg - 1 into s_slot (and
// slots_out).  The loads that need no slot -- the owner lanes' positions,
// query_start_loc for the LDS copy and whatever `prefetch` issues (the first
// rows of the copy) -- all go out before the first wait, so the chain is two
// memory round trips: those loads, then the block-table entry.  Ends with a
// barrier after which s_slot is valid.
template <typename Prefetch>
__device__ __forceinline__ void workgroup_slots(const int32_t* __restrict__ block_tables, int num_seqs,
                                                int max_blocks, const int32_t* __restrict__ positions,
                                                const int32_t* __restrict__ qsl, int num_tokens, int block_size,
                                                int64_t* __restrict__ slots_out, int t0, int* qs, int64_t* s_slot,
                                                Prefetch prefetch) {
  const int tid = threadIdx.x;
  const int t = t0 + tid;
  const bool owner = tid < kTokensPerWg && t < num_tokens;
  const int p = owner ? positions[t] : -1;
  const bool staged = num_seqs + 1 <= kQslLds;
  prefetch();
  if (staged)
    for (int i = tid; i <= num_seqs; i += 256) qs[i] = qsl[i];
  __syncthreads();
  if (tid < kTokensPerWg) {
    int64_t slot = -1;
    if (owner) {
      const int32_t* q = staged ? qs : qsl;
      int lo = 0, hi = num_seqs;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (q[mid] <= t) lo = mid; else hi = mid;
      }
      if (num_seqs > 0 && t < q[lo + 1] && p >= 0) {
        const int lb = p / block_size;
        if (lb < max_blocks) {
          const int phys = block_tables[(int64_t)lo * max_blocks + lb];
          if (phys >= 0) slot = (int64_t)phys * block_size + (p - lb * block_size);
        }
      }
      if (slots_out) slots_out[t] = slot;
    }
    s_slot[tid] = slot;
  }
  __syncthreads();
}

// Row vectors each lane loads before the slots are known (the rest of the
// workgroup's rows follow in a plain loop).
constexpr int kCopyAhead = 4;

__global__ void __launch_bounds__(256)
write_tokens_kernel(const int32_t* __restrict__ block_tables, int num_seqs, int max_blocks,
                    const int32_t* __restrict__ positions, const int32_t* __restrict__ qsl, int num_tokens,
                    int block_size, const u32x4* __restrict__ key, const u32x4* __restrict__ value,
                    u32x4* __restrict__ key_cache, u32x4* __restrict__ value_cache, int row_vecs,
                    int64_t num_slots, int64_t* __restrict__ slots_out) {
  __shared__ int qs[kQslLds];
  __shared__ int64_t s_slot[kTokensPerWg];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kTokensPerWg;
  const int n = min(kTokensPerWg, num_tokens - t0) * row_vecs;   // row vectors of this workgroup
  const int64_t base = (int64_t)t0 * row_vecs;
  u32x4 ka[kCopyAhead], va[kCopyAhead];
  workgroup_slots(block_tables, num_seqs, max_blocks, positions, qsl, num_tokens, block_size, slots_out, t0, qs,
                  s_slot, [&] {
#pragma unroll
                    for (int u = 0; u < kCopyAhead; ++u) {
                      const int i = tid + 256 * u;
                      if (i < n) {
                        ka[u] = key[base + i];
                        va[u] = value[base + i];
                      }
                    }
                  });
  auto store = [&](int i, const u32x4& k, const u32x4& v) {
    const int tl = i / row_vecs, cvec = i - tl * row_vecs;
    const int64_t slot = s_slot[tl];
    if (slot < 0 || slot >= num_slots) return;
    key_cache[slot * row_vecs + cvec] = k;
    value_cache[slot * row_vecs + cvec] = v;
  };
#pragma unroll
  for (int u = 0; u < kCopyAhead; ++u) {
    const int i = tid + 256 * u;
    if (i < n) store(i, ka[u], va[u]);
  }
  for (int i = tid + 256 * kCopyAhead; i < n; i += 256) store(i, key[base + i], value[base + i]);
}

// ------------------------------------------------------------------ FP8 stores
// The 16 input elements of output vector `v` of a row (bf16: two 16-byte
// input vectors, fp32: four) and their 16 E4M3 bytes.
template <bool BF16IN>
struct QuantIn {
  static constexpr int kVecs = BF16IN ? 2 : 4;   // 16-byte input vectors per 16 output bytes
  u32x4 x[kVecs];
  __device__ __forceinline__ void load(const void* in, int64_t v) {
    const u32x4* p = reinterpret_cast<const u32x4*>(in) + kVecs * v;
#pragma unroll
    for (int j = 0; j < kVecs; ++j) x[j] = p[j];
  }
  __device__ __forceinline__ u32x4 quant(float inv) const {
    u32x4 out;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if constexpr (BF16IN) {
        const u32x4& y = x[w >> 1];
        const uint32_t lo = y[2 * (w & 1)], hi = y[2 * (w & 1) + 1];
        out[w] = quant4(bf16_lo(lo), bf16_hi(lo), bf16_lo(hi), bf16_hi(hi), inv);
      } else {
        const f32x4 y = __builtin_bit_cast(f32x4, x[w]);
        out[w] = quant4(y[0], y[1], y[2], y[3], inv);
      }
    }
    return out;
  }
};

template <bool BF16IN>
__device__ __forceinline__ u32x4 quant16(const void* in, int64_t v, float inv) {
  QuantIn<BF16IN> x;
  x.load(in, v);
  return x.quant(inv);
}

template <bool BF16IN>
__global__ void __launch_bounds__(256)
reshape_and_cache_fp8_kernel(const void* __restrict__ key, const void* __restrict__ value,
                             u32x4* __restrict__ key_cache, u32x4* __restrict__ value_cache,
                             const int64_t* __restrict__ slots, int64_t total, int row_vecs, int64_t num_slots,
                             float k_inv, float v_inv) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / row_vecs;
    const int64_t c = i - t * row_vecs;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) continue;
    key_cache[slot * row_vecs + c] = quant16<BF16IN>(key, i, k_inv);
    value_cache[slot * row_vecs + c] = quant16<BF16IN>(value, i, v_inv);
  }
}

// write_tokens_kernel with quantising stores (same slot computation).  The
// raw input vectors of each lane's first kQuantAhead output vectors are
// loaded before the slots are known.
constexpr int kQuantAhead = 2;


template <bool BF16IN>
__global__ void __launch_bounds__(256)
write_tokens_fp8_kernel(const int32_t* __restrict__ block_tables, int num_seqs, int max_blocks,
                        const int32_t* __restrict__ positions, const int32_t* __restrict__ qsl, int num_tokens,
                        int block_size, const void* __restrict__ key, const void* __restrict__ value,
                        u32x4* __restrict__ key_cache, u32x4* __restrict__ value_cache, int row_vecs,
                        int64_t num_slots, int64_t* __restrict__ slots_out, float k_inv, float v_inv) {
  __shared__ int qs[kQslLds];
  __shared__ int64_t s_slot[kTokensPerWg];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kTokensPerWg;
  const int n = min(kTokensPerWg, num_tokens - t0) * row_vecs;   // output vectors of this workgroup
  const int64_t base = (int64_t)t0 * row_vecs;
  QuantIn<BF16IN> ka[kQuantAhead], va[kQuantAhead];
  workgroup_slots(block_tables, num_seqs, max_blocks, positions, qsl, num_tokens, block_size, slots_out, t0, qs,
                  s_slot, [&] {
#pragma unroll
                    for (int u = 0; u < kQuantAhead; ++u) {
                      const int i = tid + 256 * u;
                      if (i < n) {
                        ka[u].load(key, base + i);
                        va[u].load(value, base + i);
                      }
                    }
                  });
  auto store = [&](int i, const QuantIn<BF16IN>& k, const QuantIn<BF16IN>& v) {
    const int tl = i / row_vecs, cvec = i - tl * row_vecs;
    const int64_t slot = s_slot[tl];
    if (slot < 0 || slot >= num_slots) return;
    key_cache[slot * row_vecs + cvec] = k.quant(k_inv);
    value_cache[slot * row_vecs + cvec] = v.quant(v_inv);
  };
#pragma unroll
  for (int u = 0; u < kQuantAhead; ++u) {
    const int i = tid + 256 * u;
    if (i < n) store(i, ka[u], va[u]);
  }
  for (int i = tid + 256 * kQuantAhead; i < n; i += 256) {
    QuantIn<BF16IN> k, v;
    k.load(key, base + i);
    v.load(value, base + i);
    store(i, k, v);
  }
}

hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, void* kc, void* vc,
                                        const int64_t* slots, int num_tokens, int row_elems, int64_t num_slots,
                                        KvKind in_kind, float k_inv, float v_inv, hipStream_t stream) {
  const int row_vecs = row_elems / 16;
  const int64_t total = (int64_t)num_tokens * row_vecs;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (in_kind == KvKind::BF16)
    hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream, key, value,
                       (u32x4*)kc, (u32x4*)vc, slots, total, row_vecs, num_slots, k_inv, v_inv);
  else
    hipLaunchKernelGGL(reshape_and_cache_fp8_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream, key,
                       value, (u32x4*)kc, (u32x4*)vc, slots, total, row_vecs, num_slots, k_inv, v_inv);
  return hipGetLastError();
}

hipError_t launch_write_tokens_fp8(const int32_t* bt, int num_seqs, int max_blocks, const int32_t* pos,
                                   const int32_t* qsl, int num_tokens, int block_size, const void* key,
                                   const void* value, void* kc, void* vc, int row_elems, int64_t num_slots,
                                   int64_t* slots, KvKind in_kind, float k_inv, float v_inv, hipStream_t stream) {
  const int blocks = (num_tokens + kTokensPerWg - 1) / kTokensPerWg;
  if (in_kind == KvKind::BF16)
    hipLaunchKernelGGL(write_tokens_fp8_kernel<true>, dim3(blocks), dim3(256), 0, stream, bt, num_seqs, max_blocks,
                       pos, qsl, num_tokens, block_size, key, value, (u32x4*)kc, (u32x4*)vc, row_elems / 16,
                       num_slots, slots, k_inv, v_inv);
  else
    hipLaunchKernelGGL(write_tokens_fp8_kernel<false>, dim3(blocks), dim3(256), 0, stream, bt, num_seqs, max_blocks,
                       pos, qsl, num_tokens, block_size, key, value, (u32x4*)kc, (u32x4*)vc, row_elems / 16,
                       num_slots, slots, k_inv, v_inv);
  return hipGetLastError();
}

hipError_t launch_write_tokens(const int32_t* bt, int num_seqs, int max_blocks, const int32_t* pos,
                               const int32_t* qsl, int num_tokens, int block_size, const void* key,
                               const void* value, void* kc, void* vc, int row_bytes, int64_t num_slots,
                               int64_t* slots, hipStream_t stream) {
  const int blocks = (num_tokens + kTokensPerWg - 1) / kTokensPerWg;
  hipLaunchKernelGGL(write_tokens_kernel, dim3(blocks), dim3(256), 0, stream, bt, num_seqs, max_blocks, pos, qsl,
                     num_tokens, block_size, (const u32x4*)key, (const u32x4*)value, (u32x4*)kc, (u32x4*)vc,
                     row_bytes / 16, num_slots, slots);
  return hipGetLastError();
}

hipError_t launch_slot_mapping(const int32_t* bt, int num_seqs, int max_blocks, const int32_t* pos,
                               const int32_t* qsl, int num_tokens, int block_size, int64_t* slots,
                               hipStream_t stream) {
  const int threads = 256;
  const int blocks = (num_tokens + threads - 1) / threads;
  const int lds_n = num_seqs + 1 <= 8192 ? num_seqs + 1 : 0;
  hipLaunchKernelGGL(slot_mapping_kernel, dim3(blocks), dim3(threads), (size_t)lds_n * sizeof(int), stream,
                     bt, num_seqs, max_blocks, pos, qsl, num_tokens, block_size, slots, lds_n);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* kc, void* vc,
                                    const int64_t* slots, int num_tokens, int row_bytes,
                                    int64_t num_slots, hipStream_t stream) {
  const int row_vecs = row_bytes / 16;
  const int64_t total = (int64_t)num_tokens * row_vecs;
  const int threads = 256;
  int64_t blocks = (total + threads - 1) / threads;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream,
                     (const u32x4*)key, (const u32x4*)value, (u32x4*)kc, (u32x4*)vc, slots, total,
                     row_vecs, num_slots);
  return hipGetLastError();
}

}  // namespace pkv
