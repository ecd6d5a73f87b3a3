// Whole-block copies: copy-on-write inside the KV pools and swap between a
// GPU pool and a pinned host pool.
//
// Copy-on-write: lakecityint.com/news/209622 §3.2 (a sharer about to write
// gets a fresh block holding a copy of the shared one).  Swap: 5688vip.com
// "vLLM核心机制" §3.3 and lakecityint §2.1 (a preempted sequence's blocks move
// to CPU memory and come back later, possibly into other physical blocks).
//
// One launch serves every (src, dst) pair of the call: workgroup x takes pair
// x, workgroup y a slice of the block, and each lane keeps kUnroll 16-byte
// loads of each pool in flight before its stores.  A block is one contiguous
// run of block_size*num_kv_heads*head_dim elements in the [blocks, block_size,
// heads, head_dim] layout, so both sides are fully coalesced.  Pinned host
// memory is read or written through the device's mapping of it, over PCIe.
#include "common.h"
#include "launch.h"

namespace pkv {

constexpr int kCopyThreads = 256;
constexpr int kCopyUnroll = 4;

// NT: non-temporal loads and stores.  Device-to-device copies touch every
// byte once, and keeping them out of the caches lets the writes stream
// (+7 % on 4096 pairs of 32 KiB blocks); across PCIe to pinned host memory
// the plain form is as fast or faster.
template <bool NT>
__global__ void __launch_bounds__(kCopyThreads)
block_copy_kernel(const u32x4* __restrict__ src0, u32x4* __restrict__ dst0, const u32x4* __restrict__ src1,
                  u32x4* __restrict__ dst1, const int64_t* __restrict__ mapping, int64_t src_blocks,
                  int64_t dst_blocks, int64_t block_vecs) {
  const int64_t pair = blockIdx.x;
  const int64_t s = mapping[2 * pair];
  const int64_t d = mapping[2 * pair + 1];
  if (s < 0 || s >= src_blocks || d < 0 || d >= dst_blocks) return;   // uniform per workgroup
  const int64_t so = s * block_vecs, dof = d * block_vecs;
  const int64_t step = (int64_t)gridDim.y * kCopyThreads * kCopyUnroll;
  for (int64_t base = (int64_t)blockIdx.y * kCopyThreads * kCopyUnroll + threadIdx.x; base < block_vecs;
       base += step) {
    u32x4 a[kCopyUnroll], b[kCopyUnroll];
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = base + u * kCopyThreads;
      if (i < block_vecs) {
        a[u] = NT ? __builtin_nontemporal_load(src0 + so + i) : src0[so + i];
        if (src1) b[u] = NT ? __builtin_nontemporal_load(src1 + so + i) : src1[so + i];
      }
    }
#pragma unroll
    for (int u = 0; u < kCopyUnroll; ++u) {
      const int64_t i = base + u * kCopyThreads;
      if (i < block_vecs) {
        if (NT) {
          __builtin_nontemporal_store(a[u], dst0 + dof + i);
          if (src1) __builtin_nontemporal_store(b[u], dst1 + dof + i);
        } else {
          dst0[dof + i] = a[u];
          if (src1) dst1[dof + i] = b[u];
        }
      }
    }
  }
}

hipError_t launch_block_copy(const void* src0, void* dst0, const void* src1, void* dst1, const int64_t* mapping,
                             int num_pairs, int64_t src_blocks, int64_t dst_blocks, int64_t block_bytes,
                             bool streaming, hipStream_t stream) {
  const int64_t vecs = block_bytes / 16;
  const int64_t per_wg = (int64_t)kCopyThreads * kCopyUnroll;
  int64_t slices = (vecs + per_wg - 1) / per_wg;
  if (slices > 65535) slices = 65535;
  const dim3 grid((unsigned)num_pairs, (unsigned)slices);
  if (streaming)
    hipLaunchKernelGGL(block_copy_kernel<true>, grid, dim3(kCopyThreads), 0, stream, (const u32x4*)src0,
                       (u32x4*)dst0, (const u32x4*)src1, (u32x4*)dst1, mapping, src_blocks, dst_blocks, vecs);
  else
    hipLaunchKernelGGL(block_copy_kernel<false>, grid, dim3(kCopyThreads), 0, stream, (const u32x4*)src0,
                       (u32x4*)dst0, (const u32x4*)src1, (u32x4*)dst1, mapping, src_blocks, dst_blocks, vecs);
  return hipGetLastError();
}

}  // namespace pkv
