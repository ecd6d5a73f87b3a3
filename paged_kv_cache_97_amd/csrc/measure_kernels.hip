// A plain streaming read of a device buffer, kept beside the hot-path kernels
// as a measuring stick: the HBM read rate this part reaches in practice, to
// set next to the 8 TB/s peak the attention kernels are judged against, and
// a read-only way to push other data out of the L2s and the last-level cache
// before a cold timing.  It computes nothing of the method.
//
// Each lane keeps kReadUnroll non-temporal 16-byte loads in flight per
// iteration of a grid-stride loop; the XOR of everything read is reduced per
// wavefront and stored to sink so the loads cannot be dropped.
#include "common.h"
#include "launch.h"

namespace pkv {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;

__global__ void __launch_bounds__(kReadThreads)
stream_read_kernel(const u32x4* __restrict__ buf, int64_t nvec, uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t step = (int64_t)gridDim.x * kReadThreads * kReadUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kReadThreads * kReadUnroll + threadIdx.x; base < nvec; base += step) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const int64_t i = base + (int64_t)u * kReadThreads;
      v[u] = i < nvec ? __builtin_nontemporal_load(buf + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, d);
  if (lane_id() == 0) sink[blockIdx.x * (kReadThreads / kWave) + (threadIdx.x >> 6)] = acc;
}

hipError_t launch_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int blocks, hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kReadThreads), 0, stream,
                     static_cast<const u32x4*>(buf), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace pkv
