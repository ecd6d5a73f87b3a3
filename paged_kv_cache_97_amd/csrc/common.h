// Device-side building blocks shared by the pagedkv kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Wave-uniform value into a scalar register.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// Vector load; STREAM = non-temporal (data read once per kernel).
template <typename V, bool STREAM>
__device__ __forceinline__ V ld_v(const void* p) {
  if constexpr (STREAM) return __builtin_nontemporal_load(reinterpret_cast<const V*>(p));
  else return *reinterpret_cast<const V*>(p);
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st16f(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

// Pack the 16-bit element `t` of a and of b (a in the low half).  Each u32x4
// holds 8 consecutive 16-bit values, element 2w in the low half of dword w.
template <int T>
__device__ __forceinline__ uint32_t pick16_pair(const u32x4& a, const u32x4& b) {
  constexpr uint32_t sel = (T & 1) ? 0x07060302u : 0x05040100u;
  return __builtin_amdgcn_perm(b[T >> 1], a[T >> 1], sel);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float wave_max_across_rows(float v) {
  // reduce over the 4 rows of 16 lanes (lanes l, l^16, l^32, l^48)
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ float wave_sum_across_rows(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Inclusive prefix sum over one wavefront.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int l = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int u = __shfl_up(v, d);
    if (l >= d) v += u;
  }
  return v;
}

// Block-wide exclusive scan of f(i) for i in [0, n) into lds[0..n] (lds[0] = 0,
// lds[i+1] = f(0)+...+f(i)), for a block of kThreads threads.  Ends with a
// barrier, so every thread may read lds afterwards.
template <int kThreads, typename F>
__device__ void block_prefix_sum(int n, int* lds, F f) {
  __shared__ int wave_tot[kThreads / kWave];
  const int tid = threadIdx.x;
  const int wid = tid / kWave;
  int carry = 0;
  if (tid == 0) lds[0] = 0;
  for (int base = 0; base < n; base += kThreads) {
    const int i = base + tid;
    int x = wave_inclusive_scan(i < n ? f(i) : 0);
    if (lane_id() == kWave - 1) wave_tot[wid] = x;
    __syncthreads();
    int off = carry;
    for (int w = 0; w < wid; ++w) off += wave_tot[w];
    if (i < n) lds[i + 1] = x + off;
    int tot = 0;
    for (int w = 0; w < kThreads / kWave; ++w) tot += wave_tot[w];
    carry += tot;
    __syncthreads();
  }
}

}  // namespace pkv
