// Device-side building blocks shared by the pagedkv kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// The lane index, recomputed where it is used.  A volatile asm is never
// hoisted, so per-lane addresses built from it in rarely run code stay there
// instead of becoming loop-invariant values that hold registers (or spill)
// through a hot loop.
__device__ __forceinline__ int lane_id_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

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

// The same maximum with the gfx950 row-swap permutes: permlane16_swap pairs
// row r with row r ^ 1 and permlane32_swap the two 32-lane halves.  Each
// returns both swapped registers; whichever holds which, every lane finds its
// own value and its partner's among the two, so a max over both is the
// pairwise max.  VALU only: no LDS round trip on the softmax critical path.
__device__ __forceinline__ float wave_max_across_rows_swap(float v) {
  const uint32_t x = __float_as_uint(v);
  const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t y = __float_as_uint(m);
  const auto b = __builtin_amdgcn_permlane32_swap(y, y, false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float wave_sum_across_rows(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Four floats -> four OCP E4M3 bytes of x * inv (inv: the float32 reciprocal
// of the pool scale), saturated to +-448, the largest finite E4M3 value, and
// rounded to nearest even by v_cvt_pk_fp8_f32.  Byte k holds the k-th value.
__device__ __forceinline__ uint32_t quant4(float a, float b, float c, float d, float inv) {
  auto q = [inv](float x) { return fminf(fmaxf(x * inv, -448.f), 448.f); };
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(q(a), q(b), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(q(c), q(d), w, true);
  return (uint32_t)w;
}

// bf16 element 0 / 1 of a dword as a float (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Eight bf16 values (element 2w in the low half of dword w) -> eight E4M3 bytes.
__device__ __forceinline__ u32x2 quant8_bf16(const u32x4& x, float inv) {
  return u32x2{quant4(bf16_lo(x[0]), bf16_hi(x[0]), bf16_lo(x[1]), bf16_hi(x[1]), inv),
               quant4(bf16_lo(x[2]), bf16_hi(x[2]), bf16_lo(x[3]), bf16_hi(x[3]), inv)};
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
