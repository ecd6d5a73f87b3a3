// MFMA tile primitives shared by the decode and varlen kernels (gfx950).
//
// A "chunk" is CT consecutive logical tokens of one KV head (32, or 64 for
// the wide E4M3 decode tile), held as CT / 16 sub-tiles of 16 tokens.  With
// tokens on the M side of the MFMA tiles:
//   S^T[token, col] = K[token, :] . Q[col, :]          (A operand = K rows)
//   O^T[dim, col]  += V^T[dim, token] P^T[token, col]   (A operand = V rows)
// so a lane owns column col = lane % 16 of every accumulator, and the S^T
// accumulator's values are already the P^T operand's k-slots.
#pragma once

#include <type_traits>

#include "common.h"

namespace pkv {

template <int N> struct U32Vec;
template <> struct U32Vec<2> { typedef u32x2 type; };
template <> struct U32Vec<4> { typedef u32x4 type; };

// ------------------------------------------------------------------ bf16 tile
template <int D_, int BS_>
struct TileBf16 {
  static constexpr int D = D_;
  static constexpr int BS = BS_;
  static constexpr int CT = 32;      // tokens per chunk
  static constexpr int NSUB = 2;     // 16-token sub-tiles per chunk
  static constexpr bool kStoresInPatch = false;  // the writer calls store_new after patch_new
  static constexpr bool kDoubleBuffer = true;
  static constexpr int kWavesPerEU = 2;
  static constexpr int KK = D / 32;   // K=32 slices of the QK contraction
  static constexpr int VW = D / 16;   // dims per lane of a V row (= O^T dim tiles)
  static constexpr int NDT = D / 16;
  typedef uint16_t Elem;
  typedef uint16_t QElem;
  typedef typename U32Vec<VW / 2>::type VVec;

  struct Q { u32x4 q[KK]; };
  struct Buf { u32x4 k[2][KK]; VVec v[2][4]; };

  // Query head `i` (lane % 16) of the tile, slice kk: dims 32kk + 8c .. +7.
  static __device__ __forceinline__ void load_q(Q& q, const Elem* qb, int cols) {
    const int l = lane_id(), i = l & 15, c = l >> 4;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      q.q[kk] = (i < cols) ? ld16(qb + i * D + 32 * kk + 8 * c) : u32x4{0, 0, 0, 0};
  }

  // Column given by a per-lane pointer to its query row (zeros when !valid).
  static __device__ __forceinline__ void load_q_col(Q& q, const Elem* colp, bool valid) {
    const int c = lane_id() >> 4;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) q.q[kk] = valid ? ld16(colp + 32 * kk + 8 * c) : u32x4{0, 0, 0, 0};
  }

  // Per-lane element offsets inside a sub-tile (row 0 of the tile at the
  // uniform base pointer): K row i, dims 8c..; V rows 4c + r, dims VW*i...
  static __device__ __forceinline__ int k_lane_off(int rs) {
    const int l = lane_id();
    return (l & 15) * rs + 8 * (l >> 4);
  }
  static __device__ __forceinline__ int v_lane_off(int rs) {
    const int l = lane_id();
    return 4 * (l >> 4) * rs + VW * (l & 15);
  }

  // kp[u]/vp[u]: wave-uniform pointers to row 0 of sub-tile u for this KV head.
  // STREAM: non-temporal loads, for tiles read once per kernel (decode);
  // tiles that many wavefronts re-read (prefill) use ordinary cached loads.
  template <bool STREAM = true>
  static __device__ __forceinline__ void load(Buf& b, const Elem* const kp[2], const Elem* const vp[2],
                                              int koff, int voff, int rs) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) b.k[u][kk] = ld_v<u32x4, STREAM>(kp[u] + koff + 32 * kk);
#pragma unroll
      for (int r = 0; r < 4; ++r) b.v[u][r] = ld_v<VVec, STREAM>(vp[u] + voff + r * rs);
    }
  }

  static __device__ __forceinline__ void qk(const Buf& b, const Q& q, f32x4 s[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      s[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        s[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b.k[u][kk]),
                                                       __builtin_bit_cast(bf16x8, q.q[kk]), s[u], 0,
                                                       0, 0);
    }
  }

  static __device__ __forceinline__ void zero_v_rows(Buf& b, int valid) {
    const int c = lane_id() >> 4;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (16 * u + 4 * c + r >= valid) b.v[u][r] = VVec{};
  }

  static __device__ __forceinline__ uint32_t pick(const VVec& a, const VVec& b, int t) {
    const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
    return __builtin_amdgcn_perm(b[t >> 1], a[t >> 1], sel);
  }

  // O^T[dim tile t] += V^T P^T; k-slot 4u + r of every lane is token 16u + 4c + r.
  static __device__ __forceinline__ void pv(const Buf& b, const float p[2][4], f32x4 o[NDT]) {
    bf16x8 pb;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) pb[4 * u + r] = (__bf16)p[u][r];
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
      u32x4 a;
      a[0] = pick(b.v[0][0], b.v[0][1], t);
      a[1] = pick(b.v[0][2], b.v[0][3], t);
      a[2] = pick(b.v[1][0], b.v[1][1], t);
      a[3] = pick(b.v[1][2], b.v[1][3], t);
      o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), pb, o[t], 0, 0, 0);
    }
  }

  // ---- the step's new token (cache write fused into the attention launch)
  // Token tn (0..31) of the loaded chunk is the step's new token, whose slot
  // this launch writes: the lanes that hold its K and V rows replace them
  // with this KV head's input rows nk / nv (pool element type).
  static __device__ __forceinline__ void patch_new(Buf& b, int tn, const void* nkp, const void* nvp, float,
                                                   float) {
    const Elem* nk = static_cast<const Elem*>(nkp);
    const Elem* nv = static_cast<const Elem*>(nvp);
    const int l = lane_id_here(), i = l & 15, c = l >> 4;
    const int t = tn & 15;
    if (i == t)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const u32x4 x = ld16(nk + 8 * c + 32 * kk);
        if (tn >= 16) b.k[1][kk] = x; else b.k[0][kk] = x;
      }
    if (c == (t >> 2)) {
      const VVec x = *reinterpret_cast<const VVec*>(nv + VW * i);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * u + 4 * c + r == tn) b.v[u][r] = x;
    }
  }
  // The lanes holding token tn's rows store them at kd / vd (its slot).
  static __device__ __forceinline__ void store_new(const Buf& b, int tn, Elem* kd, Elem* vd) {
    const int l = lane_id_here(), i = l & 15, c = l >> 4;
    const int t = tn & 15;
    if (i == t)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) st16(kd + 8 * c + 32 * kk, tn >= 16 ? b.k[1][kk] : b.k[0][kk]);
    if (c == (t >> 2)) {
      VVec x = b.v[0][0];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * u + 4 * c + r == tn) x = b.v[u][r];
      *reinterpret_cast<VVec*>(vd + VW * i) = x;
    }
  }

  // Output dim held in o[dt][r] by a lane of row group c.
  static __device__ __forceinline__ int out_dim(int dt, int c, int r) { return VW * (4 * c + r) + dt; }
};

// ------------------------------------------------------------------ fp32 tile
template <int D_, int BS_>
struct TileF32 {
  static constexpr int D = D_;
  static constexpr int BS = BS_;
  static constexpr int CT = 32;      // tokens per chunk
  static constexpr int NSUB = 2;     // 16-token sub-tiles per chunk
  static constexpr bool kStoresInPatch = false;  // the writer calls store_new after patch_new
  static constexpr bool kDoubleBuffer = false;
  static constexpr int kWavesPerEU = D == 128 ? 1 : 2;  // fp32 D=128 needs > 256 VGPRs
  static constexpr int NQ = D / 16;   // float4 pieces of a row per lane
  static constexpr int NH = D / 64;   // 64-dim halves of a V row
  static constexpr int NDT = D / 16;
  typedef float Elem;
  typedef float QElem;

  struct Q { f32x4 q[NQ]; };
  struct Buf { f32x4 k[2][NQ]; f32x4 v[2][4][NH]; };

  static __device__ __forceinline__ void load_q(Q& q, const Elem* qb, int cols) {
    const int l = lane_id(), i = l & 15, c = l >> 4;
#pragma unroll
    for (int j = 0; j < NQ; ++j)
      q.q[j] = (i < cols) ? *reinterpret_cast<const f32x4*>(qb + i * D + 16 * j + 4 * c)
                          : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  static __device__ __forceinline__ void load_q_col(Q& q, const Elem* colp, bool valid) {
    const int c = lane_id() >> 4;
#pragma unroll
    for (int j = 0; j < NQ; ++j)
      q.q[j] = valid ? *reinterpret_cast<const f32x4*>(colp + 16 * j + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  static __device__ __forceinline__ int k_lane_off(int rs) {
    const int l = lane_id();
    return (l & 15) * rs + 4 * (l >> 4);
  }
  static __device__ __forceinline__ int v_lane_off(int rs) {
    const int l = lane_id();
    return 4 * (l >> 4) * rs + 4 * (l & 15);
  }

  template <bool STREAM = true>
  static __device__ __forceinline__ void load(Buf& b, const Elem* const kp[2], const Elem* const vp[2],
                                              int koff, int voff, int rs) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int j = 0; j < NQ; ++j) b.k[u][j] = ld_v<f32x4, STREAM>(kp[u] + koff + 16 * j);
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int hf = 0; hf < NH; ++hf) b.v[u][r][hf] = ld_v<f32x4, STREAM>(vp[u] + voff + r * rs + 64 * hf);
    }
  }

  // k-slot c of MFMA (j, e) is dim 16j + 4c + e.
  static __device__ __forceinline__ void qk(const Buf& b, const Q& q, f32x4 s[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      s[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NQ; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(b.k[u][j][e], q.q[j][e], s[u], 0, 0, 0);
    }
  }

  static __device__ __forceinline__ void zero_v_rows(Buf& b, int valid) {
    const int c = lane_id() >> 4;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (16 * u + 4 * c + r >= valid)
#pragma unroll
          for (int hf = 0; hf < NH; ++hf) b.v[u][r][hf] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // For token slot (u, r) the k-slot c of every lane is token 16u + 4c + r.
  static __device__ __forceinline__ void pv(const Buf& b, const float p[2][4], f32x4 o[NDT]) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int hf = 0; hf < NH; ++hf)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            o[4 * hf + e] = __builtin_amdgcn_mfma_f32_16x16x4f32(b.v[u][r][hf][e], p[u][r], o[4 * hf + e], 0, 0, 0);
  }

  // ---- the step's new token: as TileBf16 (rows of float32).
  static __device__ __forceinline__ void patch_new(Buf& b, int tn, const void* nkp, const void* nvp, float,
                                                   float) {
    const Elem* nk = static_cast<const Elem*>(nkp);
    const Elem* nv = static_cast<const Elem*>(nvp);
    const int l = lane_id_here(), i = l & 15, c = l >> 4;
    const int t = tn & 15;
    if (i == t)
#pragma unroll
      for (int j = 0; j < NQ; ++j) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(nk + 16 * j + 4 * c);
        if (tn >= 16) b.k[1][j] = x; else b.k[0][j] = x;
      }
    if (c == (t >> 2)) {
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(nv + 4 * i + 64 * hf);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * u + 4 * c + r == tn) b.v[u][r][hf] = x;
      }
    }
  }
  static __device__ __forceinline__ void store_new(const Buf& b, int tn, Elem* kd, Elem* vd) {
    const int l = lane_id_here(), i = l & 15, c = l >> 4;
    const int t = tn & 15;
    if (i == t)
#pragma unroll
      for (int j = 0; j < NQ; ++j) st16f(kd + 16 * j + 4 * c, tn >= 16 ? b.k[1][j] : b.k[0][j]);
    if (c == (t >> 2)) {
#pragma unroll
      for (int hf = 0; hf < NH; ++hf) {
        f32x4 x = b.v[0][0][hf];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * u + 4 * c + r == tn) x = b.v[u][r][hf];
        st16f(vd + 4 * i + 64 * hf, x);
      }
    }
  }

  static __device__ __forceinline__ int out_dim(int dt, int c, int r) {
    return 64 * (dt >> 2) + 16 * c + 4 * r + (dt & 3);
  }
};

// ------------------------------------------------------------------ fp8 tile
// KV pools hold OCP E4M3 bytes, the query is bf16.  Every E4M3 value is
// exactly a bf16 value, so tiles are widened in registers
// (v_cvt_scalef32_pk_bf16_fp8, scale 1) and fed to the bf16 MFMA; the pool
// scales are applied outside the tile (k_scale folded into the softmax scale,
// v_scale into the final normalisation).
//
// QK contraction order: the dot product may visit dims in any order as long
// as K and Q agree.  Load j of a K row (16 bytes per lane) gives lane
// row-group c the dims 64j + 16c .. +15, so each load instruction reads one
// contiguous 64-byte run of each of 16 rows (the way the bf16 tile's K loads
// do; a lane-contiguous 32-byte split would make two instructions each touch
// every 128-byte row at alternate 16-byte pieces); k-step kk = 2j + hh uses
// dims 64j + 16c + 8hh .. +7 of both operands.
// V keeps the bf16 tile's layout (rows 4c + r, dims VW*i ..), at one byte per
// element, and is widened before the same in-lane transpose.
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w, bool hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 r = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                      : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  return __builtin_bit_cast(uint32_t, r);
}

template <int D_, int BS_>
struct TileFp8 {
  static constexpr int D = D_;
  static constexpr int BS = BS_;
  static constexpr int CT = 32;      // tokens per chunk
  static constexpr int NSUB = 2;     // 16-token sub-tiles per chunk
  static constexpr bool kStoresInPatch = false;  // the writer calls store_new after patch_new
  static constexpr bool kDoubleBuffer = true;
  static constexpr int kWavesPerEU = 2;
  static constexpr int KK = D / 32;   // bf16 MFMA k-steps of the QK contraction
  static constexpr int KB = D / 4;    // K bytes per lane and row
  static constexpr int KV = KB / 16;  // 16-byte K loads per lane and row (load j: dims 64j + 16c ..)
  static constexpr int VW = D / 16;   // V dims (bytes) per lane and row
  static constexpr int NDT = D / 16;
  typedef uint8_t Elem;
  typedef uint16_t QElem;
  typedef typename U32Vec<VW / 2>::type VVec;                   // widened V piece (bf16)
  typedef typename std::conditional<VW == 8, u32x2, uint32_t>::type VRaw;

  struct Q { u32x4 q[KK]; };
  struct Buf { u32x4 k[2][KV]; VRaw v[2][4]; };

  // dims of k-step kk held by row-group c (see the contraction order above)
  static __device__ __forceinline__ int q_dim(int kk, int c) { return 64 * (kk >> 1) + 16 * c + 8 * (kk & 1); }

  static __device__ __forceinline__ void load_q(Q& q, const QElem* qb, int cols) {
    const int l = lane_id(), i = l & 15, c = l >> 4;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      q.q[kk] = (i < cols) ? ld16(qb + i * D + q_dim(kk, c)) : u32x4{0, 0, 0, 0};
  }

  static __device__ __forceinline__ void load_q_col(Q& q, const QElem* colp, bool valid) {
    const int c = lane_id() >> 4;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) q.q[kk] = valid ? ld16(colp + q_dim(kk, c)) : u32x4{0, 0, 0, 0};
  }

  static __device__ __forceinline__ int k_lane_off(int rs) {
    const int l = lane_id();
    return (l & 15) * rs + 16 * (l >> 4);
  }
  static __device__ __forceinline__ int v_lane_off(int rs) {
    const int l = lane_id();
    return 4 * (l >> 4) * rs + VW * (l & 15);
  }

  template <bool STREAM = true>
  static __device__ __forceinline__ void load(Buf& b, const Elem* const kp[2], const Elem* const vp[2],
                                              int koff, int voff, int rs) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
#pragma unroll
      for (int j = 0; j < KV; ++j) b.k[u][j] = ld_v<u32x4, STREAM>(kp[u] + koff + 64 * j);
#pragma unroll
      for (int r = 0; r < 4; ++r) b.v[u][r] = ld_v<VRaw, STREAM>(vp[u] + voff + r * rs);
    }
  }

  static __device__ __forceinline__ void qk(const Buf& b, const Q& q, f32x4 s[2]) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      s[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        // 8 bytes = dims q_dim(kk, c) .. +7 of this lane's K row
        const uint32_t w0 = b.k[u][kk >> 1][2 * (kk & 1)];
        const uint32_t w1 = b.k[u][kk >> 1][2 * (kk & 1) + 1];
        const u32x4 a = {fp8x2_to_bf16x2(w0, false), fp8x2_to_bf16x2(w0, true), fp8x2_to_bf16x2(w1, false),
                         fp8x2_to_bf16x2(w1, true)};
        s[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, q.q[kk]), s[u], 0, 0, 0);
      }
    }
  }

  static __device__ __forceinline__ void zero_v_rows(Buf& b, int valid) {
    const int c = lane_id() >> 4;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (16 * u + 4 * c + r >= valid) b.v[u][r] = VRaw{};
  }

  static __device__ __forceinline__ VVec widen(const VRaw& x) {
    VVec y;
    if constexpr (VW == 8) {
      y[0] = fp8x2_to_bf16x2(x[0], false);
      y[1] = fp8x2_to_bf16x2(x[0], true);
      y[2] = fp8x2_to_bf16x2(x[1], false);
      y[3] = fp8x2_to_bf16x2(x[1], true);
    } else {
      y[0] = fp8x2_to_bf16x2(x, false);
      y[1] = fp8x2_to_bf16x2(x, true);
    }
    return y;
  }

  static __device__ __forceinline__ uint32_t pick(const VVec& a, const VVec& b, int t) {
    const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
    return __builtin_amdgcn_perm(b[t >> 1], a[t >> 1], sel);
  }

  // Same k-slot order as the bf16 tile: slot 4u + r is token 16u + 4c + r.
  static __device__ __forceinline__ void pv(const Buf& b, const float p[2][4], f32x4 o[NDT]) {
    bf16x8 pb;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) pb[4 * u + r] = (__bf16)p[u][r];
    VVec w[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) w[u][r] = widen(b.v[u][r]);
#pragma unroll
    for (int t = 0; t < NDT; ++t) {
      u32x4 a;
      a[0] = pick(w[0][0], w[0][1], t);
      a[1] = pick(w[0][2], w[0][3], t);
      a[2] = pick(w[1][0], w[1][1], t);
      a[3] = pick(w[1][2], w[1][3], t);
      o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), pb, o[t], 0, 0, 0);
    }
  }

  // ---- the step's new token.  Its input rows nk / nv are bfloat16 and the
  // pool holds E4M3 codes: the lanes that hold token tn encode their pieces
  // of the input rows exactly as the quantising cache write does
  // (x * (1/scale), saturated, nearest even) and replace the loaded codes.
  static __device__ __forceinline__ void patch_new(Buf& b, int tn, const void* nkp, const void* nvp, float k_inv,
                                                   float v_inv) {
    const uint16_t* nk = static_cast<const uint16_t*>(nkp);
    const uint16_t* nv = static_cast<const uint16_t*>(nvp);
    const int l = lane_id_here(), i = l & 15, c = l >> 4;
    const int t = tn & 15;
    if (i == t)
#pragma unroll
      for (int j = 0; j < KV; ++j) {
        const u32x2 lo = quant8_bf16(ld16(nk + 64 * j + 16 * c), k_inv);
        const u32x2 hi = quant8_bf16(ld16(nk + 64 * j + 16 * c + 8), k_inv);
        const u32x4 code = {lo[0], lo[1], hi[0], hi[1]};
        if (tn >= 16) b.k[1][j] = code; else b.k[0][j] = code;
      }
    if (c == (t >> 2)) {
      const VVec x = *reinterpret_cast<const VVec*>(nv + VW * i);
      VRaw vq;
      if constexpr (VW == 8) vq = quant8_bf16(x, v_inv);
      else vq = quant4(bf16_lo(x[0]), bf16_hi(x[0]), bf16_lo(x[1]), bf16_hi(x[1]), v_inv);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * u + 4 * c + r == tn) b.v[u][r] = vq;
    }
  }
  // After patch_new: the lanes holding token tn's codes store them at kd / vd.
  static __device__ __forceinline__ void store_new(const Buf& b, int tn, Elem* kd, Elem* vd) {
    const int l = lane_id_here(), i = l & 15, c = l >> 4;
    const int t = tn & 15;
    if (i == t)
#pragma unroll
      for (int j = 0; j < KV; ++j) st16(kd + 64 * j + 16 * c, tn >= 16 ? b.k[1][j] : b.k[0][j]);
    if (c == (t >> 2)) {
      VRaw x = b.v[0][0];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (16 * u + 4 * c + r == tn) x = b.v[u][r];
      *reinterpret_cast<VRaw*>(vd + VW * i) = x;
    }
  }

  static __device__ __forceinline__ int out_dim(int dt, int c, int r) { return VW * (4 * c + r) + dt; }
};

// ------------------------------------------------------------ wide fp8 tile
// The decode kernel's E4M3 tile: 64-token chunks (four 16-token sub-tiles),
// held raw in registers until they are used.  An E4M3 chunk of 64 tokens
// takes the register bytes of a bf16 chunk of 32, so each wavefront keeps
// the same number of pool bytes in flight as the bf16 kernel (two chunks of
// 16 KB for D 128), where 32-token E4M3 chunks would keep half.  Operand
// layouts, widening and the pool scales are those of TileFp8; the PV product
// takes sub-tiles (0, 1) and (2, 3) as two k = 32 MFMA steps.
template <int D_, int BS_>
struct TileFp8W {
  static constexpr int D = D_;
  static constexpr int BS = BS_;
  static constexpr int CT = 64;
  static constexpr int NSUB = 4;
  // patch_new also stores the new token's codes (from the values it just
  // encoded): reading them back out of one of four sub-tiles would index the
  // chunk buffer dynamically and push it to scratch memory.
  static constexpr bool kStoresInPatch = true;
  static constexpr bool kDoubleBuffer = true;
  static constexpr int kWavesPerEU = 2;
  typedef TileFp8<D_, BS_> Narrow;
  static constexpr int KK = Narrow::KK, KB = Narrow::KB, KV = Narrow::KV, VW = Narrow::VW, NDT = Narrow::NDT;
  typedef uint8_t Elem;
  typedef uint16_t QElem;
  typedef typename Narrow::VVec VVec;
  typedef typename Narrow::VRaw VRaw;
  typedef typename Narrow::Q Q;

  struct Buf { u32x4 k[NSUB][KV]; VRaw v[NSUB][4]; };

  static __device__ __forceinline__ void load_q(Q& q, const QElem* qb, int cols) { Narrow::load_q(q, qb, cols); }
  static __device__ __forceinline__ void load_q_col(Q& q, const QElem* colp, bool valid) {
    Narrow::load_q_col(q, colp, valid);
  }
  static __device__ __forceinline__ int k_lane_off(int rs) { return Narrow::k_lane_off(rs); }
  static __device__ __forceinline__ int v_lane_off(int rs) { return Narrow::v_lane_off(rs); }

  template <bool STREAM = true>
  static __device__ __forceinline__ void load(Buf& b, const Elem* const kp[NSUB], const Elem* const vp[NSUB],
                                              int koff, int voff, int rs) {
#pragma unroll
    for (int u = 0; u < NSUB; ++u) {
#pragma unroll
      for (int j = 0; j < KV; ++j) b.k[u][j] = ld_v<u32x4, STREAM>(kp[u] + koff + 64 * j);
#pragma unroll
      for (int r = 0; r < 4; ++r) b.v[u][r] = ld_v<VRaw, STREAM>(vp[u] + voff + r * rs);
    }
  }

  static __device__ __forceinline__ void qk(const Buf& b, const Q& q, f32x4 s[NSUB]) {
#pragma unroll
    for (int u = 0; u < NSUB; ++u) {
      s[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const uint32_t w0 = b.k[u][kk >> 1][2 * (kk & 1)];
        const uint32_t w1 = b.k[u][kk >> 1][2 * (kk & 1) + 1];
        const u32x4 a = {fp8x2_to_bf16x2(w0, false), fp8x2_to_bf16x2(w0, true), fp8x2_to_bf16x2(w1, false),
                         fp8x2_to_bf16x2(w1, true)};
        s[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, q.q[kk]), s[u], 0, 0, 0);
      }
    }
  }

  static __device__ __forceinline__ void zero_v_rows(Buf& b, int valid) {
    const int c = lane_id() >> 4;
#pragma unroll
    for (int u = 0; u < NSUB; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) b.v[u][r] = 16 * u + 4 * c + r >= valid ? VRaw{} : b.v[u][r];
  }

  // k-step g takes sub-tiles 2g and 2g + 1: its slot 4v + r is token
  // 16(2g + v) + 4c + r, for P and for the transposed V alike.
  static __device__ __forceinline__ void pv(const Buf& b, const float p[NSUB][4], f32x4 o[NDT]) {
#pragma unroll
    for (int g = 0; g < NSUB / 2; ++g) {
      bf16x8 pb;
#pragma unroll
      for (int v = 0; v < 2; ++v)
#pragma unroll
        for (int r = 0; r < 4; ++r) pb[4 * v + r] = (__bf16)p[2 * g + v][r];
      VVec w[2][4];
#pragma unroll
      for (int v = 0; v < 2; ++v)
#pragma unroll
        for (int r = 0; r < 4; ++r) w[v][r] = Narrow::widen(b.v[2 * g + v][r]);
#pragma unroll
      for (int t = 0; t < NDT; ++t) {
        u32x4 a;
        a[0] = Narrow::pick(w[0][0], w[0][1], t);
        a[1] = Narrow::pick(w[0][2], w[0][3], t);
        a[2] = Narrow::pick(w[1][0], w[1][1], t);
        a[3] = Narrow::pick(w[1][2], w[1][3], t);
        o[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), pb, o[t], 0, 0, 0);
      }
    }
  }

  // ---- the step's new token (tn in 0..63): encoded from its bfloat16 input
  // rows exactly as the quantising cache write does, as in TileFp8, and
  // stored at kd / vd (its slot) when they are not null.
  static __device__ __forceinline__ void patch_new(Buf& b, int tn, const void* nkp, const void* nvp, float k_inv,
                                                   float v_inv, Elem* kd, Elem* vd) {
    const uint16_t* nk = static_cast<const uint16_t*>(nkp);
    const uint16_t* nv = static_cast<const uint16_t*>(nvp);
    const int l = lane_id_here(), i = l & 15, c = l >> 4;
    const int t = tn & 15, su = tn >> 4;
    if (i == t)
#pragma unroll
      for (int j = 0; j < KV; ++j) {
        const u32x2 lo = quant8_bf16(ld16(nk + 64 * j + 16 * c), k_inv);
        const u32x2 hi = quant8_bf16(ld16(nk + 64 * j + 16 * c + 8), k_inv);
        const u32x4 code = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int u = 0; u < NSUB; ++u) b.k[u][j] = u == su ? code : b.k[u][j];
        if (kd != nullptr) st16(kd + 64 * j + 16 * c, code);
      }
    if (c == (t >> 2)) {
      const VVec x = *reinterpret_cast<const VVec*>(nv + VW * i);
      VRaw vq;
      if constexpr (VW == 8) vq = quant8_bf16(x, v_inv);
      else vq = quant4(bf16_lo(x[0]), bf16_hi(x[0]), bf16_lo(x[1]), bf16_hi(x[1]), v_inv);
#pragma unroll
      for (int u = 0; u < NSUB; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) b.v[u][r] = 16 * u + 4 * c + r == tn ? vq : b.v[u][r];
      if (vd != nullptr) *reinterpret_cast<VRaw*>(vd + VW * i) = vq;
    }
  }

  static __device__ __forceinline__ int out_dim(int dt, int c, int r) { return VW * (4 * c + r) + dt; }
};

// ------------------------------------------------------------ block id window
// Lane k of `val` holds the physical id of logical block base + k (clamped to
// the pool), for the blocks a sequence owns.
struct BlockWindow {
  const int32_t* row;
  int nblk;
  int base;
  int val;
  int64_t max_id;

  __device__ __forceinline__ void fill(int b) {
    base = b;
    const int lb = b + lane_id();
    int v = 0;
    if (lb < nblk) v = row[lb];
    v = v < 0 ? 0 : v;
    val = (int64_t)v > max_id ? (int)max_id : v;
  }
  // Physical id of logical block lb (clamped to the sequence's last block).
  __device__ __forceinline__ int get(int lb) {
    lb = lb < nblk ? lb : nblk - 1;
    if (lb - base >= kWave || lb < base) fill(lb);
    return __builtin_amdgcn_readlane(val, lb - base);
  }
};

}  // namespace pkv
