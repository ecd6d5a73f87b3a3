// One wavefront's decode attention over a range of chunks of one
// (sequence, KV head, head tile) pair, and the merge of split parts.  Used
// by the decode split kernels and by the mixed varlen kernel's decode rows.
#pragma once

#include <type_traits>

#include "common.h"
#include "launch.h"
#include "tiles.h"

namespace pkv {

__device__ __forceinline__ int clamp_len(int L, int max_tok) {
  return L < 0 ? 0 : (L > max_tok ? max_tok : L);
}

// One range [c0, c1) of chunks of one pair; chunk ch covers tokens t0 + ch *
// CT .. (OFF: t0 is a multiple of 16 that the shared-prefix calls pass; the
// plain kernels start at token 0 and keep their block arithmetic).
// tn >= 0: chunk c1 - 1 is the sequence's last and its token tn is the step's
// new token (fused write); writer: this wave also stores it at element offset
// new_row of the pools.
template <class Tile, bool OFF = false>
__device__ __forceinline__ void run_segment(const DecodeArgs& a, int s, int row, int h, int ht, int L,
                                            int c0, int c1, bool single, int64_t slot, int tn, bool writer,
                                            int64_t new_row, int t0_ = 0) {
  const int t0 = OFF ? t0_ : 0;
  constexpr int D = Tile::D, BS = Tile::BS, NDT = Tile::NDT, CT = Tile::CT, NSUB = Tile::NSUB;
  typedef typename Tile::Elem Elem;
  const int l = lane_id(), col = l & 15, c = l >> 4;
  const int G = a.group;
  const int cols = min(16, G - 16 * ht);
  const int hq0 = h * G + 16 * ht;
  const int Hkv = a.num_kv_heads;
  const int rs = Hkv * D;                              // elements between token rows
  const Elem* kc = reinterpret_cast<const Elem*>(a.key_cache);
  const Elem* vc = reinterpret_cast<const Elem*>(a.value_cache);

  typename Tile::Q q;
  Tile::load_q(q, reinterpret_cast<const typename Tile::QElem*>(a.query) + ((int64_t)row * a.num_q_heads + hq0) * D,
               cols);

  BlockWindow win;
  win.row = a.block_tables + (int64_t)s * a.max_blocks;
  win.nblk = (L + BS - 1) / BS;
  win.max_id = a.num_blocks - 1;
  win.fill((t0 + c0 * CT) / BS);

  const int koff = Tile::k_lane_off(rs);
  const int voff = Tile::v_lane_off(rs);
  // Wave-uniform pointers to row 0 of the 16-token sub-tiles of chunk ch
  // (sub-tile u: tokens ch * CT + 16u ..; a 32-token block holds two).
  auto bases = [&](int ch, const Elem* kp[NSUB], const Elem* vp[NSUB]) {
    int64_t b[NSUB];
#pragma unroll
    for (int u = 0; u < NSUB; ++u) {
      if constexpr (OFF) {
        const int tok = t0 + ch * CT + 16 * u;               // a sub-tile never crosses a block
        b[u] = (((int64_t)win.get(tok / BS) * BS + tok % BS) * Hkv + h) * D;
      } else if (BS == 16)
        b[u] = ((int64_t)win.get(ch * (CT / 16) + u) * BS * Hkv + h) * D;
      else if (u % 2 == 0)
        b[u] = ((int64_t)win.get(ch * (CT / 32) + u / 2) * BS * Hkv + h) * D;
      else
        b[u] = b[u - 1] + (int64_t)16 * rs;
      kp[u] = kc + b[u];
      vp[u] = vc + b[u];
    }
  };

  float m = -INFINITY, lsum = 0.f;
  f32x4 o[NDT];
#pragma unroll
  for (int t = 0; t < NDT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // One chunk of the online softmax.  TAIL: the chunk holds the sequence's
  // last `valid` (< CT) tokens; the others are masked by select and their V
  // rows zeroed so stale slot contents never reach a product.
  auto compute = [&](typename Tile::Buf& b, auto tail_tag, int valid) {
    constexpr bool TAIL = decltype(tail_tag)::value;
    f32x4 sc[NSUB];
    Tile::qk(b, q, sc);
    if constexpr (TAIL) Tile::zero_v_rows(b, valid);
    float x[NSUB][4];
    float cm = -INFINITY;
#pragma unroll
    for (int u = 0; u < NSUB; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = sc[u][r] * a.scale_log2;
        if constexpr (TAIL) v = (16 * u + 4 * c + r < valid) ? v : -INFINITY;
        x[u][r] = v;
        cm = fmaxf(cm, v);
      }
    cm = wave_max_across_rows(cm);
    const float mn = fmaxf(m, cm);
    const float alpha = fast_exp2(m - mn);             // 0 on the first chunk (m = -inf)
    m = mn;
    float p[NSUB][4];
    float ps = 0.f;
#pragma unroll
    for (int u = 0; u < NSUB; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[u][r] = fast_exp2(x[u][r] - mn);
        ps += p[u][r];
      }
    lsum = lsum * alpha + ps;
#pragma unroll
    for (int t = 0; t < NDT; ++t) o[t] *= alpha;
    Tile::pv(b, p, o);
  };
  // The last chunk of a range may be the sequence's partial chunk, and may
  // hold the step's new token: patched in from the input rows (the patch
  // loads are issued only here, so the steady-state loop is unchanged) and
  // stored to its slot by the writer.
  auto compute_last = [&](typename Tile::Buf& b, int ch) {
    if (tn >= 0) {
      const int64_t nrow = ((int64_t)s * Hkv + h) * D;
      const auto* nk = reinterpret_cast<const typename Tile::QElem*>(a.new_k) + nrow;
      const auto* nv = reinterpret_cast<const typename Tile::QElem*>(a.new_v) + nrow;
      if constexpr (Tile::kStoresInPatch) {
        Tile::patch_new(b, tn, nk, nv, a.k_inv, a.v_inv, writer ? const_cast<Elem*>(kc) + new_row : nullptr,
                        writer ? const_cast<Elem*>(vc) + new_row : nullptr);
      } else {
        Tile::patch_new(b, tn, nk, nv, a.k_inv, a.v_inv);
        if (writer)
          Tile::store_new(b, tn, const_cast<Elem*>(kc) + new_row, const_cast<Elem*>(vc) + new_row);
      }
    }
    const int valid = uniform(L - t0 - ch * CT);
    if (valid < CT) compute(b, std::true_type{}, valid);
    else compute(b, std::false_type{}, CT);
  };

  const Elem* kp[NSUB];
  const Elem* vp[NSUB];
  if constexpr (Tile::kDoubleBuffer) {
    // Steady state: the loads of chunk ch+1 are always in flight while chunk
    // ch is computed (unconditional prefetch keeps the wait counts exact).
    typename Tile::Buf A, B;
    bases(c0, kp, vp);
    Tile::load(A, kp, vp, koff, voff, rs);
    int ch = c0;
    // sched_barrier keeps the compiler from sinking the prefetch below the
    // waits of the chunk being computed.
    while (ch + 2 < c1) {
      bases(ch + 1, kp, vp);
      Tile::load(B, kp, vp, koff, voff, rs);
      __builtin_amdgcn_sched_barrier(0);
      compute(A, std::false_type{}, CT);
      bases(ch + 2, kp, vp);
      Tile::load(A, kp, vp, koff, voff, rs);
      __builtin_amdgcn_sched_barrier(0);
      compute(B, std::false_type{}, CT);
      ch += 2;
    }
    if (ch + 1 < c1) {
      bases(ch + 1, kp, vp);
      Tile::load(B, kp, vp, koff, voff, rs);
      __builtin_amdgcn_sched_barrier(0);
      compute(A, std::false_type{}, CT);
      compute_last(B, ch + 1);
    } else {
      compute_last(A, ch);
    }
  } else {
    typename Tile::Buf A;
    for (int ch = c0; ch < c1 - 1; ++ch) {
      bases(ch, kp, vp);
      Tile::load(A, kp, vp, koff, voff, rs);
      compute(A, std::false_type{}, CT);
    }
    bases(c1 - 1, kp, vp);
    Tile::load(A, kp, vp, koff, voff, rs);
    compute_last(A, c1 - 1);
  }

  lsum = wave_sum_across_rows(lsum);
  if (col >= cols) return;
  if (single) {
    const float inv = a.v_scale / lsum;
    float* dst = a.out + ((int64_t)row * a.num_q_heads + hq0 + col) * D;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int g = 0; g < NDT / 4; ++g)
        st16f(dst + Tile::out_dim(4 * g, c, r),
              f32x4{o[4 * g][r] * inv, o[4 * g + 1][r] * inv, o[4 * g + 2][r] * inv, o[4 * g + 3][r] * inv});
  } else {
    const int64_t pidx = slot * a.tile_cols + col;
    float* dst = a.part_o + pidx * D;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int g = 0; g < NDT / 4; ++g)
        st16f(dst + Tile::out_dim(4 * g, c, r),
              f32x4{o[4 * g][r], o[4 * g + 1][r], o[4 * g + 2][r], o[4 * g + 3][r]});
    if (c == 0) {
      a.part_ml[2 * pidx] = m;
      a.part_ml[2 * pidx + 1] = lsum;
    }
  }
}

// Online merge of split parts (max m, sum l, unnormalised output o) into a
// running (M, Z, acc): parts with nothing visible (l == 0) are skipped.
struct PartMerge {
  float M = -INFINITY, Z = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  __device__ __forceinline__ void add(float mk, float lk, const f32x4& ok) {
    if (lk == 0.f) return;
    const float mn = fmaxf(M, mk);
    const float s_old = fast_exp2(M - mn), s_new = fast_exp2(mk - mn);
    Z = Z * s_old + lk * s_new;
    acc = acc * s_old + ok * s_new;
    M = mn;
  }
  // N parts from worker kb on (those past k1 count as empty): their loads
  // are issued before any of them is merged.
  template <int D, int N>
  __device__ __forceinline__ void add_batch(const float* ml, const float* o, int64_t base, int64_t cols, int col,
                                            int d4, int kb, int k1) {
    float mk[N], lk[N];
    f32x4 ok[N];
#pragma unroll
    for (int j = 0; j < N; ++j) {
      const int k = min(kb + j, k1);
      const int64_t p = (base + k) * cols + col;
      mk[j] = ml[2 * p];
      lk[j] = kb + j <= k1 ? ml[2 * p + 1] : 0.f;
      ok[j] = *reinterpret_cast<const f32x4*>(o + p * D + 4 * d4);
    }
#pragma unroll
    for (int j = 0; j < N; ++j) add(mk[j], lk[j], ok[j]);
  }
  // The parts of workers k0 .. k1 (slot = base + k; ml stride 2, o stride D
  // per slot and column) in batches of eight, then four, so that a long list
  // costs a few round trips, not one each.
  template <int D>
  __device__ __forceinline__ void add_range(const float* ml, const float* o, int64_t base, int64_t cols, int col,
                                            int d4, int k0, int k1) {
    int kb = k0;
    for (; k1 - kb >= 7; kb += 8) add_batch<D, 8>(ml, o, base, cols, col, d4, kb, k1);
    for (; kb <= k1; kb += 4) add_batch<D, 4>(ml, o, base, cols, col, d4, kb, k1);
  }
};

}  // namespace pkv
