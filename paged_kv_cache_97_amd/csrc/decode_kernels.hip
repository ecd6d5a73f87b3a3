// Paged decode attention for gfx950: a split kernel that walks block tables
// and a reduction kernel that merges split parts.
//
// What is computed (gaoleia.github.io "PagedAttention 和 Continuous
// Batching" §1.6): for sequence s and query head hq, gather the first
// seq_len tokens' K and V rows of KV head hq / G through the block table in
// logical order and return softmax(scale * q K^T) V.  Paging changes where K/V
// live, not the result.  Decode time is spent reading the KV cache (same
// page, §2.4), so the kernel is built around HBM streaming.
//
// Design (MI355X-first; the pages give no kernel):
//  * Work unit = one chunk (32 tokens; 64 for E4M3 pools, whose bytes per
//    token are half) of one (sequence, KV head, head tile) "pair".  All chunks of all pairs are laid end to end and cut into
//    `workers` equal contiguous ranges, one per wavefront (stream-K style),
//    so every wave streams the same number of KV bytes whatever the length
//    mix.  A wave whose range covers a whole pair writes the final row; other
//    ranges leave an unnormalised part (max, sum, output) in the workspace
//    and the reduction kernel merges the parts of each pair.
//  * Each wave serves all G query heads that share its KV head, so every K/V
//    byte is read once per step (GQA grouping).  Up to 16 heads form the N
//    side of the MFMA tiles:
//      S^T[token, head] = K[token, :] . Q[head, :]         (A = K rows)
//      O^T[dim, head]  += V^T[dim, token] P^T[token, head]  (A = V rows)
//    With tokens on M, the S^T accumulator already has each lane's P values
//    in the k-slots of the P^T operand, and each head's softmax state lives
//    in the lanes that own its O^T column; no LDS round trip is needed.
//  * K rows are loaded straight into MFMA A-operand registers (16 B per lane,
//    64 B runs per row).  V is loaded as whole 256-byte head rows (16 lanes x
//    16 B, four rows per instruction) and transposed inside each lane with
//    v_perm_b32 into the A operand of the PV product.
//  * bf16 uses v_mfma_f32_16x16x32_bf16 with P rounded to bf16; fp32 uses
//    v_mfma_f32_16x16x4_f32 and keeps P in fp32.  FP8 (E4M3) pools are read
//    at one byte per element, widened exactly to bf16 in registers and fed to
//    the bf16 MFMA; k_scale is folded into the softmax scale and v_scale into
//    the final normalisation.
//  * Online softmax in the log2 domain: per chunk the max over tokens is
//    reduced across the four 16-lane rows with two cross-lane xors; the sum
//    stays lane-local until the end.  Masked tokens are excluded by select
//    and their V rows zeroed, so stale NaN slots never reach a product.
//  * KV tiles are read once per step, so they are loaded non-temporally
//    (streaming hint): on MI355X this lifts the split kernel from about 5.2
//    to 5.8 TB/s on the 128-sequence GQA batch, close to the ~6 TB/s a plain
//    random 4 KB-tile gather reaches on the same part.
//  * Block ids: each wave holds a 64-entry window of its block-table row in
//    one VGPR and reads entries with v_readlane; loads of chunk n+1 are in
//    flight while chunk n is computed (bf16).
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "tiles.h"
#include "prefill_plan.h"

namespace pkv {

// One range [c0, c1) of chunks of one pair.
// tn >= 0: chunk c1 - 1 is the sequence's last and its token tn is the step's
// new token (fused write); writer: this wave also stores it at element offset
// new_row of the pools.
template <class Tile>
__device__ __forceinline__ void run_segment(const DecodeArgs& a, int s, int row, int h, int ht, int L,
                                            int c0, int c1, bool single, int64_t slot, int tn, bool writer,
                                            int64_t new_row) {
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
  win.fill((c0 * CT) / BS);

  const int koff = Tile::k_lane_off(rs);
  const int voff = Tile::v_lane_off(rs);
  // Wave-uniform pointers to row 0 of the 16-token sub-tiles of chunk ch
  // (sub-tile u: tokens ch * CT + 16u ..; a 32-token block holds two).
  auto bases = [&](int ch, const Elem* kp[NSUB], const Elem* vp[NSUB]) {
    int64_t b[NSUB];
#pragma unroll
    for (int u = 0; u < NSUB; ++u) {
      if (BS == 16)
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
    const int valid = uniform(L - ch * CT);
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

__device__ __forceinline__ int clamp_len(int L, int max_tok) {
  return L < 0 ? 0 : (L > max_tok ? max_tok : L);
}

// Chunks of CT tokens of each pair of sequence s that this launch handles,
// plus the pair's virtual start-up chunks (0 for skipped and empty sequences).
template <int CT>
__device__ __forceinline__ int seq_chunks(const DecodeArgs& a, int s, int max_tok) {
  if (a.qsl != nullptr && a.qsl[s + 1] - a.qsl[s] != 1) return 0;
  const int n = (clamp_len(a.seq_lens[s], max_tok) + CT - 1) / CT;
  return n > 0 ? n + a.seg_chunks : 0;
}

// How the chunk space [0, total) is shared out.  Chunks [0, S) go in equal
// static ranges to the `workers` wavefronts; the last chunks [S, total) form
// NU units of U chunks (the last one may be shorter), "virtual workers"
// W .. W + NU - 1, which wavefronts take from a counter once their static
// range is done, so that waves on faster compute units take more of them.
// Every range, static or not, is fixed by (total, W, dyn_permille,
// unit_chunks) alone, so the parts and their merge order do not depend on
// which wave ran a unit: results are the same from run to run.  NU <= W.
struct Split {
  int64_t total, S, U;
  int W, NU;
  __device__ __forceinline__ void init(int64_t total_, int W_, int dyn_permille, int unit_chunks) {
    total = total_;
    W = W_;
    const int64_t dyn = total * dyn_permille / 1000;
    U = max<int64_t>(max(unit_chunks, 1), (dyn + W - 1) / W);
    NU = (int)((dyn + U - 1) / U);
    S = total - dyn;
  }
  __device__ __forceinline__ int64_t begin(int k) const { return k < W ? S * k / W : S + (int64_t)(k - W) * U; }
  __device__ __forceinline__ int64_t end(int k) const {
    return k < W ? S * (k + 1) / W : min(S + (int64_t)(k - W + 1) * U, total);
  }
  // the worker (static or virtual) whose range holds chunk x < total
  __device__ __forceinline__ int owner(int64_t x) const {
    return x < S ? (int)(((x + 1) * W - 1) / S) : W + (int)((x - S) / U);
  }
};

// Attend over the chunks [x0, x1) of the sequence-major chunk space (pairs of
// sequence s at ppseq * cum[s] .., chunks of one pair consecutive) as worker k:
// segment by segment, each pair's piece written whole or as a part at slot
// pair + k.
template <class Tile>
__device__ __forceinline__ void run_range(const DecodeArgs& a, const int* cum, int64_t x0, int64_t x1, int k) {
  const int B = a.num_seqs;
  const int max_tok = a.max_blocks * Tile::BS;
  const int ppseq = a.num_kv_heads * a.head_tiles;     // pairs per sequence
  // sequence holding chunk x0: the last s with ppseq * cum[s] <= x0
  int lo = 0, hi = B;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if ((int64_t)ppseq * cum[mid] <= x0) lo = mid; else hi = mid;
  }
  int s = uniform(lo);
  int n_s = uniform(cum[s + 1] - cum[s]);
  const int64_t local = x0 - (int64_t)ppseq * uniform(cum[s]);
  int pr = (int)(local / n_s);
  int ch = (int)(local - (int64_t)pr * n_s);
  int64_t remaining = x1 - x0;
  while (true) {
    // Positions count the pair's seg_chunks virtual chunks first: [ch, ch +
    // seg) maps to the real chunks [r0, r1).
    const int seg = (int)min<int64_t>(n_s - ch, remaining);
    const int n_real = n_s - a.seg_chunks;
    const int r0 = max(ch - a.seg_chunks, 0), r1 = max(ch + seg - a.seg_chunks, 0);
    const int raw_len = uniform(a.seq_lens[s]);
    const int L = clamp_len(raw_len, max_tok);
    const int row = a.qsl ? uniform(a.qsl[s]) : s;
    const int h = pr / a.head_tiles, ht = pr % a.head_tiles;
    // Fused write: the range holding the sequence's last chunk owns the new
    // token (position L - 1) when seq_lens was not clamped and the token's
    // block id is in the pool (otherwise the slot is not written and the
    // token is read from the pool, as a separate write would leave it).
    int tn = -1;
    int64_t new_row = 0;
    if (a.new_k != nullptr && r1 == n_real && r1 > r0 && raw_len == L) {
      const int lt = L - 1;
      const int phys = uniform(a.block_tables[(int64_t)s * a.max_blocks + lt / Tile::BS]);
      if (phys >= 0 && phys < a.num_blocks) {
        tn = lt & (Tile::CT - 1);
        new_row = (((int64_t)phys * Tile::BS + lt % Tile::BS) * a.num_kv_heads + h) * Tile::D;
      }
    }
    if (r1 > r0)                                       // a range of virtual chunks only does nothing
      run_segment<Tile>(a, s, row, h, ht, L, r0, r1, r0 == 0 && r1 == n_real, (int64_t)s * ppseq + pr + k, tn,
                        ht == 0, new_row);
    remaining -= seg;
    if (remaining <= 0) break;
    ch = 0;
    if (++pr == ppseq) {
      pr = 0;
      do { ++s; } while (s < B - 1 && cum[s + 1] == cum[s]);
      if (s >= B) break;
      s = uniform(s);
      n_s = uniform(cum[s + 1] - cum[s]);
    }
  }
}

template <class Tile>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(Tile::kWavesPerEU)))
decode_split_kernel(const DecodeArgs a) {
  extern __shared__ int cum[];                         // [num_seqs + 1]
  const int B = a.num_seqs;
  const int max_tok = a.max_blocks * Tile::BS;
  block_prefix_sum<256>(B, cum, [&](int s) { return seq_chunks<Tile::CT>(a, s, max_tok); });
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i <= B; i += 256) a.cum[i] = cum[i];

  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= a.workers) return;
  const int ppseq = a.num_kv_heads * a.head_tiles;
  Split sp;
  sp.init((int64_t)ppseq * cum[B], a.workers, a.dyn_permille, a.unit_chunks);
  // The static range first, then units, first come first served (the
  // counter is zero on entry; the merge kernel of the same call resets it).
  // One call site, so the range code is inlined once.
  // A unit is claimed only when the wave is free to run it: claiming earlier
  // would hand units to waves that are still busy.
  int k = w;
  while (true) {
    const int64_t x0 = sp.begin(k), x1 = sp.end(k);
    if (x0 < x1) run_range<Tile>(a, cum, x0, x1, k);
    if (sp.NU == 0) break;
    int u = 0;
    if (lane_id() == 0) u = atomicAdd(a.counter, 1);
    u = uniform(u);
    if (u >= sp.NU) break;
    k = a.workers + u;
  }
}

// Merge the parts of one pair (blockIdx.x = s * ppseq + pr); pairs done by a
// single worker were written by the split kernel, empty sequences get zeros.
template <int D>
__global__ void __launch_bounds__(256) decode_reduce_kernel(const DecodeArgs a) {
  const int ppseq = a.num_kv_heads * a.head_tiles;
  const int pair = blockIdx.x;
  if (pair == 0 && threadIdx.x == 0) *a.counter = 0;   // the split kernel has finished with it
  if (pair == a.num_seqs * ppseq) {                    // the extra workgroup: the prefill rows' item plan
    build_prefill_plan(a.qsl, a.seq_lens, a.num_seqs, a.prefill_max_tok, a.num_kv_heads, a.group, a.prefill_plan);
    return;
  }
  const int s = pair / ppseq, pr = pair - s * ppseq;
  if (a.qsl != nullptr && a.qsl[s + 1] - a.qsl[s] != 1) return;
  const int h = pr / a.head_tiles, ht = pr - h * a.head_tiles;
  const int cols = min(16, a.group - 16 * ht);
  const int hq0 = h * a.group + 16 * ht;
  const int row = a.qsl ? a.qsl[s] : s;
  float* out = a.out + ((int64_t)row * a.num_q_heads + hq0) * D;
  const int B = a.num_seqs;
  const int n_s = a.cum[s + 1] - a.cum[s];             // real + virtual chunks per pair
  constexpr int Q4 = D / 4;
  if (n_s == 0) {
    for (int i = threadIdx.x; i < cols * Q4; i += 256) st16f(out + 4 * i, f32x4{0.f, 0.f, 0.f, 0.f});
    return;
  }
  // the workers that hold the pair's real chunks (positions seg_chunks ..)
  Split sp;
  sp.init((int64_t)ppseq * a.cum[B], a.workers, a.dyn_permille, a.unit_chunks);
  const int64_t first = (int64_t)ppseq * a.cum[s] + (int64_t)pr * n_s + a.seg_chunks;
  const int64_t last = (int64_t)ppseq * a.cum[s] + (int64_t)pr * n_s + n_s - 1;
  const int k_first = sp.owner(first), k_last = sp.owner(last);
  if (k_first == k_last) return;
  // Parts in chunk order.  When every static range holds a chunk (S >= W;
  // units are never empty) the owners of the pair's chunks are the workers
  // k_first .. k_last, so the parts' loads do not depend on each other;
  // otherwise each owner's range is followed to the owner of the next chunk.
  const bool dense = sp.S >= sp.W;
  for (int i = threadIdx.x; i < cols * Q4; i += 256) {
    const int col = i / Q4, d4 = i - col * Q4;
    // one pass with a running maximum: rescale what has been merged so far
    float M = -INFINITY, Z = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto add = [&](int k) {
      const int64_t p = ((int64_t)pair + k) * a.tile_cols + col;
      const float mk = a.part_ml[2 * p], lk = a.part_ml[2 * p + 1];
      const f32x4 ok = *reinterpret_cast<const f32x4*>(a.part_o + p * D + 4 * d4);
      const float mn = fmaxf(M, mk);
      const float s_old = fast_exp2(M - mn), s_new = fast_exp2(mk - mn);
      Z = Z * s_old + lk * s_new;
      acc = acc * s_old + ok * s_new;
      M = mn;
    };
    if (dense) {
#pragma unroll 4
      for (int k = k_first; k <= k_last; ++k) add(k);
    } else {
      for (int k = k_first;; k = sp.owner(sp.end(k))) {
        add(k);
        if (k == k_last) break;
      }
    }
    st16f(out + col * D + 4 * d4, acc * (a.v_scale / Z));
  }
}

// Workspace: the unit counter in the first word (at the same place whatever
// the call's shape, so the reset of one call holds for the next), chunk
// prefix sums [B + 1], then per slot (max, sum) and the unnormalised partial
// outputs; slots = pairs + static workers + at most as many units.
size_t decode_workspace_bytes(int num_seqs, int num_kv_heads, int group, int head_dim, int workers) {
  const int head_tiles = (group + 15) / 16;
  const int tile_cols = group < 16 ? group : 16;
  const size_t slots = (size_t)num_seqs * num_kv_heads * head_tiles + 2 * (size_t)workers;
  const size_t cum = 256 + ((size_t)(num_seqs + 1) * 4 + 255) / 256 * 256;
  const size_t ml = (slots * tile_cols * 2 * 4 + 255) / 256 * 256;
  const size_t o = slots * tile_cols * head_dim * 4;
  return cum + ml + o;
}

void decode_workspace_carve(DecodeArgs& a, void* ws, int head_dim) {
  const size_t slots = (size_t)a.num_seqs * a.num_kv_heads * a.head_tiles + 2 * (size_t)a.workers;
  char* p = static_cast<char*>(ws);
  a.counter = reinterpret_cast<int*>(p);
  p += 256;
  a.cum = reinterpret_cast<int*>(p);
  p += ((size_t)(a.num_seqs + 1) * 4 + 255) / 256 * 256;
  a.part_ml = reinterpret_cast<float*>(p);
  p += (slots * a.tile_cols * 2 * 4 + 255) / 256 * 256;
  a.part_o = reinterpret_cast<float*>(p);
  (void)head_dim;
}

template <class Tile>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  const int grid = (a.workers + 3) / 4;
  const size_t lds = (size_t)(a.num_seqs + 1) * sizeof(int);
  if (e0) (void)hipEventRecord(e0, stream);
  hipLaunchKernelGGL(decode_split_kernel<Tile>, dim3(grid), dim3(256), lds, stream, a);
  if (e1) (void)hipEventRecord(e1, stream);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int pairs = a.num_seqs * a.num_kv_heads * a.head_tiles;
  if (pairs > 0)
    hipLaunchKernelGGL(decode_reduce_kernel<Tile::D>, dim3(pairs + (a.prefill_plan != nullptr ? 1 : 0)), dim3(256), 0,
                       stream, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int head_dim, int block_size, KvKind kind,
                         hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
#define PKV_CASE(T, D, BS) \
  if (head_dim == D && block_size == BS) return launch_decode_t<T<D, BS>>(a, stream, e0, e1);
  if (kind == KvKind::FP8) {
    PKV_CASE(TileFp8W, 128, 16)
    PKV_CASE(TileFp8W, 128, 32)
    PKV_CASE(TileFp8W, 64, 16)
    PKV_CASE(TileFp8W, 64, 32)
  } else if (kind == KvKind::BF16) {
    PKV_CASE(TileBf16, 128, 16)
    PKV_CASE(TileBf16, 128, 32)
    PKV_CASE(TileBf16, 64, 16)
    PKV_CASE(TileBf16, 64, 32)
  } else {
    PKV_CASE(TileF32, 128, 16)
    PKV_CASE(TileF32, 128, 32)
    PKV_CASE(TileF32, 64, 16)
    PKV_CASE(TileF32, 64, 32)
  }
#undef PKV_CASE
  return hipErrorInvalidValue;
}

}  // namespace pkv
