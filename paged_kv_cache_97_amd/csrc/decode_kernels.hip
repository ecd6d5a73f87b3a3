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
#include "decode_segment.h"

namespace pkv {

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
    PartMerge pm;
    if (dense) {
      pm.add_range<D>(a.part_ml, a.part_o, pair, a.tile_cols, col, d4, k_first, k_last);
    } else {
      for (int k = k_first;; k = sp.owner(sp.end(k))) {
        pm.add_range<D>(a.part_ml, a.part_o, pair, a.tile_cols, col, d4, k, k);
        if (k == k_last) break;
      }
    }
    st16f(out + col * D + 4 * d4, pm.acc * (a.v_scale / pm.Z));
  }
}

// ------------------------------------------------------------------ shared prefixes
// Decode calls that name groups of sequences sharing their first tokens
// (feifeigd.github.io "vLLM 架构详解" 一, 共享前缀的 Block 复用: a shared
// prefix is held once, in blocks with a reference count above one).  The
// chunk space then starts with a prefix region: for each group, KV head and
// block of prefix_cols(D) query columns (column j * G + gh = head gh of
// member j) one "prefix pair" over the shared tokens, read once through the
// first member's table for all those columns (two or four MFMA column
// tiles).  The members' own
// pairs follow and start at their prefix end.  Prefix segments always write
// parts (one per column); the merge combines a member's prefix parts with its
// own.

struct PrefixGroup {
  int first, n, shared, ncb, nch;
};

// A group as given, clamped to the batch and to whole 16-token sub-tiles (a
// shorter prefix pass is still exact: the members read the rest through
// their own tables).
template <int CT>
__device__ __forceinline__ PrefixGroup prefix_group(const DecodeArgs& a, int g, int max_tok) {
  PrefixGroup p;
  const int B = a.num_seqs;
  p.first = min(max(a.groups[3 * g], 0), B);
  p.n = min(max(a.groups[3 * g + 1], 0), B - p.first);
  p.shared = min(max(a.groups[3 * g + 2], 0), max_tok) & ~15;
  p.ncb = (p.n * a.group + prefix_cols(a.head_dim) - 1) / prefix_cols(a.head_dim);
  p.nch = p.n > 0 ? (p.shared + CT - 1) / CT : 0;
  return p;
}

// Tokens a member reads in the prefix pass: the shared ones it attends, kept
// before its step's new token (a decode step writes that token, so it is
// never in a shared block) and rounded down to a sub-tile.
__device__ __forceinline__ int member_prefix(const DecodeArgs& a, int shared, int L) {
  const int lim = a.new_k != nullptr ? L - 1 : L;
  return max(min(shared, lim), 0) & ~15;
}

// LDS tables of the prefix calls, built by every workgroup.
struct PrefixLds {
  int* cum;    // [B + 1] chunk prefix sums of the members' own pairs
  int* start;  // [B] first token of each sequence's own pairs
  int* grp;    // [B] group of each sequence or -1
  int* gch;    // [NG + 1] prefix-region chunk prefix sums
  int* gpr;    // [NG + 1] prefix-pair prefix sums
};

// Groups are taken in order while their prefix pairs fit the workspace
// (Hkv x (NG + B x G / prefix_cols) pairs, which disjoint groups never
// exceed); groups past that point (only overlapping groups reach it) are
// left out, and their members read everything through their own tables.
template <class Tile>
__device__ void prefix_prologue(const DecodeArgs& a, const PrefixLds& t) {
  const int B = a.num_seqs, NG = a.num_groups;
  const int max_tok = a.max_blocks * Tile::BS;
  block_prefix_sum<256>(NG, t.gpr, [&](int g) {
    return a.num_kv_heads * prefix_group<Tile::CT>(a, g, max_tok).ncb;
  });
  auto enabled = [&](int g) { return t.gpr[g + 1] <= a.pre_pairs_cap; };
  for (int i = threadIdx.x; i < B; i += blockDim.x) t.grp[i] = -1;
  __syncthreads();
  for (int g = 0; g < NG && enabled(g); ++g) {
    const PrefixGroup pg = prefix_group<Tile::CT>(a, g, max_tok);
    for (int j = threadIdx.x; j < pg.n; j += blockDim.x) t.grp[pg.first + j] = g;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < B; i += blockDim.x) {
    const int L = clamp_len(a.seq_lens[i], max_tok);
    const int g = t.grp[i];
    t.start[i] = g >= 0 ? member_prefix(a, prefix_group<Tile::CT>(a, g, max_tok).shared, L) : 0;
  }
  __syncthreads();
  block_prefix_sum<256>(B, t.cum, [&](int i) {
    const int L = clamp_len(a.seq_lens[i], max_tok);
    return (L - t.start[i] + Tile::CT - 1) / Tile::CT;
  });
  block_prefix_sum<256>(NG, t.gch, [&](int g) {
    const PrefixGroup pg = prefix_group<Tile::CT>(a, g, max_tok);
    return enabled(g) ? a.num_kv_heads * pg.ncb * pg.nch : 0;
  });
}

// One range [c0, c1) of chunks of prefix pair (group pg, KV head h, column
// block cb) as worker k: attention of the block's 64 columns over those
// chunks of the shared tokens, written as a part at prefix slot `slot`.
template <class Tile>
__device__ __forceinline__ void run_prefix_segment(const DecodeArgs& a, const PrefixLds& t, const PrefixGroup& pg,
                                                   int h, int cb, int c0, int c1, int64_t slot) {
  constexpr int D = Tile::D, BS = Tile::BS, NDT = Tile::NDT, CT = Tile::CT, NSUB = Tile::NSUB;
  constexpr int PC = prefix_cols(D), NT = PC / 16;
  typedef typename Tile::Elem Elem;
  const int l = lane_id(), col = l & 15, c = l >> 4;
  const int G = a.group, Hkv = a.num_kv_heads;
  const int rs = Hkv * D;
  const Elem* kc = reinterpret_cast<const Elem*>(a.key_cache);
  const Elem* vc = reinterpret_cast<const Elem*>(a.value_cache);
  const auto* qb = reinterpret_cast<const typename Tile::QElem*>(a.query);

  typename Tile::Q q[NT];
  int lim[NT];                                         // tokens this lane's column attends in the pass
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const int f = cb * PC + 16 * tt + col;
    const int j = f / G, gh = f - j * G;
    const bool valid = j < pg.n;
    lim[tt] = valid ? t.start[pg.first + j] : 0;
    Tile::load_q_col(q[tt], qb + ((int64_t)(valid ? pg.first + j : 0) * a.num_q_heads + h * G + gh) * D, valid);
  }

  BlockWindow win;
  win.row = a.block_tables + (int64_t)pg.first * a.max_blocks;
  win.nblk = (pg.shared + BS - 1) / BS;
  win.max_id = a.num_blocks - 1;
  win.fill((c0 * CT) / BS);
  const int koff = Tile::k_lane_off(rs);
  const int voff = Tile::v_lane_off(rs);
  auto bases = [&](int ch, const Elem* kp[NSUB], const Elem* vp[NSUB]) {
#pragma unroll
    for (int u = 0; u < NSUB; ++u) {
      const int tok = ch * CT + 16 * u;
      const int64_t b = (((int64_t)win.get(tok / BS) * BS + tok % BS) * Hkv + h) * D;
      kp[u] = kc + b;
      vp[u] = vc + b;
    }
  };

  float m[NT], lsum[NT];
  f32x4 o[NT][NDT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    m[tt] = -INFINITY;
    lsum[tt] = 0.f;
#pragma unroll
    for (int d = 0; d < NDT; ++d) o[tt][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Columns attend different numbers of tokens (a member shorter than the
  // prefix, columns past the group): masked per column, and a column with
  // nothing visible yet keeps m = -inf, sum 0 and a zero output.
  auto compute = [&](typename Tile::Buf& b, int ch) {
    const int vrows = uniform(pg.shared - ch * CT);
    if (vrows < CT) Tile::zero_v_rows(b, vrows);       // rows past the shared tokens are stale
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      f32x4 sc[NSUB];
      Tile::qk(b, q[tt], sc);
      float x[NSUB][4];
      float cm = -INFINITY;
#pragma unroll
      for (int u = 0; u < NSUB; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = ch * CT + 16 * u + 4 * c + r < lim[tt] ? sc[u][r] * a.scale_log2 : -INFINITY;
          x[u][r] = v;
          cm = fmaxf(cm, v);
        }
      cm = wave_max_across_rows(cm);
      const float mn = fmaxf(m[tt], cm);
      const float ref = mn == -INFINITY ? 0.f : mn;
      const float alpha = fast_exp2(m[tt] - ref);
      m[tt] = mn;
      float p[NSUB][4];
      float ps = 0.f;
#pragma unroll
      for (int u = 0; u < NSUB; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[u][r] = fast_exp2(x[u][r] - ref);
          ps += p[u][r];
        }
      lsum[tt] = lsum[tt] * alpha + ps;
#pragma unroll
      for (int d = 0; d < NDT; ++d) o[tt][d] *= alpha;
      Tile::pv(b, p, o[tt]);
    }
  };

  const Elem* kp[NSUB];
  const Elem* vp[NSUB];
  typename Tile::Buf A, B;
  bases(c0, kp, vp);
  Tile::load(A, kp, vp, koff, voff, rs);
  int ch = c0;
  while (ch + 2 < c1) {
    bases(ch + 1, kp, vp);
    Tile::load(B, kp, vp, koff, voff, rs);
    __builtin_amdgcn_sched_barrier(0);
    compute(A, ch);
    bases(ch + 2, kp, vp);
    Tile::load(A, kp, vp, koff, voff, rs);
    __builtin_amdgcn_sched_barrier(0);
    compute(B, ch + 1);
    ch += 2;
  }
  if (ch + 1 < c1) {
    bases(ch + 1, kp, vp);
    Tile::load(B, kp, vp, koff, voff, rs);
    __builtin_amdgcn_sched_barrier(0);
    compute(A, ch);
    compute(B, ch + 1);
  } else {
    compute(A, ch);
  }

#pragma unroll
  for (int tt = 0; tt < NT; ++tt) {
    const float ls = wave_sum_across_rows(lsum[tt]);
    const int64_t pidx = slot * PC + 16 * tt + col;
    float* dst = a.pre_o + pidx * D;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int g4 = 0; g4 < NDT / 4; ++g4)
        st16f(dst + Tile::out_dim(4 * g4, c, r),
              f32x4{o[tt][4 * g4][r], o[tt][4 * g4 + 1][r], o[tt][4 * g4 + 2][r], o[tt][4 * g4 + 3][r]});
    if (c == 0) {
      a.pre_ml[2 * pidx] = m[tt];
      a.pre_ml[2 * pidx + 1] = ls;
    }
  }
}

// Chunks [x0, x1) of the prefix region as worker k.
template <class Tile>
__device__ __forceinline__ void run_prefix_range(const DecodeArgs& a, const PrefixLds& t, int64_t x0, int64_t x1,
                                                 int k) {
  const int NG = a.num_groups, Hkv = a.num_kv_heads;
  const int max_tok = a.max_blocks * Tile::BS;
  int lo = 0, hi = NG;                                  // the last group g with gch[g] <= x0
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (t.gch[mid] <= x0) lo = mid; else hi = mid;
  }
  int g = uniform(lo);
  int64_t x = x0;
  while (x < x1) {
    while (g < NG - 1 && t.gch[g + 1] <= x) ++g;
    g = uniform(g);
    const PrefixGroup pg = prefix_group<Tile::CT>(a, g, max_tok);
    const int64_t local = x - t.gch[g];
    const int qi = (int)(local / pg.nch);                // prefix pair of the group: h * ncb + cb
    const int ch = (int)(local - (int64_t)qi * pg.nch);
    const int seg = (int)min<int64_t>(pg.nch - ch, x1 - x);
    const int h = qi / pg.ncb, cb = qi - h * pg.ncb;
    (void)Hkv;
    run_prefix_segment<Tile>(a, t, pg, h, cb, ch, ch + seg, (int64_t)t.gpr[g] + qi + k);
    x += seg;
  }
}

// Chunks [x0, x1) of the members' and other sequences' own pairs (chunk 0
// of sequence s at ppseq * cum[s]) as worker k, each pair starting at the
// sequence's first own token.
template <class Tile>
__device__ __forceinline__ void run_own_range(const DecodeArgs& a, const PrefixLds& t, int64_t x0, int64_t x1,
                                              int k) {
  const int B = a.num_seqs;
  const int max_tok = a.max_blocks * Tile::BS;
  const int ppseq = a.num_kv_heads * a.head_tiles;
  const int* cum = t.cum;
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
    const int seg = (int)min<int64_t>(n_s - ch, remaining);
    const int raw_len = uniform(a.seq_lens[s]);
    const int L = clamp_len(raw_len, max_tok);
    const int st = uniform(t.start[s]);
    const bool member = uniform(t.grp[s]) >= 0;
    const int h = pr / a.head_tiles, ht = pr % a.head_tiles;
    int tn = -1;
    int64_t new_row = 0;
    if (a.new_k != nullptr && ch + seg == n_s && raw_len == L) {
      const int lt = L - 1;
      const int phys = uniform(a.block_tables[(int64_t)s * a.max_blocks + lt / Tile::BS]);
      if (phys >= 0 && phys < a.num_blocks) {
        tn = lt - st - (n_s - 1) * Tile::CT;
        new_row = (((int64_t)phys * Tile::BS + lt % Tile::BS) * a.num_kv_heads + h) * Tile::D;
      }
    }
    run_segment<Tile, true>(a, s, s, h, ht, L, ch, ch + seg, !member && ch == 0 && seg == n_s,
                            (int64_t)s * ppseq + pr + k, tn, ht == 0, new_row, st);
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
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
decode_split_prefix_kernel(const DecodeArgs a) {
  extern __shared__ int lds[];
  const int B = a.num_seqs, NG = a.num_groups;
  PrefixLds t;
  t.cum = lds;
  t.start = t.cum + B + 1;
  t.grp = t.start + B;
  t.gch = t.grp + B;
  t.gpr = t.gch + NG + 1;
  prefix_prologue<Tile>(a, t);
  if (blockIdx.x == 0) {
    for (int i = threadIdx.x; i <= B; i += 256) a.cum[i] = t.cum[i];
    for (int i = threadIdx.x; i < B; i += 256) a.seq_group[i] = t.grp[i];
    for (int i = threadIdx.x; i <= NG; i += 256) {
      a.gchunk[i] = t.gch[i];
      a.gpair[i] = t.gpr[i];
    }
  }
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (w >= a.workers) return;
  const int ppseq = a.num_kv_heads * a.head_tiles;
  const int64_t P = t.gch[NG];
  Split sp;
  sp.init(P + (int64_t)ppseq * t.cum[B], a.workers, a.dyn_permille, a.unit_chunks);
  int k = w;
  while (true) {
    const int64_t x0 = sp.begin(k), x1 = sp.end(k);
    if (x0 < min(x1, P)) run_prefix_range<Tile>(a, t, x0, min(x1, P), k);
    if (max(x0, P) < x1) run_own_range<Tile>(a, t, max(x0, P) - P, x1 - P, k);
    if (sp.NU == 0) break;
    int u = 0;
    if (lane_id() == 0) u = atomicAdd(a.counter, 1);
    u = uniform(u);
    if (u >= sp.NU) break;
    k = a.workers + u;
  }
}

// Merge for the shared-prefix calls: a member's prefix parts (from the prefix
// pair holding its column), then its own parts; other sequences as in
// decode_reduce_kernel.  Parts with nothing visible (sum 0) are skipped.
template <class Tile>
__global__ void __launch_bounds__(256) decode_reduce_prefix_kernel(const DecodeArgs a) {
  constexpr int D = Tile::D;
  const int ppseq = a.num_kv_heads * a.head_tiles;
  const int pair = blockIdx.x;
  if (pair == 0 && threadIdx.x == 0) *a.counter = 0;   // the split kernel has finished with it
  const int s = pair / ppseq, pr = pair - s * ppseq;
  const int h = pr / a.head_tiles, ht = pr - h * a.head_tiles;
  const int G = a.group;
  const int cols = min(16, G - 16 * ht);
  const int hq0 = h * G + 16 * ht;
  float* out = a.out + ((int64_t)s * a.num_q_heads + hq0) * D;
  const int B = a.num_seqs, NG = a.num_groups;
  const int max_tok = a.max_blocks * Tile::BS;
  const int n_s = a.cum[s + 1] - a.cum[s];
  const int g = a.seq_group[s];
  constexpr int Q4 = D / 4;
  const int64_t P = a.gchunk[NG];
  Split sp;
  sp.init(P + (int64_t)ppseq * a.cum[B], a.workers, a.dyn_permille, a.unit_chunks);
  const bool dense = sp.S >= sp.W;
  // owners of the own chunks
  const int64_t first = P + (int64_t)ppseq * a.cum[s] + (int64_t)pr * n_s;
  const int64_t last = first + n_s - 1;
  const int k0 = n_s > 0 ? sp.owner(first) : 0, k1 = n_s > 0 ? sp.owner(last) : -1;
  if (g < 0) {
    if (n_s == 0) {
      for (int i = threadIdx.x; i < cols * Q4; i += 256) st16f(out + 4 * i, f32x4{0.f, 0.f, 0.f, 0.f});
      return;
    }
    if (k0 == k1) return;                              // written by its only worker
  }
  PrefixGroup pg{};
  if (g >= 0) pg = prefix_group<Tile::CT>(a, g, max_tok);
  for (int i = threadIdx.x; i < cols * Q4; i += 256) {
    const int col = i / Q4, d4 = i - col * Q4;
    PartMerge pm;
    // the owners k of chunks f0 .. f1, as ranges of consecutive workers
    auto owners = [&](int64_t f0, int64_t f1, const float* ml, const float* o, int64_t base, int64_t ncol, int c) {
      const int a0 = sp.owner(f0), a1 = sp.owner(f1);
      if (dense) {
        pm.add_range<D>(ml, o, base, ncol, c, d4, a0, a1);
      } else {
        for (int k = a0;; k = sp.owner(sp.end(k))) {
          pm.add_range<D>(ml, o, base, ncol, c, d4, k, k);
          if (k == a1) break;
        }
      }
    };
    if (g >= 0 && pg.nch > 0) {
      const int f = (s - pg.first) * G + (hq0 + col - h * G);
      constexpr int PC = prefix_cols(D);
      const int cb = f / PC, ci = f - cb * PC;
      const int qi = h * pg.ncb + cb;
      const int64_t c0 = a.gchunk[g] + (int64_t)qi * pg.nch;
      owners(c0, c0 + pg.nch - 1, a.pre_ml, a.pre_o, a.gpair[g] + qi, PC, ci);
    }
    if (n_s > 0) owners(first, last, a.part_ml, a.part_o, pair, a.tile_cols, col);
    st16f(out + col * D + 4 * d4, pm.Z > 0.f ? pm.acc * (a.v_scale / pm.Z) : f32x4{0.f, 0.f, 0.f, 0.f});
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

// Prefix calls: the decode workspace, then the sequences' groups [B], the
// prefix region's chunk and pair prefix sums [NG + 1] each, and the prefix
// parts: slots = prefix pairs (at most Hkv x (NG + B x G / 64), rounded up)
// + static workers + units, 64 columns each.
static size_t prefix_pairs_cap(int num_seqs, int num_kv_heads, int group, int head_dim, int num_groups) {
  const int pc = prefix_cols(head_dim);
  return (size_t)num_kv_heads * ((size_t)num_groups + ((size_t)num_seqs * group + pc - 1) / pc);
}

static size_t prefix_slots(int num_seqs, int num_kv_heads, int group, int head_dim, int workers, int num_groups) {
  return prefix_pairs_cap(num_seqs, num_kv_heads, group, head_dim, num_groups) + 2 * (size_t)workers;
}

size_t decode_prefix_workspace_bytes(int num_seqs, int num_kv_heads, int group, int head_dim, int workers,
                                     int num_groups) {
  const size_t base = decode_workspace_bytes(num_seqs, num_kv_heads, group, head_dim, workers);
  const size_t tables = ((size_t)num_seqs * 4 + 255) / 256 * 256 + 2 * (((size_t)num_groups + 1) * 4 + 255) / 256 * 256;
  const size_t slots = prefix_slots(num_seqs, num_kv_heads, group, head_dim, workers, num_groups);
  const size_t pc = prefix_cols(head_dim);
  return base + tables + (slots * pc * 2 * 4 + 255) / 256 * 256 + slots * pc * head_dim * 4;
}

void decode_prefix_workspace_carve(DecodeArgs& a, void* ws, int head_dim) {
  decode_workspace_carve(a, ws, head_dim);
  a.pre_pairs_cap = (int)prefix_pairs_cap(a.num_seqs, a.num_kv_heads, a.group, head_dim, a.num_groups);
  char* p = static_cast<char*>(ws) + decode_workspace_bytes(a.num_seqs, a.num_kv_heads, a.group, head_dim, a.workers);
  a.seq_group = reinterpret_cast<int*>(p);
  p += ((size_t)a.num_seqs * 4 + 255) / 256 * 256;
  a.gchunk = reinterpret_cast<int*>(p);
  p += (((size_t)a.num_groups + 1) * 4 + 255) / 256 * 256;
  a.gpair = reinterpret_cast<int*>(p);
  p += (((size_t)a.num_groups + 1) * 4 + 255) / 256 * 256;
  const size_t slots = prefix_slots(a.num_seqs, a.num_kv_heads, a.group, head_dim, a.workers, a.num_groups);
  a.pre_ml = reinterpret_cast<float*>(p);
  p += (slots * prefix_cols(head_dim) * 2 * 4 + 255) / 256 * 256;
  a.pre_o = reinterpret_cast<float*>(p);
}

template <class Tile>
static hipError_t launch_decode_prefix_t(const DecodeArgs& a, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  const int grid = (a.workers + 3) / 4;
  const size_t lds = ((size_t)3 * a.num_seqs + 1 + 2 * ((size_t)a.num_groups + 1)) * sizeof(int);
  if (e0) (void)hipEventRecord(e0, stream);
  hipLaunchKernelGGL(decode_split_prefix_kernel<Tile>, dim3(grid), dim3(256), lds, stream, a);
  if (e1) (void)hipEventRecord(e1, stream);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int pairs = a.num_seqs * a.num_kv_heads * a.head_tiles;
  if (pairs > 0) hipLaunchKernelGGL(decode_reduce_prefix_kernel<Tile>, dim3(pairs), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <class Tile>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t stream, hipEvent_t e0, hipEvent_t e1) {
  if (a.num_groups > 0) {
    if constexpr (std::is_same<Tile, TileF32<Tile::D, Tile::BS>>::value) return hipErrorInvalidValue;
    else return launch_decode_prefix_t<Tile>(a, stream, e0, e1);
  }
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
