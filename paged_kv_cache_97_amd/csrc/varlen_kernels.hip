// Prefill-chunk rows of a varlen attention step (gfx950).
//
// What is computed (gaoleia.github.io "PagedAttention 和 Continuous
// Batching" §2.4: one iteration mixes decode rows with prefill rows; §2.5:
// a long prompt is processed as 512-token chunks between decodes;
// fanquanpp.github.io "vLLM服务内部" 分块预填充): a sequence with q rows and
// seq_len L has c = L - q earlier tokens already cached; row i sits at
// position c + i and attends keys 0 .. c + i.  The mask is aligned to the end
// of the key range, so processing a prompt chunk by chunk equals one causal
// pass over the whole prompt.  Rows of one-row sequences (decode rows) are
// handled by the decode kernels.
//
// Design: the same transposed MFMA tiles as decode (tokens on M), but the N
// side of each 16-column tile holds flat (row, head) pairs f = row * G + head
// of one KV head's query group, so GQA groups and consecutive rows fill the
// tiles without padding.  A wavefront owns NT tiles (16 * NT columns) and
// streams the K/V chunks of its sequence once for all of them, reusing each
// K/V register tile NT times; chunks before the diagonal need no mask, the
// diagonal chunks select per column.  Work items (sequence, KV head, column
// block) are dealt round-robin to a persistent grid.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "tiles.h"

namespace pkv {

template <class Tile, int NT>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
prefill_kernel(const PrefillArgs a) {
  constexpr int D = Tile::D, BS = Tile::BS, NDT = Tile::NDT, COLS = 16 * NT;
  typedef typename Tile::Elem Elem;
  extern __shared__ int cum[];                         // [num_seqs + 1] item prefix
  const int B = a.num_seqs, G = a.group, Hkv = a.num_kv_heads, Hq = a.num_q_heads;
  const int max_tok = a.max_blocks * BS;
  block_prefix_sum<256>(B, cum, [&](int s) {
    const int q = a.qsl[s + 1] - a.qsl[s];
    return q > 1 ? Hkv * ((q * G + COLS - 1) / COLS) : 0;
  });
  const int total = cum[B];
  const int l = lane_id(), col = l & 15, c = l >> 4;
  const int rs = Hkv * D;
  const Elem* kc = reinterpret_cast<const Elem*>(a.key_cache);
  const Elem* vc = reinterpret_cast<const Elem*>(a.value_cache);
  const typename Tile::QElem* qbase = reinterpret_cast<const typename Tile::QElem*>(a.query);
  const int koff = Tile::k_lane_off(rs);
  const int voff = Tile::v_lane_off(rs);

  // Workgroups are dispatched round-robin over the XCDs (j -> XCD j % 8).
  // Renumber them XCD-major so consecutive items -- the column blocks of one
  // (sequence, KV head), which stream the same K/V -- share one XCD's L2.
  constexpr int kXcds = 8;
  const int nwg = gridDim.x;
  int wg = blockIdx.x;
  if (nwg % kXcds == 0) wg = (blockIdx.x % kXcds) * (nwg / kXcds) + blockIdx.x / kXcds;
  for (int item = wg * 4 + (threadIdx.x >> 6); item < total; item += a.waves) {
    int lo = 0, hi = B;                                // last s with cum[s] <= item
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cum[mid] <= item) lo = mid; else hi = mid;
    }
    const int s = uniform(lo);
    const int local = uniform(item - cum[s]);
    const int qrow0 = uniform(a.qsl[s]);
    const int q_s = uniform(a.qsl[s + 1]) - qrow0;
    const int per_head = (q_s * G + COLS - 1) / COLS;
    const int h = local / per_head, cb = local - h * per_head;
    int L = uniform(a.seq_lens[s]);
    L = L < 0 ? 0 : (L > max_tok ? max_tok : L);
    const int ctx = L - q_s;                           // tokens before the chunk's first row
    const int f0 = cb * COLS, f1 = min(f0 + COLS, q_s * G);
    const int p_min = ctx + f0 / G, p_max = ctx + (f1 - 1) / G;
    if (p_max < 0) continue;                           // seq_len < rows: nothing is defined

    typename Tile::Q q[NT];
    int pos[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int f = f0 + 16 * t + col;
      const int row = f / G, head = f - row * G;
      pos[t] = ctx + row;
      Tile::load_q_col(q[t], qbase + ((int64_t)(qrow0 + row) * Hq + h * G + head) * D, f < f1);
    }

    BlockWindow win;
    win.row = a.block_tables + (int64_t)s * a.max_blocks;
    win.nblk = (L + BS - 1) / BS;
    win.max_id = a.num_blocks - 1;
    win.fill(0);
    auto bases = [&](int ch, const Elem* kp[2], const Elem* vp[2]) {
      int64_t b0, b1;
      if (BS == 16) {
        b0 = ((int64_t)win.get(2 * ch) * BS * Hkv + h) * D;
        b1 = ((int64_t)win.get(2 * ch + 1) * BS * Hkv + h) * D;
      } else {
        b0 = ((int64_t)win.get(ch) * BS * Hkv + h) * D;
        b1 = b0 + (int64_t)16 * rs;
      }
      kp[0] = kc + b0;
      kp[1] = kc + b1;
      vp[0] = vc + b0;
      vp[1] = vc + b1;
    };

    float m[NT], lsum[NT];
    f32x4 o[NT][NDT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      m[t] = -INFINITY;
      lsum[t] = 0.f;
#pragma unroll
      for (int d = 0; d < NDT; ++d) o[t][d] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // One chunk for all tiles.  MASK: some column of the item sees only part
    // of this chunk (token > its position is excluded by select); tokens past
    // every column's position get zero V rows.
    auto compute = [&](typename Tile::Buf& b, int ch, auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      const int t0 = ch * 32;
      if constexpr (MASK) {
        const int valid = p_max + 1 - t0;
        if (valid < 32) Tile::zero_v_rows(b, valid);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        f32x4 sc[2];
        Tile::qk(b, q[t], sc);
        float x[2][4];
        float cm = -INFINITY;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float v = sc[u][r] * a.scale_log2;
            if constexpr (MASK) v = (t0 + 16 * u + 4 * c + r <= pos[t]) ? v : -INFINITY;
            x[u][r] = v;
            cm = fmaxf(cm, v);
          }
        cm = wave_max_across_rows(cm);
        const float mn = fmaxf(m[t], cm);
        const float alpha = fast_exp2(m[t] - mn);
        m[t] = mn;
        float p[2][4];
        float ps = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            p[u][r] = fast_exp2(x[u][r] - mn);
            ps += p[u][r];
          }
        lsum[t] = lsum[t] * alpha + ps;
#pragma unroll
        for (int d = 0; d < NDT; ++d) o[t][d] *= alpha;
        Tile::pv(b, p, o[t]);
      }
    };
    auto compute_any = [&](typename Tile::Buf& b, int ch) {
      if (ch * 32 + 31 > p_min) compute(b, ch, std::true_type{});
      else compute(b, ch, std::false_type{});
    };

    const int nch = (p_max + 32) / 32;                 // chunks covering keys 0..p_max
    const Elem* kp[2];
    const Elem* vp[2];
    if constexpr (Tile::kDoubleBuffer) {
      typename Tile::Buf A, Bf;
      bases(0, kp, vp);
      Tile::template load<false>(A, kp, vp, koff, voff, rs);
      int ch = 0;
      while (ch + 2 < nch) {
        bases(ch + 1, kp, vp);
        Tile::template load<false>(Bf, kp, vp, koff, voff, rs);
        __builtin_amdgcn_sched_barrier(0);
        compute_any(A, ch);
        bases(ch + 2, kp, vp);
        Tile::template load<false>(A, kp, vp, koff, voff, rs);
        __builtin_amdgcn_sched_barrier(0);
        compute_any(Bf, ch + 1);
        ch += 2;
      }
      if (ch + 1 < nch) {
        bases(ch + 1, kp, vp);
        Tile::template load<false>(Bf, kp, vp, koff, voff, rs);
        __builtin_amdgcn_sched_barrier(0);
        compute_any(A, ch);
        compute_any(Bf, ch + 1);
      } else {
        compute_any(A, ch);
      }
    } else {
      typename Tile::Buf A;
      for (int ch = 0; ch < nch; ++ch) {
        bases(ch, kp, vp);
        Tile::template load<false>(A, kp, vp, koff, voff, rs);
        compute_any(A, ch);
      }
    }

#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float tot = wave_sum_across_rows(lsum[t]);
      const int f = f0 + 16 * t + col;
      if (f >= f1) continue;
      const int row = f / G, head = f - row * G;
      const float inv = a.v_scale / tot;
      float* dst = a.out + ((int64_t)(qrow0 + row) * Hq + h * G + head) * D;
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int g = 0; g < NDT / 4; ++g)
          st16f(dst + Tile::out_dim(4 * g, c, r),
                f32x4{o[t][4 * g][r] * inv, o[t][4 * g + 1][r] * inv, o[t][4 * g + 2][r] * inv,
                      o[t][4 * g + 3][r] * inv});
    }
  }
}

// Tiles per wavefront: as many as the register file holds without spilling.
template <bool BF16, int D> struct PrefillTiles { static constexpr int value = D == 128 ? 2 : 4; };
template <int D> struct PrefillTiles<false, D> { static constexpr int value = 2; };


template <class Tile, int NT>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t stream) {
  const int grid = (a.waves + 3) / 4;
  const size_t lds = (size_t)(a.num_seqs + 1) * sizeof(int);
  hipLaunchKernelGGL((prefill_kernel<Tile, NT>), dim3(grid), dim3(256), lds, stream, a);
  return hipGetLastError();
}

bool prefill_uses_plan(int head_dim, KvKind kind) {
  return (kind == KvKind::BF16 || kind == KvKind::FP8) && head_dim == 128;
}

hipError_t launch_prefill(const PrefillArgs& a, int head_dim, int block_size, KvKind kind, int cus,
                          hipStream_t stream) {
  if (prefill_uses_plan(head_dim, kind))
    return launch_prefill_lds(a, block_size, kind == KvKind::FP8, cus, stream);
#define PKV_CASE(T, B, D, BS) \
  if (head_dim == D && block_size == BS) return launch_prefill_t<T<D, BS>, PrefillTiles<B, D>::value>(a, stream);
  if (kind == KvKind::FP8) {
    PKV_CASE(TileFp8, true, 128, 16)
    PKV_CASE(TileFp8, true, 128, 32)
    PKV_CASE(TileFp8, true, 64, 16)
    PKV_CASE(TileFp8, true, 64, 32)
  } else if (kind == KvKind::BF16) {
    PKV_CASE(TileBf16, true, 128, 16)
    PKV_CASE(TileBf16, true, 128, 32)
    PKV_CASE(TileBf16, true, 64, 16)
    PKV_CASE(TileBf16, true, 64, 32)
  } else {
    PKV_CASE(TileF32, false, 128, 16)
    PKV_CASE(TileF32, false, 128, 32)
    PKV_CASE(TileF32, false, 64, 16)
    PKV_CASE(TileF32, false, 64, 32)
  }
#undef PKV_CASE
  return hipErrorInvalidValue;
}

}  // namespace pkv
