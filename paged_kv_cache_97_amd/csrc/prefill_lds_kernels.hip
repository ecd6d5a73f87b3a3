// Prefill-chunk rows for bf16, head_dim 128: the workgroup-shared variant.
//
// Same computation as prefill_kernel (gaoleia.github.io "PagedAttention 和
// Continuous Batching" §2.4-§2.5: a chunk of q rows after c cached tokens,
// row i attends keys 0 .. c + i), organised for the MFMA rate of gfx950:
//  * a workgroup of 8 waves (two per SIMD) owns an item of 256 (row, head)
//    columns of one (sequence, KV head); each 32-token K/V chunk is loaded
//    once per workgroup into LDS (K in two buffers, V in three) and read by
//    all 8 waves, each computing 2 tiles of 16 columns.  K is kept
//    token-major in XOR-swizzled 256 B rows; V token-major in 288 B rows, and
//    each lane reads its PV operand -- 8 tokens of one dim -- with two
//    transposing 8-byte LDS reads (ds_read_b64_tr_b16);
//  * the two waves of a SIMD are staggered: waves 0-3 take chunk n's scores,
//    weights and PV between two barriers, waves 4-7 the weights and PV of
//    chunk n - 1 and then chunk n's scores, so one wave's softmax VALU work
//    meets the other's MFMA work;
//  * the O^T accumulators stay in the accumulation registers: the softmax
//    reference maximum is only moved when a column's maximum grows by more
//    than 2^8 (the rescale is exact; weights up to 256 are fine in bf16/fp32),
//    and that rare rescale runs outside the hot chunk loop;
//  * items are taken from a work counter in order of decreasing sequence
//    length (the plan, built by one extra workgroup of the decode merge launch
//    just before, sorts up to 512 prefill sequences), so the
//    longest items start first.
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "tiles.h"
#include "prefill_plan.h"
#include "decode_segment.h"

namespace pkv {

namespace {
constexpr int kPfWaves = 8;                        // 2 per SIMD
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kPfTiles = 2;                        // 16-column tiles per wave
constexpr int kPfWaveCols = 16 * kPfTiles;         // 64
constexpr int kPfCols = kPfWaveCols * kPfWaves;    // 256 columns per item
static_assert(kPfCols == kPlanItemCols, "the plan counts items of the kernel's width");
constexpr float kRescaleSlack = 8.f;               // log2 units
}  // namespace

// plan (ints): header, then the processing order of the prefill sequences
// [B], their item prefix sums [B + 1], and scan scratch [B + 1].
size_t prefill_plan_bytes(int num_seqs) {
  return ((size_t)(kPlanHeader + 3 * (size_t)num_seqs + 2) * 4 + 255) / 256 * 256;
}

// max(a, b) as one v_max_f32.  The compiler's fmaxf quiets signalling NaNs
// first (an extra v_max x, x per operand) when it cannot see where a value
// came from, e.g. a cross-lane swap; the scores here are never NaN once masked.
__device__ __forceinline__ float raw_max(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Column maxima of two tiles at once.  a and b are each lane's maximum over
// its rows of tile 0 and tile 1; the row-pair swap leaves every lane with two
// values of one tile (which one depends only on the lane's row parity, and
// `tile_of_lane` below says which), the half swap combines the two row pairs
// of that tile.  Result: the column maximum over all 32 tokens of the lane's
// tile, with two cross-lane steps for both tiles.
__device__ __forceinline__ float pair_tile_max(float a, float b) {
  const auto s1 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  const float z = raw_max(__uint_as_float(s1[0]), __uint_as_float(s1[1]));
  const auto s2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(z), __float_as_uint(z), false, false);
  return raw_max(__uint_as_float(s2[0]), __uint_as_float(s2[1]));
}

// The tile (0 or 1) whose maximum pair_tile_max leaves in this lane: the same
// swap applied to the tile numbers themselves.
__device__ __forceinline__ int tile_of_lane() {
  return (int)__builtin_amdgcn_permlane16_swap(0u, 1u, false, false)[0];
}

// The other tile's maximum, from the lane of the neighbouring row: after a
// row-pair swap of r with itself a lane holds its own value and its
// neighbour's, in an order that does not matter (equal values are the same).
__device__ __forceinline__ float other_tile_max(float r) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(r), __float_as_uint(r), false, false);
  return s[0] == __float_as_uint(r) ? __uint_as_float(s[1]) : __uint_as_float(s[0]);
}

// FP8: the pools hold E4M3 bytes; the loader widens them exactly to bf16 on
// their way into LDS (waves 0-3 load K, waves 4-7 V, 16 elements per lane), so
// everything after the LDS tiles is the bf16 path.  k_scale is already in
// scale_log2; v_scale multiplies the output.
// V is token-major like K, rows padded to 288 bytes: the transposing LDS
// reads of the PV operand then hit every bank pair at most twice and their
// per-dim-tile addresses are immediate offsets.
constexpr int kRowK = 256;                         // LDS bytes of one K token row (D 128, bf16)
constexpr int kRowV = 288;                         // LDS bytes of one V token row
typedef uint8_t KBuf[32 * kRowK];                  // one 32-token K chunk
typedef uint8_t VBuf[32 * kRowV];                  // one 32-token V chunk

// A wave-uniform address as an opaque scalar value: a load from it plus a
// 32-bit lane offset then keeps a scalar base, instead of being re-associated
// into per-lane 64-bit address arithmetic around a hoisted lane term.
typedef __attribute__((address_space(1))) const char gchar;
typedef __attribute__((address_space(1))) const u32x4 gu32x4;
__device__ __forceinline__ gchar* uniform_ptr(const char* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<gchar*>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ u32x4 gld16(gchar* p) { return *reinterpret_cast<gu32x4*>(p); }

// One item: the kPfCols (row, head) columns block `local` of prefill
// sequence s (KV head local / blocks-per-head), computed by the workgroup's 8
// waves through the LDS chunk buffers kbuf[2] and vbuf[3].
template <int BS, bool FP8>
__device__ __forceinline__ void prefill_item(const PrefillArgs& a, int s, int local, KBuf* kbuf, VBuf* vbuf) {
  typedef TileBf16<128, BS> Tile;
  constexpr int D = 128, NDT = 8, RB = kRowK, VR = kRowV;
  // wave is read through readfirstlane so the compiler knows every per-wave
  // decision below is uniform: scalar branches, no exec-masked loop exits.
  const int tid = threadIdx.x, wave = uniform(tid >> 6), l = tid & 63, col = l & 15, c = l >> 4;
  const int G = a.group, Hkv = a.num_kv_heads, Hq = a.num_q_heads;
  const int max_tok = a.max_blocks * BS;
  typedef typename std::conditional<FP8, uint8_t, uint16_t>::type Elem;
  const Elem* kc = reinterpret_cast<const Elem*>(a.key_cache);
  const Elem* vc = reinterpret_cast<const Elem*>(a.value_cache);
  const uint16_t* qbase = reinterpret_cast<const uint16_t*>(a.query);
  const int ld_row = tid >> 4, ld_chunk = tid & 15;    // loader: 16 lanes per 256 B row (32 rows)
  static_assert(kPfTiles == 2, "the column maxima pair the two tiles of a wave");
  // A negative scale is folded into the query: flipping the sign bits of q
  // negates every score exactly, so the softmax below always works with a
  // non-negative scale sl2 and a column's largest raw score is its largest
  // scaled one.  inv_sl2 = 1 / sl2 (+inf for scale 0) turns a reference
  // maximum into a threshold on raw scores.
  const bool neg_scale = a.scale_log2 < 0.f;
  const float sl2 = fabsf(a.scale_log2), inv_sl2 = 1.f / sl2;
  const int my_tile = tile_of_lane();

  const int qrow0 = uniform(a.qsl[s]);
  const int q_s = uniform(a.qsl[s + 1]) - qrow0;
  const int per_head = (q_s * G + kPfCols - 1) / kPfCols;
  const int h = local / per_head;
  const int cb = per_head - 1 - (local - h * per_head);   // most rows first
  int L = uniform(a.seq_lens[s]);
  L = L < 0 ? 0 : (L > max_tok ? max_tok : L);
  const int ctx = L - q_s;
  const int f0 = cb * kPfCols, f1 = min(f0 + kPfCols, q_s * G);
  const int p_max = ctx + (f1 - 1) / G;              // last key any column of the item sees
  if (p_max < 0) return;                             // seq_len < rows: nothing is defined
  const int f0w = f0 + wave * kPfWaveCols, f1w = min(f0w + kPfWaveCols, f1);
  const bool has = f0w < f1w;
  const int p_min_w = ctx + f0w / G;
  const int p_max_w = has ? ctx + (f1w - 1) / G : -1;

  typename Tile::Q q[kPfTiles];
  int pos[kPfTiles];
#pragma unroll
  for (int t = 0; t < kPfTiles; ++t) {
    const int f = f0w + 16 * t + col;
    const int row = f / G, head = f - row * G;
    pos[t] = ctx + row;
    Tile::load_q_col(q[t], qbase + ((int64_t)(qrow0 + row) * Hq + h * G + head) * D, f < f1w);
    if (neg_scale)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) q[t].q[kk] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  }

  BlockWindow win;
  win.row = a.block_tables + (int64_t)s * a.max_blocks;
  win.nblk = (L + BS - 1) / BS;
  win.max_id = a.num_blocks - 1;
  win.fill(0);

  // Loader (bf16): piece k of this thread is 16 bytes (8 dims) of row ld_row
  // of the K chunk (k = 0) and of the V chunk (k = 1).  FP8: waves 0-3 load
  // K, waves 4-7 V (row (tid >> 3) & 31, 16 dims).  Two register sets: chunk j travels in set j & 1, so chunks
  // ch + 1 and ch + 2 are in flight while chunk ch is computed.  The loads
  // are unconditional (block ids are
  // clamped to the sequence's blocks, so every address is inside the pool)
  // which keeps the wait before a store at "all but the newest loads";
  // V rows past p_max are zeroed when stored, K rows past it only ever meet
  // masked scores.
  u32x4 S[2][2];
  const bool kthr = wave < kPfWaves / 2;             // FP8 only: this wave loads K
  // A wave's loader rows lie in one of a chunk's two 16-token blocks (bf16:
  // rows 16-31 are waves 4-7; FP8: the waves with (wave & 3) >= 2), so the
  // block base is wave-uniform and each lane adds a constant 32-bit offset:
  // the address arithmetic per chunk is scalar (3 % faster on the 8 x 512-row
  // step than per-lane 64-bit addresses).
  const bool second = BS == 16 && (FP8 ? (wave & 3) >= 2 : wave >= 4);
  const int my_row = FP8 ? ((tid >> 3) & 31) : ld_row;
  const uint32_t lane_off = (uint32_t)(((((BS == 16 ? (my_row & 15) : my_row) * Hkv + h) * D) +
                                        (FP8 ? 16 * (tid & 7) : 8 * ld_chunk)) * (int)sizeof(Elem));
  const int64_t blk_bytes = (int64_t)BS * Hkv * D * (int64_t)sizeof(Elem);
  const char* kpool = reinterpret_cast<const char*>(FP8 && !kthr ? vc : kc);
  const char* vpool = reinterpret_cast<const char*>(vc);
  auto load_chunk = [&](int ch, u32x4* R) {
    const int lb0 = (ch * 32) / BS;                          // uniform
    const int blk = uniform(second ? win.get(lb0 + 1) : win.get(lb0));
    const int64_t boff = (int64_t)blk * blk_bytes;
    R[0] = gld16(uniform_ptr(kpool + boff) + lane_off);
    if constexpr (!FP8) R[1] = gld16(uniform_ptr(vpool + boff) + lane_off);
  };
  auto store_chunk = [&](int ch, int kb, int vb, const u32x4* R) {
    if constexpr (FP8) {
      const int row = (tid >> 3) & 31, p = tid & 7;
      const bool vpast = !kthr && ch * 32 + row > p_max;
      const u32x4 x = vpast ? u32x4{0, 0, 0, 0} : R[0];
      uint32_t d[8];                                 // 16 elements widened to bf16 pairs
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        d[2 * q4] = fp8x2_to_bf16x2(x[q4], false);
        d[2 * q4 + 1] = fp8x2_to_bf16x2(x[q4], true);
      }
      if (kthr) {
        *reinterpret_cast<u32x4*>(&kbuf[kb][row * RB + (((2 * p) ^ (row & 15)) << 4)]) = u32x4{d[0], d[1], d[2], d[3]};
        *reinterpret_cast<u32x4*>(&kbuf[kb][row * RB + (((2 * p + 1) ^ (row & 15)) << 4)]) =
            u32x4{d[4], d[5], d[6], d[7]};
      } else {
        *reinterpret_cast<u32x4*>(&vbuf[vb][row * VR + 32 * p]) = u32x4{d[0], d[1], d[2], d[3]};
        *reinterpret_cast<u32x4*>(&vbuf[vb][row * VR + 32 * p + 16]) = u32x4{d[4], d[5], d[6], d[7]};
      }
    } else {
      *reinterpret_cast<u32x4*>(&kbuf[kb][ld_row * RB + ((ld_chunk ^ (ld_row & 15)) << 4)]) = R[0];
      *reinterpret_cast<u32x4*>(&vbuf[vb][ld_row * VR + 16 * ld_chunk]) =
          ch * 32 + ld_row > p_max ? u32x4{0, 0, 0, 0} : R[1];
    }
  };

  // osum: the softmax denominators, accumulated by the MFMA against an
  // all-ones A tile (every row of it is the column's sum of the bf16 weights
  // that multiply V), so the VALU does no per-element adds.
  // mref: each column's reference maximum (log2 units, scaled); mref_own:
  // that of this lane's own tile (my_tile); thr_own: the raw score above
  // which that column outgrows its reference by more than the slack.
  float mref[kPfTiles];
  float mref_own = -INFINITY, thr_own = -INFINITY;
  f32x4 o[kPfTiles][NDT], osum[kPfTiles];
#pragma unroll
  for (int t = 0; t < kPfTiles; ++t) {
    mref[t] = -INFINITY;
    osum[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < NDT; ++d) o[t][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Phase A of a chunk: scores of all tiles from the shared K tile and the
  // column maximum of this lane's tile.  Off the diagonal the scores stay
  // raw (the scale goes into the exponent's fma); on diagonal chunks they
  // are scaled first and the masked ones set to -inf, so a masked key gets
  // weight 0 whatever the scale (also 0: -inf * 0 would be NaN).
  f32x4 sc[kPfTiles][2];
  auto scores = [&](int b, int ch, auto diag_tag) -> float {
    constexpr bool DIAG = decltype(diag_tag)::value;
    const uint8_t* Kt = kbuf[b];
    u32x4 kop[2][4];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int row = 16 * u + col;
        kop[u][kk] = *reinterpret_cast<const u32x4*>(Kt + row * RB + (((4 * kk + c) ^ (row & 15)) << 4));
      }
    float lmax[kPfTiles];
#pragma unroll
    for (int t = 0; t < kPfTiles; ++t) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        sc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          sc[t][u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kop[u][kk]),
                                                             __builtin_bit_cast(bf16x8, q[t].q[kk]), sc[t][u], 0, 0, 0);
      }
      float cmax = -INFINITY;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (DIAG)
            sc[t][u][r] = (ch * 32 + 16 * u + 4 * c + r <= pos[t]) ? sc[t][u][r] * sl2 : -INFINITY;
          cmax = fmaxf(cmax, sc[t][u][r]);
        }
      lmax[t] = cmax;
    }
    return pair_tile_max(lmax[0], lmax[1]);
  };
  // Phase B: weights against the current reference maxima, then O^T += V^T P^T.
  // Row i of O^T tile dt is dim i + 16 dt; k-slot 4u + r is token 16u + 4c + r,
  // the order in which the S^T accumulator holds P.  The A operand comes
  // from two transposing LDS reads (ds_read_b64_tr_b16): within each
  // 16-lane group, lane i receives element k = element (i & 3) of the
  // 8 bytes read by lane 4k + (i >> 2).  Lane j of group c reads token
  // 16u + 4c + (j >> 2), dims 16 dt + 4 (j & 3) .. + 3, so lane i gets
  // dim 16 dt + i of tokens 16u + 4c .. + 3: k-slots 4u .. 4u + 3.
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  auto accumulate = [&](int b, float mul) {
    const uint8_t* vlane = vbuf[b] + (4 * c + (col >> 2)) * VR + 8 * (col & 3);
    bf16x8 pb[kPfTiles];
    constexpr uint32_t kOnes = 0x3F803F80u;           // two bf16 1.0
#pragma unroll
    for (int t = 0; t < kPfTiles; ++t) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          pb[t][4 * u + r] = (__bf16)fast_exp2(fmaf(sc[t][u][r], mul, -mref[t]));
      osum[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, u32x4{kOnes, kOnes, kOnes, kOnes}),
                                                       pb[t], osum[t], 0, 0, 0);
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                    (lds_v4i16*)(vlane + 32 * dt)));
      const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                                    (lds_v4i16*)(vlane + 16 * VR + 32 * dt)));
      const u32x4 av = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
      for (int t = 0; t < kPfTiles; ++t)
        o[t][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), pb[t], o[t][dt], 0, 0, 0);
    }
  };

  // If a column's maximum m (scaled on the diagonal, raw off it) outgrew
  // its reference by more than the slack (always on the first chunk; a
  // rare, wave-uniform branch) rescale that column's accumulators.  The test
  // is on raw scores against thr_own off the diagonal and on scaled ones
  // against mref_own on it.
  auto rescale_if_needed = [&](float m, bool diag) {
    if (__any(m > (diag ? mref_own + kRescaleSlack : thr_own))) {
      const float m_other = other_tile_max(m);
#pragma unroll
      for (int t = 0; t < kPfTiles; ++t) {
        const float v = t == my_tile ? m : m_other;
        const float cmx = diag ? v : v * sl2;
        const bool nt = diag ? v > mref[t] + kRescaleSlack : v > (mref[t] + kRescaleSlack) * inv_sl2;
        const float alpha = nt ? fast_exp2(mref[t] - cmx) : 1.f;       // 0 on the first chunk
        mref[t] = nt ? cmx : mref[t];
        osum[t] *= alpha;
#pragma unroll
        for (int d = 0; d < NDT; ++d) o[t][d] *= alpha;
      }
      mref_own = my_tile ? mref[1] : mref[0];
      thr_own = (mref_own + kRescaleSlack) * inv_sl2;
    }
  };

  const int nch = (p_max + 32) / 32;
  load_chunk(0, S[0]);
  load_chunk(1, S[1]);
  store_chunk(0, 0, 0, S[0]);
  load_chunk(2, S[0]);
  __syncthreads();
  // Staggered waves.  Both waves of a SIMD (w and w + 4) work between the
  // same two barriers, but in different orders, so that one wave's softmax
  // VALU work runs while the other's products keep the matrix core busy:
  //   waves 0-3, step n:  scores(n) -> weights and PV of n
  //   waves 4-7, step n:  weights and PV of n - 1 -> scores(n)
  // (a lagging wave keeps chunk n's scores in registers across the barrier).
  // Step n reads K chunk n (buffer n & 1) and V chunks n and n - 1 (buffers
  // n % 3 and (n - 1) % 3), stores chunk n + 1 (register set 1 - P, loaded
  // two steps ago) into K buffer 1 - P and V buffer (n + 1) % 3 -- both last
  // read before the previous barrier -- reloads that set with chunk n + 3,
  // then the barrier.  The loop runs one step past the last chunk for the
  // lagging waves' last PV.
  float m_lag = 0.f;                                   // lagging waves: the held chunk's maximum
  bool diag_lag = false;
  int v_prev = 2, v_cur = 0, v_next = 1;               // (n - 1) % 3, n % 3, (n + 1) % 3
  auto step = [&](int n, auto par_tag, auto lag_tag) {
    constexpr int P = decltype(par_tag)::value;
    constexpr bool LAG = decltype(lag_tag)::value;
    const bool have_n = has && n < nch && n * 32 <= p_max_w;
    if constexpr (!LAG) {
      if (have_n) {
        const bool diag = n * 32 + 31 > p_min_w;
        const float m = diag ? scores(P, n, std::true_type{}) : scores(P, n, std::false_type{});
        rescale_if_needed(m, diag);
        accumulate(v_cur, diag ? 1.f : sl2);
      }
    } else {
      if (has && n > 0 && (n - 1) * 32 <= p_max_w) {
        rescale_if_needed(m_lag, diag_lag);
        accumulate(v_prev, diag_lag ? 1.f : sl2);
      }
      if (have_n) {
        diag_lag = n * 32 + 31 > p_min_w;
        m_lag = diag_lag ? scores(P, n, std::true_type{}) : scores(P, n, std::false_type{});
      }
    }
    // Past the last chunk the loads and stores are clamped and unused.
    store_chunk(n + 1, 1 - P, v_next, S[1 - P]);
    load_chunk(n + 3, S[1 - P]);
    v_prev = v_cur;
    v_cur = v_next;
    v_next = v_next == 2 ? 0 : v_next + 1;
    __syncthreads();
  };
  // Even and odd steps alternate in straight-line code, so the compiler's
  // wait counting sees which register set is older and waits only for it.
  // One loop per role (the same barriers in the same number).
  if (wave >= kPfWaves / 2) {
    for (int n = 0; n <= nch; n += 2) {
      step(n, std::integral_constant<int, 0>{}, std::true_type{});
      step(n + 1, std::integral_constant<int, 1>{}, std::true_type{});
    }
  } else {
    for (int n = 0; n <= nch; n += 2) {
      step(n, std::integral_constant<int, 0>{}, std::false_type{});
      step(n + 1, std::integral_constant<int, 1>{}, std::false_type{});
    }
  }

#pragma unroll
  for (int t = 0; t < kPfTiles; ++t) {
    const float tot = osum[t][0];                    // every row holds the column sum
    const int f = f0w + 16 * t + col;
    if (f >= f1w) continue;
    const int row = f / G, head = f - row * G;
    const float inv = a.v_scale / tot;
    float* dst = a.out + ((int64_t)(qrow0 + row) * Hq + h * G + head) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)             // rows 4c..4c+3 of tile dt: dims 16 dt + 4c ..
      st16f(dst + 16 * dt + 4 * c,
            f32x4{o[t][dt][0] * inv, o[t][dt][1] * inv, o[t][dt][2] * inv, o[t][dt][3] * inv});
  }
}

// Last r in [0, n) with cum[r] <= item (cum[0] = 0 <= item).
__device__ __forceinline__ int item_row(const int* cum, int n, int item) {
  int lo = 0, hi = n;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (cum[mid] <= item) lo = mid; else hi = mid;
  }
  return lo;
}

template <int BS, bool FP8>
__global__ void __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(2)))
prefill_lds_kernel(const PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) KBuf kbuf[2];
  __shared__ __attribute__((aligned(16))) VBuf vbuf[3];
  __shared__ int s_item;
  const int B = a.num_seqs;
  const int* plan = a.plan;
  const int total = plan[0], P = plan[1];
  const int* order = plan + kPlanHeader;
  const int* cum = order + B;
  int* counter = a.plan + 2;
  // XCD queues.  Workgroups are dispatched to the 8 XCDs in turn, so
  // workgroup b runs on XCD b % 8, and each XCD has an L2 of its own.  With
  // a KV head count that is a multiple of 8, queue x holds the items of the
  // heads h = x (mod 8) -- per sequence in the plan's order, head by head --
  // so one (sequence, head)'s K/V is streamed through one L2, by the
  // workgroups of that XCD at about the same time.  A workgroup drains its
  // own queue, then takes items from the others in turn (8 equal queues, so
  // only the last items move).  Other head counts take items from the one
  // counter in plan order.
  const int Hkv = a.num_kv_heads;
  const bool xcd_queues = Hkv % kPlanXcdQueues == 0;
  const int x = blockIdx.x % kPlanXcdQueues, per_queue = total / kPlanXcdQueues;
  int drained = 0;                                     // thread 0: queues found empty
  while (true) {
    __syncthreads();                                   // everyone has read the previous item
    if (threadIdx.x == 0) {
      int it = total;
      if (!xcd_queues) {
        it = atomicAdd(counter, 1);
      } else {
        for (; drained < kPlanXcdQueues; ++drained) {
          const int y = (x + drained) % kPlanXcdQueues;
          const int j = atomicAdd(a.plan + 8 + y, 1);
          if (j < per_queue) {
            // Queue position j -> plan item: every sequence contributes
            // items / 8 to each queue (its item count is Hkv x column
            // blocks), so the sequence is the last r with cum[r] <= 8 j.
            const int r = item_row(cum, P, kPlanXcdQueues * j);
            const int c0 = cum[r], per_head = (cum[r + 1] - c0) / Hkv;
            const int lj = j - c0 / kPlanXcdQueues, hi = lj / per_head;
            it = c0 + (y + kPlanXcdQueues * hi) * per_head + (lj - hi * per_head);
            break;
          }
        }
      }
      s_item = it;
    }
    __syncthreads();
    const int item = s_item;
    if (item >= total) break;
    const int r = item_row(cum, P, item);
    prefill_item<BS, FP8>(a, uniform(order[r]), uniform(item - cum[r]), kbuf, vbuf);
  }
}

// ------------------------------------------------------------------ mixed steps
// A varlen step with prefill chunks and decode rows in one launch.  Every
// workgroup first builds the item order in its own LDS (the prefill
// sequences, longest first, then the decode rows by decreasing length), then
// takes items from one counter: all prefill items, then one item per decode
// (sequence, KV head, head tile) pair.  A decode item's chunks are split in
// up to 8 contiguous ranges, one per wave, each attended straight from the
// pools by the decode tiles (decode_segment.h); the workgroup then merges
// the waves' parts from its own slots of the workspace.  The memory-bound
// decode items run on the compute units that the compute-bound prefill items
// leave idle at the end, instead of in launches of their own.  An opt-in
// path: measured on MI355X it is slower than the separate launches (the
// decode code in the same kernel makes the compiler place the prefill's LDS
// reads later, and a decode item pays its own claim, start-up and merge).

// Descending-order key of a decode row's cost: two buckets per octave of
// the row's length (0 for an empty row).
__device__ __forceinline__ int length_bucket(int L) {
  if (L <= 0) return 0;
  const int e = 31 - __clz(L);
  return 1 + 2 * e + (e > 0 ? (L >> (e - 1)) & 1 : 0);   // <= 62
}

constexpr int kMixedBuckets = 64;

// order[0, P): prefill sequences in processing order (longest first, ties
// by sequence index, when P <= kSortMax; else in batch order); cum[0..P]:
// their item prefix sums; order[P, P + Dn): the decode rows, longer buckets
// first and in batch order within a bucket.  Every workgroup builds the same
// order from the same inputs (items are numbered by it), so no step may
// depend on the order of atomic updates.  pseq / plen: scratch of
// kMixedMaxSeqs ints each.  cnt[0] = P, cnt[1] = Dn.  Ends with a barrier.
__device__ void build_mixed_plan(const int32_t* __restrict__ qsl, const int32_t* __restrict__ seq_lens, int B,
                                 int max_tok, int Hkv, int G, int* order, int* cum, int* pseq, int* plen,
                                 int* hist, int* cnt) {
  const int tid = threadIdx.x;
  for (int i = tid; i < kMixedBuckets; i += kPfThreads) hist[i] = 0;
  if (tid < 2) cnt[tid] = 0;
  __syncthreads();
  // counts only: their values do not depend on the order of the updates
  for (int s = tid; s < B; s += kPfThreads) {
    const int q = qsl[s + 1] - qsl[s];
    if (q > 1) atomicAdd(&cnt[0], 1);
    else if (q == 1) atomicAdd(&hist[length_bucket(clamp_len(seq_lens[s], max_tok))], 1);
  }
  __syncthreads();
  const int P = cnt[0];
  if (tid < kWave) {
    // Wave 0: bucket starts (longest bucket first), then one pass over the
    // batch in order, 64 sequences at a time: prefill sequences are
    // compacted into pseq, each decode row goes to its bucket's next place.
    // A lane's rank among the lanes of the same bucket comes from ballots of
    // the bucket's six bits.
    const int lane = tid;
    {
      const int b = kMixedBuckets - 1 - lane;
      const int v = hist[b];
      const int x = wave_inclusive_scan(v);
      hist[b] = P + x - v;
      if (lane == kWave - 1) cnt[1] = x;
    }
    const uint64_t below = (1ull << lane) - 1;
    int np = 0;
    for (int base = 0; base < B; base += kWave) {
      const int s = base + lane;
      int q = 0, L = 0;
      if (s < B) {
        q = qsl[s + 1] - qsl[s];
        L = clamp_len(seq_lens[s], max_tok);
      }
      const uint64_t pm = __ballot(q > 1);
      if (q > 1) {
        pseq[np + __popcll(pm & below)] = s;
        plen[np + __popcll(pm & below)] = L;
      }
      np += __popcll(pm);
      const bool dec = q == 1;
      const int b = dec ? length_bucket(L) : 0;
      uint64_t m = __ballot(dec);
#pragma unroll
      for (int k = 0; k < 6; ++k) {
        const uint64_t bk = __ballot(dec && ((b >> k) & 1));
        m &= ((b >> k) & 1) ? bk : ~bk;
      }
      const int at = dec ? hist[b] : 0;                 // read by every lane of the group before any update
      if (dec) order[at + __popcll(m & below)] = s;
      if (dec && (m >> lane) == 1ull) hist[b] = at + __popcll(m);   // the group's highest lane
    }
  }
  __syncthreads();
  for (int i = tid; i < P; i += kPfThreads) {
    int rank = i;
    if (P <= kSortMax) {                               // longer first, ties by sequence index
      rank = 0;
      for (int j = 0; j < P; ++j) rank += (plen[j] > plen[i]) || (plen[j] == plen[i] && pseq[j] < pseq[i]);
    }
    order[rank] = pseq[i];
  }
  __syncthreads();
  block_prefix_sum<kPfThreads>(P, cum, [&](int r) {
    const int s = order[r];
    return Hkv * (((qsl[s + 1] - qsl[s]) * G + kPlanItemCols - 1) / kPlanItemCols);
  });
  __syncthreads();                                     // (block_prefix_sum has none when P == 0)
}

// One decode item: pair (sequence s, KV head h, head tile ht) of a row whose
// workgroup owns part slots slot0 .. slot0 + 7.
template <class Tile>
__device__ __forceinline__ void decode_item(const DecodeArgs& d, int s, int h, int ht, int64_t slot0) {
  constexpr int D = Tile::D, Q4 = D / 4;
  const int tid = threadIdx.x, wave = uniform(tid >> 6);
  const int L = uniform(clamp_len(d.seq_lens[s], d.max_blocks * Tile::BS));
  const int row = uniform(d.qsl[s]);
  const int cols = min(16, d.group - 16 * ht);
  float* out = d.out + ((int64_t)row * d.num_q_heads + h * d.group + 16 * ht) * D;
  const int n = (L + Tile::CT - 1) / Tile::CT;
  if (n == 0) {                                        // an empty row: zeros, as the decode merge writes
    for (int i = tid; i < cols * Q4; i += kPfThreads) st16f(out + 4 * i, f32x4{0.f, 0.f, 0.f, 0.f});
    return;
  }
  const int k = min(kPfWaves, n);
  if (wave < k)
    run_segment<Tile>(d, s, row, h, ht, L, wave * n / k, (wave + 1) * n / k, k == 1, slot0 + wave, -1, false, 0);
  if (k == 1) return;
  __syncthreads();                                     // every wave's part is written
  for (int i = tid; i < cols * Q4; i += kPfThreads) {
    const int col = i / Q4, d4 = i - col * Q4;
    PartMerge pm;
    pm.add_range<D>(d.part_ml, d.part_o, slot0, d.tile_cols, col, d4, 0, k - 1);
    st16f(out + col * D + 4 * d4, pm.acc * (d.v_scale / pm.Z));
  }
}

template <int BS, bool FP8>
__global__ void __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(2)))
mixed_varlen_kernel(const PrefillArgs a, const DecodeArgs d) {
  typedef typename std::conditional<FP8, TileFp8W<128, BS>, TileBf16<128, BS>>::type DTile;
  __shared__ __attribute__((aligned(16))) KBuf kbuf[2];
  __shared__ __attribute__((aligned(16))) VBuf vbuf[3];
  __shared__ int s_order[kMixedMaxSeqs];
  __shared__ int s_cum[kMixedMaxSeqs + 1];
  __shared__ int s_hist[kMixedBuckets];
  __shared__ int s_cnt[2];
  __shared__ int s_item;
  static_assert(sizeof(vbuf) >= 2 * kMixedMaxSeqs * sizeof(int), "plan scratch lives in the V buffers");
  int* scratch_seq = reinterpret_cast<int*>(&vbuf[0][0]);   // free until the first item
  build_mixed_plan(a.qsl, a.seq_lens, a.num_seqs, a.max_blocks * BS, a.num_kv_heads, a.group, s_order, s_cum,
                   scratch_seq, scratch_seq + kMixedMaxSeqs, s_hist, s_cnt);
  const int P = s_cnt[0], Dn = s_cnt[1];
  const int ptotal = s_cum[P];
  const int ppseq = d.num_kv_heads * d.head_tiles;
  const int total = ptotal + Dn * ppseq;
  int* counter = d.counter;                            // workspace words 0 (items taken) and 1 (workgroups done)
  while (true) {
    __syncthreads();                                   // everyone is done with the previous item (and the plan)
    if (threadIdx.x == 0) s_item = atomicAdd(counter, 1);
    __syncthreads();
    const int item = s_item;
    if (item < 0 || item >= total) break;              // (< 0 only from a workspace that was not zero-filled)
    if (item < ptotal) {
      const int r = item_row(s_cum, P, item);
      prefill_item<BS, FP8>(a, uniform(s_order[r]), uniform(item - s_cum[r]), kbuf, vbuf);
    } else {
      const int di = item - ptotal, r = di / ppseq, pr = di - r * ppseq;
      decode_item<DTile>(d, uniform(s_order[P + r]), pr / d.head_tiles, pr % d.head_tiles,
                         (int64_t)blockIdx.x * kPfWaves);
    }
  }
  // The last workgroup out resets both words for the next call: every
  // other workgroup has taken its last item before it counts itself done.
  if (threadIdx.x == 0 && atomicAdd(counter + 1, 1) == (int)gridDim.x - 1) {
    atomicExch(counter, 0);
    atomicExch(counter + 1, 0);
  }
}

size_t mixed_workspace_bytes(int grid, int tile_cols, int head_dim) {
  const size_t slots = (size_t)grid * kPfWaves;
  return 256 + (slots * tile_cols * 2 * 4 + 255) / 256 * 256 + slots * tile_cols * head_dim * 4;
}

hipError_t launch_mixed_varlen(const PrefillArgs& p, DecodeArgs d, void* workspace, int block_size, bool fp8,
                               int grid, hipStream_t stream) {
  char* w = static_cast<char*>(workspace);
  const size_t slots = (size_t)grid * kPfWaves;
  d.counter = reinterpret_cast<int*>(w);
  d.part_ml = reinterpret_cast<float*>(w + 256);
  d.part_o = reinterpret_cast<float*>(w + 256 + (slots * d.tile_cols * 2 * 4 + 255) / 256 * 256);
  if (block_size == 16 && !fp8)
    hipLaunchKernelGGL((mixed_varlen_kernel<16, false>), dim3(grid), dim3(kPfThreads), 0, stream, p, d);
  else if (block_size == 16)
    hipLaunchKernelGGL((mixed_varlen_kernel<16, true>), dim3(grid), dim3(kPfThreads), 0, stream, p, d);
  else if (!fp8)
    hipLaunchKernelGGL((mixed_varlen_kernel<32, false>), dim3(grid), dim3(kPfThreads), 0, stream, p, d);
  else
    hipLaunchKernelGGL((mixed_varlen_kernel<32, true>), dim3(grid), dim3(kPfThreads), 0, stream, p, d);
  return hipGetLastError();
}

hipError_t launch_prefill_lds(const PrefillArgs& a, int block_size, bool fp8, int cus, hipStream_t stream) {
  const int grid = cus > 0 ? cus : 256;
  if (block_size == 16 && !fp8)
    hipLaunchKernelGGL((prefill_lds_kernel<16, false>), dim3(grid), dim3(kPfThreads), 0, stream, a);
  else if (block_size == 16)
    hipLaunchKernelGGL((prefill_lds_kernel<16, true>), dim3(grid), dim3(kPfThreads), 0, stream, a);
  else if (!fp8)
    hipLaunchKernelGGL((prefill_lds_kernel<32, false>), dim3(grid), dim3(kPfThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((prefill_lds_kernel<32, true>), dim3(grid), dim3(kPfThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
