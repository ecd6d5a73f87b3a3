// The item plan of the workgroup-shared prefill kernel: which prefill
// sequences exist, in which order their items are taken (longest first), the
// items' prefix sums, and the work counter the kernel's workgroups take items
// from.  Built by one workgroup of 256 threads before the prefill kernel runs
// (the decode merge kernel of the same call carries that workgroup).
#pragma once

#include "common.h"

namespace pkv {

constexpr int kPlanItemCols = 256;                 // (row, head) columns per prefill item
constexpr int kPlanHeader = 16;                    // ints: [0] items, [1] prefill seqs, [2] counter,
                                                   // [8 + x] the counter of XCD x's queue
constexpr int kPlanXcdQueues = 8;
constexpr int kSortMax = 512;                      // prefill sequences the plan sorts by length

// Exclusive scan of f(i), i in [0, n), writing out(i, prefix) for i in [0, n]
// (out(n, total)); LDS use is independent of n.  Ends with a barrier.
template <typename F, typename O>
__device__ inline int block_scan_to(int n, F f, O out) {
  __shared__ int wave_tot[256 / kWave];
  const int tid = threadIdx.x, wid = tid / kWave;
  int carry = 0;
  for (int base = 0; base < n; base += 256) {
    const int i = base + tid;
    const int v = i < n ? f(i) : 0;
    int x = wave_inclusive_scan(v);
    if (lane_id() == kWave - 1) wave_tot[wid] = x;
    __syncthreads();
    int off = carry;
    for (int w = 0; w < wid; ++w) off += wave_tot[w];
    if (i < n) out(i, x + off - v);
    int tot = 0;
    for (int w = 0; w < 256 / kWave; ++w) tot += wave_tot[w];
    carry += tot;
    __syncthreads();
  }
  if (tid == 0) out(n, carry);
  __syncthreads();
  return carry;
}

__device__ inline void build_prefill_plan(const int32_t* __restrict__ qsl, const int32_t* __restrict__ seq_lens,
                                          int B, int max_tok, int Hkv, int G, int* __restrict__ plan) {
  __shared__ int s_len[kSortMax];
  __shared__ int s_seq[kSortMax];
  int* order = plan + kPlanHeader;
  int* cum = order + B;
  int* pre = cum + B + 1;                              // scratch: prefix of "is prefill"
  auto is_prefill = [&](int s) { return qsl[s + 1] - qsl[s] > 1 ? 1 : 0; };
  const int P = block_scan_to(B, is_prefill, [&](int i, int v) { pre[i] = v; });
  auto len = [&](int s) {
    const int L = seq_lens[s];
    return L < 0 ? 0 : (L > max_tok ? max_tok : L);
  };
  if (P <= kSortMax) {
    for (int s = threadIdx.x; s < B; s += 256)
      if (pre[s + 1] != pre[s]) {
        s_seq[pre[s]] = s;
        s_len[pre[s]] = len(s);
      }
    __syncthreads();
    // rank: longer first, ties by sequence index
    for (int i = threadIdx.x; i < P; i += 256) {
      int rank = 0;
      for (int j = 0; j < P; ++j)
        rank += (s_len[j] > s_len[i]) || (s_len[j] == s_len[i] && j < i);
      order[rank] = s_seq[i];
    }
  } else {
    for (int s = threadIdx.x; s < B; s += 256)
      if (pre[s + 1] != pre[s]) order[pre[s]] = s;
  }
  __syncthreads();
  auto items = [&](int r) {
    const int s = order[r];
    const int q = qsl[s + 1] - qsl[s];
    return Hkv * ((q * G + kPlanItemCols - 1) / kPlanItemCols);
  };
  const int total = block_scan_to(P, items, [&](int i, int v) { cum[i] = v; });
  if (threadIdx.x == 0) {
    plan[0] = total;
    plan[1] = P;
    plan[2] = 0;                                       // work counter
    for (int x = 0; x < kPlanXcdQueues; ++x) plan[8 + x] = 0;
  }
}


}  // namespace pkv
