// Work list of packed (jagged) launches, built on the device by every workgroup from the
// document offsets: no extra kernel, no memory, nothing the host must know about the lengths,
// so a captured graph stays valid when they change (FLAMIA reading notes, section 6,
// Algorithm 2: items of at most 256 queries per document (here one 128-token block), cost =
// the item's visible 64-token tile count, items sorted across the packed row by decreasing
// cost; the backward's key tiles ordered by cost with the heads grouped for L2).
//
// A launch has one workgroup per (rank, head) with the heads inner: blockIdx.x = rank * H + h.
// Rank r takes the r-th item in decreasing cost (ties: by document, then block), so the
// dispatcher starts the longest items first and the short ones fill the tail; workgroups go
// round-robin to the 8 XCDs, so with H a divisor of 8 each XCD keeps to a fixed set of heads
// and the items of one (document, head) share its L2. Ranks past the item count exit.
#pragma once
#include <hip/hip_runtime.h>

#include "mx_layout.h"

namespace mx {

constexpr int kPlanBlock = 128;          // tokens per item along its own axis
constexpr int kPlanTile = 64;            // tokens per cost unit along the other axis
constexpr int kPlanMaxBins = 1024;       // cost bins: max_seqlen <= 64 * (kPlanMaxBins - 1)
constexpr int kPlanMaxDocs = 1 << 16;

// What an item is and how much it costs.
//   kQueryItems: the item is a block of queries; cost = the key tiles it visits (causal: keys
//                up to the block's last query; otherwise all of the document's keys).
//   kKeyItems:   the item is a block of keys; cost = the 64-query steps that visit it (causal:
//                the queries from the block's first key on; otherwise all of them).
enum PlanKind { kQueryItems = 0, kKeyItems = 1 };

struct PlanItem {
  int doc, blk;
  bool valid;
};

// True when a packed launch uses the work list (the host sizes the grid accordingly).
__host__ __device__ inline bool plan_eligible(const Geom& g, const Geom& gk) {
  const int m = g.max_seqlen > gk.max_seqlen ? g.max_seqlen : gk.max_seqlen;
  return packed(g) && g.n_docs <= kPlanMaxDocs && m <= kPlanTile * (kPlanMaxBins - 1);
}

// Upper bound of the item count: sum over documents of ceil(n_j / 128) <= T / 128 + n_docs.
__host__ inline long long plan_items_bound(const Geom& g_items) {
  return g_items.total / kPlanBlock + g_items.n_docs;
}

// (clamped to the bins, should a document be longer than the call's stated max_seqlen)
__device__ __forceinline__ int plan_cost(PlanKind kind, bool causal, int nq, int nk, int b) {
  int c;
  if (kind == kQueryItems) {
    const int keys = causal ? min(nk, kPlanBlock * (b + 1)) : nk;
    c = (keys + kPlanTile - 1) / kPlanTile;
  } else {
    const int queries = causal ? nq - kPlanBlock * b : nq;
    c = (queries + kPlanTile - 1) / kPlanTile;
  }
  return min(max(c, 0), kPlanMaxBins - 1);
}

// Exclusive prefix sum of one value per thread over the workgroup (wave scans by lane shuffles,
// then the wave totals); wsum: kThreads / 64 ints of shared memory.
template <int kThreads>
__device__ __forceinline__ int block_exclusive_scan(int v, int* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; w++) base += wsum[w];
  __syncthreads();
  return base + x - v;
}

// The item of `rank`. kThreads: the workgroup size; smem: at least kPlanMaxBins + kThreads / 64 + 4
// ints of shared memory that nothing else uses during the call. Every thread of the workgroup
// must call it (it synchronises the workgroup) and gets the same result.
template <int kThreads>
__device__ PlanItem plan_item(const Geom& g, const Geom& gk, PlanKind kind, bool causal, int rank, int* smem) {
  int* hist = smem;                        // [kPlanMaxBins] items per cost
  int* part = smem + kPlanMaxBins;         // [kThreads / 64] wave totals of the scans
  int* pick = part + kThreads / 64;        // [4] cost, index within the cost, document, block
  const int tid = threadIdx.x;
  const int nd = g.n_docs;
  auto nq_of = [&](int j) { return g.cu[j + 1] - g.cu[j]; };
  auto nk_of = [&](int j) { return gk.cu[j + 1] - gk.cu[j]; };
  auto nitems = [&](int j) { return (kind == kQueryItems ? nq_of(j) : nk_of(j)) + kPlanBlock - 1; };
  for (int i = tid; i < kPlanMaxBins; i += kThreads) hist[i] = 0;
  if (tid < 4) pick[tid] = -1;
  __syncthreads();
  // 1. histogram of the item costs
  for (int j = tid; j < nd; j += kThreads) {
    const int nq = nq_of(j), nk = nk_of(j), nb = nitems(j) / kPlanBlock;
    for (int b = 0; b < nb; b++) atomicAdd(&hist[plan_cost(kind, causal, nq, nk, b)], 1);
  }
  __syncthreads();
  // 2. ranks start at the highest cost: start(c) = sum of hist over costs above c. Thread t
  //    scans bins [t * per, (t + 1) * per) from the top; a workgroup scan joins the pieces.
  constexpr int per = (kPlanMaxBins + kThreads - 1) / kThreads;
  int loc = 0;
  for (int i = 0; i < per; i++) {
    const int c = kPlanMaxBins - 1 - (tid * per + i);
    if (c >= 0) loc += hist[c];
  }
  {
    int start = block_exclusive_scan<kThreads>(loc, part);
    for (int i = 0; i < per; i++) {
      const int c = kPlanMaxBins - 1 - (tid * per + i);
      if (c < 0) break;
      const int h = hist[c];
      if (h > 0 && rank >= start && rank < start + h) {
        pick[0] = c;
        pick[1] = rank - start;
      }
      start += h;
    }
  }
  __syncthreads();
  const int cstar = pick[0], istar = pick[1];
  if (cstar < 0) return PlanItem{0, 0, false};      // rank past the item count (uniform)
  // 3. the istar-th item of cost cstar in (document, block) order: per-thread counts over a
  //    contiguous range of documents, a scan, and the thread whose range holds it finds it.
  const int dper = (nd + kThreads - 1) / kThreads;
  const int j0 = tid * dper, j1 = min(nd, j0 + dper);
  int cnt = 0;
  for (int j = j0; j < j1; j++) {
    const int nq = nq_of(j), nk = nk_of(j), nb = nitems(j) / kPlanBlock;
    for (int b = 0; b < nb; b++) cnt += plan_cost(kind, causal, nq, nk, b) == cstar;
  }
  int left = istar - block_exclusive_scan<kThreads>(cnt, part);
  if (left >= 0 && left < cnt) {
    for (int j = j0; j < j1 && left >= 0; j++) {
      const int nq = nq_of(j), nk = nk_of(j), nb = nitems(j) / kPlanBlock;
      for (int b = 0; b < nb; b++) {
        if (plan_cost(kind, causal, nq, nk, b) != cstar) continue;
        if (left == 0) {
          pick[2] = j;
          pick[3] = b;
        }
        left--;
      }
    }
  }
  __syncthreads();
  const PlanItem it{pick[2], pick[3], pick[2] >= 0};
  __syncthreads();                         // the shared memory is free again for the caller
  return it;
}

}  // namespace mx
