// Device-side split planner for the split-KV decode (run by the last
// workgroup of the query-absorption launch, see qabsorb.hip).
//
// Each sequence's pages are cut into contiguous work items so that all
// workgroups of one decode launch finish at about the same time.  The
// sequence lengths live on the device, so the plan is made on the device by a
// single workgroup, with no host round trip.  An item's partial result (fp32
// output rows and their log-sum-exp) is merged afterwards by the combine
// kernel; the merge is the split form of the softmax in the MLA forward pass
// (the decode-context-parallel excerpt on the "DeepSeek" tag page describes
// the same merge across GPUs).
//
// Cost model for a candidate item size c (in pages):
//   items(c) = sum_b ceil(pages_b / c)
//   big(c)   = max_b ceil(pages_b / ceil(pages_b / c))  (largest actual item)
//   time(c)  = min(ceil(items/slots) * big(c), total/slots + big(c))
//              + cost * items/slots
// where `slots` is the number of workgroups that run at once and `cost` the
// price, in pages, of one item's fixed work: its set-up and the writing and
// merging of its partial rows.
//
// Everything is wave-parallel (shuffle reductions and scans); no thread walks
// a long dependent chain through LDS.
#pragma once
#include "mla_common.h"

namespace mla {

constexpr int kPlanThreads = 256;
constexpr int kPlanWaves = kPlanThreads / 64;
constexpr int kPlanShared = 8192;  // sequences whose page counts are kept in LDS
constexpr int kCandidates = 24;
constexpr int kPlanSmemBytes = 4 * (kPlanShared + kPlanWaves + kCandidates + 1);

// Pages of a sequence, clamped to the host-side bound so that a length beyond
// the documented contract can never make the plan overflow its arrays.
__device__ __forceinline__ int clamp_pages(int len, int max_pages) {
  const int p = (len + kPage - 1) / kPage;
  return p < 1 ? 1 : (p > max_pages ? max_pages : p);
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// candidate k: 1..8 pages, then a ladder growing by about a third (the last
// entry is replaced by max_pages)
__device__ __forceinline__ int candidate(int k, int max_pages) {
  constexpr int kLadder[kCandidates] = {1,  2,  3,  4,  5,  6,  7,   8,   10,  13,  18,  24,
                                        32, 42, 56, 72, 96, 128, 168, 224, 296, 392, 512, 0};
  int c = k == kCandidates - 1 ? max_pages : kLadder[k];
  return c > max_pages ? max_pages : (c < 1 ? 1 : c);
}

struct PlanArgs {
  const int32_t* seq_lens;
  int batch, max_pages, slots, max_items, splits_hint;
  float item_cost;
  PlanView plan;
};

// The whole plan, run by one workgroup of kPlanThreads threads; `smem` holds
// kPlanSmemBytes of LDS.
__device__ void plan_block(const PlanArgs& pa, MLA_LDS char* smem) {
  const int32_t* seq_lens = pa.seq_lens;
  const int batch = pa.batch, max_pages = pa.max_pages, slots = pa.slots;
  const int max_items = pa.max_items, splits_hint = pa.splits_hint;
  const float item_cost = pa.item_cost;
  const PlanView& plan = pa.plan;
  MLA_LDS int* sh_pages = reinterpret_cast<MLA_LDS int*>(smem);
  MLA_LDS int* sh_wave = sh_pages + kPlanShared;
  MLA_LDS float* sh_cost = reinterpret_cast<MLA_LDS float*>(sh_wave + kPlanWaves);
  MLA_LDS int* sh_chosen_p = reinterpret_cast<MLA_LDS int*>(sh_cost + kCandidates);
  const int t = threadIdx.x;
  const int wave = t >> 6;
  const int lane = t & 63;
  auto pages = [&](int b) {
    return b < kPlanShared ? sh_pages[b] : clamp_pages(seq_lens[b], max_pages);
  };

  int local = 0;
  for (int b = t; b < batch; b += kPlanThreads) {
    const int p = clamp_pages(seq_lens[b], max_pages);
    if (b < kPlanShared) sh_pages[b] = p;
    local += p;
  }
  local = wave_sum(local);
  if (lane == 0) sh_wave[wave] = local;
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int w = 0; w < kPlanWaves; ++w) total += sh_wave[w];

  if (splits_hint <= 0) {
    // each wave scores kCandidates / kPlanWaves candidate sizes; their
    // per-lane sums come first and the cross-lane reductions run side by side
    // (one chain of shuffle latencies instead of one per candidate)
    constexpr int kPerWave = kCandidates / kPlanWaves;
    static_assert(kCandidates % kPlanWaves == 0, "candidates split evenly over the waves");
    int items[kPerWave], big[kPerWave];
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      items[i] = 0;
      big[i] = 0;
    }
    for (int b = lane; b < batch; b += 64) {
      const int p = pages(b);
#pragma unroll
      for (int i = 0; i < kPerWave; ++i) {
        const int c = candidate(wave + i * kPlanWaves, max_pages);
        const int n = (p + c - 1) / c;
        items[i] += n;
        big[i] = max(big[i], (p + n - 1) / n);
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
#pragma unroll
      for (int i = 0; i < kPerWave; ++i) {
        items[i] += __shfl_xor(items[i], o, 64);
        big[i] = max(big[i], __shfl_xor(big[i], o, 64));
      }
    if (lane < kPerWave) {
      // lane i publishes candidate wave + i*kPlanWaves
      int it = items[0], bg = big[0];
#pragma unroll
      for (int i = 1; i < kPerWave; ++i) {
        it = lane == i ? items[i] : it;
        bg = lane == i ? big[i] : bg;
      }
      float cost = 3.0e38f;
      if (it <= max_items) {
        const float rounds = (float)((it + slots - 1) / slots);
        const float t1 = rounds * (float)bg;
        const float t2 = (float)total / (float)slots + (float)bg;
        cost = fminf(t1, t2) + item_cost * (float)it / (float)slots;
      }
      sh_cost[wave + lane * kPlanWaves] = cost;
    }
    __syncthreads();
    if (wave == 0) {
      // arg-min over candidates, ties to the larger item size (lane = candidate)
      float best = lane < kCandidates ? sh_cost[lane] : 3.0e38f;
      int bk = lane;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) {
        const float ob = __shfl_xor(best, o, 64);
        const int ok = __shfl_xor(bk, o, 64);
        if (ob < best || (ob == best && ok > bk)) {
          best = ob;
          bk = ok;
        }
      }
      if (lane == 0) *sh_chosen_p = candidate(bk, max_pages);
    }
    __syncthreads();
  }
  const int chosen = splits_hint > 0 ? max_pages : *sh_chosen_p;
  auto split_chunk = [&](int p) {
    int splits = splits_hint > 0 ? min(splits_hint, p) : (p + chosen - 1) / chosen;
    splits = splits < 1 ? 1 : splits;
    return (p + splits - 1) / splits;
  };

  // items per thread over a contiguous range of sequences, then a block scan
  const int per = (batch + kPlanThreads - 1) / kPlanThreads;
  const int b0 = min(t * per, batch);
  const int b1 = min(b0 + per, batch);
  int mine = 0;
  for (int b = b0; b < b1; ++b) {
    const int p = pages(b);
    const int ch = split_chunk(p);
    mine += (p + ch - 1) / ch;
  }
  int incl = mine;  // inclusive scan within the wave
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  __syncthreads();
  if (lane == 63) sh_wave[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += sh_wave[w];
  if (t == kPlanThreads - 1) plan.header[0] = before + incl;
  int next = before + incl - mine;
  for (int b = b0; b < b1; ++b) {
    const int p = pages(b);
    const int ch = split_chunk(p);
    const int n = (p + ch - 1) / ch;
    plan.seq_start[b] = next;
    plan.seq_count[b] = n;
    for (int s = 0; s < n; ++s) {
      plan.item_b[next + s] = b;
      plan.item_p0[next + s] = s * ch;
      plan.item_p1[next + s] = min((s + 1) * ch, p);
    }
    next += n;
  }
}

}  // namespace mla
