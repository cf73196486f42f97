// Device-side split planner for the split-KV decode.
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
//   time(c)  = min(ceil(items/slots) * c, total/slots + c) + cost * items/slots
// where `slots` is the number of workgroups that run at once and `cost` the
// price, in pages, of writing and merging one item's partial rows.
#include "mla_common.h"

namespace mla {

constexpr int kPlanThreads = 256;
constexpr int kPlanShared = 8192;  // sequences whose page counts fit in LDS

// Pages of a sequence, clamped to the host-side bound so that a length beyond
// the documented contract can never make the plan overflow its arrays.
__device__ __forceinline__ int clamp_pages(int len, int max_pages) {
  const int p = (len + kPage - 1) / kPage;
  return p < 1 ? 1 : (p > max_pages ? max_pages : p);
}
__device__ __forceinline__ int pages_of(const int32_t* seq_lens, const int* sh, int b,
                                        int max_pages) {
  return b < kPlanShared ? sh[b] : clamp_pages(seq_lens[b], max_pages);
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(
    const int32_t* __restrict__ seq_lens, int batch, int max_pages, int slots, int max_items,
    int splits_hint, float item_cost, PlanView plan) {
  __shared__ int sh_pages[kPlanShared];
  __shared__ float sh_cost[kPlanThreads];
  __shared__ int sh_c[kPlanThreads];
  __shared__ int sh_sum[kPlanThreads];
  __shared__ int sh_total;
  const int t = threadIdx.x;
  int local = 0;
  for (int b = t; b < batch; b += kPlanThreads) {
    const int p = clamp_pages(seq_lens[b], max_pages);
    if (b < kPlanShared) sh_pages[b] = p;
    local += p;
  }
  sh_sum[t] = local;
  __syncthreads();
  if (t == 0) {
    int s = 0;
    for (int k = 0; k < kPlanThreads; ++k) s += sh_sum[k];
    sh_total = s;
  }
  __syncthreads();
  const float total = (float)sh_total;

  int chosen = max_pages;
  if (splits_hint <= 0) {
    // candidate item sizes: 1..32, then a geometric ladder, capped at max_pages
    int c = t < 32 ? t + 1 : (int)(32.0f * __builtin_powf(1.08f, (float)(t - 32)));
    c = c > max_pages ? max_pages : c;
    c = c < 1 ? 1 : c;
    long items = 0;
    for (int b = 0; b < batch; ++b) items += (pages_of(seq_lens, sh_pages, b, max_pages) + c - 1) / c;
    float cost;
    if (items > max_items) {
      cost = 3.0e38f;
    } else {
      const float rounds = (float)((items + slots - 1) / slots);
      const float t1 = rounds * (float)c;
      const float t2 = total / (float)slots + (float)c;
      cost = (t1 < t2 ? t1 : t2) + item_cost * (float)items / (float)slots;
    }
    sh_cost[t] = cost;
    sh_c[t] = c;
    __syncthreads();
    if (t == 0) {
      float best = 3.5e38f;
      int bc = max_pages;
      for (int k = 0; k < kPlanThreads; ++k) {
        if (sh_cost[k] < best || (sh_cost[k] == best && sh_c[k] > bc)) {
          best = sh_cost[k];
          bc = sh_c[k];
        }
      }
      sh_c[0] = bc;
    }
    __syncthreads();
    chosen = sh_c[0];
    __syncthreads();
  }

  // per-sequence split count; each thread owns a contiguous range of sequences
  const int per = (batch + kPlanThreads - 1) / kPlanThreads;
  const int b0 = t * per;
  const int b1 = (b0 + per < batch) ? b0 + per : batch;
  int my_items = 0;
  for (int b = b0; b < b1; ++b) {
    const int p = pages_of(seq_lens, sh_pages, b, max_pages);
    int splits = splits_hint > 0 ? (splits_hint < p ? splits_hint : p) : (p + chosen - 1) / chosen;
    splits = splits < 1 ? 1 : splits;
    const int chunk = (p + splits - 1) / splits;
    my_items += (p + chunk - 1) / chunk;
  }
  sh_sum[t] = my_items;
  __syncthreads();
  if (t == 0) {
    int s = 0;
    for (int k = 0; k < kPlanThreads; ++k) {
      const int v = sh_sum[k];
      sh_sum[k] = s;
      s += v;
    }
    plan.header[0] = s;
  }
  __syncthreads();
  int next = sh_sum[t];
  for (int b = b0; b < b1; ++b) {
    const int p = pages_of(seq_lens, sh_pages, b, max_pages);
    int splits = splits_hint > 0 ? (splits_hint < p ? splits_hint : p) : (p + chosen - 1) / chosen;
    splits = splits < 1 ? 1 : splits;
    const int chunk = (p + splits - 1) / splits;
    const int n = (p + chunk - 1) / chunk;
    plan.seq_start[b] = next;
    plan.seq_count[b] = n;
    for (int s = 0; s < n; ++s) {
      plan.item_b[next + s] = b;
      plan.item_p0[next + s] = s * chunk;
      plan.item_p1[next + s] = (s + 1) * chunk < p ? (s + 1) * chunk : p;
    }
    next += n;
  }
}

hipError_t launch_plan(const int32_t* seq_lens, int batch, int max_pages, int slots,
                       int max_items, int splits_hint, float item_cost_pages, PlanView plan,
                       hipStream_t stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, seq_lens, batch,
                     max_pages, slots, max_items, splits_hint, item_cost_pages, plan);
  return hipGetLastError();
}

}  // namespace mla
