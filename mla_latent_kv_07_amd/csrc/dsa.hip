// Sparse MLA decode (DeepSeek Sparse Attention): index scores over the cached
// tokens, top-k selection, and a gather of the selected cache rows, after
// which the regular decode path runs over them.
//
// "DeepSeek-V3.2-Exp unboxing", section 初步研读: after the KV cache is
// written, the MLA forward scores the cached tokens with an FP8 index kernel
// (FP8 queries with per-head weights, FP8 keys with a per-token scale) and
// keeps the highest-scoring tokens for the rest of the attention.  Score of
// cached position n for a sequence's new token:
//   o[n] = sum_h w[h] * (q[h] . k[n]) * k_s[n]   (E4M3 values)
// Top-k: the k largest scores, equal scores taken lower position first, the
// kept positions in ascending order.
//
// Kernels
//   index_score_kernel  one thread per cached position: the head-weighted
//                       query (sum_h w[h] q[h], fp32) is formed once per
//                       workgroup in LDS, then one 128-wide FP8 dot product per
//                       key.  HBM-bound (128 + 4 bytes per cached token).
//   topk_kernel         one 1024-thread workgroup per sequence: radix select
//                       of the k-th largest score (4 passes of 8 bits over
//                       order-preserving integer keys), then a stable
//                       compaction in position order.
//   gather_kernel       one wavefront per kept position: its 1152-byte cache
//                       row into a dense run of pages (identity block table).
#include "mla_common.h"

namespace mla {

constexpr int kIdxDim = 128;  // index key / query width

struct IndexArgs {
  const uint8_t* q;        // [B, Hi, 128] E4M3
  const float* w;          // [B, Hi]
  const uint8_t* k;        // [num_blocks, 64, 128] E4M3
  const float* k_scale;    // [num_blocks, 64]
  int bt_stride;
  const int32_t* seq_lens;
  int heads;               // Hi
  int lpad;                // row stride of `scores`
  float* scores;           // [B, lpad]
};

__global__ __launch_bounds__(256) void index_score_kernel(IndexArgs a,
                                                          const int32_t* __restrict__ block_table) {
  __shared__ float qe[kIdxDim];
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  if (tid < kIdxDim) {
    const uint8_t* qb = a.q + (int64_t)b * a.heads * kIdxDim + tid;
    const float* wb = a.w + (int64_t)b * a.heads;
    float acc = 0.f;
    for (int h = 0; h < a.heads; ++h) {
      const float v = __builtin_amdgcn_cvt_f32_fp8((uint32_t)qb[(int64_t)h * kIdxDim], 0);
      acc = fmaf(wb[h], v, acc);
    }
    qe[tid] = acc;
  }
  __syncthreads();
  const int n = blockIdx.x * 256 + tid;
  if (n >= a.seq_lens[b]) return;
  const int64_t slot = (int64_t)block_table[(int64_t)b * a.bt_stride + n / kPage] * kPage + n % kPage;
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* row = reinterpret_cast<const u32x4*>(a.k + slot * kIdxDim);
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < kIdxDim / 16; ++i) {
    const u32x4 v = row[i];
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      typedef float f32x2 __attribute__((ext_vector_type(2)));
      const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(v[wd], false);
      const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(v[wd], true);
      const int d = 16 * i + 4 * wd;
      dot = fmaf(qe[d], lo[0], dot);
      dot = fmaf(qe[d + 1], lo[1], dot);
      dot = fmaf(qe[d + 2], hi[0], dot);
      dot = fmaf(qe[d + 3], hi[1], dot);
    }
  }
  a.scores[(int64_t)b * a.lpad + n] = dot * a.k_scale[slot];
}

// order-preserving integer key of a float (larger score <-> larger key); -0
// and +0 share one key, so they tie like equal numbers
__device__ __forceinline__ uint32_t score_key(float s) {
  const uint32_t u = s == 0.f ? 0u : __float_as_uint(s);
  return (u >> 31) ? ~u : (u | 0x80000000u);
}

constexpr int kTopkThreads = 1024;

// exclusive prefix sum of v over the workgroup's 1024 threads (wave scans,
// then the 16 wave totals); `tot` gets the total
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_sums, int& tot) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wave_sums[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int s = lane < kTopkThreads / 64 ? wave_sums[lane] : 0;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int y = __shfl_up(s, o, 64);
      if (lane >= o) s += y;
    }
    if (lane < kTopkThreads / 64) wave_sums[lane] = s;  // inclusive
  }
  __syncthreads();
  tot = wave_sums[kTopkThreads / 64 - 1];
  const int before = (wave == 0 ? 0 : wave_sums[wave - 1]) + x - v;
  __syncthreads();
  return before;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores,
                                                            int lpad,
                                                            const int32_t* __restrict__ seq_lens,
                                                            int top_k, int32_t* __restrict__ out,
                                                            int32_t* __restrict__ counts) {
  __shared__ int hist[256];
  __shared__ int wave_sums[kTopkThreads / 64];
  __shared__ uint32_t s_prefix, s_mask;
  __shared__ int s_remaining;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int len = seq_lens[b];
  const int kk = min(top_k, len);
  const float* sc = scores + (int64_t)b * lpad;
  if (tid == 0) {
    s_prefix = 0;
    s_mask = 0;
    s_remaining = kk;
  }
  // radix select of the kk-th largest key, 8 bits per pass from the top
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    const uint32_t prefix = s_prefix, mask = s_mask;
    for (int n = tid; n < len; n += kTopkThreads) {
      const uint32_t key = score_key(sc[n]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int cum = 0;
      int rem = s_remaining;
      for (int d = 255; d >= 0; --d) {
        if (cum + hist[d] >= rem) {
          s_prefix = prefix | ((uint32_t)d << shift);
          s_remaining = rem - cum;
          break;
        }
        cum += hist[d];
      }
      s_mask = mask | (255u << shift);
    }
    __syncthreads();
  }
  const uint32_t thr = s_prefix;     // the kk-th largest key
  const int need_eq = s_remaining;   // how many keys equal to it are kept
  // stable compaction: thread t scans positions [t per, (t+1) per)
  const int per = (len + kTopkThreads - 1) / kTopkThreads;
  const int lo = min(tid * per, len);
  const int hi = min(lo + per, len);
  int gt = 0, eq = 0;
  for (int n = lo; n < hi; ++n) {
    const uint32_t key = score_key(sc[n]);
    gt += key > thr;
    eq += key == thr;
  }
  int tot;
  int g = block_exclusive_scan(gt, wave_sums, tot);
  int e = block_exclusive_scan(eq, wave_sums, tot);
  int32_t* ob = out + (int64_t)b * top_k;
  for (int n = lo; n < hi; ++n) {
    const uint32_t key = score_key(sc[n]);
    if (key > thr) {
      ob[g + min(e, need_eq)] = n;
      ++g;
    } else if (key == thr) {
      if (e < need_eq) ob[g + e] = n;
      ++e;
    }
  }
  for (int s = kk + tid; s < top_k; s += kTopkThreads) ob[s] = -1;
  if (tid == 0 && counts) counts[b] = kk;
}

__global__ __launch_bounds__(256) void gather_kernel(const uint16_t* __restrict__ cache,
                                                     const int32_t* __restrict__ block_table,
                                                     int bt_stride,
                                                     const int32_t* __restrict__ kept, int top_k,
                                                     const int32_t* __restrict__ counts, int kpages,
                                                     uint16_t* __restrict__ dense,
                                                     int32_t* __restrict__ dense_bt) {
  const int b = blockIdx.y;
  if (blockIdx.x == 0)
    for (int p = threadIdx.x; p < kpages; p += 256) dense_bt[(int64_t)b * kpages + p] = b * kpages + p;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (j >= counts[b]) return;
  const int p = kept[(int64_t)b * top_k + j];
  const int64_t src_slot =
      (int64_t)block_table[(int64_t)b * bt_stride + p / kPage] * kPage + p % kPage;
  const int64_t dst_slot = ((int64_t)b * kpages + j / kPage) * kPage + j % kPage;
  const u16x8* src = reinterpret_cast<const u16x8*>(cache + src_slot * kEntry);
  u16x8* dst = reinterpret_cast<u16x8*>(dense + dst_slot * kEntry);
  dst[lane] = src[lane];                            // pieces 0 .. 63
  if (lane < kChunk16 - 64) dst[64 + lane] = src[64 + lane];  // pieces 64 .. 71
}

hipError_t launch_index_scores(const uint8_t* index_q, const float* index_w, int index_heads,
                               const uint8_t* index_k, const float* index_k_scale,
                               const int32_t* block_table, int bt_stride, const int32_t* seq_lens,
                               int batch, int max_seq_len, float* scores, int lpad,
                               hipStream_t stream) {
  IndexArgs ia{index_q, index_w, index_k, index_k_scale, bt_stride, seq_lens, index_heads, lpad,
               scores};
  hipLaunchKernelGGL(index_score_kernel, dim3((max_seq_len + 255) / 256, batch), dim3(256), 0,
                     stream, ia, block_table);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int lpad, const int32_t* seq_lens, int batch,
                       int top_k, int32_t* kept, int32_t* counts, hipStream_t stream) {
  hipLaunchKernelGGL(topk_kernel, dim3(batch), dim3(kTopkThreads), 0, stream, scores, lpad,
                     seq_lens, top_k, kept, counts);
  return hipGetLastError();
}

hipError_t launch_gather(const uint16_t* cache, const int32_t* block_table, int bt_stride,
                         const int32_t* kept, int top_k, const int32_t* counts, int batch,
                         int kpages, uint16_t* dense, int32_t* dense_bt, hipStream_t stream) {
  hipLaunchKernelGGL(gather_kernel, dim3((top_k + 3) / 4, batch), dim3(256), 0, stream, cache,
                     block_table, bt_stride, kept, top_k, counts, kpages, dense, dense_bt);
  return hipGetLastError();
}

}  // namespace mla
