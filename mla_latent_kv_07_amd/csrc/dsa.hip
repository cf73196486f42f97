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
//   index_score_kernel  the head-weighted query (sum_h w[h] q[h], fp32) is
//                       formed once per workgroup of 512 positions, then one
//                       128-wide FP8 dot product per key, 8 lanes per key row.
//                       HBM-bound (128 + 4 bytes read, 4 written per position).
//   topk_kernel         one 1024-thread workgroup per sequence, the scores in
//                       registers (up to 16384 positions; longer sequences
//                       re-read them): radix select of the k-th largest score
//                       (4 passes of 8 bits over order-preserving integer
//                       keys), then a stable compaction in position order.
//   gather_kernel       8 kept rows per wavefront: their cache rows (1152-byte
//                       bf16 or 656-byte FP8 rows) into a dense run of pages
//                       (identity block table).
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
  int max_len;             // host-side bound on seq_lens (lengths are clamped to it)
};

constexpr int kIdxRowsPerWG = 512;  // cached positions per index-score workgroup

// E4M3 byte -> fp32
__device__ __forceinline__ float e4m3(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8(byte, 0);
}

// Index scores.  256 threads = 4 wavefronts; a wavefront reads 8 key rows
// (1 KB, one load per lane: 16 bytes of one row) per load instruction, each
// lane keeps its 16 dimensions of the weighted query in registers, and the
// 8 lanes of a row add their partial dot products with 3 cross-lane steps.
// Each wavefront takes whole 64-row pages, one per loop iteration: one scalar
// block-table lookup, then the page's 8 row groups and scales in flight.
__global__ __launch_bounds__(256) void index_score_kernel(IndexArgs a,
                                                          const int32_t* __restrict__ block_table) {
  __shared__ float part[2][kIdxDim];
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  // (a length beyond the documented bound is clamped: no score row, block
  // table row or kept list is ever addressed past its size)
  const int len = min(a.seq_lens[b], a.max_len);
  const int n0 = blockIdx.x * kIdxRowsPerWG;
  if (n0 >= len) return;  // uniform over the workgroup
  {
    // weighted query: thread (d = tid % 128, half = tid / 128) sums the heads
    // h = half, half + 2, ...; 32 heads' loads are issued together per round
    const int d = tid & (kIdxDim - 1), half = tid >> 7;
    const uint8_t* qb = a.q + (int64_t)b * a.heads * kIdxDim + d;
    const float* wb = a.w + (int64_t)b * a.heads;
    float acc = 0.f;
    for (int h0 = half; h0 < a.heads; h0 += 64) {
      uint32_t qv[32];
      float wv[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int h = h0 + 2 * i;
        qv[i] = h < a.heads ? qb[(int64_t)h * kIdxDim] : 0u;
        wv[i] = h < a.heads ? wb[h] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) acc = fmaf(wv[i], e4m3(qv[i]), acc);
    }
    part[half][d] = acc;
  }
  __syncthreads();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keep it scalar
  const int p = lane & 7;     // this lane's 16 dimensions: 16p .. 16p + 15
  const int rl = lane >> 3;   // this lane's row within an 8-row group
  float qe[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) qe[e] = part[0][16 * p + e] + part[1][16 * p + e];
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const int32_t* bt = block_table + (int64_t)b * a.bt_stride;
  const int wrow0 = n0 + wave * (kIdxRowsPerWG / 4);
  constexpr int kGroups = kIdxRowsPerWG / 4 / 8;  // 8-row groups per wavefront
  constexpr int kUnroll = kPage / 8;  // one page per iteration
  static_assert(kIdxRowsPerWG / 4 % kPage == 0, "a wavefront's rows are whole pages");
#pragma unroll 1
  for (int g0 = 0; g0 < kGroups; g0 += kUnroll) {
    const int page_row = wrow0 + g0 * 8;  // uniform, a multiple of 64
    if (page_row >= len) break;
    const int64_t base = (int64_t)bt[page_row / kPage] * kPage;  // scalar load
    u32x4 v[kUnroll];
    float ks[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      // the key rows and their scales are all requested before any is used
      const int r = page_row + u * 8 + rl;
      const int64_t slot = base + u * 8 + rl;
      v[u] = r < len ? *reinterpret_cast<const u32x4*>(a.k + slot * kIdxDim + 16 * p)
                     : u32x4{0u, 0u, 0u, 0u};
      ks[u] = r < len ? a.k_scale[slot] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float dot = 0.f;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(v[u][wd], false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(v[u][wd], true);
        dot = fmaf(qe[4 * wd], lo[0], dot);
        dot = fmaf(qe[4 * wd + 1], lo[1], dot);
        dot = fmaf(qe[4 * wd + 2], hi[0], dot);
        dot = fmaf(qe[4 * wd + 3], hi[1], dot);
      }
      dot += __shfl_xor(dot, 1, 64);
      dot += __shfl_xor(dot, 2, 64);
      dot += __shfl_xor(dot, 4, 64);
      const int r = wrow0 + (g0 + u) * 8 + rl;
      if (p == 0 && r < len) a.scores[(int64_t)b * a.lpad + r] = dot * ks[u];
    }
  }
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

constexpr int kTopkRegs = 16;  // positions per thread held in registers (len <= 16384)

// One radix-select digit: which 8-bit digit (at `shift`) the rem-th largest
// key among those matching `prefix` under `mask` has, and how many keys with
// that digit are still needed.  Histogram in LDS, then wavefront 0 finds the
// digit: lane l owns bins 4l .. 4l + 3, a suffix sum over the lanes finds the
// lane, the lane walks its four bins.
template <bool REGS>
__device__ __forceinline__ void select_digit(const float* sc, int lo, int cnt,
                                             const uint32_t (&key)[REGS ? kTopkRegs : 1],
                                             int shift, uint32_t& prefix, uint32_t mask, int& rem,
                                             int* hist, uint32_t* s_prefix, int* s_rem) {
  const int tid = threadIdx.x;
  if (tid < 256) hist[tid] = 0;
  __syncthreads();
  if constexpr (REGS) {
#pragma unroll
    for (int i = 0; i < kTopkRegs; ++i)
      if (i < cnt && (key[i] & mask) == prefix) atomicAdd(&hist[(key[i] >> shift) & 255], 1);
  } else {
    for (int i = 0; i < cnt; ++i) {
      const uint32_t k = score_key(sc[lo + i]);
      if ((k & mask) == prefix) atomicAdd(&hist[(k >> shift) & 255], 1);
    }
  }
  __syncthreads();
  if (tid < 64) {
    const int lane = tid;
    const int c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2],
              c3 = hist[4 * lane + 3];
    const int own = c0 + c1 + c2 + c3;
    int x = own;  // becomes the count of keys in bins >= 4 lane
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_down(x, o, 64);
      if (lane + o < 64) x += y;
    }
    // x is non-increasing in the lane: the lanes with x >= rem form a prefix
    const uint64_t ok = __ballot(x >= rem);
    const int ls = 63 - __clzll((long long)ok);
    if (lane == ls) {
      int above = x - own;  // keys in the bins above this lane's four
      int d;
      if (above + c3 >= rem) {
        d = 3;
      } else if (above + c3 + c2 >= rem) {
        d = 2;
        above += c3;
      } else if (above + c3 + c2 + c1 >= rem) {
        d = 1;
        above += c3 + c2;
      } else {
        d = 0;
        above += c3 + c2 + c1;
      }
      *s_prefix = prefix | ((uint32_t)(4 * ls + d) << shift);
      *s_rem = rem - above;
    }
  }
  __syncthreads();
  prefix = *s_prefix;
  rem = *s_rem;
}

template <bool REGS>
__device__ __forceinline__ void topk_body(const float* sc, int len, int kk, int32_t* ob,
                                          int* hist, int* wave_sums, uint32_t* s_prefix,
                                          int* s_rem, const int32_t* btb, int32_t* sl) {
  const int tid = threadIdx.x;
  // a kept position at its rank, and (sl != nullptr: the decode reads the kept
  // rows in place) its cache row index at the same rank
  auto put = [&](int rank, int pos) {
    ob[rank] = pos;
    if (sl) sl[rank] = btb[pos / kPage] * kPage + pos % kPage;
  };
  // thread t owns the contiguous positions [lo, lo + cnt)
  const int per = (len + kTopkThreads - 1) / kTopkThreads;
  const int lo = min(tid * per, len);
  const int cnt = min(per, len - lo);
  uint32_t key[REGS ? kTopkRegs : 1];
  if constexpr (REGS) {
#pragma unroll
    for (int i = 0; i < kTopkRegs; ++i) key[i] = i < cnt ? score_key(sc[lo + i]) : 0u;
  } else {
    key[0] = 0u;
  }
  uint32_t prefix = 0, mask = 0;
  int rem = kk;
  for (int shift = 24; shift >= 0; shift -= 8) {
    select_digit<REGS>(sc, lo, cnt, key, shift, prefix, mask, rem, hist, s_prefix, s_rem);
    mask |= 255u << shift;
  }
  const uint32_t thr = prefix;  // the kk-th largest key
  const int need_eq = rem;      // keys equal to it that are kept (lowest positions)
  int gt = 0, eq = 0;
  if constexpr (REGS) {
#pragma unroll
    for (int i = 0; i < kTopkRegs; ++i) {
      gt += (i < cnt && key[i] > thr) ? 1 : 0;
      eq += (i < cnt && key[i] == thr) ? 1 : 0;
    }
  } else {
    for (int i = 0; i < cnt; ++i) {
      const uint32_t k = score_key(sc[lo + i]);
      gt += k > thr ? 1 : 0;
      eq += k == thr ? 1 : 0;
    }
  }
  int tot;
  int g = block_exclusive_scan(gt, wave_sums, tot);
  int e = block_exclusive_scan(eq, wave_sums, tot);
  // each kept position at its rank: the kept positions before it are the
  // larger keys before it and the first need_eq equal keys
  if constexpr (REGS) {
#pragma unroll
    for (int i = 0; i < kTopkRegs; ++i) {
      if (i < cnt) {
        const uint32_t k = key[i];
        if (k > thr) {
          put(g + min(e, need_eq), lo + i);
          ++g;
        } else if (k == thr) {
          if (e < need_eq) put(g + e, lo + i);
          ++e;
        }
      }
    }
  } else {
    for (int i = 0; i < cnt; ++i) {
      const uint32_t k = score_key(sc[lo + i]);
      if (k > thr) {
        put(g + min(e, need_eq), lo + i);
        ++g;
      } else if (k == thr) {
        if (e < need_eq) put(g + e, lo + i);
        ++e;
      }
    }
  }
}

// Top-k of one sequence per 1024-thread workgroup: radix select of the k-th
// largest key (four 8-bit digits from the top), then a stable compaction in
// position order (the keys above it, and the lowest-positioned keys equal to
// it, each at its rank among the kept positions).
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(const float* __restrict__ scores,
                                                            int lpad,
                                                            const int32_t* __restrict__ seq_lens,
                                                            int max_len, int top_k,
                                                            int32_t* __restrict__ out,
                                                            int32_t* __restrict__ counts,
                                                            const int32_t* __restrict__ block_table,
                                                            int bt_stride,
                                                            int32_t* __restrict__ slots,
                                                            int slot_stride) {
  __shared__ int hist[256];
  __shared__ int wave_sums[kTopkThreads / 64];
  __shared__ uint32_t s_prefix;
  __shared__ int s_rem;
  const int b = blockIdx.x;
  const int tid = threadIdx.x;
  const int len = min(seq_lens[b], max_len);  // clamped as in the index scores
  const int kk = min(top_k, len);
  const float* sc = scores + (int64_t)b * lpad;
  int32_t* ob = out + (int64_t)b * top_k;
  const int32_t* btb = slots ? block_table + (int64_t)b * bt_stride : nullptr;
  int32_t* sl = slots ? slots + (int64_t)b * slot_stride : nullptr;
  if (kk > 0) {  // uniform
    if (len <= kTopkThreads * kTopkRegs)
      topk_body<true>(sc, len, kk, ob, hist, wave_sums, &s_prefix, &s_rem, btb, sl);
    else
      topk_body<false>(sc, len, kk, ob, hist, wave_sums, &s_prefix, &s_rem, btb, sl);
  }
  for (int s = kk + tid; s < top_k; s += kTopkThreads) ob[s] = -1;
  if (tid == 0 && counts) counts[b] = kk;
}

constexpr int kGatherRows = 8;  // kept rows per wavefront

// Gather: each wavefront copies kGatherRows kept rows of ROW bytes (consecutive
// kept ranks, so consecutive dense rows); lanes 0 .. 7 look up the rows' cache
// slots, every lane then issues all of its 16-byte loads before its stores.
// ROW: 1152 (bf16 rows) or 656 (FP8 rows).
template <int ROW>
__global__ __launch_bounds__(256) void gather_kernel(const char* __restrict__ cache,
                                                     const int32_t* __restrict__ block_table,
                                                     int bt_stride,
                                                     const int32_t* __restrict__ kept, int top_k,
                                                     const int32_t* __restrict__ counts, int kpages,
                                                     char* __restrict__ dense,
                                                     int32_t* __restrict__ dense_bt) {
  constexpr int kPieces = ROW / 16;                         // 16-byte pieces per row
  constexpr int kLoads = (kGatherRows * kPieces + 63) / 64;  // per lane
  static_assert(ROW % 16 == 0, "rows of whole 16-byte pieces");
  const int b = blockIdx.y;
  if (blockIdx.x == 0)
    for (int p = threadIdx.x; p < kpages; p += 256) dense_bt[(int64_t)b * kpages + p] = b * kpages + p;
  const int lane = threadIdx.x & 63;
  const int j0 = (blockIdx.x * 4 + (threadIdx.x >> 6)) * kGatherRows;  // first kept rank
  const int n = counts[b];
  if (j0 >= n) return;  // uniform over the wavefront
  int64_t my_slot = 0;
  if (lane < kGatherRows && j0 + lane < n) {
    const int p = kept[(int64_t)b * top_k + j0 + lane];
    my_slot = (int64_t)block_table[(int64_t)b * bt_stride + p / kPage] * kPage + p % kPage;
  }
  // dense rows of sequence b are contiguous: rank j sits at row b * kpages * 64 + j
  u16x8* dst = reinterpret_cast<u16x8*>(dense + ((int64_t)b * kpages * kPage + j0) * ROW);
  u16x8 v[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int q = i * 64 + lane;  // piece of the wavefront's rows
    const int r = q / kPieces;
    const int64_t slot = __shfl(my_slot, r < kGatherRows ? r : 0, 64);
    if (q < kGatherRows * kPieces && j0 + r < n)
      v[i] = reinterpret_cast<const u16x8*>(cache + slot * ROW)[q - r * kPieces];
  }
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int q = i * 64 + lane;
    if (q < kGatherRows * kPieces && j0 + q / kPieces < n) dst[q] = v[i];
  }
}

hipError_t launch_index_scores(const uint8_t* index_q, const float* index_w, int index_heads,
                               const uint8_t* index_k, const float* index_k_scale,
                               const int32_t* block_table, int bt_stride, const int32_t* seq_lens,
                               int batch, int max_seq_len, float* scores, int lpad,
                               hipStream_t stream) {
  IndexArgs ia{index_q, index_w, index_k, index_k_scale, bt_stride, seq_lens, index_heads, lpad,
               scores, max_seq_len};
  hipLaunchKernelGGL(index_score_kernel,
                     dim3((max_seq_len + kIdxRowsPerWG - 1) / kIdxRowsPerWG, batch), dim3(256), 0,
                     stream, ia, block_table);
  return hipGetLastError();
}

hipError_t launch_topk(const float* scores, int lpad, const int32_t* seq_lens, int max_seq_len,
                       int batch, int top_k, int32_t* kept, int32_t* counts, hipStream_t stream,
                       const int32_t* block_table, int bt_stride, int32_t* slots,
                       int slot_stride) {
  hipLaunchKernelGGL(topk_kernel, dim3(batch), dim3(kTopkThreads), 0, stream, scores, lpad,
                     seq_lens, max_seq_len, top_k, kept, counts, block_table, bt_stride, slots,
                     slot_stride);
  return hipGetLastError();
}

hipError_t launch_gather(bool fp8, const void* cache, const int32_t* block_table, int bt_stride,
                         const int32_t* kept, int top_k, const int32_t* counts, int batch,
                         int kpages, void* dense, int32_t* dense_bt, hipStream_t stream) {
  const dim3 grid((top_k + 4 * kGatherRows - 1) / (4 * kGatherRows), batch);
  if (fp8)
    hipLaunchKernelGGL(gather_kernel<kFp8EntryBytes>, grid, dim3(256), 0, stream,
                       static_cast<const char*>(cache), block_table, bt_stride, kept, top_k, counts,
                       kpages, static_cast<char*>(dense), dense_bt);
  else
    hipLaunchKernelGGL(gather_kernel<kEntryBytes>, grid, dim3(256), 0, stream,
                       static_cast<const char*>(cache), block_table, bt_stride, kept, top_k, counts,
                       kpages, static_cast<char*>(dense), dense_bt);
  return hipGetLastError();
}


}  // namespace mla
