// Cache insert kernels (bf16 and FP8 rows): one wavefront per new token, the
// work of insert_dev.h.  Bound by launch latency (1152 bytes in and out per
// token).
#include "insert_dev.h"

namespace mla {

__global__ __launch_bounds__(64) void insert_kernel(InsertArgs a) {
  const int pos = token_pos(a, blockIdx.x);
  double c, s;
  rope_angle(pos, a.freq[threadIdx.x & 31], c, s);
  insert_token_bf16(a, blockIdx.x, threadIdx.x, pos, c, s);
}

__global__ __launch_bounds__(64) void insert_fp8_kernel(InsertArgs a) {
  const int pos = token_pos(a, blockIdx.x);
  double c, s;
  rope_angle(pos, a.freq[threadIdx.x & 31], c, s);
  insert_token_fp8(a, blockIdx.x, threadIdx.x, pos, c, s);
}

hipError_t launch_insert(const uint16_t* kv_a, const uint16_t* rms_w, float eps, float rope_base,
                         const int32_t* block_table, int bt_stride, const int32_t* seq_lens,
                         int batch, int q_len, uint16_t* cache, hipStream_t stream) {
  const InsertArgs a = with_rope_freq(InsertArgs{kv_a, rms_w, (double)eps, (double)rope_base,
                                                  block_table, bt_stride, seq_lens, q_len, cache});
  hipLaunchKernelGGL(insert_kernel, dim3(batch * q_len), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_insert_fp8(const uint16_t* kv_a, const uint16_t* rms_w, float eps,
                             float rope_base, const int32_t* block_table, int bt_stride,
                             const int32_t* seq_lens, int batch, int q_len, uint8_t* cache,
                             hipStream_t stream) {
  const InsertArgs a = with_rope_freq(InsertArgs{kv_a, rms_w, (double)eps, (double)rope_base,
                                                  block_table, bt_stride, seq_lens, q_len, cache});
  hipLaunchKernelGGL(insert_fp8_kernel, dim3(batch * q_len), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace mla
