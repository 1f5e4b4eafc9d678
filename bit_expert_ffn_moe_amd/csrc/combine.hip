// combine.hip -- S7: out[t] = y[shared row] + sum_j w[t][j] * y[row_of[t][j]].
//
// The shared expert is added with weight 1 and the routed experts with their
// renormalised gate weights, after the down projection (tcti.cn post,
// section "DeepSeek-V4-Flash的可能性": the shared expert sits beside the
// routed ones).  fp32 in the order shared, slot 0, ..., slot k-1, then bf16
// (nearest even) or fp32.  HBM-bound: 16-byte loads/stores, one thread per 4
// consecutive outputs.
#include "common.h"
#include "kernels.h"

namespace bef {

template <bool BF16OUT>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ topk_w, int T,
                                                      int k, int H, void* __restrict__ out) {
  const int t = blockIdx.x;  // tokens in x: more than 65535 of them are valid
  const int m4 = blockIdx.y * 256 + threadIdx.x;
  if (4 * m4 >= H) return;
  const int32_t* ro = row_of + (size_t)t * (k + 1);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  const int rs = ro[k];
  if (rs >= 0) acc = reinterpret_cast<const float4*>(y + (size_t)rs * H)[m4];
  for (int j = 0; j < k; ++j) {
    const int r = ro[j];
    if (r < 0) continue;
    const float wj = topk_w[(size_t)t * k + j];
    const float4 v = reinterpret_cast<const float4*>(y + (size_t)r * H)[m4];
    acc.x = fmaf(wj, v.x, acc.x);
    acc.y = fmaf(wj, v.y, acc.y);
    acc.z = fmaf(wj, v.z, acc.z);
    acc.w = fmaf(wj, v.w, acc.w);
  }
  if (BF16OUT) {
    uint2 o;
    o.x = (uint32_t)f32_to_bf16(acc.x) | ((uint32_t)f32_to_bf16(acc.y) << 16);
    o.y = (uint32_t)f32_to_bf16(acc.z) | ((uint32_t)f32_to_bf16(acc.w) << 16);
    reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + (size_t)t * H)[m4] = o;
  } else {
    reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + (size_t)t * H)[m4] = acc;
  }
}

hipError_t launch_combine(const float* y, const int32_t* row_of, const float* topk_w, int T, int k,
                          int H, void* out, bool bf16, hipStream_t st) {
  const dim3 grid(T, (H / 4 + 255) / 256);
  if (bf16)
    combine_kernel<true><<<grid, 256, 0, st>>>(y, row_of, topk_w, T, k, H, out);
  else
    combine_kernel<false><<<grid, 256, 0, st>>>(y, row_of, topk_w, T, k, H, out);
  return hipGetLastError();
}

}  // namespace bef
