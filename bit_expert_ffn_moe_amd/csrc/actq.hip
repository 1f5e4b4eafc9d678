// actq.hip -- S3, activation quantisation to E4M3 with one fp32 scale per 128
// (tcti.cn post, section "补齐软件栈缺失": act_quant feeds the FP8/FP4
// linears; dpshk.com article, section "核心实现四": one quantised input
// serves gate and up).
//
// HBM-bound elementwise work: one 128-block per 16 lanes, 8 consecutive
// elements per lane (16 B of bf16 or 32 B of f32 in, 8 B of codes out), the
// block max reduced across the 16 lanes by cross-lane steps (actq.h).  No
// LDS.
#include "actq.h"
#include "common.h"
#include "kernels.h"

namespace bef {

template <bool BF16>
__global__ __launch_bounds__(256) void act_quant_kernel(const void* __restrict__ x,
                                                        int64_t nblocks, uint8_t* __restrict__ q,
                                                        float* __restrict__ s) {
  act_quant_lanes<BF16>(x, nblocks, q, s, (int64_t)blockIdx.x * 256 + threadIdx.x);
}

hipError_t launch_act_quant(const void* x, bool bf16, int64_t rows, int32_t cols, uint8_t* q,
                            float* s, hipStream_t st) {
  const int64_t nblocks = rows * (cols / 128);
  const int64_t threads = nblocks * 16;
  const int64_t grid = (threads + 255) / 256;
  if (bf16)
    act_quant_kernel<true><<<dim3((unsigned)grid), dim3(256), 0, st>>>(x, nblocks, q, s);
  else
    act_quant_kernel<false><<<dim3((unsigned)grid), dim3(256), 0, st>>>(x, nblocks, q, s);
  return hipGetLastError();
}

}  // namespace bef
