// actq.h -- S3, activation quantisation to E4M3 with one fp32 scale per 128
// (tcti.cn post, section "补齐软件栈缺失": act_quant feeds the FP8/FP4
// linears), as a device routine: the act_quant kernel runs it, and so do the
// router launches that quantise x in the same launch.
//
// Thread gt of the flattened range quantises elements 8 gt .. 8 gt + 7 of x
// (16 lanes per 128-block, the block max reduced across them): s = amax/448
// by IEEE division, q = E4M3(x / s), an all-zero block gives s = 0, q = 0.
// Lanes past nblocks*16 take part in the reduction with zeros and store
// nothing.  Called with all 64 lanes of a wave (the 16-lane reduction).
#pragma once
#include "common.h"

namespace bef {

template <bool BF16>
__device__ __forceinline__ void act_quant_lanes(const void* __restrict__ x, int64_t nblocks,
                                                uint8_t* __restrict__ q, float* __restrict__ s,
                                                int64_t gt) {
  const int64_t blk = gt >> 4;
  const bool valid = blk < nblocks;
  float v[8];
  if (valid) {
    if (BF16) {
      const uint4 r = reinterpret_cast<const uint4*>(x)[gt];
      v[0] = bf16_to_f32(r.x & 0xffffu);
      v[1] = bf16_to_f32(r.x >> 16);
      v[2] = bf16_to_f32(r.y & 0xffffu);
      v[3] = bf16_to_f32(r.y >> 16);
      v[4] = bf16_to_f32(r.z & 0xffffu);
      v[5] = bf16_to_f32(r.z >> 16);
      v[6] = bf16_to_f32(r.w & 0xffffu);
      v[7] = bf16_to_f32(r.w >> 16);
    } else {
      const float4 a = reinterpret_cast<const float4*>(x)[2 * gt];
      const float4 b = reinterpret_cast<const float4*>(x)[2 * gt + 1];
      v[0] = a.x, v[1] = a.y, v[2] = a.z, v[3] = a.w;
      v[4] = b.x, v[5] = b.y, v[6] = b.z, v[7] = b.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
  amax = group_max<16>(amax);
  const float sc = amax / 448.0f;
  uint32_t lo = 0, hi = 0;
  if (amax != 0.0f) {
    lo = e4m3_pack4(v[0] / sc, v[1] / sc, v[2] / sc, v[3] / sc);
    hi = e4m3_pack4(v[4] / sc, v[5] / sc, v[6] / sc, v[7] / sc);
  }
  if (valid) {
    reinterpret_cast<uint2*>(q)[gt] = make_uint2(lo, hi);
    if ((gt & 15) == 0) s[blk] = sc;
  }
}

}  // namespace bef
