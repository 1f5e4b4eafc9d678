// route.hip -- S1 router logits and S2 top-k + renormalisation.
//
// The router runs first and picks each token's experts (dpshk.com article,
// section "核心实现一"); 6 of 256 per token (ai-muninn.com
// "[洋垃圾跑大模型 #3]").  Logits are fp32 in one fixed order so that the
// chosen ids are reproducible bit for bit: 64-wide chunk partials, each a
// chain of fused multiply-adds in ascending h starting from +0, then the
// partials summed in ascending chunk order (the row keeps
// one fixed accumulation order, as dpshk.com "核心实现四" does for its rows).
// Every kernel below computes exactly that order; they differ only in how
// the (token, expert, chunk) work is spread over the GPU.
//
// Selection: order by (logit desc, id asc), keep k in rank order; weights
// sigmoid(logit) renormalised over the chosen k (fp32, device expf).
#include <float.h>

#include "common.h"
#include "kernels.h"

namespace bef {

// One wavefront picks the top-k of E <= 256 logits held in LDS and writes
// ids / weights.  Lane e owns experts e, e+64, e+128, e+192.
__device__ __forceinline__ void topk_wave(const float* __restrict__ z, int E, int k,
                                          int32_t* __restrict__ ids_out,
                                          float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  float v[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    v[i] = (e < E) ? z[e] : -FLT_MAX;
  }
  uint32_t taken = 0;
  float my_z = 0.0f;
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      const bool ok = (e < E) && !((taken >> i) & 1u);
      if (ok && (v[i] > bv || (v[i] == bv && e < bi))) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(bv, m, kWave);
      const int oi = __shfl_xor(bi, m, kWave);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == j) {
      my_z = bv;
      my_id = bi;
    }
  }
  const float sg = (lane < k) ? 1.0f / (1.0f + expf(-my_z)) : 0.0f;
  const float sum = wave_sum(sg);
  if (lane < k) {
    ids_out[lane] = my_id;
    w_out[lane] = sg / sum;
  }
}

// ---------------------------------------------------------------------------
// Small T (decode, T <= kRouteSmallT): block c computes the chunk-c partials
// of every (token, expert) -- thread e reads column e of the router, so a
// block streams 64 rows x E bf16 with coalesced loads -- and the last block
// to finish (arrival counter in the workspace) sums the partials in chunk
// order and runs the top-k.  The counter is returned to zero by that block.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_small_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int H, int E, int k,
    float* __restrict__ part /* [H/64][T][E] */, uint32_t* __restrict__ counter,
    int32_t* __restrict__ ids, float* __restrict__ w) {
  const int c = blockIdx.x;
  const int nc = gridDim.x;
  const int e = threadIdx.x;
  __shared__ float sx[kRouteSmallT][64];
  __shared__ float sz[kRouteSmallT][256];
  __shared__ int s_last;
  for (int i = threadIdx.x; i < T * 64; i += 256)
    sx[i / 64][i % 64] = bf16_to_f32(x[(size_t)(i / 64) * H + 64 * c + (i % 64)]);
  __syncthreads();
  if (e < E) {
    float p[kRouteSmallT];
#pragma unroll
    for (int t = 0; t < kRouteSmallT; ++t) p[t] = 0.0f;
    const uint16_t* col = wr + (size_t)(64 * c) * E + e;
#pragma unroll 8
    for (int h = 0; h < 64; ++h) {
      const float wv = bf16_to_f32(col[(size_t)h * E]);
#pragma unroll
      for (int t = 0; t < kRouteSmallT; ++t)
        if (t < T) p[t] = fmaf(sx[t][h], wv, p[t]);
    }
#pragma unroll
    for (int t = 0; t < kRouteSmallT; ++t)
      if (t < T) part[((size_t)c * T + t) * E + e] = p[t];
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(counter, 1u) == (uint32_t)(nc - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (e < E) {
    // partials of 16 chunks are loaded together, then summed in chunk order
    for (int t = 0; t < T; ++t) {
      float acc = 0.0f;
      for (int c0 = 0; c0 < nc; c0 += 16) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i)
          v[i] = (c0 + i < nc) ? part[((size_t)(c0 + i) * T + t) * E + e] : 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (c0 + i < nc) acc = (c0 + i == 0) ? v[i] : acc + v[i];
      }
      sz[t][e] = acc;
    }
  }
  __syncthreads();
  const int wv = threadIdx.x >> 6;
  if (wv < T) topk_wave(sz[wv], E, k, ids + (size_t)wv * k, w + (size_t)wv * k);
  if (threadIdx.x == 0) *counter = 0u;
}

// ---------------------------------------------------------------------------
// Large T: a block owns 32 tokens x all E (<= 256) experts.  Per 64-wide
// chunk it stages x (as fp32) and the router rows (bf16) in LDS; thread
// (ty, tx) accumulates tokens 4ty..4ty+3 x experts tx + 32j (j < 8), each in
// the fixed order.  The block's logits then go through LDS to 4 waves that
// run the top-k, 8 tokens each.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_tile_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ wr, int T,
                                                         int H, int E, int k,
                                                         int32_t* __restrict__ ids,
                                                         float* __restrict__ w) {
  __shared__ float sx[32][65];
  __shared__ uint16_t sw[64][256];
  __shared__ float sz[32][257];
  const int t0 = blockIdx.x * 32;
  const int tid = threadIdx.x;
  const int ty = tid >> 5, tx = tid & 31;
  float acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
  const int nc = H / 64;
  for (int c = 0; c < nc; ++c) {
    {
      const int row = tid >> 3, col8 = (tid & 7) * 8;
      const int t = t0 + row;
      uint4 r = make_uint4(0, 0, 0, 0);
      if (t < T) r = *reinterpret_cast<const uint4*>(x + (size_t)t * H + 64 * c + col8);
      sx[row][col8 + 0] = bf16_to_f32(r.x & 0xffffu);
      sx[row][col8 + 1] = bf16_to_f32(r.x >> 16);
      sx[row][col8 + 2] = bf16_to_f32(r.y & 0xffffu);
      sx[row][col8 + 3] = bf16_to_f32(r.y >> 16);
      sx[row][col8 + 4] = bf16_to_f32(r.z & 0xffffu);
      sx[row][col8 + 5] = bf16_to_f32(r.z >> 16);
      sx[row][col8 + 6] = bf16_to_f32(r.w & 0xffffu);
      sx[row][col8 + 7] = bf16_to_f32(r.w >> 16);
    }
    if (E == 256) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = tid + 256 * i;  // 16-byte chunk: row q/32, 8 experts (q%32)*8..
        const int h = q >> 5, e8 = (q & 31) * 8;
        *reinterpret_cast<uint4*>(&sw[h][e8]) =
            *reinterpret_cast<const uint4*>(wr + (size_t)(64 * c + h) * 256 + e8);
      }
    } else {
      for (int q = tid; q < 64 * 256; q += 256) {
        const int h = q >> 8, e = q & 255;
        sw[h][e] = (e < E) ? wr[(size_t)(64 * c + h) * E + e] : (uint16_t)0;
      }
    }
    __syncthreads();
    float p[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) p[i][j] = 0.0f;
#pragma unroll 4
    for (int h = 0; h < 64; ++h) {
      float xv[4], wv[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[i] = sx[4 * ty + i][h];
#pragma unroll
      for (int j = 0; j < 8; ++j) wv[j] = bf16_to_f32(sw[h][tx + 32 * j]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) p[i][j] = fmaf(xv[i], wv[j], p[i][j]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = (c == 0) ? p[i][j] : acc[i][j] + p[i][j];
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) sz[4 * ty + i][tx + 32 * j] = acc[i][j];
  __syncthreads();
  const int wv = tid >> 6;
  for (int tt = wv; tt < 32; tt += 4) {
    const int t = t0 + tt;
    if (t < T) topk_wave(sz[tt], E, k, ids + (size_t)t * k, w + (size_t)t * k);
  }
}

hipError_t launch_route(const uint16_t* x, const uint16_t* wr, int T, int H, int E, int k,
                        int32_t* ids, float* w, float* part, uint32_t* counter, hipStream_t st) {
  if (T <= kRouteSmallT) {
    route_small_kernel<<<dim3(H / 64), dim3(256), 0, st>>>(x, wr, T, H, E, k, part, counter, ids,
                                                           w);
  } else {
    route_tile_kernel<<<dim3((T + 31) / 32), dim3(256), 0, st>>>(x, wr, T, H, E, k, ids, w);
  }
  return hipGetLastError();
}

}  // namespace bef
