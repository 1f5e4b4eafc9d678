// gemv.hip -- S5/S6 for one token: fused low-bit GEMV on the VALU.
//
// Decode moves every byte of its experts' weights for one token, so it is
// HBM-bound (tcti.cn post, section "DeepSeek-V4-Flash的可能性": decode is
// memory-bound and needs its own operators; smzdm.com roundup: MoE saves
// compute, not bandwidth).  FP4 weights stay FP4 in HBM and are unpacked in
// registers inside the dot product (dpshk.com article, section "核心实现四";
// tcti.cn post, section "硬件的骨头怎么啃": FP4 stays FP4 and is unpacked on
// the device).  On gfx950 that is one v_cvt_scalef32_pk_f16_fp4 per two
// weights and one v_dot2_f32_f16 per two products; the UE8M0 scale is an
// exact ldexp per 32 weights, the activation scale one multiply per 32.
//
// Layout per wave: lane l owns 32-element chunk l (+64i) of every row it
// touches, so each 16-byte load of a weight row is exactly one UE8M0 scale
// block, and a wave reads a 1 KiB contiguous stretch per load instruction.
// Each wave issues the loads of all its rows before any arithmetic, to keep
// many bytes in flight per CU.
#include "common.h"
#include "kernels.h"

namespace bef {

// Loads two 16-byte halves of a 32-code E4M3 chunk and converts to fp16.
__device__ __forceinline__ void load_act32(const uint8_t* __restrict__ p, Act16& a0, Act16& a1) {
  const uint4 q0 = *reinterpret_cast<const uint4*>(p);
  const uint4 q1 = *reinterpret_cast<const uint4*>(p + 16);
  e4m3x16_to_h2(q0, a0);
  e4m3x16_to_h2(q1, a1);
}

// ---------------------------------------------------------------------------
// gate + up + SwiGLU.  grid = (I / (4*RPW), active group slots); the slot's
// group is found from offsets (no host round trip).  Wave w of block b owns
// weight rows n = (4b + w)*RPW .. +RPW-1 of gate and up of that group, for
// every row (token) of the group.  h = silu(g) * u is written fp32 to
// h[row][n].
// ---------------------------------------------------------------------------
template <int NB, int RPW>
__global__ __launch_bounds__(256) void gemv_gate_up_fp4_kernel(
    const uint8_t* __restrict__ gq, const uint8_t* __restrict__ gs,
    const uint8_t* __restrict__ uq, const uint8_t* __restrict__ us,
    const uint8_t* __restrict__ xq, const float* __restrict__ xs,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ row_token, int E, int H,
    int I, float* __restrict__ h) {
  __shared__ int stmp[8];
  int unused;
  const int g = find_group_item(
      offsets, E + 1, blockIdx.y, [](int c) { return c > 0 ? 1 : 0; }, stmp, &unused);
  if (g < 0) return;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n0 = (blockIdx.x * 4 + wv) * RPW;
  const int nch = H >> 5;
  const size_t rowq = (size_t)(H >> 1), rows_ = (size_t)nch;

  uint4 wg[RPW][NB], wu[RPW][NB];
  uint32_t sg[RPW][NB], su[RPW][NB];
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    const size_t row = (size_t)g * I + n0 + i;
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      const int ch = lane + 64 * c;
      if (ch < nch) {
        wg[i][c] = *reinterpret_cast<const uint4*>(gq + row * rowq + 16 * ch);
        wu[i][c] = *reinterpret_cast<const uint4*>(uq + row * rowq + 16 * ch);
        sg[i][c] = gs[row * rows_ + ch];
        su[i][c] = us[row * rows_ + ch];
      } else {
        wg[i][c] = wu[i][c] = make_uint4(0, 0, 0, 0);
        sg[i][c] = su[i][c] = 127;
      }
    }
  }
  const int r_end = offsets[g + 1];
  for (int r = offsets[g]; r < r_end; ++r) {
    const int t = row_token[r];
    Act16 a0[NB], a1[NB];
    float xsc[NB];
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      const int ch = lane + 64 * c;
      if (ch < nch) {
        load_act32(xq + (size_t)t * H + 32 * ch, a0[c], a1[c]);
        xsc[c] = xs[(size_t)t * (H >> 7) + (ch >> 2)];
      } else {
        xsc[c] = 0.0f;
        e4m3x16_to_h2(make_uint4(0, 0, 0, 0), a0[c]);
        e4m3x16_to_h2(make_uint4(0, 0, 0, 0), a1[c]);
      }
    }
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      float ag = 0.0f, au = 0.0f;
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        ag += scale_ue8m0(dot32_fp4(wg[i][c], a0[c], a1[c]), sg[i][c]) * xsc[c];
        au += scale_ue8m0(dot32_fp4(wu[i][c], a0[c], a1[c]), su[i][c]) * xsc[c];
      }
      ag = wave_sum(ag);
      au = wave_sum(au);
      if (lane == 0) h[(size_t)r * I + n0 + i] = silu_mul_accurate(ag, au);
    }
  }
}

// ---------------------------------------------------------------------------
// down (+ combine for a single token).  Every block first requantises all R
// (<= RMAX) rows of h to E4M3 per 128 into LDS (the same rule as act_quant;
// block 0 also stores the codes/scales to the workspace for inspection).
// Wave w of block b owns output rows m = (4b + w)*RPW .. +RPW-1; for each
// row r (expert e_r) it loads W_down[e_r][m] (one 16-byte chunk per lane for
// I = 2048), issuing every load before any arithmetic.  COMBINE writes
// out[m] = y[shared] + sum_j w_j y[row_of[j]] (T = 1); otherwise y_rows.
// ---------------------------------------------------------------------------
template <int NB, int RMAX, int RPW, bool COMBINE>
__global__ __launch_bounds__(256) void gemv_down_fp4_kernel(
    const uint8_t* __restrict__ dq, const uint8_t* __restrict__ ds, const float* __restrict__ h,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ row_of,
    const float* __restrict__ topk_w, int E, int H, int I, int k, float* __restrict__ y_rows,
    void* __restrict__ out, int out_bf16, uint8_t* __restrict__ hq_ws,
    float* __restrict__ hs_ws) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_rowexp[RMAX];
  const int R = offsets[E + 1];
  uint8_t* s_hq = smem;                                            // [R][I]
  float* s_hs = reinterpret_cast<float*>(smem + (size_t)RMAX * I);  // [R][I/128]
  const int tid = threadIdx.x;
  // row -> expert
  for (int g = tid; g <= E; g += 256) {
    const int a = offsets[g], b = offsets[g + 1];
    for (int r = a; r < b && r < RMAX; ++r) s_rowexp[r] = g;
  }
  // requantise h: 16 lanes per 128-block, 8 elements per lane
  const int nq = R * (I >> 3);
  for (int idx = tid; idx < ((nq + 255) & ~255); idx += 256) {
    const bool ok = idx < nq;
    float v[8];
    if (ok) {
      const float4 p0 = reinterpret_cast<const float4*>(h)[2 * idx];
      const float4 p1 = reinterpret_cast<const float4*>(h)[2 * idx + 1];
      v[0] = p0.x, v[1] = p0.y, v[2] = p0.z, v[3] = p0.w;
      v[4] = p1.x, v[5] = p1.y, v[6] = p1.z, v[7] = p1.w;
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
    if (ok) {
      reinterpret_cast<uint2*>(s_hq)[idx] = make_uint2(lo, hi);
      if ((idx & 15) == 0) s_hs[idx >> 4] = sc;
      if (blockIdx.x == 0) {
        reinterpret_cast<uint2*>(hq_ws)[idx] = make_uint2(lo, hi);
        if ((idx & 15) == 0) hs_ws[idx >> 4] = sc;
      }
    }
  }
  __syncthreads();

  const int lane = tid & 63, wv = tid >> 6;
  const int m0 = (blockIdx.x * 4 + wv) * RPW;
  const int nch = I >> 5;
  const size_t rowq = (size_t)(I >> 1), rows_ = (size_t)nch;
  uint4 w[RMAX][RPW][NB];
  uint32_t sb[RMAX][RPW][NB];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    if (r < R) {
      const int e = s_rowexp[r];
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const size_t row = (size_t)e * H + m0 + i;
#pragma unroll
        for (int c = 0; c < NB; ++c) {
          const int ch = lane + 64 * c;
          if (ch < nch) {
            w[r][i][c] = *reinterpret_cast<const uint4*>(dq + row * rowq + 16 * ch);
            sb[r][i][c] = ds[row * rows_ + ch];
          } else {
            w[r][i][c] = make_uint4(0, 0, 0, 0);
            sb[r][i][c] = 127;
          }
        }
      }
    }
  }
  float y[RMAX][RPW];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
#pragma unroll
    for (int i = 0; i < RPW; ++i) y[r][i] = 0.0f;
    if (r < R) {
      Act16 a0[NB], a1[NB];
      float hsc[NB];
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nch) {
          const uint4 q0 = *reinterpret_cast<const uint4*>(s_hq + (size_t)r * I + 32 * ch);
          const uint4 q1 = *reinterpret_cast<const uint4*>(s_hq + (size_t)r * I + 32 * ch + 16);
          e4m3x16_to_h2(q0, a0[c]);
          e4m3x16_to_h2(q1, a1[c]);
          hsc[c] = s_hs[r * (I >> 7) + (ch >> 2)];
        } else {
          e4m3x16_to_h2(make_uint4(0, 0, 0, 0), a0[c]);
          e4m3x16_to_h2(make_uint4(0, 0, 0, 0), a1[c]);
          hsc[c] = 0.0f;
        }
      }
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < NB; ++c)
          acc += scale_ue8m0(dot32_fp4(w[r][i][c], a0[c], a1[c]), sb[r][i][c]) * hsc[c];
        y[r][i] = wave_sum(acc);
      }
    }
  }
  if (COMBINE) {
    if (lane < RPW) {
      // lane i writes output row m0 + i (T = 1: token 0)
      float yi[RMAX];
#pragma unroll
      for (int r = 0; r < RMAX; ++r) {
        float v = y[r][0];
#pragma unroll
        for (int i = 1; i < RPW; ++i) v = (lane == i) ? y[r][i] : v;
        yi[r] = v;
      }
      auto pick = [&](int rr) {
        float v = 0.0f;
#pragma unroll
        for (int r = 0; r < RMAX; ++r) v = (r == rr) ? yi[r] : v;
        return v;
      };
      const int rs = row_of[k];
      float o = (rs >= 0) ? pick(rs) : 0.0f;
      for (int j = 0; j < k; ++j) {
        const int rj = row_of[j];
        if (rj >= 0) o = fmaf(topk_w[j], pick(rj), o);
      }
      const int m = m0 + lane;
      if (out_bf16)
        reinterpret_cast<uint16_t*>(out)[m] = f32_to_bf16(o);
      else
        reinterpret_cast<float*>(out)[m] = o;
    }
  } else {
    if (lane < RPW) {
#pragma unroll
      for (int r = 0; r < RMAX; ++r) {
        if (r < R) {
          float v = y[r][0];
#pragma unroll
          for (int i = 1; i < RPW; ++i) v = (lane == i) ? y[r][i] : v;
          y_rows[(size_t)r * H + m0 + lane] = v;
        }
      }
    }
  }
}

template <int NB>
static hipError_t launch_gate_up_nb(const GemvArgs& a, hipStream_t st) {
  constexpr int RPW = 2;
  const dim3 grid(a.I / (4 * RPW), a.n_slots);
  gemv_gate_up_fp4_kernel<NB, RPW><<<grid, 256, 0, st>>>(a.gq, a.gs, a.uq, a.us, a.xq, a.xs,
                                                         a.offsets, a.row_token, a.E, a.H, a.I,
                                                         a.h);
  return hipGetLastError();
}

template <int NB, bool COMBINE>
static hipError_t launch_down_nb(const GemvArgs& a, hipStream_t st) {
  constexpr int RMAX = kGemvMaxRows, RPW = 2;
  const dim3 grid(a.H / (4 * RPW));
  const size_t lds = (size_t)RMAX * a.I + (size_t)RMAX * (a.I / 128) * sizeof(float);
  gemv_down_fp4_kernel<NB, RMAX, RPW, COMBINE><<<grid, 256, lds, st>>>(
      a.dq, a.ds, a.h, a.offsets, a.row_of, a.topk_w, a.E, a.H, a.I, a.k, a.y_rows, a.out,
      a.out_bf16, a.hq_ws, a.hs_ws);
  return hipGetLastError();
}

hipError_t launch_gemv_gate_up(const GemvArgs& a, hipStream_t st) {
  const int nb = (a.H / 32 + 63) / 64;
  if (nb <= 1) return launch_gate_up_nb<1>(a, st);
  if (nb <= 2) return launch_gate_up_nb<2>(a, st);
  return launch_gate_up_nb<4>(a, st);
}

hipError_t launch_gemv_down(const GemvArgs& a, bool combine, hipStream_t st) {
  const int nb = (a.I / 32 + 63) / 64;
  if (combine) {
    if (nb <= 1) return launch_down_nb<1, true>(a, st);
    if (nb <= 2) return launch_down_nb<2, true>(a, st);
    return launch_down_nb<4, true>(a, st);
  }
  if (nb <= 1) return launch_down_nb<1, false>(a, st);
  if (nb <= 2) return launch_down_nb<2, false>(a, st);
  return launch_down_nb<4, false>(a, st);
}

}  // namespace bef
