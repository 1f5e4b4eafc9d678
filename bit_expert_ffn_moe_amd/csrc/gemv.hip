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
// block, and a wave reads a 1 KiB contiguous stretch per load instruction
// (gemv_body.h).
#include "common.h"
#include "gemv_body.h"
#include "kernels.h"

namespace bef {

// ---------------------------------------------------------------------------
// gate + up + SwiGLU.  Block b serves group slot b / (I/(4 RUN)): the slot's
// group and rows come from `active` ({group, first row, end row}, written by
// the front kernel) or, without it, from the offsets table (no host round
// trip either way).  Wave w streams RUN rows from n0 = (4 (b mod bpg) + w) RUN
// for every activation row of the group, activations from xq/xs.
// ---------------------------------------------------------------------------
template <int NB, int DEPTH>
__global__ __launch_bounds__(256) void gemv_gate_up_fp4_kernel(
    GUWeights w, const uint8_t* __restrict__ xq, const float* __restrict__ xs,
    const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ row_token, const int4* __restrict__ active,
    float* __restrict__ h) {
  __shared__ int stmp[8];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  constexpr int RUN = kGemvRun;
  const int bpg = w.I / (4 * RUN);
  const int slot = blockIdx.x / bpg;
  int g, r0 = 0, r1 = 0;
  if (active) {
    const int4 a = active[slot];
    g = a.x, r0 = a.y, r1 = a.z;
  } else {
    int unused;
    g = find_group_item(
        offsets, w.E + 1, slot, [](int c) { return c > 0 ? 1 : 0; }, stmp, &unused);
    if (g >= 0) r0 = offsets[g], r1 = offsets[g + 1];
  }
  if (g < 0) return;
  const int n0 = ((blockIdx.x - slot * bpg) * 4 + wv) * RUN;
  for (int r = r0; r < r1; ++r) {
    const int t = row_token[r];
    Act16 a0[NB], a1[NB];
    float xsc[NB];
    act_from_codes<NB>(xq + (size_t)t * w.H, xs + (size_t)t * (w.H >> 7), w.H, lane, a0, a1, xsc);
    gate_up_rows<NB, DEPTH>(w, g, n0, r, lane, a0, a1, xsc, h);
  }
}

// ---------------------------------------------------------------------------
// down (+ combine for a single token).  Wave w of block b owns output rows
// m = (4b + w)*RUN .. +RUN-1.  Once the row -> expert map is known, every
// W_down load of the wave (R rows x RUN outputs, one 16-byte chunk per lane
// for I = 2048) is issued; while they fly the block requantises all R rows
// of h to E4M3 per 128 into LDS (the act_quant rule; block 0 also stores the
// codes/scales to the workspace for inspection).  COMBINE writes
// out[m] = y[shared] + sum_j w_j y[row_of[j]] (T = 1); otherwise y_rows.
// ---------------------------------------------------------------------------
template <int NB, int RMAX, int RUN, bool COMBINE>
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
  for (int g = tid; g <= E; g += 256) {
    const int a = offsets[g], b = offsets[g + 1];
    for (int r = a; r < b && r < RMAX; ++r) s_rowexp[r] = g;
  }
  __syncthreads();

  const int lane = tid & 63, wv = tid >> 6;
  const int m0 = (blockIdx.x * 4 + wv) * RUN;
  const int nch = I >> 5;
  const size_t rowq = (size_t)(I >> 1), rows_ = (size_t)nch;
  uint4 w[RMAX][RUN][NB];
  uint32_t sb[RMAX][RUN][NB];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    if (r < R) {
      const size_t row0 = (size_t)s_rowexp[r] * H + m0;
#pragma unroll
      for (int i = 0; i < RUN; ++i)
#pragma unroll
        for (int c = 0; c < NB; ++c) {
          const int ch = lane + 64 * c;
          if (ch < nch) {
            w[r][i][c] = *reinterpret_cast<const uint4*>(dq + (row0 + i) * rowq + 16 * ch);
            sb[r][i][c] = ds[(row0 + i) * rows_ + ch];
          } else {
            w[r][i][c] = make_uint4(0, 0, 0, 0);
            sb[r][i][c] = 127;
          }
        }
    }
  }
  // requantise h: 16 lanes per 128-block, 8 elements per lane; the loads of
  // QB chunks per thread are issued together before any is quantised
  const int nq = R * (I >> 3);
  constexpr int QB = 8;
  for (int base = 0; base < nq; base += 256 * QB) {
    float4 p[QB][2];
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int idx = base + q * 256 + tid;
      if (idx < nq) {
        p[q][0] = reinterpret_cast<const float4*>(h)[2 * idx];
        p[q][1] = reinterpret_cast<const float4*>(h)[2 * idx + 1];
      } else {
        p[q][0] = p[q][1] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
#pragma unroll
    for (int q = 0; q < QB; ++q) {
      const int idx = base + q * 256 + tid;
      const float v[8] = {p[q][0].x, p[q][0].y, p[q][0].z, p[q][0].w,
                          p[q][1].x, p[q][1].y, p[q][1].z, p[q][1].w};
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
      if (idx < nq) {
        reinterpret_cast<uint2*>(s_hq)[idx] = make_uint2(lo, hi);
        if ((idx & 15) == 0) s_hs[idx >> 4] = sc;
        if (blockIdx.x == 0) {
          reinterpret_cast<uint2*>(hq_ws)[idx] = make_uint2(lo, hi);
          if ((idx & 15) == 0) hs_ws[idx >> 4] = sc;
        }
      }
    }
  }
  __syncthreads();

  // per-lane partials of y[r][i] (r < RMAX rows, i < RUN outputs), one
  // butterfly, then every lane holds the total of j = r*RUN + i
  static_assert(RMAX * RUN == 16, "butterfly16 layout");
  float part[RMAX * RUN];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
#pragma unroll
    for (int i = 0; i < RUN; ++i) part[r * RUN + i] = 0.0f;
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
      for (int i = 0; i < RUN; ++i) {
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < NB; ++c)
          acc += scale_ue8m0(dot32_fp4(w[r][i][c], a0[c], a1[c]), sb[r][i][c]) * hsc[c];
        part[r * RUN + i] = acc;
      }
    }
  }
  const float tot = butterfly16(part);       // j = 8*bit5 + 4*bit4 + 2*bit3 + bit2
  const int jr = (lane >> 3) & 7, ji = (lane >> 2) & 1;  // j = 2*jr + ji
  if (COMBINE) {
    __shared__ float s_y[4][RMAX][RUN];
    if ((lane & 3) == 0) s_y[wv][jr][ji] = tot;
    __syncthreads();
    if (lane < RUN) {
      // lane i finishes output row m0 + i (T = 1: token 0), shared first, then
      // the routed slots in rank order
      const int rs = row_of[k];
      float o = (rs >= 0) ? s_y[wv][rs][lane] : 0.0f;
      for (int j = 0; j < k; ++j) {
        const int rj = row_of[j];
        if (rj >= 0) o = fmaf(topk_w[j], s_y[wv][rj][lane], o);
      }
      const int m = m0 + lane;
      if (out_bf16)
        reinterpret_cast<uint16_t*>(out)[m] = f32_to_bf16(o);
      else
        reinterpret_cast<float*>(out)[m] = o;
    }
  } else {
    if ((lane & 3) == 0 && jr < R) y_rows[(size_t)jr * H + m0 + ji] = tot;
  }
}

template <int NB>
static hipError_t launch_gate_up_nb(const GemvArgs& a, hipStream_t st) {
  constexpr int RUN = kGemvRun, DEPTH = 3;
  if (a.I % (4 * RUN) != 0) return hipErrorInvalidValue;
  const GUWeights w = {a.gq, a.gs, a.uq, a.us, a.E, a.H, a.I};
  const dim3 grid((a.I / (4 * RUN)) * a.n_slots);
  gemv_gate_up_fp4_kernel<NB, DEPTH><<<grid, 256, 0, st>>>(
      w, a.xq, a.xs, a.offsets, a.row_token, a.active, a.h);
  return hipGetLastError();
}

template <int NB, bool COMBINE>
static hipError_t launch_down_nb(const GemvArgs& a, hipStream_t st) {
  constexpr int RMAX = kGemvMaxRows, RUN = 2;
  if (a.H % (4 * RUN) != 0) return hipErrorInvalidValue;
  const dim3 grid(a.H / (4 * RUN));
  const size_t lds = (size_t)RMAX * a.I + (size_t)RMAX * (a.I / 128) * sizeof(float);
  gemv_down_fp4_kernel<NB, RMAX, RUN, COMBINE><<<grid, 256, lds, st>>>(
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
    return launch_down_nb<2, true>(a, st);
  }
  if (nb <= 1) return launch_down_nb<1, false>(a, st);
  return launch_down_nb<2, false>(a, st);
}

}  // namespace bef
