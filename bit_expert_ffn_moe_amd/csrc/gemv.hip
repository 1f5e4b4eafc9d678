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
#include <hip/hip_ext.h>

#include "common.h"
#include "gemv_body.h"
#include "kernels.h"

namespace bef {

// ---------------------------------------------------------------------------
// gate + up + SwiGLU.  Block b serves group slot b / (I/(4 RUN)): the slot's
// group and rows come from `active` ({group, first row, end row}, written by
// the front kernel) or, without it, from the offsets table (no host round
// trip either way).  Wave w streams RUN rows from n0 = (4 (b mod bpg) + w) RUN
// for every activation row of the group, activations from xq/xs; the last
// block of each 128-wide block of h requantises it (publish_h).
// ---------------------------------------------------------------------------
template <int NB>
__global__ __launch_bounds__(256) void gemv_gate_up_fp4_kernel(
    GUWeights w, const uint8_t* __restrict__ xq, const float* __restrict__ xs,
    const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ row_token, const int4* __restrict__ active,
    HExchange hx) {
  __shared__ int stmp[8];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
  constexpr int RUN = kGuRun;
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
  const int n0b = (blockIdx.x - slot * bpg) * 4 * RUN;
  const int n0 = n0b + wv * RUN;
  for (int r = r0; r < r1; ++r) {
    const int t = row_token[r];
    uint4 aq[NB][2];
    float xsc[NB];
    load_act_codes<NB>(xq + (size_t)t * w.H, xs + (size_t)t * (w.H >> 7), w.H, lane, aq, xsc);
    const float hv = gate_up_rows<NB>(w, g, n0, lane, aq, xsc);
    publish_h(hx, hv, r, w.I, n0, n0b, tid, lane);
  }
}

// ---------------------------------------------------------------------------
// down (+ combine for a single token).  Block b owns output rows m0 = 8b ..
// 8b+7, one wave per routed row r < R <= 8: wave r multiplies row r of the
// requantised h (E4M3 codes + scales from the gate+up kernel; only its own
// row, 2 KB for I = 2048) by rows m0..m0+7 of its group's W_down, streamed
// through a 3-deep register pipeline held in order by a dependency-carrying
// empty asm statement (as in gate_up_rows).  A butterfly gives the 8 totals;
// COMBINE then adds them per output row in LDS -- the shared row first, then
// the routed slots in rank order, out[m] = y[shared] + sum_j w_j y[row_of[j]]
// (T = 1); otherwise the totals go to y_rows.
// A row's group comes from the active list when the front kernel wrote one
// (a few uniform loads; the last row is the shared expert's), else from the
// offsets table through LDS.  The combine's row_of / topk_w are loaded at
// the start, so the kernel's tail has no dependent load.
// ---------------------------------------------------------------------------
template <int NB, bool COMBINE>
__global__ __launch_bounds__(512) void gemv_down_fp4_kernel(
    const uint8_t* __restrict__ dq, const uint8_t* __restrict__ ds,
    const uint8_t* __restrict__ hq, const float* __restrict__ hs,
    const int32_t* __restrict__ offsets, const int4* __restrict__ active, int n_slots,
    int n_rows, const int32_t* __restrict__ row_of, const float* __restrict__ topk_w, int E,
    int H, int I, int k, float* __restrict__ y_rows, void* __restrict__ out, int out_bf16) {
  constexpr int RMAX = kGemvMaxRows, RUN = 8, DEPTH = 3;
  __shared__ int s_rowexp[RMAX];
  __shared__ float s_y[RMAX][RUN];
  const int tid = threadIdx.x, lane = tid & 63;
  const int r = __builtin_amdgcn_readfirstlane(tid >> 6);
  int ro[RMAX];
  float twj[RMAX];
  if (COMBINE) {
#pragma unroll
    for (int j = 0; j < RMAX; ++j) {
      ro[j] = (j <= k) ? row_of[j] : -1;
      twj[j] = (j < k) ? topk_w[j] : 0.0f;
    }
  }
  int R, g = 0;
  if (active) {
    R = min(n_rows, RMAX);
    g = E;  // the last row: the shared expert
    if (r < R - 1) {
      g = 0;
      for (int q = 0; q < n_slots; ++q) {
        const int4 v = active[q];
        if (v.x >= 0 && r >= v.y && r < v.z) g = v.x;
      }
    }
  } else {
    R = min(offsets[E + 1], RMAX);
    for (int gg = tid; gg <= E; gg += 512) {
      const int a = offsets[gg], b = offsets[gg + 1];
      for (int rr = a; rr < b && rr < RMAX; ++rr) s_rowexp[rr] = gg;
    }
    __syncthreads();
    if (r < R) g = s_rowexp[r];
  }
  const int m0 = blockIdx.x * RUN;
  if (r < R) {
    const int nch = I >> 5;
    const size_t rowq = (size_t)(I >> 1), rows_ = (size_t)nch;
    // chunk indices clamped into the row (unconditional loads); a chunk past
    // the end gets scale 0 and adds exactly 0
    int ch[NB];
    uint4 aq[NB][2];
    float hs_raw[NB];
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      ch[c] = min(lane + 64 * c, nch - 1);
      const uint8_t* p = hq + (size_t)r * I + 32 * ch[c];
      aq[c][0] = *reinterpret_cast<const uint4*>(p);
      aq[c][1] = *reinterpret_cast<const uint4*>(p + 16);
      hs_raw[c] = hs[(size_t)r * (I >> 7) + (ch[c] >> 2)];
    }
    const size_t row0 = (size_t)g * H + m0;
    const uint8_t* wb = dq + row0 * rowq;
    const uint8_t* sbb = ds + row0 * rows_;
    uint4 w[DEPTH][NB];
    uint32_t sb[DEPTH][NB];
    int dep = 0;
#define BEF_DN_LOAD(SLOT, ROW)                                                         \
  _Pragma("unroll") for (int c = 0; c < NB; ++c) {                                     \
    w[SLOT][c] = *reinterpret_cast<const uint4*>(wb + (ROW) * rowq + 16 * ch[c] + dep); \
    sb[SLOT][c] = sbb[(ROW) * rows_ + ch[c] + dep];                                    \
  }
#pragma unroll
    for (int d = 0; d < DEPTH - 1; ++d) {
      BEF_DN_LOAD(d, d)
    }
    // the activations, once the first rows are in flight
    Act16 a0[NB], a1[NB];
    float hsc[NB];
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      e4m3x16_to_h2(aq[c][0], a0[c]);
      e4m3x16_to_h2(aq[c][1], a1[c]);
      hsc[c] = (lane + 64 * c < nch) ? hs_raw[c] : 0.0f;
    }
    float part[RUN];
#pragma unroll
    for (int i = 0; i < RUN; ++i) {
      if (i + DEPTH - 1 < RUN) {
        BEF_DN_LOAD((i + DEPTH - 1) % DEPTH, i + DEPTH - 1)
      }
      float acc = 0.0f;
#pragma unroll
      for (int c = 0; c < NB; ++c)
        acc += scale_ue8m0(dot32_fp4(w[i % DEPTH][c], a0[c], a1[c]), sb[i % DEPTH][c]) * hsc[c];
      part[i] = acc;
      asm volatile("" : "+v"(dep) : "v"(acc));
    }
#undef BEF_DN_LOAD
    const float tot = butterfly8(part);  // j = 4*bit5 + 2*bit4 + bit3
    if ((lane & 7) == 0) s_y[r][lane >> 3] = tot;
  }
  __syncthreads();
  if (COMBINE) {
    if (tid < RUN) {
      const int rs = ro[k & (RMAX - 1)];
      float o = (rs >= 0 && rs < RMAX) ? s_y[rs][tid] : 0.0f;
      for (int j = 0; j < k; ++j) {
        const int rj = ro[j & (RMAX - 1)];
        if (rj >= 0 && rj < RMAX) o = fmaf(twj[j & (RMAX - 1)], s_y[rj][tid], o);
      }
      const int m = m0 + tid;
      if (out_bf16)
        reinterpret_cast<uint16_t*>(out)[m] = f32_to_bf16(o);
      else
        reinterpret_cast<float*>(out)[m] = o;
    }
  } else if (tid < R * RUN) {
    y_rows[(size_t)(tid / RUN) * H + m0 + (tid % RUN)] = s_y[tid / RUN][tid % RUN];
  }
}

template <int NB>
static hipError_t launch_gate_up_nb(const GemvArgs& a, hipStream_t st) {
  constexpr int RUN = kGuRun;
  if (a.I % 128 != 0 || a.I > kHSlotStride) return hipErrorInvalidValue;
  const GUWeights w = {a.gq, a.gs, a.uq, a.us, a.E, a.H, a.I};
  const dim3 grid((a.I / (4 * RUN)) * a.n_slots);
  const HExchange hx = {a.h_slots, a.h, a.hq_ws, a.hs_ws, a.status};
  const KernelTimer& tm = g_kernel_timer[MOE_KERNEL_GEMV_GATE_UP];
  if (tm.start)
    hipExtLaunchKernelGGL(gemv_gate_up_fp4_kernel<NB>, grid, dim3(256), 0, st, tm.start, tm.stop,
                          0, w, a.xq, a.xs, a.offsets, a.row_token, a.active, hx);
  else
    gemv_gate_up_fp4_kernel<NB><<<grid, 256, 0, st>>>(w, a.xq, a.xs, a.offsets, a.row_token,
                                                      a.active, hx);
  return hipGetLastError();
}

template <int NB, bool COMBINE>
static hipError_t launch_down_nb(const GemvArgs& a, hipStream_t st) {
  if (a.H % 8 != 0) return hipErrorInvalidValue;
  if (COMBINE && a.k + 1 > kGemvMaxRows) return hipErrorInvalidValue;
  gemv_down_fp4_kernel<NB, COMBINE><<<dim3(a.H / 8), 512, 0, st>>>(
      a.dq, a.ds, a.hq_ws, a.hs_ws, a.offsets, a.active, a.n_slots, a.n_rows, a.row_of,
      a.topk_w, a.E, a.H, a.I, a.k, a.y_rows, a.out, a.out_bf16);
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
