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
// for every activation row of the group, activations from xq/xs; the last
// block of each 128-wide block of h requantises it (publish_h).
// ---------------------------------------------------------------------------
template <int NB, int DEPTH>
__global__ __launch_bounds__(256) void gemv_gate_up_fp4_kernel(
    GUWeights w, const uint8_t* __restrict__ xq, const float* __restrict__ xs,
    const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ row_token, const int4* __restrict__ active,
    HExchange hx) {
  __shared__ int stmp[8];
  __shared__ uint32_t s_ticket;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar registers
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
  const int n0b = (blockIdx.x - slot * bpg) * 4 * RUN;
  const int n0 = n0b + wv * RUN;
  for (int r = r0; r < r1; ++r) {
    const int t = row_token[r];
    Act16 a0[NB], a1[NB];
    float xsc[NB];
    act_from_codes<NB>(xq + (size_t)t * w.H, xs + (size_t)t * (w.H >> 7), w.H, lane, a0, a1, xsc);
    const float hv = gate_up_rows<NB, DEPTH>(w, g, n0, lane, a0, a1, xsc);
    publish_h(hx, hv, r, w.I, n0, n0b, tid, lane, &s_ticket);
  }
}

// ---------------------------------------------------------------------------
// down (+ combine for a single token).  Wave w of block b owns output rows
// m = (4b + w)*RUN .. +RUN-1.  Once the row -> expert map is known, every
// load of the wave is issued at once: the E4M3 codes and scales of h (R rows,
// requantised by the gate+up kernel), then every W_down chunk (R rows x RUN
// outputs, one 16-byte chunk per lane for I = 2048) with its UE8M0 scale.
// COMBINE writes out[m] = y[shared] + sum_j w_j y[row_of[j]] (T = 1);
// otherwise y_rows.
// ---------------------------------------------------------------------------
template <int NB, int RMAX, int RUN, bool COMBINE>
__global__ __launch_bounds__(256) void gemv_down_fp4_kernel(
    const uint8_t* __restrict__ dq, const uint8_t* __restrict__ ds,
    const uint8_t* __restrict__ hq, const float* __restrict__ hs,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ row_of,
    const float* __restrict__ topk_w, int E, int H, int I, int k, float* __restrict__ y_rows,
    void* __restrict__ out, int out_bf16) {
  __shared__ int s_rowexp[RMAX];
  const int R = min(offsets[E + 1], RMAX);
  const int tid = threadIdx.x;
  for (int g = tid; g <= E; g += 256) {
    const int a = offsets[g], b = offsets[g + 1];
    for (int r = a; r < b && r < RMAX; ++r) s_rowexp[r] = g;
  }
  __syncthreads();

  const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m0 = (blockIdx.x * 4 + wv) * RUN;
  const int nch = I >> 5;
  const size_t rowq = (size_t)(I >> 1), rows_ = (size_t)nch;
  // chunk indices clamped into the row (unconditional loads); a chunk past
  // the end gets scale 0 and adds exactly 0
  int ch[NB];
#pragma unroll
  for (int c = 0; c < NB; ++c) ch[c] = min(lane + 64 * c, nch - 1);
  uint4 aq[RMAX][NB][2];
  float asc[RMAX][NB];
#pragma unroll
  for (int r = 0; r < RMAX; ++r)
    if (r < R)
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        const uint8_t* p = hq + (size_t)r * I + 32 * ch[c];
        aq[r][c][0] = *reinterpret_cast<const uint4*>(p);
        aq[r][c][1] = *reinterpret_cast<const uint4*>(p + 16);
        asc[r][c] = hs[r * (I >> 7) + (ch[c] >> 2)];
      }
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
          w[r][i][c] = *reinterpret_cast<const uint4*>(dq + (row0 + i) * rowq + 16 * ch[c]);
          sb[r][i][c] = ds[(row0 + i) * rows_ + ch[c]];
        }
    }
  }

  // per-lane partials of y[r][i] (r < RMAX rows, i < RUN outputs), one
  // butterfly, then every lane holds the total of j = r*RUN + i
  static_assert(RMAX * RUN == 16, "butterfly16 layout");
  float part[RMAX * RUN];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
#pragma unroll
    for (int i = 0; i < RUN; ++i) part[r * RUN + i] = 0.0f;
    if (r < R) {
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        Act16 a0, a1;
        e4m3x16_to_h2(aq[r][c][0], a0);
        e4m3x16_to_h2(aq[r][c][1], a1);
        const float hsc = (lane + 64 * c < nch) ? asc[r][c] : 0.0f;
#pragma unroll
        for (int i = 0; i < RUN; ++i)
          part[r * RUN + i] += scale_ue8m0(dot32_fp4(w[r][i][c], a0, a1), sb[r][i][c]) * hsc;
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
  if (a.I % 128 != 0 || a.I > kHSlotStride) return hipErrorInvalidValue;
  const GUWeights w = {a.gq, a.gs, a.uq, a.us, a.E, a.H, a.I};
  const dim3 grid((a.I / (4 * RUN)) * a.n_slots);
  gemv_gate_up_fp4_kernel<NB, DEPTH><<<grid, 256, 0, st>>>(
      w, a.xq, a.xs, a.offsets, a.row_token, a.active,
      HExchange{a.hq_arrive, a.h_slots, a.h, a.hq_ws, a.hs_ws, a.status});
  return hipGetLastError();
}

template <int NB, bool COMBINE>
static hipError_t launch_down_nb(const GemvArgs& a, hipStream_t st) {
  constexpr int RMAX = kGemvMaxRows, RUN = 2;
  if (a.H % (4 * RUN) != 0) return hipErrorInvalidValue;
  const dim3 grid(a.H / (4 * RUN));
  gemv_down_fp4_kernel<NB, RMAX, RUN, COMBINE><<<grid, 256, 0, st>>>(
      a.dq, a.ds, a.hq_ws, a.hs_ws, a.offsets, a.row_of, a.topk_w, a.E, a.H, a.I, a.k, a.y_rows,
      a.out, a.out_bf16);
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
