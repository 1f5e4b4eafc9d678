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
// for every activation row of the group (a second token of the group finds
// the rows in L2), activations from xq/xs; the last block of each 128-wide
// block of h requantises it (publish_h).  FMT 1: FP4 weights, 2: FP8.
// ---------------------------------------------------------------------------
template <int NB, int FMT>
__global__ __launch_bounds__(256) void gemv_gate_up_kernel(
    GUWeights w, const uint8_t* __restrict__ xq, const float* __restrict__ xs,
    const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ row_token, const int4* __restrict__ active,
    const uint8_t* __restrict__ group_mask, HExchange hx) {
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
        offsets, w.E + 1, slot,
        [group_mask](int gg, int c) { return (c > 0 && (!group_mask || group_mask[gg])) ? 1 : 0; },
        stmp, &unused);
    if (g >= 0) r0 = offsets[g], r1 = offsets[g + 1];
  }
  if (g < 0) return;
  const int n0b = (blockIdx.x - slot * bpg) * 4 * RUN;
  const int n0 = n0b + wv * RUN;
  for (int r = r0; r < r1; ++r) {
    // the row's token is looked up once its first weight rows are in flight
    auto acts = [&](uint4 (&aq)[NB][2], float (&xsc)[NB]) {
      const int t = row_token[r];
      load_act_codes<NB>(xq + (size_t)t * w.H, xs + (size_t)t * (w.H >> 7), w.H, lane, aq, xsc);
    };
    float hv;
    if (FMT == 1) {
      hv = gate_up_rows<NB>(w, g, n0, lane, acts);
    } else {
      const GUWeights8 w8 = {w.gq, w.uq, reinterpret_cast<const float*>(w.gs),
                             reinterpret_cast<const float*>(w.us), w.E, w.H, w.I};
      hv = gate_up_rows_fp8<NB>(w8, g, n0, lane, acts);
    }
    publish_h(hx, hv, r, w.I, n0, n0b, tid, lane);
  }
}

// ---------------------------------------------------------------------------
// down (+ combine).  Block b owns output rows m0 = 8b .. 8b+7; wave w takes
// the h rows r = w, w+8, w+16, w+24 (< R = T*k + T <= 32) in turn: it
// multiplies row r of the requantised h (E4M3 codes + scales from the
// gate+up kernel; only its own row, 2 KB for I = 2048) by rows m0..m0+7 of
// its group's W_down, streamed through a 3-deep register pipeline held in
// order by a dependency-carrying empty asm statement (as in gate_up_rows).
// A butterfly gives the 8 totals; COMBINE then adds them per token and
// output row in LDS -- the shared row first, then the routed slots in rank
// order, out[t][m] = y[shared] + sum_j w_j y[row_of[t][j]]; otherwise the
// totals go to y_rows.
// A row's group comes from the active list when the front kernel wrote one
// (a few uniform loads; the last T rows are the shared expert's), else from
// the offsets table through LDS.  The combine's row_of / topk_w are loaded
// at the start, so the kernel's tail has no dependent load.
// FMT 1: FP4 W_down [E+1][H][I/2] + UE8M0 [E+1][H][I/32]; 2: FP8 W_down
// [E+1][H][I] + fp32 [E+1][H/128][I/128] (rows m0..m0+7 share a 128-row
// block, so one scale per 32-wide chunk of a row of h).
// ---------------------------------------------------------------------------
template <int NB, bool COMBINE, int FMT>
__global__ __launch_bounds__(512) void gemv_down_kernel(
    const uint8_t* __restrict__ dq, const uint8_t* __restrict__ ds,
    const uint8_t* __restrict__ hq, const float* __restrict__ hs,
    const int32_t* __restrict__ offsets, const int4* __restrict__ active, int n_slots,
    int n_rows, const int32_t* __restrict__ row_of, const float* __restrict__ topk_w, int E,
    int H, int I, int k, int T, const uint8_t* __restrict__ group_mask,
    float* __restrict__ y_rows, void* __restrict__ out, int out_bf16) {
  constexpr int RMAX = kHSlotRows, KMAX = kGemvMaxRows, RUN = 8, DEPTH = 3, NW = 8;
  __shared__ int s_rowexp[RMAX];
  __shared__ float s_y[RMAX][RUN];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  int ro[KMAX];
  float twj[KMAX];
  if (COMBINE) {
    const int t = min(tid / RUN, T - 1);  // thread tid < T*RUN combines token tid / RUN
#pragma unroll
    for (int j = 0; j < KMAX; ++j) {
      ro[j] = (j <= k) ? row_of[(size_t)t * (k + 1) + j] : -1;
      twj[j] = (j < k) ? topk_w[(size_t)t * k + j] : 0.0f;
    }
  }
  int R;
  if (active) {
    R = min(n_rows, RMAX);
  } else {
    R = min(offsets[E + 1], RMAX);
    for (int gg = tid; gg <= E; gg += 512) {
      const int a = offsets[gg], b = offsets[gg + 1];
      for (int rr = a; rr < b && rr < RMAX; ++rr) s_rowexp[rr] = gg;
    }
    __syncthreads();
  }
  const int m0 = blockIdx.x * RUN;
  const int nch = I >> 5;
  for (int r = wv; r < R; r += NW) {
    int g = E;  // rows past the T*k routed ones: the shared expert
    if (active) {
      if (r < n_rows - T) {
        // the slot holding row r (the slots' row ranges are disjoint): lane j
        // loads entry q0 + j, a ballot finds the match -- one load round trip
        // for up to 64 slots, where a loop of scalar loads waited for each
        // entry in turn
        g = 0;
        for (int q0 = 0; q0 < n_slots; q0 += 64) {
          const int4 v = active[min(q0 + lane, n_slots - 1)];
          const uint64_t m =
              __ballot((q0 + lane < n_slots) & (v.x >= 0) & (r >= v.y) & (r < v.z));
          if (m) g = __builtin_amdgcn_readlane(v.x, __ffsll((long long)m) - 1);
        }
      }
    } else {
      g = s_rowexp[r];
      if (group_mask && !group_mask[g]) continue;  // a skipped group: row left untouched
    }
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
    float part[RUN];
    int dep = 0;
    if (FMT == 1) {
      const size_t rowq = (size_t)(I >> 1), rows_ = (size_t)nch;
      const uint8_t* wb = dq + row0 * rowq;
      const uint8_t* sbb = ds + row0 * rows_;
      uint4 w[DEPTH][NB];
      uint32_t sb[DEPTH][NB];
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
    } else {
      const size_t rowq = (size_t)I;
      const uint8_t* wb = dq + row0 * rowq;
      const float* sc8 = reinterpret_cast<const float*>(ds) +
                         ((size_t)g * (H >> 7) + (m0 >> 7)) * (size_t)(I >> 7);
      uint4 w[DEPTH][NB][2];
#define BEF_DN8_LOAD(SLOT, ROW)                                                             \
  _Pragma("unroll") for (int c = 0; c < NB; ++c) {                                          \
    w[SLOT][c][0] = *reinterpret_cast<const uint4*>(wb + (ROW) * rowq + 32 * ch[c] + dep);   \
    w[SLOT][c][1] = *reinterpret_cast<const uint4*>(wb + (ROW) * rowq + 32 * ch[c] + 16 + dep); \
  }
#pragma unroll
      for (int d = 0; d < DEPTH - 1; ++d) {
        BEF_DN8_LOAD(d, d)
      }
      Act16 a0[NB], a1[NB];
      float hsc[NB];
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        const float wsc = sc8[ch[c] >> 2];
        e4m3x16_to_h2(aq[c][0], a0[c]);
        e4m3x16_to_h2(aq[c][1], a1[c]);
        hsc[c] = (lane + 64 * c < nch) ? hs_raw[c] * wsc : 0.0f;
      }
#pragma unroll
      for (int i = 0; i < RUN; ++i) {
        if (i + DEPTH - 1 < RUN) {
          BEF_DN8_LOAD((i + DEPTH - 1) % DEPTH, i + DEPTH - 1)
        }
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < NB; ++c)
          acc += dot32_fp8(w[i % DEPTH][c][0], w[i % DEPTH][c][1], a0[c], a1[c]) * hsc[c];
        part[i] = acc;
        asm volatile("" : "+v"(dep) : "v"(acc));
      }
#undef BEF_DN8_LOAD
    }
    const float tot = butterfly8(part);  // j = 4*bit5 + 2*bit4 + bit3
    if ((lane & 7) == 0) s_y[r][lane >> 3] = tot;
  }
  __syncthreads();
  if (COMBINE) {
    if (tid < T * RUN) {
      const int t = tid / RUN, mm = tid - t * RUN;
      const int rs = ro[k & (KMAX - 1)];
      float o = (rs >= 0 && rs < RMAX) ? s_y[rs][mm] : 0.0f;
      for (int j = 0; j < k; ++j) {
        const int rj = ro[j & (KMAX - 1)];
        if (rj >= 0 && rj < RMAX) o = fmaf(twj[j & (KMAX - 1)], s_y[rj][mm], o);
      }
      const size_t m = (size_t)t * H + m0 + mm;
      if (out_bf16)
        reinterpret_cast<uint16_t*>(out)[m] = f32_to_bf16(o);
      else
        reinterpret_cast<float*>(out)[m] = o;
    }
  } else {
    for (int i = tid; i < R * RUN; i += 512)
      if (active || !group_mask || group_mask[s_rowexp[i / RUN]])
        y_rows[(size_t)(i / RUN) * H + m0 + (i % RUN)] = s_y[i / RUN][i % RUN];
  }
}

template <int NB, int FMT>
static hipError_t launch_gate_up_nb(const GemvArgs& a, hipStream_t st) {
  constexpr int RUN = kGuRun;
  if (a.I % 128 != 0 || a.I > kHSlotStride) return hipErrorInvalidValue;
  const GUWeights w = {a.gq, a.gs, a.uq, a.us, a.E, a.H, a.I};
  const dim3 grid((a.I / (4 * RUN)) * a.n_slots);
  const HExchange hx = {a.h_slots, a.h, a.hq_ws, a.hs_ws, a.status};
  const KernelTimer& tm = g_kernel_timer[MOE_KERNEL_GEMV_GATE_UP];
  if (tm.start)
    hipExtLaunchKernelGGL(gemv_gate_up_kernel<NB, FMT>, grid, dim3(256), 0, st, tm.start,
                          tm.stop, 0, w, a.xq, a.xs, a.offsets, a.row_token, a.active,
                          a.group_mask, hx);
  else
    gemv_gate_up_kernel<NB, FMT><<<grid, 256, 0, st>>>(w, a.xq, a.xs, a.offsets, a.row_token,
                                                       a.active, a.group_mask, hx);
  return hipGetLastError();
}

template <int NB, bool COMBINE, int FMT>
static hipError_t launch_down_nb(const GemvArgs& a, hipStream_t st) {
  if (a.H % 8 != 0 || a.T < 1 || a.T * (a.k + 1) > kHSlotRows) return hipErrorInvalidValue;
  if (COMBINE && a.k + 1 > kGemvMaxRows) return hipErrorInvalidValue;
  const KernelTimer& tm = g_kernel_timer[MOE_KERNEL_GEMV_DOWN];
  if (tm.start)
    hipExtLaunchKernelGGL(gemv_down_kernel<NB, COMBINE, FMT>, dim3(a.H / 8), dim3(512), 0, st,
                          tm.start, tm.stop, 0, a.dq, a.ds, a.hq_ws, a.hs_ws, a.offsets,
                          a.active, a.n_slots, a.n_rows, a.row_of, a.topk_w, a.E, a.H, a.I, a.k,
                          a.T, a.group_mask, a.y_rows, a.out, a.out_bf16);
  else
    gemv_down_kernel<NB, COMBINE, FMT><<<dim3(a.H / 8), 512, 0, st>>>(
        a.dq, a.ds, a.hq_ws, a.hs_ws, a.offsets, a.active, a.n_slots, a.n_rows, a.row_of,
        a.topk_w, a.E, a.H, a.I, a.k, a.T, a.group_mask, a.y_rows, a.out, a.out_bf16);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_gemv_gate_up_f(const GemvArgs& a, hipStream_t st) {
  const int nb = (a.H / 32 + 63) / 64;
  if (nb <= 1) return launch_gate_up_nb<1, FMT>(a, st);
  if (nb <= 2) return launch_gate_up_nb<2, FMT>(a, st);
  return launch_gate_up_nb<4, FMT>(a, st);
}

hipError_t launch_gemv_gate_up(const GemvArgs& a, hipStream_t st) {
  return a.fmt == 2 ? launch_gemv_gate_up_f<2>(a, st) : launch_gemv_gate_up_f<1>(a, st);
}

template <int FMT>
static hipError_t launch_gemv_down_f(const GemvArgs& a, bool combine, hipStream_t st) {
  const int nb = (a.I / 32 + 63) / 64;
  if (combine) {
    if (nb <= 1) return launch_down_nb<1, true, FMT>(a, st);
    return launch_down_nb<2, true, FMT>(a, st);
  }
  if (nb <= 1) return launch_down_nb<1, false, FMT>(a, st);
  return launch_down_nb<2, false, FMT>(a, st);
}

hipError_t launch_gemv_down(const GemvArgs& a, bool combine, hipStream_t st) {
  return a.fmt == 2 ? launch_gemv_down_f<2>(a, combine, st)
                    : launch_gemv_down_f<1>(a, combine, st);
}

}  // namespace bef
