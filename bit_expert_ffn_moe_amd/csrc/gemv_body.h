// gemv_body.h -- the one-token FP4 gate+up GEMV as device functions, shared
// by the gate+up kernel (gemv.hip) and the front kernel (route.hip), which
// runs the shared expert's rows while the router's reduction is in flight.
//
// Layout: lane l owns 32-element chunk l + 64c (c < NB) of every row; one
// 16-byte load of a weight row is exactly one UE8M0 scale block; FP4 -> fp16
// with v_cvt_scalef32_pk_f16_fp4, E4M3 -> fp16 with
// v_cvt_scalef32_pk_f16_fp8, products with v_dot2_f32_f16, the UE8M0 scale
// by an exact ldexp and the activation scale by one multiply per 32 weights
// (dpshk.com article, section "核心实现四": dequantise inside the GEMV; gate
// and up share one quantised input).
#pragma once
#include "common.h"
#include "kernels.h"

namespace bef {

struct GUWeights {
  const uint8_t *gq, *gs, *uq, *us;
  int E, H, I;
};

// This lane's activation chunks as raw E4M3 codes (two 16-byte halves per
// chunk) and their block scales, loaded unconditionally (chunk index clamped
// into the row; gate_up_rows masks the chunks past the end): the conversion
// happens in gate_up_rows after the first weight row's loads are issued, so
// the wait for these loads overlaps the weight stream.
template <int NB>
__device__ __forceinline__ void load_act_codes(const uint8_t* __restrict__ xq_row,
                                               const float* __restrict__ xs_row, int H, int lane,
                                               uint4 (&aq)[NB][2], float (&xsc)[NB]) {
  const int nch = H >> 5;
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const int ch = min(lane + 64 * c, nch - 1);
    aq[c][0] = *reinterpret_cast<const uint4*>(xq_row + 32 * ch);
    aq[c][1] = *reinterpret_cast<const uint4*>(xq_row + 32 * ch + 16);
    xsc[c] = xs_row[ch >> 2];
  }
}

// This lane's activation chunks quantised on the fly from the bf16 row, with
// exactly the act_quant rule: the 128-block of chunk ch is spread over the 4
// lanes 4j..4j+3 (ch = 4j..4j+3), so its amax is a 4-lane max; s = amax/448
// (IEEE division), code = E4M3(x/s), a zero block gives s = 0 and code 0.
// Requires H/32 to be a multiple of 4 per 64-lane pass (H % 128 == 0).
template <int NB>
__device__ __forceinline__ void quant_act_codes(const uint16_t* __restrict__ x_row, int H, int lane,
                                                uint4 (&aq)[NB][2], float (&xsc)[NB]) {
  const int nch = H >> 5;
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const int ch = lane + 64 * c;
    uint4 r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      r[i] = (ch < nch) ? *reinterpret_cast<const uint4*>(x_row + 32 * ch + 8 * i)
                        : make_uint4(0, 0, 0, 0);
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * i + 0] = bf16_to_f32(r[i].x & 0xffffu), v[8 * i + 1] = bf16_to_f32(r[i].x >> 16);
      v[8 * i + 2] = bf16_to_f32(r[i].y & 0xffffu), v[8 * i + 3] = bf16_to_f32(r[i].y >> 16);
      v[8 * i + 4] = bf16_to_f32(r[i].z & 0xffffu), v[8 * i + 5] = bf16_to_f32(r[i].z >> 16);
      v[8 * i + 6] = bf16_to_f32(r[i].w & 0xffffu), v[8 * i + 7] = bf16_to_f32(r[i].w >> 16);
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = group_max<4>(amax);
    const float sc = amax / 448.0f;
    uint4 q0 = make_uint4(0, 0, 0, 0), q1 = make_uint4(0, 0, 0, 0);
    if (amax != 0.0f) {
      q0.x = e4m3_pack4(v[0] / sc, v[1] / sc, v[2] / sc, v[3] / sc);
      q0.y = e4m3_pack4(v[4] / sc, v[5] / sc, v[6] / sc, v[7] / sc);
      q0.z = e4m3_pack4(v[8] / sc, v[9] / sc, v[10] / sc, v[11] / sc);
      q0.w = e4m3_pack4(v[12] / sc, v[13] / sc, v[14] / sc, v[15] / sc);
      q1.x = e4m3_pack4(v[16] / sc, v[17] / sc, v[18] / sc, v[19] / sc);
      q1.y = e4m3_pack4(v[20] / sc, v[21] / sc, v[22] / sc, v[23] / sc);
      q1.z = e4m3_pack4(v[24] / sc, v[25] / sc, v[26] / sc, v[27] / sc);
      q1.w = e4m3_pack4(v[28] / sc, v[29] / sc, v[30] / sc, v[31] / sc);
    }
    aq[c][0] = q0;
    aq[c][1] = q1;
    xsc[c] = sc;
  }
}

// Streams 4 consecutive rows n0.. of group g's gate and up matrices for one
// activation row, whose codes and scales acts(aq, xs) loads once the first
// weight rows are in flight (so a lookup of the row's token does not delay
// the weight stream), through a DEPTH-deep register pipeline: the loads of row
// i+DEPTH-1 are issued after row i-1's products, which an empty asm
// statement enforces by passing a zero that depends on those sums into the
// next row's addresses (without it the compiler hoists every load to the
// top, and in the gate+up kernel, where many waves share the stream, the
// higher register count costs more than the deeper pipeline gains).  The
// front kernel's shared-expert rows, which run beside the router's latency
// chain with few waves, take DEPTH = 4: all four rows in flight at once
// (decode step -1%).  One butterfly
// reduce-scatter then gives every lane one of the 8 totals (4 gate, 4 up),
// and 4 lanes finish h[n] = silu(g_n) * u_n in parallel (returned in those
// lanes).
constexpr int kGuRun = 4;
template <int NB, int DEPTH = 2, class Acts>
__device__ __forceinline__ float gate_up_rows(const GUWeights& w, int g, int n0, int lane,
                                              Acts&& acts) {
  constexpr int RUN = kGuRun;
  const int H = w.H, I = w.I;
  const int nch = H >> 5;
  const size_t rowq = (size_t)(H >> 1), rows_ = (size_t)nch;
  // chunk offsets clamped into the row: the loads are unconditional, so no
  // select on a loaded value forces an early wait; a chunk past the row end
  // meets activation codes of 0 and scale 0 and adds exactly 0
  // (the lane index is made opaque so that a caller's loop cannot hoist the
  // 64-bit row addresses out and keep them all live across iterations)
  int ln = lane;
  asm volatile("" : "+v"(ln));
  int co[NB], cs[NB];
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const int ch = min(ln + 64 * c, nch - 1);
    co[c] = 16 * ch;
    cs[c] = ch;
  }
  const uint8_t* gqb = w.gq + ((size_t)g * I + n0) * rowq;
  const uint8_t* uqb = w.uq + ((size_t)g * I + n0) * rowq;
  const uint8_t* gsb = w.gs + ((size_t)g * I + n0) * rows_;
  const uint8_t* usb = w.us + ((size_t)g * I + n0) * rows_;
  uint4 pg[DEPTH][NB], pu[DEPTH][NB];
  uint32_t psg[DEPTH][NB], psu[DEPTH][NB];
  int dep = 0;
#define BEF_GU_LOAD(SLOT, ROW)                                                        \
  _Pragma("unroll") for (int c = 0; c < NB; ++c) {                                    \
    pg[SLOT][c] = *reinterpret_cast<const uint4*>(gqb + (ROW) * rowq + co[c] + dep);  \
    pu[SLOT][c] = *reinterpret_cast<const uint4*>(uqb + (ROW) * rowq + co[c] + dep);  \
    psg[SLOT][c] = gsb[(ROW) * rows_ + cs[c] + dep];                                  \
    psu[SLOT][c] = usb[(ROW) * rows_ + cs[c] + dep];                                  \
  }
#pragma unroll
  for (int d = 0; d + 1 < DEPTH; ++d) {
    BEF_GU_LOAD(d, d)
  }
  // the activation loads, once the first rows are in flight (the compiler
  // barrier keeps acts' loads, and any lookup they wait for, behind them)
  uint4 aq[NB][2];
  float xs_raw[NB];
  asm volatile("" ::: "memory");
  acts(aq, xs_raw);
  Act16 a0[NB], a1[NB];
  float xsc[NB];
  float part[2 * RUN];  // [0..3] gate rows, [4..7] up rows
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    if (i + DEPTH - 1 < RUN) {
      BEF_GU_LOAD((i + DEPTH - 1) % DEPTH, i + DEPTH - 1)
    }
    if (i == 0) {
      // converted after the next row's loads are issued (the wait for the
      // activations then leaves them in flight); chunks past the row end get
      // scale 0
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        e4m3x16_to_h2(aq[c][0], a0[c]);
        e4m3x16_to_h2(aq[c][1], a1[c]);
        xsc[c] = (lane + 64 * c < nch) ? xs_raw[c] : 0.0f;
      }
    }
    const int sl = i % DEPTH;
    float ag = 0.0f, au = 0.0f;
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      ag += scale_ue8m0(dot32_fp4(pg[sl][c], a0[c], a1[c]), psg[sl][c]) * xsc[c];
      au += scale_ue8m0(dot32_fp4(pu[sl][c], a0[c], a1[c]), psu[sl][c]) * xsc[c];
    }
    part[i] = ag;
    part[RUN + i] = au;
    asm volatile("" : "+v"(dep) : "v"(ag), "v"(au));
  }
#undef BEF_GU_LOAD
  const float tot = butterfly8(part);  // j = 4*bit5 + 2*bit4 + bit3
  const float up = xchg32(tot);        // lanes with bit5 = 0 receive the same row's up total
  return silu_mul_accurate(tot, up);   // valid in h_lane() lanes
}

// FP8 weights (fp8_gemm at decode: tcti.cn post, section "补齐软件栈缺失"):
// codes [E+1][I][H] u8 and one fp32 scale per 128x128 block
// [E+1][I/128][H/128].  A 32-element chunk of a row is 32 bytes (two 16-byte
// loads); codes go to fp16 pairwise (exact) and into v_dot2_f32_f16 with the
// activation pairs; the block scale of rows n0..n0+3 (one 128-row block, n0
// a multiple of 4) and the chunk's 128 columns is folded into the
// activation scale, once per chunk.
struct GUWeights8 {
  const uint8_t *gq, *uq;
  const float *gs, *us;
  int E, H, I;
};

__device__ __forceinline__ float dot32_fp8(const uint4 w0, const uint4 w1, const Act16& a0,
                                           const Act16& a1) {
  Act16 b0, b1;
  e4m3x16_to_h2(w0, b0);
  e4m3x16_to_h2(w1, b1);
  float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    acc0 = dot2(b0.p[i], a0.p[i], acc0);
    acc1 = dot2(b1.p[i], a1.p[i], acc1);
  }
  return acc0 + acc1;
}

template <int NB, int DEPTH = 2, class Acts>
__device__ __forceinline__ float gate_up_rows_fp8(const GUWeights8& w, int g, int n0, int lane,
                                                  Acts&& acts) {
  constexpr int RUN = kGuRun;
  const int H = w.H, I = w.I;
  const int nch = H >> 5;
  const size_t rowq = (size_t)H;
  int ln = lane;
  asm volatile("" : "+v"(ln));
  int co[NB];
  float wsg[NB], wsu[NB];
  const size_t sb = ((size_t)g * (I >> 7) + (n0 >> 7)) * (size_t)(H >> 7);
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const int ch = min(ln + 64 * c, nch - 1);
    co[c] = 32 * ch;
    wsg[c] = w.gs[sb + (ch >> 2)];
    wsu[c] = w.us[sb + (ch >> 2)];
  }
  const uint8_t* gqb = w.gq + ((size_t)g * I + n0) * rowq;
  const uint8_t* uqb = w.uq + ((size_t)g * I + n0) * rowq;
  uint4 pg[DEPTH][NB][2], pu[DEPTH][NB][2];
  int dep = 0;
#define BEF_GU8_LOAD(SLOT, ROW)                                                           \
  _Pragma("unroll") for (int c = 0; c < NB; ++c) {                                        \
    pg[SLOT][c][0] = *reinterpret_cast<const uint4*>(gqb + (ROW) * rowq + co[c] + dep);   \
    pg[SLOT][c][1] = *reinterpret_cast<const uint4*>(gqb + (ROW) * rowq + co[c] + 16 + dep); \
    pu[SLOT][c][0] = *reinterpret_cast<const uint4*>(uqb + (ROW) * rowq + co[c] + dep);   \
    pu[SLOT][c][1] = *reinterpret_cast<const uint4*>(uqb + (ROW) * rowq + co[c] + 16 + dep); \
  }
#pragma unroll
  for (int d = 0; d + 1 < DEPTH; ++d) {
    BEF_GU8_LOAD(d, d)
  }
  uint4 aq[NB][2];
  float xs_raw[NB];
  asm volatile("" ::: "memory");
  acts(aq, xs_raw);
  Act16 a0[NB], a1[NB];
  float sg[NB], su[NB];
  float part[2 * RUN];
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    if (i + DEPTH - 1 < RUN) {
      BEF_GU8_LOAD((i + DEPTH - 1) % DEPTH, i + DEPTH - 1)
    }
    if (i == 0) {
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        e4m3x16_to_h2(aq[c][0], a0[c]);
        e4m3x16_to_h2(aq[c][1], a1[c]);
        const float xsc = (lane + 64 * c < nch) ? xs_raw[c] : 0.0f;
        sg[c] = xsc * wsg[c];
        su[c] = xsc * wsu[c];
      }
    }
    const int sl = i % DEPTH;
    float ag = 0.0f, au = 0.0f;
#pragma unroll
    for (int c = 0; c < NB; ++c) {
      ag += dot32_fp8(pg[sl][c][0], pg[sl][c][1], a0[c], a1[c]) * sg[c];
      au += dot32_fp8(pu[sl][c][0], pu[sl][c][1], a0[c], a1[c]) * su[c];
    }
    part[i] = ag;
    part[RUN + i] = au;
    asm volatile("" : "+v"(dep) : "v"(ag), "v"(au));
  }
#undef BEF_GU8_LOAD
  const float tot = butterfly8(part);
  const float up = xchg32(tot);
  return silu_mul_accurate(tot, up);
}

// The same with the activation codes and scales already in registers.
template <int NB>
struct ActRegs {
  const uint4 (&aq)[NB][2];
  const float (&xs)[NB];
  __device__ __forceinline__ void operator()(uint4 (&q)[NB][2], float (&s)[NB]) const {
#pragma unroll
    for (int c = 0; c < NB; ++c) q[c][0] = aq[c][0], q[c][1] = aq[c][1], s[c] = xs[c];
  }
};
template <int NB, int DEPTH = 2>
__device__ __forceinline__ float gate_up_rows(const GUWeights& w, int g, int n0, int lane,
                                              const uint4 (&aq)[NB][2],
                                              const float (&xs_raw)[NB]) {
  return gate_up_rows<NB, DEPTH>(w, g, n0, lane, ActRegs<NB>{aq, xs_raw});
}
template <int NB, int DEPTH = 2>
__device__ __forceinline__ float gate_up_rows_fp8(const GUWeights8& w, int g, int n0, int lane,
                                                  const uint4 (&aq)[NB][2],
                                                  const float (&xs_raw)[NB]) {
  return gate_up_rows_fp8<NB, DEPTH>(w, g, n0, lane, ActRegs<NB>{aq, xs_raw});
}

// The lanes that hold a finished h value after gate_up_rows (bit 5 = 0 and
// bits 2..0 = 0: one per row), and the row n0 + h_row(lane) they hold.
__device__ __forceinline__ bool h_lane(int lane) { return (lane & 39) == 0; }
__device__ __forceinline__ int h_row(int lane) { return (lane >> 3) & 3; }

// The requantisation of h ahead of the down projection, done once, with no
// device-scope fence (on this chip a release fence writes back the whole L2
// of the XCD) and no round trip for the blocks that only write.  h moves
// between blocks through 64-bit atomics, which are coherent across the XCDs:
//  * every block producing rows of (row r, 128-wide block c of h) sends its
//    values out as {kSlotValid, value bits} words (atomic exchange) -- it
//    reads nothing first, so its weight stream starts at once;
//  * the last of the 8 blocks of (r, c) in launch order reads the 128 words
//    (atomic loads) until every one carries kSlotValid -- a bounded wait:
//    past kSpinLimit rounds it flags MOE_STATUS_SYNC_TIMEOUT and carries on
//    --, returns them to zero for the next launch (each slot is written once
//    per launch, so nothing can land after that reset), and writes the E4M3
//    codes and scale with the act_quant rule (s = amax / 448 by IEEE
//    division, code = E4M3(v / s), zero block -> s = 0, code 0; tcti.cn
//    post, section "补齐软件栈缺失": act_quant feeds the FP8/FP4 linears).
// The slots start zeroed (workspace initialisation); after a timeout a late
// write could outlive the reset, so a workspace that reported one must be
// initialised again.
constexpr int kHSlotStride = 4096;   // largest I on the one-token path
constexpr int kHSlotRows = kHSlotRowsHost;   // rows T*k + T of the VALU path
constexpr uint32_t kSpinLimit = 1u << 16;
constexpr uint32_t kStatusSyncTimeout = 2u;  // MOE_STATUS_SYNC_TIMEOUT
constexpr uint64_t kSlotValid = 1ull << 32;
constexpr uint64_t kSlotTagMask = 0xffffffff00000000ull;

struct HExchange {
  uint64_t* slots;     // [kHSlotRows][kHSlotStride] {kSlotValid, value bits} or 0
  float* h;            // [rows][I] plain copy of h (inspection)
  uint8_t* hq;         // [rows][I] E4M3 codes
  float* hs;           // [rows][I/128] scales
  uint32_t* status;
};

// Called by every thread of a block whose waves hold h values hv (in the
// h_lane lanes) for rows n0 .. n0+3 of h row r; the block's rows start at
// n0b.
__device__ __forceinline__ void publish_h(const HExchange& x, float hv, int r, int I, int n0,
                                          int n0b, int tid, int lane) {
  constexpr int kRowsPerBlock = 4 * kGuRun;
  const int c = n0b >> 7;
  unsigned long long* slot = reinterpret_cast<unsigned long long*>(x.slots) + r * kHSlotStride;
  if (h_lane(lane)) {
    const int n = n0 + h_row(lane);
    x.h[(size_t)r * I + n] = hv;
    atomicExch(slot + n, kSlotValid | __float_as_uint(hv));
  }
  if (n0b + kRowsPerBlock != 128 * (c + 1) || tid >= 64) return;
  // the reader: the last block of this 128-wide block of h
  const int n = 128 * c + 2 * tid;
  unsigned long long w0 = 0, w1 = 0;
  uint32_t spins = 0;
  bool ok = false;
  for (;;) {
    if ((w0 & kSlotTagMask) != kSlotValid)
      w0 = __hip_atomic_load(slot + n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((w1 & kSlotTagMask) != kSlotValid)
      w1 = __hip_atomic_load(slot + n + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    ok = (w0 & kSlotTagMask) == kSlotValid && (w1 & kSlotTagMask) == kSlotValid;
    if (__all(ok) || ++spins >= kSpinLimit) break;
    __builtin_amdgcn_s_sleep(1);
  }
  if (!ok) atomicOr(x.status, kStatusSyncTimeout);
  __hip_atomic_store(slot + n, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(slot + n + 1, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const float v0 = __uint_as_float((uint32_t)w0), v1 = __uint_as_float((uint32_t)w1);
  const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
  const float sc = amax / 448.0f;
  uint32_t q = 0;
  if (amax != 0.0f) q = e4m3_pack4(v0 / sc, v1 / sc, 0.0f, 0.0f);
  const size_t e = (size_t)r * I + n;
  reinterpret_cast<uint16_t*>(x.hq + e)[0] = (uint16_t)q;
  if (tid == 0) x.hs[(size_t)r * (I >> 7) + c] = sc;
}

}  // namespace bef
