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

namespace bef {

struct GUWeights {
  const uint8_t *gq, *gs, *uq, *us;
  int E, H, I;
};

// Loads a 32-code E4M3 chunk and converts it to fp16 pairs.
__device__ __forceinline__ void load_act32(const uint8_t* __restrict__ p, Act16& a0, Act16& a1) {
  const uint4 q0 = *reinterpret_cast<const uint4*>(p);
  const uint4 q1 = *reinterpret_cast<const uint4*>(p + 16);
  e4m3x16_to_h2(q0, a0);
  e4m3x16_to_h2(q1, a1);
}

// This lane's activation chunks from already-quantised codes and scales.
template <int NB>
__device__ __forceinline__ void act_from_codes(const uint8_t* __restrict__ xq_row,
                                               const float* __restrict__ xs_row, int H, int lane,
                                               Act16 (&a0)[NB], Act16 (&a1)[NB],
                                               float (&xsc)[NB]) {
  const int nch = H >> 5;
#pragma unroll
  for (int c = 0; c < NB; ++c) {
    const int ch = lane + 64 * c;
    if (ch < nch) {
      load_act32(xq_row + 32 * ch, a0[c], a1[c]);
      xsc[c] = xs_row[ch >> 2];
    } else {
      xsc[c] = 0.0f;
      e4m3x16_to_h2(make_uint4(0, 0, 0, 0), a0[c]);
      e4m3x16_to_h2(make_uint4(0, 0, 0, 0), a1[c]);
    }
  }
}

// This lane's activation chunks quantised on the fly from the bf16 row, with
// exactly the act_quant rule: the 128-block of chunk ch is spread over the 4
// lanes 4j..4j+3 (ch = 4j..4j+3), so its amax is a 4-lane max; s = amax/448
// (IEEE division), code = E4M3(x/s), a zero block gives s = 0 and code 0.
// Requires H/32 to be a multiple of 4 per 64-lane pass (H % 128 == 0).
template <int NB>
__device__ __forceinline__ void act_from_bf16(const uint16_t* __restrict__ x_row, int H, int lane,
                                              Act16 (&a0)[NB], Act16 (&a1)[NB],
                                              float (&xsc)[NB]) {
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
    e4m3x16_to_h2(q0, a0[c]);
    e4m3x16_to_h2(q1, a1[c]);
    xsc[c] = (ch < nch) ? sc : 0.0f;
  }
}

// Streams 8 consecutive rows n0.. of group g's gate and up matrices for one
// activation row with a DEPTH-deep register pipeline (the loads of row
// i+DEPTH-1 are in flight while row i is multiplied), keeping each row's
// per-lane partial sums; one butterfly reduce-scatter then gives every lane
// one of the 16 totals (8 gate, 8 up), and 8 lanes finish
// h[n] = silu(g_n) * u_n in parallel (returned in those lanes).
template <int NB, int DEPTH>
__device__ __forceinline__ float gate_up_rows(const GUWeights& w, int g, int n0, int lane,
                                              const Act16 (&a0)[NB], const Act16 (&a1)[NB],
                                              const float (&xsc)[NB]) {
  constexpr int RUN = 8;
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
#define BEF_GU_LOAD(SLOT, ROW)                                                      \
  _Pragma("unroll") for (int c = 0; c < NB; ++c) {                                  \
    pg[SLOT][c] = *reinterpret_cast<const uint4*>(gqb + (ROW) * rowq + co[c]);      \
    pu[SLOT][c] = *reinterpret_cast<const uint4*>(uqb + (ROW) * rowq + co[c]);      \
    psg[SLOT][c] = gsb[(ROW) * rows_ + cs[c]];                                      \
    psu[SLOT][c] = usb[(ROW) * rows_ + cs[c]];                                      \
  }
#pragma unroll
  for (int d = 0; d < DEPTH - 1; ++d) {
    BEF_GU_LOAD(d, d)
  }
  float part[2 * RUN];  // [0..7] gate rows, [8..15] up rows
#pragma unroll
  for (int i = 0; i < RUN; ++i) {
    if (i + DEPTH - 1 < RUN) {
      BEF_GU_LOAD((i + DEPTH - 1) % DEPTH, i + DEPTH - 1)
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
    // keep the next row's loads from being hoisted above this row's math: the
    // pipeline then holds DEPTH rows, not the whole run, and the arithmetic of
    // early rows overlaps the transfer of later ones
    __builtin_amdgcn_sched_barrier(0);
  }
#undef BEF_GU_LOAD
  const float tot = butterfly16(part);  // j = 8*bit5 + 4*bit4 + 2*bit3 + bit2
  const float up = xchg32(tot);         // lanes with bit5 = 0 receive the same row's up total
  return silu_mul_accurate(tot, up);    // valid in h_lane() lanes
}

// The lanes that hold a finished h value after gate_up_rows (bit 5 = 0 and
// bits 1..0 = 0: one per row), and the row n0 + h_row(lane) they hold.
__device__ __forceinline__ bool h_lane(int lane) { return (lane & 35) == 0; }
__device__ __forceinline__ int h_row(int lane) { return (lane >> 2) & 7; }

// The requantisation of h ahead of the down projection, done once, with no
// device-scope fence (on this chip a release fence writes back the whole L2
// of the XCD).  h moves between blocks only through 64-bit atomic
// read-modify-writes, which are coherent across the XCDs:
//  * each block that has finished rows n0b .. n0b+31 of h row r takes a
//    ticket from the arrival counter of the 128-wide block n0b / 128; the 4
//    tickets of one launch share tag = ticket / 4 + 1 (never 0; the slots
//    start zeroed);
//  * its 32 values go out as {tag, value bits} words (atomic exchange);
//  * the block that drew the 4th ticket reads the 128 words (atomic or with
//    0) until every tag is its own -- a bounded wait: past kSpinLimit
//    rounds it flags MOE_STATUS_SYNC_TIMEOUT and carries on -- and writes
//    the E4M3 codes and scale with the act_quant rule (s = amax / 448 by IEEE
//    division, code = E4M3(v / s), zero block -> s = 0, code 0; dpshk.com
//    article, section "核心实现二").
// Slots have a fixed row stride of kHSlotStride so that a slot always
// belongs to the same counter, whatever I a call uses.
constexpr int kHSlotStride = 4096;   // largest I on the one-token path
constexpr int kHSlotRows = 8;
constexpr uint32_t kSpinLimit = 1u << 16;
constexpr uint32_t kStatusSyncTimeout = 2u;  // MOE_STATUS_SYNC_TIMEOUT

struct HExchange {
  uint32_t* arrive;    // [kHSlotRows][kHSlotStride / 128] tickets
  uint64_t* slots;     // [kHSlotRows][kHSlotStride] {tag, value bits}
  float* h;            // [rows][I] plain copy of h (inspection)
  uint8_t* hq;         // [rows][I] E4M3 codes
  float* hs;           // [rows][I/128] scales
  uint32_t* status;
};

__device__ __forceinline__ void publish_h(const HExchange& x, float hv, int r, int I, int n0,
                                          int n0b, int tid, int lane, uint32_t* s_ticket) {
  constexpr uint32_t kBlocks = 128 / 32;
  const int c = n0b >> 7;
  __syncthreads();  // readers of the previous ticket are done with it
  if (tid == 0) *s_ticket = atomicAdd(x.arrive + r * (kHSlotStride / 128) + c, 1u);
  __syncthreads();
  const uint32_t ticket = *s_ticket;
  const uint64_t tag = (uint64_t)(ticket / kBlocks + 1) << 32;
  unsigned long long* slot = reinterpret_cast<unsigned long long*>(x.slots) + r * kHSlotStride;
  if (h_lane(lane)) {
    const int n = n0 + h_row(lane);
    x.h[(size_t)r * I + n] = hv;
    atomicExch(slot + n, tag | __float_as_uint(hv));
  }
  if (ticket % kBlocks == kBlocks - 1 && tid < 64) {
    const int n = 128 * c + 2 * tid;
    unsigned long long w0 = 0, w1 = 0;
    uint32_t spins = 0;
    bool ok = false;
    for (;;) {
      if ((w0 & 0xffffffff00000000ull) != tag) w0 = atomicOr(slot + n, 0ull);
      if ((w1 & 0xffffffff00000000ull) != tag) w1 = atomicOr(slot + n + 1, 0ull);
      ok = (w0 & 0xffffffff00000000ull) == tag && (w1 & 0xffffffff00000000ull) == tag;
      if (__all(ok) || ++spins >= kSpinLimit) break;
      __builtin_amdgcn_s_sleep(1);
    }
    if (!ok) atomicOr(x.status, kStatusSyncTimeout);
    const float v0 = __uint_as_float((uint32_t)w0), v1 = __uint_as_float((uint32_t)w1);
    const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
    const float sc = amax / 448.0f;
    uint32_t q = 0;
    if (amax != 0.0f) q = e4m3_pack4(v0 / sc, v1 / sc, 0.0f, 0.0f);
    const size_t e = (size_t)r * I + n;
    reinterpret_cast<uint16_t*>(x.hq + e)[0] = (uint16_t)q;
    if (tid == 0) x.hs[(size_t)r * (I >> 7) + c] = sc;
  }
}

}  // namespace bef
