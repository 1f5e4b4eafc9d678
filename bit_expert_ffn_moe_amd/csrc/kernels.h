// kernels.h -- launchers of the gfx950 kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace bef {

constexpr int kRouteSmallT = 4;           // router: per-chunk blocks + last-block top-k
constexpr int kRouteMaxGroups = 32;       // router: 256-row groups, H <= 8192
constexpr int kRouteSplitT = 256;         // router: experts also split in quarters below this T
constexpr int kRouteMfmaRows = 512;       // router from kRouteSplitT tokens: rows per group sum
constexpr int kPermuteSmallPairs = 2048;  // permute: single block up to this many pairs
constexpr int kPermuteTokBlock = 256;     // permute: tokens per block above that
constexpr int kGemvMaxRows = 8;           // VALU GEMV path: rows (k + 1) per token
constexpr int kGemvMaxT = 4;              // VALU GEMV path: at most this many tokens
constexpr int kHSlotRowsHost = 32;        // VALU GEMV path: rows T*(k+1) (h exchange slots)
constexpr uint32_t MOE_STATUS_BAD_EXPERT_ID_DEV = 1u;

// Optional start/stop events of one kernel's launches (debug timing; set by
// moe_debug_time_kernel, index MOE_KERNEL_*).
struct KernelTimer {
  hipEvent_t start, stop;
};
extern KernelTimer g_kernel_timer[6];

struct GemvArgs {
  const uint8_t *gq, *gs, *uq, *us, *dq, *ds;
  const uint8_t* xq;
  const float* xs;
  const int4* active;      // set: {group, first row, end row} per slot
  const int32_t *offsets, *row_token, *row_of;
  const float* topk_w;
  int E, H, I, k, n_slots;
  float* h;
  float* y_rows;
  void* out;
  int out_bf16;
  uint8_t* hq_ws;
  float* hs_ws;
  uint64_t* h_slots;    // tagged slots of the h exchange (zero between launches)
  uint32_t* status;
  int n_rows;           // down with an active list: T*k + T rows, the last T the shared ones
  int fmt;              // 1: FP4 weights, 2: FP8
  int T;                // tokens
  const uint8_t* group_mask;  // [E+1] or null: groups with 0 are skipped (no active list)
};

struct GemmArgs {
  int fmt;
  const uint8_t *gq, *uq, *dq;
  const void *gs, *us, *ds;
  const uint8_t* xq;
  const float* xs;
  const int32_t *offsets, *row_token;
  int T, k, E, H, I;
  uint8_t* hq;
  float* hs;
  float* y_rows;
  float* h_dbg;   // debug: fp32 h [T*k+T][I] of the gate+up kernels when set
  const uint8_t* group_mask;  // [E+1] or null: groups with 0 are skipped
};

// The one-token fused expert kernel (decode.hip): 16 output rows per block
// (one block per CU), 12 waves, at most 8 h rows (k + 1).
constexpr int kDecRowsPerBlock = 16;
constexpr int kDecWaves = 12;
constexpr int kDecMaxRows = 8;
struct DecodeArgs {
  const uint8_t *gq, *gs, *uq, *us, *dq, *ds;  // FP4 weights [E+1][...]
  const uint8_t* xq;          // the token's E4M3 codes [H] and scales [H/128]
  const float* xs;
  const int4* active;         // routed slots {group, row, row + 1} (rows 0 .. k-1)
  const int32_t* row_of;      // [k+1]: h row of rank j, then the shared row
  const float* topk_w;        // [k]
  int E, H, I, k;
  float* h;                   // [k+1][I] fp32 h (inspection)
  uint8_t* hq;                // [k+1][I] requantised h (row k: the shared expert's, read)
  float* hs;                  // [k+1][I/128]
  uint64_t* dec_h;            // WsCtl::dec_h, dec_c, dec_epoch, dec_done
  uint64_t* dec_c;
  uint32_t* epoch;
  uint32_t* done;
  uint32_t* cnt;              // [8][16] published gate+up units per 128-block
  uint32_t* status;
  void* out;                  // [H] f32 or bf16
  int out_bf16;
};
bool decode_ffn_fits(int fmt, int T, int k, int H, int I);
hipError_t launch_decode_ffn(const DecodeArgs& a, hipStream_t st);

// Debug sink of the grouped GEMM's fp32 h (moe_debug_store_h).
struct HSink {
  float* h;
  size_t n;
};
extern HSink g_h_sink;

// Small-T front of the layer: router (+ act_quant of x when xq is set,
// + permutation tables when offsets is set).
struct WsCtl;
struct FrontArgs {
  const uint16_t* x;
  const uint16_t* wr;
  int T, H, E, k;
  uint64_t* slots;        // [H/256][T][E] tagged group sums (zero between launches)
  int32_t* ids;
  float* w;
  uint8_t* xq;
  float* xs;
  int32_t *offsets, *row_token, *row_of;
  int4* active;           // routed groups {group, first row, end row}, -1 padded
  int n_active_slots;
  // shared expert's gate+up rows run in the same kernel when sh_h is set
  // (fmt 1: FP4 weights, 2: FP8)
  const uint8_t *sh_gq, *sh_gs, *sh_uq, *sh_us;
  int fmt;
  int I;
  float* sh_h;
  uint8_t* sh_hq;         // requantised h (rows of the shared expert)
  float* sh_hs;
  uint64_t* h_slots;
  uint32_t* status;
};
void set_route_sync(FrontArgs& a, WsCtl* ctl);
hipError_t launch_route_front(const FrontArgs& a, hipStream_t st);

hipError_t launch_act_quant(const void* x, bool bf16, int64_t rows, int32_t cols, uint8_t* q,
                            float* s, hipStream_t st);
// T > kRouteSmallT needs gsum: (H/256) * T * E floats of workspace (group sums;
// from kRouteSplitT tokens on, H/kRouteMfmaRows of them are used), and from
// kRouteSplitT tokens on wrT: E * H bf16 (the router matrix transposed).
// xq/xs set: the act_quant of x runs in the same launch (T > kRouteSmallT) or
// in the front kernel (T <= kRouteSmallT).
hipError_t launch_route(const uint16_t* x, const uint16_t* wr, int T, int H, int E, int k,
                        int32_t* ids, float* w, WsCtl* ctl, float* gsum, uint16_t* wrT,
                        hipStream_t st, uint8_t* xq = nullptr, float* xs = nullptr);
hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* offsets,
                          int32_t* row_token, int32_t* row_of, int32_t* cnt,
                          uint32_t* status, hipStream_t st);
hipError_t launch_combine(const float* y, const int32_t* row_of, const float* topk_w, int T, int k,
                          int H, void* out, bool bf16, hipStream_t st);
hipError_t launch_gemv_gate_up(const GemvArgs& a, hipStream_t st);
hipError_t launch_gemv_down(const GemvArgs& a, bool combine, hipStream_t st);
hipError_t launch_gemm_gate_up(const GemmArgs& a, hipStream_t st);
hipError_t launch_gemm_down(const GemmArgs& a, hipStream_t st);
hipError_t launch_zero_words(uint32_t* p, int n, hipStream_t st);

}  // namespace bef
