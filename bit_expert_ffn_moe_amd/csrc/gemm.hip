// gemm.hip -- S5/S6 for many tokens: grouped GEMM on the CDNA4 matrix cores.
//
// Prefill and batched verification are compute-heavy (tcti.cn post, section
// "DeepSeek-V4-Flash的可能性": prefill and decode need different operators);
// tokens are grouped by expert so that each expert's weights stream once for
// all of its tokens (dpshk.com article, section "核心实现三").  The products
// are fp4_gemm (FP8-quantised activation x FP4 packed weight) and fp8_gemm
// (tcti.cn post, section "补齐软件栈缺失"), dequantised inside the MFMA
// (dpshk.com article, section "核心实现四"):
//   v_mfma_scale_f32_16x16x128_f8f6f4, taken transposed: A = weight rows
//   (E2M1 with their UE8M0 scale per 32 K as the hardware A scale, or E4M3
//   with an fp32 128x128 block scale applied below), B = E4M3 token rows.
// The fp32 activation scale (amax/448 per 128 of K) cannot ride in the MFMA
// scale operand, so each 128-deep K step is issued into a fresh result and
// folded into the running sum with one FMA per output: acc += s_x * d (times
// the weight block scale for FP8).  In the transposed form a lane holds 4
// weight rows of one token, so s_x is one value per lane.
//
// Operand layout of the 16x16x128 f8f6f4 MFMA (measured on gfx950 with a
// one-hot probe): lane l supplies row/column l%16; lane group q = l/16 holds
// K = 32q..32q+31 contiguously for an FP4 operand (16 bytes, its UE8M0 scale
// covering exactly those 32), but K = 16q..16q+15 and 64+16q..64+16q+15 for
// an FP8 operand (two 16-byte halves).  The result holds rows 4q..4q+3 of
// column l%16.
//
// Shapes: an expert sees ~200 tokens in a uniformly routed 8192-token
// prefill, so its weights carry ~2x200 flops per byte -- below the chip's
// ~600 flop/byte balance point: the weights must stream from HBM once.  A
// tile is 256 weight rows (gate+up: 128 rows of each matrix for the same 128
// columns of I, so SwiGLU and the per-128 requant of h finish in the tile) x
// TM tokens (256, 128 or 64 by the groups' average size); 8 waves as 2
// (rows) x 4 (tokens).  Per 128-deep K step the block stages its weight rows
// and gathered token rows in LDS with direct global->LDS loads
// (global_load_lds_dwordx4), as many stages as fit (at most 6), each waited
// for explicitly so that the younger stages' loads fly while one is
// multiplied; the 16-byte chunk positions are XOR-swizzled by row so the
// MFMA operand reads are conflict-free.  The per-row scales go to rings of
// their own where they fit (GemmPlan below).
//
// The grid is persistent (one block per CU, two for the small FP4 tiles) and
// XCD-aware: the work items (expert M-tile, N-block), N-blocks of one M-tile
// adjacent, are split into 8 contiguous ranges, one per XCD (block b runs on
// XCD b mod 8).  The blocks of an XCD thus work on neighbouring items
// together: the N-blocks of an M-tile share its token rows in the XCD's L2,
// and the M-tiles of one expert read the same weight rows at about the same
// time, so those stream from HBM about once.
#include <hip/hip_ext.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace bef {

constexpr int kGThreads = 512;


// SwiGLU in the grouped GEMM's epilogue uses the fast exponential and the
// hardware reciprocal (v_rcp_f32, ~1 ulp): h there already carries the
// MFMA's own accumulation error (its 128-term sums are not exactly rounded),
// next to which a few ulp of the SiLU are negligible.  The requantisation of
// h, however, follows the act_quant rule exactly (e4m3_div2).
__device__ __forceinline__ float silu_mul_fast(float g, float u) {
  return g * u * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

__device__ __forceinline__ uint32_t e4m3_1(float v) {
  v = __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xffu;
}

__device__ __forceinline__ uint32_t e4m3_2(float a, float b) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// E4M3 codes (bytes 0 and 1) of fl32(a / s) and fl32(b / s): the act_quant
// rule (IEEE division, then round to nearest even, saturating), without a
// division per element.  With r = v_rcp_f32(s) (within 1 ulp of 1/s), t =
// v * r is within 2^-22 |t| of fl32(v / s); the E4M3 rounding is monotone,
// so when t (1 - 2^-20) and t (1 + 2^-20) get the same code, that is the
// code of fl32(v / s).  Only an element whose bracket holds a rounding
// midpoint (about 2^-16 of them) takes the correctly rounded division; so
// does every element when s is an fp32 subnormal (its reciprocal is then not
// within 1 ulp).
__device__ __forceinline__ uint32_t e4m3_div2(float a, float b, float s, float r) {
  const float ta = a * r, tb = b * r;
  const float dn = 1.0f - 0x1p-20f, up = 1.0f + 0x1p-20f;
  const uint32_t lo = e4m3_2(ta * dn, tb * dn), hi = e4m3_2(ta * up, tb * up);
  const bool tiny = s < 0x1p-126f;
  if (lo == hi && !tiny) return lo;
  const uint32_t ca = ((lo ^ hi) & 0xffu) || tiny ? e4m3_1(a / s) : (lo & 0xffu);
  const uint32_t cb = ((lo ^ hi) & 0xff00u) || tiny ? e4m3_1(b / s) : (lo >> 8);
  return ca | (cb << 8);
}

// LDS byte offset of 16-byte chunk c of row r: rows of 128 bytes (E4M3, one
// K step) swizzle by bits 3..1 of r, rows of 64 bytes (E2M1) by bits 2..1.
// Measured with the fragment read (rows r = lane mod 16, chunk lane / 16,
// ds_read_b128): both run at ~142 B/clk per CU, while 64-byte rows unswizzled
// or swizzled by bits 3..2 reach only ~116 (bank conflicts).
__device__ __forceinline__ int sw128(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }
__device__ __forceinline__ int sw64(int r, int c) { return r * 64 + ((c ^ ((r >> 1) & 3)) << 4); }

// ---------------------------------------------------------------------------
// The kernel.  Tile: 256 weight rows (gate+up: rows nb*128 .. +127 of W_gate
// then the same rows of W_up; down: rows nb*256 .. +255 of W_down) x 256
// tokens of one group.  The product is taken transposed, D[n][t] =
// sum_k W[n][k] X[t][k]: the weights are the MFMA's A operand (FP4 with its
// UE8M0 scale as the hardware A scale, or FP8), the activations its B
// operand, so a lane holds 4 consecutive weight rows of one token and the
// token's activation scale is one value per lane.  8 waves as 2 (weight
// rows) x 4 (tokens), 128 x 64 outputs each: weight fragments i = 0..7 are,
// for gate+up, gate rows 64 wn + 16 i (i < 4) and the same up rows (i >= 4),
// so SwiGLU pairs stay in one lane; for down, rows 128 wn + 16 i.
// ---------------------------------------------------------------------------
constexpr int kTN2 = 256;   // weight rows per tile

// TM = tokens per tile (256, or 128 / 64 when groups are small): wave tile
// 128 weight rows x TM/4 tokens.  FP4 tiles of 64 tokens, and the FP4 down
// tiles of 128, run two blocks per CU (their registers fit four waves per
// SIMD and their stages half of the LDS): two independent pipelines, whose
// barriers do not hold each other up (measured: 32-token verify step -6%,
// 4096-token FP4 prefill -4% when both of its GEMMs ran so).  The FP4
// gate+up tiles of 128 tokens run one block per CU since the scale rings
// below, which need the registers of two waves per SIMD (4096-token FP4
// prefill gate+up -6% against two blocks per CU without them).  The FP8
// stages are too large for two blocks.
constexpr bool gemm_two_per_cu(int fmt, int tm, bool gu) {
  return fmt == 1 && (tm <= 64 || (tm == 128 && !gu));
}

// Per-tile LDS plan.  Stages: as many as fit in ~156 KB of LDS (~76 KB with
// two blocks per CU), at most 6.  Scale rings: the scales are tiny next to
// the codes (4 bytes per weight row or token per K step) but each comes
// from its own 128-byte line (a row's scales are K/32 bytes, a token's K/32
// as well), and those lines fell out of L2 between K steps: per-step 4-byte
// scale loads cost the 4096-token FP4 gate+up's loads about 30% of their
// time.  With the rings the FP4 weight scales (RW) and the activation scales
// (RX) leave the stages for two buffers of their own, filled a few K steps
// ahead with the scales of four K steps per row in one 16-byte load when K
// is a multiple of 512 (else of one step), so each line is fetched about a
// quarter as often.  Used where the registers allow: at one block per CU
// where the rings fit beside the same number of stages, and at two blocks
// per CU for the 64-token FP4 tiles (two stages instead of three; 32-token
// verify: gate+up -14%, down -11%) and the 128-token FP4 down tiles
// (4096-token FP4 prefill down -7%).  The 128-token FP4 gate+up tiles at two
// blocks per CU spilled address registers inside the K loop with them (hence
// one block per CU for those).
template <int FMT, bool GU, int TM>
struct GemmPlan {
  static constexpr bool kTwo = gemm_two_per_cu(FMT, TM, GU);
  static constexpr int KB_A = TM * 128;                           // E4M3 activations per K step
  static constexpr int KB_B = FMT == 1 ? kTN2 * 64 : kTN2 * 128;  // weight codes per K step
  static constexpr int kStage = KB_A + KB_B + (FMT == 1 ? kTN2 * 4 : 0) + TM * 4;
  static constexpr int kLdsBudget = kTwo ? 77568 : 159744;
  static constexpr int NST0 = (kLdsBudget / kStage) > 6 ? 6 : (kLdsBudget / kStage);
  static constexpr int kTotalLds = kTwo ? 81920 : 163840;
  static constexpr int kMisc = 12 * TM + 1576 + 512;  // the kernel's small arrays, and slack
  static constexpr int kCodes = KB_A + KB_B;
  static constexpr int kRingW = FMT == 1 ? 2 * kTN2 * 16 : 0, kRingX = 2 * TM * 16;
  static constexpr int NSTR0 = (kTotalLds - kRingW - kRingX - kMisc) / kCodes;
  static constexpr int NSTR = NSTR0 < NST0 ? NSTR0 : NST0;  // stages beside the rings
  static constexpr bool kRings = (!kTwo || TM == 64 || !GU) && NSTR >= 2 && (NSTR == NST0 || kTwo);
  static constexpr bool RX = kRings, RW = kRings && FMT == 1;
  static constexpr int NST = kRings ? NSTR : NST0;
};

template <int FMT, bool GU, int TM, bool SS4>
__global__ __launch_bounds__(kGThreads, gemm_two_per_cu(FMT, TM, GU) ? 4 : 2) void gemm_kernel(
    GemmArgs a) {
  using P = GemmPlan<FMT, GU, TM>;
  constexpr int NT = TM / 64;  // token fragments per wave
  constexpr int KB_A = P::KB_A, KB_B = P::KB_B, NST = P::NST;
  constexpr bool RX = P::RX, RW = P::RW;
  static_assert(NST >= 2, "LDS stages");
  constexpr int XL = TM / 8;                               // act-scale DMA lanes per wave
  constexpr int NAI = KB_A / 8192;                         // A DMA instructions per wave
  constexpr int NBI = KB_B / 8192;                         // B DMA instructions per wave
  constexpr int kLoads = NAI + NBI + (FMT == 1 && !RW ? 1 : 0) + (RX ? 0 : 1);  // + scales in the stage
  // stage buffers: activation codes, weight codes, FP4 weight scales (4
  // UE8M0 bytes per weight row), activation scales of the K step
#define BEF_STAGE(i)                                                        \
  __shared__ __align__(16) uint8_t sA##i[NST > i ? KB_A : 16];              \
  __shared__ __align__(16) uint8_t sB##i[NST > i ? KB_B : 16];              \
  __shared__ __align__(16) uint32_t sS##i[FMT == 1 && !RW && NST > i ? kTN2 : 4]; \
  __shared__ __align__(16) float sX##i[!RX && NST > i ? TM : 4];
  BEF_STAGE(0) BEF_STAGE(1) BEF_STAGE(2) BEF_STAGE(3) BEF_STAGE(4) BEF_STAGE(5)
#undef BEF_STAGE
  __shared__ __align__(16) uint32_t sRW[RW ? 2 * kTN2 * 4 : 4];  // [buffer][row][4 K steps]
  __shared__ __align__(16) float sRX[RX ? 2 * TM * 4 : 4];       // [buffer][token][4 K steps]
  __shared__ float s_amax[2][TM];
  __shared__ float s_wsc[2][64];  // FP8 weight block scales of the tile, per K step
  __shared__ int s_mtp[258];      // m-tile prefix per group
  __shared__ int s_tok[TM];
  __shared__ int stmp[kGThreads / 64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = w & 1, wt = w >> 1, q = lane >> 4;
  const int E = a.E, H = a.H, I = a.I;
  const int K = GU ? H : I;  // contraction length
  const int KS = K >> 7;
  // N-blocks per M-tile.  For down, H may end in half an N-block (H = 128
  // mod 256): that block's second 128 weight rows are clamped to row H-1 in
  // the loads and never stored.
  const int NB = GU ? (I >> 7) : ((H + kTN2 - 1) / kTN2);

  // m-tiles per group and their exclusive prefix (groups 0..E, E = shared)
  {
    int my_mt = 0;
    if (tid <= E && (!a.group_mask || a.group_mask[tid])) {
      const int c = a.offsets[tid + 1] - a.offsets[tid];
      my_mt = (c + TM - 1) / TM;
    }
    int inc = my_mt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int t = __shfl_up(inc, d, kWave);
      if (lane >= d) inc += t;
    }
    if (lane == 63) stmp[w] = inc;
    __syncthreads();
    int base = 0, total = 0;
#pragma unroll
    for (int i = 0; i < kGThreads / 64; ++i) {
      base += (i < w) ? stmp[i] : 0;
      total += stmp[i];
    }
    if (tid <= E) s_mtp[tid] = base + inc - my_mt;
    if (tid == 0) s_mtp[E + 1] = total;
    __syncthreads();
  }
  const int total_mt = s_mtp[E + 1];
  const int W = total_mt * NB;
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3, per_xcd = gridDim.x >> 3;
  const int w_lo = (int)(((long long)xcd * W) >> 3), w_hi = (int)(((long long)(xcd + 1) * W) >> 3);

  for (int wi = w_lo + local; wi < w_hi; wi += per_xcd) {
    // work item -> (group, M-tile, N-block).  A group's items are
    // consecutive; within it the N-blocks of an M-tile are adjacent (they
    // share its token rows) -- except for the FP4 gate+up in a group of
    // several M-tiles, where the M-tiles of an N-block are adjacent instead,
    // so that the blocks streaming the same weight rows run side by side and
    // share them in L2 (4096-token FP4 prefill: gate+up -2.9%; the same order
    // for down slowed the 8192-token FP8 prefill by 2%, and its gate+up
    // gained nothing)
    constexpr bool kMFirst = GU && FMT == 1;
    const int mt0 = __builtin_amdgcn_readfirstlane(wi / NB);
    int lo = 0, hi = E + 2;  // first index with s_mtp > mt0
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_mtp[mid] <= mt0) lo = mid + 1; else hi = mid;
    }
    const int g = __builtin_amdgcn_readfirstlane(lo - 1);
    const int nmt = kMFirst ? __builtin_amdgcn_readfirstlane(s_mtp[g + 1] - s_mtp[g]) : 1;
    const int loc = __builtin_amdgcn_readfirstlane(wi - s_mtp[g] * NB);
    const int nb = kMFirst ? __builtin_amdgcn_readfirstlane(loc / nmt) : wi - mt0 * NB;
    const int mtg = kMFirst ? __builtin_amdgcn_readfirstlane(s_mtp[g] + loc - nb * nmt) : mt0;
    const int row0 = __builtin_amdgcn_readfirstlane(a.offsets[g] + (mtg - s_mtp[g]) * TM);
    const int nrows = __builtin_amdgcn_readfirstlane(min(TM, a.offsets[g + 1] - row0));
    if (GU) {
      for (int i = tid; i < TM; i += kGThreads) s_tok[i] = a.row_token[row0 + min(i, nrows - 1)];
      __syncthreads();
    }

    // ---- DMA sources of this tile (K offset 0): a wave-uniform base and a
    // 32-bit per-lane offset ----
    const uint8_t* baseA = GU ? a.xq : a.hq + (size_t)row0 * I;
    uint32_t offA[NAI];
#pragma unroll
    for (int i = 0; i < NAI; ++i) {
      const int p = (w * NAI + i) * 64 + lane, r = p >> 3, c = (p & 7) ^ ((r >> 1) & 7);
      const int rr = min(r, nrows - 1);
      offA[i] = (GU ? (uint32_t)s_tok[rr] * (uint32_t)H : (uint32_t)rr * (uint32_t)I) + 16u * c;
    }
    const uint32_t brow_bytes = FMT == 1 ? (uint32_t)(K >> 1) : (uint32_t)K;
    const size_t rows_per_expert = GU ? (size_t)I : (size_t)H;
    const uint8_t* baseG = (GU ? a.gq : a.dq) + (size_t)g * rows_per_expert * brow_bytes;
    const uint8_t* baseU = (GU ? a.uq : a.dq) + (size_t)g * rows_per_expert * brow_bytes;
    const uint32_t row_base = GU ? (uint32_t)nb * 128u : (uint32_t)nb * kTN2;
    uint32_t offB[NBI];
#pragma unroll
    for (int i = 0; i < NBI; ++i) {
      const int p = (w * NBI + i) * 64 + lane;
      const int r = FMT == 1 ? (p >> 2) : (p >> 3);
      const int c = FMT == 1 ? ((p & 3) ^ ((r >> 1) & 3)) : ((p & 7) ^ ((r >> 1) & 7));
      const uint32_t row = GU ? row_base + (uint32_t)(r & 127) : min(row_base + (uint32_t)r, (uint32_t)H - 1u);
      offB[i] = row * brow_bytes + 16u * c;
    }
    // FP4 scales: weight row w*32 + lane (lanes < 32; gate rows are waves 0-3)
    const uint32_t sbytes = (uint32_t)(K >> 5);
    const uint8_t* baseS = nullptr;
    uint32_t offS = 0;
    if (FMT == 1) {
      const uint8_t* sm = (GU && w >= 4) ? (const uint8_t*)a.us : (const uint8_t*)(GU ? a.gs : a.ds);
      baseS = sm + (size_t)g * rows_per_expert * sbytes;
      const int r = w * 32 + (lane & 31);
      offS = (GU ? row_base + (uint32_t)(r & 127) : min(row_base + (uint32_t)r, (uint32_t)H - 1u)) * sbytes;
    }
    // activation scales: token w*XL + lane (lanes < XL)
    const float* baseX = GU ? a.xs : a.hs + (size_t)row0 * KS;
    uint32_t offX;
    {
      const int rr = min(w * XL + (lane & (XL - 1)), nrows - 1);
      offX = (GU ? (uint32_t)s_tok[rr] : (uint32_t)rr) * (uint32_t)KS;
    }
    // FP8 weight block scales of the tile into LDS, once: [0] gate (GU) or
    // rows 0..127 (down), [1] up (GU) or rows 128..255 (down)
    if (FMT == 2) {
      for (int t = tid; t < 2 * KS; t += kGThreads) {
        const int hsel = t >= KS, ks = t - hsel * KS;
        const float* src = GU ? (const float*)(hsel ? a.us : a.gs) + ((size_t)g * (I >> 7) + nb) * KS
                              : (const float*)a.ds + ((size_t)g * (H >> 7) + min(nb * 2 + hsel, (H >> 7) - 1)) * KS;
        s_wsc[hsel][ks] = src[ks];
      }
      __syncthreads();
    }

    // The K steps of a tile run in rotated order, from step ks0 round to
    // ks0 - 1: weight rows H bytes apart (a power of two) read in lockstep
    // at one K offset by the neighbouring tiles of an XCD land on few HBM
    // channels; starting each tile elsewhere spreads them (the order of the
    // per-step fp32 sums changes, nothing else).  The start follows the work
    // item, except in a group of several M-tiles: there it follows (group,
    // N-block), so the M-tiles that stream the same weight rows -- running
    // side by side on one XCD -- read them in step and share them in its L2
    // (4096-token FP4 prefill, whose hot experts and shared expert have many
    // M-tiles: gate+up -2.3%).  Pairs of neighbouring items share a start, so
    // that two N-blocks read a token tile's K steps together (verify_t32 and
    // both prefills: -0.3 to -0.6%).
    const int rot = (s_mtp[g + 1] - s_mtp[g] > 1 ? g * NB + nb : wi) >> 1;
    // (with four K steps per scale load, the start is rounded down to a
    // multiple of 4, so that each group of four steps is contiguous in K)
    constexpr bool ss4 = (RW || RX) && SS4;
    static_assert(!SS4 || RW || RX, "four-step scale loads only with a ring");
    const int ks0 = (int)(((uint32_t)rot * 7u) % (uint32_t)KS) & (ss4 ? ~3 : ~0);
    auto kr = [&](int ks) {
      const int k = ks + ks0;
      return k >= KS ? k - KS : k;
    };
    auto issue = [&](int ks_, uint8_t* sA, uint8_t* sB, uint32_t* sS, float* sX) {
      const uint32_t ks = (uint32_t)kr(ks_);
#pragma unroll
      for (int i = 0; i < NAI; ++i) dma16(baseA, offA[i] + ks * 128u, sA + (w * NAI + i) * 1024);
#pragma unroll
      for (int i = 0; i < NBI; ++i) {
        // weight rows >= 128 of a gate+up tile are up rows: uniform per instruction
        const uint8_t* bb = (GU && (w * NBI + i) * 64 >= 128 * (FMT == 1 ? 4 : 8)) ? baseU : baseG;
        dma16(bb, offB[i] + ks * (FMT == 1 ? 64u : 128u), sB + (w * NBI + i) * 1024);
      }
      if (FMT == 1 && !RW && lane < 32) dma4(baseS, offS + ks * 4u, sS + w * 32);
      if (!RX && lane < XL) dma4((const uint8_t*)baseX, (offX + ks) * 4u, sX + w * XL);
    };
    // the scale rings: the scales of loop steps s .. s+3 (s a multiple of 4)
    // or of step s alone, into buffer (s/4) mod 2 or s mod 2
    auto issue_scales = [&](int s_) {
      const uint32_t k = (uint32_t)kr(s_);
      const int buf = ss4 ? ((s_ >> 2) & 1) : (s_ & 1);
      if (RW && lane < 32) {
        uint32_t* d = sRW + buf * (kTN2 * 4) + (ss4 ? w * 128 : w * 32);
        if (ss4) dma16(baseS, offS + k * 4u, d);
        else dma4(baseS, offS + k * 4u, d);
      }
      if (RX && lane < XL) {
        float* d = sRX + buf * (TM * 4) + (ss4 ? w * XL * 4 : w * XL);
        if (ss4) dma16((const uint8_t*)baseX, (offX + k) * 4u, d);
        else dma4((const uint8_t*)baseX, (offX + k) * 4u, d);
      }
    };
    // the ring slot of row / token i at loop step ks
    auto ring_at = [&](int ks, int i, int n) {
      return ss4 ? ((ks >> 2) & 1) * (n * 4) + i * 4 + (ks & 3) : (ks & 1) * (n * 4) + i;
    };

    v4f_t acc[8][NT];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int ti = 0; ti < NT; ++ti) acc[i][ti] = (v4f_t){0.0f, 0.0f, 0.0f, 0.0f};
    // Token fragments of 16 per wave: NT for a full tile; in a 256-token
    // tile, NT - 1 when the group's rows fit in three quarters of it (each
    // token wave then takes
    // 16 (NT - 1) tokens, so a tile of at most 3/4 TM rows spends a quarter
    // fewer multiplies and token fragment reads, all four SIMDs still
    // equally busy).  A wave whose tokens are all past the group's rows
    // skips the multiplies (the tokens of a partly filled band are
    // multiplied anyway: clamped copies of a real row, never stored).
    const bool part = NT == 4 && nrows <= 64 * (NT - 1);
    const int TS = part ? 16 * (NT - 1) : 16 * NT;  // tokens per token wave
    const bool live = nrows > wt * TS;
    auto wrow = [&](int i) {
      return GU ? ((i < 4 ? 0 : 128) + 64 * wn + 16 * (i & 3) + (lane & 15))
                : (128 * wn + 16 * i + (lane & 15));
    };

    auto compute = [&](auto ntl, int ks, const uint8_t* sA, const uint8_t* sB,
                       const uint32_t* sS, const float* sX) {
      constexpr int NTL = decltype(ntl)::value;  // token fragments of this wave
      if (!live) return;
      auto read_w = [&](int i, v8i_t& wv, int& sw) {
        const int n = wrow(i);
        if (FMT == 1) {
          const uint4 b0 = *reinterpret_cast<const uint4*>(sB + sw64(n, q));
          wv = (v8i_t){(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, 0, 0, 0, 0};
          sw = (int)(((RW ? sRW[ring_at(ks, n, kTN2)] : sS[n]) >> (8 * q)) & 0xffu);
        } else {
          const uint4 b0 = *reinterpret_cast<const uint4*>(sB + sw128(n, q));
          const uint4 b1 = *reinterpret_cast<const uint4*>(sB + sw128(n, q + 4));
          wv = (v8i_t){(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                       (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
          sw = 127;
        }
      };
      // LDS reads in the order of first use (the hardware returns them in
      // order): the scales (a few bytes; the first fold needs them), weight
      // fragment 0, then the wave's 4 token fragments, so that the first
      // MFMA waits only for its own two fragments
      float cx[NTL], cy[NTL];
#pragma unroll
      for (int ti = 0; ti < NTL; ++ti) {
        const int t = wt * 16 * NTL + 16 * ti + (lane & 15);
        const float x = RX ? sRX[ring_at(ks, t, TM)] : sX[t];
        cx[ti] = x;
        cy[ti] = x;
      }
      float f0 = 1.0f, f1 = 1.0f;
      if (FMT == 2) {
        // the FP8 weight block scales: gate / up halves (down: this wave's rows)
        f0 = s_wsc[GU ? 0 : wn][kr(ks)];
        f1 = GU ? s_wsc[1][kr(ks)] : f0;
      }
      v8i_t wv[2];
      int sw[2];
      read_w(0, wv[0], sw[0]);
      v8i_t tv[NTL];
#pragma unroll
      for (int ti = 0; ti < NTL; ++ti) {
        const int r = wt * 16 * NTL + 16 * ti + (lane & 15);
        const uint4 a0 = *reinterpret_cast<const uint4*>(sA + sw128(r, q));
        const uint4 a1 = *reinterpret_cast<const uint4*>(sA + sw128(r, q + 4));
        tv[ti] = (v8i_t){(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                         (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      }
      if (FMT == 2) {
#pragma unroll
        for (int ti = 0; ti < NTL; ++ti) {
          cy[ti] = cx[ti] * f1;
          cx[ti] = cx[ti] * f0;
        }
      }
      const v4f_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        // fragment i+1 is read while fragment i multiplies
        if (i + 1 < 8) read_w(i + 1, wv[(i + 1) & 1], sw[(i + 1) & 1]);
        v4f_t d[NTL];
#pragma unroll
        for (int ti = 0; ti < NTL; ++ti)
          d[ti] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              wv[i & 1], tv[ti], zero, FMT == 1 ? 4 : 0, 0, 0, sw[i & 1], 0, 127);
#pragma unroll
        for (int ti = 0; ti < NTL; ++ti) {
          const float c = (GU && i >= 4) ? cy[ti] : cx[ti];
          acc[i][ti][0] = fmaf(c, d[ti][0], acc[i][ti][0]);
          acc[i][ti][1] = fmaf(c, d[ti][1], acc[i][ti][1]);
          acc[i][ti][2] = fmaf(c, d[ti][2], acc[i][ti][2]);
          acc[i][ti][3] = fmaf(c, d[ti][3], acc[i][ti][3]);
        }
      }
    };

    // ---- K loop: NST stages.  Step ks waits for its own DMA of stage ks
    // (the younger stages' loads may stay in flight), passes a barrier --
    // after which the stage is complete and every wave is done with step
    // ks-1 --, issues step ks+NST-1 into step ks-1's stage, then
    // multiplies. ----
    struct Stage {
      uint8_t* a;
      uint8_t* b;
      uint32_t* s;
      float* x;
    };
    auto stage = [&](int i) -> Stage {
      switch (i) {
        case 0: return {sA0, sB0, sS0, sX0};
        case 1: return {sA1, sB1, sS1, sX1};
        case 2: return {sA2, sB2, sS2, sX2};
        case 3: return {sA3, sB3, sS3, sX3};
        case 4: return {sA4, sB4, sS4, sX4};
        default: return {sA5, sB5, sS5, sX5};
      }
    };
    // wait until at most `newer` stages of this wave's loads are in flight
    auto wait_stages = [&](int newer) {
      switch (newer) {
        case 0: __builtin_amdgcn_s_waitcnt(waitcnt_vm(0)); break;
        case 1: __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLoads)); break;
        case 2: __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * kLoads)); break;
        case 3: __builtin_amdgcn_s_waitcnt(waitcnt_vm(3 * kLoads)); break;
        default: __builtin_amdgcn_s_waitcnt(waitcnt_vm(4 * kLoads)); break;
      }
    };
    if (RW || RX) issue_scales(0);
#pragma unroll
    for (int i = 0; i < NST - 1; ++i) {
      if (i < KS) {
        const Stage st = stage(i);
        issue(i, st.a, st.b, st.s, st.x);
      }
    }
    // the loop, for NTL token fragments per wave.  (Measured on the
    // compiler at hand: the 256-token tile runs faster with its two loops in
    // a generic lambda, the smaller tiles, with one loop, without: written
    // once as a macro, it serves both.)
#define BEF_KLOOP(NTL)                                                      \
  for (int kb = 0; kb < KS; kb += NST) {                                    \
    _Pragma("unroll") for (int j = 0; j < NST; ++j) {                       \
      const int ks = kb + j;                                                \
      if (ks < KS) {                                                        \
        wait_stages(min(NST - 2, KS - 1 - ks));                             \
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);                             \
        block_barrier();                                                    \
        if (RW || RX) {                                                     \
          if (ss4) {                                                        \
            if ((ks & 3) == 1 && ks + 3 < KS) issue_scales(ks + 3);         \
          } else if (ks + 1 < KS) {                                         \
            issue_scales(ks + 1);                                           \
          }                                                                 \
        }                                                                   \
        if (ks + NST - 1 < KS) {                                            \
          const Stage nx = stage((j + NST - 1) % NST);                      \
          issue(ks + NST - 1, nx.a, nx.b, nx.s, nx.x);                      \
        }                                                                   \
        const Stage cu = stage(j);                                          \
        compute(std::integral_constant<int, NTL>{}, ks, cu.a, cu.b, cu.s, cu.x); \
      }                                                                     \
    }                                                                       \
  }
    if constexpr (NT == 4) {
      auto kloop = [&](auto ntl) { BEF_KLOOP(decltype(ntl)::value) };
      if (part)
        kloop(std::integral_constant<int, 3>{});
      else
        kloop(std::integral_constant<int, 4>{});
    } else {
      BEF_KLOOP(NT)
    }
#undef BEF_KLOOP
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    block_barrier();

    if (GU) {
      // ---- epilogue: h = silu(g) * u for the lane's token (16 ti + lane%16)
      // and h columns 64 wn + 16 i + 4 q + v; per-token amax over the tile's
      // 128 columns (4 lanes of a column group, then the 2 column waves),
      // E4M3 codes and scale (the act_quant rule) ----
      // h overwrites the gate accumulators: acc[i][ti][v], i < 4
      float m[NT];
#pragma unroll
      for (int ti = 0; ti < NT; ++ti) m[ti] = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int ti = 0; ti < NT; ++ti)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            acc[i][ti][v] = silu_mul_fast(acc[i][ti][v], acc[i + 4][ti][v]);
            m[ti] = fmaxf(m[ti], fabsf(acc[i][ti][v]));
          }
#pragma unroll
      for (int ti = 0; ti < NT; ++ti) {
        m[ti] = fmaxf(m[ti], __shfl_xor(m[ti], 16, kWave));
        m[ti] = fmaxf(m[ti], __shfl_xor(m[ti], 32, kWave));
        if (q == 0 && (!part || ti < NT - 1)) s_amax[wn][wt * TS + 16 * ti + lane] = m[ti];
      }
      __syncthreads();
      uint8_t* s_out = sA0;  // [token][128 codes]
      const int I128 = I >> 7;
#pragma unroll
      for (int ti = 0; ti < NT; ++ti) {
        if (part && ti == NT - 1) continue;
        const int t = wt * TS + 16 * ti + (lane & 15);
        const float am = fmaxf(s_amax[0][t], s_amax[1][t]);
        const float sc = am / 448.0f;
        const float rsc = __builtin_amdgcn_rcpf(sc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t cw = 0;
          if (am != 0.0f) {
            cw = e4m3_div2(acc[i][ti][0], acc[i][ti][1], sc, rsc) |
                 (e4m3_div2(acc[i][ti][2], acc[i][ti][3], sc, rsc) << 16);
          }
          *reinterpret_cast<uint32_t*>(&s_out[t * 128 + 64 * wn + 16 * i + 4 * q]) = cw;
          if (a.h_dbg && t < nrows)
            *reinterpret_cast<float4*>(a.h_dbg + (size_t)(row0 + t) * I + nb * 128 + 64 * wn +
                                       16 * i + 4 * q) =
                make_float4(acc[i][ti][0], acc[i][ti][1], acc[i][ti][2], acc[i][ti][3]);
        }
        if (wn == 0 && q == 0 && t < nrows) a.hs[(size_t)(row0 + t) * I128 + nb] = sc;
      }
      __syncthreads();
      for (int t = tid; t < TM * 8; t += kGThreads) {
        const int R = t >> 3, c16 = t & 7;
        if (R < nrows)
          *reinterpret_cast<uint4*>(a.hq + (size_t)(row0 + R) * I + nb * 128 + 16 * c16) =
              *reinterpret_cast<const uint4*>(&s_out[R * 128 + 16 * c16]);
      }
      __syncthreads();
    } else {
#pragma unroll
      for (int ti = 0; ti < NT; ++ti) {
        const int t = wt * TS + 16 * ti + (lane & 15);
        if (live && (!part || ti < NT - 1) && t < nrows && nb * kTN2 + 128 * wn < H) {
          float* yp = a.y_rows + (size_t)(row0 + t) * H + nb * kTN2 + 128 * wn + 4 * q;
#pragma unroll
          for (int i = 0; i < 8; ++i)
            *reinterpret_cast<float4*>(yp + 16 * i) =
                make_float4(acc[i][ti][0], acc[i][ti][1], acc[i][ti][2], acc[i][ti][3]);
        }
      }
    }
  }
}

// Blocks of the persistent grid: one per CU, a multiple of 8 (the XCDs).
static int g_cu_count[64];

static int grid_blocks() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  if (g_cu_count[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
      (void)hipGetLastError();
      n = 256;
    }
    g_cu_count[dev] = n >= 8 ? (n & ~7) : 8;
  }
  return g_cu_count[dev];
}

template <int FMT, bool GU, int TM, bool SS4>
static hipError_t launch_g4(const GemmArgs& a, hipStream_t st) {
  const KernelTimer& tm = g_kernel_timer[GU ? MOE_KERNEL_GEMM_GATE_UP : MOE_KERNEL_GEMM_DOWN];
  const dim3 grid((gemm_two_per_cu(FMT, TM, GU) ? 2 : 1) * grid_blocks());
  if (tm.start)
    hipExtLaunchKernelGGL(gemm_kernel<FMT, GU, TM, SS4>, grid, dim3(kGThreads), 0, st, tm.start,
                          tm.stop, 0, a);
  else
    gemm_kernel<FMT, GU, TM, SS4><<<grid, dim3(kGThreads), 0, st>>>(a);
  return hipGetLastError();
}

// with scale rings, the contraction length decides their form: four K
// steps per scale load when it is a multiple of 512
template <int FMT, bool GU, int TM>
static hipError_t launch_g(const GemmArgs& a, hipStream_t st) {
  if (a.E + 1 > 257 || (GU ? a.I : a.H) % 128 != 0) return hipErrorInvalidValue;
  using P = GemmPlan<FMT, GU, TM>;
  if constexpr (P::RW || P::RX) {
    if ((GU ? a.H : a.I) % 512 == 0) return launch_g4<FMT, GU, TM, true>(a, st);
  }
  return launch_g4<FMT, GU, TM, false>(a, st);
}

// Token tile by the routed groups' average size: 256 from 128 rows (each
// expert's weights then stream once for all of its tokens), 128 from 32,
// else 64 (small stages: more K steps in flight while little multiplies).
template <bool GU>
static hipError_t launch_gg(const GemmArgs& a, hipStream_t st) {
  const int64_t rows = (int64_t)a.T * a.k;
  const int tm = rows >= (int64_t)128 * a.E ? 256 : rows >= (int64_t)32 * a.E ? 128 : 64;
  if (a.fmt == 1) {
    if (tm == 256) return launch_g<1, GU, 256>(a, st);
    if (tm == 128) return launch_g<1, GU, 128>(a, st);
    return launch_g<1, GU, 64>(a, st);
  }
  if (tm == 256) return launch_g<2, GU, 256>(a, st);
  if (tm == 128) return launch_g<2, GU, 128>(a, st);
  return launch_g<2, GU, 64>(a, st);
}

hipError_t launch_gemm_gate_up(const GemmArgs& a, hipStream_t st) { return launch_gg<true>(a, st); }

hipError_t launch_gemm_down(const GemmArgs& a, hipStream_t st) { return launch_gg<false>(a, st); }

}  // namespace bef
