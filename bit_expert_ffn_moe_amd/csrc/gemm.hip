// gemm.hip -- S5/S6 for many tokens: grouped GEMM on the CDNA4 matrix cores.
//
// Prefill and batched verification are compute-heavy (tcti.cn post, section
// "DeepSeek-V4-Flash的可能性": prefill and decode need different operators);
// tokens are grouped by expert so that each expert's weights stream once for
// all of its tokens (dpshk.com article, section "核心实现三").  The products
// are fp4_gemm (FP8-quantised activation x FP4 packed weight) and fp8_gemm
// (tcti.cn post, section "补齐软件栈缺失"), dequantised inside the MFMA
// (dpshk.com article, section "核心实现四"):
//   v_mfma_scale_f32_16x16x128_f8f6f4, A = E4M3 activations (scale 2^0),
//   B = E2M1 weights with their UE8M0 scale per 32 K as the hardware B scale
//   (FP4), or B = E4M3 weights (FP8, fp32 block scale applied below).
// The fp32 activation scale (amax/448 per 128 of K) cannot ride in the MFMA
// scale operand, so each 128-deep K step is issued into a fresh result and
// folded into the running sum with one FMA per output: acc += s_x * d (times
// the weight block scale for FP8).
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
// tile is 128 tokens x 256 output columns (gate+up: 128 columns of I for both
// matrices, so SwiGLU and the per-128 requant of h finish in the tile); 4
// waves, one per SIMD, as 2 (M) x 2 (N), 64 x 128 outputs each (128 fp32
// accumulators per lane, up to 512 registers per wave).  Per 128-deep K step
// the block stages its A rows (gathered token rows) and B rows (weight rows)
// in LDS with direct global->LDS loads (global_load_lds_dwordx4), three
// stages deep in separate LDS objects so that the compiler's wait tracking
// lets the next stages' loads fly while one is multiplied; the 16-byte chunk
// positions are XOR-swizzled by row so the MFMA operand reads are
// conflict-free.
//
// The grid is persistent (one block per CU) and XCD-aware: the work items
// (expert M-tile, N-block), N-blocks of one M-tile adjacent, are split into 8
// contiguous ranges, one per XCD (block b runs on XCD b mod 8).  The 32
// blocks of an XCD thus work on neighbouring items together: the N-blocks of
// an M-tile share its activation rows in the XCD's L2, and the M-tiles of
// one expert (16 items apart for I = 2048) read the same weight rows at the
// same time, so those stream from HBM about once.
#include <hip/hip_ext.h>

#include "common.h"
#include "kernels.h"

namespace bef {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* glb_ptr_t;

constexpr int kTM = 128;      // tokens per tile
constexpr int kTN = 256;      // output columns per tile
constexpr int kGThreads = 512;

// s_waitcnt immediates (gfx9: vmcnt [3:0] + [15:14], expcnt [6:4], lgkmcnt [11:8])
constexpr int waitcnt_vm(int n) { return 0xF70 | (n & 0xF) | ((n >> 4) << 14); }
constexpr int kWaitLgkm0 = 0xC07F;

// Workgroup barrier that is also a compiler barrier for memory accesses: the
// s_barrier builtin is modelled as touching no memory, so LDS reads could be
// moved across it; an asm statement with a memory clobber cannot be.  (It
// waits for nothing: the callers wait for their own loads explicitly.)
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

__device__ __forceinline__ void dma16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((glb_ptr_t)g, (lds_ptr_t)l, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds((glb_ptr_t)g, (lds_ptr_t)l, 4, 0, 0);
}

// SwiGLU and requantisation in the grouped GEMM's epilogue use the fast
// exponential and reciprocals: h there already carries the MFMA's own
// accumulation error (its 128-term sums are not exactly rounded), next to
// which a few ulp of the SiLU and of v * (1/s) instead of v / s are
// negligible.  The one-token GEMV keeps the IEEE forms (its h is exact to
// fp32 rounding).
__device__ __forceinline__ float silu_mul_fast(float g, float u) {
  return g * u * __frcp_rn(1.0f + __expf(-g));
}

__device__ __forceinline__ uint32_t e4m3_1(float v) {
  v = __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xffu;
}

// LDS byte offset of 16-byte chunk c of row r: rows of 128 bytes (E4M3, one
// K step) swizzle by bits 3..1 of r, rows of 64 bytes (E2M1) by bits 3..2.
__device__ __forceinline__ int sw128(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }
__device__ __forceinline__ int sw64(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }

template <int FMT>
struct StageBytes {
  static constexpr int kB = FMT == 1 ? kTN * 64 : kTN * 128;
};

// GU = gate+up (+SwiGLU, requant of h), else down.
template <int FMT, bool GU>
__global__ __launch_bounds__(kGThreads) void gemm_kernel(GemmArgs a) {
  constexpr int KB = StageBytes<FMT>::kB;
  constexpr int NAI = 2;                 // A DMA instructions per wave per K step
  constexpr int NBI = FMT == 1 ? 2 : 4;  // B DMA instructions per wave per K step
  constexpr int kLoads = NAI + NBI + (FMT == 1 ? 2 : 1);  // DMA instructions per wave per stage
  __shared__ __align__(16) uint8_t sA0[kTM * 128];
  __shared__ __align__(16) uint8_t sA1[kTM * 128];
  __shared__ __align__(16) uint8_t sA2[kTM * 128];
  __shared__ __align__(16) uint8_t sB0[KB];
  __shared__ __align__(16) uint8_t sB1[KB];
  __shared__ __align__(16) uint8_t sB2[KB];
  __shared__ __align__(16) uint32_t sS0[FMT == 1 ? kTN : 1];  // FP4: 4 UE8M0 bytes per B row
  __shared__ __align__(16) uint32_t sS1[FMT == 1 ? kTN : 1];
  __shared__ __align__(16) uint32_t sS2[FMT == 1 ? kTN : 1];
  __shared__ __align__(16) float sX0[kTM];  // activation scales of the K step
  __shared__ __align__(16) float sX1[kTM];
  __shared__ __align__(16) float sX2[kTM];
  __shared__ float s_amax[4][kTM];
  __shared__ float s_wsc[2][64];  // FP8 weight block scales of the tile, per K step
  __shared__ int s_mtp[258];  // m-tile prefix per group
  __shared__ int s_tok[kTM];
  __shared__ int stmp[kGThreads / 64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w & 1, wn = w >> 1, q = lane >> 4;  // 2 (M) x 4 (N) waves of 64 x 64
  const int E = a.E, H = a.H, I = a.I;
  const int K = GU ? H : I;  // contraction length
  const int KS = K >> 7;
  const int NB = GU ? (I >> 7) : (H / kTN);  // N-blocks per M-tile

  // m-tiles per group and their exclusive prefix (groups 0..E, E = shared)
  {
    int my_mt = 0;
    if (tid <= E) {
      const int c = a.offsets[tid + 1] - a.offsets[tid];
      my_mt = (c + kTM - 1) / kTM;
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
    const int mtg = __builtin_amdgcn_readfirstlane(wi / NB);
    const int nb = __builtin_amdgcn_readfirstlane(wi - mtg * NB);
    int lo = 0, hi = E + 2;  // first index with s_mtp > mtg
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (s_mtp[mid] <= mtg) lo = mid + 1; else hi = mid;
    }
    // block-uniform values in scalar registers (scalar loads of the scales)
    const int g = __builtin_amdgcn_readfirstlane(lo - 1);
    const int row0 = __builtin_amdgcn_readfirstlane(a.offsets[g] + (mtg - s_mtp[g]) * kTM);
    const int nrows = __builtin_amdgcn_readfirstlane(min(kTM, a.offsets[g + 1] - row0));
    if (GU) {
      for (int i = tid; i < kTM; i += kGThreads) s_tok[i] = a.row_token[row0 + min(i, nrows - 1)];
      __syncthreads();
    }

    // ---- DMA sources of this tile (K offset 0): a wave-uniform 64-bit base
    // (scalar registers) and a 32-bit per-lane offset ----
    const uint8_t* baseA = GU ? a.xq : a.hq + (size_t)row0 * I;
    uint32_t offA[NAI];
#pragma unroll
    for (int i = 0; i < NAI; ++i) {
      const int p = (w * NAI + i) * 64 + lane, r = p >> 3, c = (p & 7) ^ ((r >> 1) & 7);
      const int rr = min(r, nrows - 1);
      offA[i] = (GU ? (uint32_t)s_tok[rr] * (uint32_t)H : (uint32_t)rr * (uint32_t)I) + 16u * c;
    }
    const uint32_t brow_bytes = FMT == 1 ? (uint32_t)(K >> 1) : (uint32_t)K;
    // B row r of the tile: gate rows 0..127 and up rows 128..255 of I-block
    // nb (gate+up), or rows nb*256 + r of W_down (down)
    const size_t rows_per_expert = GU ? (size_t)I : (size_t)H;
    const uint8_t* baseG = (GU ? a.gq : a.dq) + (size_t)g * rows_per_expert * brow_bytes;
    const uint8_t* baseU = (GU ? a.uq : a.dq) + (size_t)g * rows_per_expert * brow_bytes;
    const uint32_t row_base = GU ? (uint32_t)nb * 128u : (uint32_t)nb * kTN;
    uint32_t offB[NBI];
#pragma unroll
    for (int i = 0; i < NBI; ++i) {
      const int p = (w * NBI + i) * 64 + lane;
      const int r = FMT == 1 ? (p >> 2) : (p >> 3);
      const int c = FMT == 1 ? ((p & 3) ^ ((r >> 2) & 3)) : ((p & 7) ^ ((r >> 1) & 7));
      offB[i] = (row_base + (uint32_t)(GU ? (r & 127) : r)) * brow_bytes + 16u * c;
    }
    // FP4 scales: B row w*32 + lane (lanes < 32; uniform matrix per wave)
    const uint32_t sbytes = (uint32_t)(K >> 5);
    const uint8_t* baseS = nullptr;
    uint32_t offS = 0;
    if (FMT == 1) {
      const uint8_t* sm = (GU && w >= 4) ? (const uint8_t*)a.us : (const uint8_t*)(GU ? a.gs : a.ds);
      baseS = sm + (size_t)g * rows_per_expert * sbytes;
      const int r = w * 32 + (lane & 31);
      offS = (row_base + (uint32_t)(GU ? (r & 127) : r)) * sbytes;
    }
    // activation scales: A row w*16 + lane (lanes < 16)
    const float* baseX = GU ? a.xs : a.hs + (size_t)row0 * KS;
    uint32_t offX;
    {
      const int rr = min(w * 16 + (lane & 15), nrows - 1);
      offX = (GU ? (uint32_t)s_tok[rr] : (uint32_t)rr) * (uint32_t)KS;
    }
    // FP8 weight block scales of the tile into LDS, once: [0] gate (GU) or
    // columns 0..127 (down), [1] up (GU) or columns 128..255 (down)
    if (FMT == 2) {
      for (int t = tid; t < 2 * KS; t += kGThreads) {
        const int hsel = t >= KS, ks = t - hsel * KS;
        const float* src = GU ? (const float*)(hsel ? a.us : a.gs) + ((size_t)g * (I >> 7) + nb) * KS
                              : (const float*)a.ds + ((size_t)g * (H >> 7) + nb * 2 + hsel) * KS;
        s_wsc[hsel][ks] = src[ks];
      }
      __syncthreads();
    }

    // The K steps of a tile run in rotated order, from step ks0 round to
    // ks0 - 1: weight rows H bytes apart (a power of two) read in lockstep
    // at one K offset by the neighbouring tiles of an XCD land on few HBM
    // channels; starting each tile elsewhere spreads them (the order of the
    // per-step fp32 sums changes, nothing else).
    const int ks0 = (int)(((uint32_t)wi * 7u) % (uint32_t)KS);
    auto kr = [&](int ks) {
      const int k = ks + ks0;
      return k >= KS ? k - KS : k;
    };
    auto issue = [&](int ks_, uint8_t* sA, uint8_t* sB, uint32_t* sS, float* sX) {
      const uint32_t ks = (uint32_t)kr(ks_);
#pragma unroll
      for (int i = 0; i < NAI; ++i) dma16(baseA + (offA[i] + ks * 128u), sA + (w * NAI + i) * 1024);
#pragma unroll
      for (int i = 0; i < NBI; ++i) {
        // B rows >= 128 of a gate+up tile are up rows: uniform per instruction
        const uint8_t* bb = (GU && (w * NBI + i) * 64 >= 128 * (FMT == 1 ? 4 : 8)) ? baseU : baseG;
        dma16(bb + (offB[i] + ks * (FMT == 1 ? 64u : 128u)), sB + (w * NBI + i) * 1024);
      }
      if (FMT == 1 && lane < 32) dma4(baseS + (offS + ks * 4u), sS + w * 32);
      if (lane < 16) dma4(baseX + (offX + ks), sX + w * 16);
    };

    v4f_t acc[4][4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[mi][j] = (v4f_t){0.0f, 0.0f, 0.0f, 0.0f};
    // a wave whose 64 rows hold no token skips the multiplies (the rows of a
    // partly filled 64-row band are multiplied anyway: clamped copies of a
    // real row, never stored)
    const bool live = nrows > wm * 64;

    // one K step's operands of this wave, read from a stage into registers
    v8i_t f_av[4], f_bv[4];
    int f_sb[4];
    float4 f_xs[4];
    auto read_frags = [&](const uint8_t* sA, const uint8_t* sB, const uint32_t* sS,
                          const float* sX) {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int r = wm * 64 + 16 * mi + (lane & 15);
        const uint4 a0 = *reinterpret_cast<const uint4*>(sA + sw128(r, q));
        const uint4 a1 = *reinterpret_cast<const uint4*>(sA + sw128(r, q + 4));
        f_av[mi] = (v8i_t){(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                           (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        f_xs[mi] = *reinterpret_cast<const float4*>(sX + wm * 64 + 16 * mi + 4 * q);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // sub-tile j: gate+up -- j < 2 gate, j >= 2 up, I-columns
        // 32 wn + 16 (j & 1) + (lane & 15) of the block; down -- H-columns
        // 64 wn + 16 j + (lane & 15)
        const int n = GU ? ((j < 2 ? 0 : 128) + 32 * wn + 16 * (j & 1) + (lane & 15))
                         : (64 * wn + 16 * j + (lane & 15));
        if (FMT == 1) {
          const uint4 b0 = *reinterpret_cast<const uint4*>(sB + sw64(n, q));
          f_bv[j] = (v8i_t){(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, 0, 0, 0, 0};
          f_sb[j] = (int)((sS[n] >> (8 * q)) & 0xffu);
        } else {
          const uint4 b0 = *reinterpret_cast<const uint4*>(sB + sw128(n, q));
          const uint4 b1 = *reinterpret_cast<const uint4*>(sB + sw128(n, q + 4));
          f_bv[j] = (v8i_t){(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w,
                            (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
          f_sb[j] = 127;
        }
      }
    };
    auto mma = [&](int ks) {
      // activation scales times the FP8 weight block scale (gate / up halves)
      float f0 = 1.0f, f1 = 1.0f;
      if (FMT == 2) {
        f0 = s_wsc[GU ? 0 : (wn >> 1)][kr(ks)];
        f1 = GU ? s_wsc[1][kr(ks)] : f0;
      }
      const v4f_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
      // sub-tile j+1's MFMAs are issued before sub-tile j's scale FMAs, so
      // the FMAs never wait on a result just issued (two result sets live)
      v4f_t d[2][4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        d[0][mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
            f_av[mi], f_bv[0], zero, 0, FMT == 1 ? 4 : 0, 0, 127, 0, f_sb[0]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (j + 1 < 4) {
#pragma unroll
          for (int mi = 0; mi < 4; ++mi)
            d[(j + 1) & 1][mi] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                f_av[mi], f_bv[j + 1], zero, 0, FMT == 1 ? 4 : 0, 0, 127, 0, f_sb[j + 1]);
        }
        __builtin_amdgcn_sched_barrier(0);
        const float fj = (GU && j >= 2) ? f1 : f0;
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const v4f_t& dd = d[j & 1][mi];
          acc[mi][j][0] = fmaf(FMT == 2 ? f_xs[mi].x * fj : f_xs[mi].x, dd[0], acc[mi][j][0]);
          acc[mi][j][1] = fmaf(FMT == 2 ? f_xs[mi].y * fj : f_xs[mi].y, dd[1], acc[mi][j][1]);
          acc[mi][j][2] = fmaf(FMT == 2 ? f_xs[mi].z * fj : f_xs[mi].z, dd[2], acc[mi][j][2]);
          acc[mi][j][3] = fmaf(FMT == 2 ? f_xs[mi].w * fj : f_xs[mi].w, dd[3], acc[mi][j][3]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };

    // ---- K loop, two wave groups in ping-pong: waves 0-3 (one per SIMD)
    // and waves 4-7 run half a step apart, so that one group reads its
    // operands from LDS while the other multiplies from registers.  Per step
    // ks a wave passes barrier 1, issues the DMA of step ks+2 into the stage
    // every wave has finished reading, reads stage ks, waits for its own DMA
    // of step ks+1, passes barrier 2 and multiplies.  Group 1 starts one
    // barrier late; at every barrier both groups have waited for the DMA of
    // the stage read next, and the stage refilled next was read by both
    // before the previous barrier. ----
    const bool grp1 = w >= 4;
    issue(0, sA0, sB0, sS0, sX0);
    if (KS > 1) issue(1, sA1, sB1, sS1, sX1);
    if (KS > 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLoads));
    else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    if (grp1) block_barrier();
#define BEF_GEMM_STEP(KS_, SA, SB, SS, SX, NA, NB_, NS, NX)                   \
    {                                                                        \
      block_barrier();                                                       \
      if ((KS_) + 2 < KS) issue((KS_) + 2, NA, NB_, NS, NX);                 \
      if (live) read_frags(SA, SB, SS, SX);                                  \
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);                                \
      if ((KS_) + 2 < KS) __builtin_amdgcn_s_waitcnt(waitcnt_vm(kLoads));    \
      else __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));                        \
      block_barrier();                                                       \
      if (live) mma((KS_));                                                  \
    }
    for (int ks = 0; ks < KS; ks += 3) {
      BEF_GEMM_STEP(ks, sA0, sB0, sS0, sX0, sA2, sB2, sS2, sX2)
      if (ks + 1 >= KS) break;
      BEF_GEMM_STEP(ks + 1, sA1, sB1, sS1, sX1, sA0, sB0, sS0, sX0)
      if (ks + 2 >= KS) break;
      BEF_GEMM_STEP(ks + 2, sA2, sB2, sS2, sX2, sA1, sB1, sS1, sX1)
    }
#undef BEF_GEMM_STEP
    if (!grp1) block_barrier();
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    block_barrier();

    if (GU) {
      // ---- epilogue: h = silu(g) * u, per-row amax over the tile's 128
      // columns of I, E4M3 codes and scale (the act_quant rule) ----
      float hv[4][2][4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            hv[mi][jj][v] = silu_mul_fast(acc[mi][jj][v], acc[mi][jj + 2][v]);
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float m = fmaxf(fabsf(hv[mi][0][v]), fabsf(hv[mi][1][v]));
          m = group_max<16>(m);
          const int R = wm * 64 + 16 * mi + 4 * q + v;
          if ((lane & 15) == 0) s_amax[wn][R] = m;
        }
      __syncthreads();
      uint8_t* s_out = sA0;
      const int I128 = I >> 7;
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int R = wm * 64 + 16 * mi + 4 * q + v;
          const float am = fmaxf(fmaxf(s_amax[0][R], s_amax[1][R]), fmaxf(s_amax[2][R], s_amax[3][R]));
          const float sc = am / 448.0f;
          const float rsc = __frcp_rn(sc);
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int col = 32 * wn + 16 * jj + (lane & 15);
            s_out[R * 128 + col] = (uint8_t)((am != 0.0f) ? e4m3_1(hv[mi][jj][v] * rsc) : 0u);
          }
          if (wn == 0 && (lane & 15) == 0 && R < nrows)
            a.hs[(size_t)(row0 + R) * I128 + nb] = sc;
        }
      __syncthreads();
      for (int t = tid; t < kTM * 8; t += kGThreads) {
        const int R = t >> 3, c16 = t & 7;
        if (R < nrows)
          *reinterpret_cast<uint4*>(a.hq + (size_t)(row0 + R) * I + nb * 128 + 16 * c16) =
              *reinterpret_cast<const uint4*>(&s_out[R * 128 + 16 * c16]);
      }
      __syncthreads();
    } else {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int R = wm * 64 + 16 * mi + 4 * q + v;
          if (R < nrows) {
            float* yp = a.y_rows + (size_t)(row0 + R) * H + nb * kTN + 64 * wn + (lane & 15);
#pragma unroll
            for (int j = 0; j < 4; ++j) yp[16 * j] = acc[mi][j][v];
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

template <int FMT, bool GU>
static hipError_t launch_g(const GemmArgs& a, hipStream_t st) {
  if (a.E + 1 > 257 || (GU ? (a.I % 128) : (a.H % kTN)) != 0) return hipErrorInvalidValue;
  const KernelTimer& tm = g_kernel_timer[MOE_KERNEL_GEMM_GATE_UP];
  if (GU && tm.start)
    hipExtLaunchKernelGGL(gemm_kernel<FMT, GU>, dim3(grid_blocks()), dim3(kGThreads), 0, st,
                          tm.start, tm.stop, 0, a);
  else
    gemm_kernel<FMT, GU><<<dim3(grid_blocks()), dim3(kGThreads), 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_gemm_gate_up(const GemmArgs& a, hipStream_t st) {
  if (a.fmt == 1) return launch_g<1, true>(a, st);
  return launch_g<2, true>(a, st);
}

hipError_t launch_gemm_down(const GemmArgs& a, hipStream_t st) {
  if (a.fmt == 1) return launch_g<1, false>(a, st);
  return launch_g<2, false>(a, st);
}

}  // namespace bef
