// gemm.hip -- S5/S6 for many tokens: grouped GEMM on the CDNA4 matrix cores.
//
// Prefill and batched verification are compute-bound (tcti.cn post, section
// "DeepSeek-V4-Flash的可能性": prefill and decode need different operators);
// tokens are grouped by expert so that each expert's weights stream once for
// all of its tokens (dpshk.com article, section "核心实现三").  The products
// are fp4_gemm (FP8-quantised activation x FP4 packed weight) and fp8_gemm
// (tcti.cn post, section "补齐软件栈缺失"), dequantised inside the MFMA
// (dpshk.com article, section "核心实现四"):
//   v_mfma_scale_f32_16x16x128_f8f6f4, A = E4M3 activations (scale 2^0),
//   B = E2M1 weights with their UE8M0 scale per 32 K as the hardware B scale
//   (FP4), or B = E4M3 weights (FP8, block scale applied below).
// The fp32 activation scale (amax/448 per 128 of K) cannot ride in the MFMA
// scale operand, so each 128-deep K step is issued into a fresh accumulator
// and folded into the running sum with one FMA per output: acc += s_x * d
// (times the fp32 weight block scale for FP8).
//
// Operand layout of the 16x16x128 f8f6f4 MFMA (measured on gfx950 with a
// one-hot probe): lane l supplies row/column l%16; lane group q = l/16 holds
// K = 32q..32q+31 contiguously for an FP4 operand (16 bytes, its UE8M0 scale
// covering exactly those 32), but K = 16q..16q+15 and 64+16q..64+16q+15 for
// an FP8 operand (two 16-byte halves).  The result holds rows 4q..4q+3 of
// column l%16.
//
// Tile: BM tokens x BN columns, K step 128, 256 threads = 4 waves, wave w
// owning BN/4 columns for all BM rows.  A (gathered token rows) is staged in
// LDS, double buffered, with the 16-byte chunk index XOR-swizzled by row so
// the MFMA operand reads are conflict-free; B is read straight from HBM into
// registers (each lane's 16 or 32 bytes are contiguous in a weight row) and
// prefetched one K step ahead.  A group's tiles are found from the offsets
// table inside the block; surplus blocks of the upper-bound grid exit.
#include "common.h"
#include "kernels.h"

namespace bef {

__device__ __forceinline__ uint32_t e4m3_1(float v) {
  v = __builtin_amdgcn_fmed3f(v, -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.0f, 0, false) & 0xffu;
}

template <int FMT>
struct BFrag;
template <>
struct BFrag<1> {  // FP4: 16 bytes + one UE8M0 byte per lane
  uint4 q;
  uint32_t s;
};
template <>
struct BFrag<2> {  // FP8: 32 bytes per lane
  uint4 q0, q1;
};

// Main loop shared by both GEMMs.  Rows: a_row[j] points at the token row of
// A chunk j (K offset 0), xs_row at that row's scale row (only threads < BM).
// B: bsrc[j] points at this lane's first bytes of weight row j (K offset 0);
// bscale[j] at its UE8M0 scales (FP4) -- for FP8 wsc[j] points at the fp32
// block scales along K of the column block of sub-tile j.
template <int BM, int NJ, int FMT>
__device__ __forceinline__ void mfma_mainloop(const uint8_t* const (&a_row)[BM / 32],
                                              const int (&a_dst)[BM / 32], const float* xs_row,
                                              const uint8_t* const (&bsrc)[NJ],
                                              const uint8_t* const (&bscale)[NJ],
                                              const float* const (&wsc)[NJ], int KS,
                                              uint8_t (*sA)[BM * 128], float (*sXs)[BM],
                                              v4f_t (&acc)[BM / 16][NJ]) {
  constexpr int MT = BM / 16;
  constexpr int ACH = BM / 32;
  const int tid = threadIdx.x, lane = tid & 63;
  const int kq = lane >> 4;
  uint4 a_stage[ACH];
  float xs_stage = 0.0f;
  BFrag<FMT> bc[NJ], bn[NJ];
  float fc[NJ], fn[NJ];

  auto load_a = [&](int ks) {
#pragma unroll
    for (int j = 0; j < ACH; ++j) a_stage[j] = *reinterpret_cast<const uint4*>(a_row[j] + ks * 128);
    if (tid < BM) xs_stage = xs_row[ks];
  };
  auto store_a = [&](int buf) {
#pragma unroll
    for (int j = 0; j < ACH; ++j) *reinterpret_cast<uint4*>(&sA[buf][a_dst[j]]) = a_stage[j];
    if (tid < BM) sXs[buf][tid] = xs_stage;
  };
  auto load_b = [&](int ks, BFrag<FMT>(&b)[NJ], float(&f)[NJ]) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if constexpr (FMT == 1) {
        b[j].q = *reinterpret_cast<const uint4*>(bsrc[j] + ks * 64);
        b[j].s = bscale[j][ks * 4];
        f[j] = 1.0f;
      } else {
        b[j].q0 = *reinterpret_cast<const uint4*>(bsrc[j] + ks * 128);
        b[j].q1 = *reinterpret_cast<const uint4*>(bsrc[j] + ks * 128 + 64);
        f[j] = wsc[j][ks];
      }
    }
  };

  load_a(0);
  load_b(0, bc, fc);
  store_a(0);
  __syncthreads();
  const v4f_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int ks = 0; ks < KS; ++ks) {
    const int buf = ks & 1;
    const bool more = ks + 1 < KS;
    if (more) {
      load_a(ks + 1);
      load_b(ks + 1, bn, fn);
    }
#pragma unroll
    for (int mi = 0; mi < MT; ++mi) {
      const int r = 16 * mi + (lane & 15);
      const uint8_t* rowp = &sA[buf][r * 128];
      const uint4 a0 = *reinterpret_cast<const uint4*>(rowp + ((kq ^ (r & 7)) << 4));
      const uint4 a1 = *reinterpret_cast<const uint4*>(rowp + (((kq + 4) ^ (r & 7)) << 4));
      const v8i_t av = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                        (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
      const float4 xsv = *reinterpret_cast<const float4*>(&sXs[buf][16 * mi + 4 * kq]);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        v4f_t d;
        if constexpr (FMT == 1) {
          const v8i_t bv = {(int)bc[j].q.x, (int)bc[j].q.y, (int)bc[j].q.z, (int)bc[j].q.w,
                            0, 0, 0, 0};
          d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, zero, 0, 4, 0, 127, 0,
                                                               (int)bc[j].s);
          acc[mi][j][0] = fmaf(xsv.x, d[0], acc[mi][j][0]);
          acc[mi][j][1] = fmaf(xsv.y, d[1], acc[mi][j][1]);
          acc[mi][j][2] = fmaf(xsv.z, d[2], acc[mi][j][2]);
          acc[mi][j][3] = fmaf(xsv.w, d[3], acc[mi][j][3]);
        } else {
          const v8i_t bv = {(int)bc[j].q0.x, (int)bc[j].q0.y, (int)bc[j].q0.z, (int)bc[j].q0.w,
                            (int)bc[j].q1.x, (int)bc[j].q1.y, (int)bc[j].q1.z, (int)bc[j].q1.w};
          d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, zero, 0, 0, 0, 127, 0, 127);
          const float f = fc[j];
          acc[mi][j][0] = fmaf(xsv.x * f, d[0], acc[mi][j][0]);
          acc[mi][j][1] = fmaf(xsv.y * f, d[1], acc[mi][j][1]);
          acc[mi][j][2] = fmaf(xsv.z * f, d[2], acc[mi][j][2]);
          acc[mi][j][3] = fmaf(xsv.w * f, d[3], acc[mi][j][3]);
        }
      }
    }
    if (more) store_a(buf ^ 1);
    __syncthreads();
    if (more) {
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        bc[j] = bn[j];
        fc[j] = fn[j];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// gate + up + SwiGLU + requantisation of h.  BN = 128 columns of I for both
// gate and up: wave w owns columns 32w..32w+31 of each, as sub-tiles
// j = 0,1 (gate) and j = 2,3 (up) of the same columns, so h = silu(g)*u is
// formed in registers.  A 128-column tile is exactly one quantisation block
// of h, so the E4M3 requantisation (amax/448 per 128, as act_quant) finishes
// inside the tile: per-row max across the 16 lanes of a column group, then
// across the 4 waves through LDS.  grid = (I/128, m-tile slots).
// ---------------------------------------------------------------------------
template <int BM, int FMT>
__global__ __launch_bounds__(256) void gemm_gate_up_kernel(
    const uint8_t* __restrict__ gq, const void* __restrict__ gsv, const uint8_t* __restrict__ uq,
    const void* __restrict__ usv, const uint8_t* __restrict__ xq, const float* __restrict__ xs,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ row_token, int E, int H,
    int I, uint8_t* __restrict__ hq, float* __restrict__ hs) {
  constexpr int MT = BM / 16, ACH = BM / 32, NJ = 4;
  __shared__ int stmp[8];
  __shared__ int s_tok[BM];
  __shared__ __align__(16) uint8_t sA[2][BM * 128];
  __shared__ __align__(16) float sXs[2][BM];
  __shared__ float s_amax[4][BM];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, kq = lane >> 4;
  int mt;
  const int g = find_group_item(
      offsets, E + 1, blockIdx.y, [](int c) { return (c + BM - 1) / BM; }, stmp, &mt);
  if (g < 0) return;
  const int nb = blockIdx.x;
  const int row0 = offsets[g] + mt * BM;
  const int nrows = min(BM, offsets[g + 1] - row0);
  for (int i = tid; i < BM; i += 256) s_tok[i] = row_token[row0 + (i < nrows ? i : 0)];
  __syncthreads();

  const int KS = H >> 7;
  const uint8_t* a_row[ACH];
  int a_dst[ACH];
#pragma unroll
  for (int j = 0; j < ACH; ++j) {
    const int q = tid + 256 * j, row = q >> 3, c16 = q & 7;
    a_row[j] = xq + (size_t)s_tok[row] * H + 16 * c16;
    a_dst[j] = row * 128 + ((c16 ^ (row & 7)) << 4);
  }
  const float* xs_row = xs + (size_t)s_tok[tid < BM ? tid : 0] * KS;

  const uint8_t* bsrc[NJ];
  const uint8_t* bscale[NJ];
  const float* wsc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const uint8_t* mat = (j < 2) ? gq : uq;
    const void* sc = (j < 2) ? gsv : usv;
    const int n = nb * 128 + 32 * wv + 16 * (j & 1) + (lane & 15);
    if constexpr (FMT == 1) {
      bsrc[j] = mat + ((size_t)g * I + n) * (H >> 1) + 16 * kq;
      bscale[j] = reinterpret_cast<const uint8_t*>(sc) + ((size_t)g * I + n) * (H >> 5) + kq;
      wsc[j] = nullptr;
    } else {
      bsrc[j] = mat + ((size_t)g * I + n) * H + 16 * kq;
      bscale[j] = nullptr;
      wsc[j] = reinterpret_cast<const float*>(sc) + ((size_t)g * (I >> 7) + nb) * KS;
    }
  }

  v4f_t acc[MT][NJ];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[mi][j] = (v4f_t){0.0f, 0.0f, 0.0f, 0.0f};
  mfma_mainloop<BM, NJ, FMT>(a_row, a_dst, xs_row, bsrc, bscale, wsc, KS, sA, sXs, acc);

  // epilogue: h, per-row amax over the 128 columns, E4M3 codes
  float hv[MT][2][4];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int v = 0; v < 4; ++v) hv[mi][jj][v] = silu_mul_accurate(acc[mi][jj][v], acc[mi][jj + 2][v]);
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      float m = fmaxf(fabsf(hv[mi][0][v]), fabsf(hv[mi][1][v]));
      m = group_max<16>(m);
      if ((lane & 15) == 0) s_amax[wv][16 * mi + 4 * kq + v] = m;
    }
  __syncthreads();
  uint8_t* s_out = sA[0];
  const int I128 = I >> 7;
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 16 * mi + 4 * kq + v;
      const float am = fmaxf(fmaxf(s_amax[0][row], s_amax[1][row]), fmaxf(s_amax[2][row], s_amax[3][row]));
      const float sc = am / 448.0f;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int col = 32 * wv + 16 * jj + (lane & 15);
        s_out[row * 128 + col] = (uint8_t)((am != 0.0f) ? e4m3_1(hv[mi][jj][v] / sc) : 0u);
      }
      if (wv == 0 && (lane & 15) == 0 && row < nrows) hs[(size_t)(row0 + row) * I128 + nb] = sc;
    }
  __syncthreads();
  for (int q = tid; q < BM * 8; q += 256) {
    const int row = q >> 3, c16 = q & 7;
    if (row < nrows)
      *reinterpret_cast<uint4*>(hq + (size_t)(row0 + row) * I + nb * 128 + 16 * c16) =
          *reinterpret_cast<const uint4*>(&s_out[row * 128 + 16 * c16]);
  }
}

// ---------------------------------------------------------------------------
// down: y_rows[r] = W_down[g] . deq(hq[r]).  Rows of a group are contiguous
// in hq (no gather).  BN columns of H per block, wave w owning BN/4 of them
// as NJ = BN/64 sub-tiles.  grid = (H/BN, m-tile slots).
// ---------------------------------------------------------------------------
template <int BM, int BN, int FMT>
__global__ __launch_bounds__(256) void gemm_down_kernel(
    const uint8_t* __restrict__ dq, const void* __restrict__ dsv, const uint8_t* __restrict__ hq,
    const float* __restrict__ hs, const int32_t* __restrict__ offsets, int E, int H, int I,
    float* __restrict__ y_rows) {
  constexpr int MT = BM / 16, ACH = BM / 32, NJ = BN / 64;
  __shared__ int stmp[8];
  __shared__ __align__(16) uint8_t sA[2][BM * 128];
  __shared__ __align__(16) float sXs[2][BM];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, kq = lane >> 4;
  int mt;
  const int g = find_group_item(
      offsets, E + 1, blockIdx.y, [](int c) { return (c + BM - 1) / BM; }, stmp, &mt);
  if (g < 0) return;
  const int nb = blockIdx.x;
  const int row0 = offsets[g] + mt * BM;
  const int nrows = min(BM, offsets[g + 1] - row0);
  const int KS = I >> 7;

  const uint8_t* a_row[ACH];
  int a_dst[ACH];
#pragma unroll
  for (int j = 0; j < ACH; ++j) {
    const int q = tid + 256 * j, row = q >> 3, c16 = q & 7;
    a_row[j] = hq + (size_t)(row0 + (row < nrows ? row : 0)) * I + 16 * c16;
    a_dst[j] = row * 128 + ((c16 ^ (row & 7)) << 4);
  }
  const int xr = (tid < BM && tid < nrows) ? tid : 0;
  const float* xs_row = hs + (size_t)(row0 + xr) * KS;

  const uint8_t* bsrc[NJ];
  const uint8_t* bscale[NJ];
  const float* wsc[NJ];
  int cols[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = nb * BN + (BN / 4) * wv + 16 * j + (lane & 15);
    cols[j] = c;
    if constexpr (FMT == 1) {
      bsrc[j] = dq + ((size_t)g * H + c) * (I >> 1) + 16 * kq;
      bscale[j] = reinterpret_cast<const uint8_t*>(dsv) + ((size_t)g * H + c) * (I >> 5) + kq;
      wsc[j] = nullptr;
    } else {
      bsrc[j] = dq + ((size_t)g * H + c) * I + 16 * kq;
      bscale[j] = nullptr;
      wsc[j] = reinterpret_cast<const float*>(dsv) + ((size_t)g * (H >> 7) + (c >> 7)) * KS;
    }
  }
  v4f_t acc[MT][NJ];
#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[mi][j] = (v4f_t){0.0f, 0.0f, 0.0f, 0.0f};
  mfma_mainloop<BM, NJ, FMT>(a_row, a_dst, xs_row, bsrc, bscale, wsc, KS, sA, sXs, acc);

#pragma unroll
  for (int mi = 0; mi < MT; ++mi)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int row = 16 * mi + 4 * kq + v;
      if (row < nrows) {
        float* yp = y_rows + (size_t)(row0 + row) * H;
#pragma unroll
        for (int j = 0; j < NJ; ++j) yp[cols[j]] = acc[mi][j][v];
      }
    }
}

int gemm_mtile_slots(int T, int k, int E, int BM) {
  const long long routed = (long long)T * k;
  const long long partial = routed < E ? routed : E;
  return (int)(routed / BM + partial + (T + BM - 1) / BM + 1);
}

template <int BM, int FMT>
static hipError_t launch_gu(const GemmArgs& a, hipStream_t st) {
  const dim3 grid(a.I / 128, gemm_mtile_slots(a.T, a.k, a.E, BM));
  gemm_gate_up_kernel<BM, FMT><<<grid, 256, 0, st>>>(a.gq, a.gs, a.uq, a.us, a.xq, a.xs,
                                                     a.offsets, a.row_token, a.E, a.H, a.I, a.hq,
                                                     a.hs);
  return hipGetLastError();
}

template <int BM, int BN, int FMT>
static hipError_t launch_dn(const GemmArgs& a, hipStream_t st) {
  const dim3 grid(a.H / BN, gemm_mtile_slots(a.T, a.k, a.E, BM));
  gemm_down_kernel<BM, BN, FMT><<<grid, 256, 0, st>>>(a.dq, a.ds, a.hq, a.hs, a.offsets, a.E,
                                                      a.H, a.I, a.y_rows);
  return hipGetLastError();
}

hipError_t launch_gemm_gate_up(const GemmArgs& a, hipStream_t st) {
  if (a.fmt == 1) return launch_gu<kGemmBM, 1>(a, st);
  return launch_gu<kGemmBM, 2>(a, st);
}

hipError_t launch_gemm_down(const GemmArgs& a, hipStream_t st) {
  if (a.H % 256 == 0) {
    if (a.fmt == 1) return launch_dn<kGemmBM, 256, 1>(a, st);
    return launch_dn<kGemmBM, 256, 2>(a, st);
  }
  if (a.fmt == 1) return launch_dn<kGemmBM, 128, 1>(a, st);
  return launch_dn<kGemmBM, 128, 2>(a, st);
}

}  // namespace bef
