// decode.hip -- S5, S6 and S7 for one token in one persistent kernel: the
// routed experts' gate+up+SwiGLU, the requantisation of h, the down
// projection of every expert (routed and shared) and the combine.
//
// A decoded token pays a fixed cost per step beyond moving its weights
// (ai-muninn.com "[洋垃圾跑大模型 #3]", section "軟地板大約 18": scheduling,
// launches, expert selection); here that cost is the gap between the
// gate+up and down launches and the exchange of h between them, during
// which HBM would idle.  The kernel keeps HBM busy across it: one block per
// CU owns 16 output rows; its waves stream the routed gate+up rows from
// registers, then copy those 16 rows of every selected expert's W_down (and
// the shared expert's) into the block's LDS by direct global->LDS loads --
// 7 x 16 rows x 1088 bytes = 119 KB at hidden 4096, intermediate 2048, FP4:
// the 31 MB of down weights fit in the chip's LDS -- while h is exchanged.
// Once every 128-wide block of h is requantised, the down products and the
// combine run out of LDS.
//
// Measured on MI355X at those shapes (6 routed experts + shared): 30.5 us
// for the kernel against 14.8 + 11.1 us for the separate gate+up and
// down+combine kernels.  Per-block timestamps put the gate+up stream's last
// waves at 19-23 us (the separate gate+up kernel ends at ~14.5 us) and the
// exchange chain after it (requantisation, code words, down, combine) at
// ~7 us.  Neither the order of the copies (before or after the gate+up
// rows) nor 12 instead of 16 waves per block changed the time; dealing the
// gate+up rows out to the blocks in 16-row groups, as the separate kernel's
// blocks get them, made it slower (35 us).  So the library keeps the
// separate kernels by default and runs this one only when asked
// (moe_debug_set_decode_fused).
//
// The arithmetic is that of the two one-token kernels (gemv.hip) step by
// step -- the same device functions for the gate+up rows, the same
// requantisation (tcti.cn post, section "补齐软件栈缺失": act_quant feeds
// the FP8/FP4 linears), the same per-chunk down products and butterfly, the
// same combine order -- so the output is bit-identical to theirs.
//
// h moves between blocks without a device-scope fence, through 64-bit
// atomics carrying {launch tag, value} (a tag that no other launch uses, so
// nothing is ever cleared):
//  * each gate+up wave sends its h values out (atomic exchanges) and counts
//    its unit in the 128-wide block of h it belongs to;
//  * the wave whose count completes a block reads the block's 128 values
//    until all carry the tag (a bounded wait: past kSpinLimit rounds it
//    flags MOE_STATUS_SYNC_TIMEOUT and carries on), writes the E4M3 codes
//    and scale with the act_quant rule and sends them out as 32 words of
//    four codes and one scale word;
//  * every block, once all of its own waves are through, reads the code
//    words of all routed rows into LDS until all carry the tag (bounded).
// The counts only say who looks when (the tags decide validity), and no
// wave polls while the others of its block still stream weights.
// The shared expert's h was requantised by the front kernel (route.hip) and
// is read from the workspace.  The last block to finish advances the epoch.
// Every wait is on work that does not wait itself, so the kernel completes
// when its blocks are co-resident (one per CU, the LDS allows no second);
// otherwise the waits run out and the status says so.
#include <hip/hip_ext.h>

#include "common.h"
#include "gemv_body.h"
#include "kernels.h"

namespace bef {

constexpr int kDecThreads = kDecWaves * 64;
constexpr int kDecI = 2048;                  // largest intermediate size
constexpr int kDecCodeWords = 36;            // per 128-block: 32 code words, 1 scale word, pad
// code words of all routed rows per thread: (kDecMaxRows - 1) x 16 x 33 at most
constexpr int kDecWordsPerThread = ((kDecMaxRows - 1) * 16 * 33 + kDecThreads - 1) / kDecThreads;

template <int NB>
__global__ __launch_bounds__(kDecThreads) void decode_ffn_kernel(DecodeArgs a) {
  // LDS: W_down rows of the block (codes, then UE8M0 scales) per h row, the
  // requantised h rows, the down totals
  __shared__ __align__(16) uint8_t sW[kDecMaxRows][kDecRowsPerBlock * kDecI / 2];
  __shared__ __align__(16) uint8_t sS[kDecMaxRows][1024];
  __shared__ __align__(16) uint8_t sH[kDecMaxRows][kDecI];
  __shared__ float sHS[kDecMaxRows][kDecI / 128];
  __shared__ float sY[kDecMaxRows][kDecRowsPerBlock];
  __shared__ int sG[kDecMaxRows];  // each h row's expert

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = a.E, H = a.H, I = a.I, k = a.k, R = k + 1;
  const int I4 = I >> 2, I128 = I >> 7, nch = I >> 5;
  const int m0 = blockIdx.x * kDecRowsPerBlock;
  const uint32_t ep = __hip_atomic_load(a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const uint64_t tag = (uint64_t)(ep | 0x80000000u) << 32;

  // the experts of the h rows, once (loads inside the copy loop would each
  // wait for every copy issued before them: one counter for both)
  if (tid < R) sG[tid] = tid < k ? a.active[tid].x : E;
  __syncthreads();

  // ---- requantisation of the 128-wide block c of h row r, by the wave whose
  // unit completed it: waits (bounded) until the block's 128 words carry
  // the tag, then sends out the codes and the scale ----
  bool ok = true;
  auto requant = [&](int r, int c) {
    const int n = 128 * c + 2 * lane;
    const unsigned long long* hw = reinterpret_cast<const unsigned long long*>(a.dec_h) + r * kDecI;
    unsigned long long w0 = 0, w1 = 0;
    bool got = false;
    for (uint32_t spins = 0;;) {
      if ((w0 & kSlotTagMask) != tag)
        w0 = __hip_atomic_load(hw + n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((w1 & kSlotTagMask) != tag)
        w1 = __hip_atomic_load(hw + n + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      got = (w0 & kSlotTagMask) == tag && (w1 & kSlotTagMask) == tag;
      if (__all(got) || ++spins >= kSpinLimit) break;
      __builtin_amdgcn_s_sleep(1);
    }
    ok &= got;
    const float v0 = __uint_as_float((uint32_t)w0), v1 = __uint_as_float((uint32_t)w1);
    const float amax = wave_max(fmaxf(fabsf(v0), fabsf(v1)));
    const float sc = amax / 448.0f;
    uint32_t q = 0;
    if (amax != 0.0f) q = e4m3_pack4(v0 / sc, v1 / sc, 0.0f, 0.0f);
    reinterpret_cast<uint16_t*>(a.hq + (size_t)r * I + n)[0] = (uint16_t)q;
    if (lane == 0) a.hs[(size_t)r * I128 + c] = sc;
    // four codes per word: lanes 2i and 2i+1 hold codes 4i..4i+1 and 4i+2..4i+3
    const uint32_t q2 = (uint32_t)__shfl_down((int)q, 1, 64);
    unsigned long long* cw =
        reinterpret_cast<unsigned long long*>(a.dec_c) + (r * 16 + c) * kDecCodeWords;
    if ((lane & 1) == 0) atomicExch(cw + (lane >> 1), tag | ((q & 0xffffu) | (q2 << 16)));
    if (lane == 0) atomicExch(cw + 32, tag | __float_as_uint(sc));
  };

  // ---- routed gate+up: wave w takes units u_lo + w, + kDecWaves, ... ----
  const int units = k * I4;  // gate+up units: 4 rows of h each
  const int ub = (units + (int)gridDim.x - 1) / (int)gridDim.x;  // units per block
  const int u_lo = blockIdx.x * ub, u_hi = min(u_lo + ub, units);
  const GUWeights w = {a.gq, a.gs, a.uq, a.us, E, H, I};
  for (int u = u_lo + wv; u < u_hi; u += kDecWaves) {
    const int r = u / I4, n0 = (u - r * I4) * 4;
    const int g = __builtin_amdgcn_readfirstlane(sG[r]);
    uint4 aq[NB][2];
    float xsc[NB];
    load_act_codes<NB>(a.xq, a.xs, H, lane, aq, xsc);
    const float hv = gate_up_rows<NB>(w, g, n0, lane, aq, xsc);
    if (h_lane(lane)) {
      const int n = n0 + h_row(lane);
      a.h[(size_t)r * I + n] = hv;
      atomicExch(reinterpret_cast<unsigned long long*>(a.dec_h) + r * kDecI + n,
                 tag | __float_as_uint(hv));
    }
    // count the unit in its 128-block; the wave that completes the count
    // requantises the block (and returns the count to zero for the next
    // launch: all 32 increments are in)
    uint32_t prev = 0;
    uint32_t* cnt = a.cnt + r * 16 + (n0 >> 7);
    if (lane == 0) prev = atomicAdd(cnt, 1u);
    prev = __builtin_amdgcn_readfirstlane(prev);
    if (prev == 31) {
      if (lane == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      requant(r, n0 >> 7);
    }
  }
  // ---- the down rows m0 .. m0+15 of every h row's expert into LDS, once
  // this wave's gate+up work is out (the gate+up rows go first) ----
  {
    const int cw = kDecRowsPerBlock * (I >> 1);   // code bytes per h row (multiple of 1024)
    const int sb = kDecRowsPerBlock * (I >> 5);   // scale bytes per h row (64 .. 1024)
    const int per_row = cw / 1024 + 1;
    for (int i = wv; i < R * per_row; i += kDecWaves) {
      const int r = i / per_row, j = i - r * per_row;
      const int g = __builtin_amdgcn_readfirstlane(sG[r]);
      if (j + 1 < per_row) {
        const uint8_t* src = a.dq + ((size_t)g * H + m0) * (size_t)(I >> 1);
        dma16(src, (uint32_t)(1024 * j + 16 * lane), &sW[r][1024 * j]);
      } else {
        const uint8_t* src = a.ds + ((size_t)g * H + m0) * (size_t)(I >> 5);
        dma16(src, (uint32_t)min(16 * lane, sb - 16), &sS[r][0]);
      }
    }
  }
  // every wave of the block is done with its own work before any waits for
  // the others' (waiting waves would slow the streaming ones)
  __syncthreads();

  // ---- all routed code words into LDS; the shared row from the workspace ----
  {
    const int nw = k * I128 * 33;
    unsigned long long wd[kDecWordsPerThread];
#pragma unroll
    for (int q = 0; q < kDecWordsPerThread; ++q) wd[q] = 0;
    const unsigned long long* cw = reinterpret_cast<const unsigned long long*>(a.dec_c);
    auto word_at = [&](int i) {
      const int rc = i / 33, j = i - rc * 33;  // rc = r * I128 + c
      const int r = rc / I128, c = rc - r * I128;
      return cw + (r * 16 + c) * kDecCodeWords + j;
    };
    for (uint32_t spins = 0;;) {
      bool all = true;
#pragma unroll
      for (int q = 0; q < kDecWordsPerThread; ++q) {
        const int i = tid + q * kDecThreads;
        if (i < nw && (wd[q] & kSlotTagMask) != tag) {
          wd[q] = __hip_atomic_load(word_at(i), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          all &= (wd[q] & kSlotTagMask) == tag;
        }
      }
      if (__all(all)) break;
      if (++spins >= kSpinLimit) {
        ok = false;
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
#pragma unroll
    for (int q = 0; q < kDecWordsPerThread; ++q) {
      const int i = tid + q * kDecThreads;
      if (i < nw) {
        const int rc = i / 33, j = i - rc * 33;
        const int r = rc / I128, c = rc - r * I128;
        if (j < 32)
          *reinterpret_cast<uint32_t*>(&sH[r][128 * c + 4 * j]) = (uint32_t)wd[q];
        else
          sHS[r][c] = __uint_as_float((uint32_t)wd[q]);
      }
    }
    for (int i = tid; i < I / 16; i += kDecThreads)
      *reinterpret_cast<uint4*>(&sH[k][16 * i]) =
          *reinterpret_cast<const uint4*>(a.hq + (size_t)k * I + 16 * i);
    for (int i = tid; i < I128; i += kDecThreads) sHS[k][i] = a.hs[(size_t)k * I128 + i];
  }
  if (!ok) atomicOr(a.status, kStatusSyncTimeout);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's copies into LDS (and everything else)
  __syncthreads();

  // ---- down: item i < 2R (waves in turn) is h row r = i / 2 and output rows m0 + 8 (i % 2) + 0..7
  // (the per-chunk products and the butterfly of gemv_down_kernel) ----
  for (int it = wv; it < 2 * R; it += kDecWaves) {
    const int r = it >> 1, i0 = 8 * (it & 1);
    const int ch = min(lane, nch - 1);
    const uint4 a0q = *reinterpret_cast<const uint4*>(&sH[r][32 * ch]);
    const uint4 a1q = *reinterpret_cast<const uint4*>(&sH[r][32 * ch + 16]);
    Act16 a0, a1;
    e4m3x16_to_h2(a0q, a0);
    e4m3x16_to_h2(a1q, a1);
    const float hsc = (lane < nch) ? sHS[r][ch >> 2] : 0.0f;
    const int rowq = I >> 1, rows_ = nch;
    float part[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 wq = *reinterpret_cast<const uint4*>(&sW[r][(i0 + i) * rowq + 16 * ch]);
      const uint32_t sb = sS[r][(i0 + i) * rows_ + ch];
      float acc = 0.0f;
      acc += scale_ue8m0(dot32_fp4(wq, a0, a1), sb) * hsc;
      part[i] = acc;
    }
    const float tot = butterfly8(part);
    if ((lane & 7) == 0) sY[r][i0 + (lane >> 3)] = tot;
  }
  __syncthreads();

  // ---- combine (the order of gemv_down_kernel): the shared row first, then
  // the routed rows in rank order ----
  if (tid < kDecRowsPerBlock) {
    const int rs = a.row_of[k];
    float o = (rs >= 0 && rs < R) ? sY[rs][tid] : 0.0f;
    for (int j = 0; j < k; ++j) {
      const int rj = a.row_of[j];
      if (rj >= 0 && rj < R) o = fmaf(a.topk_w[j], sY[rj][tid], o);
    }
    const size_t m = (size_t)m0 + tid;
    if (a.out_bf16)
      reinterpret_cast<uint16_t*>(a.out)[m] = f32_to_bf16(o);
    else
      reinterpret_cast<float*>(a.out)[m] = o;
  }
  // ---- the last block to finish advances the epoch for the next launch ----
  if (tid == 0) {
    const uint32_t prev = atomicAdd(a.done, 1u);
    if (prev == gridDim.x - 1) {
      __hip_atomic_store(a.done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.epoch, (ep + 1u) & 0x7fffffffu, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Blocks: H / 16, one per CU; hidden <= 4096 (activation chunks NB <= 2:
// the registers of 16 waves per CU hold no more).
static int dec_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return n;
}

bool decode_ffn_fits(int fmt, int T, int k, int H, int I) {
  if (fmt != MOE_W_FP4_E2M1_UE8M0_K32 || T != 1 || k < 1 || k + 1 > kDecMaxRows) return false;
  if (I > kDecI || I % 128 != 0 || H % kDecRowsPerBlock != 0 || H > 4096) return false;
  return H / kDecRowsPerBlock <= dec_cu_count();
}

template <int NB>
static void launch_nb(const DecodeArgs& a, hipStream_t st) {
  const dim3 grid(a.H / kDecRowsPerBlock), block(kDecThreads);
  const KernelTimer& tm = g_kernel_timer[MOE_KERNEL_DECODE_FFN];
  if (tm.start)
    hipExtLaunchKernelGGL(decode_ffn_kernel<NB>, grid, block, 0, st, tm.start, tm.stop, 0, a);
  else
    decode_ffn_kernel<NB><<<grid, block, 0, st>>>(a);
}

hipError_t launch_decode_ffn(const DecodeArgs& a, hipStream_t st) {
  if (!decode_ffn_fits(MOE_W_FP4_E2M1_UE8M0_K32, 1, a.k, a.H, a.I)) return hipErrorInvalidValue;
  if (a.H <= 2048)
    launch_nb<1>(a, st);
  else
    launch_nb<2>(a, st);
  return hipGetLastError();
}

}  // namespace bef
