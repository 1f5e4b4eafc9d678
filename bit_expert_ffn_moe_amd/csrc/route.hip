// route.hip -- S1 router logits and S2 top-k + renormalisation.
//
// The router runs first and picks each token's experts (dpshk.com article,
// section "核心实现一"); 6 of 256 per token (ai-muninn.com
// "[洋垃圾跑大模型 #3]").  Logits are fp32 in one fixed order so that the
// chosen ids are reproducible bit for bit: 64-wide chunk partials, each a
// chain of fused multiply-adds in ascending h starting from +0; sums of 4
// consecutive chunks (256 rows) in ascending chunk order; then those group
// sums in ascending group order (the row keeps one fixed accumulation order,
// as dpshk.com "核心实现四" does for its rows; the pages leave the order
// open).  Every kernel below computes exactly that order; they differ only
// in how the (token, expert, chunk) work is spread over the GPU.
//
// Selection: order by (logit desc, id asc), keep k in rank order; weights
// sigmoid(logit) renormalised over the chosen k (fp32, device expf).  The
// pages give no order for a NaN logit: it ranks below every number.
#include <float.h>
#include <limits.h>

#include "actq.h"
#include "common.h"
#include "gemv_body.h"
#include "kernels.h"

namespace bef {

// One wavefront picks the top-k of E <= 256 logits held in LDS and writes
// ids / weights.  Lane l owns experts l, l+64, l+128, l+192, as integer keys
// that order like the logits (-0 made +0; a NaN below every number, an
// expert beyond E below that), sorted in the lane by (key desc, id asc).
// Each of the k rounds takes the wave maximum of the lanes' leading keys
// (wave_max_all: fused DPP steps and row swaps) -- when several lanes hold
// it, the lowest of their ids by the same minimum -- and the winning lane
// moves on to its next key.
__device__ __forceinline__ void topk_wave(const float* __restrict__ z, int E, int k,
                                          int32_t* __restrict__ ids_out,
                                          float* __restrict__ w_out) {
  constexpr int kAbsent = INT_MIN, kNaN = INT_MIN + 1;
  const int lane = threadIdx.x & 63;
  int key[4], sl[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;  // < 256: z holds 256 entries, those from E on unused
    const float v = z[e];
    const int b = __float_as_int(v + 0.0f);
    const int kv = (v != v) ? kNaN : (b >= 0 ? b : b ^ 0x7fffffff);
    key[i] = (e >= E) ? kAbsent : kv;
    sl[i] = i;
  }
  // a 4-input sorting network on (key desc, slot asc)
  auto ce = [&](int a, int b) {
    const bool sw = key[b] > key[a] || (key[b] == key[a] && sl[b] < sl[a]);
    const int ka = key[a], sa = sl[a];
    key[a] = sw ? key[b] : ka;
    sl[a] = sw ? sl[b] : sa;
    key[b] = sw ? ka : key[b];
    sl[b] = sw ? sa : sl[b];
  };
  ce(0, 1);
  ce(2, 3);
  ce(0, 2);
  ce(1, 3);
  ce(1, 2);
  int my_id = 0;
  // k <= 16 (checked by the launchers): unrolled, so the lane's list shifts
  // are register renamings rather than copies carried around a loop
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j >= k) continue;  // uniform; no early exit, so the loop unrolls fully
    const int m = wave_max_all(key[0]);
    const uint64_t cand = __ballot(key[0] == m);
    int wl;
    if (__popcll(cand) == 1) {
      wl = __ffsll((long long)cand) - 1;
    } else {
      const int id = ((cand >> lane) & 1ull) ? lane + 64 * sl[0] : 0x7fffffff;
      wl = __builtin_amdgcn_readfirstlane(wave_min_all(id)) & 63;
    }
    const int win = __builtin_amdgcn_readlane(lane + 64 * sl[0], wl);
    if (lane == j) my_id = win;
    const bool pop = lane == wl;
    key[0] = pop ? key[1] : key[0], sl[0] = pop ? sl[1] : sl[0];
    key[1] = pop ? key[2] : key[1], sl[1] = pop ? sl[2] : sl[1];
    key[2] = pop ? key[3] : key[2], sl[2] = pop ? sl[3] : sl[2];
    key[3] = pop ? kAbsent : key[3];
  }
  const float my_z = (lane < k) ? z[my_id] : 0.0f;
  const float sg = (lane < k) ? 1.0f / (1.0f + expf(-my_z)) : 0.0f;
  const float sum = wave_sum_dpp(sg);
  if (lane < k) {
    ids_out[lane] = my_id;
    w_out[lane] = sg / sum;
  }
}

// ---------------------------------------------------------------------------
// Small T (decode, T <= kRouteSmallT): the front of the layer in one kernel.
//  * Router blocks (group g, quarter q), g < H/256, q < E/64: wave j computes
//    the chunk 4g+j partials of experts 64q .. 64q+63 for every token -- lane
//    l streams 64 rows of column 64q+l, all loads issued before the
//    multiply-adds -- and the block publishes the group sums as
//    {kSlotValid, value} words through 64-bit atomic exchanges (no
//    device-scope fence, and nothing read first).
//  * When sh_h is set (single-token FP4 path), the next I/(4 RUN) blocks per
//    token run the shared expert's gate+up GEMV rows (it needs no routing):
//    its 8.9 MB stream overlaps the router's reduction chain; the last block
//    of each 128-wide block of h requantises it.
//  * Then, when xq is set, act_quant blocks of x (16 lanes per 128-block).
//  * The last router block (in launch order) reads the group sums with
//    atomic loads until each carries kSlotValid (a bounded wait), returns
//    the slots to zero for the next launch, adds the sums in group order,
//    runs the top-k (one wave per token), computes the weights and, when
//    asked, writes the permutation tables (the single-block form of S4) and
//    the list of active routed groups.
// ---------------------------------------------------------------------------
template <int NB, int FMT>
__global__ __launch_bounds__(256) void route_front_kernel(FrontArgs a) {
  const int nc = a.H / 64;                 // 64-row chunks
  const int ng = (nc + 3) / 4;             // groups of 4 chunks
  const int nq4 = (a.E + 63) / 64;         // 64-expert quarters
  const int nr = ng * nq4;                 // router blocks
  const int tid = threadIdx.x;
  const int T = a.T, H = a.H, E = a.E, k = a.k;
  int b = (int)blockIdx.x - nr;
  if (b >= 0 && a.sh_h) {
    const int bpg = a.I / (4 * kGuRun);
    if (b < bpg * T) {
      const int t = b / bpg, lane = tid & 63;
      const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
      const int n0b = (b - t * bpg) * 4 * kGuRun;
      const HExchange hx = {a.h_slots, a.sh_h, a.sh_hq, a.sh_hs, a.status};
      uint4 aq[NB][2];
      float xsc[NB];
      quant_act_codes<NB>(a.x + (size_t)t * H, H, lane, aq, xsc);
      const int n0 = n0b + wv * kGuRun;
      float hv;
      if (FMT == 1) {
        const GUWeights w = {a.sh_gq, a.sh_gs, a.sh_uq, a.sh_us, E, H, a.I};
        hv = gate_up_rows<NB, kGuRun>(w, E, n0, lane, aq, xsc);
      } else {
        const GUWeights8 w = {a.sh_gq, a.sh_uq, reinterpret_cast<const float*>(a.sh_gs),
                              reinterpret_cast<const float*>(a.sh_us), E, H, a.I};
        hv = gate_up_rows_fp8<NB, kGuRun>(w, E, n0, lane, aq, xsc);
      }
      publish_h(hx, hv, T * k + t, a.I, n0, n0b, tid, lane);
      return;
    }
    b -= bpg * T;
  }
  if (b >= 0) {
    // act_quant of x: 16 lanes per 128-block, 8 elements per lane
    act_quant_lanes<true>(a.x, (int64_t)T * (H / 128), a.xq, a.xs, (int64_t)b * 256 + tid);
    return;
  }
  // router block (group g, quarter q): rows 256g .. 256g+255 (chunks 4g ..
  // 4g+3, one per wave) x experts 64q .. 64q+63 (one per lane)
  const int w = tid >> 6, lane = tid & 63;
  const int g = (int)blockIdx.x / nq4, q = (int)blockIdx.x - g * nq4;
  const int c = 4 * g + w, e = 64 * q + lane;
  __shared__ float sx[kRouteSmallT][256];
  __shared__ float sp[4][kRouteSmallT][64];
  __shared__ float sz[kRouteSmallT][256];
  __shared__ int s_ids[kRouteSmallT * 16];
  __shared__ float s_w[kRouteSmallT * 16];
  __shared__ int s_sorted[kRouteSmallT * 16];
  __shared__ int s_rank[kRouteSmallT * 16];
  for (int i = tid; i < T * 256; i += 256) {
    const int t = i >> 8, h = 256 * g + (i & 255);
    sx[t][i & 255] = (h < H) ? bf16_to_f32(a.x[(size_t)t * H + h]) : 0.0f;
  }
  const bool mine = c < nc && e < E;
  uint32_t wv[64];
  if (mine) {
    const uint16_t* col = a.wr + (size_t)(64 * c) * E + e;
#pragma unroll
    for (int h = 0; h < 64; ++h) wv[h] = col[(size_t)h * E];
  }
  __syncthreads();
  if (mine) {
    for (int t = 0; t < T; ++t) {
      float p = 0.0f;
#pragma unroll
      for (int h = 0; h < 64; ++h) p = fmaf(sx[t][64 * w + h], bf16_to_f32(wv[h]), p);
      sp[w][t][lane] = p;
    }
  }
  __syncthreads();
  unsigned long long* slots = reinterpret_cast<unsigned long long*>(a.slots);
  if (tid < T * 64) {
    // the group sum of this (token, expert)
    const int t = tid >> 6, eg = 64 * q + lane;
    if (eg < E) {
      float G = sp[0][t][lane];
      for (int jc = 1; jc < 4 && 4 * g + jc < nc; ++jc) G = G + sp[jc][t][lane];
      atomicExch(slots + ((size_t)g * T + t) * E + eg, kSlotValid | __float_as_uint(G));
    }
  }
  if ((int)blockIdx.x != nr - 1) return;

  // the last router block: logits in the fixed order (group sums added in
  // ascending group order), waiting -- bounded -- until every group sum of
  // this launch is visible, then clearing the slots; thread ez owns expert
  // ez (each slot is written once per launch, so the clear cannot race a
  // write of this launch)
  // (the loads go out together, unconditionally: H <= 2048 NB, so ng <=
  // 8 NB = GMAX and a clamped index repeats the last group only when H is
  // not a multiple of 2048; a branch per load would issue them one by one)
  constexpr int GMAX = 8 * NB;
  const int ez = tid;
  bool ok = true;
  for (int t = 0; t < T; ++t) {
    float acc = -INFINITY;  // experts beyond E never rank
    if (ez < E) {
      unsigned long long* st = slots + (size_t)t * E + ez;
      const size_t gstride = (size_t)T * E;
      unsigned long long v[GMAX];
#pragma unroll
      for (int i = 0; i < GMAX; ++i)
        v[i] = __hip_atomic_load(st + (size_t)min(i, ng - 1) * gstride, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      for (uint32_t spins = 0;;) {
        bool all = true;
#pragma unroll
        for (int i = 0; i < GMAX; ++i) all &= (v[i] & kSlotTagMask) == kSlotValid;
        if (all) break;
        if (++spins >= kSpinLimit) {
          ok = false;
          break;
        }
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int i = 0; i < GMAX; ++i)
          if ((v[i] & kSlotTagMask) != kSlotValid)
            v[i] = __hip_atomic_load(st + (size_t)min(i, ng - 1) * gstride, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int i = 0; i < GMAX; ++i)
        if (i < ng)
          __hip_atomic_store(st + (size_t)i * gstride, 0ull, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      acc = __uint_as_float((uint32_t)v[0]);
#pragma unroll
      for (int i = 1; i < GMAX; ++i)
        if (i < ng) acc = acc + __uint_as_float((uint32_t)v[i]);
    }
    sz[t][ez] = acc;
  }
  if (!ok) atomicOr(a.status, kStatusSyncTimeout);
  __syncthreads();
  // top-k: wave t ranks token t (order: logit desc, id asc).  Results stay
  // in LDS until the last barrier: a barrier after global stores would wait
  // for them to complete.
  if (w < T) topk_wave(sz[w], E, k, s_ids + w * k, s_w + w * k);
  __syncthreads();
  const int P = T * k;
  if (a.offsets && w == 0) {
    // permutation order: the P = T*k <= 64 pairs sorted by (expert, pair
    // index) -- the stable counting-sort order of the general path
    const int id = (lane < P) ? s_ids[lane] : 0x7fffffff;
    int rank = 0;
    for (int qq = 0; qq < P; ++qq) {
      const int iq = __builtin_amdgcn_readlane(id, qq);  // P <= 64: the pairs are lanes
      rank += (iq < id) | ((iq == id) & (qq < lane));
    }
    if (lane < P) {
      s_sorted[rank] = id;
      s_rank[lane] = rank;
    }
  }
  __syncthreads();
  if (tid < P) {
    a.ids[tid] = s_ids[tid];
    a.w[tid] = s_w[tid];
  }
  if (a.offsets) {
    if (tid < P) {
      a.row_token[s_rank[tid]] = tid / k;
      a.row_of[(size_t)(tid / k) * (k + 1) + (tid % k)] = s_rank[tid];
    }
    if (tid < T) {
      a.row_token[P + tid] = tid;
      a.row_of[(size_t)tid * (k + 1) + k] = P + tid;
    }
    // offsets[g] = number of pairs with expert < g (lower bound in the
    // sorted ids); the shared group E holds one row per token
    for (int g2 = tid; g2 <= E + 1; g2 += 256) {
      int v = P + T;
      if (g2 <= E) {
        int lo = 0, hi = P;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (s_sorted[mid] < g2) lo = mid + 1; else hi = mid;
        }
        v = lo;
      }
      a.offsets[g2] = v;
    }
    if (a.active && w == 1) {
      // one entry per distinct routed expert, in expert order
      const bool start = lane < P && (lane == 0 || s_sorted[lane] != s_sorted[lane - 1]);
      const uint64_t m = __ballot(start);
      if (start) {
        const uint64_t after = m & ~((2ull << lane) - 1ull);
        const int end = after ? __ffsll((long long)after) - 1 : P;
        a.active[__popcll(m & ((1ull << lane) - 1ull))] = make_int4(s_sorted[lane], lane, end, 0);
      }
      for (int i = __popcll(m) + lane; i < a.n_active_slots; i += 64)
        a.active[i] = make_int4(-1, 0, 0, 0);
    }
  }
}

// The act_quant of x riding along the router launch of 4 < T < kRouteSplitT
// tokens: blocks past the router's groups in x run thread-blocks b < nb of
// the act_quant kernel's range (b counts over the extra blocks in launch
// order); q == nullptr: none.
struct ActQuantArgs {
  const uint16_t* x;
  uint8_t* q;
  float* s;
  int64_t nblocks;  // 128-element blocks of x
  int64_t nb;       // act_quant thread-blocks of 256 threads
  __device__ __forceinline__ void run(int64_t b, int tid) const {
    if (q && b < nb) act_quant_lanes<true>(x, nblocks, q, s, b * 256 + tid);
  }
};

// ---------------------------------------------------------------------------
// T > 4, in two kernels: the group sums G[g][t][e] over rows 256 g .. 256 g +
// 255 (route_group_quarter_kernel) or, from kRouteSplitT tokens on, over
// rows 512 g .. 512 g + 511 (route_group_mfma_kernel, after the router
// matrix is transposed), then
// route_reduce_kernel: a block per 4 tokens adds the group sums in
// ascending group order (thread e owns expert e) and one wave per token runs
// the top-k.  Splitting over H keeps the GPU busy at moderate T.
// ---------------------------------------------------------------------------
// The router matrix transposed, wr [H][E] -> wrT [E][H] (bf16), in 64 x 64
// tiles through LDS with 16-byte global accesses (8 consecutive experts of
// one row in -- element by element when E is not a multiple of 8 -- and 8
// consecutive rows of one expert out): the matrix-core router below then
// copies 16-byte runs of h per expert straight into LDS.
__global__ __launch_bounds__(256) void route_transpose_kernel(const uint16_t* __restrict__ wr,
                                                              int H, int E,
                                                              uint16_t* __restrict__ wrT) {
  __shared__ uint16_t tile[64][66];  // [h][e], rows padded against bank conflicts
  const int h0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
  const int tid = threadIdx.x;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = 256 * j + tid, h = i >> 3, e8 = (i & 7) * 8;
    const uint16_t* src = wr + (size_t)(h0 + h) * E + e0 + e8;
    if (E % 8 == 0) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (h0 + h < H && e0 + e8 < E) v = *reinterpret_cast<const uint4*>(src);
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        tile[h][e8 + 2 * m] = (uint16_t)(u[m] & 0xffffu);
        tile[h][e8 + 2 * m + 1] = (uint16_t)(u[m] >> 16);
      }
    } else {
#pragma unroll
      for (int m = 0; m < 8; ++m)
        tile[h][e8 + m] = (h0 + h < H && e0 + e8 + m < E) ? src[m] : (uint16_t)0;
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = 256 * j + tid, e = i >> 3, h8 = (i & 7) * 8;
    if (e0 + e < E && h0 + h8 < H) {
      uint32_t u[4];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        u[m] = (uint32_t)tile[h8 + 2 * m][e] | ((uint32_t)tile[h8 + 2 * m + 1][e] << 16);
      *reinterpret_cast<uint4*>(wrT + (size_t)(e0 + e) * H + h0 + h8) =
          make_uint4(u[0], u[1], u[2], u[3]);
    }
  }
}

// The group sums on the matrix cores (T >= kRouteSplitT): block (g, tile)
// takes rows kRouteMfmaRows g .. +kRouteMfmaRows-1 (fewer in the last
// group) for 256 tokens and all E <= 256 experts with
// v_mfma_f32_16x16x32_bf16 (bf16 products are exact; the matrix cores add
// them in fp32 in an order of their own, so the ids are a top-k of these
// logits like the VALU kernels').  The rows pass through LDS 256 at a time:
// per pass, direct global->LDS loads copy each expert's 256 h values (512
// bytes, 32 runs of 16) from wrT, run c of expert e stored at run position
// c xor (e mod 16), so that the 16 lanes of a fragment read (16 experts,
// one run) hit distinct banks.  The products of every pass accumulate in
// the same MFMA results.  8 waves, each 32 tokens x all experts (2 x 16
// tiles of 16 x 16); a lane's token fragment (8 consecutive h of one token,
// 16 contiguous bytes) comes straight from x, a pass's fragments loaded
// before its router rows.  Writes G[g][t][e] for the reduce: with 512 rows
// a group, the group sums of an 8192-token batch take half the bytes they
// take with 256 (67 instead of 134 MB, written and read again).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(512) void route_group_mfma_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ wrT,
                                                               int T, int H, int E,
                                                               float* __restrict__ gsum) {
  __shared__ __align__(16) uint8_t swt[256 * 512];  // [expert][32 runs of 16 bytes]
  const int g = blockIdx.x, t0 = blockIdx.y * 256;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int q = lane >> 4, r = lane & 15;
  constexpr int KS = 8;  // 32-row MFMA steps per pass of 256 rows
  const uint8_t* wbase = reinterpret_cast<const uint8_t*>(wrT);
  v4f_t acc[2][16];
#pragma unroll
  for (int mf = 0; mf < 2; ++mf)
#pragma unroll
    for (int f = 0; f < 16; ++f) acc[mf][f] = (v4f_t){0.0f, 0.0f, 0.0f, 0.0f};
  for (int pass = 0; pass < kRouteMfmaRows / 256; ++pass) {
    const int h0 = kRouteMfmaRows * g + 256 * pass;
    if (h0 >= H) break;  // block-uniform
    const int nh = min(256, H - h0);  // rows of this pass (a multiple of 64)
    // this lane's token fragments for every K step of the pass, loads issued first
    uint4 av[KS][2];
#pragma unroll
    for (int mf = 0; mf < 2; ++mf) {
      const int t = min(t0 + 32 * w + 16 * mf + r, T - 1);
      const uint16_t* xr = x + (size_t)t * H + h0 + 8 * q;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        av[ks][mf] = (32 * ks < nh) ? *reinterpret_cast<const uint4*>(xr + 32 * ks)
                                    : make_uint4(0, 0, 0, 0);
    }
    // every wave is done with the previous pass's rows before they are replaced
    if (pass > 0) {
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      block_barrier();
    }
    // the router rows: LDS run position s = 512 i + tid holds run
    // (s mod 32) xor (e mod 16) of expert e = s / 32 (experts past E repeat
    // the last one, runs past the pass's rows repeat its last run: neither
    // is read)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int sp = 512 * i + tid, e = sp >> 5, c = (sp & 31) ^ (e & 15);
      const uint32_t off = ((uint32_t)min(e, E - 1) * (uint32_t)H + (uint32_t)(h0 + min(8 * c, nh - 8))) * 2u;
      dma16(wbase, off, swt + (size_t)(512 * i + 64 * w) * 16);
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
    block_barrier();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (32 * ks >= nh) break;
      const bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, av[ks][0]);
      const bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, av[ks][1]);
#pragma unroll
      for (int f = 0; f < 16; ++f) {
        const uint4 bv =
            *reinterpret_cast<const uint4*>(swt + (size_t)((16 * f + r) * 32 + ((4 * ks + q) ^ r)) * 16);
        const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bv);
        acc[0][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b, acc[0][f], 0, 0, 0);
        acc[1][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b, acc[1][f], 0, 0, 0);
      }
    }
  }
  // tile (mf, f): lane holds experts 16 f + r, tokens 16 mf + 4 q + v of the wave's 32
#pragma unroll
  for (int mf = 0; mf < 2; ++mf)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int t = t0 + 32 * w + 16 * mf + 4 * q + v;
      if (t >= T) continue;
      float* dst = gsum + ((size_t)g * T + t) * E;
#pragma unroll
      for (int f = 0; f < 16; ++f)
        if (16 * f + r < E) dst[16 * f + r] = acc[mf][f][v];
    }
}

// Fewer tokens (T < kRouteSplitT): the same group sums with the experts split
// in quarters as well, block (g, quarter, 32-token tile), so that a 32-token
// batch still spreads over 64 blocks; thread (ty, tx) accumulates token ty x
// experts 64 quarter + 8tx .. +7 in the same fixed order.
__global__ __launch_bounds__(256) void route_group_quarter_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int H, int E,
    float* __restrict__ gsum, ActQuantArgs aq) {
  __shared__ __align__(16) float sx[32][68];   // [token][h of the chunk], padded rows
  __shared__ __align__(16) float sw[64][64];   // [h of the chunk][expert of the quarter]
  const int g = blockIdx.x, e00 = 64 * blockIdx.y, t0 = blockIdx.z * 32;
  const int tid = threadIdx.x;
  const int ng = (H / 64 + 3) / 4;
  if (g >= ng) {
    aq.run(((int64_t)(g - ng) * gridDim.z + blockIdx.z) * gridDim.y + blockIdx.y, tid);
    return;
  }
  const int ty = tid >> 3, tx = tid & 7;
  const int nc = H / 64;
  const int c0 = 4 * g, c1 = min(4 * g + 4, nc);
  // this thread's share of a chunk: x row tid/8, 8 bf16 at (tid%8)*8; router
  // 16-byte pieces q = tid + 256 i (i < 2): row q/8, experts e00 + (q%8)*8 .. +7
  const int xr = tid >> 3, xc = (tid & 7) * 8;
  const bool xin = t0 + xr < T;
  uint4 px, pw[2];
  auto load_chunk = [&](int c) {
    px = xin ? *reinterpret_cast<const uint4*>(x + (size_t)(t0 + xr) * H + 64 * c + xc)
             : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 256 * i, h = q >> 3, e8 = e00 + (q & 7) * 8;
      const uint16_t* src = wr + (size_t)(64 * c + h) * E + e8;
      if (e8 + 8 <= E && (E & 7) == 0) {
        pw[i] = *reinterpret_cast<const uint4*>(src);
      } else {
        uint16_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = (e8 + u < E) ? src[u] : (uint16_t)0;
        pw[i] = make_uint4(v[0] | ((uint32_t)v[1] << 16), v[2] | ((uint32_t)v[3] << 16),
                           v[4] | ((uint32_t)v[5] << 16), v[6] | ((uint32_t)v[7] << 16));
      }
    }
  };
  auto store_chunk = [&]() {
    *reinterpret_cast<float4*>(&sx[xr][xc]) =
        make_float4(bf16_to_f32(px.x & 0xffffu), bf16_to_f32(px.x >> 16),
                    bf16_to_f32(px.y & 0xffffu), bf16_to_f32(px.y >> 16));
    *reinterpret_cast<float4*>(&sx[xr][xc + 4]) =
        make_float4(bf16_to_f32(px.z & 0xffffu), bf16_to_f32(px.z >> 16),
                    bf16_to_f32(px.w & 0xffffu), bf16_to_f32(px.w >> 16));
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = tid + 256 * i, h = q >> 3, e8 = (q & 7) * 8;
      const uint4 r = pw[i];
      *reinterpret_cast<float4*>(&sw[h][e8]) =
          make_float4(bf16_to_f32(r.x & 0xffffu), bf16_to_f32(r.x >> 16),
                      bf16_to_f32(r.y & 0xffffu), bf16_to_f32(r.y >> 16));
      *reinterpret_cast<float4*>(&sw[h][e8 + 4]) =
          make_float4(bf16_to_f32(r.z & 0xffffu), bf16_to_f32(r.z >> 16),
                      bf16_to_f32(r.w & 0xffffu), bf16_to_f32(r.w >> 16));
    }
  };
  float grp[8];
  load_chunk(c0);
  for (int c = c0; c < c1; ++c) {
    store_chunk();
    __syncthreads();
    if (c + 1 < c1) load_chunk(c + 1);  // in flight while this chunk multiplies
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) p[j] = 0.0f;
#pragma unroll 4
    for (int h4 = 0; h4 < 64; h4 += 4) {
      const float4 xv = *reinterpret_cast<const float4*>(&sx[ty][h4]);
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        const float4 w0 = *reinterpret_cast<const float4*>(&sw[h4 + hh][8 * tx]);
        const float4 w1 = *reinterpret_cast<const float4*>(&sw[h4 + hh][8 * tx + 4]);
        const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        const float xs = hh == 0 ? xv.x : hh == 1 ? xv.y : hh == 2 ? xv.z : xv.w;
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = fmaf(xs, wv[j], p[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) grp[j] = (c == c0) ? p[j] : grp[j] + p[j];
    __syncthreads();
  }
  const int t = t0 + ty, e0 = e00 + 8 * tx;
  if (t >= T) return;
  float* dst = gsum + ((size_t)g * T + t) * E;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if (e0 + j < E) dst[e0 + j] = grp[j];
}

// The logits of 4 tokens per block: the ng group sums added in ascending
// group order (thread e owns expert e; all group loads issued before the
// adds, GMAX >= ng of them, the index clamped to the last group), then one
// wave per token runs the top-k.
template <int GMAX>
__global__ __launch_bounds__(256) void route_reduce_kernel(const float* __restrict__ gsum, int T,
                                                           int ng, int E, int k,
                                                           int32_t* __restrict__ ids,
                                                           float* __restrict__ w) {
  __shared__ float sz[4][256];
  const int t0 = blockIdx.x * 4, tid = threadIdx.x;
  const int e = min(tid, E - 1);
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int t = min(t0 + tt, T - 1);
    float v[GMAX];
#pragma unroll
    for (int g = 0; g < GMAX; ++g)
      v[g] = gsum[((size_t)min(g, ng - 1) * T + t) * E + e];
    float acc = v[0];
#pragma unroll
    for (int g = 1; g < GMAX; ++g)
      if (g < ng) acc = acc + v[g];
    sz[tt][tid] = (t0 + tt < T && tid < E) ? acc : 0.0f;
  }
  __syncthreads();
  const int wv = tid >> 6, t = t0 + wv;
  if (t < T) topk_wave(sz[wv], E, k, ids + (size_t)t * k, w + (size_t)t * k);
}

hipError_t launch_route(const uint16_t* x, const uint16_t* wr, int T, int H, int E, int k,
                        int32_t* ids, float* w, WsCtl* ctl, float* gsum, uint16_t* wrT,
                        hipStream_t st, uint8_t* xq, float* xs) {
  if (T <= kRouteSmallT) {
    FrontArgs a = {};
    a.x = x, a.wr = wr, a.T = T, a.H = H, a.E = E, a.k = k;
    a.ids = ids, a.w = w;
    a.xq = xq, a.xs = xs;
    set_route_sync(a, ctl);
    return launch_route_front(a, st);
  }
  if (!gsum || E > 256 || H % 64 != 0 || (H / 64 + 3) / 4 > kRouteMaxGroups)
    return hipErrorInvalidValue;
  const int ng = (H / 64 + 3) / 4;
  if (T < kRouteSplitT) {
    // act_quant of x (when xq is set) in extra x-slices of the router's grid:
    // one launch fewer.  (From kRouteSplitT tokens on, the matrix-core
    // router's blocks hold 132 KB of LDS each, and the act_quant runs as a
    // launch of its own.)
    ActQuantArgs aq = {x, xq, xs, (int64_t)T * (H / 128), 0};
    if (xq) aq.nb = (aq.nblocks * 16 + 255) / 256;
    const int ny = (E + 63) / 64, nz = (T + 31) / 32;
    const int nqx = (int)((aq.nb + ny * nz - 1) / (ny * nz));
    route_group_quarter_kernel<<<dim3(ng + nqx, ny, nz), dim3(256), 0, st>>>(x, wr, T, H, E,
                                                                            gsum, aq);
    route_reduce_kernel<kRouteMaxGroups>
        <<<dim3((T + 3) / 4), dim3(256), 0, st>>>(gsum, T, ng, E, k, ids, w);
  } else {
    if (!wrT || (size_t)E * H * 2 > 0xffffffffu) return hipErrorInvalidValue;
    const int ngm = (H + kRouteMfmaRows - 1) / kRouteMfmaRows;
    route_transpose_kernel<<<dim3((H + 63) / 64, (E + 63) / 64), dim3(256), 0, st>>>(wr, H, E,
                                                                                   wrT);
    route_group_mfma_kernel<<<dim3(ngm, (T + 255) / 256), dim3(512), 0, st>>>(x, wrT, T, H, E,
                                                                             gsum);
    route_reduce_kernel<kRouteMaxGroups * 256 / kRouteMfmaRows>
        <<<dim3((T + 3) / 4), dim3(256), 0, st>>>(gsum, T, ngm, E, k, ids, w);
  }
  if (xq && T >= kRouteSplitT) return launch_act_quant(x, true, T, H, xq, xs, st);
  return hipGetLastError();
}

void set_route_sync(FrontArgs& a, WsCtl* ctl) {
  a.slots = ctl->route_slots;
  a.status = &ctl->status;
}

hipError_t launch_route_front(const FrontArgs& a, hipStream_t st) {
  if (a.T < 1 || a.T > kRouteSmallT || a.k > 16 || a.E > 256 || a.H % 64 != 0 ||
      (a.H / 64 + 3) / 4 > kRouteMaxGroups || !a.slots || !a.status)
    return hipErrorInvalidValue;
  int nq = 0, nsh = 0;
  if (a.xq) nq = (int)(((int64_t)a.T * (a.H / 128) * 16 + 255) / 256);
  if (a.sh_h) {
    if (a.I % 128 != 0 || a.I > kHSlotStride || a.T * (a.k + 1) > kHSlotRows)
      return hipErrorInvalidValue;
    nsh = (a.I / (4 * kGuRun)) * a.T;
  }
  const int nr = (a.H / 64 + 3) / 4 * ((a.E + 63) / 64);
  const dim3 grid(nr + nsh + nq);
  const int nb = (a.H / 32 + 63) / 64;
  const bool f8 = a.sh_h && a.fmt == 2;  // the shared expert's rows are FP8
  if (nb <= 1) {
    if (f8) route_front_kernel<1, 2><<<grid, dim3(256), 0, st>>>(a);
    else route_front_kernel<1, 1><<<grid, dim3(256), 0, st>>>(a);
  } else if (nb <= 2) {
    if (f8) route_front_kernel<2, 2><<<grid, dim3(256), 0, st>>>(a);
    else route_front_kernel<2, 1><<<grid, dim3(256), 0, st>>>(a);
  } else {
    if (f8) route_front_kernel<4, 2><<<grid, dim3(256), 0, st>>>(a);
    else route_front_kernel<4, 1><<<grid, dim3(256), 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace bef
