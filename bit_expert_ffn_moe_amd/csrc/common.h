// common.h -- device helpers shared by the gfx950 kernels of this library.
//
// Format conversions use the CDNA4 hardware converters:
//   v_cvt_pk_fp8_f32            two fp32 -> two E4M3 codes, round to nearest even
//   v_cvt_scalef32_pk_f16_fp8   two E4M3 codes -> two fp16 (exact: every E4M3
//                               value is an fp16 value)
//   v_cvt_scalef32_pk_f16_fp4   one byte of two E2M1 codes -> two fp16 (exact)
// and products of those exact fp16 values are summed with v_dot2_f32_f16
// (fp32 accumulate).  E4M3 and E2M1 are the OCP formats (OCP 8-bit Floating
// Point rev 1.0; OCP Microscaling Formats v1.0).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bef {

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* glb_ptr_t;

// s_waitcnt immediates (gfx9: vmcnt [3:0] + [15:14], expcnt [6:4], lgkmcnt [11:8])
constexpr int waitcnt_vm(int n) { return 0xF70 | (n & 0xF) | ((n >> 4) << 14); }
// s_waitcnt immediate of lgkmcnt(0) (vmcnt and expcnt left at their maxima)
constexpr int kWaitLgkm0 = 0xC07F;

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v4f_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// Workgroup barrier that is also a compiler barrier for memory accesses: the
// s_barrier builtin is modelled as touching no memory, so LDS reads could be
// moved across it; an asm statement with a memory clobber cannot be.  (It
// waits for nothing: the callers wait for their own loads explicitly.)
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Direct global->LDS loads of 16 or 4 bytes per lane: global address base +
// voff (base wave-uniform), LDS address M0 + size x lane, with M0 the
// wave-uniform LDS base l.  Written as asm statements (no register output,
// LDS written, hence the memory clobber): the compiler's tracking of the
// builtin form marks the LDS counter out of order, so every later LDS read
// then waits for all outstanding ones (lgkmcnt(0)) and the first MFMA of a
// K step waits for all of the step's operand reads.  Unseen by the compiler,
// these loads are waited for explicitly (vmcnt before the barrier that precedes
// the first LDS read of the copied data).
__device__ __forceinline__ uint32_t lds_addr(void* l) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)l);
}
__device__ __forceinline__ void dma16(const uint8_t* base, uint32_t voff, void* l) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds_addr(l))
               : "memory");
}
__device__ __forceinline__ void dma4(const uint8_t* base, uint32_t voff, void* l) {
  asm volatile("global_load_lds_dword %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds_addr(l))
               : "memory");
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// E4M3 code of v: clamp to +-448 first (the conversion then rounds to
// nearest even; values in (448, 464) round to 448 either way, so the clamp
// only turns would-be overflows into the saturated code; -0 stays -0).
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
  d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
  uint32_t v = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, (int)v, true);
  return v;
}

// Two E4M3 codes (bytes 0-1 or 2-3 of v) -> (lo element, hi element) fp16.
__device__ __forceinline__ h2_t e4m3x2_lo(uint32_t v) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, false);
}
__device__ __forceinline__ h2_t e4m3x2_hi(uint32_t v) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, true);
}

// Two E2M1 codes in byte B of v (element 2j in bits 0-3, 2j+1 in bits 4-7)
// -> (element 2j, element 2j+1) fp16.
template <int B>
__device__ __forceinline__ h2_t e2m1x2(uint32_t v) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, B);
}

__device__ __forceinline__ float dot2(h2_t a, h2_t b, float c) {
  return __builtin_amdgcn_fdot2(a, b, c, false);
}

// Eight fp16 pairs of activations (elements 0..15 of a 16-code group, from
// four dwords of E4M3 codes).
struct Act16 {
  h2_t p[8];
};

__device__ __forceinline__ void e4m3x16_to_h2(const uint4 q, Act16& a) {
  a.p[0] = e4m3x2_lo(q.x);
  a.p[1] = e4m3x2_hi(q.x);
  a.p[2] = e4m3x2_lo(q.y);
  a.p[3] = e4m3x2_hi(q.y);
  a.p[4] = e4m3x2_lo(q.z);
  a.p[5] = e4m3x2_hi(q.z);
  a.p[6] = e4m3x2_lo(q.w);
  a.p[7] = e4m3x2_hi(q.w);
}

// Sum of 16 products: E2M1 codes in one dword w (elements 8d..8d+7 for the
// bytes 0..3) against activation pairs a.p[...]: the dword holds 8 weights,
// matching activation pairs p0..p3.
__device__ __forceinline__ float dot8_fp4(uint32_t w, h2_t p0, h2_t p1, h2_t p2, h2_t p3,
                                          float acc) {
  acc = dot2(e2m1x2<0>(w), p0, acc);
  acc = dot2(e2m1x2<1>(w), p1, acc);
  acc = dot2(e2m1x2<2>(w), p2, acc);
  acc = dot2(e2m1x2<3>(w), p3, acc);
  return acc;
}

// 32 E2M1 weights (16 bytes) . 32 activations (two Act16) -> fp32, as two
// independent accumulation chains (instruction-level parallelism).
__device__ __forceinline__ float dot32_fp4(const uint4 w, const Act16& a0, const Act16& a1) {
  float acc0 = dot8_fp4(w.x, a0.p[0], a0.p[1], a0.p[2], a0.p[3], 0.0f);
  float acc1 = dot8_fp4(w.z, a1.p[0], a1.p[1], a1.p[2], a1.p[3], 0.0f);
  acc0 = dot8_fp4(w.y, a0.p[4], a0.p[5], a0.p[6], a0.p[7], acc0);
  acc1 = dot8_fp4(w.w, a1.p[4], a1.p[5], a1.p[6], a1.p[7], acc1);
  return acc0 + acc1;
}

// 2^(b - 127) applied exactly (UE8M0 scale byte b).
__device__ __forceinline__ float scale_ue8m0(float v, uint32_t b) {
  return __builtin_amdgcn_ldexpf(v, (int)b - 127);
}

// Cross-lane data movement through DPP (GFX9 encodings: quad_perm, row
// mirrors, row_bcast15/31).
template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, BANK_MASK, true));
}

// Sum over the 64 lanes, result valid in every lane: pairs, quads, half
// rows, rows of 16 by DPP, then rows combined through row_bcast15/31 into
// lane 63, read back as a scalar.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_f<0xB1>(v);        // quad_perm [1,0,3,2]
  v += dpp_f<0x4E>(v);        // quad_perm [2,3,0,1]
  v += dpp_f<0x141>(v);       // row_half_mirror
  v += dpp_f<0x140>(v);       // row_mirror
  v += dpp_f<0x142, 0xA>(v);  // row_bcast15 into rows 1 and 3
  v += dpp_f<0x143, 0xC>(v);  // row_bcast31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Maximum / minimum over the 64 lanes, in every lane: inside each row of 16
// by DPP (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror,
// row_mirror; every source lane exists, so each step fuses into one
// v_max/min_i32_dpp), then across rows by the gfx950 row swaps
// (v_permlane16_swap: rows 0<->1 and 2<->3; v_permlane32_swap: halves).
template <int CTRL>
__device__ __forceinline__ int dpp_row(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ int wave_max_all(int v) {
  v = max(v, dpp_row<0xB1>(v));
  v = max(v, dpp_row<0x4E>(v));
  v = max(v, dpp_row<0x141>(v));
  v = max(v, dpp_row<0x140>(v));
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max((int)a[0], (int)a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((int)b[0], (int)b[1]);
}
__device__ __forceinline__ int wave_min_all(int v) {
  v = min(v, dpp_row<0xB1>(v));
  v = min(v, dpp_row<0x4E>(v));
  v = min(v, dpp_row<0x141>(v));
  v = min(v, dpp_row<0x140>(v));
  const auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = min((int)a[0], (int)a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return min((int)b[0], (int)b[1]);
}

// Butterfly reduce-scatter over the 64 lanes.  Each lane starts with N
// partial sums v[0..N-1]; at each step it keeps the half of its values picked
// by one bit of its lane id and adds the partner lane's copy of that half, the
// partner differing in that bit and agreeing in the bits already used.  xor 32
// and xor 16 go through ds_bpermute; the lower bits use DPP: row_mirror
// (i <-> 15-i) flips bit 3, row_half_mirror (i <-> 7-i) flips bit 2, and the
// quad permutations flip bits 1 and 0 -- each pairing also flips lower bits,
// which is harmless because those have not been used yet.
// The value of lane l ^ 32 / l ^ 16 by the gfx950 row swaps (no LDS round
// trip): with both operands a, v_permlane32_swap returns {lanes 0-31 of a
// in both halves, lanes 32-63 of a in both halves} and v_permlane16_swap
// {the even rows of a in both rows of each pair, the odd rows likewise}.
__device__ __forceinline__ float xchg32(float a) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false,
                                                  false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}
__device__ __forceinline__ float xchg16(float a) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false,
                                                  false);
  return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}
__device__ __forceinline__ float xchg_b3(float a) { return dpp_f<0x140>(a); }
__device__ __forceinline__ float xchg_b2(float a) { return dpp_f<0x141>(a); }
__device__ __forceinline__ float xchg_b1(float a) { return dpp_f<0x4E>(a); }
__device__ __forceinline__ float xchg_b0(float a) { return dpp_f<0xB1>(a); }

// 16 values: on return every lane holds the 64-lane total of value
// j = 8*bit5 + 4*bit4 + 2*bit3 + bit2 of its lane id.
__device__ __forceinline__ float butterfly16(const float (&v)[16]) {
  const int lane = threadIdx.x & 63;
  const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8, b2 = lane & 4;
  float a[8], b[4], c[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) a[j] = (b5 ? v[8 + j] : v[j]) + xchg32(b5 ? v[j] : v[8 + j]);
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = (b4 ? a[4 + j] : a[j]) + xchg16(b4 ? a[j] : a[4 + j]);
#pragma unroll
  for (int j = 0; j < 2; ++j) c[j] = (b3 ? b[2 + j] : b[j]) + xchg_b3(b3 ? b[j] : b[2 + j]);
  float d = (b2 ? c[1] : c[0]) + xchg_b2(b2 ? c[0] : c[1]);
  d += xchg_b1(d);
  d += xchg_b0(d);
  return d;
}

// 8 values: every lane ends with the total of value
// j = 4*bit5 + 2*bit4 + bit3 of its lane id.
__device__ __forceinline__ float butterfly8(const float (&v)[8]) {
  const int lane = threadIdx.x & 63;
  const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
  float a[4], b[2];
#pragma unroll
  for (int j = 0; j < 4; ++j) a[j] = (b5 ? v[4 + j] : v[j]) + xchg32(b5 ? v[j] : v[4 + j]);
#pragma unroll
  for (int j = 0; j < 2; ++j) b[j] = (b4 ? a[2 + j] : a[j]) + xchg16(b4 ? a[j] : a[2 + j]);
  float c = (b3 ? b[1] : b[0]) + xchg_b3(b3 ? b[0] : b[1]);
  c += xchg_b2(c);
  c += xchg_b1(c);
  c += xchg_b0(c);
  return c;
}

// 32 values: every lane ends with the total of value
// j = 16*bit5 + 8*bit4 + 4*bit3 + 2*bit2 + bit1 of its lane id.
__device__ __forceinline__ float butterfly32(const float (&v)[32]) {
  const int lane = threadIdx.x & 63;
  const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8, b2 = lane & 4, b1 = lane & 2;
  float a[16], b[8], c[4], d[2];
#pragma unroll
  for (int j = 0; j < 16; ++j) a[j] = (b5 ? v[16 + j] : v[j]) + xchg32(b5 ? v[j] : v[16 + j]);
#pragma unroll
  for (int j = 0; j < 8; ++j) b[j] = (b4 ? a[8 + j] : a[j]) + xchg16(b4 ? a[j] : a[8 + j]);
#pragma unroll
  for (int j = 0; j < 4; ++j) c[j] = (b3 ? b[4 + j] : b[j]) + xchg_b3(b3 ? b[j] : b[4 + j]);
#pragma unroll
  for (int j = 0; j < 2; ++j) d[j] = (b2 ? c[2 + j] : c[j]) + xchg_b2(b2 ? c[j] : c[2 + j]);
  float e = (b1 ? d[1] : d[0]) + xchg_b1(b1 ? d[0] : d[1]);
  e += xchg_b0(e);
  return e;
}

// Max over aligned groups of G lanes (G = 2, 4, 8, 16, 32 or 64), in every
// lane of the group: DPP inside rows of 16 (quad_perm [1,0,3,2], quad_perm
// [2,3,0,1], row_half_mirror, row_mirror -- each pairs the halves of the
// next larger group), the gfx950 row swaps above.  A maximum does not depend
// on the order of its operands, so this is the same value as any other tree.
template <int CTRL>
__device__ __forceinline__ float dpp_rowf(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int G>
__device__ __forceinline__ float group_max(float v) {
  static_assert(G == 2 || G == 4 || G == 8 || G == 16 || G == 32 || G == 64, "group size");
  v = fmaxf(v, dpp_rowf<0xB1>(v));
  if constexpr (G >= 4) v = fmaxf(v, dpp_rowf<0x4E>(v));
  if constexpr (G >= 8) v = fmaxf(v, dpp_rowf<0x141>(v));
  if constexpr (G >= 16) v = fmaxf(v, dpp_rowf<0x140>(v));
  if constexpr (G >= 32) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  }
  if constexpr (G >= 64) {
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    v = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
  }
  return v;
}
__device__ __forceinline__ float wave_max(float v) { return group_max<64>(v); }

__device__ __forceinline__ float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

// Workspace control block: word 0 = status bits, then the tagged slots of
// the fence-free exchanges (zero between launches).
struct WsCtl {
  uint32_t status;
  uint32_t pad[63];
  // VALU GEMV path: h slots [row 32][4096] (publish_h)
  uint64_t h_slots[32 * 4096];
  // small-T router: group sums [H/256 <= 32][T <= 4][E <= 256]
  uint64_t route_slots[32 * 4 * 256];
  // one-token fused expert kernel (decode.hip): the launch epoch, the count
  // of its finished blocks, per-128-block counts of published gate+up units,
  // then words tagged with the epoch
  // (never cleared): h values [row 8][2048] and requantised h [row 8][16
  // blocks of 128][32 code words + 1 scale word, padded to 36]
  uint32_t dec_epoch, dec_done;
  uint32_t pad2[62];
  uint32_t dec_cnt[8 * 16];  // per 128-block of h: gate+up units published (zero between launches)
  uint64_t dec_h[8 * 2048];
  uint64_t dec_c[8 * 16 * 36];
};

__device__ __forceinline__ void set_status(uint32_t* st, uint32_t bit) { atomicOr(st, bit); }

__device__ __forceinline__ float silu_mul_accurate(float g, float u) {
  return g / (1.0f + expf(-g)) * u;
}

// Exclusive prefix sum of v over a block of exactly 256 threads.  s_tmp holds
// >= 4 ints.  Returns the prefix; *total receives the block sum.  All
// threads must call it.
__device__ __forceinline__ int block256_exclusive_scan(int v, int* s_tmp, int* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int inc = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int t = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += t;
  }
  if (lane == 63) s_tmp[wv] = inc;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int s = s_tmp[i];
    base += (i < wv) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return base + inc - v;
}

// Group lookup for ragged grouped work.  Groups g = 0..G-1 (G <= 512) own
// units[g] consecutive work items, units[g] = f(count of rows of g) with
// count = offsets[g+1]-offsets[g].  Given a linear item index `item`, find
// (group, index inside the group).  Returns the group or -1 when `item` is
// past the last item.  All 256 threads of the block must call it.
template <typename UnitsOf>
__device__ __forceinline__ int find_group_item(const int32_t* __restrict__ offsets, int G, int item,
                                               UnitsOf units_of, int* s_tmp /* >= 6 ints */,
                                               int* local_item) {
  const int t = threadIdx.x;
  const int ga = t, gb = t + 256;
  int ca = 0, cb = 0;
  if (ga < G) ca = offsets[ga + 1] - offsets[ga];
  if (gb < G) cb = offsets[gb + 1] - offsets[gb];
  const int ua = (ga < G) ? units_of(ga, ca) : 0;
  const int ub = (gb < G) ? units_of(gb, cb) : 0;
  if (t == 0) {
    s_tmp[4] = -1;
    s_tmp[5] = 0;
  }
  int tot_a, tot_b;
  const int pa = block256_exclusive_scan(ua, s_tmp, &tot_a);
  const int pb = block256_exclusive_scan(ub, s_tmp, &tot_b) + tot_a;
  if (ua > 0 && item >= pa && item < pa + ua) {
    s_tmp[4] = ga;
    s_tmp[5] = item - pa;
  }
  if (ub > 0 && item >= pb && item < pb + ub) {
    s_tmp[4] = gb;
    s_tmp[5] = item - pb;
  }
  __syncthreads();
  const int g = s_tmp[4];
  *local_item = s_tmp[5];
  __syncthreads();
  return g;
}

}  // namespace bef
