// permute.hip -- S4, the stable counting sort of (token, slot) pairs by expert.
//
// Reading each expert's weights once for all of its tokens is what makes
// batching pay (dpshk.com article, section "核心实现三").  The sort is
// stable and deterministic: experts' counts come from LDS atomic adds (the
// order of the adds does not change a count), and a pair's row is its
// expert's base plus the number of earlier pairs of the same expert, counted
// a chunk of 256 pairs at a time -- inside a wave from ballots over the id
// bits, across the waves of a chunk from per-wave counts in LDS, across
// chunks from a running count -- so rows inside an expert are in ascending
// token order and repeated runs give identical tables.
//
// Tables: offsets[E+2] (group g = expert g, group E = the shared expert with
// every token), row_token[T*k+T], row_of[T][k+1].  An id outside [0, E) is
// dropped: row_of = -1 and the status bit is set.
#include "common.h"
#include "kernels.h"

namespace bef {

// Stable ranks of one chunk of 256 consecutive pairs, pair c0 + tid held by
// thread tid with expert e (valid: e in [0, E), E <= 256).  Returns the
// number of earlier pairs of the same expert in this chunk plus s_run[e],
// the count from the chunks before; then adds this chunk's counts to s_run.
// The lanes of a wave holding the same expert come from 8 ballots (one per
// bit of e); the counts of the earlier waves of the chunk go through
// s_hist, which must be zero on entry and is zero again on return.  All 256
// threads must call it (it holds barriers).
__device__ __forceinline__ int chunk_rank(int e, bool valid, int* s_run, int (*s_hist)[256]) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  uint64_t m = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    const bool on = (e >> bit) & 1;
    const uint64_t bb = __ballot(valid && on);
    m &= on ? bb : ~bb;
  }
  const int before = __popcll(m & ((1ull << lane) - 1ull));
  if (valid && before == 0) s_hist[w][e] = __popcll(m);
  __syncthreads();
  int r = 0;
  if (valid) {
    r = s_run[e] + before;
    for (int w2 = 0; w2 < w; ++w2) r += s_hist[w2][e];
  }
  __syncthreads();
  s_run[tid] += s_hist[0][tid] + s_hist[1][tid] + s_hist[2][tid] + s_hist[3][tid];
  s_hist[0][tid] = 0, s_hist[1][tid] = 0, s_hist[2][tid] = 0, s_hist[3][tid] = 0;
  __syncthreads();
  return r;
}

__device__ __forceinline__ void clear_rank_state(int* s_run, int (*s_hist)[256]) {
  const int tid = threadIdx.x;
  s_run[tid] = 0;
  s_hist[0][tid] = 0, s_hist[1][tid] = 0, s_hist[2][tid] = 0, s_hist[3][tid] = 0;
}

// One block for small T*k (<= kPermuteSmallPairs): counts by LDS atomics,
// block scan for the offsets, then the rows chunk by chunk.
__global__ __launch_bounds__(256) void permute_small_kernel(
    const int32_t* __restrict__ ids, int T, int k, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_token, int32_t* __restrict__ row_of, uint32_t* __restrict__ status) {
  __shared__ int s_cnt[256], s_run[256], s_hist[4][256];
  __shared__ int stmp[8];
  __shared__ int s_bad;
  const int P = T * k;
  const int tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  s_cnt[tid] = 0;
  clear_rank_state(s_run, s_hist);
  __syncthreads();
  for (int p = tid; p < P; p += 256) {
    const int e = ids[p];
    if (e < 0 || e >= E) {
      row_of[(size_t)(p / k) * (k + 1) + (p % k)] = -1;
      s_bad = 1;
    } else {
      atomicAdd(&s_cnt[e], 1);
    }
  }
  __syncthreads();
  const int cnt = tid < E ? s_cnt[tid] : 0;
  int total;
  const int pre = block256_exclusive_scan(cnt, stmp, &total);
  s_cnt[tid] = pre;  // each thread rewrites only the entry it read
  if (tid < E) offsets[tid] = pre;
  if (tid == 0) {
    offsets[E] = total;
    offsets[E + 1] = total + T;
    if (s_bad) set_status(status, MOE_STATUS_BAD_EXPERT_ID_DEV);
  }
  __syncthreads();
  for (int c0 = 0; c0 < P; c0 += 256) {
    const int p = c0 + tid;
    const int e = p < P ? ids[p] : -1;
    const bool valid = e >= 0 && e < E;
    const int r = chunk_rank(e, valid, s_run, s_hist);
    if (valid) {
      const int row = s_cnt[e] + r, t = p / k;
      row_token[row] = t;
      row_of[(size_t)t * (k + 1) + (p % k)] = row;
    }
  }
  for (int t = tid; t < T; t += 256) {
    row_token[total + t] = t;
    row_of[(size_t)t * (k + 1) + k] = total + t;
  }
}

// Large T: two passes over token blocks of kPermuteTokBlock tokens.
// Pass 1: per-block counts cnt[b][e] (LDS atomics).
__global__ __launch_bounds__(256) void permute_count_kernel(const int32_t* __restrict__ ids,
                                                            int T, int k, int E,
                                                            int32_t* __restrict__ cnt,
                                                            int32_t* __restrict__ row_of,
                                                            uint32_t* __restrict__ status) {
  __shared__ int s_cnt[256];
  const int b = blockIdx.x;
  const int t0 = b * kPermuteTokBlock;
  const int nt = min(kPermuteTokBlock, T - t0);
  const int P = nt * k;
  const int tid = threadIdx.x;
  s_cnt[tid] = 0;
  __syncthreads();
  int bad = 0;
  for (int p = tid; p < P; p += 256) {
    const int e = ids[(size_t)t0 * k + p];
    if (e < 0 || e >= E) {
      row_of[(size_t)(t0 + p / k) * (k + 1) + (p % k)] = -1;
      bad = 1;
    } else {
      atomicAdd(&s_cnt[e], 1);
    }
  }
  if (bad) set_status(status, MOE_STATUS_BAD_EXPERT_ID_DEV);
  __syncthreads();
  if (tid < E) cnt[(size_t)b * E + tid] = s_cnt[tid];
}

// Pass 2: block b forms its experts' bases from the counts of every block
// -- tot[e] = sum over all blocks, base[e] = offsets[e] + sum over blocks
// before b, with offsets the exclusive scan of tot over experts (block 0
// writes it) -- then its pairs get their rows chunk by chunk.
__global__ __launch_bounds__(256) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int T, int k, int E, int nblk,
    const int32_t* __restrict__ cnt, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_token, int32_t* __restrict__ row_of) {
  __shared__ int s_base[256], s_run[256], s_hist[4][256];
  __shared__ int stmp[8];
  const int b = blockIdx.x;
  const int t0 = b * kPermuteTokBlock;
  const int nt = min(kPermuteTokBlock, T - t0);
  const int P = nt * k;
  const int tid = threadIdx.x;
  int before = 0, tot = 0;
  if (tid < E) {
    // 8 counts in flight at a time
    for (int b0 = 0; b0 < nblk; b0 += 8) {
      int c[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        c[j] = (b0 + j < nblk) ? cnt[(size_t)(b0 + j) * E + tid] : 0;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        tot += c[j];
        before += (b0 + j < b) ? c[j] : 0;
      }
    }
  }
  int total;
  const int pre = block256_exclusive_scan(tid < E ? tot : 0, stmp, &total);
  s_base[tid] = tid < E ? pre + before : 0;
  if (b == 0) {
    if (tid < E) offsets[tid] = pre;
    if (tid == 0) {
      offsets[E] = total;
      offsets[E + 1] = total + T;
    }
  }
  clear_rank_state(s_run, s_hist);
  __syncthreads();
  for (int c0 = 0; c0 < P; c0 += 256) {
    const int p = c0 + tid;
    const int e = p < P ? ids[(size_t)t0 * k + p] : -1;
    const bool valid = e >= 0 && e < E;
    const int r = chunk_rank(e, valid, s_run, s_hist);
    if (valid) {
      const int row = s_base[e] + r, t = t0 + p / k;
      row_token[row] = t;
      row_of[(size_t)t * (k + 1) + (p % k)] = row;
    }
  }
  for (int i = tid; i < nt; i += 256) {
    const int t = t0 + i;
    row_token[total + t] = t;
    row_of[(size_t)t * (k + 1) + k] = total + t;
  }
}

hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* offsets,
                          int32_t* row_token, int32_t* row_of, int32_t* cnt,
                          uint32_t* status, hipStream_t st) {
  if (E < 1 || E > 256 || k < 1) return hipErrorInvalidValue;  // one thread per expert
  if ((int64_t)T * k <= kPermuteSmallPairs) {
    permute_small_kernel<<<1, 256, 0, st>>>(ids, T, k, E, offsets, row_token, row_of, status);
    return hipGetLastError();
  }
  const int nblk = (T + kPermuteTokBlock - 1) / kPermuteTokBlock;
  permute_count_kernel<<<nblk, 256, 0, st>>>(ids, T, k, E, cnt, row_of, status);
  permute_scatter_kernel<<<nblk, 256, 0, st>>>(ids, T, k, E, nblk, cnt, offsets, row_token,
                                              row_of);
  return hipGetLastError();
}

}  // namespace bef
