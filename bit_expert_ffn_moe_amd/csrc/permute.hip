// permute.hip -- S4, the stable counting sort of (token, slot) pairs by expert.
//
// Reading each expert's weights once for all of its tokens is what makes
// batching pay (dpshk.com article, section "核心实现三").  The sort is
// deterministic and atomic-free: every expert's rows are assigned by one
// thread walking the pairs in token order, so rows inside an expert are in
// ascending token order and repeated runs give identical tables.
//
// Tables: offsets[E+2] (group g = expert g, group E = the shared expert with
// every token), row_token[T*k+T], row_of[T][k+1].  An id outside [0, E) is
// dropped: row_of = -1 and the status bit is set.
#include "common.h"
#include "kernels.h"

namespace bef {

// One block for small T*k (<= kPermuteSmallPairs): ids staged in LDS, thread e
// counts expert e, block scan gives the offsets, thread e then walks the
// pairs again and assigns its rows.
__global__ __launch_bounds__(256) void permute_small_kernel(
    const int32_t* __restrict__ ids, int T, int k, int E, int32_t* __restrict__ offsets,
    int32_t* __restrict__ row_token, int32_t* __restrict__ row_of, uint32_t* __restrict__ status) {
  __shared__ int32_t sid[kPermuteSmallPairs];
  __shared__ int stmp[8];
  __shared__ int s_bad;
  const int P = T * k;
  const int tid = threadIdx.x;
  if (tid == 0) s_bad = 0;
  for (int p = tid; p < P; p += 256) sid[p] = ids[p];
  __syncthreads();
  int bad = 0;
  for (int p = tid; p < P; p += 256) {
    const int e = sid[p];
    if (e < 0 || e >= E) {
      row_of[(size_t)(p / k) * (k + 1) + (p % k)] = -1;
      bad = 1;
    }
  }
  if (bad) s_bad = 1;
  int cnt = 0;
  if (tid < E)
    for (int p = 0; p < P; ++p) cnt += (sid[p] == tid);
  int total;
  const int pre = block256_exclusive_scan(tid < E ? cnt : 0, stmp, &total);
  if (tid < E) offsets[tid] = pre;
  if (tid == 0) {
    offsets[E] = total;
    offsets[E + 1] = total + T;
    if (s_bad) set_status(status, MOE_STATUS_BAD_EXPERT_ID_DEV);
  }
  if (tid < E && cnt > 0) {
    int r = pre;
    for (int p = 0; p < P; ++p) {
      if (sid[p] == tid) {
        row_token[r] = p / k;
        row_of[(size_t)(p / k) * (k + 1) + (p % k)] = r;
        ++r;
      }
    }
  }
  for (int t = tid; t < T; t += 256) {
    row_token[total + t] = t;
    row_of[(size_t)t * (k + 1) + k] = total + t;
  }
}

// Large T: three passes over token blocks of kPermuteTokBlock tokens.
// Pass 1: per-block counts cnt[b][e] (thread e walks the block's pairs).
__global__ __launch_bounds__(256) void permute_count_kernel(const int32_t* __restrict__ ids,
                                                            int T, int k, int E,
                                                            int32_t* __restrict__ cnt,
                                                            int32_t* __restrict__ row_of,
                                                            uint32_t* __restrict__ status) {
  __shared__ int32_t sid[kPermuteTokBlock * 16];
  const int b = blockIdx.x;
  const int t0 = b * kPermuteTokBlock;
  const int nt = min(kPermuteTokBlock, T - t0);
  const int P = nt * k;
  const int tid = threadIdx.x;
  int bad = 0;
  for (int p = tid; p < P; p += 256) {
    const int e = ids[(size_t)t0 * k + p];
    sid[p] = e;
    if (e < 0 || e >= E) {
      row_of[(size_t)(t0 + p / k) * (k + 1) + (p % k)] = -1;
      bad = 1;
    }
  }
  if (bad) set_status(status, MOE_STATUS_BAD_EXPERT_ID_DEV);
  __syncthreads();
  if (tid < E) {
    int c = 0;
    for (int p = 0; p < P; ++p) c += (sid[p] == tid);
    cnt[(size_t)b * E + tid] = c;
  }
}

// Pass 2 (one block): running sums over blocks per expert, scan over experts.
// base[b][e] = offsets[e] + sum_{b' < b} cnt[b'][e].
__global__ __launch_bounds__(256) void permute_scan_kernel(int nblk, int T, int E,
                                                           const int32_t* __restrict__ cnt,
                                                           int32_t* __restrict__ base,
                                                           int32_t* __restrict__ offsets) {
  __shared__ int stmp[8];
  const int e = threadIdx.x;
  int tot = 0;
  if (e < E)
    for (int b = 0; b < nblk; ++b) tot += cnt[(size_t)b * E + e];
  int total;
  const int pre = block256_exclusive_scan(e < E ? tot : 0, stmp, &total);
  if (e < E) {
    offsets[e] = pre;
    int run = pre;
    for (int b = 0; b < nblk; ++b) {
      base[(size_t)b * E + e] = run;
      run += cnt[(size_t)b * E + e];
    }
  }
  if (e == 0) {
    offsets[E] = total;
    offsets[E + 1] = total + T;
  }
}

// Pass 3: thread e walks its block's pairs in order and assigns its rows.
__global__ __launch_bounds__(256) void permute_scatter_kernel(
    const int32_t* __restrict__ ids, int T, int k, int E, const int32_t* __restrict__ base,
    const int32_t* __restrict__ offsets, int32_t* __restrict__ row_token,
    int32_t* __restrict__ row_of) {
  __shared__ int32_t sid[kPermuteTokBlock * 16];
  const int b = blockIdx.x;
  const int t0 = b * kPermuteTokBlock;
  const int nt = min(kPermuteTokBlock, T - t0);
  const int P = nt * k;
  const int tid = threadIdx.x;
  for (int p = tid; p < P; p += 256) sid[p] = ids[(size_t)t0 * k + p];
  __syncthreads();
  if (tid < E) {
    int r = base[(size_t)b * E + tid];
    for (int p = 0; p < P; ++p) {
      if (sid[p] == tid) {
        const int t = t0 + p / k;
        row_token[r] = t;
        row_of[(size_t)t * (k + 1) + (p % k)] = r;
        ++r;
      }
    }
  }
  const int shared0 = offsets[E];
  for (int i = tid; i < nt; i += 256) {
    const int t = t0 + i;
    row_token[shared0 + t] = t;
    row_of[(size_t)t * (k + 1) + k] = shared0 + t;
  }
}

hipError_t launch_permute(const int32_t* ids, int T, int k, int E, int32_t* offsets,
                          int32_t* row_token, int32_t* row_of, int32_t* cnt, int32_t* base,
                          uint32_t* status, hipStream_t st) {
  if ((int64_t)T * k <= kPermuteSmallPairs) {
    permute_small_kernel<<<1, 256, 0, st>>>(ids, T, k, E, offsets, row_token, row_of, status);
    return hipGetLastError();
  }
  const int nblk = (T + kPermuteTokBlock - 1) / kPermuteTokBlock;
  permute_count_kernel<<<nblk, 256, 0, st>>>(ids, T, k, E, cnt, row_of, status);
  permute_scan_kernel<<<1, 256, 0, st>>>(nblk, T, E, cnt, base, offsets);
  permute_scatter_kernel<<<nblk, 256, 0, st>>>(ids, T, k, E, base, offsets, row_token, row_of);
  return hipGetLastError();
}

}  // namespace bef
