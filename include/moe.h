/*
 * moe.h -- C ABI of the MI355X (gfx950) routed-expert MoE FFN library.
 *
 * The layer: 256 routed experts, top-6 per token, plus one always-on shared
 * expert (tcti.cn post on DeepSeek-V4-Flash on 4x RTX 2080 Ti, section
 * "DeepSeek-V4-Flash的可能性"; ai-muninn.com "[洋垃圾跑大模型 #3]", section
 * "目標不是「載得進去」...").  Expert weights are FP4 E2M1 with one UE8M0
 * scale per 32 inputs, or FP8 E4M3 with one fp32 scale per 128x128 block;
 * activations are FP8 E4M3 with one fp32 scale (amax/448) per 128.  The
 * pages name the operators this ABI exposes: act_quant feeding the low-bit
 * linears, fp4_gemm (FP8-quantised activation x FP4 packed weight) and
 * fp8_gemm (tcti.cn post, section "补齐软件栈缺失"); the router picks the
 * token's experts first (dpshk.com article on deepseek-v4-flash-0731-in-c,
 * section "核心实现一"); each expert is read once for all of its tokens
 * (same article, "核心实现三"); dequantisation happens inside the product,
 * gate and up share one quantised input, and workspaces are allocated once
 * and reused (same article, "核心实现四").
 *
 * Conventions for every call:
 *  - Every buffer is a DEVICE pointer owned by the caller.  The library never
 *    allocates, frees or synchronises inside these calls (the debug helpers
 *    at the end are the only exceptions and say so).
 *  - Arguments are validated on the host first; on any error nothing is
 *    enqueued and a negative MOE_E* status is returned.  Otherwise the work
 *    is enqueued on `stream` (a hipStream_t passed as void*; NULL = the
 *    default stream) and MOE_OK is returned.  MOE_ELAUNCH means the HIP
 *    launch itself failed (the HIP error is cleared).
 *  - All device pointers must be 16-byte aligned (MOE_EALIGN otherwise);
 *    `ws` must be 256-byte aligned.
 *  - bf16 values are passed as their uint16_t bit patterns.
 *  - Expert ids outside [0, E) found on the device are skipped (their rows
 *    produce zero contribution) and set bit MOE_STATUS_BAD_EXPERT_ID in the
 *    workspace status word; no memory is accessed out of bounds.
 *  - Calls are reentrant for distinct workspaces; two calls in flight on the
 *    same workspace race.
 *  - Limits: 1 <= E <= 256, 1 <= k <= min(E, 16), H and I multiples of 128,
 *    128 <= H <= 8192, 128 <= I <= 8192, 0 <= T <= 262144 (MOE_ENOTSUP
 *    beyond the size limits, MOE_EINVAL for malformed values).  The device must be a
 *    gfx950 (MOE_ENOTSUP otherwise).
 *  - T = 0 (rows = 0 for act_quant_fp8) is an empty batch: the other
 *    arguments are checked as usual, then MOE_OK is returned with nothing
 *    read, written or enqueued (no device is needed for that answer).
 */
#ifndef BEF_MOE_H
#define BEF_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_OK = 0,
  MOE_EINVAL = -1,     /* null pointer, bad size, unknown dtype            */
  MOE_ENOTSUP = -2,    /* not a gfx950 device, unknown format, size limit   */
  MOE_EALIGN = -3,     /* pointer not 16-byte (ws: 256-byte) aligned        */
  MOE_EWORKSPACE = -4, /* workspace smaller than moe_workspace_bytes()      */
  MOE_ELAUNCH = -5     /* a HIP launch failed                               */
};

/* Weight formats. */
enum {
  MOE_W_FP4_E2M1_UE8M0_K32 = 1, /* E2M1 codes 2/byte (element 2j in bits 0-3),
                                   one UE8M0 byte per 32 inputs               */
  MOE_W_FP8_E4M3_F32_B128 = 2   /* E4M3 codes, one fp32 per 128x128 block     */
};

/* Activation / output dtypes. */
enum { MOE_DT_BF16 = 1, MOE_DT_F32 = 2 };

/* Device status word bits (see moe_device_status).  MOE_STATUS_SYNC_TIMEOUT:
 * on the small-T router or the one-token path, a block waiting for the
 * values of other blocks gave up after its bounded wait; the results of that
 * call are invalid, and the workspace must go through moe_workspace_init
 * again before its next use (a late value could outlive the clean-up). */
enum { MOE_STATUS_BAD_EXPERT_ID = 1u, MOE_STATUS_SYNC_TIMEOUT = 2u };

/* Stacked expert weights, expert-major; slot E (the last) is the shared
 * expert, which must have the same intermediate size as the routed ones.
 * Matrices are [out][in] row-major.
 *   FP4: gate_q/up_q [E+1][I][H/2] u8, gate_s/up_s [E+1][I][H/32] u8,
 *        down_q [E+1][H][I/2] u8,     down_s [E+1][H][I/32] u8.
 *   FP8: gate_q/up_q [E+1][I][H] u8,   gate_s/up_s [E+1][I/128][H/128] f32,
 *        down_q [E+1][H][I] u8,       down_s [E+1][H/128][I/128] f32.
 * The descriptor itself is host memory, read during the call only. */
typedef struct moe_weights {
  int32_t format;    /* MOE_W_*                      */
  int32_t n_experts; /* E, routed experts            */
  int32_t hidden;    /* H                            */
  int32_t inter;     /* I, expert intermediate size  */
  const void* gate_q;
  const void* gate_s;
  const void* up_q;
  const void* up_s;
  const void* down_q;
  const void* down_s;
} moe_weights;

/* Bytes of workspace needed by any call below for up to `max_tokens` tokens
 * at top-k `top_k` (router partials, quantised activations, routing tables,
 * intermediate h, y rows, status word).  0 if the arguments are invalid or
 * max_tokens < 1.
 * Allocate once, call moe_workspace_init once, then reuse for every call
 * (dpshk.com article, section "核心实现四": workspaces preallocated). */
size_t moe_workspace_bytes(const moe_weights* w, int32_t max_tokens, int32_t top_k);

/* Enqueue a zero-fill of the workspace's control block (about 1.3 MB: the
 * status word and the slots through which blocks of one launch hand each
 * other router partials and h values without device-scope fences; a slot
 * holds a valid mark with its value, and the block that consumes it clears
 * it, so the slots must start zeroed).  Call once after allocating a
 * workspace, before its first use (and again after MOE_STATUS_SYNC_TIMEOUT);
 * the kernels keep the control block consistent from then on. */
int moe_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* S1+S2, the router (dpshk.com article, section "核心实现一"; top-6 of 256:
 * ai-muninn.com "[洋垃圾跑大模型 #3]").
 *   x        [T][H] bf16 activations
 *   w_router [H][E] bf16
 *   topk_ids [T][k] int32 out: experts ordered by (logit desc, id asc)
 *   topk_w   [T][k] f32 out: sigmoid(logit) renormalised over the k chosen
 * Logits are fp32 sums of the exact bf16 x bf16 products in a fixed order
 * for a given T: below 256 tokens, 64-wide chunk partials (chains of fused
 * multiply-adds in ascending h from +0), sums of 4 consecutive chunks in
 * ascending order, those group sums in ascending order; from 256 tokens on,
 * sums over 512-row groups formed on the matrix cores (bf16 MFMA, fp32
 * accumulation in the hardware's order), added in ascending group order.
 * The ids are deterministic.  They are the
 * exact top-k of these logits; logits summed in any other order differ by
 * rounding only, so another order can rank two experts differently only
 * where their logits lie within rounding distance of each other.
 * ws: workspace of at least moe_workspace_bytes(.., T, k). */
int moe_route(const uint16_t* x, const uint16_t* w_router, int32_t T, int32_t H, int32_t E,
              int32_t k, int32_t* topk_ids, float* topk_w, void* ws, size_t ws_bytes,
              void* stream);

/* S3, act_quant (tcti.cn post, section "补齐软件栈缺失"): per row and per
 * 128 columns, s = amax/448 (fp32, IEEE division) and
 * q = E4M3(x / s) rounded to nearest even, saturating at +-448, sign kept;
 * an all-zero block gives s = 0 and q = 0.
 *   x      [rows][cols] bf16 (x_dtype MOE_DT_BF16) or f32 (MOE_DT_F32)
 *   q      [rows][cols] u8 E4M3 codes out
 *   scales [rows][cols/128] f32 out
 * cols must be a multiple of 128; rows >= 0. */
int act_quant_fp8(const void* x, int32_t x_dtype, int64_t rows, int32_t cols, uint8_t* q,
                  float* scales, void* stream);

/* S4, permute (dpshk.com article, section "核心实现三": each expert read
 * once for all of its tokens): a stable counting sort of the T*k
 * (token, slot) pairs by expert, tokens ascending within an expert, then
 * the shared-expert group (index E) holding tokens 0..T-1.
 *   offsets   [E+2] out: group g is rows offsets[g] .. offsets[g+1]-1
 *   row_token [T*k+T] out: token of each row
 *   row_of    [T][k+1] out: row of (t, slot j); row_of[t][k] = shared row;
 *             -1 for a pair whose id is outside [0, E)
 * Rows that a dropped pair would have used are never written. */
int moe_permute(const int32_t* topk_ids, int32_t T, int32_t k, int32_t E, int32_t* offsets,
                int32_t* row_token, int32_t* row_of, void* ws, size_t ws_bytes, void* stream);

/* S5+S6, the experts (tcti.cn post, section "补齐软件栈缺失": fp4_gemm and
 * fp8_gemm; dpshk.com article, section "核心实现四": dequantise inside the
 * product, gate and up share one quantised input).  For every row r of
 * group g (expert g, or the shared expert for g = E) and its token t:
 *   g = W_gate[g] . deq(xq[t]),  u = W_up[g] . deq(xq[t])   (fp32 accumulate)
 *   h = silu(g) * u, requantised to E4M3 per 128 exactly as act_quant_fp8
 *   y_rows[r] = W_down[g] . deq(hq)
 *   xq [T][H] u8, xs [T][H/128] f32 (act_quant_fp8 of x)
 *   offsets, row_token as produced by moe_permute
 *   y_rows [T*k+T][H] f32 out (rows of dropped pairs are left untouched)
 * A few tokens -- 1 <= T <= 4 with k+1 <= 8, T*(k+1) <= 32, H <= 8192 and
 * I <= 4096, either weight format -- run the VALU GEMV kernels (weights
 * streamed from HBM into registers, no matrix-core tile to fill); any other
 * shape runs the MFMA grouped GEMM kernels. */
int moe_expert_ffn(const moe_weights* w, const uint8_t* xq, const float* xs, int32_t T, int32_t k,
                   const int32_t* offsets, const int32_t* row_token, float* y_rows, void* ws,
                   size_t ws_bytes, void* stream);

/* S5 alone: gate + up + SwiGLU for every row, h requantised to E4M3 per 128
 * and kept in `ws` for moe_expert_down (same kernels moe_expert_ffn runs
 * first; arguments as moe_expert_ffn). */
int moe_expert_gate_up(const moe_weights* w, const uint8_t* xq, const float* xs, int32_t T,
                       int32_t k, const int32_t* offsets, const int32_t* row_token, void* ws,
                       size_t ws_bytes, void* stream);

/* S6 alone (+ S7): the down projection of the h that moe_expert_gate_up left
 * in `ws` (same T, k, offsets), into y_rows [T*k+T][H] f32.  When `out` is
 * set the combine (S7) follows, using row_of and topk_w: on the VALU GEMV
 * path (see moe_expert_ffn) it is fused into the down kernel and y_rows may
 * be NULL; on the MFMA path y_rows is required and a combine kernel runs. */
int moe_expert_down(const moe_weights* w, int32_t T, int32_t k, const int32_t* offsets,
                    const int32_t* row_of, const float* topk_w, float* y_rows, void* out,
                    int32_t out_dtype, void* ws, size_t ws_bytes, void* stream);

/* S7, combine: the always-on shared expert's output plus the token's routed
 * experts' outputs weighted by their gate weights (tcti.cn post, section
 * "DeepSeek-V4-Flash的可能性": top-6 routed experts beside one shared
 * expert; the rows come back from the expert-major order of the batch,
 * dpshk.com article, section "核心实现三"):
 *   out[t] = y_rows[row_of[t][k]] + sum_{j<k} topk_w[t][j] * y_rows[row_of[t][j]]
 * in fp32 in that order (rows of -1 contribute 0), written as bf16 (nearest
 * even) or f32.
 *   y_rows [rows][H] f32, row_of [T][k+1] int32, topk_w [T][k] f32
 *   out [T][H] (out_dtype MOE_DT_BF16 or MOE_DT_F32)
 * Limits as for every call: 1 <= k <= 16, 0 <= T <= 262144, H a multiple of
 * 128 up to 8192. */
int moe_combine(const float* y_rows, const int32_t* row_of, const float* topk_w, int32_t T,
                int32_t k, int32_t H, void* out, int32_t out_dtype, void* stream);

/* The whole layer, S1..S7, on x [T][H] bf16 -> out [T][H] (bf16 or f32).
 * routing_ids/routing_w [T][k] (both NULL, or both set) inject routing
 * (e.g. a drawn routing, or a speculative-verification batch whose routing
 * is known, dpshk.com article section "核心实现三"); when NULL the router
 * runs on x. */
int dsv4_moe_forward(const moe_weights* w, const uint16_t* w_router, const uint16_t* x, int32_t T,
                     int32_t k, const int32_t* routing_ids, const float* routing_w, void* out,
                     int32_t out_dtype, void* ws, size_t ws_bytes, void* stream);

/* The whole layer as dsv4_moe_forward, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): no workspace argument, no allocation of
 * any kind.  The workspace is a file-scope device array of the library,
 * MOE_NOALLOC_SCRATCH_BYTES bytes on each GPU it runs on, held until the
 * process ends; its device address is looked up on the first call on a
 * device (that device current), and its control block is then cleared by a
 * fill kernel enqueued on `stream`.  A call whose workspace need
 * (moe_workspace_bytes(w, T, k)) exceeds the array returns MOE_ENOTSUP with
 * nothing enqueued -- about 100 tokens at hidden 4096, intermediate 2048,
 * top-6.  Every call on one GPU shares that array: two calls in flight at
 * once on one GPU (different streams, or different threads) race and give
 * wrong results.  Results equal dsv4_moe_forward's bit for bit (same
 * kernels).  Its status word cannot be read (moe_device_status needs a
 * workspace); bad expert ids are still skipped. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
int dsv4_moe_forward_noalloc(const moe_weights* w, const uint16_t* w_router, const uint16_t* x,
                             int32_t T, int32_t k, const int32_t* routing_ids,
                             const float* routing_w, void* out, int32_t out_dtype, void* stream);

/* ---- Host-resident experts ------------------------------------------------
 * For layers whose routed experts do not all fit in HBM, the pages keep the
 * routed experts in host memory and move each to the GPU when a token needs
 * it, computing on arrival, with a per-layer LRU cache of experts on the GPU
 * and double-buffered copies (dpshk.com article, sections "核心实现一" and
 * "核心实现二"; tcti.cn post, section "DeepSeek-V4-Flash的可能性": routed
 * experts in host memory).  Here: one layer's cache is n_slots expert slots
 * in HBM plus one slot for the shared expert; a call routes on the GPU,
 * reads the ids back (it synchronises `stream` once for that), keeps hits in
 * their slots, copies each miss into a free or least-recently-used slot on
 * `copy_stream`, runs the experts already resident at once and the copied
 * ones when `copies_done` (recorded after the last copy) has fired, then
 * combines.  Expert math and the combine order are those of
 * dsv4_moe_forward.
 *
 * The cache state lives in caller-owned HOST memory:
 *   n_experts = E of the layer, n_slots = slots in HBM (1..E),
 *   slot_of [E] (slot of expert e or -1), expert_of [n_slots] (-1 if free),
 *   last_use [n_slots] (call count of last use), initially all -1 / -1 / 0,
 *   calls = 0, shared_resident = 0 (the first call copies the shared
 *   expert into slot n_slots, where it stays); hits, misses, bytes_copied
 *   count distinct experts per call and bytes sent to the GPU. */
typedef struct moe_expert_cache {
  int32_t n_experts;
  int32_t n_slots;
  int32_t* slot_of;
  int32_t* expert_of;
  uint64_t* last_use;
  uint64_t calls;
  int32_t shared_resident;
  int32_t pad_;
  uint64_t hits, misses, bytes_copied;
} moe_expert_cache;

/* Workspace bytes (device) of moe_forward_host_experts for up to max_tokens
 * tokens of the layer `host_w` (0 on invalid arguments). */
size_t moe_host_experts_workspace_bytes(const moe_weights* host_w, int32_t max_tokens,
                                        int32_t top_k);

/* Pinned host scratch bytes of moe_forward_host_experts (ids read back, slot
 * ids and group masks staged for upload). */
size_t moe_host_experts_scratch_bytes(int32_t n_experts, int32_t max_tokens, int32_t top_k);

/* The whole layer with routed experts in host memory (see above).
 *   host_w: the layer's E+1 experts in HOST memory (pinned for asynchronous
 *           copies), layout as moe_weights;
 *   slot_w: the cache's slots in DEVICE memory, n_experts = n_slots: slot s
 *           of each array holds one expert, slot n_slots the shared expert;
 *   w_router [H][E], x [T][H] bf16 on the device; out [T][H] bf16 or f32;
 *   ws: device workspace of moe_host_experts_workspace_bytes (moe_workspace_init
 *       once), host_scratch: pinned host memory of
 *       moe_host_experts_scratch_bytes;
 *   copies_done: a hipEvent_t (void*) the call records on copy_stream;
 *   stream: compute stream; copy_stream: host-to-device copies.
 * Requires every expert of a call to fit at once: T*k <= n_slots unless
 * n_slots = E (MOE_ENOTSUP otherwise).  Synchronises `stream` once (the ids
 * must reach the host to choose the copies); returns with the copies and the
 * layer enqueued.  Reentrant only for distinct caches, slots, workspaces and
 * streams. */
int moe_forward_host_experts(const moe_weights* host_w, const moe_weights* slot_w,
                             moe_expert_cache* cache, const uint16_t* w_router, const uint16_t* x,
                             int32_t T, int32_t k, void* out, int32_t out_dtype, void* ws,
                             size_t ws_bytes, void* host_scratch, size_t host_scratch_bytes,
                             void* copies_done, void* stream, void* copy_stream);

/* A static string naming a status code. */
const char* moe_status_string(int status);

/* DEBUG/TESTS ONLY -- synchronises `stream`.  Reads the workspace status
 * word into *status (MOE_STATUS_* bits) and clears it when `clear` != 0. */
int moe_device_status(void* ws, void* stream, uint32_t* status, int clear);

/* DEBUG/TESTS ONLY -- device pointers to the intermediate activations that
 * the last moe_expert_ffn / dsv4_moe_forward call with the same (w, T, k)
 * left in `ws`: h [T*k+T][I] f32 (VALU path only, else NULL), and
 * hq [T*k+T][I] u8 with hs [T*k+T][I/128] f32 (both paths).  T >= 1 (an
 * empty batch leaves none: MOE_EINVAL). */
int moe_debug_intermediates(const moe_weights* w, int32_t T, int32_t k, void* ws,
                            size_t ws_bytes, float** h, uint8_t** hq, float** hs);

/* DEBUG/TESTS ONLY -- while set, every MFMA grouped-GEMM gate+up launch of
 * a call with (T*k+T)*I <= n_floats also stores its fp32 h (SwiGLU output,
 * before requantisation) into h [T*k+T][I] (device memory owned by the
 * caller, 16-byte aligned); the VALU path keeps its h in the workspace (see
 * moe_debug_intermediates).  NULL and 0 clear it.  Process-wide and not
 * thread-safe.  MOE_EINVAL if exactly one of h, n_floats is zero. */
int moe_debug_store_h(float* h, size_t n_floats);

/* DEBUG/TESTS ONLY -- device pointers to the expert ids [T][k] int32 and
 * weights [T][k] f32 that the router of the last dsv4_moe_forward call with
 * the same (w, T, k) and no injected routing left in `ws`.  T >= 1. */
int moe_debug_routing(const moe_weights* w, int32_t T, int32_t k, void* ws, size_t ws_bytes,
                      int32_t** ids, float** topk_w);

/* Kernels that moe_debug_time_kernel can time: the gate+up and the down
 * kernels of the VALU path (GEMV) and of the grouped GEMM, and the fused
 * one-token expert kernel (gate+up, down and combine in one launch). */
enum {
  MOE_KERNEL_GEMV_GATE_UP = 1,
  MOE_KERNEL_GEMM_GATE_UP = 2,
  MOE_KERNEL_GEMV_DOWN = 3,
  MOE_KERNEL_GEMM_DOWN = 4,
  MOE_KERNEL_DECODE_FFN = 5
};

/* DEBUG/BENCHMARK ONLY -- the one-token path of dsv4_moe_forward with the
 * router on the device and FP4 weights: `fused` = 1 runs the routed experts'
 * gate+up, the down projection of all k + 1 experts and the combine as one
 * persistent kernel wherever it fits (T = 1, k + 1 <= 8, inter <= 2048,
 * hidden <= 4096 and a multiple of 16 with hidden / 16 <= the device's
 * compute units), 0 (the default: measured faster) the separate gate+up and
 * down+combine kernels.  Both give bit-identical outputs.  The fused kernel runs one block per compute unit
 * and its blocks wait on each other's results (bounded waits): it expects
 * the device to itself for its duration; when other work holds compute
 * units, the waits may run out, which sets MOE_STATUS_SYNC_TIMEOUT.
 * Process-wide and not thread-safe; MOE_EINVAL for other values. */
int moe_debug_set_decode_fused(int32_t fused);

/* DEBUG/BENCHMARK ONLY -- kernel timing.  While set, every launch of kernel
 * `which` (MOE_KERNEL_*) records `start_event` and `stop_event` (hipEvent_t
 * passed as void*) at that kernel's own begin and end, as part of its
 * dispatch (hipExtLaunchKernelGGL), so their elapsed time is the kernel's
 * duration without queueing gaps.  Two NULL events clear it.  Process-wide
 * and not thread-safe.  MOE_EINVAL for an unknown kernel. */
int moe_debug_time_kernel(int32_t which, void* start_event, void* stop_event);

/* DEBUG/BENCHMARK ONLY -- enqueue a plain streaming read of `bytes` (a
 * multiple of 16) at `src` by `blocks` blocks of 512 threads (16-byte
 * loads, four in flight per lane): the practical HBM read ceiling the
 * kernels are measured against.  `sink` (4 bytes of device memory) is
 * written only if the XOR of the data read equals an arbitrary constant. */
int moe_debug_stream_read(const void* src, size_t bytes, uint32_t* sink, int32_t blocks,
                          void* stream);

#ifdef __cplusplus
}
#endif
#endif /* BEF_MOE_H */
