/*
 * moe_oracle.h -- plain, slow CPU oracle of the routed-expert MoE FFN layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load or call this library.  The GPU
 * library never includes, links or calls it, and it includes nothing from
 * the GPU library: the two share no code, headers, tables or constants.
 *
 * Sources (cited by page and section; the pages print no formulas, so every
 * step below is the plainest reading of what they name):
 *   [tcti]   tcti.cn repost of the LINUX DO post on running DeepSeek-V4-Flash
 *            on 4x RTX 2080 Ti -- sections "DeepSeek-V4-Flash的可能性"
 *            (routed experts stored FP4, top-6 activation, shared expert) and
 *            "补齐软件栈缺失" (act_quant feeds the FP8/FP4 linears; fp4_gemm
 *            multiplies an FP8-quantised activation by FP4 packed weights;
 *            fp8_gemm is FP8 x FP8).
 *   [dpshk]  dpshk.com article on deepseek-v4-flash-0731-in-c -- sections
 *            "核心实现一" (router first picks the token's experts),
 *            "核心实现三" (layer-major batching: an expert read once serves
 *            all of its tokens) and "核心实现四" (FP4/FP8 dequantised inside
 *            the GEMV, gate and up share one quantised input, each row keeps
 *            a fixed accumulation order).
 *   [muninn] ai-muninn.com "[洋垃圾跑大模型 #3]" -- section "目標不是「載得
 *            進去」..." (256 routed experts per block, 6 chosen per token).
 *   [OCP-MX] OCP Microscaling Formats (MX) v1.0: E2M1 element, E8M0 scale,
 *            E4M3 (the "FN" variant: no infinities, NaN = S.1111.111,
 *            max 448).
 * The layer's formats and rules (E2M1 packed two per byte with one UE8M0
 * scale per 32 inputs; E4M3 activations with one fp32 scale = amax/448 per
 * 128; sigmoid scores; top-k renormalised to sum 1; ties to the lower expert
 * id; SwiGLU; one always-on shared expert; an FP8-weight variant with one
 * fp32 scale per 128x128 block) come from the workload definitions that
 * accompany the pages.  Every point the sources leave open is resolved by a
 * stated reading (see the comments at each function).
 *
 * Precision: all FFN arithmetic is fp64.  The two places where a floating
 * point value decides an integer -- the E4M3 code of an activation and the
 * choice of experts -- take that decision in fp32, the precision the layer
 * stores those values in, exactly as the definition states.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_FMT_FP4 = 1, ORC_FMT_FP8 = 2 };

/* Stacked expert weights, expert-major; slot E (the last) is the shared
 * expert.  Matrices are [out][in] row-major.
 *   FP4 (ORC_FMT_FP4): gate/up codes [E+1][I][H/2] u8, element 2j in bits
 *     0-3 and element 2j+1 in bits 4-7; scales [E+1][I][H/32] u8 (UE8M0).
 *     down codes [E+1][H][I/2]; scales [E+1][H][I/32].
 *   FP8 (ORC_FMT_FP8): gate/up codes [E+1][I][H] u8 (E4M3); scales
 *     [E+1][I/128][H/128] f32.  down codes [E+1][H][I]; scales
 *     [E+1][H/128][I/128] f32. */
typedef struct {
  int32_t format, E, H, I;
  const uint8_t *gate_q, *up_q, *down_q;
  const void *gate_s, *up_s, *down_s;
} orc_weights;

/* ---- element codecs ---------------------------------------------------- */
double orc_e2m1_value(unsigned code4);
double orc_ue8m0_value(unsigned byte);
double orc_e4m3_value(unsigned byte);
double orc_bf16_value(uint16_t bits);
unsigned orc_e4m3_encode(float v);
void orc_e4m3_encode_n(const float* v, int64_t n, uint8_t* out);

/* ---- S3: activation quantisation --------------------------------------- */
void orc_act_quant_f32(const float* x, int64_t rows, int32_t cols, uint8_t* q, float* s);
void orc_act_quant_bf16(const uint16_t* x, int64_t rows, int32_t cols, uint8_t* q, float* s);

/* ---- S1/S2: router ------------------------------------------------------ */
void orc_router_logits(const uint16_t* x, const uint16_t* wr, int32_t T, int32_t H, int32_t E,
                       float* z);
void orc_topk(const float* z, int32_t T, int32_t E, int32_t k, int32_t* ids, double* w);
void orc_topk_weights(const float* z, int32_t T, int32_t E, int32_t k, const int32_t* ids,
                      double* w);

/* ---- S4: permutation ---------------------------------------------------- */
int orc_permute(const int32_t* ids, int32_t T, int32_t k, int32_t E, int32_t* offsets,
                int32_t* row_token, int32_t* row_of);

/* ---- S5/S6: one expert on one row -------------------------------------- */
double orc_weight(const orc_weights* w, int mat, int32_t e, int32_t row, int32_t col);
void orc_gate_up(const orc_weights* w, int32_t e, const uint8_t* xq, const float* xs, double* g,
                 double* u);
void orc_swiglu(const double* g, const double* u, int32_t n, float* h);
void orc_down(const orc_weights* w, int32_t e, const uint8_t* hq, const float* hs, double* y);
void orc_expert_row(const orc_weights* w, int32_t e, const uint8_t* xq, const float* xs, float* h,
                    uint8_t* hq, float* hs, double* y);

/* ---- whole layer -------------------------------------------------------- */
int orc_moe_forward(const orc_weights* w, const uint16_t* wr, const uint16_t* x, int32_t T,
                    int32_t k, const int32_t* ids_in, const float* w_in, const int32_t* tokens,
                    int32_t n_tokens, double* out, int32_t n_threads);

#ifdef __cplusplus
}
#endif
#endif
