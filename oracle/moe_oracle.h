/*
 * Plain CPU oracle for the routed MXFP4 MoE feed-forward (TEST INFRASTRUCTURE ONLY).
 * Host pointers, fp64 arithmetic. Shares nothing with the HIP library.
 * Layouts match the library's documented layouts: row-major and contiguous,
 *   logits f32[T,E]; x bf16 bits u16[T,H];
 *   w13_q u8[E,2I,H/2] (rows [0,I) gate, [I,2I) up; low nibble = even element), w13_s u8[E,2I,H/32];
 *   w2_q u8[E,H,I/2], w2_s u8[E,H,I/32];
 *   topk_ids i32[T,k], topk_w f64[T,k]; pairs are numbered p = t*k + j.
 * Return codes: 0 ok, -2 bad argument, -3 out of host memory.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_SCORE_SOFTMAX = 0, ORACLE_SCORE_SIGMOID = 1 };
enum { ORACLE_ACT_NONE = 0, ORACLE_ACT_MXFP8 = 1, ORACLE_ACT_MXFP4 = 2 };

double oracle_e2m1_value(int code);
double oracle_e8m0_value(int byte);
double oracle_bf16_to_double(uint16_t bits);
uint16_t oracle_double_to_bf16(double v);
double oracle_mxfp4_element(const uint8_t* q, const uint8_t* s, int K, long n, long kk);

double oracle_e4m3_value(int code);
int oracle_e4m3_encode(double v);
int oracle_e2m1_encode(double v);
double oracle_mx_element(int fmt, int code);
int oracle_mx_quantize_block(const double* v, int fmt, uint8_t* codes);

int oracle_route_topk(const float* logits, int T, int E, int k, int score_fn, int renorm,
                      int32_t* topk_ids, double* topk_w);

int oracle_group_tokens(const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_pair, int32_t* pair_pos, int32_t* active,
                        int32_t* n_active);

/* y_pairs (optional, may be NULL): f64[T*k, H], each pair's down-projection output before weighting.
 * out_ref (optional): f64[T,H], the combined output before rounding. out_bf16 (optional): the
 * combined output rounded once to bfloat16. clamp_limit <= 0 disables the clamp. nthreads <= 0 uses
 * the OpenMP default; pairs are independent, so the thread count does not change any result. */
int oracle_mxfp4_ffn(const uint16_t* x_bf16, int T, int H, int I, int E, int k,
                     const uint8_t* w13_q, const uint8_t* w13_s, const uint8_t* w2_q,
                     const uint8_t* w2_s, const int32_t* topk_ids, const double* topk_w,
                     double clamp_limit, int nthreads, double* y_pairs, double* out_ref,
                     uint16_t* out_bf16);

/* As oracle_mxfp4_ffn with the GEMMs' activations quantised to an MX format (act_fmt); see the .c.
 * h_pairs (optional): f64[T*k, I], each pair's h before its quantisation (rounded to binary32 when
 * act_fmt quantises). */
int oracle_mxfp4_ffn_act(const uint16_t* x_bf16, int T, int H, int I, int E, int k,
                         const uint8_t* w13_q, const uint8_t* w13_s, const uint8_t* w2_q,
                         const uint8_t* w2_s, const int32_t* topk_ids, const double* topk_w,
                         double clamp_limit, int act_fmt, int nthreads, double* y_pairs, double* h_pairs,
                         double* out_ref, uint16_t* out_bf16);

/* Router logits f64[T,E] = x . w^T for bfloat16 x[T,H] and w[E,H] (fp64, h ascending). */
int oracle_router_logits(const uint16_t* x_bf16, const uint16_t* w_bf16, int T, int H, int E,
                         int nthreads, double* logits);

int oracle_num_threads(int nthreads);

#ifdef __cplusplus
}
#endif
#endif
