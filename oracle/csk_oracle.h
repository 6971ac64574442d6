/*
 * csk_oracle.h - plain CPU oracle for hybrid compressed attention (CSA + HCA).
 *
 * TEST INFRASTRUCTURE ONLY. This library is the slow, obviously-correct
 * reference the GPU library is checked against. Only the test suite, the
 * smoke check and the benchmark's CPU-baseline leg may load it. It shares no
 * source, header, table or helper with the GPU library.
 *
 * Sources (web pages about the DeepSeek-V4 technical report):
 *   [P1] "Техотчёт DeepSeek-V4 (2026): миллион токенов контекста" (ai.flicky.cc)
 *   [P2] "Статья DeepSeek V4: Ключевые технические находки официального отчёта" (framia.pro)
 *   [P3] aixai.ru blog post on the V4 million-token context, section
 *        "Гибридный attention: CSA и HCA"
 *   [P4] "Технический отчёт DeepSeek-V4 — часть 1/2" (aifinder.ae mirror)
 *
 * Conventions: every pointer is a host pointer to a dense row-major array.
 * Floating-point inputs arrive as float (bf16 inputs are widened exactly by
 * the caller); all internal arithmetic is double unless a function states an
 * fp32 operation order. Functions return 0 on success and a negative value on
 * invalid arguments. Nothing here allocates device memory or prints.
 */
#ifndef CSK_ORACLE_H
#define CSK_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Partial RoPE, in place, on one vector of length D: the last d_rope
 * channels are rotated in interleaved pairs, pair j by angle
 * pos * base^(-2j/d_rope). [P4], paragraph on partial RoPE (only the last 64
 * dims are rotated). */
void csk_ref_rope(double* x, int D, int d_rope, double pos, double base);

/* CSA compression. ca, za, cb, zb: [B,S,D]; bias_a, bias_b: [m,D];
 * entry_pos: [B,S/m] or NULL (then entry i sits at position m*i).
 * out: [B,S/m,D] double, before any output rounding.
 * [P1] «CSA: сжать в 4 раза и выбрать top-k», step 1; exercise 2 in
 * «Что сделать руками»; [P4] (2m tokens with stride m). */
int csk_ref_csa_compress(const float* ca, const float* za, const float* cb, const float* zb,
                         const float* bias_a, const float* bias_b, int B, int S, int D, int m,
                         int d_rope, double rope_base, const int32_t* entry_pos, double* out);

/* HCA compression: softmax-gated pooling of each non-overlapping block of m
 * tokens. c, z: [B,S,D]; bias: [m,D]; out: [B,S/m,D] double.
 * [P1] «HCA: сжать в 128 раз, но смотреть на всё». */
int csk_ref_hca_compress(const float* c, const float* z, const float* bias, int B, int S, int D,
                         int m, int d_rope, double rope_base, const int32_t* entry_pos, double* out);

/* Round-to-nearest-even of double values to bf16 bit patterns / to float. */
void csk_ref_round_bf16(const double* x, uint16_t* y, int64_t n);
void csk_ref_round_f32(const double* x, float* y, int64_t n);

/* MXFP4 (E2M1 elements, one power-of-two E8M0 scale per 1x32 tile).
 * x: [rows, cols] with cols % 32 == 0. codes: [rows, cols/2] (element 2j in
 * the low nibble of byte j); scales: [rows, cols/32].
 * [P1] «FP4 с учётом квантования» (MXFP4, FP4 = E2M1, 1x32 tiles). */
int csk_ref_mxfp4_encode(const float* x, int64_t rows, int cols, uint8_t* codes, uint8_t* scales);
int csk_ref_mxfp4_decode(const uint8_t* codes, const uint8_t* scales, int64_t rows, int cols,
                         float* x);

/* Lightning-indexer scores I[t,s] = sum_h w[t,h] * ReLU(q[t,h] . k[s]) for
 * the listed query rows. dtype 0: fp32 q [B,T,HI,dI] and k [B,Nmax,dI];
 * dtype 2: MXFP4 q codes/scales [B,T,HI,dI/2]/[B,T,HI,dI/32] and k codes/
 * scales [B,Nmax,dI/2]/[B,Nmax,dI/32]. rows: n_rows pairs (b, t).
 * scores: [n_rows, Nmax] (entries past the visible count are -inf);
 * n_vis: [n_rows]. [P1] «CSA: сжать в 4 раза и выбрать top-k», step 2;
 * [P3] lightning indexer paragraph. */
int csk_ref_indexer_scores(const float* qf, const uint8_t* qc, const uint8_t* qs, const float* w,
                           const float* kf, const uint8_t* kc, const uint8_t* ks,
                           const int32_t* q_pos, const int32_t* n_entries, int B, int T, int HI,
                           int dI, int Nmax, int m, int dtype, const int32_t* rows, int n_rows,
                           float* scores, int32_t* n_vis);

/* FP8 KV entries ([P2] FP8 storage; [P1] «Почему это так сильно экономит»,
 * item 1): the D - d_rope non-RoPE dims as OCP E4M3 codes with one
 * power-of-two scale byte per 32 dims (the block maximum scaled into
 * [128, 256)), the d_rope RoPE dims as bf16. Entry layout: [codes][rope
 * bf16][scales], zero-padded to a multiple of 16 bytes. x: [rows, D] fp32;
 * out: [rows, entry_bytes]. Decode is exact (to fp32). */
int csk_ref_fp8kv_entry_bytes(int D, int d_rope);
int csk_ref_fp8kv_encode(const float* x, int64_t rows, int D, int d_rope, uint8_t* out);
int csk_ref_fp8kv_decode(const uint8_t* in, int64_t rows, int D, int d_rope, float* x);

/* BF16 indexer scores: each fp32 score rounded once to the nearest bf16
 * (ties to even), in place. [P1] «FP4 с учётом квантования» (BF16 scores
 * for the top-k). */
void csk_ref_scores_bf16(float* scores, int64_t n);

/* Top-k per row: the min(k, n_vis) highest scores, ties to the lower index,
 * returned in ascending index order and padded with -1 (score -inf).
 * scores: [n_rows, Nmax]; idx, out_scores: [n_rows, k]. */
int csk_ref_topk(const float* scores, const int32_t* n_vis, int n_rows, int Nmax, int k,
                 int32_t* idx, float* out_scores);

/* CSA sparse MQA attention over the selected compressed entries, the
 * sliding window of uncompressed tokens and the sink, for the listed rows.
 * q: [B,T,H,D] (unrotated); q_pos: [B,T]; kv_c: [B,Nmax,D] (rotated);
 * idx: [B,T,k]; kv_w: [B,S_w,D] (rotated), row r at position w_pos0[b]+r;
 * sink: [H] or NULL. out: [n_rows,H,dv] double; lse: [n_rows,H] double.
 * [P1] «CSA: сжать в 4 раза и выбрать top-k», step 3; «HCA…» (window);
 * [P4] (SWA branch, attention sink, partial RoPE). */
int csk_ref_sparse_attn(const float* q, const int32_t* q_pos, const float* kv_c, int Nmax,
                        const int32_t* idx, int k, const float* kv_w, const int32_t* w_pos0,
                        int S_w, int W, const float* sink, int B, int T, int H, int D, int dv,
                        int d_rope, double rope_base, double scale, const int32_t* rows,
                        int n_rows, double* out, double* lse);

/* HCA dense attention: as csk_ref_sparse_attn, but the compressed
 * candidates are every entry i < n_entries[b] with m*(i+1)-1 <= q_pos.
 * [P1] «HCA: сжать в 128 раз, но смотреть на всё»; [P3] HCA paragraph. */
int csk_ref_dense_attn(const float* q, const int32_t* q_pos, const float* kv_c, int Nmax,
                       const int32_t* n_entries, int m, const float* kv_w, const int32_t* w_pos0,
                       int S_w, int W, const float* sink, int B, int T, int H, int D, int dv,
                       int d_rope, double rope_base, double scale, const int32_t* rows,
                       int n_rows, double* out, double* lse);

/* Grouped output projection ([P1] «CSA: сжать в 4 раза и выбрать top-k»,
 * step 4). o: [R, H*dv] (head h's outputs at h*dv); the g groups hold H/g
 * consecutive heads each; w1: [g, dg, (H/g)*dv] (group i's projection to
 * dg intermediate features, [out, in]); w2: [d, g*dg]. u_out: [R, g*dg]
 * (the intermediate, rounded once to bf16) or NULL; y: [R, d] double. */
int csk_ref_grouped_out_proj(const float* o, const float* w1, const float* w2, int R, int H, int dv,
                             int g, int dg, int d, float* u_out, double* y);

/* RMSNorm of each row of x [rows, D] over all D values:
 * y = x * gamma / sqrt(mean(x^2) + eps) ([P1] «Muon и борьба с
 * нестабильностью»: queries and KV entries normalised by RMSNorm; [P4]: QK
 * norms). y: [rows, D] double. */
int csk_ref_rmsnorm(const float* x, const float* gamma, int64_t rows, int D, double eps, double* y);

/* Projection then compression ([P1] «CSA…» step 1: the series come from
 * the hidden states). x: [B,S,hidden]; w: [4,D,hidden] (csa = 1: W_ca,
 * W_za, W_cb, W_zb) or [2,D,hidden] (csa = 0: W_c, W_z), [out, in]; the
 * series X W^T pool as csk_ref_csa_compress / csk_ref_hca_compress (bias_b
 * unused for HCA); gamma [D] or NULL: RMSNorm of each entry before RoPE.
 * out: [B,S/m,D] double. */
int csk_ref_project_compress(const float* x, const float* w, const float* bias_a, const float* bias_b,
                             const float* gamma, double eps, int csa, int B, int S, int hidden, int D,
                             int m, int d_rope, double rope_base, const int32_t* entry_pos, double* out);

/* Number of OpenMP threads the oracle runs with. */
int csk_ref_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
