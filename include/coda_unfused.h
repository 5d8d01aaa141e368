/*
 * coda_unfused.h - the unfused baseline of libcoda.so: standalone bandwidth
 * kernels that, behind the plain GEMMs of coda.h (coda_gemm, and the
 * store-only data/weight-gradient calls), form the conventional sequence
 * that the fused calls replace.
 *
 * "CODA: Rewriting Transformer Blocks as GEMM-Epilogue Programs" (abstract;
 * Figure 1) describes that sequence: each memory-bound operation is its own
 * kernel that reads its input from global memory and writes its output back.
 * These kernels do that, with the same arithmetic as the fused epilogues
 * (reading notes "CODA GEMM-Epilogue Programming" sections 2 and 3), so the
 * two paths can be timed against each other on the same tensors.
 *
 * Conventions are those of coda.h: row-major bf16 matrices with a leading
 * dimension in elements (16-byte aligned base, ld % 8 == 0), widths % 8 == 0,
 * caller-owned device pointers, no allocation or synchronisation, launch on
 * `stream`, coda_status return codes, validation before any HIP call.
 * Each kernel rounds its bf16 outputs to nearest-even and computes in fp32.
 */
#ifndef CODA_UNFUSED_H_
#define CODA_UNFUSED_H_

#include "coda.h"

#ifdef __cplusplus
extern "C" {
#endif

/* C = bf16(A + B), all [M x N]: the standalone residual add (the residual of
 * "GEMM -> residual -> RMSNorm -> GEMM", notes section 2).  C may alias A or B
 * when it has the same leading dimension. */
coda_status coda_unfused_add(const coda_bf16* A, int lda, const coda_bf16* B, int ldb,
                             coda_bf16* C, int ldc, int M, int N, hipStream_t stream);

/* Residual add followed by RMSNorm, one row per workgroup (notes section 2;
 * paper Figure 4 shows the same computation split across two GEMMs):
 *   U = bf16(Y + Z)                  (Z opt: NULL means U = Y)
 *   r_i = 1 / sqrt(mean_j U_ij^2 + eps)     (fp32, over the bf16 U)
 *   N2 = bf16(r_i * U_ij * gamma_j)
 * U may alias Y.  r: fp32 [M]; gamma: bf16 [d]. */
coda_status coda_unfused_add_rmsnorm(const coda_bf16* Y, int ldy, const coda_bf16* Z, int ldz,
                                     const coda_bf16* gamma, float eps, coda_bf16* U, int ldu,
                                     coda_bf16* N2, int ldn, float* r, int M, int d, hipStream_t stream);

/* RoPE in place on Y [M x N] (paper Figure 7; RoFormer): every adjacent pair
 * (c, c+1), c even and c < n_rope, rotated by pos_i * theta^(-2k/head_dim),
 * k = (c mod head_dim)/2; columns >= n_rope are left unchanged.  inverse != 0
 * rotates by the negative angle.  pos: int32 [M].  n_rope % head_dim == 0,
 * head_dim even. */
coda_status coda_unfused_rope(coda_bf16* Y, int ldy, const int32_t* pos, float theta, int head_dim,
                              int n_rope, int inverse, int M, int N, hipStream_t stream);

/* SwiGLU (paper Figure 7): Pre [M x 2F] holds (gate, up) interleaved at
 * columns (2j, 2j+1); Act [M x F], Act_ij = g * sigmoid(g) * v. */
coda_status coda_unfused_swiglu(const coda_bf16* Pre, int ldp, coda_bf16* Act, int lda, int M, int F,
                                hipStream_t stream);

/* SwiGLU backward (notes section 3): dA [M x F], Pre [M x 2F] ->
 * dPre [M x 2F], (dg, dv) = (da v s (1 + g (1 - s)), da g s), s = sigmoid(g). */
coda_status coda_unfused_swiglu_bwd(const coda_bf16* dA, int ldda, const coda_bf16* Pre, int ldp,
                                    coda_bf16* dPre, int lddp, int M, int F, hipStream_t stream);

/* Rows per dgamma partial of coda_unfused_rmsnorm_bwd: gpart has
 * coda_unfused_rmsnorm_bwd_parts(M) rows of d floats. */
int coda_unfused_rmsnorm_bwd_parts(int M);

/* RMSNorm backward in its canonical form (notes section 3), one row at a time:
 * with G = dN2 [M x d] (gradient of N2 = r U gamma),
 *   c_i = sum_j G_ij gamma_j U_ij,
 *   dU_ij = dRes_ij + r_i G_ij gamma_j - r_i^3 U_ij c_i / d   (dRes opt),
 *   gpart[q, j] = sum over rows i of block q of G_ij r_i U_ij (dgamma partials;
 *                 reduce them with coda_col_reduce).
 * r: fp32 [M] from the forward; gpart: fp32 dense
 * [coda_unfused_rmsnorm_bwd_parts(M) x d], opt.  d <= 8192. */
coda_status coda_unfused_rmsnorm_bwd(const coda_bf16* G, int ldg, const coda_bf16* U, int ldu,
                                     const coda_bf16* gamma, const float* r, const coda_bf16* dRes,
                                     int ldr, coda_bf16* dU, int lddu, float* gpart, int M, int d,
                                     hipStream_t stream);

/* Cross-entropy over materialised logits L [M x V] (bf16, e.g. from
 * coda_gemm): lse_i = log sum_j exp(L_ij), loss_row_i = lse_i - L_{i,y_i}
 * (NaN when the label is outside [0, V)), loss_mean = mean_i loss_row_i
 * (opt).  One workgroup per row; fixed reduction order. */
coda_status coda_unfused_cross_entropy(const coda_bf16* L, int ldl, const int32_t* labels, float* lse,
                                       float* loss_row, float* loss_mean, int M, int V,
                                       hipStream_t stream);

/* Cross-entropy backward over the materialised logits: D = bf16((exp(L - lse_i)
 * - [j == y_i]) * grad_scale), D [M x V] (may alias L when ldd == ldl). */
coda_status coda_unfused_cross_entropy_bwd(const coda_bf16* L, int ldl, const int32_t* labels,
                                           const float* lse, float grad_scale, coda_bf16* D, int ldd,
                                           int M, int V, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CODA_UNFUSED_H_ */
