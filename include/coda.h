/*
 * coda.h - C ABI of the MI355X (gfx950) CODA GEMM-epilogue library, libcoda.so.
 *
 * Each fused call is one bf16 MFMA GEMM whose epilogue performs the
 * non-attention Transformer-block work on the output tile while it is still in
 * registers, before the global store, as described in "CODA: Rewriting
 * Transformer Blocks as GEMM-Epilogue Programs" (abstract; Figure 3) and in
 * the reading notes "CODA GEMM-Epilogue Programming" (section 1, "The Epilogue
 * Concept").  The auxiliary reductions are small bandwidth kernels.
 *
 * Conventions (every entry point):
 *  - Matrices are row-major with a leading dimension ld* in elements.
 *    Weights are stored [in x out] (K x N), so a forward projection is X W.
 *  - bf16 is bfloat16 bits (coda_bf16); the GEMM accumulates in fp32 and
 *    rounds its bf16 outputs to nearest-even.  Row/column statistics,
 *    losses and weight gradients are fp32.
 *  - All pointers are DEVICE pointers owned by the caller.  The library never
 *    allocates, frees or synchronises; calls are asynchronous and ordered on
 *    `stream` (NULL = default stream).  Its global state: a per-device cache
 *    of two device properties (the gfx950 check and the compute-unit count)
 *    and of the address of the 64 MiB device array behind
 *    coda_lmhead_ce_noalloc, each written once per device with atomic stores
 *    and safe to read from any thread; that array itself (one per device,
 *    held until the process ends); the environment switches below, read
 *    once; and, in the timeline build only, the timeline buffer installed by
 *    coda_timeline_set (coda_probe.h), read under a lock.
 *  - Requirements: bf16 base pointers 16-byte aligned and bf16 ld % 8 == 0;
 *    fp32 matrix pointers 16-byte aligned and fp32 ld % 4 == 0; every output
 *    width (N, F, d, V) % 8 == 0, except the SwiGLU activation width F
 *    (coda_gemm_swiglu: F % 4 == 0 and ldact % 4 == 0); the reduction length
 *    K % 8 == 0 when the operand is contiguous along K (every forward and
 *    data-gradient call).  The token count M is arbitrary; ragged edge tiles
 *    are masked.
 *  - Errors: validation happens before any launch and returns a status
 *    without touching the device.  CODA_ERR_HIP reports a launch error
 *    (hipGetLastError); device faults surface at the caller's next sync.
 *    Optional outputs ("opt") are skipped when NULL.
 *  - Environment: CODA_LOG=1 prints each call's name and sizes to stderr.
 *    CODA_DEBUG=1 checks, before any launch, that every matrix and vector
 *    argument's byte extent ((rows - 1) * ld + cols elements) lies inside the
 *    device allocation holding its base pointer, and returns CODA_ERR_BOUNDS
 *    otherwise (coda_debug_extent is that check on its own).
 *  - Outputs must not alias inputs unless stated.  Results are deterministic:
 *    no atomics, fixed reduction order.
 */
#ifndef CODA_H_
#define CODA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t coda_bf16;

typedef enum coda_status {
  CODA_OK = 0,
  CODA_ERR_NULL = 1,        /* a required pointer is NULL                     */
  CODA_ERR_SHAPE = 2,       /* a size or leading dimension is invalid         */
  CODA_ERR_ALIGN = 3,       /* a pointer or leading dimension is misaligned   */
  CODA_ERR_UNSUPPORTED = 4, /* device is not gfx950, or an untiled constraint */
  CODA_ERR_HIP = 5,         /* the HIP runtime reported an error              */
  CODA_ERR_WORKSPACE = 6,   /* workspace missing or too small                 */
  CODA_ERR_BOUNDS = 7       /* CODA_DEBUG: an argument leaves its allocation  */
} coda_status;

/* Human-readable text of a status code (static storage). */
const char* coda_status_str(coda_status s);

/* Library version string, e.g. "coda-gfx950 0.1". */
const char* coda_version(void);

/* CODA_DEBUG's extent check on its own: CODA_OK if [p, p + bytes) lies
 * inside the device allocation that holds p (or p is NULL, or bytes is 0),
 * CODA_ERR_BOUNDS otherwise.  Host-side query; launches nothing. */
coda_status coda_debug_extent(const void* p, size_t bytes);

/* Number of per-row partial columns a fused call writes for an output of
 * width N (one per 128-wide wavefront output tile): ceil(N / 128).  These
 * are per-tile row reductions, the fourth epilogue primitive class of the
 * reading notes "CODA GEMM-Epilogue Programming" (section 1), and the first
 * level of the paper's two-level RMSNorm reduction (Figure 4). */
int coda_nparts(int N);

/* Number of per-column partial rows written by coda_gemm_rowscale_bwd for M
 * tokens (one per 128-token wavefront output tile): ceil(M / 128).  The
 * per-tile column reductions of the same primitive class (reading notes
 * section 1, class 4), used for dgamma. */
int coda_mparts(int M);

/* Tile plan of a fused GEMM with F output features (N, F or V of the call)
 * and T tokens (M) on a device with `cus` compute units.  Output tiles are
 * 256 features x 256 tokens, one per compute unit at a time; when that
 * leaves the last round of tiles mostly empty, the features from
 * 256 * split on are computed in 256 x 128 tiles by the same dispatch.
 * Returns split (0: no such split).  A problem of at most cus/2 tiles of
 * 256 x 256 (under half a round) instead runs entirely in 256 x 128 tiles,
 * on twice as many compute units.  Both apply to every GEMM of the library
 * except coda_gemm_rowscale_bwd, whose dgamma column partials are laid out
 * per 256-token tile.  This plans the fixed mainloop that every call shares
 * (paper abstract and Figure 3: the mainloop stays as it is and only the
 * epilogue changes).  Host-only: touches no device. */
int coda_tile_split(int F, int T, int cus);

/* When neither of the above applies: the number tb of 256-token tiles that
 * stay 256 x 256, the tokens from 256 * tb on being computed in 256 x 128
 * tiles by the same dispatch (0: no such split).  It is chosen with the same
 * round-count model (a 256 x 128 tile costs 0.6 of a 256 x 256 one) and must
 * save 0.2 rounds, as for the weight gradient 14336 x 4096 over 8192 tokens
 * (3.5 rounds of 256 x 256 tiles: tb = 48 gives 3 + 0.6).  Same scope as
 * coda_tile_split.  Host-only: touches no device. */
int coda_tile_split_tokens(int F, int T, int cus);

/* Plan of coda_gemm_swiglu_bwd_overlap for M tokens, F features and
 * reduction length N on `cus` compute units: the number U (1 or 2) of
 * pair-map units that each k-tile of the GEMM mainloop carries, or 0 for the
 * plain kernel.  With U > 0 the call is a persistent kernel of one workgroup
 * per compute unit, whose tile epilogue stores da in fp32 into the dPre
 * bytes of that tile (32 bytes per token and 8 features either way), and
 * whose next k-loop reads it back and applies the pair map in 64 units per
 * wave, U per k-tile; the last tile's units run after its k-loop.  It
 * applies when no tile split does (coda_tile_split,
 * coda_tile_split_tokens, the 256 x 128 small-problem plan), the problem
 * has more than one round of 256 x 256 tiles, and N >= 2048 (32 k-tiles of
 * 64).  Host-only: touches no device. */
int coda_swiglu_bwd_units(int M, int F, int N, int cus);

/* Workspace bytes coda_lmhead_ce needs for M rows and vocabulary V: the
 * per-tile max and sum-exp statistics and the gathered target logits that
 * the epilogue writes and the auxiliary reduction combines (reading notes
 * section 2, "Cross-entropy loss"). */
size_t coda_lmhead_ce_workspace(int M, int V);

/* Minimal workspace bytes coda_lmhead_ce_bwd needs (one 256-row chunk of
 * bf16 dlogits of the recomputed logits, reading notes section 2,
 * "Cross-entropy loss"); a larger workspace processes more rows per chunk,
 * up to M * V * 2 bytes (no chunking). */
size_t coda_lmhead_ce_bwd_workspace(int M, int V, int d);

/* ---------------------------------------------------------------------------
 * Plain GEMM, store-only epilogue: Y[M x N] = bf16(X[M x K] W[K x N]).
 * The "fixed mainloop" every fused call shares; also the unfused baseline.
 * ------------------------------------------------------------------------- */
coda_status coda_gemm(const coda_bf16* X, int ldx, const coda_bf16* W, int ldw,
                      coda_bf16* Y, int ldy, int M, int N, int K, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Forward
 * ------------------------------------------------------------------------- */

/* GEMM1 of GEMM -> residual -> RMSNorm -> GEMM (reading notes section 2;
 * paper Figure 4 and Listing 2):
 *   u = X W + Z                       -> U  (bf16, M x N)
 *   h2 = u * gamma (per column)       -> H2 (bf16, opt; needs gamma)
 *   part[i, p] = sum_{j in part p} u_ij^2 of the UNSCALED fp32 u
 *                                     -> part (fp32, opt, M x coda_nparts(N),
 *                                        row stride coda_nparts(N))
 * Z may be NULL (no residual).  With gamma, H2 and part all NULL this is a
 * GEMM plus residual add (e.g. an MLP down projection). */
coda_status coda_gemm_res_sumsq(const coda_bf16* X, int ldx, const coda_bf16* W, int ldw,
                                const coda_bf16* Z, int ldz, const coda_bf16* gamma,
                                coda_bf16* U, int ldu, coda_bf16* H2, int ldh, float* part,
                                int M, int N, int K, hipStream_t stream);

/* Auxiliary reduction (paper Figure 4 / Figure 5 caption):
 *   r_i = 1 / sqrt( sum_p part[i, p] / d + eps )
 * part is fp32 [M x nparts] (row stride nparts), r is fp32 [M]. */
coda_status coda_row_rms(const float* part, int nparts, int M, int d, float eps, float* r,
                         hipStream_t stream);

/* GEMM2 with the delayed RMSNorm row scale (reading notes section 2):
 *   Y = bf16( r_i * (A W)_ij ),  A = h2 [M x K], W [K x N], r fp32 [M]. */
coda_status coda_gemm_rowscale(const coda_bf16* A, int lda, const coda_bf16* W, int ldw,
                               const float* r, coda_bf16* Y, int ldy, int M, int N, int K,
                               hipStream_t stream);

/* GEMM + RoPE pair map (paper Figure 7; RoFormer rotation):
 *   t = r_i * (A W)_ij  (r opt: NULL means 1)
 *   for each even column c < n_rope, k = (c mod head_dim) / 2,
 *   ang = pos_i * theta^(-2k / head_dim):
 *     (y_c, y_c+1) = (t_c cos - t_c+1 sin, t_c sin + t_c+1 cos)
 *   columns >= n_rope pass through.  pos is int32 [M].
 * Needs head_dim even, n_rope % head_dim == 0, n_rope % 8 == 0 and
 * n_rope <= N. */
coda_status coda_gemm_rope(const coda_bf16* A, int lda, const coda_bf16* W, int ldw,
                           const float* r, const int32_t* pos, float theta, int head_dim,
                           int n_rope, coda_bf16* Y, int ldy, int M, int N, int K,
                           hipStream_t stream);

/* GEMM + SwiGLU pair map (paper Figure 7; reading notes section 2):
 *   (g, v) = r_i * ((A Wgu)_i,2j , (A Wgu)_i,2j+1)   (r opt)
 *   Act_ij = g * sigmoid(g) * v         -> Act (bf16, M x F)
 *   Pre = bf16(g, v) interleaved        -> Pre (bf16, opt, M x 2F)
 * Wgu is [K x 2F] with gate columns even and up columns odd. */
coda_status coda_gemm_swiglu(const coda_bf16* A, int lda, const coda_bf16* Wgu, int ldw,
                             const float* r, coda_bf16* Act, int ldact, coda_bf16* Pre,
                             int ldp, int M, int F, int K, hipStream_t stream);

/* LM head + cross-entropy (reading notes section 2, "Cross-entropy loss"):
 * logits l = H W (fp32, never stored); the GEMM epilogue writes per-tile
 * (max, sum exp) and gathers the target logit; an auxiliary kernel forms
 *   lse_i = log sum_k exp(l_ik),  loss_row_i = lse_i - l_{i,label_i},
 *   loss_mean = sum_i loss_row_i / M  (fixed order).
 * A label outside [0, V) gives a NaN row loss.  H [M x d], W [d x V],
 * labels int32 [M]; lse, loss_row fp32 [M] (loss_row opt), loss_mean fp32 [1]
 * (opt); ws >= coda_lmhead_ce_workspace(M, V) bytes, 16-byte aligned. */
coda_status coda_lmhead_ce(const coda_bf16* H, int ldh, const coda_bf16* W, int ldw,
                           const int32_t* labels, float* lse, float* loss_row, float* loss_mean,
                           void* ws, size_t ws_bytes, int M, int V, int d, hipStream_t stream);

/* coda_lmhead_ce for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and arguments without the workspace.  The partials
 * live in a 64 MiB array that the library holds in device memory, one per
 * GPU, from the first call on that device until the process ends
 * (coda_lmhead_ce_noalloc_max_bytes() returns its size); a call whose
 * coda_lmhead_ce_workspace(M, V) exceeds it returns CODA_ERR_WORKSPACE.
 * It calls no allocation routine.  Every call on one GPU shares that array:
 * calls that overlap on one GPU (other streams, other threads) race and give
 * wrong results; calls ordered on one stream are safe (each writes every
 * entry it reads). */
coda_status coda_lmhead_ce_noalloc(const coda_bf16* H, int ldh, const coda_bf16* W, int ldw,
                                   const int32_t* labels, float* lse, float* loss_row,
                                   float* loss_mean, int M, int V, int d, hipStream_t stream);

/* Size in bytes of the array coda_lmhead_ce_noalloc uses (67108864). */
size_t coda_lmhead_ce_noalloc_max_bytes(void);

/* coda_lmhead_ce that also keeps the logits: the same statistics, taken from
 * the fp32 logits, plus logits (bf16, M x V, leading dimension ldl, required)
 * written by the same epilogue.  For coda_lmhead_ce_bwd_logits, which then
 * needs no recompute GEMM; this trades the Cut-Cross-Entropy-style recompute
 * (reading notes section 2) for 2 M V bytes of HBM. */
coda_status coda_lmhead_ce_logits(const coda_bf16* H, int ldh, const coda_bf16* W, int ldw,
                                  const int32_t* labels, float* lse, float* loss_row,
                                  float* loss_mean, coda_bf16* logits, int ldl, void* ws,
                                  size_t ws_bytes, int M, int V, int d, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Backward ("reverse fusion", reading notes section 3; paper Figure 9)
 * ------------------------------------------------------------------------- */

/* Data-gradient GEMM with the SwiGLU backward pair map (1 -> 2):
 *   da = dOut Wd^T   (dOut [M x N], Wd [F x N] used transposed)
 *   with (g, v) = Pre_i,2j , Pre_i,2j+1 and s = sigmoid(g):
 *   dPre_i,2j = da v s (1 + g (1 - s)),  dPre_i,2j+1 = da g s
 *   spart[i, p] = sum_{j in part p} (dPre_2j g + dPre_2j+1 v)  (fp32, opt,
 *   M x coda_nparts(F)): the partial of sumcols(dY * y) that the RMSNorm
 *   backward statistic s needs (reading notes section 3). */
coda_status coda_gemm_swiglu_bwd(const coda_bf16* dOut, int ldd, const coda_bf16* Wd, int ldw,
                                 const coda_bf16* Pre, int ldp, coda_bf16* dPre, int lddp,
                                 float* spart, int M, int F, int N, hipStream_t stream);

/* coda_gemm_swiglu_bwd with each output tile's epilogue overlapped with the
 * next tile's MFMA work: the PingPong-style overlap of epilogue and
 * tensor-core work that the social thread "CODA reparameterizes
 * memory-bound operations" names (paper Figure 3: the epilogue is
 * tile-local).  Same arguments, outputs and errors; dPre is also used as the
 * tiles' staging: until the call completes it holds da in fp32 (the 8
 * features f..f+7 of a token are 32 bytes either way), so it must not alias
 * any input (as for every call; here a dPre that shares a byte with dOut,
 * Wd or Pre is rejected with CODA_ERR_SHAPE).  Where coda_swiglu_bwd_units(M, F, N, CUs)
 * is 0 it runs coda_gemm_swiglu_bwd's kernel.  Measured on gfx950 at the
 * 1B- and 8B-like MLP shapes it is 1.5-2x slower than coda_gemm_swiglu_bwd:
 * one wave per SIMD holds the 256 accumulators, and the pair map's VALU work
 * placed between its MFMAs does not overlap them, while reading da back in
 * the accumulator layout (32 bytes of each of 32 rows per load) costs more
 * than the plain epilogue's staged row loads. */
coda_status coda_gemm_swiglu_bwd_overlap(const coda_bf16* dOut, int ldd, const coda_bf16* Wd, int ldw,
                                         const coda_bf16* Pre, int ldp, coda_bf16* dPre, int lddp,
                                         float* spart, int M, int F, int N, hipStream_t stream);

/* Auxiliary reduction of the RMSNorm backward statistic (reading notes
 * section 3): s_i = sum_p spart[i, p] / d, d = the RMSNorm width. */
coda_status coda_row_rms_bwd(const float* spart, int nparts, int M, int d, float* s,
                             hipStream_t stream);

/* Data-gradient GEMM with the RMSNorm backward epilogue:
 *   G = dY W1^T   (dY [M x N], W1 [d x N] used transposed)
 *   dU = dRes + r_i (G * gamma) - r_i^2 s_i u          (bf16, M x d)
 *   N2 = bf16(r_i u * gamma)  (opt; the weight-gradient operand)
 *   gpart[q, j] = sum_{i in token part q} r_i G_ij u_ij (fp32, opt,
 *   coda_mparts(M) x d): the column partials of dgamma.
 * U is the RMSNorm input [M x d]; r, s fp32 [M]; dRes opt. */
coda_status coda_gemm_rowscale_bwd(const coda_bf16* dY, int ldd, const coda_bf16* W1, int ldw,
                                   const coda_bf16* U, int ldu, const coda_bf16* gamma,
                                   const float* r, const float* s, const coda_bf16* dRes, int ldr,
                                   coda_bf16* dU, int lddu, coda_bf16* N2, int ldn, float* gpart,
                                   int M, int d, int N, hipStream_t stream);

/* Column reduction of the dgamma partials: dgamma_j = sum_q gpart[q, j]
 * (the auxiliary step after the epilogue's per-tile column reductions,
 * reading notes section 1, class 4; dgamma of the RMSNorm backward,
 * section 3).  gpart fp32 [mparts x d], dgamma fp32 [d]. */
coda_status coda_col_reduce(const float* gpart, int mparts, int d, float* dgamma,
                            hipStream_t stream);

/* RoPE backward epilogue: same arguments as coda_gemm_rope; applies the
 * inverse rotation (ang -> -ang) after the optional row scale.  The
 * rotation is orthogonal, so its derivative map is the inverse rotation,
 * fused into the GEMM that produces the gradient of the rotated output
 * (reading notes section 3, "Reverse Fusion"; paper Figure 7). */
coda_status coda_gemm_rope_bwd(const coda_bf16* A, int lda, const coda_bf16* W, int ldw,
                               const float* r, const int32_t* pos, float theta, int head_dim,
                               int n_rope, coda_bf16* Y, int ldy, int M, int N, int K,
                               hipStream_t stream);

/* Backward of u = X W + Z (reading notes section 3: the gradient of the
 * GEMM input is dU W^T, and the residual's gradient path is added in the
 * same GEMM's epilogue):
 *   dX = dU W^T (+ dRes)   (bf16, M x K)       W [K x N] used transposed
 *   dW = X^T dU            (fp32, opt, K x N)  */
coda_status coda_gemm_res_sumsq_bwd(const coda_bf16* dU, int ldu, const coda_bf16* W, int ldw,
                                    const coda_bf16* X, int ldx, const coda_bf16* dRes, int ldr,
                                    coda_bf16* dX, int lddx, float* dW, int lddw,
                                    int M, int N, int K, hipStream_t stream);

/* Weight gradient: dW[K x N] = X^T dY (fp32); accumulate != 0 adds into dW.
 * X [M x K], dY [M x N]; M (the reduction) is arbitrary.  The weight
 * gradient of every GEMM of the block (reading notes section 3), on the same
 * fixed mainloop with an fp32 store epilogue. */
coda_status coda_gemm_wgrad(const coda_bf16* X, int ldx, const coda_bf16* dY, int ldd,
                            float* dW, int lddw, int M, int K, int N, int accumulate,
                            hipStream_t stream);

/* LM head + cross-entropy backward of loss = grad_scale * sum_i loss_row_i
 * (grad_scale = 1/M for the mean):
 *   recompute l = H W; dlogits D = (exp(l - lse_i) - [k == label_i]) grad_scale
 *   (bf16, in ws, row chunks); dH = D W^T (bf16, M x d); dW = H^T D (fp32, d x V).
 * lse comes from coda_lmhead_ce.  ws >= coda_lmhead_ce_bwd_workspace(M,V,d). */
coda_status coda_lmhead_ce_bwd(const coda_bf16* H, int ldh, const coda_bf16* W, int ldw,
                               const int32_t* labels, const float* lse, float grad_scale,
                               coda_bf16* dH, int lddh, float* dW, int lddw, void* ws,
                               size_t ws_bytes, int M, int V, int d, hipStream_t stream);

/* The same backward with the dlogits never round-tripping HBM: the
 * vocabulary is cut into chunks of vchunk columns (vchunk % 8 == 0), and
 * per chunk
 *   1) the recompute GEMM's epilogue forms D_c = (exp(l - lse_i) -
 *      [k == label_i]) grad_scale (bf16, M x vchunk, in ws) with ordinary
 *      stores, so that the chunk stays in the 256 MB Infinity Cache;
 *   2) dW[:, chunk] = H^T D_c (fp32; every column of dW is written once);
 *   3) dH += D_c W[:, chunk]^T, accumulated in fp32 in ws and rounded to bf16
 *      after the last chunk.
 * This is the reading notes' cross-entropy (section 2, "Cross-entropy loss")
 * backward in the form the social thread's third pattern names (the logits
 * recomputed as in Cut Cross Entropy), with the two consumer GEMMs of each
 * chunk reading it from the cache instead of HBM.  The default chunk for
 * M = 8192 is 8192 columns (134 MB of dlogits).  ws: 256-byte aligned,
 * >= coda_lmhead_ce_bwd_vchunk_workspace(M, V, d, vchunk) bytes. */
size_t coda_lmhead_ce_bwd_vchunk_workspace(int M, int V, int d, int vchunk);

coda_status coda_lmhead_ce_bwd_vchunk(const coda_bf16* H, int ldh, const coda_bf16* W, int ldw,
                                      const int32_t* labels, const float* lse, float grad_scale,
                                      coda_bf16* dH, int lddh, float* dW, int lddw, void* ws,
                                      size_t ws_bytes, int M, int V, int d, int vchunk,
                                      hipStream_t stream);

/* The same backward from the logits coda_lmhead_ce_logits kept: an
 * auxiliary kernel overwrites logits (bf16, M x V, ldl) in place with
 *   D = (exp(l - lse_i) - [k == label_i]) grad_scale  (bf16),
 * then dH = D W^T (bf16, M x d) and dW = H^T D (fp32, d x V, overwritten).
 * The logits buffer holds D afterwards.  No workspace. */
coda_status coda_lmhead_ce_bwd_logits(const coda_bf16* H, int ldh, const coda_bf16* W, int ldw,
                                      const int32_t* labels, const float* lse, float grad_scale,
                                      coda_bf16* logits, int ldl, coda_bf16* dH, int lddh,
                                      float* dW, int lddw, int M, int V, int d,
                                      hipStream_t stream);

/* ---------------------------------------------------------------------------
 * LayerNorm variant.  The paper's review page asks for LayerNorm gradients as
 * an epilogue composition (referee report, major comment 1; simulated
 * rebuttal, point 1).  With n = r (u - mu) gamma + beta, the mean and the
 * scale both move past GEMM2's projection W, as the reading notes move r
 * (section 2): n W = r ((u gamma) W - mu (gamma^T W)) + beta^T W, so GEMM2's
 * epilogue applies a row scale plus a rank-1 correction with the fp32
 * weight-side vectors c = gamma^T W and b = beta^T W.  In the backward the
 * two row statistics a = mean_j(G gamma) and s = mean_j(G gamma xhat)
 * (G = dL/dn, xhat = r (u - mu)) are, by the substitution of section 3,
 * a = (dY . c) / d and s = (sumcols(dY * y) - dY . b) / d: the next layer's
 * backward epilogue accumulates them.
 * ------------------------------------------------------------------------- */

/* GEMM1 with LayerNorm statistics: as coda_gemm_res_sumsq (U = XW + Z,
 * H2 = U * gamma opt), but the per-row partials are, per 128-feature wave
 * tile p, the tile's mean of the fp32 u (pmean) and its sum of squared
 * deviations from that mean (pm2), both fp32 [M x coda_nparts(N)] and
 * required. */
coda_status coda_gemm_res_lnstats(const coda_bf16* X, int ldx, const coda_bf16* W, int ldw,
                                  const coda_bf16* Z, int ldz, const coda_bf16* gamma,
                                  coda_bf16* U, int ldu, coda_bf16* H2, int ldh, float* pmean,
                                  float* pm2, int M, int N, int K, hipStream_t stream);

/* Auxiliary merge of those partials into the row statistics (tile p holds
 * min(128, d - 128 p) features; pairwise-update merge):
 *   mu_i = mean_j u_ij,  r_i = 1 / sqrt(mean_j (u_ij - mu_i)^2 + eps).
 * nparts must equal coda_nparts(d).  mu, r fp32 [M]. */
coda_status coda_row_ln(const float* pmean, const float* pm2, int nparts, int M, int d,
                        float eps, float* mu, float* r, hipStream_t stream);

/* Weight-side vectors of the mean correction: c_j = sum_k gamma_k W_kj and
 * (beta and bvec both given, or both NULL) b_j = sum_k beta_k W_kj, fp32 [N],
 * 16-byte aligned; W [K x N] bf16.  Computed once per weight. */
coda_status coda_ln_colvec(const coda_bf16* W, int ldw, const coda_bf16* gamma,
                           const coda_bf16* beta, int K, int N, float* cvec, float* bvec,
                           hipStream_t stream);

/* GEMM2 with the LayerNorm row transform: A = h2 = u * gamma [M x K],
 *   Y = bf16( r_i ((A W)_ij - mu_i c_j) + b_j )   (b opt: NULL means 0). */
coda_status coda_gemm_ln_rowscale(const coda_bf16* A, int lda, const coda_bf16* W, int ldw,
                                  const float* r, const float* mu, const float* cvec,
                                  const float* bvec, coda_bf16* Y, int ldy, int M, int N, int K,
                                  hipStream_t stream);

/* coda_gemm_swiglu after the LayerNorm row transform: the pre-activation is
 *   pre_ij = r_i ((A Wgu)_ij - mu_i c_j) + b_j over the interleaved 2F
 * columns (c, b fp32 [2F]), then Act = silu(gate) * up; Pre opt. */
coda_status coda_gemm_ln_swiglu(const coda_bf16* A, int lda, const coda_bf16* Wgu, int ldw,
                                const float* r, const float* mu, const float* cvec,
                                const float* bvec, coda_bf16* Act, int ldact, coda_bf16* Pre,
                                int ldp, int M, int F, int K, hipStream_t stream);

/* coda_gemm_swiglu_bwd whose epilogue accumulates the two LayerNorm row
 * statistics of the layer whose output Pre is (c, b = gamma^T Wgu,
 * beta^T Wgu of that layer, fp32 [2F]; b opt):
 *   spart[i, p] = sum_{j in part p} dPre_ij (Pre_ij - b_j)
 *   apart[i, p] = sum_{j in part p} dPre_ij c_j      (fp32 [M x coda_nparts(F)]). */
coda_status coda_gemm_swiglu_bwd_ln(const coda_bf16* dOut, int ldd, const coda_bf16* Wd, int ldw,
                                    const coda_bf16* Pre, int ldp, coda_bf16* dPre, int lddp,
                                    const float* cvec, const float* bvec, float* spart,
                                    float* apart, int M, int F, int N, hipStream_t stream);

/* Auxiliary reduction of those partials: s_i = sum_p spart[i, p] / d and
 * a_i = sum_p apart[i, p] / d, d = the LayerNorm width. */
coda_status coda_row_ln_bwd(const float* spart, const float* apart, int nparts, int M, int d,
                            float* s, float* a, hipStream_t stream);

/* Data-gradient GEMM with the delayed LayerNorm backward epilogue:
 *   G = dY W1^T;  dU = dRes + r_i (G * gamma) - r_i a_i - r_i^2 s_i (u - mu_i)
 *   N2 = bf16(r_i (u - mu_i) gamma + beta)   (opt; the weight-gradient operand)
 *   gpart[q, j] = sum_{i in part q} r_i G_ij (u_ij - mu_i)   (dgamma partials)
 *   bgpart[q, j] = sum_{i in part q} G_ij                     (dbeta partials)
 * both fp32 [coda_mparts(M) x d], reduced by coda_col_reduce; beta opt. */
coda_status coda_gemm_ln_bwd(const coda_bf16* dY, int ldd, const coda_bf16* W1, int ldw,
                             const coda_bf16* U, int ldu, const coda_bf16* gamma,
                             const coda_bf16* beta, const float* r, const float* mu,
                             const float* s, const float* a, const coda_bf16* dRes, int ldr,
                             coda_bf16* dU, int lddu, coda_bf16* N2, int ldn, float* gpart,
                             float* bgpart, int M, int d, int N, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CODA_H_ */
