// coda_api.hip - C ABI of libcoda.so: argument validation, kernel selection
// and launch of the fused GEMM-epilogue kernels and the auxiliary reductions.
//
// Every entry point validates its arguments before any HIP call, launches on
// the caller's stream and returns; nothing is allocated or synchronised.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "../../include/coda.h"
#include "coda_epilogues.hpp"
#include "coda_host.hpp"
#include "coda_mainloop_occ2.hpp"

using namespace coda;
using namespace coda_host;

namespace {

// ---------------------------------------------------------------------------
// Auxiliary reductions.  Bandwidth/latency-bound: every load instruction of a
// wave reads contiguous floats, the summation order is fixed (deterministic).
// ---------------------------------------------------------------------------

// Row sums of per-row partials [M x nparts] (row-major, ld = nparts), G lanes
// per row: lane k adds elements k, k+G, ..., then a butterfly over the G lanes.
// RMS: out_i = 1/sqrt(sum/d + eps) (paper Figure 4 / Figure 5 caption);
// otherwise out_i = sum/d (the backward statistic s, reading notes section 3).
template <int G, bool RMS>
__global__ void __launch_bounds__(256) row_reduce_kernel(const float* __restrict__ part, int nparts,
                                                         int M, float inv_d, float eps,
                                                         float* __restrict__ out) {
  const int row = blockIdx.x * (256 / G) + (int)threadIdx.x / G;
  const int k = (int)threadIdx.x % G;
  float s = 0.0f;
  if (row < M) {
    const float* p = part + (size_t)row * nparts;
#pragma unroll 4
    for (int j = k; j < nparts; j += G) s += p[j];
  }
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if (row < M && k == 0) out[row] = RMS ? 1.0f / sqrtf(s * inv_d + eps) : s * inv_d;
}

template <bool RMS>
void launch_row_reduce(const float* part, int nparts, int M, float inv_d, float eps, float* out,
                       hipStream_t stream) {
  if (nparts <= 4)
    hipLaunchKernelGGL((row_reduce_kernel<4, RMS>), dim3(cdiv(M, 64)), dim3(256), 0, stream, part,
                       nparts, M, inv_d, eps, out);
  else if (nparts <= 16)
    hipLaunchKernelGGL((row_reduce_kernel<16, RMS>), dim3(cdiv(M, 16)), dim3(256), 0, stream, part,
                       nparts, M, inv_d, eps, out);
  else
    hipLaunchKernelGGL((row_reduce_kernel<64, RMS>), dim3(cdiv(M, 4)), dim3(256), 0, stream, part,
                       nparts, M, inv_d, eps, out);
}

// dgamma_j = sum_q gpart[q, j]: a workgroup takes 32 columns, its eight
// waves-halves take every eighth partial row, and the eight slice sums are
// added in a fixed order.
constexpr int CR_COLS = 32, CR_SLICES = 8;
__global__ void __launch_bounds__(256) col_reduce_kernel(const float* __restrict__ gpart, int mparts,
                                                         int d, float* __restrict__ out) {
  __shared__ float sh[CR_SLICES][CR_COLS];
  const int c = (int)threadIdx.x % CR_COLS, sl = (int)threadIdx.x / CR_COLS;
  const int j = blockIdx.x * CR_COLS + c;
  float s = 0.0f;
  if (j < d) {
#pragma unroll 4
    for (int q = sl; q < mparts; q += CR_SLICES) s += gpart[(size_t)q * d + j];
  }
  sh[sl][c] = s;
  __syncthreads();
  if (sl == 0 && j < d) {
    float t = 0.0f;
#pragma unroll
    for (int k = 0; k < CR_SLICES; ++k) t += sh[k][c];
    out[j] = t;
  }
}

// Merge of per-tile (max, sum exp) into lse and the row loss (reading notes
// section 2, "Cross-entropy loss").  Partials are part-major ([nparts x ldp]).
// A workgroup takes 32 tokens; each of its 32 slices merges every 32nd part
// with one exponential per part (the smaller of the two maxima is rescaled),
// and the 32 slice states of a token are merged in a fixed order.
constexpr int CE_TOK = 32, CE_SLICES = 32;
__global__ void __launch_bounds__(1024) ce_reduce_kernel(const float* __restrict__ pm,
                                                         const float* __restrict__ ps,
                                                         const float* __restrict__ tgt,
                                                         const int32_t* __restrict__ labels,
                                                         int nparts, int M, int ldp, int V,
                                                         float* __restrict__ lse,
                                                         float* __restrict__ loss) {
  __shared__ float shm[CE_SLICES][CE_TOK], shs[CE_SLICES][CE_TOK];
  const int tl = (int)threadIdx.x % CE_TOK, sl = (int)threadIdx.x / CE_TOK;
  const int i = blockIdx.x * CE_TOK + tl;
  float m = -INFINITY, s = 0.0f;
  if (i < M) {
#pragma unroll 4
    for (int j = sl; j < nparts; j += CE_SLICES) {
      const float a = pm[(size_t)j * ldp + i], b = ps[(size_t)j * ldp + i];
      if (a > -INFINITY) {
        const float dl = a - m;
        const bool up = dl > 0.0f;
        const float e = expf(-fabsf(dl));
        s = up ? fmaf(s, e, b) : fmaf(b, e, s);
        m = up ? a : m;
      }
    }
  }
  shm[sl][tl] = m;
  shs[sl][tl] = s;
  __syncthreads();
  if (sl == 0 && i < M) {
    float L = -INFINITY;
#pragma unroll
    for (int k = 0; k < CE_SLICES; ++k) L = fmaxf(L, shm[k][tl]);
    float S = 0.0f;
#pragma unroll
    for (int k = 0; k < CE_SLICES; ++k)
      S += shm[k][tl] > -INFINITY ? shs[k][tl] * expf(shm[k][tl] - L) : 0.0f;
    const float l = L + logf(S);
    lse[i] = l;
    const int y = labels[i];
    loss[i] = (y >= 0 && y < V) ? (l - tgt[i]) : __builtin_nanf("");
  }
}

// dlogits from stored bf16 logits, in place: D_ik = (exp(l_ik - lse_i) -
// [k == label_i]) * scale, the gradient of scale * sum_i loss_i (reading
// notes section 2, "Cross-entropy loss").  A thread takes one 16-byte chunk
// (8 logits) of every gridDim.y-th row.
__global__ void __launch_bounds__(256) ce_dlogits_kernel(uint16_t* __restrict__ L, int ldl,
                                                         const int32_t* __restrict__ labels,
                                                         const float* __restrict__ lse, float scale,
                                                         int M, int V) {
  const int c = blockIdx.x * 256 + (int)threadIdx.x;
  if (8 * c >= V) return;
  for (int i = blockIdx.y; i < M; i += gridDim.y) {
    uint16_t* p = L + (size_t)i * ldl + 8 * c;
    const float ls = lse[i];
    const int y = labels[i] - 8 * c;
    float v[8];
    unpack8(ld16(p), v);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      v[e] = (__builtin_amdgcn_exp2f((v[e] - ls) * LOG2E) - (y == e ? 1.0f : 0.0f)) * scale;
    st16(p, pack8(v));
  }
}

// Deterministic mean of the row losses: one workgroup, fixed-order tree.
__global__ void __launch_bounds__(1024) mean_kernel(const float* __restrict__ x, int M,
                                                    float* __restrict__ out) {
  __shared__ float sh[1024];
  float s = 0.0f;
  for (int i = threadIdx.x; i < M; i += 1024) s += x[i];
  sh[threadIdx.x] = s;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) sh[threadIdx.x] += sh[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = sh[0] / (float)M;
}

// Launch one fused GEMM: features F (output columns), tokens T (output rows).
// Epilogues that work on any wave-tile width (all but the dgamma column
// partials, which are laid out per 128-token wave tile).
template <class Epi>
struct AnyWaveWidth : std::true_type {};
template <bool A, bool B, bool C>
struct AnyWaveWidth<EpiRowscaleBwd<A, B, C>> : std::false_type {};

#ifndef CODA_OCC2
#define CODA_OCC2 0
#endif

// Two workgroups per CU (256 x 128 tiles, coda_mainloop_occ2.hpp).
template <bool WK, class Epi>
coda_status launch_gemm_occ2(const uint16_t* W, int ldw, const uint16_t* X, int ldx, int F, int T, int K,
                             const Epi& epi, hipStream_t stream) {
  Problem p;
  p.W = W;
  p.X = X;
  p.ldw = ldw;
  p.ldx = ldx;
  p.F = F;
  p.T = T;
  p.K = K;
  p.nTF = cdiv(F, occ2::BF);
  p.nTT = cdiv(T, occ2::BT);
  p.f_base = 0;
  const int nb = p.nTF * p.nTT;
  if (nb == 0) return CODA_OK;
  hipLaunchKernelGGL((occ2::gemm_epi_kernel_occ2<WK, Epi>), dim3(nb), dim3(NT), 0, stream, p, epi);
  return launched();
}

// Tile-count quantization.  One 256x256 tile per CU at a time: when the tile
// count leaves the last round of tiles partly empty (8192 x 3072 has 384
// tiles = 1.5 rounds on 256 CUs), the trailing feature range can instead be
// covered by 256-feature x 128-token tiles, two per big tile, each taking
// about 0.6 of a big tile's time (measured on 8192 x 3072 x 2048).  Returns
// the number of 256-wide feature tiles to keep in big tiles (the rest go to
// the half tiles), or 0 to keep every tile big.  Cost model in rounds: a big
// round is 1, a half-tile round 0.6; a split must save at least 0.2 rounds.
inline int quantization_split(int nTF, int nTT, int nTT_half, int cus) {
  if (cus <= 0 || nTF < 2) return 0;
  const double base = (double)cdiv(nTF * nTT, cus);
  double best = base - 0.2;
  int split = 0;
  for (int f1 = 1; f1 < nTF; ++f1) {
    const double c = (double)cdiv(f1 * nTT, cus) + 0.6 * (double)cdiv((nTF - f1) * nTT_half, cus);
    if (c < best) {
      best = c;
      split = f1;
    }
  }
  return split;
}

template <bool WK, bool XK, int BT = 256, class Epi>
coda_status launch_gemm(const uint16_t* W, int ldw, const uint16_t* X, int ldx, int F, int T, int K,
                        const Epi& epi, hipStream_t stream) {
  if constexpr (CODA_OCC2 && XK && AnyWaveWidth<Epi>::value && EpiLds<Epi>::value == 0) {
    return launch_gemm_occ2<WK>(W, ldw, X, ldx, F, T, K, epi, stream);
  }
  constexpr int BF = 256;
  Problem p;
  p.W = W;
  p.X = X;
  p.ldw = ldw;
  p.ldx = ldx;
  p.F = F;
  p.T = T;
  p.K = K;
  p.nTF = cdiv(F, BF);
  p.nTT = cdiv(T, BT);
  p.f_base = 0;
  const int nb = p.nTF * p.nTT;
  if (nb == 0) return CODA_OK;
  if constexpr (BT == 256 && XK && AnyWaveWidth<Epi>::value) {
    const int cus = device_cus();
    const int split = coda_tile_split(F, T, cus);
    if (split > 0) {
      Problem big = p, half = p;
      big.nTF = split;
      half.f_base = split * BF;
      half.nTF = p.nTF - split;
      half.nTT = cdiv(T, 128);
      hipLaunchKernelGGL((gemm_epi_kernel_split<WK, XK, Epi>), dim3(big.nTF * big.nTT + half.nTF * half.nTT),
                         dim3(NT), 0, stream, big, half, epi);
      return launched();
    }
    // Under half a round of big tiles: 256 x 128 tiles run on twice as many
    // CUs in the same single round, so each CU's k-loop and epilogue (the
    // whole cost of a small GEMM) are about half as long.
    if (cus > 0 && 2 * nb <= cus && cdiv(T, 128) > p.nTT) {
      Problem none = p, half = p;
      none.nTF = 0;
      half.nTT = cdiv(T, 128);
      hipLaunchKernelGGL((gemm_epi_kernel_split<WK, XK, Epi>), dim3(half.nTF * half.nTT), dim3(NT), 0,
                         stream, none, half, epi);
      return launched();
    }
  }
  hipLaunchKernelGGL((gemm_epi_kernel<BF, BT, WK, XK, Epi>), dim3(nb), dim3(NT), 0, stream, p, epi);
  return launched();
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================

extern "C" {

const char* coda_status_str(coda_status s) {
  switch (s) {
    case CODA_OK: return "ok";
    case CODA_ERR_NULL: return "a required pointer is NULL";
    case CODA_ERR_SHAPE: return "invalid size or leading dimension";
    case CODA_ERR_ALIGN: return "pointer or leading dimension misaligned";
    case CODA_ERR_UNSUPPORTED: return "unsupported device or parameter combination";
    case CODA_ERR_HIP: return "HIP runtime error";
    case CODA_ERR_WORKSPACE: return "workspace missing or too small";
  }
  return "unknown status";
}

const char* coda_version(void) { return "coda-gfx950 0.1"; }

int coda_nparts(int N) { return N <= 0 ? 0 : cdiv(N, WAVE_F); }
int coda_mparts(int M) { return M <= 0 ? 0 : cdiv(M, WAVE_T); }
int coda_tile_split(int F, int T, int cus) {
  if (F <= 0 || T <= 0) return 0;
  return quantization_split(cdiv(F, 256), cdiv(T, 256), cdiv(T, 128), cus);
}

size_t coda_lmhead_ce_workspace(int M, int V) {
  if (M <= 0 || V <= 0) return 0;
  const size_t np = (size_t)coda_nparts(V);
  return (2 * (size_t)M * np + 2 * (size_t)M) * sizeof(float);
}

static const int kCeBwdMinRows = 256;

size_t coda_lmhead_ce_bwd_workspace(int M, int V, int d) {
  (void)d;
  if (M <= 0 || V <= 0) return 0;
  const size_t rows = (size_t)(M < kCeBwdMinRows ? M : kCeBwdMinRows);
  return rows * (size_t)V * 2;
}

coda_status coda_gemm(const coda_bf16* X, int ldx, const coda_bf16* W, int ldw, coda_bf16* Y,
                      int ldy, int M, int N, int K, hipStream_t stream) {
  Check c;
  c.shape(M >= 0 && N >= 0 && K >= 0);
  c.bmat(X, ldx, K, true, M);
  c.bmat(W, ldw, N);
  c.bmat(Y, ldy, N, true, M);
  c.shape(N % 8 == 0 && K % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || N == 0) return CODA_OK;
  if (coda_status s = device_ok()) return s;
  EpiLinear<false, false> e{nullptr, nullptr, 0, Y, ldy};
  return launch_gemm<false, true>(W, ldw, X, ldx, N, M, K, e, stream);
}

coda_status coda_gemm_res_sumsq(const coda_bf16* X, int ldx, const coda_bf16* W, int ldw,
                                const coda_bf16* Z, int ldz, const coda_bf16* gamma, coda_bf16* U,
                                int ldu, coda_bf16* H2, int ldh, float* part, int M, int N, int K,
                                hipStream_t stream) {
  Check c;
  c.shape(M >= 0 && N >= 0 && K >= 0);
  c.bmat(X, ldx, K, true, M);
  c.bmat(W, ldw, N);
  c.bmat(Z, ldz, N, false, M);
  c.bmat(U, ldu, N, true, M);
  c.bmat(H2, ldh, N, false, M);
  if (H2) c.vec(gamma, true, true);
  c.vec(part, false, false, M);
  c.shape(N % 8 == 0 && K % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || N == 0) return CODA_OK;
  if (coda_status s = device_ok()) return s;
  const int np = coda_nparts(N);
#define CODA_RS(HZ, HH, HP)                                                              \
  {                                                                                      \
    EpiResSumsq<HZ, HH, HP> e{Z, ldz, gamma, U, ldu, H2, ldh, part, np};                 \
    return launch_gemm<false, true>(W, ldw, X, ldx, N, M, K, e, stream);                 \
  }
  const bool hz = Z != nullptr, hh = H2 != nullptr, hp = part != nullptr;
  if (hz && hh && hp) CODA_RS(true, true, true)
  if (hz && hh && !hp) CODA_RS(true, true, false)
  if (hz && !hh && hp) CODA_RS(true, false, true)
  if (hz && !hh && !hp) CODA_RS(true, false, false)
  if (!hz && hh && hp) CODA_RS(false, true, true)
  if (!hz && hh && !hp) CODA_RS(false, true, false)
  if (!hz && !hh && hp) CODA_RS(false, false, true)
  CODA_RS(false, false, false)
#undef CODA_RS
}

coda_status coda_row_rms(const float* part, int nparts, int M, int d, float eps, float* r,
                         hipStream_t stream) {
  Check c;
  c.shape(M >= 0 && nparts >= 1 && d >= 1 && eps >= 0.0f);
  c.vec(part, true, false, M);
  c.vec(r, true, false, M);
  if (c.st != CODA_OK) return c.st;
  if (M == 0) return CODA_OK;
  if (coda_status s = device_ok()) return s;
  launch_row_reduce<true>(part, nparts, M, 1.0f / (float)d, eps, r, stream);
  return launched();
}

coda_status coda_gemm_rowscale(const coda_bf16* A, int lda, const coda_bf16* W, int ldw,
                               const float* r, coda_bf16* Y, int ldy, int M, int N, int K,
                               hipStream_t stream) {
  Check c;
  c.shape(M >= 0 && N >= 0 && K >= 0);
  c.bmat(A, lda, K, true, M);
  c.bmat(W, ldw, N);
  c.vec(r, true, false, M);
  c.bmat(Y, ldy, N, true, M);
  c.shape(N % 8 == 0 && K % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || N == 0) return CODA_OK;
  if (coda_status s = device_ok()) return s;
  EpiLinear<true, false> e{r, nullptr, 0, Y, ldy};
  return launch_gemm<false, true>(W, ldw, A, lda, N, M, K, e, stream);
}

static coda_status rope_common(const coda_bf16* A, int lda, const coda_bf16* W, int ldw,
                               const float* r, const int32_t* pos, float theta, int head_dim,
                               int n_rope, coda_bf16* Y, int ldy, int M, int N, int K, bool inv,
                               hipStream_t stream) {
  Check c;
  c.shape(M >= 0 && N >= 0 && K >= 0);
  c.bmat(A, lda, K, true, M);
  c.bmat(W, ldw, N);
  c.vec(r, false, false, M);
  c.vec(pos, true, false, M);
  c.bmat(Y, ldy, N, true, M);
  c.shape(N % 8 == 0 && K % 8 == 0);
  c.unsupported(head_dim >= 2 && head_dim % 2 == 0 && n_rope >= 0 && n_rope <= N &&
                n_rope % head_dim == 0 && n_rope % 8 == 0 && theta > 0.0f);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || N == 0) return CODA_OK;
  if (coda_status s = device_ok()) return s;
  const float l2t = (float)std::log2((double)theta);
#define CODA_RP(HR, INV)                                                   \
  {                                                                        \
    EpiRope<HR, INV> e{r, pos, l2t, head_dim, n_rope, Y, ldy};             \
    return launch_gemm<false, true>(W, ldw, A, lda, N, M, K, e, stream);   \
  }
  if (r && !inv) CODA_RP(true, false)
  if (!r && !inv) CODA_RP(false, false)
  if (r && inv) CODA_RP(true, true)
  CODA_RP(false, true)
#undef CODA_RP
}

coda_status coda_gemm_rope(const coda_bf16* A, int lda, const coda_bf16* W, int ldw,
                           const float* r, const int32_t* pos, float theta, int head_dim,
                           int n_rope, coda_bf16* Y, int ldy, int M, int N, int K,
                           hipStream_t stream) {
  return rope_common(A, lda, W, ldw, r, pos, theta, head_dim, n_rope, Y, ldy, M, N, K, false,
                     stream);
}

coda_status coda_gemm_rope_bwd(const coda_bf16* A, int lda, const coda_bf16* W, int ldw,
                               const float* r, const int32_t* pos, float theta, int head_dim,
                               int n_rope, coda_bf16* Y, int ldy, int M, int N, int K,
                               hipStream_t stream) {
  return rope_common(A, lda, W, ldw, r, pos, theta, head_dim, n_rope, Y, ldy, M, N, K, true,
                     stream);
}

coda_status coda_gemm_swiglu(const coda_bf16* A, int lda, const coda_bf16* Wgu, int ldw,
                             const float* r, coda_bf16* Act, int ldact, coda_bf16* Pre, int ldp,
                             int M, int F, int K, hipStream_t stream) {
  Check c;
  c.shape(M >= 0 && F >= 0 && K >= 0);
  c.shape(F <= (1 << 29));
  if (c.st != CODA_OK) return c.st;
  c.bmat(A, lda, K, true, M);
  c.bmat(Wgu, ldw, 2 * F);
  c.vec(r, false, false, M);
  c.vec(Act, true, false, M);
  if (c.st == CODA_OK && (ldact < F)) c.st = CODA_ERR_SHAPE;
  if (c.st == CODA_OK && (!al16(Act) || ldact % 4 != 0)) c.st = CODA_ERR_ALIGN;
  c.bmat(Pre, ldp, 2 * F, false, M);
  c.shape(F % 4 == 0 && K % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || F == 0) return CODA_OK;
  if (coda_status s = device_ok()) return s;
#define CODA_SW(HR, HP)                                                          \
  {                                                                              \
    EpiSwiglu<HR, HP> e{r, Act, ldact, Pre, ldp};                                \
    return launch_gemm<false, true>(Wgu, ldw, A, lda, 2 * F, M, K, e, stream);   \
  }
  if (r && Pre) CODA_SW(true, true)
  if (r && !Pre) CODA_SW(true, false)
  if (!r && Pre) CODA_SW(false, true)
  CODA_SW(false, false)
#undef CODA_SW
}

static coda_status lmhead_ce_common(const coda_bf16* H, int ldh, const coda_bf16* W, int ldw,
                                    const int32_t* labels, float* lse, float* loss_row,
                                    float* loss_mean, coda_bf16* logits, int ldl, bool keep,
                                    void* ws, size_t ws_bytes, int M, int V, int d,
                                    hipStream_t stream) {
  Check c;
  c.shape(M >= 0 && V >= 0 && d >= 0);
  c.bmat(H, ldh, d, true, M);
  c.bmat(W, ldw, V);
  c.vec(labels, true, false, M);
  c.vec(lse, true, false, M);
  c.vec(loss_row, false);
  c.vec(loss_mean, false);
  if (keep) c.bmat(logits, ldl, V, true, M);
  c.shape(V % 8 == 0 && d % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || V == 0) return CODA_OK;
  if (ws == nullptr || !al16(ws) || ws_bytes < coda_lmhead_ce_workspace(M, V))
    return CODA_ERR_WORKSPACE;
  if (coda_status s = device_ok()) return s;
  const int np = coda_nparts(V);
  float* pm = static_cast<float*>(ws);
  float* ps = pm + (size_t)M * np;
  float* tgt = ps + (size_t)M * np;
  float* lrow = tgt + M;
  if (loss_row == nullptr) loss_row = lrow;
  if (keep) {
    EpiCE<true> e{labels, pm, ps, tgt, M, logits, ldl};
    if (coda_status s = launch_gemm<false, true>(W, ldw, H, ldh, V, M, d, e, stream)) return s;
  } else {
    EpiCE<false> e{labels, pm, ps, tgt, M, nullptr, 0};
    if (coda_status s = launch_gemm<false, true>(W, ldw, H, ldh, V, M, d, e, stream)) return s;
  }
  hipLaunchKernelGGL(ce_reduce_kernel, dim3(cdiv(M, CE_TOK)), dim3(CE_TOK * CE_SLICES), 0, stream,
                     pm, ps, tgt, labels, np, M, M, V, lse, loss_row);
  if (coda_status s = launched()) return s;
  if (loss_mean) {
    hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(1024), 0, stream, loss_row, M, loss_mean);
    return launched();
  }
  return CODA_OK;
}

coda_status coda_lmhead_ce(const coda_bf16* H, int ldh, const coda_bf16* W, int ldw,
                           const int32_t* labels, float* lse, float* loss_row, float* loss_mean,
                           void* ws, size_t ws_bytes, int M, int V, int d, hipStream_t stream) {
  return lmhead_ce_common(H, ldh, W, ldw, labels, lse, loss_row, loss_mean, nullptr, 0, false, ws,
                          ws_bytes, M, V, d, stream);
}

coda_status coda_lmhead_ce_logits(const coda_bf16* H, int ldh, const coda_bf16* W, int ldw,
                                  const int32_t* labels, float* lse, float* loss_row,
                                  float* loss_mean, coda_bf16* logits, int ldl, void* ws,
                                  size_t ws_bytes, int M, int V, int d, hipStream_t stream) {
  return lmhead_ce_common(H, ldh, W, ldw, labels, lse, loss_row, loss_mean, logits, ldl, true, ws,
                          ws_bytes, M, V, d, stream);
}

coda_status coda_gemm_swiglu_bwd(const coda_bf16* dOut, int ldd, const coda_bf16* Wd, int ldw,
                                 const coda_bf16* Pre, int ldp, coda_bf16* dPre, int lddp,
                                 float* spart, int M, int F, int N, hipStream_t stream) {
  Check c;
  c.shape(M >= 0 && F >= 0 && N >= 0 && F <= (1 << 29));
  if (c.st != CODA_OK) return c.st;
  c.bmat(dOut, ldd, N, true, M);
  c.bmat(Wd, ldw, N);
  c.bmat(Pre, ldp, 2 * F, true, M);
  c.bmat(dPre, lddp, 2 * F, true, M);
  c.vec(spart, false, false, M);
  c.shape(F % 8 == 0 && N % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || F == 0) return CODA_OK;
  if (coda_status s = device_ok()) return s;
  const int np = coda_nparts(F);
  // da[M x F] = dOut[M x N] Wd^T: features = F (rows of Wd, K-major), tokens = M.
  if (spart) {
    EpiSwigluBwd<true> e{Pre, ldp, dPre, lddp, spart, np};
    return launch_gemm<true, true>(Wd, ldw, dOut, ldd, F, M, N, e, stream);
  }
  EpiSwigluBwd<false> e{Pre, ldp, dPre, lddp, nullptr, np};
  return launch_gemm<true, true>(Wd, ldw, dOut, ldd, F, M, N, e, stream);
}

coda_status coda_row_rms_bwd(const float* spart, int nparts, int M, int d, float* s,
                             hipStream_t stream) {
  Check c;
  c.shape(M >= 0 && nparts >= 1 && d >= 1);
  c.vec(spart, true, false, M);
  c.vec(s, true, false, M);
  if (c.st != CODA_OK) return c.st;
  if (M == 0) return CODA_OK;
  if (coda_status st = device_ok()) return st;
  launch_row_reduce<false>(spart, nparts, M, 1.0f / (float)d, 0.0f, s, stream);
  return launched();
}

coda_status coda_gemm_rowscale_bwd(const coda_bf16* dY, int ldd, const coda_bf16* W1, int ldw,
                                   const coda_bf16* U, int ldu, const coda_bf16* gamma,
                                   const float* r, const float* s, const coda_bf16* dRes, int ldr,
                                   coda_bf16* dU, int lddu, coda_bf16* N2, int ldn, float* gpart,
                                   int M, int d, int N, hipStream_t stream) {
  Check c;
  c.shape(M >= 0 && d >= 0 && N >= 0);
  c.bmat(dY, ldd, N, true, M);
  c.bmat(W1, ldw, N);
  c.bmat(U, ldu, d, true, M);
  c.vec(gamma, true, true);
  c.vec(r, true, false, M);
  c.vec(s, true, false, M);
  c.bmat(dRes, ldr, d, false, M);
  c.bmat(dU, lddu, d, true, M);
  c.bmat(N2, ldn, d, false, M);
  c.vec(gpart, false);
  c.shape(d % 8 == 0 && N % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || d == 0) return CODA_OK;
  if (coda_status st = device_ok()) return st;
#define CODA_RB(HR, HN, HG)                                                             \
  {                                                                                     \
    EpiRowscaleBwd<HR, HN, HG> e{U, ldu, gamma, r, s, dRes, ldr, dU, lddu, N2, ldn,     \
                                 gpart, d};                                             \
    return launch_gemm<true, true, 256>(W1, ldw, dY, ldd, d, M, N, e, stream);          \
  }
  const bool hr = dRes != nullptr, hn = N2 != nullptr, hg = gpart != nullptr;
  if (hr && hn && hg) CODA_RB(true, true, true)
  if (hr && hn && !hg) CODA_RB(true, true, false)
  if (hr && !hn && hg) CODA_RB(true, false, true)
  if (hr && !hn && !hg) CODA_RB(true, false, false)
  if (!hr && hn && hg) CODA_RB(false, true, true)
  if (!hr && hn && !hg) CODA_RB(false, true, false)
  if (!hr && !hn && hg) CODA_RB(false, false, true)
  CODA_RB(false, false, false)
#undef CODA_RB
}

coda_status coda_col_reduce(const float* gpart, int mparts, int d, float* dgamma,
                            hipStream_t stream) {
  Check c;
  c.shape(mparts >= 1 && d >= 0);
  c.vec(gpart);
  c.vec(dgamma);
  if (c.st != CODA_OK) return c.st;
  if (d == 0) return CODA_OK;
  if (coda_status st = device_ok()) return st;
  hipLaunchKernelGGL(col_reduce_kernel, dim3(cdiv(d, CR_COLS)), dim3(256), 0, stream, gpart, mparts,
                     d, dgamma);
  return launched();
}

coda_status coda_gemm_wgrad(const coda_bf16* X, int ldx, const coda_bf16* dY, int ldd, float* dW,
                            int lddw, int M, int K, int N, int accumulate, hipStream_t stream) {
  Check c;
  c.shape(M >= 0 && K >= 0 && N >= 0);
  c.bmat(X, ldx, K, true, M);
  c.bmat(dY, ldd, N, true, M);
  c.fmat(dW, lddw, N);
  c.shape(K % 8 == 0 && N % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (K == 0 || N == 0) return CODA_OK;
  if (coda_status st = device_ok()) return st;
  // dW[K x N] = X^T dY: features = N (dY, contiguous along N -> MN-major),
  // tokens = K (X, contiguous along K -> MN-major), reduction = M.
  if (accumulate) {
    EpiF32<true> e{dW, lddw};
    return launch_gemm<false, false>(dY, ldd, X, ldx, N, K, M, e, stream);
  }
  EpiF32<false> e{dW, lddw};
  return launch_gemm<false, false>(dY, ldd, X, ldx, N, K, M, e, stream);
}

coda_status coda_gemm_res_sumsq_bwd(const coda_bf16* dU, int ldu, const coda_bf16* W, int ldw,
                                    const coda_bf16* X, int ldx, const coda_bf16* dRes, int ldr,
                                    coda_bf16* dX, int lddx, float* dW, int lddw, int M, int N,
                                    int K, hipStream_t stream) {
  Check c;
  c.shape(M >= 0 && N >= 0 && K >= 0);
  c.bmat(dU, ldu, N, true, M);
  c.bmat(W, ldw, N);
  c.bmat(dRes, ldr, K, false, M);
  c.bmat(dX, lddx, K, true, M);
  if (dW) {
    c.bmat(X, ldx, K, true, M);
    c.fmat(dW, lddw, N);
  }
  c.shape(N % 8 == 0 && K % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 && dW == nullptr) return CODA_OK;
  if (coda_status st = device_ok()) return st;
  if (M > 0 && K > 0) {
    // dX[M x K] = dU[M x N] W^T: features = K (rows of W, K-major over N).
    coda_status s2;
    if (dRes) {
      EpiLinear<false, true> e{nullptr, dRes, ldr, dX, lddx};
      s2 = launch_gemm<true, true>(W, ldw, dU, ldu, K, M, N, e, stream);
    } else {
      EpiLinear<false, false> e{nullptr, nullptr, 0, dX, lddx};
      s2 = launch_gemm<true, true>(W, ldw, dU, ldu, K, M, N, e, stream);
    }
    if (s2 != CODA_OK) return s2;
  }
  if (dW) return coda_gemm_wgrad(X, ldx, dU, ldu, dW, lddw, M, K, N, 0, stream);
  return CODA_OK;
}

coda_status coda_lmhead_ce_bwd(const coda_bf16* H, int ldh, const coda_bf16* W, int ldw,
                               const int32_t* labels, const float* lse, float grad_scale,
                               coda_bf16* dH, int lddh, float* dW, int lddw, void* ws,
                               size_t ws_bytes, int M, int V, int d, hipStream_t stream) {
  Check c;
  c.shape(M >= 0 && V >= 0 && d >= 0);
  c.bmat(H, ldh, d, true, M);
  c.bmat(W, ldw, V);
  c.vec(labels, true, false, M);
  c.vec(lse, true, false, M);
  c.bmat(dH, lddh, d, true, M);
  c.fmat(dW, lddw, V);
  c.shape(V % 8 == 0 && d % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (V == 0 || d == 0) return CODA_OK;
  if (M > 0 && (ws == nullptr || !al16(ws) || ws_bytes < coda_lmhead_ce_bwd_workspace(M, V, d)))
    return CODA_ERR_WORKSPACE;
  if (coda_status st = device_ok()) return st;
  if (M == 0)  // no rows: dW = H^T D over an empty reduction = 0
    return coda_gemm_wgrad(H, ldh, nullptr, V, dW, lddw, 0, d, V, 0, stream);
  // Rows per chunk: as many as the workspace holds, a multiple of 256.
  size_t rows = ws_bytes / ((size_t)V * 2);
  if (rows >= (size_t)M) rows = (size_t)M;
  else rows = (rows / 256) * 256;
  if (rows == 0) rows = (size_t)M;  // M < 256 and the workspace holds all rows
  uint16_t* D = static_cast<uint16_t*>(ws);
  for (int m0 = 0; m0 < M; m0 += (int)rows) {
    const int mc = (M - m0) < (int)rows ? (M - m0) : (int)rows;
    const uint16_t* Hc = H + (size_t)m0 * ldh;
    // 1) recompute logits and form dlogits D[mc x V] (bf16) in the epilogue
    EpiCEBwd e1{labels + m0, lse + m0, grad_scale, D, V};
    if (coda_status s = launch_gemm<false, true>(W, ldw, Hc, ldh, V, mc, d, e1, stream)) return s;
    // 2) dH[mc x d] = D W^T: features = d (rows of W, contiguous along V)
    EpiLinear<false, false> e2{nullptr, nullptr, 0, dH + (size_t)m0 * lddh, lddh};
    if (coda_status s = launch_gemm<true, true>(W, ldw, D, V, d, mc, V, e2, stream)) return s;
    // 3) dW[d x V] (+)= Hc^T D
    if (coda_status s = coda_gemm_wgrad(Hc, ldh, D, V, dW, lddw, mc, d, V, m0 > 0, stream))
      return s;
  }
  return CODA_OK;
}

coda_status coda_lmhead_ce_bwd_logits(const coda_bf16* H, int ldh, const coda_bf16* W, int ldw,
                                      const int32_t* labels, const float* lse, float grad_scale,
                                      coda_bf16* logits, int ldl, coda_bf16* dH, int lddh,
                                      float* dW, int lddw, int M, int V, int d,
                                      hipStream_t stream) {
  Check c;
  c.shape(M >= 0 && V >= 0 && d >= 0);
  c.bmat(H, ldh, d, true, M);
  c.bmat(W, ldw, V);
  c.vec(labels, true, false, M);
  c.vec(lse, true, false, M);
  c.bmat(logits, ldl, V, true, M);
  c.bmat(dH, lddh, d, true, M);
  c.fmat(dW, lddw, V);
  c.shape(V % 8 == 0 && d % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (V == 0 || d == 0) return CODA_OK;
  if (coda_status st = device_ok()) return st;
  if (M == 0)  // no rows: dW = H^T D over an empty reduction = 0
    return coda_gemm_wgrad(H, ldh, nullptr, V, dW, lddw, 0, d, V, 0, stream);
  // 1) dlogits in place of the logits
  hipLaunchKernelGGL(ce_dlogits_kernel, dim3(cdiv(V / 8, 256), M < 2048 ? M : 2048), dim3(256), 0,
                     stream, logits, ldl, labels, lse, grad_scale, M, V);
  if (coda_status s = launched()) return s;
  // 2) dH[M x d] = D W^T: features = d (rows of W, contiguous along V)
  EpiLinear<false, false> e2{nullptr, nullptr, 0, dH, lddh};
  if (coda_status s = launch_gemm<true, true>(W, ldw, logits, ldl, d, M, V, e2, stream)) return s;
  // 3) dW[d x V] = H^T D
  return coda_gemm_wgrad(H, ldh, logits, ldl, dW, lddw, M, d, V, 0, stream);
}

}  // extern "C"
