// coda_ln.hip - the LayerNorm variant of the GEMM -> residual -> norm -> GEMM
// composition, forward and backward, on the same fixed mainloop.
//
// The paper's review page asks for LayerNorm gradients as an epilogue
// composition (referee report, major comment 1) and the simulated rebuttal
// promises the LayerNorm backward pass with its residual-gradient path
// (point 1).  LayerNorm adds a mean to RMSNorm's scale: n = r (u - mu) gamma +
// beta.  Both move past GEMM2's projection W the way the reading notes move r
// (section 2): n W = r ((u gamma) W - mu gamma^T W) + beta^T W, a row scale
// plus a rank-1 correction with the weight-side vectors c = gamma^T W and
// b = beta^T W.  In the backward, the two row statistics a = mean(G gamma)
// and s = mean(G gamma xhat) (G = dL/dn) are, by the substitution of section
// 3, sumcols of the next GEMM's output side: a = dY c / d and
// s = (sumcols(dY y) - dY b) / d, so the next layer's backward epilogue
// accumulates them.
//
// Every entry point validates its arguments before any HIP call, launches on
// the caller's stream and returns; nothing is allocated or synchronised.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/coda.h"
#include "coda_launch.hpp"

using namespace coda;
using namespace coda_host;
using namespace coda_launch;

namespace {

// Row LayerNorm statistics from the per-wave-tile (mean, M2) partials of
// coda_gemm_res_lnstats: tile t holds n_t = min(128, d - 128 t) features, so
// mu = sum_t n_t m_t / d and M2 = sum_t (M2_t + n_t (m_t - mu)^2) (the
// pairwise-update merge); r = 1 / sqrt(M2 / d + eps).  G lanes per row: lane
// k takes tiles k, k + G, ...; butterflies over the G lanes finish both sums.
template <int G>
__global__ void __launch_bounds__(256) row_ln_kernel(const float* __restrict__ pmean,
                                                     const float* __restrict__ pm2, int nparts, int M,
                                                     int d, float eps, float* __restrict__ mu,
                                                     float* __restrict__ r) {
  const int row = blockIdx.x * (256 / G) + (int)threadIdx.x / G;
  const int k = (int)threadIdx.x % G;
  const bool on = row < M;
  const float* pm = pmean + (size_t)(on ? row : 0) * nparts;
  const float* pq = pm2 + (size_t)(on ? row : 0) * nparts;
  float s = 0.0f;
  if (on) {
    for (int j = k; j < nparts; j += G) {
      const int nt = min(WAVE_F, d - WAVE_F * j);
      s = fmaf((float)nt, pm[j], s);
    }
  }
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) s += __shfl_xor(s, o);
  const float m = s / (float)d;
  float q = 0.0f;
  if (on) {
    for (int j = k; j < nparts; j += G) {
      const int nt = min(WAVE_F, d - WAVE_F * j);
      const float dm = pm[j] - m;
      q += fmaf((float)nt * dm, dm, pq[j]);
    }
  }
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) q += __shfl_xor(q, o);
  if (on && k == 0) {
    mu[row] = m;
    r[row] = 1.0f / sqrtf(q / (float)d + eps);
  }
}

// The backward row statistics: s = sum spart / d and a = sum apart / d.
template <int G>
__global__ void __launch_bounds__(256) row_ln_bwd_kernel(const float* __restrict__ spart,
                                                         const float* __restrict__ apart, int nparts,
                                                         int M, float inv_d, float* __restrict__ s,
                                                         float* __restrict__ a) {
  const int row = blockIdx.x * (256 / G) + (int)threadIdx.x / G;
  const int k = (int)threadIdx.x % G;
  float ss = 0.0f, sa = 0.0f;
  if (row < M) {
    const float* ps = spart + (size_t)row * nparts;
    const float* pa = apart + (size_t)row * nparts;
    for (int j = k; j < nparts; j += G) {
      ss += ps[j];
      sa += pa[j];
    }
  }
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) {
    ss += __shfl_xor(ss, o);
    sa += __shfl_xor(sa, o);
  }
  if (row < M && k == 0) {
    s[row] = ss * inv_d;
    a[row] = sa * inv_d;
  }
}

// G lanes per row: the smallest of 4, 16, 64 that covers nparts (at most 64).
inline int lanes_per_row(int nparts) { return nparts <= 4 ? 4 : nparts <= 16 ? 16 : 64; }

// c = gamma^T W and b = beta^T W for W [K x N] (the weight-side vectors of
// the mean correction).  A workgroup takes 256 columns: 32 lanes of 8
// columns (one 16-byte load per row) times 8 row slices, whose sums are
// added in a fixed order through the LDS.
constexpr int CV_LANES = 32, CV_SLICES = 8, CV_COLS = 8 * CV_LANES;
__global__ void __launch_bounds__(256) ln_colvec_kernel(const uint16_t* __restrict__ W, int ldw,
                                                        const uint16_t* __restrict__ gamma,
                                                        const uint16_t* __restrict__ beta, int K, int N,
                                                        float* __restrict__ cvec, float* __restrict__ bvec) {
  __shared__ float shc[CV_SLICES][CV_COLS], shb[CV_SLICES][CV_COLS];
  const int c = (int)threadIdx.x % CV_LANES, sl = (int)threadIdx.x / CV_LANES;
  const int j0 = blockIdx.x * CV_COLS + 8 * c;
  float ac[8], ab[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) ac[e] = ab[e] = 0.0f;
  if (j0 < N) {
    for (int k = sl; k < K; k += CV_SLICES) {
      float w[8];
      unpack8(ld16(W + (size_t)k * ldw + j0), w);
      const float gk = __uint_as_float((uint32_t)gamma[k] << 16);
      const float bk = beta ? __uint_as_float((uint32_t)beta[k] << 16) : 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ac[e] = fmaf(gk, w[e], ac[e]);
        ab[e] = fmaf(bk, w[e], ab[e]);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    shc[sl][8 * c + e] = ac[e];
    shb[sl][8 * c + e] = ab[e];
  }
  __syncthreads();
  if (sl == 0 && j0 < N) {
    float tc[8], tb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      tc[e] = 0.0f;
      tb[e] = 0.0f;
#pragma unroll
      for (int q = 0; q < CV_SLICES; ++q) {
        tc[e] += shc[q][8 * c + e];
        tb[e] += shb[q][8 * c + e];
      }
    }
    *reinterpret_cast<f32x4*>(cvec + j0) = (f32x4){tc[0], tc[1], tc[2], tc[3]};
    *reinterpret_cast<f32x4*>(cvec + j0 + 4) = (f32x4){tc[4], tc[5], tc[6], tc[7]};
    if (bvec) {
      *reinterpret_cast<f32x4*>(bvec + j0) = (f32x4){tb[0], tb[1], tb[2], tb[3]};
      *reinterpret_cast<f32x4*>(bvec + j0 + 4) = (f32x4){tb[4], tb[5], tb[6], tb[7]};
    }
  }
}

}  // namespace

extern "C" {

coda_status coda_gemm_res_lnstats(const coda_bf16* X, int ldx, const coda_bf16* W, int ldw, const coda_bf16* Z,
                                  int ldz, const coda_bf16* gamma, coda_bf16* U, int ldu, coda_bf16* H2,
                                  int ldh, float* pmean, float* pm2, int M, int N, int K, hipStream_t stream) {
  trace("coda_gemm_res_lnstats", "M=%d N=%d K=%d Z=%d H2=%d", M, N, K, Z != nullptr, H2 != nullptr);
  Check c;
  c.shape(M >= 0 && N >= 0 && K >= 0);
  c.bmat(X, ldx, K, M);
  c.bmat(W, ldw, N, K);
  c.bmat(Z, ldz, N, M, false);
  c.bmat(U, ldu, N, M);
  c.bmat(H2, ldh, N, M, false);
  if (H2) c.vec(gamma, N, 2, true, true);
  c.vec(pmean, (long long)M * coda_nparts(N), 4);
  c.vec(pm2, (long long)M * coda_nparts(N), 4);
  c.shape(N % 8 == 0 && K % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || N == 0) return CODA_OK;
  if (coda_status s = c.device()) return s;
  const int np = coda_nparts(N);
#define CODA_LS(HZ, HH)                                                                  \
  {                                                                                      \
    EpiResSumsq<HZ, HH, true, true> e{Z, ldz, gamma, U, ldu, H2, ldh, pmean, np, pm2};   \
    return launch_gemm<false, true>(W, ldw, X, ldx, N, M, K, e, stream);                 \
  }
  const bool hz = Z != nullptr, hh = H2 != nullptr;
  if (hz && hh) CODA_LS(true, true)
  if (hz && !hh) CODA_LS(true, false)
  if (!hz && hh) CODA_LS(false, true)
  CODA_LS(false, false)
#undef CODA_LS
}

coda_status coda_row_ln(const float* pmean, const float* pm2, int nparts, int M, int d, float eps, float* mu,
                        float* r, hipStream_t stream) {
  trace("coda_row_ln", "nparts=%d M=%d d=%d eps=%g", nparts, M, d, (double)eps);
  Check c;
  c.shape(M >= 0 && d >= 1 && eps >= 0.0f && nparts == coda_nparts(d));
  c.vec(pmean, (long long)M * nparts, 4);
  c.vec(pm2, (long long)M * nparts, 4);
  c.vec(mu, M, 4);
  c.vec(r, M, 4);
  if (c.st != CODA_OK) return c.st;
  if (M == 0) return CODA_OK;
  if (coda_status s = c.device()) return s;
  switch (lanes_per_row(nparts)) {
    case 4:
      hipLaunchKernelGGL(row_ln_kernel<4>, dim3(cdiv(M, 64)), dim3(256), 0, stream, pmean, pm2, nparts, M, d, eps,
                         mu, r);
      break;
    case 16:
      hipLaunchKernelGGL(row_ln_kernel<16>, dim3(cdiv(M, 16)), dim3(256), 0, stream, pmean, pm2, nparts, M, d, eps,
                         mu, r);
      break;
    default:
      hipLaunchKernelGGL(row_ln_kernel<64>, dim3(cdiv(M, 4)), dim3(256), 0, stream, pmean, pm2, nparts, M, d, eps,
                         mu, r);
  }
  return launched();
}

coda_status coda_ln_colvec(const coda_bf16* W, int ldw, const coda_bf16* gamma, const coda_bf16* beta, int K,
                           int N, float* cvec, float* bvec, hipStream_t stream) {
  trace("coda_ln_colvec", "K=%d N=%d beta=%d", K, N, beta != nullptr);
  Check c;
  c.shape(K >= 0 && N >= 0 && N % 8 == 0);
  c.bmat(W, ldw, N, K);
  c.vec(gamma, K, 2);
  c.vec(beta, K, 2, false);
  c.vec(cvec, N, 4, true, true);
  c.vec(bvec, N, 4, beta != nullptr, true);
  if (c.st == CODA_OK && (beta == nullptr) != (bvec == nullptr)) c.st = CODA_ERR_NULL;
  if (c.st != CODA_OK) return c.st;
  if (N == 0) return CODA_OK;
  if (coda_status s = c.device()) return s;
  hipLaunchKernelGGL(ln_colvec_kernel, dim3(cdiv(N, CV_COLS)), dim3(256), 0, stream, W, ldw, gamma, beta, K, N,
                     cvec, bvec);
  return launched();
}

coda_status coda_gemm_ln_rowscale(const coda_bf16* A, int lda, const coda_bf16* W, int ldw, const float* r,
                                  const float* mu, const float* cvec, const float* bvec, coda_bf16* Y, int ldy,
                                  int M, int N, int K, hipStream_t stream) {
  trace("coda_gemm_ln_rowscale", "M=%d N=%d K=%d beta=%d", M, N, K, bvec != nullptr);
  Check c;
  c.shape(M >= 0 && N >= 0 && K >= 0);
  c.bmat(A, lda, K, M);
  c.bmat(W, ldw, N, K);
  c.vec(r, M, 4);
  c.vec(mu, M, 4);
  c.vec(cvec, N, 4, true, true);
  c.vec(bvec, N, 4, false, true);
  c.bmat(Y, ldy, N, M);
  c.shape(N % 8 == 0 && K % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || N == 0) return CODA_OK;
  if (coda_status s = c.device()) return s;
  EpiLinear<true, false, true> e{r, nullptr, 0, Y, ldy, mu, cvec, bvec};
  return launch_gemm<false, true>(W, ldw, A, lda, N, M, K, e, stream);
}

coda_status coda_gemm_ln_swiglu(const coda_bf16* A, int lda, const coda_bf16* Wgu, int ldw, const float* r,
                                const float* mu, const float* cvec, const float* bvec, coda_bf16* Act, int ldact,
                                coda_bf16* Pre, int ldp, int M, int F, int K, hipStream_t stream) {
  trace("coda_gemm_ln_swiglu", "M=%d F=%d K=%d Pre=%d beta=%d", M, F, K, Pre != nullptr, bvec != nullptr);
  Check c;
  c.shape(M >= 0 && F >= 0 && K >= 0 && F <= (1 << 29));
  if (c.st != CODA_OK) return c.st;
  c.bmat(A, lda, K, M);
  c.bmat(Wgu, ldw, 2 * F, K);
  c.vec(r, M, 4);
  c.vec(mu, M, 4);
  c.vec(cvec, 2LL * F, 4, true, true);
  c.vec(bvec, 2LL * F, 4, false, true);
  c.mat(Act, ldact, F, M, true, 2, 4);
  c.bmat(Pre, ldp, 2 * F, M, false);
  c.shape(F % 4 == 0 && K % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || F == 0) return CODA_OK;
  if (coda_status s = c.device()) return s;
  if (Pre) {
    EpiSwiglu<true, true, true> e{r, Act, ldact, Pre, ldp, mu, cvec, bvec};
    return launch_gemm<false, true>(Wgu, ldw, A, lda, 2 * F, M, K, e, stream);
  }
  EpiSwiglu<true, false, true> e{r, Act, ldact, nullptr, 0, mu, cvec, bvec};
  return launch_gemm<false, true>(Wgu, ldw, A, lda, 2 * F, M, K, e, stream);
}

coda_status coda_gemm_swiglu_bwd_ln(const coda_bf16* dOut, int ldd, const coda_bf16* Wd, int ldw,
                                    const coda_bf16* Pre, int ldp, coda_bf16* dPre, int lddp, const float* cvec,
                                    const float* bvec, float* spart, float* apart, int M, int F, int N,
                                    hipStream_t stream) {
  trace("coda_gemm_swiglu_bwd_ln", "M=%d F=%d N=%d beta=%d", M, F, N, bvec != nullptr);
  Check c;
  c.shape(M >= 0 && F >= 0 && N >= 0 && F <= (1 << 29));
  if (c.st != CODA_OK) return c.st;
  c.bmat(dOut, ldd, N, M);
  c.bmat(Wd, ldw, N, F);
  c.bmat(Pre, ldp, 2 * F, M);
  c.bmat(dPre, lddp, 2 * F, M);
  c.vec(cvec, 2LL * F, 4, true, true);
  c.vec(bvec, 2LL * F, 4, false, true);
  c.vec(spart, (long long)M * coda_nparts(F), 4);
  c.vec(apart, (long long)M * coda_nparts(F), 4);
  c.shape(F % 8 == 0 && N % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || F == 0) return CODA_OK;
  if (coda_status s = c.device()) return s;
  EpiSwigluBwd<true, true> e{Pre, ldp, dPre, lddp, spart, coda_nparts(F), cvec, bvec, apart};
  return launch_gemm<true, true>(Wd, ldw, dOut, ldd, F, M, N, e, stream);
}

coda_status coda_row_ln_bwd(const float* spart, const float* apart, int nparts, int M, int d, float* s, float* a,
                            hipStream_t stream) {
  trace("coda_row_ln_bwd", "nparts=%d M=%d d=%d", nparts, M, d);
  Check c;
  c.shape(M >= 0 && nparts >= 1 && d >= 1);
  c.vec(spart, (long long)M * nparts, 4);
  c.vec(apart, (long long)M * nparts, 4);
  c.vec(s, M, 4);
  c.vec(a, M, 4);
  if (c.st != CODA_OK) return c.st;
  if (M == 0) return CODA_OK;
  if (coda_status st = c.device()) return st;
  const float inv_d = 1.0f / (float)d;
  switch (lanes_per_row(nparts)) {
    case 4:
      hipLaunchKernelGGL(row_ln_bwd_kernel<4>, dim3(cdiv(M, 64)), dim3(256), 0, stream, spart, apart, nparts, M,
                         inv_d, s, a);
      break;
    case 16:
      hipLaunchKernelGGL(row_ln_bwd_kernel<16>, dim3(cdiv(M, 16)), dim3(256), 0, stream, spart, apart, nparts, M,
                         inv_d, s, a);
      break;
    default:
      hipLaunchKernelGGL(row_ln_bwd_kernel<64>, dim3(cdiv(M, 4)), dim3(256), 0, stream, spart, apart, nparts, M,
                         inv_d, s, a);
  }
  return launched();
}

coda_status coda_gemm_ln_bwd(const coda_bf16* dY, int ldd, const coda_bf16* W1, int ldw, const coda_bf16* U,
                             int ldu, const coda_bf16* gamma, const coda_bf16* beta, const float* r,
                             const float* mu, const float* s, const float* a, const coda_bf16* dRes, int ldr,
                             coda_bf16* dU, int lddu, coda_bf16* N2, int ldn, float* gpart, float* bgpart, int M,
                             int d, int N, hipStream_t stream) {
  trace("coda_gemm_ln_bwd", "M=%d d=%d N=%d dRes=%d N2=%d beta=%d", M, d, N, dRes != nullptr, N2 != nullptr,
        beta != nullptr);
  Check c;
  c.shape(M >= 0 && d >= 0 && N >= 0);
  c.bmat(dY, ldd, N, M);
  c.bmat(W1, ldw, N, d);
  c.bmat(U, ldu, d, M);
  c.vec(gamma, d, 2, true, true);
  c.vec(beta, d, 2, false, true);
  c.vec(r, M, 4);
  c.vec(mu, M, 4);
  c.vec(s, M, 4);
  c.vec(a, M, 4);
  c.bmat(dRes, ldr, d, M, false);
  c.bmat(dU, lddu, d, M);
  c.bmat(N2, ldn, d, M, false);
  c.vec(gpart, (long long)coda_mparts(M) * d, 4);
  c.vec(bgpart, (long long)coda_mparts(M) * d, 4);
  c.shape(d % 8 == 0 && N % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || d == 0) return CODA_OK;
  if (coda_status st = c.device()) return st;
#define CODA_LB(HR, HN)                                                                                    \
  {                                                                                                        \
    EpiRowscaleBwd<HR, HN, true, true> e{U, ldu, gamma, r, s, dRes, ldr, dU, lddu, N2, ldn, gpart, d, mu, a, \
                                         beta, bgpart};                                                    \
    return launch_gemm<true, true, 256>(W1, ldw, dY, ldd, d, M, N, e, stream);                             \
  }
  const bool hr = dRes != nullptr, hn = N2 != nullptr;
  if (hr && hn) CODA_LB(true, true)
  if (hr && !hn) CODA_LB(true, false)
  if (!hr && hn) CODA_LB(false, true)
  CODA_LB(false, false)
#undef CODA_LB
}

}  // extern "C"
