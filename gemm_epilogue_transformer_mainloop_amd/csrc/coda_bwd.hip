// coda_bwd.hip - the backward ("reverse fusion") GEMM-epilogue calls: the
// SwiGLU backward pair map with the s partials, the RMSNorm backward with the
// delayed statistic, the data gradient with residual and the weight gradient.
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

extern "C" {

// The SwiGLU backward call's arguments, checked; CODA_OK to launch (or the
// status to return, a no-op being CODA_OK with *empty set).
static coda_status check_swiglu_bwd(const coda_bf16* dOut, int ldd, const coda_bf16* Wd, int ldw,
                                    const coda_bf16* Pre, int ldp, coda_bf16* dPre, int lddp, float* spart,
                                    int M, int F, int N, bool* empty) {
  Check c;
  c.shape(M >= 0 && F >= 0 && N >= 0 && F <= (1 << 29));
  if (c.st != CODA_OK) return c.st;
  c.bmat(dOut, ldd, N, M);
  c.bmat(Wd, ldw, N, F);
  c.bmat(Pre, ldp, 2 * F, M);
  c.bmat(dPre, lddp, 2 * F, M);
  c.vec(spart, (long long)M * coda_nparts(F), 4, false);
  c.shape(F % 8 == 0 && N % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  *empty = M == 0 || F == 0;
  if (*empty) return CODA_OK;
  return c.device();
}

// da[M x F] = dOut[M x N] Wd^T: features = F (rows of Wd, K-major), tokens = M.
static coda_status launch_swiglu_bwd(const coda_bf16* dOut, int ldd, const coda_bf16* Wd, int ldw,
                                     const coda_bf16* Pre, int ldp, coda_bf16* dPre, int lddp, float* spart,
                                     int M, int F, int N, hipStream_t stream) {
  const int np = coda_nparts(F);
  if (spart) {
    EpiSwigluBwd<true> e{Pre, ldp, dPre, lddp, spart, np};
    return launch_gemm<true, true>(Wd, ldw, dOut, ldd, F, M, N, e, stream);
  }
  EpiSwigluBwd<false> e{Pre, ldp, dPre, lddp, nullptr, np};
  return launch_gemm<true, true>(Wd, ldw, dOut, ldd, F, M, N, e, stream);
}

coda_status coda_gemm_swiglu_bwd(const coda_bf16* dOut, int ldd, const coda_bf16* Wd, int ldw,
                                 const coda_bf16* Pre, int ldp, coda_bf16* dPre, int lddp,
                                 float* spart, int M, int F, int N, hipStream_t stream) {
  trace("coda_gemm_swiglu_bwd", "M=%d F=%d N=%d spart=%d", M, F, N, spart != nullptr);
  bool empty = false;
  if (coda_status s = check_swiglu_bwd(dOut, ldd, Wd, ldw, Pre, ldp, dPre, lddp, spart, M, F, N, &empty)) return s;
  if (empty) return CODA_OK;
  return launch_swiglu_bwd(dOut, ldd, Wd, ldw, Pre, ldp, dPre, lddp, spart, M, F, N, stream);
}

// Whether the byte ranges of two row-major bf16 matrices (rows x cols, leading
// dimension ld) intersect.
static bool bmat_overlap(const coda_bf16* a, int lda, int arows, int acols, const coda_bf16* b, int ldb, int brows,
                         int bcols) {
  if (arows <= 0 || acols <= 0 || brows <= 0 || bcols <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a, a1 = a0 + 2 * ((size_t)(arows - 1) * lda + acols);
  const uintptr_t b0 = (uintptr_t)b, b1 = b0 + 2 * ((size_t)(brows - 1) * ldb + bcols);
  return a0 < b1 && b0 < a1;
}

coda_status coda_gemm_swiglu_bwd_overlap(const coda_bf16* dOut, int ldd, const coda_bf16* Wd, int ldw,
                                         const coda_bf16* Pre, int ldp, coda_bf16* dPre, int lddp,
                                         float* spart, int M, int F, int N, hipStream_t stream) {
  trace("coda_gemm_swiglu_bwd_overlap", "M=%d F=%d N=%d spart=%d", M, F, N, spart != nullptr);
  // dPre holds da in fp32 before the inputs are all read: it must not share
  // a byte with them (checked here, since the result would be silently wrong).
  if (dPre && (bmat_overlap(dPre, lddp, M, 2 * F, Pre, ldp, M, 2 * F) ||
               bmat_overlap(dPre, lddp, M, 2 * F, dOut, ldd, M, N) ||
               bmat_overlap(dPre, lddp, M, 2 * F, Wd, ldw, F, N)))
    return CODA_ERR_SHAPE;
  bool empty = false;
  if (coda_status s = check_swiglu_bwd(dOut, ldd, Wd, ldw, Pre, ldp, dPre, lddp, spart, M, F, N, &empty)) return s;
  if (empty) return CODA_OK;
  const int units = coda_swiglu_bwd_units(M, F, N, device_cus());
  if (units == 0) return launch_swiglu_bwd(dOut, ldd, Wd, ldw, Pre, ldp, dPre, lddp, spart, M, F, N, stream);
  const Problem p = whole_problem(Wd, ldw, dOut, ldd, F, M, N, 256);
  const EpiSwigluBwdDump dump{dPre, lddp};
  const SwigluBwdCarryArgs ca{Pre, ldp, dPre, lddp, spart, coda_nparts(F), F, M};
  if (spart)
    return units == 1 ? launch_persistent<true, true, EpiSwigluBwdDump, SwigluBwdCarry<1, true>>(p, dump, ca, stream)
                      : launch_persistent<true, true, EpiSwigluBwdDump, SwigluBwdCarry<2, true>>(p, dump, ca, stream);
  return units == 1 ? launch_persistent<true, true, EpiSwigluBwdDump, SwigluBwdCarry<1, false>>(p, dump, ca, stream)
                    : launch_persistent<true, true, EpiSwigluBwdDump, SwigluBwdCarry<2, false>>(p, dump, ca, stream);
}

coda_status coda_gemm_rowscale_bwd(const coda_bf16* dY, int ldd, const coda_bf16* W1, int ldw,
                                   const coda_bf16* U, int ldu, const coda_bf16* gamma,
                                   const float* r, const float* s, const coda_bf16* dRes, int ldr,
                                   coda_bf16* dU, int lddu, coda_bf16* N2, int ldn, float* gpart,
                                   int M, int d, int N, hipStream_t stream) {
  trace("coda_gemm_rowscale_bwd", "M=%d d=%d N=%d dRes=%d N2=%d gpart=%d", M, d, N, dRes != nullptr, N2 != nullptr, gpart != nullptr);
  Check c;
  c.shape(M >= 0 && d >= 0 && N >= 0);
  c.bmat(dY, ldd, N, M);
  c.bmat(W1, ldw, N, d);
  c.bmat(U, ldu, d, M);
  c.vec(gamma, d, 2, true, true);
  c.vec(r, M, 4);
  c.vec(s, M, 4);
  c.bmat(dRes, ldr, d, M, false);
  c.bmat(dU, lddu, d, M);
  c.bmat(N2, ldn, d, M, false);
  c.vec(gpart, (long long)coda_mparts(M) * d, 4, false);
  c.shape(d % 8 == 0 && N % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || d == 0) return CODA_OK;
  if (coda_status st = c.device()) return st;
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

coda_status coda_gemm_wgrad(const coda_bf16* X, int ldx, const coda_bf16* dY, int ldd, float* dW,
                            int lddw, int M, int K, int N, int accumulate, hipStream_t stream) {
  trace("coda_gemm_wgrad", "M=%d K=%d N=%d accumulate=%d", M, K, N, accumulate);
  Check c;
  c.shape(M >= 0 && K >= 0 && N >= 0);
  c.bmat(X, ldx, K, M);
  c.bmat(dY, ldd, N, M);
  c.fmat(dW, lddw, N, K);
  c.shape(K % 8 == 0 && N % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (K == 0 || N == 0) return CODA_OK;
  if (coda_status st = c.device()) return st;
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
  trace("coda_gemm_res_sumsq_bwd", "M=%d N=%d K=%d dRes=%d dW=%d", M, N, K, dRes != nullptr, dW != nullptr);
  Check c;
  c.shape(M >= 0 && N >= 0 && K >= 0);
  c.bmat(dU, ldu, N, M);
  c.bmat(W, ldw, N, K);
  c.bmat(dRes, ldr, K, M, false);
  c.bmat(dX, lddx, K, M);
  if (dW) {
    c.bmat(X, ldx, K, M);
    c.fmat(dW, lddw, N, K);
  }
  c.shape(N % 8 == 0 && K % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 && dW == nullptr) return CODA_OK;
  if (coda_status st = c.device()) return st;
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

}  // extern "C"
