// coda_fwd.hip - the forward fused GEMM-epilogue calls of GEMM -> residual ->
// RMSNorm -> GEMM: the plain GEMM, GEMM1 (residual + sum-of-squares partials)
// and GEMM2 (the delayed row scale).
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

coda_status coda_gemm(const coda_bf16* X, int ldx, const coda_bf16* W, int ldw, coda_bf16* Y,
                      int ldy, int M, int N, int K, hipStream_t stream) {
  trace("coda_gemm", "M=%d N=%d K=%d", M, N, K);
  Check c;
  c.shape(M >= 0 && N >= 0 && K >= 0);
  c.bmat(X, ldx, K, M);
  c.bmat(W, ldw, N, K);
  c.bmat(Y, ldy, N, M);
  c.shape(N % 8 == 0 && K % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || N == 0) return CODA_OK;
  if (coda_status s = c.device()) return s;
  EpiLinear<false, false> e{nullptr, nullptr, 0, Y, ldy};
  return launch_gemm<false, true>(W, ldw, X, ldx, N, M, K, e, stream);
}

coda_status coda_gemm_res_sumsq(const coda_bf16* X, int ldx, const coda_bf16* W, int ldw,
                                const coda_bf16* Z, int ldz, const coda_bf16* gamma, coda_bf16* U,
                                int ldu, coda_bf16* H2, int ldh, float* part, int M, int N, int K,
                                hipStream_t stream) {
  trace("coda_gemm_res_sumsq", "M=%d N=%d K=%d Z=%d H2=%d part=%d", M, N, K, Z != nullptr, H2 != nullptr, part != nullptr);
  Check c;
  c.shape(M >= 0 && N >= 0 && K >= 0);
  c.bmat(X, ldx, K, M);
  c.bmat(W, ldw, N, K);
  c.bmat(Z, ldz, N, M, false);
  c.bmat(U, ldu, N, M);
  c.bmat(H2, ldh, N, M, false);
  if (H2) c.vec(gamma, N, 2, true, true);
  c.vec(part, (long long)M * coda_nparts(N), 4, false);
  c.shape(N % 8 == 0 && K % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || N == 0) return CODA_OK;
  if (coda_status s = c.device()) return s;
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

coda_status coda_gemm_rowscale(const coda_bf16* A, int lda, const coda_bf16* W, int ldw,
                               const float* r, coda_bf16* Y, int ldy, int M, int N, int K,
                               hipStream_t stream) {
  trace("coda_gemm_rowscale", "M=%d N=%d K=%d", M, N, K);
  Check c;
  c.shape(M >= 0 && N >= 0 && K >= 0);
  c.bmat(A, lda, K, M);
  c.bmat(W, ldw, N, K);
  c.vec(r, M, 4);
  c.bmat(Y, ldy, N, M);
  c.shape(N % 8 == 0 && K % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || N == 0) return CODA_OK;
  if (coda_status s = c.device()) return s;
  EpiLinear<true, false> e{r, nullptr, 0, Y, ldy};
  return launch_gemm<false, true>(W, ldw, A, lda, N, M, K, e, stream);
}

}  // extern "C"
