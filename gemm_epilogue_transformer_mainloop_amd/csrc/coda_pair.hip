// coda_pair.hip - the fused GEMM-epilogue calls with pairwise maps on
// register-resident adjacent outputs: RoPE (2 -> 2, and its inverse) and
// SwiGLU (2 -> 1).
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

static coda_status rope_common(const coda_bf16* A, int lda, const coda_bf16* W, int ldw,
                               const float* r, const int32_t* pos, float theta, int head_dim,
                               int n_rope, coda_bf16* Y, int ldy, int M, int N, int K, bool inv,
                               hipStream_t stream) {
  Check c;
  c.shape(M >= 0 && N >= 0 && K >= 0);
  c.bmat(A, lda, K, M);
  c.bmat(W, ldw, N, K);
  c.vec(r, M, 4, false);
  c.vec(pos, M, 4);
  c.bmat(Y, ldy, N, M);
  c.shape(N % 8 == 0 && K % 8 == 0);
  c.unsupported(head_dim >= 2 && head_dim % 2 == 0 && n_rope >= 0 && n_rope <= N &&
                n_rope % head_dim == 0 && n_rope % 8 == 0 && theta > 0.0f);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || N == 0) return CODA_OK;
  if (coda_status s = c.device()) return s;
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
  trace("coda_gemm_rope", "M=%d N=%d K=%d head_dim=%d n_rope=%d theta=%g r=%d", M, N, K, head_dim, n_rope, (double)theta, r != nullptr);
  return rope_common(A, lda, W, ldw, r, pos, theta, head_dim, n_rope, Y, ldy, M, N, K, false,
                     stream);
}

coda_status coda_gemm_rope_bwd(const coda_bf16* A, int lda, const coda_bf16* W, int ldw,
                               const float* r, const int32_t* pos, float theta, int head_dim,
                               int n_rope, coda_bf16* Y, int ldy, int M, int N, int K,
                               hipStream_t stream) {
  trace("coda_gemm_rope_bwd", "M=%d N=%d K=%d head_dim=%d n_rope=%d theta=%g r=%d", M, N, K, head_dim, n_rope, (double)theta, r != nullptr);
  return rope_common(A, lda, W, ldw, r, pos, theta, head_dim, n_rope, Y, ldy, M, N, K, true,
                     stream);
}

coda_status coda_gemm_swiglu(const coda_bf16* A, int lda, const coda_bf16* Wgu, int ldw,
                             const float* r, coda_bf16* Act, int ldact, coda_bf16* Pre, int ldp,
                             int M, int F, int K, hipStream_t stream) {
  trace("coda_gemm_swiglu", "M=%d F=%d K=%d r=%d Pre=%d", M, F, K, r != nullptr, Pre != nullptr);
  Check c;
  c.shape(M >= 0 && F >= 0 && K >= 0);
  c.shape(F <= (1 << 29));
  if (c.st != CODA_OK) return c.st;
  c.bmat(A, lda, K, M);
  c.bmat(Wgu, ldw, 2 * F, K);
  c.vec(r, M, 4, false);
  c.mat(Act, ldact, F, M, true, 2, 4);  // act rows may end on a half chunk: ld % 4
  c.bmat(Pre, ldp, 2 * F, M, false);
  c.shape(F % 4 == 0 && K % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || F == 0) return CODA_OK;
  if (coda_status s = c.device()) return s;
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

}  // extern "C"
