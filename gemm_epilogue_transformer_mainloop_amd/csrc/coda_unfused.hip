// coda_unfused.hip - the unfused baseline (include/coda_unfused.h): standalone
// bandwidth kernels that, behind the plain GEMMs, form the conventional
// sequence the fused GEMM-epilogue calls replace ("CODA: Rewriting Transformer
// Blocks as GEMM-Epilogue Programs", abstract and Figure 1).
//
// Every kernel moves 16-byte vectors (8 bf16) per thread access, computes in
// fp32 and rounds bf16 outputs to nearest-even.  Row reductions use one
// workgroup of 256 threads per row with a fixed-order tree, so results are
// deterministic.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "../../include/coda_unfused.h"
#include "coda_host.hpp"
#include "coda_mainloop.hpp"

using namespace coda;
using namespace coda_host;

namespace {

constexpr int RT = 256;          // threads per row workgroup
constexpr int MAX_CHUNKS = 4;    // 16-byte chunks per thread in the row kernels: d <= 8192
constexpr int BWD_ROWS = 16;     // rows per dgamma partial of the RMSNorm backward

// Sum of v over the 256 threads of the workgroup; every thread gets the result.
__device__ __forceinline__ float block_sum(float v, float* sh) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6;
  __syncthreads();  // sh may still be read by a previous call
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  return (sh[0] + sh[1]) + (sh[2] + sh[3]);
}

__host__ __device__ inline long long nchunks(int M, int N) { return (long long)M * (N / 8); }
inline int grid_for(long long n) {
  const long long b = (n + RT - 1) / RT;
  return (int)(b < (1 << 30) ? b : (1 << 30));
}

// ---------------------------------------------------------------------------
// Residual add
// ---------------------------------------------------------------------------
// C may alias A or B (same element, read before written): no __restrict__.
__global__ void __launch_bounds__(RT) add_kernel(const uint16_t* A, int lda, const uint16_t* B, int ldb,
                                                 uint16_t* C, int ldc, int M, int N) {
  const long long n = nchunks(M, N), per = N / 8;
  for (long long i = (long long)blockIdx.x * RT + threadIdx.x; i < n; i += (long long)gridDim.x * RT) {
    const int row = (int)(i / per), c = (int)(i % per) * 8;
    float a[8], b[8];
    unpack8(ld16(A + (size_t)row * lda + c), a);
    unpack8(ld16(B + (size_t)row * ldb + c), b);
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] += b[e];
    st16(C + (size_t)row * ldc + c, pack8(a));
  }
}

// ---------------------------------------------------------------------------
// Residual add + RMSNorm (one row per workgroup)
// ---------------------------------------------------------------------------
// U may alias Y (each chunk is read before it is written, by the same thread).
__global__ void __launch_bounds__(RT) add_rmsnorm_kernel(const uint16_t* Y, int ldy,
                                                         const uint16_t* __restrict__ Z, int ldz,
                                                         const uint16_t* __restrict__ gamma, float eps,
                                                         uint16_t* U, int ldu,
                                                         uint16_t* __restrict__ N2, int ldn,
                                                         float* __restrict__ r, int d) {
  __shared__ float sh[4];
  const int row = blockIdx.x, nc = d / 8;
  u32x4 uc[MAX_CHUNKS];
  float ss = 0.0f;
#pragma unroll
  for (int k = 0; k < MAX_CHUNKS; ++k) {
    const int c = threadIdx.x + k * RT;
    if (c < nc) {
      float y[8];
      unpack8(ld16(Y + (size_t)row * ldy + c * 8), y);
      if (Z) {
        float z[8];
        unpack8(ld16(Z + (size_t)row * ldz + c * 8), z);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] += z[e];
      }
      uc[k] = pack8(y);
      float u[8];
      unpack8(uc[k], u);  // the statistic is taken over the stored bf16 residual stream
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += u[e] * u[e];
      st16(U + (size_t)row * ldu + c * 8, uc[k]);
    }
  }
  const float tot = block_sum(ss, sh);
  const float ri = 1.0f / sqrtf(tot / (float)d + eps);
  if (threadIdx.x == 0) r[row] = ri;
#pragma unroll
  for (int k = 0; k < MAX_CHUNKS; ++k) {
    const int c = threadIdx.x + k * RT;
    if (c < nc) {
      float u[8], g[8];
      unpack8(uc[k], u);
      unpack8(ld16(gamma + c * 8), g);
#pragma unroll
      for (int e = 0; e < 8; ++e) u[e] = (ri * u[e]) * g[e];
      st16(N2 + (size_t)row * ldn + c * 8, pack8(u));
    }
  }
}

// ---------------------------------------------------------------------------
// RoPE (in place)
// ---------------------------------------------------------------------------
// One thread per 8-column chunk of the rotated range and group of rows: the
// chunk's four frequencies are computed once and reused down the rows.  The
// angle is reduced to revolutions and rotated with the hardware sine/cosine,
// as in the fused epilogue.
constexpr int ROPE_RC = 64, ROPE_RR = RT / ROPE_RC;  // chunks x rows per block
__global__ void __launch_bounds__(RT) rope_kernel(uint16_t* __restrict__ Y, int ldy, const int32_t* __restrict__ pos,
                                                  float log2_theta, int head_dim, int n_rope, float sgn, int M) {
  const int c0 = (blockIdx.x * ROPE_RC + (int)threadIdx.x % ROPE_RC) * 8;
  if (c0 >= n_rope) return;
  constexpr float INV_2PI = 0.15915494309189535f;
  const float c_exp = log2_theta / (float)head_dim;
  const int base = c0 % head_dim;
  float fr[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    int j = base + 2 * q;  // (c0 + 2q) mod head_dim: head_dim >= 2 wraps at most three times
    j -= j >= head_dim ? head_dim : 0;
    j -= j >= head_dim ? head_dim : 0;
    j -= j >= head_dim ? head_dim : 0;
    fr[q] = exp2f(-(float)j * c_exp) * INV_2PI;
  }
  for (int row = blockIdx.y * ROPE_RR + (int)threadIdx.x / ROPE_RC; row < M; row += gridDim.y * ROPE_RR) {
    uint16_t* p = Y + (size_t)row * ldy + c0;
    float v[8];
    unpack8(ld16(p), v);
    const float ps = (float)pos[row];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (c0 + 2 * q >= n_rope) break;
      float rev = ps * fr[q];
      rev -= floorf(rev);
      const float sn = sgn * __builtin_amdgcn_sinf(rev), cs = __builtin_amdgcn_cosf(rev);
      const float a = v[2 * q], b = v[2 * q + 1];
      v[2 * q] = a * cs - b * sn;
      v[2 * q + 1] = a * sn + b * cs;
    }
    st16(p, pack8(v));
  }
}

// ---------------------------------------------------------------------------
// SwiGLU forward / backward
// ---------------------------------------------------------------------------
__device__ __forceinline__ float sigm(float x) { return 1.0f / (1.0f + expf(-x)); }

__global__ void __launch_bounds__(RT) swiglu_kernel(const uint16_t* __restrict__ Pre, int ldp,
                                                    uint16_t* __restrict__ Act, int lda, int M, int F) {
  const long long n = nchunks(M, F), per = F / 8;
  for (long long i = (long long)blockIdx.x * RT + threadIdx.x; i < n; i += (long long)gridDim.x * RT) {
    const int row = (int)(i / per), j0 = (int)(i % per) * 8;
    float p0[8], p1[8], a[8];
    unpack8(ld16(Pre + (size_t)row * ldp + 2 * j0), p0);
    unpack8(ld16(Pre + (size_t)row * ldp + 2 * j0 + 8), p1);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      a[q] = p0[2 * q] * sigm(p0[2 * q]) * p0[2 * q + 1];
      a[4 + q] = p1[2 * q] * sigm(p1[2 * q]) * p1[2 * q + 1];
    }
    st16(Act + (size_t)row * lda + j0, pack8(a));
  }
}

__global__ void __launch_bounds__(RT) swiglu_bwd_kernel(const uint16_t* __restrict__ dA, int ldda,
                                                        const uint16_t* __restrict__ Pre, int ldp,
                                                        uint16_t* __restrict__ dPre, int lddp, int M, int F) {
  const long long n = nchunks(M, F), per = F / 8;
  for (long long i = (long long)blockIdx.x * RT + threadIdx.x; i < n; i += (long long)gridDim.x * RT) {
    const int row = (int)(i / per), j0 = (int)(i % per) * 8;
    float da[8], p[2][8], o[2][8];
    unpack8(ld16(dA + (size_t)row * ldda + j0), da);
    unpack8(ld16(Pre + (size_t)row * ldp + 2 * j0), p[0]);
    unpack8(ld16(Pre + (size_t)row * ldp + 2 * j0 + 8), p[1]);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float g = p[h][2 * q], v = p[h][2 * q + 1], d = da[4 * h + q];
        const float s = sigm(g);
        o[h][2 * q] = d * v * s * (1.0f + g * (1.0f - s));
        o[h][2 * q + 1] = d * g * s;
      }
    st16(dPre + (size_t)row * lddp + 2 * j0, pack8(o[0]));
    st16(dPre + (size_t)row * lddp + 2 * j0 + 8, pack8(o[1]));
  }
}

// ---------------------------------------------------------------------------
// RMSNorm backward (canonical form), BWD_ROWS rows per workgroup
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(RT) rmsnorm_bwd_kernel(const uint16_t* __restrict__ G, int ldg,
                                                         const uint16_t* __restrict__ U, int ldu,
                                                         const uint16_t* __restrict__ gamma,
                                                         const float* __restrict__ r,
                                                         const uint16_t* __restrict__ dRes, int ldr,
                                                         uint16_t* __restrict__ dU, int lddu,
                                                         float* __restrict__ gpart, int M, int d) {
  __shared__ float sh[4];
  const int nc = d / 8, q = blockIdx.x;
  float gm[MAX_CHUNKS][8], dg[MAX_CHUNKS][8];
#pragma unroll
  for (int k = 0; k < MAX_CHUNKS; ++k) {
    const int c = threadIdx.x + k * RT;
#pragma unroll
    for (int e = 0; e < 8; ++e) dg[k][e] = 0.0f;
    if (c < nc) unpack8(ld16(gamma + c * 8), gm[k]);
  }
  for (int ii = 0; ii < BWD_ROWS; ++ii) {
    const int row = q * BWD_ROWS + ii;
    if (row >= M) break;  // uniform over the workgroup
    const float ri = r[row];
    float gv[MAX_CHUNKS][8], uv[MAX_CHUNKS][8];
    float cs = 0.0f;
#pragma unroll
    for (int k = 0; k < MAX_CHUNKS; ++k) {
      const int c = threadIdx.x + k * RT;
      if (c < nc) {
        unpack8(ld16(G + (size_t)row * ldg + c * 8), gv[k]);
        unpack8(ld16(U + (size_t)row * ldu + c * 8), uv[k]);
#pragma unroll
        for (int e = 0; e < 8; ++e) cs += gv[k][e] * gm[k][e] * uv[k][e];
      }
    }
    const float ci = block_sum(cs, sh);
    const float c3 = ri * ri * ri * ci / (float)d;
#pragma unroll
    for (int k = 0; k < MAX_CHUNKS; ++k) {
      const int c = threadIdx.x + k * RT;
      if (c < nc) {
        float o[8];
        if (dRes) {
          unpack8(ld16(dRes + (size_t)row * ldr + c * 8), o);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          o[e] += ri * (gv[k][e] * gm[k][e]) - c3 * uv[k][e];
          dg[k][e] += gv[k][e] * (ri * uv[k][e]);
        }
        st16(dU + (size_t)row * lddu + c * 8, pack8(o));
      }
    }
  }
  if (gpart) {
#pragma unroll
    for (int k = 0; k < MAX_CHUNKS; ++k) {
      const int c = threadIdx.x + k * RT;
      if (c < nc) {
        float* o = gpart + (size_t)q * d + c * 8;
        *reinterpret_cast<f32x4*>(o) = (f32x4){dg[k][0], dg[k][1], dg[k][2], dg[k][3]};
        *reinterpret_cast<f32x4*>(o + 4) = (f32x4){dg[k][4], dg[k][5], dg[k][6], dg[k][7]};
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Cross-entropy over materialised logits (one row per workgroup)
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(RT) ce_kernel(const uint16_t* __restrict__ L, int ldl,
                                                const int32_t* __restrict__ labels, float* __restrict__ lse,
                                                float* __restrict__ loss, int V) {
  __shared__ float shm[RT], shs[RT], sht[1];
  const int row = blockIdx.x, nc = V / 8;
  const int y = labels[row];
  float m = -INFINITY, s = 0.0f;
  for (int c = threadIdx.x; c < nc; c += RT) {
    float v[8];
    unpack8(ld16(L + (size_t)row * ldl + c * 8), v);
    float cm = v[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cm = fmaxf(cm, v[e]);
    const float nm = fmaxf(m, cm);
    float cs = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) cs += expf(v[e] - nm);
    s = s * expf(m - nm) + cs;  // exp(-inf) = 0 on the first chunk
    m = nm;
    if (y >= c * 8 && y < c * 8 + 8) sht[0] = v[y - c * 8];
  }
  shm[threadIdx.x] = m;
  shs[threadIdx.x] = s;
  __syncthreads();
  for (int w = RT / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      const float m1 = shm[threadIdx.x], m2 = shm[threadIdx.x + w];
      const float mm = fmaxf(m1, m2);
      const float s1 = m1 == -INFINITY ? 0.0f : shs[threadIdx.x] * expf(m1 - mm);
      const float s2 = m2 == -INFINITY ? 0.0f : shs[threadIdx.x + w] * expf(m2 - mm);
      shm[threadIdx.x] = mm;
      shs[threadIdx.x] = s1 + s2;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const float l = shm[0] + logf(shs[0]);
    lse[row] = l;
    loss[row] = (y >= 0 && y < V) ? l - sht[0] : __builtin_nanf("");
  }
}

__global__ void __launch_bounds__(1024) mean_kernel(const float* __restrict__ x, int M, float* __restrict__ out) {
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

// D may alias L (same element, read before written): no __restrict__ on them.
__global__ void __launch_bounds__(RT) ce_bwd_kernel(const uint16_t* L, int ldl,
                                                    const int32_t* __restrict__ labels,
                                                    const float* __restrict__ lse, float scale,
                                                    uint16_t* D, int ldd, int M, int V) {
  const long long n = nchunks(M, V), per = V / 8;
  for (long long i = (long long)blockIdx.x * RT + threadIdx.x; i < n; i += (long long)gridDim.x * RT) {
    const int row = (int)(i / per), c0 = (int)(i % per) * 8;
    float v[8];
    unpack8(ld16(L + (size_t)row * ldl + c0), v);
    const float l = lse[row];
    const int y = labels[row];
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (expf(v[e] - l) - (c0 + e == y ? 1.0f : 0.0f)) * scale;
    st16(D + (size_t)row * ldd + c0, pack8(v));
  }
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================

extern "C" {

coda_status coda_unfused_add(const coda_bf16* A, int lda, const coda_bf16* B, int ldb, coda_bf16* C, int ldc,
                             int M, int N, hipStream_t stream) {
  trace("coda_unfused_add", "M=%d N=%d", M, N);
  Check c;
  c.shape(M >= 0 && N >= 0 && N % 8 == 0);
  c.bmat(A, lda, N, M);
  c.bmat(B, ldb, N, M);
  c.bmat(C, ldc, N, M);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || N == 0) return CODA_OK;
  if (coda_status s = c.device()) return s;
  hipLaunchKernelGGL(add_kernel, dim3(grid_for(nchunks(M, N))), dim3(RT), 0, stream, A, lda, B, ldb, C, ldc, M, N);
  return launched();
}

coda_status coda_unfused_add_rmsnorm(const coda_bf16* Y, int ldy, const coda_bf16* Z, int ldz,
                                     const coda_bf16* gamma, float eps, coda_bf16* U, int ldu, coda_bf16* N2,
                                     int ldn, float* r, int M, int d, hipStream_t stream) {
  trace("coda_unfused_add_rmsnorm", "M=%d d=%d", M, d);
  Check c;
  c.shape(M >= 0 && d >= 8 && d % 8 == 0);
  c.unsupported(d <= MAX_CHUNKS * RT * 8);
  c.bmat(Y, ldy, d, M);
  c.bmat(Z, ldz, d, M, false);
  c.vec(gamma, d, 2, true, true);
  c.bmat(U, ldu, d, M);
  c.bmat(N2, ldn, d, M);
  c.vec(r, M, 4);
  c.shape(eps >= 0.0f);
  if (c.st != CODA_OK) return c.st;
  if (M == 0) return CODA_OK;
  if (coda_status s = c.device()) return s;
  hipLaunchKernelGGL(add_rmsnorm_kernel, dim3(M), dim3(RT), 0, stream, Y, ldy, Z, ldz, gamma, eps, U, ldu, N2,
                     ldn, r, d);
  return launched();
}

coda_status coda_unfused_rope(coda_bf16* Y, int ldy, const int32_t* pos, float theta, int head_dim, int n_rope,
                              int inverse, int M, int N, hipStream_t stream) {
  trace("coda_unfused_rope", "M=%d N=%d head_dim=%d n_rope=%d", M, N, head_dim, n_rope);
  Check c;
  c.shape(M >= 0 && N >= 0 && N % 8 == 0);
  c.bmat(Y, ldy, N, M);
  c.vec(pos, M, 4);
  c.unsupported(head_dim >= 2 && head_dim % 2 == 0 && n_rope >= 0 && n_rope <= N && n_rope % head_dim == 0);
  c.shape(theta > 0.0f);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || N == 0 || n_rope == 0) return CODA_OK;
  if (coda_status s = c.device()) return s;
  const int chunks = (n_rope + 7) / 8;
  const int gx = (chunks + ROPE_RC - 1) / ROPE_RC;
  const int gy = std::min((M + ROPE_RR - 1) / ROPE_RR, 16384);
  hipLaunchKernelGGL(rope_kernel, dim3(gx, gy), dim3(RT), 0, stream, Y, ldy, pos, log2f(theta), head_dim, n_rope,
                     inverse ? -1.0f : 1.0f, M);
  return launched();
}

coda_status coda_unfused_swiglu(const coda_bf16* Pre, int ldp, coda_bf16* Act, int lda, int M, int F,
                                hipStream_t stream) {
  trace("coda_unfused_swiglu", "M=%d F=%d", M, F);
  Check c;
  c.shape(M >= 0 && F >= 0 && F % 8 == 0 && F <= (1 << 29));
  c.bmat(Pre, ldp, 2 * F, M);
  c.bmat(Act, lda, F, M);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || F == 0) return CODA_OK;
  if (coda_status s = c.device()) return s;
  hipLaunchKernelGGL(swiglu_kernel, dim3(grid_for(nchunks(M, F))), dim3(RT), 0, stream, Pre, ldp, Act, lda, M, F);
  return launched();
}

coda_status coda_unfused_swiglu_bwd(const coda_bf16* dA, int ldda, const coda_bf16* Pre, int ldp, coda_bf16* dPre,
                                    int lddp, int M, int F, hipStream_t stream) {
  trace("coda_unfused_swiglu_bwd", "M=%d F=%d", M, F);
  Check c;
  c.shape(M >= 0 && F >= 0 && F % 8 == 0 && F <= (1 << 29));
  c.bmat(dA, ldda, F, M);
  c.bmat(Pre, ldp, 2 * F, M);
  c.bmat(dPre, lddp, 2 * F, M);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || F == 0) return CODA_OK;
  if (coda_status s = c.device()) return s;
  hipLaunchKernelGGL(swiglu_bwd_kernel, dim3(grid_for(nchunks(M, F))), dim3(RT), 0, stream, dA, ldda, Pre, ldp,
                     dPre, lddp, M, F);
  return launched();
}

int coda_unfused_rmsnorm_bwd_parts(int M) { return M <= 0 ? 0 : cdiv(M, BWD_ROWS); }

coda_status coda_unfused_rmsnorm_bwd(const coda_bf16* G, int ldg, const coda_bf16* U, int ldu,
                                     const coda_bf16* gamma, const float* r, const coda_bf16* dRes, int ldr,
                                     coda_bf16* dU, int lddu, float* gpart, int M, int d, hipStream_t stream) {
  trace("coda_unfused_rmsnorm_bwd", "M=%d d=%d", M, d);
  Check c;
  c.shape(M >= 0 && d >= 8 && d % 8 == 0);
  c.unsupported(d <= MAX_CHUNKS * RT * 8);
  c.bmat(G, ldg, d, M);
  c.bmat(U, ldu, d, M);
  c.vec(gamma, d, 2, true, true);
  c.vec(r, M, 4);
  c.bmat(dRes, ldr, d, M, false);
  c.bmat(dU, lddu, d, M);
  c.vec(gpart, (long long)coda_unfused_rmsnorm_bwd_parts(M) * d, 4, false, true);
  if (c.st != CODA_OK) return c.st;
  if (M == 0) return CODA_OK;
  if (coda_status s = c.device()) return s;
  hipLaunchKernelGGL(rmsnorm_bwd_kernel, dim3(cdiv(M, BWD_ROWS)), dim3(RT), 0, stream, G, ldg, U, ldu, gamma, r,
                     dRes, ldr, dU, lddu, gpart, M, d);
  return launched();
}

coda_status coda_unfused_cross_entropy(const coda_bf16* L, int ldl, const int32_t* labels, float* lse,
                                       float* loss_row, float* loss_mean, int M, int V, hipStream_t stream) {
  trace("coda_unfused_cross_entropy", "M=%d V=%d", M, V);
  Check c;
  c.shape(M >= 0 && V >= 8 && V % 8 == 0);
  c.bmat(L, ldl, V, M);
  c.vec(labels, M, 4);
  c.vec(lse, M, 4);
  c.vec(loss_row, M, 4);
  if (c.st != CODA_OK) return c.st;
  if (M == 0) return CODA_OK;
  if (coda_status s = c.device()) return s;
  hipLaunchKernelGGL(ce_kernel, dim3(M), dim3(RT), 0, stream, L, ldl, labels, lse, loss_row, V);
  if (loss_mean) hipLaunchKernelGGL(mean_kernel, dim3(1), dim3(1024), 0, stream, loss_row, M, loss_mean);
  return launched();
}

coda_status coda_unfused_cross_entropy_bwd(const coda_bf16* L, int ldl, const int32_t* labels, const float* lse,
                                           float grad_scale, coda_bf16* D, int ldd, int M, int V,
                                           hipStream_t stream) {
  trace("coda_unfused_cross_entropy_bwd", "M=%d V=%d", M, V);
  Check c;
  c.shape(M >= 0 && V >= 8 && V % 8 == 0);
  c.bmat(L, ldl, V, M);
  c.vec(labels, M, 4);
  c.vec(lse, M, 4);
  c.bmat(D, ldd, V, M);
  if (c.st != CODA_OK) return c.st;
  if (M == 0) return CODA_OK;
  if (coda_status s = c.device()) return s;
  hipLaunchKernelGGL(ce_bwd_kernel, dim3(grid_for(nchunks(M, V))), dim3(RT), 0, stream, L, ldl, labels, lse,
                     grad_scale, D, ldd, M, V);
  return launched();
}

}  // extern "C"
