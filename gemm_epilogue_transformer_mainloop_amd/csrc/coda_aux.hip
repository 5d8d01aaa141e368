// coda_aux.hip - the auxiliary reductions of the CODA path (row statistics
// from per-tile partials, dgamma column sums) and the host-only queries.
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

}  // namespace

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
    case CODA_ERR_BOUNDS: return "an argument's extent leaves its device allocation (CODA_DEBUG)";
  }
  return "unknown status";
}

const char* coda_version(void) { return "coda-gfx950 0.2"; }

coda_status coda_debug_extent(const void* p, size_t bytes) { return extent_ok(p, bytes); }

int coda_nparts(int N) { return N <= 0 ? 0 : cdiv(N, WAVE_F); }
int coda_mparts(int M) { return M <= 0 ? 0 : cdiv(M, WAVE_T); }
int coda_tile_split(int F, int T, int cus) {
  if (F <= 0 || T <= 0) return 0;
  return quantization_split(cdiv(F, 256), cdiv(T, 256), cdiv(T, 128), cus);
}
int coda_tile_split_tokens(int F, int T, int cus) {
  if (F <= 0 || T <= 0 || cus <= 0) return 0;
  const int nTF = cdiv(F, 256), nTT = cdiv(T, 256);
  if (coda_tile_split(F, T, cus) > 0) return 0;                    // the feature split applies
  if (2 * nTF * nTT <= cus && cdiv(T, 128) > nTT) return 0;        // all 256 x 128 tiles
  return token_split(nTF, nTT, T, cus);
}

int coda_swiglu_bwd_units(int M, int F, int N, int cus) {
  if (M <= 0 || F <= 0 || N <= 0 || cus < 8) return 0;
  const int nTF = cdiv(F, 256), nTT = cdiv(M, 256);
  if (coda_tile_split(F, M, cus) > 0 || coda_tile_split_tokens(F, M, cus) > 0) return 0;
  if (2 * nTF * nTT <= cus && cdiv(M, 128) > nTT) return 0;  // all 256 x 128 tiles
  if ((long long)nTF * nTT <= cus) return 0;                  // a single round: nothing to overlap
  const int nk = cdiv(N, 64);
  return nk >= 64 ? 1 : nk >= 32 ? 2 : 0;
}


coda_status coda_row_rms(const float* part, int nparts, int M, int d, float eps, float* r,
                         hipStream_t stream) {
  trace("coda_row_rms", "nparts=%d M=%d d=%d eps=%g", nparts, M, d, (double)eps);
  Check c;
  c.shape(M >= 0 && nparts >= 1 && d >= 1 && eps >= 0.0f);
  c.vec(part, (long long)M * nparts, 4);
  c.vec(r, M, 4);
  if (c.st != CODA_OK) return c.st;
  if (M == 0) return CODA_OK;
  if (coda_status s = c.device()) return s;
  launch_row_reduce<true>(part, nparts, M, 1.0f / (float)d, eps, r, stream);
  return launched();
}

coda_status coda_row_rms_bwd(const float* spart, int nparts, int M, int d, float* s,
                             hipStream_t stream) {
  trace("coda_row_rms_bwd", "nparts=%d M=%d d=%d", nparts, M, d);
  Check c;
  c.shape(M >= 0 && nparts >= 1 && d >= 1);
  c.vec(spart, (long long)M * nparts, 4);
  c.vec(s, M, 4);
  if (c.st != CODA_OK) return c.st;
  if (M == 0) return CODA_OK;
  if (coda_status st = c.device()) return st;
  launch_row_reduce<false>(spart, nparts, M, 1.0f / (float)d, 0.0f, s, stream);
  return launched();
}

coda_status coda_col_reduce(const float* gpart, int mparts, int d, float* dgamma,
                            hipStream_t stream) {
  trace("coda_col_reduce", "mparts=%d d=%d", mparts, d);
  Check c;
  c.shape(mparts >= 1 && d >= 0);
  c.vec(gpart, (long long)mparts * d, 4);
  c.vec(dgamma, d, 4);
  if (c.st != CODA_OK) return c.st;
  if (d == 0) return CODA_OK;
  if (coda_status st = c.device()) return st;
  hipLaunchKernelGGL(col_reduce_kernel, dim3(cdiv(d, CR_COLS)), dim3(256), 0, stream, gpart, mparts,
                     d, dgamma);
  return launched();
}

}  // extern "C"
