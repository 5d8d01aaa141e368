// coda_probe.hip - the matrix-core clock probe of include/coda_probe.h.
//
// Each wave runs eight independent accumulation chains of the 32x32x16 bf16
// MFMA (one issue every 8 passes per SIMD; eight chains keep each
// accumulator's previous result ready before it is needed again), between two
// readings of the shader-clock and reference-clock counters.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/coda_probe.h"
#include "coda_host.hpp"
#include "coda_mainloop.hpp"

using namespace coda;
using namespace coda_host;

namespace {

constexpr int PROBE_LDS = 96 * 1024;  // over half of the 160 KiB: one workgroup per CU

__global__ void __launch_bounds__(256) mfma_probe_kernel(int iters, unsigned long long* __restrict__ out) {
  __shared__ char lds[PROBE_LDS];
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)(float)((lane + e) & 7);
    b[e] = (__bf16)(float)((lane * 3 + e) & 7);
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = (f32x16){};
  lds[threadIdx.x] = (char)(lane & 7);  // the workgroup owns its LDS allocation
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0];
  s += (float)lds[(threadIdx.x + 64) & 255];
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = t1 - t0;
    // s is a sum of products of small integers: never negative.  The
    // comparison keeps the MFMA results live.
    out[2 * blockIdx.x + 1] = (s < 0.0f) ? 0ull : (r1 - r0);
  }
}

}  // namespace

extern "C" {

coda_status coda_probe_mfma(int blocks, int iters, unsigned long long* out, hipStream_t stream) {
  trace("coda_probe_mfma", "blocks=%d iters=%d", blocks, iters);
  Check c;
  c.shape(blocks >= 1 && blocks <= 65536 && iters >= 1 && iters <= 1000000);
  c.vec(out, 2LL * blocks, 8);
  if (c.st != CODA_OK) return c.st;
  if (coda_status s = c.device()) return s;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, stream, iters, out);
  return launched();
}

coda_status coda_timeline_set(unsigned long long* buf, int waves) {
  trace("coda_timeline_set", "buf=%p waves=%d", (void*)buf, waves);
  if (!coda::kTimeline) return CODA_ERR_UNSUPPORTED;
  if (waves < 0 || (buf == nullptr && waves > 0)) return CODA_ERR_SHAPE;
  if (buf != nullptr && (reinterpret_cast<uintptr_t>(buf) & 7u) != 0) return CODA_ERR_ALIGN;
  std::lock_guard<std::mutex> lock(g_tl_mu);
  g_tl_buf = waves > 0 ? buf : nullptr;
  g_tl_waves = waves > 0 ? waves : 0;
  return CODA_OK;
}

int coda_timeline_words(void) { return coda::TL_WORDS; }

}  // extern "C"
