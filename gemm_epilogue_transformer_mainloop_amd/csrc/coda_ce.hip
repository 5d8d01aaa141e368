// coda_ce.hip - the LM-head cross-entropy calls: the fused statistics GEMM
// and its merge kernels, and the two backward forms.
//
// Every entry point validates its arguments before any HIP call, launches on
// the caller's stream and returns; nothing is allocated or synchronised.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/coda.h"
#include "coda_launch.hpp"

using namespace coda;
using namespace coda_host;
using namespace coda_launch;

// The allocation-free LM-head statistics call (coda_lmhead_ce_noalloc) keeps
// its partials workspace in this array: 64 MiB per device (one copy per GPU
// the library runs on, held until the process ends), enough for the
// coda_lmhead_ce workspace of M = 8192 tokens at a 128256-entry vocabulary
// (65.8 MB).  Host code never passes the array's name to a kernel: it uses the
// device address hipGetSymbolAddress returns for the current device.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

// Device address of `scratch` on the current device, looked up once per
// device (each GPU holds its own copy at its own address).
std::atomic<void*> g_scratch[64];

coda_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return CODA_ERR_HIP;
  if (dev < 0 || dev >= 64) return CODA_ERR_UNSUPPORTED;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
      (void)hipGetLastError();
      return CODA_ERR_HIP;
    }
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return CODA_OK;
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

// out = bf16(in) for an fp32 [M x N] matrix (N % 8 == 0), 8 elements per
// thread.
__global__ void __launch_bounds__(256) f32_to_bf16_kernel(const float* __restrict__ in, int ldi,
                                                          uint16_t* __restrict__ out, int ldo, int M, int N) {
  const long long per = N / 8, n = (long long)M * per;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) {
    const int row = (int)(i / per), c = (int)(i % per) * 8;
    const float* p = in + (size_t)row * ldi + c;
    const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
    const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    st16(out + (size_t)row * ldo + c, pack8(v));
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

}  // namespace

extern "C" {

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

static coda_status lmhead_ce_common(const coda_bf16* H, int ldh, const coda_bf16* W, int ldw,
                                    const int32_t* labels, float* lse, float* loss_row,
                                    float* loss_mean, coda_bf16* logits, int ldl, bool keep,
                                    void* ws, size_t ws_bytes, int M, int V, int d,
                                    hipStream_t stream, bool use_scratch = false) {
  Check c;
  c.shape(M >= 0 && V >= 0 && d >= 0);
  c.bmat(H, ldh, d, M);
  c.bmat(W, ldw, V, d);
  c.vec(labels, M, 4);
  c.vec(lse, M, 4);
  c.vec(loss_row, M, 4, false);
  c.vec(loss_mean, 1, 4, false);
  if (keep) c.bmat(logits, ldl, V, M);
  c.shape(V % 8 == 0 && d % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (M == 0 || V == 0) return CODA_OK;
  if (use_scratch) {
    if (coda_lmhead_ce_workspace(M, V) > kScratchBytes) return CODA_ERR_WORKSPACE;
    if (coda_status s = c.device()) return s;
    if (coda_status s = scratch_address(&ws)) return s;
    ws_bytes = kScratchBytes;
  } else {
    if (ws == nullptr || !al16(ws) || ws_bytes < coda_lmhead_ce_workspace(M, V))
      return CODA_ERR_WORKSPACE;
    if (coda_status s = c.device()) return s;
  }
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
  trace("coda_lmhead_ce", "M=%d V=%d d=%d ws_bytes=%zu", M, V, d, ws_bytes);
  return lmhead_ce_common(H, ldh, W, ldw, labels, lse, loss_row, loss_mean, nullptr, 0, false, ws,
                          ws_bytes, M, V, d, stream);
}

size_t coda_lmhead_ce_noalloc_max_bytes(void) { return kScratchBytes; }

coda_status coda_lmhead_ce_noalloc(const coda_bf16* H, int ldh, const coda_bf16* W, int ldw,
                                   const int32_t* labels, float* lse, float* loss_row, float* loss_mean,
                                   int M, int V, int d, hipStream_t stream) {
  trace("coda_lmhead_ce_noalloc", "M=%d V=%d d=%d", M, V, d);
  // Every partial, target and row-loss entry the merge kernel reads is written
  // earlier in the same call, so the array needs no clearing between calls.
  return lmhead_ce_common(H, ldh, W, ldw, labels, lse, loss_row, loss_mean, nullptr, 0, false, nullptr, 0,
                          M, V, d, stream, true);
}

coda_status coda_lmhead_ce_logits(const coda_bf16* H, int ldh, const coda_bf16* W, int ldw,
                                  const int32_t* labels, float* lse, float* loss_row,
                                  float* loss_mean, coda_bf16* logits, int ldl, void* ws,
                                  size_t ws_bytes, int M, int V, int d, hipStream_t stream) {
  trace("coda_lmhead_ce_logits", "M=%d V=%d d=%d ws_bytes=%zu", M, V, d, ws_bytes);
  return lmhead_ce_common(H, ldh, W, ldw, labels, lse, loss_row, loss_mean, logits, ldl, true, ws,
                          ws_bytes, M, V, d, stream);
}

coda_status coda_lmhead_ce_bwd(const coda_bf16* H, int ldh, const coda_bf16* W, int ldw,
                               const int32_t* labels, const float* lse, float grad_scale,
                               coda_bf16* dH, int lddh, float* dW, int lddw, void* ws,
                               size_t ws_bytes, int M, int V, int d, hipStream_t stream) {
  trace("coda_lmhead_ce_bwd", "M=%d V=%d d=%d ws_bytes=%zu", M, V, d, ws_bytes);
  Check c;
  c.shape(M >= 0 && V >= 0 && d >= 0);
  c.bmat(H, ldh, d, M);
  c.bmat(W, ldw, V, d);
  c.vec(labels, M, 4);
  c.vec(lse, M, 4);
  c.bmat(dH, lddh, d, M);
  c.fmat(dW, lddw, V, d);
  c.shape(V % 8 == 0 && d % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (V == 0 || d == 0) return CODA_OK;
  if (M > 0 && (ws == nullptr || !al16(ws) || ws_bytes < coda_lmhead_ce_bwd_workspace(M, V, d)))
    return CODA_ERR_WORKSPACE;
  if (coda_status st = c.device()) return st;
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
    EpiCEBwd<true> e1{labels + m0, lse + m0, grad_scale, D, V};
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

// Vocabulary-chunked CE backward: the dlogits chunk [M x vc] bf16 (ld = vc,
// 256-byte aligned) and, with more than one chunk, the fp32 dH accumulator
// [M x d] after it.
static size_t vchunk_d_bytes(int M, int vc) { return ((size_t)M * (size_t)vc * 2 + 255) / 256 * 256; }

size_t coda_lmhead_ce_bwd_vchunk_workspace(int M, int V, int d, int vchunk) {
  if (M <= 0 || V <= 0 || d <= 0 || vchunk <= 0 || vchunk % 8 != 0) return 0;
  const int vc = vchunk < V ? vchunk : V;
  const bool multi = vc < V;
  return vchunk_d_bytes(M, vc) + (multi ? (size_t)M * (size_t)d * 4 : 0);
}

coda_status coda_lmhead_ce_bwd_vchunk(const coda_bf16* H, int ldh, const coda_bf16* W, int ldw,
                                      const int32_t* labels, const float* lse, float grad_scale, coda_bf16* dH,
                                      int lddh, float* dW, int lddw, void* ws, size_t ws_bytes, int M, int V, int d,
                                      int vchunk, hipStream_t stream) {
  trace("coda_lmhead_ce_bwd_vchunk", "M=%d V=%d d=%d vchunk=%d ws_bytes=%zu", M, V, d, vchunk, ws_bytes);
  Check c;
  c.shape(M >= 0 && V >= 0 && d >= 0 && vchunk > 0 && vchunk % 8 == 0);
  c.bmat(H, ldh, d, M);
  c.bmat(W, ldw, V, d);
  c.vec(labels, M, 4);
  c.vec(lse, M, 4);
  c.bmat(dH, lddh, d, M);
  c.fmat(dW, lddw, V, d);
  c.shape(V % 8 == 0 && d % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (V == 0 || d == 0) return CODA_OK;
  if (M > 0 && (ws == nullptr || ((uintptr_t)ws & 255) != 0 ||
                ws_bytes < coda_lmhead_ce_bwd_vchunk_workspace(M, V, d, vchunk)))
    return CODA_ERR_WORKSPACE;
  if (coda_status st = c.device()) return st;
  if (M == 0)  // no rows: dW = H^T D over an empty reduction = 0
    return coda_gemm_wgrad(H, ldh, nullptr, V, dW, lddw, 0, d, V, 0, stream);
  const int vc = vchunk < V ? vchunk : V;
  const int nch = cdiv(V, vc);
  uint16_t* D = static_cast<uint16_t*>(ws);
  float* dh = reinterpret_cast<float*>(static_cast<char*>(ws) + vchunk_d_bytes(M, vc));
  for (int ch = 0; ch < nch; ++ch) {
    const int v0 = ch * vc, vcc = (V - v0) < vc ? (V - v0) : vc;
    // 1) recompute the chunk's logits and form its dlogits D [M x vcc] (bf16,
    //    ordinary stores: the two GEMMs below read it back from the caches)
    EpiCEBwd<false> e1{labels, lse, grad_scale, D, vc, v0};
    if (coda_status s = launch_gemm<false, true>(W + v0, ldw, H, ldh, vcc, M, d, e1, stream)) return s;
    // 2) dW[:, v0 : v0 + vcc] = H^T D: every column of dW is written once
    if (coda_status s = coda_gemm_wgrad(H, ldh, D, vc, dW + v0, lddw, M, d, vcc, 0, stream)) return s;
    // 3) dH (+)= D W[:, chunk]^T: features = d (rows of W, contiguous along V)
    if (nch == 1) {
      EpiLinear<false, false> e3{nullptr, nullptr, 0, dH, lddh};
      if (coda_status s = launch_gemm<true, true>(W + v0, ldw, D, vc, d, M, vcc, e3, stream)) return s;
    } else if (ch == 0) {
      EpiF32<false> e3{dh, d};
      if (coda_status s = launch_gemm<true, true>(W + v0, ldw, D, vc, d, M, vcc, e3, stream)) return s;
    } else {
      EpiF32<true> e3{dh, d};
      if (coda_status s = launch_gemm<true, true>(W + v0, ldw, D, vc, d, M, vcc, e3, stream)) return s;
    }
  }
  if (nch > 1) {
    const long long n = (long long)M * (d / 8);
    const long long blocks = (n + 255) / 256;
    hipLaunchKernelGGL(f32_to_bf16_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256), 0, stream,
                       dh, d, dH, lddh, M, d);
    return launched();
  }
  return CODA_OK;
}

coda_status coda_lmhead_ce_bwd_logits(const coda_bf16* H, int ldh, const coda_bf16* W, int ldw,
                                      const int32_t* labels, const float* lse, float grad_scale,
                                      coda_bf16* logits, int ldl, coda_bf16* dH, int lddh,
                                      float* dW, int lddw, int M, int V, int d,
                                      hipStream_t stream) {
  trace("coda_lmhead_ce_bwd_logits", "M=%d V=%d d=%d", M, V, d);
  Check c;
  c.shape(M >= 0 && V >= 0 && d >= 0);
  c.bmat(H, ldh, d, M);
  c.bmat(W, ldw, V, d);
  c.vec(labels, M, 4);
  c.vec(lse, M, 4);
  c.bmat(logits, ldl, V, M);
  c.bmat(dH, lddh, d, M);
  c.fmat(dW, lddw, V, d);
  c.shape(V % 8 == 0 && d % 8 == 0);
  if (c.st != CODA_OK) return c.st;
  if (V == 0 || d == 0) return CODA_OK;
  if (coda_status st = c.device()) return st;
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
