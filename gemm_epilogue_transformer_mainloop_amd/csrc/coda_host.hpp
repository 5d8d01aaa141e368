// coda_host.hpp - host-side helpers shared by the C ABI translation units:
// argument validation, the gfx950 device check and launch status.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "../../include/coda.h"

namespace coda_host {

// ---------------------------------------------------------------------------
// Validation helpers
// ---------------------------------------------------------------------------

inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Check {
  coda_status st = CODA_OK;
  void need(const void* p) {
    if (st == CODA_OK && p == nullptr) st = CODA_ERR_NULL;
  }
  // A bf16 matrix of `rows` x `cols`, leading dimension ld (NULL allowed when
  // optional or when it has no rows).
  void bmat(const void* p, int ld, int cols, bool required = true, int rows = 1) {
    if (st != CODA_OK) return;
    if (p == nullptr) {
      if (required && rows > 0) st = CODA_ERR_NULL;
      return;
    }
    if (ld < cols || ld <= 0) { st = CODA_ERR_SHAPE; return; }
    if (!al16(p) || (ld % 8) != 0) st = CODA_ERR_ALIGN;
  }
  void fmat(const void* p, int ld, int cols, bool required = true, int rows = 1) {
    if (st != CODA_OK) return;
    if (p == nullptr) {
      if (required && rows > 0) st = CODA_ERR_NULL;
      return;
    }
    if (ld < cols || ld <= 0) { st = CODA_ERR_SHAPE; return; }
    if (!al16(p) || (ld % 4) != 0) st = CODA_ERR_ALIGN;
  }
  void vec(const void* p, bool required = true, bool aligned16 = false, int n = 1) {
    if (st != CODA_OK) return;
    if (p == nullptr) {
      if (required && n > 0) st = CODA_ERR_NULL;
      return;
    }
    if (aligned16 && !al16(p)) st = CODA_ERR_ALIGN;
  }
  void shape(bool ok) {
    if (st == CODA_OK && !ok) st = CODA_ERR_SHAPE;
  }
  void unsupported(bool ok) {
    if (st == CODA_OK && !ok) st = CODA_ERR_UNSUPPORTED;
  }
};

// One gfx950 check per device, cached (architecture never changes).
inline std::atomic<int> g_arch_ok[64];

inline coda_status device_ok() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return CODA_ERR_HIP;
  if (dev < 0 || dev >= 64) return CODA_ERR_UNSUPPORTED;
  int v = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return CODA_ERR_HIP;
    v = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_ok[dev].store(v, std::memory_order_relaxed);
  }
  return v == 1 ? CODA_OK : CODA_ERR_UNSUPPORTED;
}

// Compute units of the current device, cached per device (0 if unknown).
inline std::atomic<int> g_cus[64];

inline int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int v = g_cus[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) return 0;
    g_cus[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

inline coda_status launched() { return hipGetLastError() == hipSuccess ? CODA_OK : CODA_ERR_HIP; }

inline int cdiv(int a, int b) { return (a + b - 1) / b; }

}  // namespace coda_host
