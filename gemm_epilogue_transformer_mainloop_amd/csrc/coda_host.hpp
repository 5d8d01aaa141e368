// coda_host.hpp - host-side helpers shared by the C ABI translation units:
// argument validation, the optional host-side extent check and call log, the
// gfx950 device check and launch status.
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/coda.h"

namespace coda_host {

// ---------------------------------------------------------------------------
// Environment switches (read once per process)
// ---------------------------------------------------------------------------

inline bool env_on(const char* name) {
  const char* v = std::getenv(name);
  return v != nullptr && v[0] != '\0' && !(v[0] == '0' && v[1] == '\0');
}

// CODA_LOG=1: every entry point prints its name and sizes to stderr.
inline bool log_on() {
  static const bool on = env_on("CODA_LOG");
  return on;
}

// CODA_DEBUG=1: before any launch, every matrix and vector argument's byte
// extent is checked against the device allocation that holds its base
// pointer (hipMemGetAddressRange); an extent that leaves its allocation
// fails with CODA_ERR_BOUNDS.  (A caching allocator's allocation may be
// larger than the tensor the caller means, so this catches escapes from the
// allocation, not from the tensor.)
inline bool debug_on() {
  static const bool on = env_on("CODA_DEBUG");
  return on;
}

inline void trace(const char* fn, const char* fmt, ...) {
  if (!log_on()) return;
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  std::fprintf(stderr, "[coda] %s(%s)\n", fn, buf);
}

// Does [p, p + bytes) lie inside one device allocation?
inline coda_status extent_ok(const void* p, size_t bytes) {
  if (p == nullptr || bytes == 0) return CODA_OK;
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of a failed query
    return CODA_ERR_BOUNDS;
  }
  const uintptr_t b = reinterpret_cast<uintptr_t>(base), q = reinterpret_cast<uintptr_t>(p);
  return (q >= b && q - b <= size && bytes <= size - (q - b)) ? CODA_OK : CODA_ERR_BOUNDS;
}

// ---------------------------------------------------------------------------
// Validation
// ---------------------------------------------------------------------------

inline bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// One gfx950 check per device, cached (the architecture never changes).
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

// Argument checks of one call.  Each matrix / vector check also records the
// argument's byte extent, which device() verifies under CODA_DEBUG=1.
struct Check {
  static constexpr int MAXEXT = 24;
  coda_status st = CODA_OK;
  const void* ep[MAXEXT];
  size_t eb[MAXEXT];
  int ne = 0;

  void extent(const void* p, size_t bytes) {
    if (p != nullptr && bytes > 0 && ne < MAXEXT) {
      ep[ne] = p;
      eb[ne] = bytes;
      ++ne;
    }
  }
  // A row-major matrix of `rows` x `cols` elements of `esize` bytes with
  // leading dimension ld (NULL allowed when optional or when it has no rows).
  void mat(const void* p, int ld, int cols, int rows, bool required, int esize, int ldmul) {
    if (st != CODA_OK) return;
    if (p == nullptr) {
      if (required && rows > 0) st = CODA_ERR_NULL;
      return;
    }
    if (ld < cols || ld <= 0) { st = CODA_ERR_SHAPE; return; }
    if (!al16(p) || (ld % ldmul) != 0) { st = CODA_ERR_ALIGN; return; }
    if (rows > 0 && cols > 0) extent(p, ((size_t)(rows - 1) * (size_t)ld + (size_t)cols) * (size_t)esize);
  }
  void bmat(const void* p, int ld, int cols, int rows, bool required = true) { mat(p, ld, cols, rows, required, 2, 8); }
  void fmat(const void* p, int ld, int cols, int rows, bool required = true) { mat(p, ld, cols, rows, required, 4, 4); }
  // A vector of n elements of esize bytes.
  void vec(const void* p, long long n, int esize, bool required = true, bool aligned16 = false) {
    if (st != CODA_OK) return;
    if (p == nullptr) {
      if (required && n > 0) st = CODA_ERR_NULL;
      return;
    }
    if (aligned16 && !al16(p)) { st = CODA_ERR_ALIGN; return; }
    if (n > 0) extent(p, (size_t)n * (size_t)esize);
  }
  void shape(bool ok) {
    if (st == CODA_OK && !ok) st = CODA_ERR_SHAPE;
  }
  void unsupported(bool ok) {
    if (st == CODA_OK && !ok) st = CODA_ERR_UNSUPPORTED;
  }
  // The device check, then (CODA_DEBUG=1) the recorded extents.
  coda_status device() const {
    if (coda_status s = device_ok()) return s;
    if (debug_on())
      for (int i = 0; i < ne; ++i)
        if (coda_status s = extent_ok(ep[i], eb[i])) return s;
    return CODA_OK;
  }
};

// The timeline buffer of timeline builds (coda_timeline_set), read by every
// GEMM launch of such a build under g_tl_mu.
inline std::mutex g_tl_mu;
inline unsigned long long* g_tl_buf = nullptr;
inline int g_tl_waves = 0;

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
