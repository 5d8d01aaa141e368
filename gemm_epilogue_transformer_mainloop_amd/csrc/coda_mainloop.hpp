// coda_mainloop.hpp - the fixed bf16 MFMA mainloop of every CODA call on gfx950.
//
// The paper "CODA: Rewriting Transformer Blocks as GEMM-Epilogue Programs"
// (abstract; Figure 3) keeps the GEMM mainloop fixed and moves the block's
// memory-bound work into the epilogue.  This file is that fixed mainloop for
// CDNA4; coda_epilogues.hpp holds the epilogues.
//
// Orientation.  The kernel computes D[f][t] = sum_k Wop[f][k] * Xop[k][t] with
// the FEATURE operand (weights; output columns of the user's GEMM) as MFMA
// operand A and the TOKEN operand (activations; output rows) as operand B.
// The gfx950 32x32x16 bf16 MFMA leaves, in lane l, token column l%32 and the
// accumulator rows 8*(v/4) + 4*(l/32) + v%4 (v = 0..15).  Feature row f of the
// wave tile is routed to MFMA row phi^-1(f) when operand A is read from LDS,
// where phi(8g + 4h + v) = 16*(g/2) + 8*h + 4*(g%2) + v, so that accumulator
// element 8*half + e of lane l holds feature 16*half + 8*(l/32) + e: every lane
// owns runs of 8 consecutive output features of one token.  Pair maps
// (SwiGLU, RoPE) are then register-local, as the reading notes "CODA
// GEMM-Epilogue Programming" section 2 require of the accumulator layout, row
// reductions are in-lane adds plus one exchange between lanes l and l^32, and
// every store is a 16-byte vector store.
//
// Operand layouts.  Each operand is either K-contiguous ("K-major") or
// contiguous along its feature/token index ("MN-major").  Both are staged to
// the same K-major, XOR-swizzled LDS tile: K-major tiles are copied with
// 16-byte loads; MN-major tiles are read as 8x8 bf16 blocks (eight coalesced
// 16-byte loads) and transposed in registers before the LDS write, so the
// MFMA fragment read is always one ds_read_b128 per lane.
//
// Pipeline.  256 threads = 4 waves in a 2x2 grid over a BF x BT output tile
// (BF = 256 features, BT = 256 tokens), BK = 64, two LDS stages (128 KiB):
// the global loads of k-tile kt+1 are issued before the MFMAs of k-tile kt
// and written to the other LDS stage after them; one barrier per k-tile.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coda {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

constexpr int BK = 64;          // k-tile depth (elements)
constexpr int NT = 256;         // threads per workgroup (4 waves of 64)
constexpr int ROW_BYTES = BK * 2;  // one LDS tile row: 64 bf16 = 128 bytes
constexpr int WAVE_F = 128;     // features per wave tile (row-partial granularity)
constexpr int WAVE_T = 128;     // tokens per wave tile (column-partial granularity)

// ---------------------------------------------------------------------------
// bf16 helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round two floats to bf16 (nearest-even, v_cvt_pk_bf16_f32) and pack (a low, b high).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ void unpack8(const u32x4 w, float (&v)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = bf_lo(w[i]);
    v[2 * i + 1] = bf_hi(w[i]);
  }
}

__device__ __forceinline__ u32x4 pack8(const float (&v)[8]) {
  return (u32x4){pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                 pack_bf16x2(v[6], v[7])};
}

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// ---------------------------------------------------------------------------
// LDS tile addressing: row-major [rows][64 bf16], 16-byte chunks XOR-swizzled
// by (row ^ row>>3) & 7 so that 16 consecutive rows reading the same logical
// chunk, and the transposed writer's 8-row blocks, hit distinct banks.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * ROW_BYTES + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

// Feature permutation of one 32-row MFMA block (see file header).
__device__ __forceinline__ int phi32(int i) {
  const int g = i >> 3, h = (i >> 2) & 1, v = i & 3;
  return ((g >> 1) << 4) + (h << 3) + ((g & 1) << 2) + v;
}

// ---------------------------------------------------------------------------
// Global -> register -> LDS tile copy of one operand (ROWS x BK).
// ---------------------------------------------------------------------------

template <int ROWS, bool KMAJ>
struct TileCopy {
  static_assert(ROWS == 128 || ROWS == 256, "tile rows");
  static constexpr int KCH = BK / 8;                    // 16-byte chunks per row
  static constexpr int NCH = KMAJ ? (ROWS * KCH) / NT : 8;
  static constexpr int NBLK = ROWS;                     // 8x8 blocks (MN-major)
  u32x4 v[NCH];

  // K-major: element (row, k) at g[row * ld + k].  MN-major: at g[k * ld + row].
  __device__ __forceinline__ void load(const uint16_t* __restrict__ g, int ld, int row0, int nrows,
                                       int k0, int K, int tid) {
    if constexpr (KMAJ) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int idx = i * NT + tid;
        const int row = idx / KCH, ck = idx % KCH;
        const int gr = row0 + row, gk = k0 + ck * 8;
        if (gr < nrows && gk < K)
          v[i] = ld16(g + (size_t)gr * ld + gk);
        else
          v[i] = (u32x4){0u, 0u, 0u, 0u};
      }
    } else {
      const int rb = tid % (ROWS / 8), kb = tid / (ROWS / 8);
      const int gr = row0 + rb * 8;
      const bool act = tid < NBLK && gr < nrows;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int gk = k0 + kb * 8 + j;
        if (act && gk < K)
          v[j] = ld16(g + (size_t)gk * ld + gr);
        else
          v[j] = (u32x4){0u, 0u, 0u, 0u};
      }
    }
  }

  __device__ __forceinline__ void store(char* s, int tid) const {
    if constexpr (KMAJ) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int idx = i * NT + tid;
        const int row = idx / KCH, ck = idx % KCH;
        st16(s + lds_off(row, ck), v[i]);
      }
    } else {
      if (tid >= NBLK) return;
      const int rb = tid % (ROWS / 8), kb = tid / (ROWS / 8);
      // v[j] holds k = kb*8 + j for rows rb*8 .. rb*8+7 (row 2d in the low half
      // of dword d).  Row r of the transposed block packs k pairs (2i, 2i+1).
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t a = v[2 * i][r >> 1], b = v[2 * i + 1][r >> 1];
          o[i] = (r & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        }
        st16(s + lds_off(rb * 8 + r, kb), o);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Problem description and epilogue geometry
// ---------------------------------------------------------------------------

struct Problem {
  const uint16_t* W;  // feature operand
  const uint16_t* X;  // token operand
  int ldw, ldx;
  int F, T, K;        // output features, tokens, reduction length
  int nTF, nTT;       // tile counts along F and T
};

// What one lane needs to place its accumulators.
struct Geom {
  int fw0;   // first feature of the wave tile
  int tw0;   // first token of the wave tile
  int lane, lt, hh;  // lane, token column (lane % 32), half (lane / 32)
  int F, T;
  int pf;    // wave-feature part index (fw0 / WAVE_F)
  int pt;    // wave-token part index (tw0 / WAVE_T)
};

// Token of MFMA column ci and first feature of run (ri, half) for this lane.
template <class G>
__device__ __forceinline__ int tok_of(const G& g, int ci) { return g.tw0 + ci * 32 + g.lt; }
template <class G>
__device__ __forceinline__ int feat_of(const G& g, int ri, int half) {
  return g.fw0 + ri * 32 + half * 16 + g.hh * 8;
}

// XCD-aware tile order: dispatch ids go round-robin over the 8 XCDs, so give
// each XCD a contiguous range of tile ids, then walk tiles in groups of
// GROUP_T token tiles so concurrently running tiles share operand panels in
// that XCD's L2.
__device__ __forceinline__ void tile_coords(int bid, int nb, int nTF, int nTT, int& tf, int& tt) {
  constexpr int NXCD = 8, GROUP_T = 4;
  const int q = nb / NXCD, rem = nb % NXCD;
  const int x = bid % NXCD, local = bid / NXCD;
  const int pid = x * q + (x < rem ? x : rem) + local;
  const int width = GROUP_T * nTF;
  const int group = pid / width;
  const int first_t = group * GROUP_T;
  const int gsz = (nTT - first_t) < GROUP_T ? (nTT - first_t) : GROUP_T;
  const int in = pid - group * width;
  tt = first_t + in % gsz;
  tf = in / gsz;
}

// ---------------------------------------------------------------------------
// The kernel
// ---------------------------------------------------------------------------

template <int BF, int BT, bool WK, bool XK, class Epi>
__global__ void __launch_bounds__(NT) gemm_epi_kernel(const Problem p, const Epi epi) {
  static_assert(BF == 256 && (BT == 256 || BT == 128), "tile shape");
  constexpr int WGF = 2, WGT = 2;           // 2 x 2 waves
  constexpr int WF = BF / WGF, WT = BT / WGT;
  static_assert(WF == WAVE_F, "row partials assume 128-feature wave tiles");
  constexpr int RI = WF / 32, CI = WT / 32;
  constexpr int A_BYTES = BF * ROW_BYTES, STAGE = (BF + BT) * ROW_BYTES;

  __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wf = wave % WGF, wt = wave / WGF;
  const int lt = lane & 31, hh = lane >> 5;
  int tf, tt;
  tile_coords(blockIdx.x, gridDim.x, p.nTF, p.nTT, tf, tt);
  const int f0 = tf * BF, t0 = tt * BT;

  TileCopy<BF, WK> ca;
  TileCopy<BT, XK> cb;
  f32x16 acc[RI][CI];
#pragma unroll
  for (int i = 0; i < RI; ++i)
#pragma unroll
    for (int j = 0; j < CI; ++j) acc[i][j] = (f32x16){};

  // Per-lane LDS byte offsets of the MFMA fragments (chunk added per k-step).
  int a_row[RI], b_row[CI];
#pragma unroll
  for (int i = 0; i < RI; ++i) a_row[i] = wf * WF + i * 32 + phi32(lt);
#pragma unroll
  for (int j = 0; j < CI; ++j) b_row[j] = wt * WT + j * 32 + lt;

  const int nk = (p.K + BK - 1) / BK;
  ca.load(p.W, p.ldw, f0, p.F, 0, p.K, tid);
  cb.load(p.X, p.ldx, t0, p.T, 0, p.K, tid);
  ca.store(smem, tid);
  cb.store(smem + A_BYTES, tid);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    char* cur = smem + (kt & 1) * STAGE;
    char* nxt = smem + ((kt + 1) & 1) * STAGE;
    const bool more = kt + 1 < nk;
    if (more) {
      ca.load(p.W, p.ldw, f0, p.F, (kt + 1) * BK, p.K, tid);
      cb.load(p.X, p.ldx, t0, p.T, (kt + 1) * BK, p.K, tid);
    }
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      const int ck = 2 * s + hh;
      bf16x8 a[RI], b[CI];
#pragma unroll
      for (int i = 0; i < RI; ++i)
        a[i] = __builtin_bit_cast(bf16x8, ld16(cur + lds_off(a_row[i], ck)));
#pragma unroll
      for (int j = 0; j < CI; ++j)
        b[j] = __builtin_bit_cast(bf16x8, ld16(cur + A_BYTES + lds_off(b_row[j], ck)));
#pragma unroll
      for (int i = 0; i < RI; ++i)
#pragma unroll
        for (int j = 0; j < CI; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      ca.store(nxt, tid);
      cb.store(nxt + A_BYTES, tid);
    }
    __syncthreads();
  }

  Geom g;
  g.fw0 = f0 + wf * WF;
  g.tw0 = t0 + wt * WT;
  g.lane = lane;
  g.lt = lt;
  g.hh = hh;
  g.F = p.F;
  g.T = p.T;
  g.pf = g.fw0 / WAVE_F;
  g.pt = g.tw0 / WT;
  epi.template apply<RI, CI>(acc, g);
}

}  // namespace coda
