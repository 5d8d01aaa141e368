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
// (BF = 256 features, BT = 256 tokens), BK = 64, two LDS stages (128 KiB).
// MFMA fragments are double-buffered in registers (the reads of k-step s+1
// overlap the MFMAs of k-step s); global loads run two k-tiles ahead through
// one register staging set; one barrier per k-tile, placed inside its last
// k-step so that MFMAs are queued on both sides of it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
  uint32_t ok = 0;  // bit i: chunk i is inside the matrix (else it is stored as zeros)

  // Load chunk i of the k-tile starting at k0.  K-major: element (row, k) at
  // g[row * ld + k]; MN-major: at g[k * ld + row], chunk i = the 16 bytes of
  // k-row kb*8 + i of this thread's 8x8 block.  Raw buffer loads through a
  // scalar descriptor based at the tile origin (range 4 GiB, so no hardware
  // range check is relied on); a masked chunk loads offset 0 (a valid
  // element) and is zeroed when written to LDS: branch-free and wait-free.
  __device__ __forceinline__ void load_chunk(const uint16_t* __restrict__ g, int ld, int row0, int nrows,
                                             int k0, int K, int tid, int i) {
    bool in;
    uint32_t off;
    __amdgpu_buffer_rsrc_t rs;
    if constexpr (KMAJ) {
      rs = __builtin_amdgcn_make_buffer_rsrc((void*)(g + (size_t)row0 * ld + k0), (short)0, -1, 0x00020000);
      const int idx = i * NT + tid;
      const int row = idx / KCH, ck = idx % KCH;
      in = row0 + row < nrows && k0 + ck * 8 < K;
      off = (uint32_t)(row * ld + ck * 8) * 2u;
    } else {
      rs = __builtin_amdgcn_make_buffer_rsrc((void*)(g + (size_t)k0 * ld + row0), (short)0, -1, 0x00020000);
      const int rb = tid % (ROWS / 8), kb = tid / (ROWS / 8);
      in = tid < NBLK && row0 + rb * 8 < nrows && k0 + kb * 8 + i < K;
      off = (uint32_t)((kb * 8 + i) * ld + rb * 8) * 2u;
    }
    ok = (ok & ~(1u << i)) | ((uint32_t)in << i);
    v[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, in ? off : 0u, 0, 0));
  }

  __device__ __forceinline__ u32x4 masked(int i) const {
    return ((ok >> i) & 1u) ? v[i] : (u32x4){0u, 0u, 0u, 0u};
  }

  // Write chunk i to the K-major LDS tile.  MN-major: row i of the transposed
  // 8x8 block (needs all eight loaded chunks).
  __device__ __forceinline__ void store_chunk(char* s, int tid, int i) const {
    if constexpr (KMAJ) {
      const int idx = i * NT + tid;
      const int row = idx / KCH, ck = idx % KCH;
      st16(s + lds_off(row, ck), masked(i));
    } else {
      if constexpr (NBLK < NT) {
        if (tid >= NBLK) return;
      }
      const int rb = tid % (ROWS / 8), kb = tid / (ROWS / 8);
      // chunk j holds k = kb*8 + j for rows rb*8 .. rb*8+7 (row 2d in the low
      // half of dword d); transposed row i packs k pairs (2q, 2q+1).
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t a = masked(2 * q)[i >> 1], b = masked(2 * q + 1)[i >> 1];
        o[q] = (i & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
      }
      st16(s + lds_off(rb * 8 + i, kb), o);
    }
  }

  __device__ __forceinline__ void load(const uint16_t* __restrict__ g, int ld, int row0, int nrows, int k0,
                                       int K, int tid) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) load_chunk(g, ld, row0, nrows, k0, K, tid, i);
  }
  __device__ __forceinline__ void store(char* s, int tid) const {
#pragma unroll
    for (int i = 0; i < NCH; ++i) store_chunk(s, tid, i);
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

  // ---- building blocks of the explicitly scheduled k-loop -------------------
  constexpr int NP = RI * CI / 2;     // MFMA pairs per k-step
  constexpr int NRD = RI + CI;        // fragment reads per k-step
  constexpr int RPP = (NRD + NP - 1) / NP;
  constexpr int NCA = TileCopy<BF, WK>::NCH, NCB = TileCopy<BT, XK>::NCH;
  constexpr int APP = (NCA + NP - 1) / NP, BPP = (NCB + NP - 1) / NP;
  constexpr int HP = NP / 2;          // pairs before the barrier in step 3

  auto read_one = [&](const char* st, int s, int q, bf16x8 (&a)[RI], bf16x8 (&b)[CI]) {
    const int ck = 2 * s + hh;
    if (q < RI)
      a[q] = __builtin_bit_cast(bf16x8, ld16(st + lds_off(a_row[q], ck)));
    else if (q < NRD)
      b[q - RI] = __builtin_bit_cast(bf16x8, ld16(st + A_BYTES + lds_off(b_row[q - RI], ck)));
  };
  auto mfma_pair = [&](const bf16x8 (&a)[RI], const bf16x8 (&b)[CI], int pr) {
    constexpr int JP = CI / 2;
    const int i = pr / JP, j = 2 * (pr % JP);
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    acc[i][j + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j + 1], acc[i][j + 1], 0, 0, 0);
  };
  auto load_a = [&](int k0, int i) { ca.load_chunk(p.W, p.ldw, f0, p.F, k0, p.K, tid, i); };
  auto load_b = [&](int k0, int i) { cb.load_chunk(p.X, p.ldx, t0, p.T, k0, p.K, tid, i); };

  // Prologue: k-tile 0 to LDS stage 0, k-tile 1 to the staging registers.
  // With no k-tile (K == 0) nothing is loaded: an empty operand may have no
  // storage at all, and masked chunks read the tile origin, which then does
  // not exist.  Every load below has k0 < K and a tile origin inside the
  // matrix, so its offset-0 fallback is a real element.
  bf16x8 fa0[RI], fb0[CI], fa1[RI], fb1[CI];
  if (nk > 0) {
    ca.load(p.W, p.ldw, f0, p.F, 0, p.K, tid);
    cb.load(p.X, p.ldx, t0, p.T, 0, p.K, tid);
    ca.store(smem, tid);
    cb.store(smem + A_BYTES, tid);
    if (nk > 1) {
      ca.load(p.W, p.ldw, f0, p.F, BK, p.K, tid);
      cb.load(p.X, p.ldx, t0, p.T, BK, p.K, tid);
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < NRD; ++q) read_one(smem, 0, q, fa0, fb0);
  }

  // One k-tile: four k-steps of NP MFMA pairs.  Each pair carries side work:
  // the fragment reads of the next k-step (into the other register set); in
  // step 2 the write of k-tile kt+1 from the staging registers to the other
  // LDS stage and, for K-major operands, the refill of each chunk with
  // k-tile kt+2; in step 3 the refill of MN-major operands, then the single
  // barrier, then the first fragment reads of k-tile kt+1.  sched_barrier
  // fences keep every piece in this order.
  auto ktile = [&](int kt, auto has1_c, auto has2_c) {
    constexpr bool HAS1 = decltype(has1_c)::value, HAS2 = decltype(has2_c)::value;
    const char* cur = smem + (kt & 1) * STAGE;
    char* nxt = smem + ((kt + 1) & 1) * STAGE;
    const int k2 = (kt + 2) * BK;
    // steps 0 and 1
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
      mfma_pair(fa0, fb0, pr);
#pragma unroll
      for (int r = 0; r < RPP; ++r) read_one(cur, 1, pr * RPP + r, fa1, fb1);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
      mfma_pair(fa1, fb1, pr);
#pragma unroll
      for (int r = 0; r < RPP; ++r) read_one(cur, 2, pr * RPP + r, fa0, fb0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // step 2
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
      mfma_pair(fa0, fb0, pr);
#pragma unroll
      for (int r = 0; r < RPP; ++r) read_one(cur, 3, pr * RPP + r, fa1, fb1);
      if constexpr (HAS1) {
#pragma unroll
        for (int c = 0; c < APP; ++c) {
          const int i = pr * APP + c;
          if (i < NCA) {
            ca.store_chunk(nxt, tid, i);
            if constexpr (HAS2 && WK) load_a(k2, i);
          }
        }
#pragma unroll
        for (int c = 0; c < BPP; ++c) {
          const int i = pr * BPP + c;
          if (i < NCB) {
            cb.store_chunk(nxt + A_BYTES, tid, i);
            if constexpr (HAS2 && XK) load_b(k2, i);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // step 3, first half: MN-major refills
#pragma unroll
    for (int pr = 0; pr < HP; ++pr) {
      mfma_pair(fa1, fb1, pr);
      if constexpr (HAS2 && !WK) {
#pragma unroll
        for (int c = 0; c < (NCA + HP - 1) / HP; ++c)
          if (pr * ((NCA + HP - 1) / HP) + c < NCA) load_a(k2, pr * ((NCA + HP - 1) / HP) + c);
      }
      if constexpr (HAS2 && !XK) {
#pragma unroll
        for (int c = 0; c < (NCB + HP - 1) / HP; ++c)
          if (pr * ((NCB + HP - 1) / HP) + c < NCB) load_b(k2, pr * ((NCB + HP - 1) / HP) + c);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    // step 3, second half: first fragments of k-tile kt+1
    constexpr int RPH = (NRD + (NP - HP) - 1) / (NP - HP);
#pragma unroll
    for (int pr = HP; pr < NP; ++pr) {
      mfma_pair(fa1, fb1, pr);
      if constexpr (HAS1) {
#pragma unroll
        for (int r = 0; r < RPH; ++r) read_one(nxt, 0, (pr - HP) * RPH + r, fa0, fb0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  int kt = 0;
  for (; kt + 2 < nk; ++kt) ktile(kt, T_{}, T_{});
  if (kt + 1 < nk) ktile(kt++, T_{}, F_{});
  if (kt < nk) ktile(kt, F_{}, F_{});

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
