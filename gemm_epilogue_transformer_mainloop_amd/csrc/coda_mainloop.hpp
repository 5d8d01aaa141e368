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
// k-step so that MFMAs are queued on both sides of it.  Interior tiles with
// K % 64 == 0 take an unmasked copy path; edge tiles a masked one.
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
// LDS tile layout ("k-step major").  One operand tile of ROWS rows x BK = 64
// k is stored as four slabs, one per 16-wide MFMA k-step; a slab holds, for
// each row, 32 bytes (two 16-byte halves: k 0-7 and k 8-15 of the step).
// Rows are grouped by 8 (256 bytes per group); inside a group the row's
// 32-byte slot is (row & 7) ^ ((row >> 4) & 7) and its halves are swapped
// when (row >> 3) is odd.  With this swizzle every 16-lane phase of
//   - an MFMA fragment read (16 consecutive rows, one half),
//   - a K-major tile write (8 rows x both halves),
//   - a transposed MN-major tile write (16 row groups, one row each)
// touches 16 distinct 16-byte slots of a 256-byte window, i.e. all 64 banks
// once; and the fragment address of a lane depends only on its row, so the
// k-step and the LDS stage become immediate offsets of ds_read_b128.
// ---------------------------------------------------------------------------

__device__ __forceinline__ int slab_off(int row, int half) {
  return ((row >> 3) << 8) + ((((row & 7) ^ ((row >> 4) & 7))) << 5) + ((half ^ ((row >> 3) & 1)) << 4);
}

// Feature permutation of one 32-row MFMA block (see file header).
__device__ __forceinline__ int phi32(int i) {
  const int g = i >> 3, h = (i >> 2) & 1, v = i & 3;
  return ((g >> 1) << 4) + (h << 3) + ((g & 1) << 2) + v;
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t rs, uint32_t voff, int soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0));
}

// ---------------------------------------------------------------------------
// Global -> register -> LDS copy of one operand tile (ROWS x BK).
//
// K-major (element (row, k) at g[row * ld + k]): chunk i of thread
// (wave w, lane l) is row i*32 + w*8 + ((l>>1)&7), k-chunk 2*(l>>4) + (l&1);
// a wave instruction reads 8 whole 128-byte rows.  MN-major (element at
// g[k * ld + row], ROWS == 256): thread t owns the 8x8 block of rows
// (t%32)*8.. and k (t/32)*8..; chunk j is k-row j of the block (a wave
// instruction reads two 512-byte row segments) and is transposed in
// registers before the LDS write.
//
// Loads are raw buffer loads through a scalar descriptor based at the tile
// origin of the k-tile (range 4 GiB; no hardware range check is relied on).
// The per-chunk stride goes in the scalar soffset.  MASKED variants (edge
// tiles, ragged K) replace an out-of-matrix chunk's offset by 0 (the tile
// origin, a real element) and zero the chunk when it is written to LDS.
// ---------------------------------------------------------------------------

template <int ROWS, bool KMAJ>
struct TileCopy {
  static_assert(ROWS == 128 || ROWS == 256, "tile rows");
  static_assert(KMAJ || ROWS == 256, "MN-major operands use 256-row tiles");
  static constexpr int NCH = KMAJ ? ROWS / 32 : 8;   // 16-byte chunks per thread
  static constexpr int SLAB = ROWS * 32;               // bytes per k-step slab
  static constexpr int REGION = ROWS * BK * 2;         // bytes per LDS stage
  u32x4 v[NCH];
  uint32_t ok = 0;      // MASKED only: bit i set = chunk i is inside the matrix
  uint32_t voff = 0;    // per-thread byte offset of chunk 0 from the tile origin
  int wbase[4];         // LDS write offsets (K-major: chunks i and i+4; MN-major: wbase[0])
  int sld2 = 0;         // 2 * ld (bytes per k-row or per row)
  int lrow = 0, lk = 0; // (MASKED) row and k of chunk 0 relative to the tile origin

  __device__ __forceinline__ void init(int ld, int tid) {
    const int w = tid >> 6, l = tid & 63;
    sld2 = 2 * ld;
    if constexpr (KMAJ) {
      const int q = (l >> 1) & 7, ck = 2 * (l >> 4) + (l & 1);
      lrow = w * 8 + q;
      lk = ck * 8;
      voff = (uint32_t)(lrow * ld + lk) * 2u;
      const int s = l >> 4, h = l & 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) wbase[i] = s * SLAB + slab_off(i * 32 + lrow, h);
    } else {
      const int rb = tid & 31, kb = tid >> 5;
      lrow = rb * 8;
      lk = kb * 8;
      voff = (uint32_t)(lk * ld + lrow) * 2u;
      wbase[0] = (kb >> 1) * SLAB + slab_off(rb * 8, kb & 1);  // row 0 of the block
    }
  }

  // Stride of chunk i from chunk 0, in bytes (uniform).
  __device__ __forceinline__ int soff(int i) const { return KMAJ ? i * 32 * sld2 : i * sld2; }

  template <bool MASKED>
  __device__ __forceinline__ void load_chunk(const uint16_t* __restrict__ g, int ld, int row0, int nrows,
                                             int k0, int K, int i) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(g + (KMAJ ? (size_t)row0 * ld + k0 : (size_t)k0 * ld + row0)), (short)0, -1, 0x00020000);
    if constexpr (!MASKED) {
      v[i] = buf_load16(rs, voff, soff(i));
    } else {
      const bool in = KMAJ ? (row0 + lrow + 32 * i < nrows && k0 + lk < K)
                           : (row0 + lrow < nrows && k0 + lk + i < K);
      ok = (ok & ~(1u << i)) | ((uint32_t)in << i);
      v[i] = buf_load16(rs, in ? voff + (uint32_t)soff(i) : 0u, 0);
    }
  }

  template <bool MASKED>
  __device__ __forceinline__ u32x4 chunk(int i) const {
    if constexpr (!MASKED) return v[i];
    return ((ok >> i) & 1u) ? v[i] : (u32x4){0u, 0u, 0u, 0u};
  }

  // Write chunk i (MN-major: transposed row i of the thread's block).
  template <bool MASKED>
  __device__ __forceinline__ void store_chunk(char* s, int i) const {
    if constexpr (KMAJ) {
      st16(s + wbase[i & 3] + (i >> 2) * 4096, chunk<MASKED>(i));
    } else {
      u32x4 o;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t a = chunk<MASKED>(2 * q)[i >> 1], b = chunk<MASKED>(2 * q + 1)[i >> 1];
        o[q] = (i & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
      }
      st16(s + (wbase[0] ^ (i << 5)), o);
    }
  }
};

// First-use order of the RI + CI fragments of one k-step for the MFMA pair
// sequence pr -> (i = pr / (CI/2), j = 2*(pr % (CI/2)), j+1): a0, b0..b(CI-1),
// a1..a(RI-1).  Returns the fragment index (< RI: operand A row block i,
// else RI + column block j).
template <int RI, int CI>
__device__ __forceinline__ constexpr int frag_order(int n) {
  return n == 0 ? 0 : (n <= CI ? RI + n - 1 : n - CI);
}

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
  using CA = TileCopy<BF, WK>;
  using CB = TileCopy<BT, XK>;
  // LDS: A stage 0 | A stage 1 | B stage 0 | B stage 1
  constexpr int A_REG = CA::REGION, B_REG = CB::REGION, B_OFF = 2 * A_REG;

  __shared__ __attribute__((aligned(16))) char smem[2 * (A_REG + B_REG)];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wf = wave % WGF, wt = wave / WGF;
  const int lt = lane & 31, hh = lane >> 5;
  int tf, tt;
  tile_coords(blockIdx.x, gridDim.x, p.nTF, p.nTT, tf, tt);
  const int f0 = tf * BF, t0 = tt * BT;

  f32x16 acc[RI][CI];
#pragma unroll
  for (int i = 0; i < RI; ++i)
#pragma unroll
    for (int j = 0; j < CI; ++j) acc[i][j] = (f32x16){};

  // Per-lane LDS fragment offsets (k-step and stage are immediates).
  int a_off[RI], b_off[CI];
#pragma unroll
  for (int i = 0; i < RI; ++i) a_off[i] = slab_off(wf * WF + i * 32 + phi32(lt), hh);
#pragma unroll
  for (int j = 0; j < CI; ++j) b_off[j] = B_OFF + slab_off(wt * WT + j * 32 + lt, hh);

  CA ca;
  CB cb;
  ca.init(p.ldw, tid);
  cb.init(p.ldx, tid);

  const int nk = (p.K + BK - 1) / BK;
  const bool interior = f0 + BF <= p.F && t0 + BT <= p.T && p.K % BK == 0;

  constexpr int NP = RI * CI / 2;     // MFMA pairs per k-step
  constexpr int NRD = RI + CI;        // fragment reads per k-step
  constexpr int RPP = (NRD + NP - 1) / NP;
  constexpr int HP = NP / 2;          // pairs before the barrier in step 3
  constexpr int RPH = (NRD + (NP - HP) - 1) / (NP - HP);

  bf16x8 fa0[RI], fb0[CI], fa1[RI], fb1[CI];

  // stage = 0 or 1 (runtime): byte offsets stage*A_REG / stage*B_REG are one
  // VALU add per fragment per k-tile; the k-step is an immediate offset.
  auto read_one = [&](int stage, int s, int n, bf16x8 (&a)[RI], bf16x8 (&b)[CI]) {
    if (n >= NRD) return;
    const int q = frag_order<RI, CI>(n);
    if (q < RI)
      a[q] = __builtin_bit_cast(bf16x8, ld16(smem + (a_off[q] + stage * A_REG) + s * CA::SLAB));
    else
      b[q - RI] = __builtin_bit_cast(bf16x8, ld16(smem + (b_off[q - RI] + stage * B_REG) + s * CB::SLAB));
  };
  auto mfma_pair = [&](const bf16x8 (&a)[RI], const bf16x8 (&b)[CI], int pr) {
    constexpr int JP = CI / 2;
    const int i = pr / JP, j = 2 * (pr % JP);
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    acc[i][j + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j + 1], acc[i][j + 1], 0, 0, 0);
  };

  // The whole k-loop for one masking mode (uniform per workgroup).
  auto mainloop = [&](auto masked_c) {
    constexpr bool MASKED = decltype(masked_c)::value;
    auto load_a = [&](int k0, int i) { ca.template load_chunk<MASKED>(p.W, p.ldw, f0, p.F, k0, p.K, i); };
    auto load_b = [&](int k0, int i) { cb.template load_chunk<MASKED>(p.X, p.ldx, t0, p.T, k0, p.K, i); };

    // Prologue: k-tile 0 to LDS stage 0, k-tile 1 to the staging registers.
    // Every load has k0 < K and a tile origin inside its matrix, so the
    // offset-0 fallback of a masked chunk is a real element; with no k-tile
    // nothing is loaded (an empty operand may have no storage at all).
    if (nk > 0) {
#pragma unroll
      for (int i = 0; i < CA::NCH; ++i) load_a(0, i);
#pragma unroll
      for (int i = 0; i < CB::NCH; ++i) load_b(0, i);
#pragma unroll
      for (int i = 0; i < CA::NCH; ++i) ca.template store_chunk<MASKED>(smem, i);
#pragma unroll
      for (int i = 0; i < CB::NCH; ++i) cb.template store_chunk<MASKED>(smem + B_OFF, i);
      if (nk > 1) {
#pragma unroll
        for (int i = 0; i < CA::NCH; ++i) load_a(BK, i);
#pragma unroll
        for (int i = 0; i < CB::NCH; ++i) load_b(BK, i);
      }
      __syncthreads();
#pragma unroll
      for (int n = 0; n < NRD; ++n) read_one(0, 0, n, fa0, fb0);
    }

    // One k-tile: four k-steps of NP MFMA pairs.  Each pair carries side
    // work: a fragment read of the next k-step (other register set, in
    // first-use order); in step 2 the write of k-tile kt+1 from the staging
    // registers to the other LDS stage and, for K-major operands, the refill
    // of each chunk with k-tile kt+2; in step 3 the refill of MN-major
    // operands, then the single barrier, then the first fragment reads of
    // k-tile kt+1.  sched_barrier fences keep every piece in this order.
    auto ktile = [&](int kt, auto has1_c, auto has2_c) {
      const int ST = kt & 1, NS = ST ^ 1;
      constexpr bool HAS1 = decltype(has1_c)::value, HAS2 = decltype(has2_c)::value;
      const int k2 = (kt + 2) * BK;
      constexpr int APP = (CA::NCH + NP - 1) / NP, BPP = (CB::NCH + NP - 1) / NP;
#pragma unroll
      for (int pr = 0; pr < NP; ++pr) {
        mfma_pair(fa0, fb0, pr);
#pragma unroll
        for (int r = 0; r < RPP; ++r) read_one(ST, 1, pr * RPP + r, fa1, fb1);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int pr = 0; pr < NP; ++pr) {
        mfma_pair(fa1, fb1, pr);
#pragma unroll
        for (int r = 0; r < RPP; ++r) read_one(ST, 2, pr * RPP + r, fa0, fb0);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int pr = 0; pr < NP; ++pr) {
        mfma_pair(fa0, fb0, pr);
#pragma unroll
        for (int r = 0; r < RPP; ++r) read_one(ST, 3, pr * RPP + r, fa1, fb1);
        if constexpr (HAS1) {
#pragma unroll
          for (int c = 0; c < APP; ++c) {
            const int i = pr * APP + c;
            if (i < CA::NCH) {
              ca.template store_chunk<MASKED>(smem + NS * A_REG, i);
              if constexpr (HAS2 && WK) load_a(k2, i);
            }
          }
#pragma unroll
          for (int c = 0; c < BPP; ++c) {
            const int i = pr * BPP + c;
            if (i < CB::NCH) {
              cb.template store_chunk<MASKED>(smem + B_OFF + NS * B_REG, i);
              if constexpr (HAS2 && XK) load_b(k2, i);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      constexpr int AH = (CA::NCH + HP - 1) / HP, BH = (CB::NCH + HP - 1) / HP;
#pragma unroll
      for (int pr = 0; pr < HP; ++pr) {
        mfma_pair(fa1, fb1, pr);
        if constexpr (HAS2 && !WK) {
#pragma unroll
          for (int c = 0; c < AH; ++c)
            if (pr * AH + c < CA::NCH) load_a(k2, pr * AH + c);
        }
        if constexpr (HAS2 && !XK) {
#pragma unroll
          for (int c = 0; c < BH; ++c)
            if (pr * BH + c < CB::NCH) load_b(k2, pr * BH + c);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __syncthreads();
#pragma unroll
      for (int pr = HP; pr < NP; ++pr) {
        mfma_pair(fa1, fb1, pr);
        if constexpr (HAS1) {
#pragma unroll
          for (int r = 0; r < RPH; ++r) read_one(NS, 0, (pr - HP) * RPH + r, fa0, fb0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    // k-tile kt lives in LDS stage kt & 1.
    int kt = 0;
    for (; kt + 2 < nk; ++kt) ktile(kt, T_{}, T_{});
    if (kt + 1 < nk) ktile(kt++, T_{}, F_{});
    if (kt < nk) ktile(kt, F_{}, F_{});
  };
  if (interior)
    mainloop(std::false_type{});
  else
    mainloop(std::true_type{});

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
