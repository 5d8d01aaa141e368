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
// Operand staging.  Both operand tiles go from global memory straight to LDS
// with the gfx950 LDS-DMA buffer load (16 bytes per lane; lane L of one
// instruction lands at LDS base + 16 L), so no VGPR staging or ds_write is
// spent on them.  A K-contiguous ("K-major") tile is stored row-contiguous
// (128 bytes per row, 16-byte chunks XOR-swizzled by (row >> 1) & 7) and each
// MFMA fragment is one ds_read_b128.  A tile contiguous along its
// feature/token index ("MN-major") is stored as 64 k-rows (32-byte blocks
// XOR-swizzled by (k & 3) << 1) and its fragments come from two transposing
// reads (ds_read_b64_tr_b16): within a group of 16 lanes, lane j receives
// element j % 4 of the 8 bytes addressed by lane j / 4 + 4 m (m = 0..3).  All
// DMA writes cover whole 128/256/512-byte global rows per instruction, and every
// fragment read phase touches each LDS bank once.  Out-of-matrix chunks use an
// offset beyond the descriptor's range, for which the hardware writes zeros.
//
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

// Timeline builds (CODA_TIMELINE=1, a separate library) record per-wave
// timestamps of every tile; the default build compiles none of it.
#ifndef CODA_TIMELINE
#define CODA_TIMELINE 0
#endif
constexpr bool kTimeline = CODA_TIMELINE;
constexpr int TL_WORDS = 12;    // 64-bit words per wave record

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

// Feature permutation of one 32-row MFMA block (see file header).
__device__ __forceinline__ int phi32(int i) {
  const int g = i >> 3, h = (i >> 2) & 1, v = i & 3;
  return ((g >> 1) << 4) + (h << 3) + ((g & 1) << 2) + v;
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// The 32-bit LDS address of a pointer into the workgroup's LDS.  Converting a
// generic pointer costs a 64-bit add, a null test and a select; the kernels
// convert their LDS base once and add offsets to it.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_ptr_t)const_cast<void*>(p);
}

// One LDS-DMA instruction: 16 bytes per lane from buffer(base, range) at
// byte offset voff to LDS address dst + 16 * lane (dst wave-uniform).  Issued as
// inline assembly so that the compiler's wait insertion does not make every
// later LDS read wait for all DMA in flight; completion is awaited explicitly
// (wait_vmcnt) before the barrier that publishes the stage.  vmcnt counts in
// issue order, so waits the compiler inserts for its own later loads stay
// correct (they may only wait longer).
// NT marks the load non-temporal (data read once, e.g. an epilogue's input
// tile), so it does not displace the GEMM operands in the caches.
template <bool NT = false>
__device__ __forceinline__ void dma16(const void* base, uint32_t range, uint32_t voff, uint32_t dst) {
  typedef __attribute__((ext_vector_type(4))) int i32x4;
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  i32x4 rs;
  rs[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  rs[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));  // stride 0
  rs[2] = __builtin_amdgcn_readfirstlane((int)range);
  rs[3] = 0x00020000;
  const int m0 = __builtin_amdgcn_readfirstlane((int)dst);
  // A SALU write of M0 needs one wait state before an LDS-DMA instruction
  // reads it; s_nop 1 gives two.
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 1\n\t"
        "buffer_load_dwordx4 %0, %1, 0 offen nt lds"
        :
        : "v"(voff), "s"(rs), "s"(m0)
        : "memory", "m0");
  else
    asm volatile(
        "s_mov_b32 m0, %2\n\t"
        "s_nop 1\n\t"
        "buffer_load_dwordx4 %0, %1, 0 offen lds"
        :
        : "v"(voff), "s"(rs), "s"(m0)
        : "memory", "m0");
}

// s_waitcnt vmcnt(N), other counters unconstrained (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
// s_waitcnt lgkmcnt(0), other counters unconstrained.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (3 << 14)); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// wait_vmcnt<n> for an n known after unrolling (0, 16, 32 or 48; anything
// else waits for everything, which is always safe).
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  switch (n) {
    case 16: wait_vmcnt<16>(); break;
    case 32: wait_vmcnt<32>(); break;
    case 48: wait_vmcnt<48>(); break;
    default: wait_vmcnt<0>(); break;
  }
}

// ---------------------------------------------------------------------------
// One operand tile: ROWS rows (features or tokens) x BK = 64 k, in one LDS
// stage of REGION bytes.  Thread (wave w, lane l) issues NCH DMA instructions
// per k-tile; instruction i of wave w fills the 1 KiB LDS block 4 i + w.
//
// K-major (element (row, k) at g[row * ld + k]): block 4i+w holds rows
//   (4i+w)*8 .. +7; lane l loads row (4i+w)*8 + l/8, logical chunk
//   (l%8) ^ sw(row), sw(row) = (row >> 1) & 7 = (4w + l/16) & 7.
// MN-major (element (row, k) at g[k * ld + row]): k-rows of 2 ROWS bytes, KPR =
//   1024 / (2 ROWS) of them per block: block 4i+w holds k-rows (4i+w)*KPR ..
//   +KPR-1; lane l loads k-row (4i+w)*KPR + l/(64/KPR), logical chunk c with
//   32-byte block (p/2) ^ ((k & 3) << 1), p = l % (64/KPR).
// ---------------------------------------------------------------------------

template <int ROWS, bool KMAJ>
struct Operand {
  static_assert(ROWS == 128 || ROWS == 256, "tile rows");
  static constexpr int REGION = ROWS * BK * 2;           // bytes per stage
  static constexpr int NCH = REGION / (NT * 16);          // DMA instructions per thread
  // MN-major: instructions [0, NCH/2) fill k-rows 0..31 (k-steps 0 and 1),
  // which are free for the next k-tile half a k-tile earlier than the rest.
  // K-major rows hold all 64 k, so the whole region is released at once.
  static constexpr int NEARLY = KMAJ ? 0 : NCH / 2;
  uint32_t voff = 0;  // byte offset of chunk 0 from the k-tile origin
  uint32_t vstep = 0; // byte offset between chunks i and i+1
  int lrow = 0;       // (masking) row or k-row of chunk 0 relative to the tile origin
  int lcol = 0;       // (masking) k (K-major) or row (MN-major) of chunk 0

  __device__ __forceinline__ void init(int ld, int w, int l) {
    if constexpr (KMAJ) {
      const int row = w * 8 + (l >> 3);
      const int c = (l & 7) ^ ((w * 4 + (l >> 4)) & 7);
      lrow = row;
      lcol = c * 8;
      voff = (uint32_t)(row * ld + c * 8) * 2u;
      vstep = (uint32_t)(32 * ld) * 2u;
    } else {
      // KPR k-rows of 2 ROWS bytes per 1 KiB block, 64 / KPR lanes per k-row.
      constexpr int KPR = 1024 / (2 * ROWS), LPK = 64 / KPR;
      const int kr = w * KPR + l / LPK, pp = l % LPK;
      const int c = (((pp >> 1) ^ ((kr & 3) << 1)) << 1) | (pp & 1);
      lrow = kr;
      lcol = c * 8;
      voff = (uint32_t)(kr * ld + c * 8) * 2u;
      vstep = (uint32_t)(4 * KPR * ld) * 2u;
    }
  }

  // DMA chunk i of the k-tile at k0 into the stage at LDS byte offset `stage`
  // from the LDS address lds_base (wave-uniform: instruction i of wave w
  // writes block 4 i + w).
  template <bool MASKED>
  __device__ __forceinline__ void dma(const uint16_t* __restrict__ g, int ld, int row0, int nrows, int k0,
                                      int K, uint32_t lds_base, int stage, int w, int i) const {
    const uint16_t* base = KMAJ ? g + (size_t)row0 * ld + k0 : g + (size_t)k0 * ld + row0;
    uint32_t off = voff + (uint32_t)i * vstep;
    int range = 0x7fffffff;
    if constexpr (MASKED) {
      // Bytes from the tile origin to the end of the last valid row (K-major)
      // or k-row (MN-major); chunks beyond it, or past K / nrows inside a
      // row, get an offset beyond the range and are written as zeros.
      const long long span = KMAJ ? (long long)(nrows - row0 - 1) * ld + (K - k0)
                                  : (long long)(K - k0 - 1) * ld + (nrows - row0);
      range = (int)(span * 2 < 0x7fffffffLL ? span * 2 : 0x7fffffffLL);
      const bool in = KMAJ ? (k0 + lcol < K) : (row0 + lcol < nrows);
      off = in ? off : 0x80000000u;
    }
    dma16(base, (uint32_t)range, off, lds_base + (uint32_t)(stage + (4 * i + w) * 1024));
  }
};

// Per-lane LDS byte offset (within an operand's stage region) of an MFMA
// fragment: K-major row `row`, k half `hh` of k-step 0 (other k-steps: XOR
// (s << 5)); MN-major: the transposing-read address for feature/token block
// starting at `row0` (32 rows), k half hh, k-step 0, sub-read 0 (other
// k-steps / sub-reads: + (16 s + 4 u) * 512).
__device__ __forceinline__ int kmaj_frag_off(int row, int hh) {
  return row * 128 + ((hh ^ ((row >> 1) & 7)) << 4);
}
template <bool PHI, int PITCH = 512>
__device__ __forceinline__ int mnmaj_frag_off(int row0, int lane) {
  const int G = lane >> 4, q = lane & 15;
  const int kr = 8 * (G >> 1) + (q >> 2);
  const int r = 16 * (G & 1) + 4 * (q & 3);
  const int f = row0 + (PHI ? phi32(r) : r);
  const int blk = f >> 4;
  return kr * PITCH + ((blk ^ ((kr & 3) << 1)) << 5) + ((f & 15) << 1);
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
  int f_base;         // first feature of this launch (tiles cover [f_base, F))
  int t_base;         // first token of this launch (tiles cover [t_base, T))
  unsigned long long* tl;  // timeline records (timeline builds; else null)
  int tl_waves;            // records tl holds
};

// Timeline mark `slot` (0 tile start, 1 k-loop start, 2 k-loop end, 3
// epilogue end) of this wave: record blk * 4 + wave (blk: the dispatch block,
// or the tile of a persistent workgroup) holds the
// reference-clock (100 MHz) stamps in words 0-3, the shader-clock stamps in
// words 4-7, then the tile's token width, its k-tile count, and the HW_ID and
// XCC_ID registers (which compute unit ran it).
__device__ __forceinline__ void timeline_mark(const Problem& p, int slot, int bt, int nk, int blk) {
  if constexpr (kTimeline) {
    const unsigned long long rt = __builtin_amdgcn_s_memrealtime();
    const unsigned long long ct = __builtin_amdgcn_s_memtime();
    const int rec = blk * 4 + (int)(threadIdx.x >> 6);
    if ((threadIdx.x & 63) == 0 && rec < p.tl_waves) {
      unsigned long long* r = p.tl + (size_t)rec * TL_WORDS;
      r[slot] = rt;
      r[4 + slot] = ct;
      if (slot == 0) {
        r[8] = (unsigned long long)bt;
        r[9] = (unsigned long long)nk;
        r[10] = __builtin_amdgcn_s_getreg((31 << 11) | 4);   // HW_ID
        r[11] = __builtin_amdgcn_s_getreg((31 << 11) | 20);  // XCC_ID
      }
    }
  }
}

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

// What the k-loop carries besides the GEMM: by default nothing.  A carry's
// prime(nk) runs in the prologue, after the first two k-tiles' DMA (its
// kPrimeOps memory operations are the last ones the prologue's wait allows in
// flight); slot(kt, step, pr) runs after MFMA pair pr of k-step `step` (0..3)
// of k-tile kt, inside that pair's scheduling fence; its last kTailOps memory
// operations of a k-tile (stores, issued after the k-tile's DMA) stay in
// flight through the next k-tile's wait; drain(nk) runs after the k-loop,
// pend(g) after the epilogue.  kPersistent: one workgroup runs several tiles
// (timeline records are then kept per tile, not per workgroup).
struct NoCarry {
  static constexpr bool kPersistent = false;
  static constexpr int kPrimeOps = 0;  // memory operations prime() issues
  static constexpr int kTailOps = 0;   // stores slot() issues after the k-tile's last DMA
  __device__ __forceinline__ void prime(int) {}
  __device__ __forceinline__ void slot(int, int, int) {}
  __device__ __forceinline__ void drain(int) {}
  __device__ __forceinline__ void pend(const Geom&) {}
};

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

// LDS bytes an epilogue stages its tile I/O through after the main loop
// (Epi::LDS_BYTES; 0 for epilogues that work from registers alone).
template <class E, class = void>
struct EpiLds : std::integral_constant<int, 0> {};
template <class E>
struct EpiLds<E, std::void_t<decltype(E::LDS_BYTES)>> : std::integral_constant<int, E::LDS_BYTES> {};

// LDS bytes of one workgroup: two stages of both operand tiles.
template <int BF, int BT, bool WK, bool XK>
constexpr int lds_bytes() {
  return 2 * (Operand<BF, WK>::REGION + Operand<BT, XK>::REGION);
}

// One BF x BT output tile: block `bid` of `nb` blocks working on problem p,
// with the workgroup's LDS at `smem` (lds_bytes<BF, BT, WK, XK>() bytes).
template <int BF, int BT, bool WK, bool XK, class Epi, class Carry>
__device__ __forceinline__ void gemm_epi_tile(const Problem& p, const Epi& epi, char* smem, int bid, int nb,
                                              Carry& carry) {
  static_assert(BF == 256 && (BT == 256 || BT == 128), "tile shape");
  constexpr int WGF = 2, WGT = 2;           // 2 x 2 waves
  constexpr int WF = BF / WGF, WT = BT / WGT;
  static_assert(WF == WAVE_F, "row partials assume 128-feature wave tiles");
  constexpr int RI = WF / 32, CI = WT / 32;
  using OA = Operand<BF, WK>;
  using OB = Operand<BT, XK>;
  // LDS: A stage 0 | A stage 1 | B stage 0 | B stage 1
  constexpr int A_REG = OA::REGION, B_REG = OB::REGION, B_OFF = 2 * A_REG;
  constexpr int A_PITCH = 2 * BF, B_PITCH = 2 * BT;  // MN-major k-row bytes

  int tid = threadIdx.x;
  // A persistent workgroup recomputes its per-lane offsets for every tile
  // rather than keeping them live across the epilogue and the carry's work.
  if constexpr (Carry::kPersistent) asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf = wave % WGF, wt = wave / WGF;
  const int lt = lane & 31, hh = lane >> 5;
  int tf, tt;
  tile_coords(bid, nb, p.nTF, p.nTT, tf, tt);
  const int f0 = p.f_base + tf * BF, t0 = p.t_base + tt * BT;

  f32x16 acc[RI][CI];
#pragma unroll
  for (int i = 0; i < RI; ++i)
#pragma unroll
    for (int j = 0; j < CI; ++j) acc[i][j] = (f32x16){};

  // Per-lane fragment offsets (stage and k-step are added per read).
  int a_off[RI], b_off[CI];
#pragma unroll
  for (int i = 0; i < RI; ++i)
    a_off[i] = WK ? kmaj_frag_off(wf * WF + i * 32 + phi32(lt), hh) : mnmaj_frag_off<true, A_PITCH>(wf * WF + i * 32, lane);
#pragma unroll
  for (int j = 0; j < CI; ++j)
    b_off[j] = B_OFF + (XK ? kmaj_frag_off(wt * WT + j * 32 + lt, hh) : mnmaj_frag_off<false, B_PITCH>(wt * WT + j * 32, lane));

  OA oa;
  OB ob;
  oa.init(p.ldw, wave, lane);
  ob.init(p.ldx, wave, lane);
  const uint32_t lds0 = lds_addr(smem);

  const int nk = (p.K + BK - 1) / BK;
  const int blk = Carry::kPersistent ? bid : (int)blockIdx.x;
  timeline_mark(p, 0, BT, nk, blk);
  const bool interior = f0 + BF <= p.F && t0 + BT <= p.T && p.K % BK == 0;

  constexpr int NP = RI * CI / 2;           // MFMA pairs per k-step
  constexpr int NRA = WK ? RI : 2 * RI;     // LDS reads for operand A per k-step
  constexpr int NRB = XK ? CI : 2 * CI;
  constexpr int NRD = NRA + NRB;
  constexpr int RPP = (NRD + NP - 1) / NP;
  constexpr int NDMA = OA::NCH + OB::NCH;

  // Fragments are read two k-steps ahead into four register sets (set s
  // holds k-step s), so every fragment of a k-tile is in registers by the
  // start of its step 2: the stage is released there and the DMA of k-tile
  // kt+2 spreads over steps 2 and 3 (and, for the k-rows of MN-major operands
  // read by k-steps 0 and 1, over steps 0 and 1).  The texture unit takes
  // about 57 B/clk per CU; one k-tile's 64 KiB of DMA issued within a single
  // k-step (8 pairs) stalls the issuing waves.
  bf16x8 fa0[RI], fb0[CI], fa1[RI], fb1[CI], fa2[RI], fb2[CI], fa3[RI], fb3[CI];

  // Read n (first-use order: a0, b0.., a1..) of k-step s from `stage` (0/1).
  // MN-major fragments take two transposing reads (n and n+1 of the same
  // fragment fill its low and high halves).
  auto read_one = [&](int stage, int s, int n, bf16x8 (&a)[RI], bf16x8 (&b)[CI]) {
    if (n >= NRD) return;
    // order: fragment index q and (for MN-major) sub-read u
    int q, u = 0;
    {
      const int na = WK ? 1 : 2;  // reads per A fragment
      const int nb = XK ? 1 : 2;
      if (n < na) {
        q = 0;
        u = n;
      } else if (n < na + CI * nb) {
        q = RI + (n - na) / nb;
        u = (n - na) % nb;
      } else {
        q = 1 + (n - na - CI * nb) / na;
        u = (n - na - CI * nb) % na;
      }
    }
    if (q < RI) {
      if constexpr (WK) {
        a[q] = __builtin_bit_cast(bf16x8, ld16(smem + ((a_off[q] ^ (s << 5)) + stage * A_REG)));
      } else {
        typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
        const bf16x4 h = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(lds_ptr_t)(smem + a_off[q] + stage * A_REG + (16 * s + 4 * u) * A_PITCH));
#pragma unroll
        for (int e = 0; e < 4; ++e) a[q][4 * u + e] = h[e];
      }
    } else {
      const int j = q - RI;
      if constexpr (XK) {
        b[j] = __builtin_bit_cast(bf16x8, ld16(smem + ((b_off[j] ^ (s << 5)) + stage * B_REG)));
      } else {
        typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
        const bf16x4 h = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(lds_ptr_t)(smem + b_off[j] + stage * B_REG + (16 * s + 4 * u) * B_PITCH));
#pragma unroll
        for (int e = 0; e < 4; ++e) b[j][4 * u + e] = h[e];
      }
    }
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
    // DMA instruction d (0..NDMA-1) of the k-tile at k0 into stage `st`.
    auto dma = [&](int k0, int st, int d) {
      if (d < OA::NCH)
        oa.template dma<MASKED>(p.W, p.ldw, f0, p.F, k0, p.K, lds0, st * A_REG, wave, d);
      else if (d < NDMA)
        ob.template dma<MASKED>(p.X, p.ldx, t0, p.T, k0, p.K, lds0 + B_OFF, st * B_REG, wave, d - OA::NCH);
    };

    // The DMA of a k-tile in two parts: the early part (the k-rows 0..31 of
    // MN-major operands) and the late part (the rest).  Part 0 instruction d
    // (0..NE-1), part 1 instruction d (0..NL-1).
    constexpr int NE = OA::NEARLY + OB::NEARLY, NL = NDMA - NE;
    auto dma_part = [&](int k0, int st, int part, int d) {
      if (part == 0) {
        if (d < OA::NEARLY) dma(k0, st, d);
        else dma(k0, st, OA::NCH + d - OA::NEARLY);
      } else {
        if (d < OA::NCH - OA::NEARLY) dma(k0, st, OA::NEARLY + d);
        else dma(k0, st, OA::NCH + OB::NEARLY + d - (OA::NCH - OA::NEARLY));
      }
    };
    // The instructions of one part over the 2 NP MFMA pairs of two k-steps:
    // those due at pair pw.
    auto dma_window = [&](int k0, int st, int part, int pw) {
      constexpr int NPW = 2 * NP;
      if (part == 0) {
#pragma unroll
        for (int d = 0; d < NE; ++d)
          if ((d * NPW) / NE == pw) dma_part(k0, st, 0, d);
      } else {
#pragma unroll
        for (int d = 0; d < NL; ++d)
          if ((d * NPW) / NL == pw) dma_part(k0, st, 1, d);
      }
    };

    // Prologue: k-tiles 0 and 1 into stages 0 and 1 (each early part, then
    // late part).  With no k-tile nothing is loaded (an empty operand may have
    // no storage at all).  Every DMA has k0 < K and a tile origin inside its
    // matrix.
    if (nk > 0) {
#pragma unroll
      for (int d = 0; d < NE; ++d) dma_part(0, 0, 0, d);
#pragma unroll
      for (int d = 0; d < NL; ++d) dma_part(0, 0, 1, d);
      if (nk > 1) {
#pragma unroll
        for (int d = 0; d < NE; ++d) dma_part(BK, 1, 0, d);
#pragma unroll
        for (int d = 0; d < NL; ++d) dma_part(BK, 1, 1, d);
        carry.prime(nk);
        wait_vmcnt<NDMA + Carry::kPrimeOps>();
      } else {
        carry.prime(nk);
        wait_vmcnt<0>();
      }
      __syncthreads();
#pragma unroll
      for (int n = 0; n < NRD; ++n) read_one(0, 0, n, fa0, fb0);
#pragma unroll
      for (int n = 0; n < NRD; ++n) read_one(0, 1, n, fa1, fb1);
    }

    // One k-tile: four k-steps of NP MFMA pairs.  Steps 0 and 1 carry the
    // fragment reads of steps 2 and 3 and the early part of k-tile kt+2's DMA
    // (its target, k-rows 0..31 of stage kt & 1, was read into registers
    // during k-tile kt-1; a barrier first makes sure every wave is done).
    // Then wait for k-tile kt+1's DMA and barrier (every wave holds all of
    // k-tile kt's fragments, so its stage is free); steps 2 and 3 carry the
    // fragment reads of k-tile kt+1's steps 0 and 1 and the late part of
    // k-tile kt+2's DMA.  Per wave the parts are issued in the order E(t),
    // L(t), E(t+1), L(t+1), ...  sched_barrier fences keep the order.
    auto ktile = [&](int kt, auto has1_c, auto has2_c) {
      constexpr bool HAS1 = decltype(has1_c)::value, HAS2 = decltype(has2_c)::value;
      const int ST = kt & 1, NS = ST ^ 1;
      const int k2 = (kt + 2) * BK;
      if constexpr (HAS2 && NE > 0) __syncthreads();
#pragma unroll
      for (int pr = 0; pr < NP; ++pr) {
        mfma_pair(fa0, fb0, pr);
#pragma unroll
        for (int r = 0; r < RPP; ++r) read_one(ST, 2, pr * RPP + r, fa2, fb2);
        if constexpr (HAS2 && NE > 0) dma_window(k2, ST, 0, pr);
        carry.slot(kt, 0, pr);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int pr = 0; pr < NP; ++pr) {
        mfma_pair(fa1, fb1, pr);
#pragma unroll
        for (int r = 0; r < RPP; ++r) read_one(ST, 3, pr * RPP + r, fa3, fb3);
        if constexpr (HAS2 && NE > 0) dma_window(k2, ST, 0, NP + pr);
        carry.slot(kt, 1, pr);
        __builtin_amdgcn_sched_barrier(0);
      }
      // k-tile kt+1 has landed; the early part of kt+2 may still be in flight.
      if constexpr (HAS1) wait_vmcnt<(HAS2 ? NE : 0) + Carry::kTailOps>();
      __syncthreads();
#pragma unroll
      for (int pr = 0; pr < NP; ++pr) {
        mfma_pair(fa2, fb2, pr);
        if constexpr (HAS1) {
#pragma unroll
          for (int r = 0; r < RPP; ++r) read_one(NS, 0, pr * RPP + r, fa0, fb0);
        }
        if constexpr (HAS2) dma_window(k2, ST, 1, pr);
        carry.slot(kt, 2, pr);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int pr = 0; pr < NP; ++pr) {
        mfma_pair(fa3, fb3, pr);
        if constexpr (HAS1) {
#pragma unroll
          for (int r = 0; r < RPP; ++r) read_one(NS, 1, pr * RPP + r, fa1, fb1);
        }
        if constexpr (HAS2) dma_window(k2, ST, 1, NP + pr);
        carry.slot(kt, 3, pr);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    // k-tile kt lives in LDS stage kt & 1.
    timeline_mark(p, 1, BT, nk, blk);
    int kt = 0;
    for (; kt + 2 < nk; ++kt) ktile(kt, T_{}, T_{});
    if (kt + 1 < nk) ktile(kt++, T_{}, F_{});
    if (kt < nk) ktile(kt, F_{}, F_{});
  };
  if (interior)
    mainloop(std::false_type{});
  else
    mainloop(std::true_type{});
  timeline_mark(p, 2, BT, nk, blk);
  carry.drain(nk);

  // The epilogues copy accumulators out of their AGPRs with inline asm, which
  // the compiler's hazard check does not see: 24 wait states cover the
  // longest MFMA-write to VALU-read distance the ISA requires.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
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
  if constexpr (EpiLds<Epi>::value > 0) {
    __syncthreads();  // every wave is done with the operand stages
    epi.template apply<RI, CI>(acc, g, smem);
  } else {
    epi.template apply<RI, CI>(acc, g);
  }
  carry.pend(g);
  timeline_mark(p, 3, BT, nk, blk);
}

template <int BF, int BT, bool WK, bool XK, class Epi>
__global__ void __launch_bounds__(NT) gemm_epi_kernel(const Problem p, const Epi epi) {
  // The operand stages, or more when the epilogue stages more (at most the
  // 160 KiB of a gfx950 CU).
  constexpr int LDS = EpiLds<Epi>::value > lds_bytes<BF, BT, WK, XK>() ? EpiLds<Epi>::value
                                                                       : lds_bytes<BF, BT, WK, XK>();
  static_assert(LDS <= 160 * 1024, "epilogue staging exceeds the LDS");
  __shared__ __attribute__((aligned(1024))) char smem[LDS];
  NoCarry none;
  gemm_epi_tile<BF, BT, WK, XK, Epi>(p, epi, smem, blockIdx.x, gridDim.x, none);
}

// Two tile shapes in one dispatch (tile-count split): blocks [0, nbig) cover
// problem p in 256 x 256 tiles, the others cover q (the trailing features) in
// 256 x 128 tiles; the hardware dispatches those as the first ones finish.
template <bool WK, bool XK, class Epi>
__global__ void __launch_bounds__(NT) gemm_epi_kernel_split(const Problem p, const Problem q, const Epi epi) {
  constexpr int BIG = lds_bytes<256, 256, WK, XK>(), HALF = lds_bytes<256, 128, WK, XK>();
  constexpr int OPS = BIG > HALF ? BIG : HALF;
  constexpr int LDS = EpiLds<Epi>::value > OPS ? EpiLds<Epi>::value : OPS;
  static_assert(LDS <= 160 * 1024, "epilogue staging exceeds the LDS");
  __shared__ __attribute__((aligned(1024))) char smem[LDS];
  const int nbig = p.nTF * p.nTT;
  NoCarry none;
  if ((int)blockIdx.x < nbig)
    gemm_epi_tile<256, 256, WK, XK, Epi>(p, epi, smem, blockIdx.x, nbig, none);
  else
    gemm_epi_tile<256, 128, WK, XK, Epi>(q, epi, smem, blockIdx.x - nbig, gridDim.x - nbig, none);
}

// Persistent form: workgroup b runs tiles b, b + G, b + 2G, ... (G =
// gridDim.x) of p's 256 x 256 tiles, and the carry takes work from one tile
// into the next tile's k-loop; finish() completes the last tile's.  G is a
// multiple of 8 whenever it is below the tile count, so every tile runs on the
// XCD that tile_coords gives it.  The epilogue works from registers (no LDS
// staging).
template <bool WK, bool XK, class Epi, class Carry>
__global__ void __launch_bounds__(NT) gemm_epi_kernel_persistent(const Problem p, const Epi epi,
                                                                 const typename Carry::Args ca) {
  static_assert(EpiLds<Epi>::value == 0, "the persistent kernel's epilogue works from registers");
  __shared__ __attribute__((aligned(1024))) char smem[lds_bytes<256, 256, WK, XK>()];
  Carry carry(ca);
  const int nb = p.nTF * p.nTT;
  for (int tile = blockIdx.x; tile < nb; tile += gridDim.x) {
    gemm_epi_tile<256, 256, WK, XK, Epi>(p, epi, smem, tile, nb, carry);
    __syncthreads();  // every wave is done with the operand stages before the next prologue
  }
  carry.finish();
}

}  // namespace coda
