// coda_mainloop_occ2.hpp - the same fixed bf16 MFMA mainloop, sized so that
// TWO workgroups share each CU and overlap one tile's epilogue with the other
// tile's MFMAs.
//
// The paper "CODA: Rewriting Transformer Blocks as GEMM-Epilogue Programs"
// notes that epilogues can overlap with tensor-core work (its Hopper design
// alternates two consumer warpgroups, "PingPong").  On CDNA4 the hardware
// already interleaves the waves of co-resident workgroups on each SIMD, so
// the overlap comes from fitting two workgroups per CU:
//  - output tile 256 features x 128 tokens; 4 waves of 128 x 64 (RI = 4,
//    CI = 2): 128 accumulator AGPRs and at most 128 VGPRs per wave, so two
//    waves fit per SIMD (__launch_bounds__(256, 2));
//  - three LDS stages of BK = 32 (72 KiB per workgroup, 144 KiB per CU).
// While one workgroup loads z/pre, computes and stores its epilogue, the
// other keeps the MFMA pipe busy, and its DMA issue stalls are covered the
// same way.  The accumulator layout, the epilogue functors and the feature
// permutation are those of coda_mainloop.hpp; the token operand is always
// K-major (forward activations, data-gradient upstream gradients).
//
// LDS layouts (per stage):
//  - K-major operand: 64-byte rows (four 16-byte chunks; chunk c at position
//    c ^ kswz(row)); for the feature operand the DMA places global row
//    (P & ~31) + phi32(P & 31) in LDS row P, so fragment reads walk
//    consecutive rows, which kswz keeps on distinct banks.
//  - MN-major feature operand: 32 k-rows of 512 bytes, as in
//    coda_mainloop.hpp.
#pragma once

#include "coda_mainloop.hpp"

namespace coda {
namespace occ2 {

constexpr int BK = 32;      // k-tile depth: two MFMA k-steps
constexpr int NSTAGE = 3;   // LDS stages
constexpr int BF = 256;     // features per workgroup tile
constexpr int BT = 128;     // tokens per workgroup tile

__device__ __forceinline__ int kswz(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

template <int ROWS, bool KMAJ, bool PHI>
struct Operand {
  static_assert(KMAJ || ROWS == 256, "MN-major operands use 256-row tiles");
  static constexpr int REGION = ROWS * BK * 2;            // bytes per stage
  static constexpr int NCH = REGION / (NT * 16);          // DMA instructions per thread
  uint32_t voff = 0, vstep = 0;
  int lcol = 0;

  __device__ __forceinline__ void init(int ld, int w, int l) {
    if constexpr (KMAJ) {
      // block 4i+w holds LDS rows (4i+w)*16 .. +15; lane l fills row
      // (4i+w)*16 + l/4 at chunk position l%4 (kswz is the same for all i)
      const int P = w * 16 + (l >> 2);
      const int c = (l & 3) ^ kswz(P);
      const int grow = PHI ? (P & ~31) + phi32(P & 31) : P;
      lcol = c * 8;
      voff = (uint32_t)(grow * ld + c * 8) * 2u;
      vstep = (uint32_t)(64 * ld) * 2u;
    } else {
      const int kr = w * 2 + (l >> 5), pp = l & 31;
      const int c = (((pp >> 1) ^ ((kr & 3) << 1)) << 1) | (pp & 1);
      lcol = c * 8;
      voff = (uint32_t)(kr * ld + c * 8) * 2u;
      vstep = (uint32_t)(8 * ld) * 2u;
    }
  }

  template <bool MASKED>
  __device__ __forceinline__ void dma(const uint16_t* __restrict__ g, int ld, int row0, int nrows, int k0,
                                      int K, char* smem_base, int stage, int w, int i) const {
    const uint16_t* base = KMAJ ? g + (size_t)row0 * ld + k0 : g + (size_t)k0 * ld + row0;
    uint32_t off = voff + (uint32_t)i * vstep;
    int range = 0x7fffffff;
    if constexpr (MASKED) {
      const long long span = KMAJ ? (long long)(nrows - row0 - 1) * ld + (K - k0)
                                  : (long long)(K - k0 - 1) * ld + (nrows - row0);
      range = (int)(span * 2 < 0x7fffffffLL ? span * 2 : 0x7fffffffLL);
      const bool in = KMAJ ? (k0 + lcol < K) : (row0 + lcol < nrows);
      off = in ? off : 0x80000000u;
    }
    char* dst = smem_base + stage + (4 * i + w) * 1024;
    dma16(base, (uint32_t)range, off, dst);
  }
};

// K-major fragment offset: LDS row `row`, k half hh of k-step 0 (k-step 1: XOR 32).
__device__ __forceinline__ int kmaj_frag_off(int row, int hh) { return row * 64 + ((hh ^ kswz(row)) << 4); }

// Workgroup barrier that does not wait for DMA in flight (see wait_vmcnt).
__device__ __forceinline__ void stage_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <bool WK, class Epi>
__global__ void __launch_bounds__(NT, 2) gemm_epi_kernel_occ2(const Problem p, const Epi epi) {
  constexpr int WGF = 2;                    // 2 x 2 waves
  constexpr int WF = BF / 2, WT = BT / 2;   // 128 x 64 per wave
  static_assert(WF == WAVE_F, "row partials assume 128-feature wave tiles");
  constexpr int RI = WF / 32, CI = WT / 32;
  using OA = Operand<BF, WK, true>;
  using OB = Operand<BT, true, false>;
  constexpr int A_REG = OA::REGION, B_REG = OB::REGION, B_OFF = NSTAGE * A_REG;
  __shared__ __attribute__((aligned(1024))) char smem[NSTAGE * (A_REG + B_REG)];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wf = wave % WGF, wt = wave / WGF;
  const int lt = lane & 31, hh = lane >> 5;
  int tf, tt;
  tile_coords(blockIdx.x, gridDim.x, p.nTF, p.nTT, tf, tt);
  const int f0 = p.f_base + tf * BF, t0 = tt * BT;

  f32x16 acc[RI][CI];
#pragma unroll
  for (int i = 0; i < RI; ++i)
#pragma unroll
    for (int j = 0; j < CI; ++j) acc[i][j] = (f32x16){};

  int a_off[RI], b_off[CI];
#pragma unroll
  for (int i = 0; i < RI; ++i)
    a_off[i] = WK ? kmaj_frag_off(wf * WF + i * 32 + lt, hh) : mnmaj_frag_off<true>(wf * WF + i * 32, lane);
#pragma unroll
  for (int j = 0; j < CI; ++j) b_off[j] = B_OFF + kmaj_frag_off(wt * WT + j * 32 + lt, hh);

  OA oa;
  OB ob;
  oa.init(p.ldw, wave, lane);
  ob.init(p.ldx, wave, lane);

  const int nk = (p.K + BK - 1) / BK;
  const bool interior = f0 + BF <= p.F && t0 + BT <= p.T && p.K % BK == 0;

  constexpr int NP = RI * CI / 2;           // MFMA pairs per k-step (4)
  constexpr int NRA = WK ? RI : 2 * RI;     // LDS reads for operand A per k-step
  constexpr int NRD = NRA + CI;
  constexpr int RPP = (NRD + NP - 1) / NP;
  constexpr int HP = 1;                     // pairs of k-step 1 before the barrier
  constexpr int RPH = (NRD + (NP - HP) - 1) / (NP - HP);
  constexpr int NDMA = OA::NCH + OB::NCH;   // DMA instructions per k-tile and thread (6)
  constexpr int DPP = (NDMA + NP - 1) / NP;
  static_assert(NDMA * (NSTAGE - 2) < 64, "pipeline depth");

  bf16x8 fa0[RI], fb0[CI], fa1[RI], fb1[CI];

  auto read_one = [&](int sa, int sb, int s, int n, bf16x8 (&a)[RI], bf16x8 (&b)[CI]) {
    if (n >= NRD) return;
    int q, u = 0;
    {
      const int na = WK ? 1 : 2;
      if (n < na) {
        q = 0;
        u = n;
      } else if (n < na + CI) {
        q = RI + (n - na);
      } else {
        q = 1 + (n - na - CI) / na;
        u = (n - na - CI) % na;
      }
    }
    typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
    if (q < RI) {
      if constexpr (WK) {
        a[q] = __builtin_bit_cast(bf16x8, ld16(smem + ((a_off[q] ^ (s << 5)) + sa)));
      } else {
        const bf16x4 h = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (__attribute__((address_space(3))) bf16x4*)(lds_ptr_t)(smem + a_off[q] + sa + (16 * s + 4 * u) * 512));
#pragma unroll
        for (int e = 0; e < 4; ++e) a[q][4 * u + e] = h[e];
      }
    } else {
      const int j = q - RI;
      b[j] = __builtin_bit_cast(bf16x8, ld16(smem + ((b_off[j] ^ (s << 5)) + sb)));
    }
  };
  auto mfma_pair = [&](const bf16x8 (&a)[RI], const bf16x8 (&b)[CI], int pr) {
    constexpr int JP = CI / 2;
    const int i = pr / JP, j = 2 * (pr % JP);
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    acc[i][j + 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j + 1], acc[i][j + 1], 0, 0, 0);
  };

  // Pipeline (k-tile j in stage j % NSTAGE): the DMA of k-tile kt+NSTAGE-1
  // is issued during k-step 0 of k-tile kt into the stage k-tile kt-1
  // released at the previous barrier; halfway through k-step 1 each wave
  // waits for its DMA of k-tile kt+1 (NSTAGE-2 newer k-tiles may stay in
  // flight) and its LDS reads, then the barrier publishes stage (kt+1).
  auto mainloop = [&](auto masked_c) {
    constexpr bool MASKED = decltype(masked_c)::value;
    auto dma = [&](int kt, int st, int d) {
      const int k0 = kt * BK;
      if (d < OA::NCH)
        oa.template dma<MASKED>(p.W, p.ldw, f0, p.F, k0, p.K, smem, st * A_REG, wave, d);
      else if (d < NDMA)
        ob.template dma<MASKED>(p.X, p.ldx, t0, p.T, k0, p.K, smem + B_OFF, st * B_REG, wave, d - OA::NCH);
    };
    auto wait_tiles = [&](int newer) {  // at most `newer` k-tiles of DMA outstanding
      if (newer <= 0)
        wait_vm<0>();
      else
        wait_vm<NDMA>();
    };
    static_assert(NSTAGE == 3, "wait_tiles covers 0 or 1 newer k-tiles");

    if (nk == 0) return;
#pragma unroll
    for (int j = 0; j < NSTAGE - 1; ++j) {
      if (j < nk) {
#pragma unroll
        for (int d = 0; d < NDMA; ++d) dma(j, j, d);
      }
    }
    wait_tiles(nk - 1 < NSTAGE - 2 ? nk - 1 : NSTAGE - 2);
    stage_barrier();
#pragma unroll
    for (int n = 0; n < NRD; ++n) read_one(0, 0, 0, n, fa0, fb0);

    int st_cur = 0;
    auto ktile = [&](int kt, auto full_c) {
      constexpr bool FULL = decltype(full_c)::value;  // kt + NSTAGE - 1 < nk
      const int st_nxt = st_cur + 1 == NSTAGE ? 0 : st_cur + 1;
      const int st_dma = st_cur == 0 ? NSTAGE - 1 : st_cur - 1;
      const bool do_dma = FULL || kt + NSTAGE - 1 < nk;
      const bool has_next = FULL || kt + 1 < nk;
      const int sa = st_cur * A_REG, sb = st_cur * B_REG;
#pragma unroll
      for (int pr = 0; pr < NP; ++pr) {
        mfma_pair(fa0, fb0, pr);
#pragma unroll
        for (int r = 0; r < RPP; ++r) read_one(sa, sb, 1, pr * RPP + r, fa1, fb1);
        if (do_dma) {
#pragma unroll
          for (int r = 0; r < DPP; ++r) dma(kt + NSTAGE - 1, st_dma, pr * DPP + r);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int pr = 0; pr < HP; ++pr) {
        mfma_pair(fa1, fb1, pr);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (has_next) {
        if constexpr (FULL)
          wait_vm<(NSTAGE - 2) * NDMA>();
        else
          wait_tiles(nk - kt - 2);
        stage_barrier();
      }
      __builtin_amdgcn_sched_barrier(0);
      const int na = st_nxt * A_REG, nb = st_nxt * B_REG;
#pragma unroll
      for (int pr = HP; pr < NP; ++pr) {
        mfma_pair(fa1, fb1, pr);
        if (has_next) {
#pragma unroll
          for (int r = 0; r < RPH; ++r) read_one(na, nb, 0, (pr - HP) * RPH + r, fa0, fb0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      st_cur = st_nxt;
    };
    int kt = 0;
    for (; kt + NSTAGE - 1 < nk; ++kt) ktile(kt, std::true_type{});
    for (; kt < nk; ++kt) ktile(kt, std::false_type{});
  };
  if (interior)
    mainloop(std::false_type{});
  else
    mainloop(std::true_type{});

  // 24 wait states between the last MFMA and the epilogue's inline-asm AGPR
  // reads (the compiler's hazard check does not see inline assembly).
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
  epi.template apply<RI, CI>(acc, g);
}

}  // namespace occ2
}  // namespace coda
