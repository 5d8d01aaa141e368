// coda_epilogues.hpp - epilogue functors of the CODA GEMM-epilogue calls.
//
// Each functor receives the wave's fp32 accumulators in the layout documented
// in coda_mainloop.hpp (lane = one token; accumulator element 8*half + e of
// block (ri, ci) = feature fw0 + 32 ri + 16 half + 8 (lane/32) + e) and turns
// them into the call's outputs before anything is written to global memory.
// They are the five primitive classes of the reading notes "CODA
// GEMM-Epilogue Programming" section 1: element/pairwise maps, vector loads
// (gamma, r, s, lse, labels, positions), tile loads (z, u, dRes, pre), tile
// reductions (sum of squares, the s statistic, dgamma column sums) and
// stateful transforms (running max / sum-exp of the cross-entropy).
//
// Memory access.  Every tile load and store goes through a raw buffer
// descriptor based at the wave tile's origin; an access outside the matrix
// (token >= M or feature >= N) uses an offset beyond the descriptor range,
// for which the hardware returns zeros (loads) or drops the write (stores).
// The epilogues are therefore branch-free: a functor first issues all its
// tile loads (or those of the next 32-token column, for functors that read
// two tiles), then computes and stores, so load latencies overlap instead of
// adding up.
#pragma once

#include "coda_mainloop.hpp"

namespace coda {

constexpr float LOG2E = 1.4426950408889634f;
constexpr uint32_t OOB = 0x80000000u;  // an offset beyond every descriptor range

__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * LOG2E); }
__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.0f + fast_exp(-x)); }

// Sum over the two lanes (l, l^32) that hold the same token.
__device__ __forceinline__ float sum_halves(float v) { return v + __shfl_xor(v, 32); }

// A row-major matrix restricted to one wave tile: element (t, f) of the tile
// (t = token offset, f = feature offset from the wave tile origin).
template <int ESIZE>
struct TileView {
  __amdgpu_buffer_rsrc_t rs;
  int ld;
  __device__ __forceinline__ TileView(const void* base, int ld_, int t0, int f0) : ld(ld_) {
    const char* b = reinterpret_cast<const char*>(base) + ((size_t)t0 * ld_ + f0) * ESIZE;
    rs = __builtin_amdgcn_make_buffer_rsrc((void*)b, (short)0, 0x7fffffff, 0x00020000);
  }
  __device__ __forceinline__ uint32_t off(int t, int f, bool ok) const {
    return ok ? (uint32_t)(t * ld + f) * (uint32_t)ESIZE : OOB;
  }
  __device__ __forceinline__ u32x4 load16(int t, int f, bool ok) const {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off(t, f, ok), 0, 0));
  }
  __device__ __forceinline__ void store16(int t, int f, bool ok, u32x4 v) const {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, off(t, f, ok), 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
  // Non-temporal store (output streamed once, not re-read by this kernel).
  __device__ __forceinline__ void store16_nt(int t, int f, bool ok, u32x4 v) const {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, off(t, f, ok), 0, 2);
    __builtin_amdgcn_sched_barrier(0);
  }
  __device__ __forceinline__ void store8(int t, int f, bool ok, u32x2 v) const {
    __builtin_amdgcn_raw_buffer_store_b64(v, rs, off(t, f, ok), 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
};

// Lane geometry inside the wave tile.
struct Lane {
  int T, F;       // tokens / features remaining from the wave tile origin
  int lt, hh;
  __device__ __forceinline__ Lane(const Geom& g) : T(g.T - g.tw0), F(g.F - g.fw0), lt(g.lt), hh(g.hh) {}
  __device__ __forceinline__ int t(int ci) const { return ci * 32 + lt; }
  __device__ __forceinline__ int f(int ri, int half) const { return ri * 32 + half * 16 + hh * 8; }
  __device__ __forceinline__ bool tok(int ci) const { return t(ci) < T; }
  __device__ __forceinline__ bool ok(int ci, int ri, int half) const { return t(ci) < T && f(ri, half) < F; }
};

// Vector element loads with the index clamped into range (always valid).
template <class T_>
__device__ __forceinline__ T_ vload(const T_* v, int i, int n) { return v[i < n ? i : n - 1]; }
__device__ __forceinline__ u32x4 vload16_bf16(const uint16_t* v, int i, int n) {
  return ld16(v + (i < n ? i : n - 8));
}

// Eight consecutive fp32 vector entries v[f .. f+7] (f clamped into range;
// n % 8 == 0), or zeros when v is NULL (a uniform branch).
__device__ __forceinline__ void load8f(const float* v, int f, int n, float (&o)[8]) {
  if (v == nullptr) {
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = 0.0f;
    return;
  }
  const float* p = v + (f < n ? f : n - 8);
  const f32x4 a = *reinterpret_cast<const f32x4*>(p), b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[e] = a[e];
    o[4 + e] = b[e];
  }
}

// Eight fp32 values from 32 bytes of LDS.
__device__ __forceinline__ void unpack_f32x8(const char* p, float (&o)[8]) {
  const f32x4 a = __builtin_bit_cast(f32x4, ld16(p)), b = __builtin_bit_cast(f32x4, ld16(p + 16));
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    o[e] = a[e];
    o[4 + e] = b[e];
  }
}

// The LayerNorm form of GEMM2's delayed row transform (the mean-corrected
// commutation of LayerNorm with the projection W): with h3 = (u * gamma) W
// in the accumulator, y = r (h3 - mu c) + b, c = gamma^T W, b = beta^T W.
__device__ __forceinline__ void ln_row(float (&v)[8], float r, float mu, const float (&c)[8], const float (&b)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = fmaf(r, fmaf(-mu, c[e], v[e]), b[e]);
}

// Eight accumulator elements of block (ri, ci), copied from their AGPRs at
// this point of the program.  Left to itself the register allocator copies
// all 256 accumulators into VGPRs where the main loop ends, which takes every
// VGPR and makes the epilogue spill; the explicit per-element reads (volatile,
// so they keep their place between the stores) avoid that.
template <int RI, int CI>
__device__ __forceinline__ void acc8(const f32x16 (&acc)[RI][CI], int ri, int ci, int half, float (&v)[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v[e]) : "a"(acc[ri][ci][8 * half + e]));
}

// A wave's bf16 output tile (CI x 32 tokens x 128 features) staged through
// the wave's 32 KiB slice of the LDS the main loop has released.  put()
// writes one lane-layout run (8 features of one token); flush() reads whole
// rows back and stores each as one 256-byte segment, four rows per
// instruction, so global stores cover whole rows instead of 16-byte pieces
// of 32 rows.  Chunk c (8 features) of row r sits at position c ^ (r & 15):
// both access patterns are free of bank conflicts.  Writes and reads are
// the same wave's, which the LDS serves in order.
constexpr int STAGE_LDS = 4 * 32768;  // bytes for the four waves

struct Stage {
  char* reg;
  __device__ __forceinline__ explicit Stage(char* smem)
      : reg(smem + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) * 32768) {}
  __device__ __forceinline__ void put(const Geom& g, int ci, int ri, int h, u32x4 v) const {
    const int r = ci * 32 + g.lt, c = 4 * ri + 2 * h + g.hh;
    st16(reg + r * 256 + ((c ^ (r & 15)) << 4), v);
  }
  // NT: non-temporal stores, for large outputs that this kernel streams
  // out once and that would otherwise displace the GEMM operands.
  template <int CI, bool NT = false>
  __device__ __forceinline__ void flush(const Geom& g, const TileView<2>& out) const {
    const int T = g.T - g.tw0, F = g.F - g.fw0;
    const int rlo = g.lane >> 4, pos = g.lane & 15;
#pragma unroll
    for (int i0 = 0; i0 < CI * 8; i0 += 8) {
      u32x4 sv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) sv[i] = ld16(reg + (i0 + i) * 1024 + 16 * g.lane);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 4 * (i0 + i) + rlo, c = pos ^ (r & 15);
        if constexpr (NT)
          out.store16_nt(r, 8 * c, r < T && 8 * c < F, sv[i]);
        else
          out.store16(r, 8 * c, r < T && 8 * c < F, sv[i]);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Store-only / row-scale / residual epilogue:  Y = bf16( r_t * acc + res )
// (plain GEMM; GEMM2's delayed RMSNorm scale; data-gradient + residual)
// ---------------------------------------------------------------------------
// LN: the LayerNorm form of the delayed transform (ln_row), with per-token
// mu and per-feature c = gamma^T W, b = beta^T W (b may be NULL).
template <bool HAS_R, bool HAS_RES, bool LN = false>
struct EpiLinear {
  const float* r;
  const uint16_t* res;
  int ldres;
  uint16_t* Y;
  int ldy;
  const float* mu = nullptr;
  const float* cvec = nullptr;
  const float* bvec = nullptr;

  static constexpr int LDS_BYTES = STAGE_LDS;

  template <int RI, int CI>
  __device__ __forceinline__ void apply(const f32x16 (&acc)[RI][CI], const Geom& g, char* smem) const {
    const Lane L(g);
    const Stage stage(smem);
    const TileView<2> y(Y, ldy, g.tw0, g.fw0);
    float rsv[CI];
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) rsv[ci] = HAS_R ? vload(r, g.tw0 + L.t(ci), g.T) : 1.0f;
    u32x4 rv[CI][RI][2];
    if constexpr (HAS_RES) {
      const TileView<2> rz(res, ldres, g.tw0, g.fw0);
#pragma unroll
      for (int ci = 0; ci < CI; ++ci)
#pragma unroll
        for (int ri = 0; ri < RI; ++ri)
#pragma unroll
          for (int h = 0; h < 2; ++h) rv[ci][ri][h] = rz.load16(L.t(ci), L.f(ri, h), L.ok(ci, ri, h));
    }
    if constexpr (LN) {
      // feature runs outer, so c and b are loaded once per run
      float mus[CI];
#pragma unroll
      for (int ci = 0; ci < CI; ++ci) mus[ci] = vload(mu, g.tw0 + L.t(ci), g.T);
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float cv[8], bv[8];
          load8f(cvec, g.fw0 + L.f(ri, h), g.F, cv);
          load8f(bvec, g.fw0 + L.f(ri, h), g.F, bv);
#pragma unroll
          for (int ci = 0; ci < CI; ++ci) {
            float v[8];
            acc8(acc, ri, ci, h, v);
            ln_row(v, rsv[ci], mus[ci], cv, bv);
            if constexpr (HAS_RES) {
              float z[8];
              unpack8(rv[ci][ri][h], z);
#pragma unroll
              for (int e = 0; e < 8; ++e) v[e] += z[e];
            }
            stage.put(g, ci, ri, h, pack8(v));
          }
        }
    } else {
#pragma unroll
      for (int ci = 0; ci < CI; ++ci) {
        const float rs = rsv[ci];
#pragma unroll
        for (int ri = 0; ri < RI; ++ri)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            float v[8];
            acc8(acc, ri, ci, h, v);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] *= rs;
            if constexpr (HAS_RES) {
              float z[8];
              unpack8(rv[ci][ri][h], z);
#pragma unroll
              for (int e = 0; e < 8; ++e) v[e] += z[e];
            }
            stage.put(g, ci, ri, h, pack8(v));
          }
      }
    }
    stage.flush<CI, HAS_RES>(g, y);  // residual-stream outputs: non-temporal
  }
};

// ---------------------------------------------------------------------------
// GEMM1 of GEMM -> residual -> RMSNorm -> GEMM (notes sec. 2; paper Fig. 4,
// Listing 2): u = acc + z; U = bf16(u); H2 = bf16(u * gamma);
// part[t, pf] = sum over the wave's features of u^2 (unscaled, fp32).
// ---------------------------------------------------------------------------
// LN: instead of the sum of squares, the LayerNorm statistics of the wave
// tile: part = the tile's mean of u, part2 = its sum of squared deviations
// from that mean (runs of 8 features, each exact in two passes, merged with
// the pairwise-update formula of Chan, Golub and LeVeque).
template <bool HAS_Z, bool HAS_H2, bool HAS_PART, bool LN = false>
struct EpiResSumsq {
  const uint16_t* z;
  int ldz;
  const uint16_t* gamma;
  uint16_t* U;
  int ldu;
  uint16_t* H2;
  int ldh;
  float* part;
  int nparts;
  float* part2 = nullptr;

  static constexpr int LDS_BYTES = STAGE_LDS;

  // u goes out through the LDS stage (whole-row stores); h2, formed from the
  // same unrounded u, is stored directly.
  template <int RI, int CI>
  __device__ __forceinline__ void apply(const f32x16 (&acc)[RI][CI], const Geom& g, char* smem) const {
    const Lane L(g);
    const Stage stage(smem);
    const TileView<2> uo(U, ldu, g.tw0, g.fw0);
    u32x4 gv[RI][2];
    if constexpr (HAS_H2) {
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int h = 0; h < 2; ++h) gv[ri][h] = vload16_bf16(gamma, g.fw0 + L.f(ri, h), g.F);
    }
    // The wave's whole z tile, loaded before anything else is stored.
    const TileView<2> zi(z, ldz, g.tw0, g.fw0);
    u32x4 zv[CI][RI][2];
    if constexpr (HAS_Z) {
#pragma unroll
      for (int ci = 0; ci < CI; ++ci)
#pragma unroll
        for (int ri = 0; ri < RI; ++ri)
#pragma unroll
          for (int h = 0; h < 2; ++h) zv[ci][ri][h] = zi.load16(L.t(ci), L.f(ri, h), L.ok(ci, ri, h));
    }
    auto u8 = [&](int ci, int ri, int h, float (&v)[8]) {
      acc8(acc, ri, ci, h, v);
      if constexpr (HAS_Z) {
        float zz[8];
        unpack8(zv[ci][ri][h], zz);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] += zz[e];
      }
    };
    const TileView<2> ho(H2, ldh, g.tw0, g.fw0);
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) {
      float ss = 0.0f;
      float na = 0.0f, ma = 0.0f;  // LN: count and mean of the runs merged so far (M2 in ss)
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bool ok = L.ok(ci, ri, h);
          float v[8];
          u8(ci, ri, h, v);
          stage.put(g, ci, ri, h, pack8(v));
          if constexpr (LN) {
            float sm = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) sm += v[e];
            const float mb = sm * 0.125f;
            float m2b = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) m2b = fmaf(v[e] - mb, v[e] - mb, m2b);
            const float nb = ok ? 8.0f : 0.0f, nn = na + nb;
            const float w = nn > 0.0f ? nb / nn : 0.0f, dl = mb - ma;
            ma = fmaf(dl, w, ma);
            ss += (ok ? m2b : 0.0f) + dl * dl * na * w;
            na = nn;
          } else {
            float sq = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) sq += v[e] * v[e];
            ss += ok ? sq : 0.0f;
          }
          if constexpr (HAS_H2) {
            float gm[8], hv[8];
            unpack8(gv[ri][h], gm);
#pragma unroll
            for (int e = 0; e < 8; ++e) hv[e] = v[e] * gm[e];
            ho.store16(L.t(ci), L.f(ri, h), ok, pack8(hv));
          }
        }
      if constexpr (LN) {
        // merge with the other half of the token's 128 features (lane l ^ 32)
        const float nb = __shfl_xor(na, 32), mb = __shfl_xor(ma, 32), m2b = __shfl_xor(ss, 32);
        const float nn = na + nb;
        const float w = nn > 0.0f ? nb / nn : 0.0f, dl = mb - ma;
        const float mt = fmaf(dl, w, ma), m2t = ss + m2b + dl * dl * na * w;
        const bool wr = g.hh == 0 && L.tok(ci) && L.F > 0;
        const int t = g.tw0 + L.t(ci);
        if (wr) {
          part[(size_t)t * nparts + g.pf] = mt;
          part2[(size_t)t * nparts + g.pf] = m2t;
        }
      } else if constexpr (HAS_PART) {
        ss = sum_halves(ss);
        const bool w = g.hh == 0 && L.tok(ci) && L.F > 0;
        const int t = g.tw0 + L.t(ci);
        if (w) part[(size_t)t * nparts + g.pf] = ss;
      }
    }
    stage.flush<CI>(g, uo);
  }
};

// ---------------------------------------------------------------------------
// RoPE pair map (paper Fig. 7; RoFormer): t = r * acc, then rotate each
// adjacent pair (c, c+1), c < n_rope, by pos * theta^(-2k/hd), k = (c mod hd)/2.
// INV applies the inverse rotation (backward epilogue).
// ---------------------------------------------------------------------------
template <bool HAS_R, bool INV>
struct EpiRope {
  const float* r;
  const int32_t* pos;
  float log2_theta;  // log2(theta)
  int head_dim;
  int n_rope;
  uint16_t* Y;
  int ldy;

  static constexpr int LDS_BYTES = STAGE_LDS;

  template <int RI, int CI>
  __device__ __forceinline__ void apply(const f32x16 (&acc)[RI][CI], const Geom& g, char* smem) const {
    const Lane L(g);
    const Stage stage(smem);
    const TileView<2> y(Y, ldy, g.tw0, g.fw0);
    float rsv[CI], psv[CI];
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) {
      const int t = g.tw0 + L.t(ci);
      rsv[ci] = HAS_R ? vload(r, t, g.T) : 1.0f;
      psv[ci] = (float)vload(pos, t, g.T);
    }
    // Per-lane frequencies in revolutions per position: theta^(-2k/hd) / (2 pi);
    // 0 for pass-through columns (angle 0 rotates by the identity).
    // The pair at column c = f + 2q (f a multiple of 8) has 2k = c mod head_dim:
    // one modulo per 8-column run, then at most three wraps (head_dim >= 2).
    constexpr float INV_2PI = 0.15915494309189535f;
    const float c_exp = log2_theta / (float)head_dim;
    float fr[RI][2][4];
#pragma unroll
    for (int ri = 0; ri < RI; ++ri)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int f = g.fw0 + L.f(ri, h);
        const int base = f % head_dim;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int j = base + 2 * q;
          j -= j >= head_dim ? head_dim : 0;
          j -= j >= head_dim ? head_dim : 0;
          j -= j >= head_dim ? head_dim : 0;
          const float w = exp2f(-(float)j * c_exp) * INV_2PI;
          fr[ri][h][q] = f < n_rope ? w : 0.0f;
        }
      }
    // One 32-token column.  P = 0: the wave tile lies past n_rope (scale
    // only).  Otherwise sine and cosine are evaluated for ri < P and reused
    // for ri + P, ri + 2P, ...: the lane's features f and f + 32 P have the
    // same angle when head_dim divides 32 P and the whole wave tile is
    // rotated (head_dim 64: two heads per 128-feature wave tile, P = 2).
    auto column = [&](int ci, auto p_c) {
      constexpr int P = decltype(p_c)::value;
      const float rs = rsv[ci], ps = psv[ci];
      float sn[P > 0 ? P : 1][2][4], cs[P > 0 ? P : 1][2][4];
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float v[8];
          acc8(acc, ri, ci, h, v);
          if constexpr (P == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] *= rs;
          } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              if (ri < P) {
                float rev = ps * fr[ri][h][q];
                rev -= floorf(rev);
                sn[ri][h][q] = INV ? -__builtin_amdgcn_sinf(rev) : __builtin_amdgcn_sinf(rev);
                cs[ri][h][q] = __builtin_amdgcn_cosf(rev);
              }
              const float sq = sn[ri % P][h][q], cq = cs[ri % P][h][q];
              const float a = v[2 * q] * rs, b = v[2 * q + 1] * rs;
              v[2 * q] = a * cq - b * sq;
              v[2 * q + 1] = a * sq + b * cq;
            }
          }
          stage.put(g, ci, ri, h, pack8(v));
        }
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    using PR = std::integral_constant<int, RI>;
    const bool whole = g.fw0 + 32 * RI <= n_rope;
    if (g.fw0 >= n_rope) {
#pragma unroll
      for (int ci = 0; ci < CI; ++ci) column(ci, P0{});
    } else if (whole && 32 % head_dim == 0) {
#pragma unroll
      for (int ci = 0; ci < CI; ++ci) column(ci, P1{});
    } else if (whole && 64 % head_dim == 0) {
#pragma unroll
      for (int ci = 0; ci < CI; ++ci) column(ci, P2{});
    } else {
#pragma unroll
      for (int ci = 0; ci < CI; ++ci) column(ci, PR{});
    }
    stage.flush<CI>(g, y);
  }
};

// The SwiGLU output tile (CI x 32 tokens x 64 act columns, 128-byte rows)
// staged the same way through the wave's LDS slice: chunk c (8 columns) of
// row r sits at position c ^ (r & 7); flush() stores eight whole rows per
// instruction, non-temporal.  Fa = act columns left from the wave tile
// origin (a multiple of 4: the last chunk may hold only 4 valid columns).
struct StageAct {
  char* reg;
  __device__ __forceinline__ explicit StageAct(char* smem)
      : reg(smem + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) * 32768) {}
  __device__ __forceinline__ void put(const Geom& g, int ci, int ri, u32x4 v) const {
    const int r = ci * 32 + g.lt, c = 2 * ri + g.hh;
    st16(reg + r * 128 + ((c ^ (r & 7)) << 4), v);
  }
  template <int CI>
  __device__ __forceinline__ void flush(const Geom& g, const TileView<2>& out, int Fa) const {
    const int T = g.T - g.tw0;
    const int rlo = g.lane >> 3, pos = g.lane & 7;
#pragma unroll
    for (int i0 = 0; i0 < CI * 4; i0 += 8) {
      u32x4 sv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) sv[i] = ld16(reg + (i0 + i) * 1024 + 16 * g.lane);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 8 * (i0 + i) + rlo, c = pos ^ (r & 7);
        const bool full = r < T && 8 * c + 8 <= Fa;
        const bool half = r < T && 8 * c + 4 <= Fa && !full;
        out.store16_nt(r, 8 * c, full, sv[i]);
        out.store8(r, 8 * c, half, (u32x2){sv[i][0], sv[i][1]});
      }
    }
  }
};

// ---------------------------------------------------------------------------
// SwiGLU pair map 2 -> 1 (paper Fig. 7): (g, v) = r * (acc_2j, acc_2j+1),
// a_j = g sigmoid(g) v; optional Pre = bf16(g, v) for the backward pass.
// The GEMM's feature space is the interleaved 2F columns.
// ---------------------------------------------------------------------------
// LN: the pre-activation is the LayerNorm form r (acc - mu c) + b (ln_row)
// over the interleaved 2F columns, c = gamma^T Wgu, b = beta^T Wgu.
template <bool HAS_R, bool HAS_PRE, bool LN = false>
struct EpiSwiglu {
  const float* r;
  uint16_t* act;
  int ldact;
  uint16_t* pre;
  int ldp;
  const float* mu = nullptr;
  const float* cvec = nullptr;
  const float* bvec = nullptr;

  // pre (when kept) and then act leave through the released LDS.
  static constexpr int LDS_BYTES = STAGE_LDS;

  template <int RI, int CI>
  __device__ __forceinline__ void apply(const f32x16 (&acc)[RI][CI], const Geom& g, char* smem) const {
    const Lane L(g);
    const TileView<2> ao(act, ldact, g.tw0, g.fw0 >> 1);
    const TileView<2> po(pre, ldp, g.tw0, g.fw0);
    const StageAct sa(smem);
    float rsv[CI], mus[CI];
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) {
      rsv[ci] = HAS_R ? vload(r, g.tw0 + L.t(ci), g.T) : 1.0f;
      mus[ci] = LN ? vload(mu, g.tw0 + L.t(ci), g.T) : 0.0f;
    }
    u32x4 aout[CI][RI];
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) {
      const float rs = rsv[ci];
#pragma unroll
      for (int ri = 0; ri < RI; ++ri) {
        // a-columns of this lane: 16 ri + 8 h + 4 hh + q (q = 0..3) for half h
        u32x2 ah[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float v[8];
          acc8(acc, ri, ci, h, v);
          if constexpr (LN) {
            float cv[8], bv[8];
            load8f(cvec, g.fw0 + L.f(ri, h), g.F, cv);
            load8f(bvec, g.fw0 + L.f(ri, h), g.F, bv);
            ln_row(v, rs, mus[ci], cv, bv);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] *= rs;
          }
          float a[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float gg = v[2 * q], uu = v[2 * q + 1];
            a[q] = gg * sigmoidf_(gg) * uu;
          }
          ah[h] = (u32x2){pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
          if constexpr (HAS_PRE) Stage(smem).put(g, ci, ri, h, pack8(v));
        }
        // Exchange with lane l ^ 32 so that each lane holds 8 consecutive
        // a-columns (16 ri + 8 hh + 0..7).
        const u32x2 give = g.hh ? ah[0] : ah[1];
        const u32x2 got = {(uint32_t)__shfl_xor((int)give[0], 32), (uint32_t)__shfl_xor((int)give[1], 32)};
        aout[ci][ri] = g.hh ? (u32x4){got[0], got[1], ah[1][0], ah[1][1]}
                            : (u32x4){ah[0][0], ah[0][1], got[0], got[1]};
        if constexpr (!HAS_PRE) sa.put(g, ci, ri, aout[ci][ri]);
      }
    }
    if constexpr (HAS_PRE) {
      // The slice is free again once flush() has its rows back in registers
      // (its stores consume them; the LDS serves one wave's accesses in
      // order); then act takes it.
      Stage(smem).flush<CI, true>(g, po);
#pragma unroll
      for (int ci = 0; ci < CI; ++ci)
#pragma unroll
        for (int ri = 0; ri < RI; ++ri) sa.put(g, ci, ri, aout[ci][ri]);
    }
    sa.flush<CI>(g, ao, L.F >> 1);
  }
};

// ---------------------------------------------------------------------------
// LM-head cross-entropy statistics (notes sec. 2 "Cross-entropy loss"):
// per (token, wave feature tile) running max m and sum exp(l - m) of the fp32
// logits, plus the gathered target logit.  The statistics come from the fp32
// logits; KEEP also writes the logits rounded to bf16 (through the released
// LDS, whole rows per store), for a backward that does not recompute them.
// ---------------------------------------------------------------------------
template <bool KEEP>
struct EpiCE {
  const int32_t* labels;
  float* part_m;  // [nparts x ldpart], ldpart >= M
  float* part_s;
  float* tgt;
  int ldpart;
  uint16_t* logits;  // KEEP: bf16 [M x V], leading dimension ldl
  int ldl;

  static constexpr int LDS_BYTES = KEEP ? STAGE_LDS : 0;

  template <int RI, int CI>
  __device__ __forceinline__ void apply(const f32x16 (&acc)[RI][CI], const Geom& g, char* smem = nullptr) const {
    const Lane L(g);
    [[maybe_unused]] const Stage stage(smem);
    int lab[CI];
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) lab[ci] = vload(labels, g.tw0 + L.t(ci), g.T);
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) {
      const int t = g.tw0 + L.t(ci);
      const bool tok_ok = L.tok(ci);
      // Label position relative to the wave tile: 8-feature group grp (held by
      // this lane when grp == 4 ri + 2 h + hh) and element eo inside it.
      const int rel = tok_ok ? lab[ci] - g.fw0 : -1;
      const int grp = rel >> 3, eo = rel & 7;
      const bool b0 = (eo & 1) != 0, b1 = (eo & 2) != 0, b2 = (eo & 4) != 0;
      float l[RI][2][8];
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          acc8(acc, ri, ci, h, l[ri][h]);
          if constexpr (KEEP) stage.put(g, ci, ri, h, pack8(l[ri][h]));
        }
      // Max and sum-exp per 8-feature group; a group lies entirely inside or
      // entirely past the vocabulary (V % 8 == 0), so masking is per group.
      float m = -INFINITY;
      bool gv[RI][2];
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float gm = l[ri][h][0];
#pragma unroll
          for (int e = 1; e < 8; ++e) gm = fmaxf(gm, l[ri][h][e]);
          gv[ri][h] = L.f(ri, h) < L.F;
          m = gv[ri][h] ? fmaxf(m, gm) : m;
        }
      const float ml = m * LOG2E;
      float s = 0.0f;
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float gs = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) gs += __builtin_amdgcn_exp2f(fmaf(l[ri][h][e], LOG2E, -ml));
          s += gv[ri][h] ? gs : 0.0f;
        }
      // Target gather: the group that holds the label (one compare per
      // group), then its element eo by a 3-level select.
      float gsel[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) gsel[e] = 0.0f;
      bool hit = false;
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bool hg = grp == ri * 4 + h * 2 + g.hh;
#pragma unroll
          for (int e = 0; e < 8; ++e) gsel[e] = hg ? l[ri][h][e] : gsel[e];
          hit = hit || hg;
        }
      const float s01 = b0 ? gsel[1] : gsel[0], s23 = b0 ? gsel[3] : gsel[2];
      const float s45 = b0 ? gsel[5] : gsel[4], s67 = b0 ? gsel[7] : gsel[6];
      const float s03 = b1 ? s23 : s01, s47 = b1 ? s67 : s45;
      const float tv = b2 ? s47 : s03;
      if (hit) tgt[t] = tv;
      // merge the two half-wave states of this token
      const float m2 = __shfl_xor(m, 32), s2 = __shfl_xor(s, 32);
      const float mm = fmaxf(m, m2);
      const float st = (m == -INFINITY ? 0.0f : s * fast_exp(m - mm)) +
                       (m2 == -INFINITY ? 0.0f : s2 * fast_exp(m2 - mm));
      if (g.hh == 0 && tok_ok && L.F > 0) {
        // part-major [nparts x M]: the 32 lanes write 128 contiguous bytes
        part_m[(size_t)g.pf * ldpart + t] = mm;
        part_s[(size_t)g.pf * ldpart + t] = st;
      }
    }
    if constexpr (KEEP) stage.flush<CI, true>(g, TileView<2>(logits, ldl, g.tw0, g.fw0));
  }
};

// ---------------------------------------------------------------------------
// dlogits of the LM-head cross-entropy backward (recomputed logits):
// D = (exp(l - lse_t) - [f == label_t]) * scale, bf16.
// ---------------------------------------------------------------------------
// NT: non-temporal stores (a dlogits buffer too large to stay in the caches);
// temporal when the consumer GEMMs read it back from the Infinity Cache.
// voff: the vocabulary index of the GEMM's feature 0 (vocabulary chunks).
template <bool NT = true>
struct EpiCEBwd {
  const int32_t* labels;
  const float* lse;
  float scale;
  uint16_t* D;
  int ldd;
  int voff = 0;

  static constexpr int LDS_BYTES = STAGE_LDS;

  template <int RI, int CI>
  __device__ __forceinline__ void apply(const f32x16 (&acc)[RI][CI], const Geom& g, char* smem) const {
    const Lane L(g);
    const Stage stage(smem);
    const TileView<2> d(D, ldd, g.tw0, g.fw0);
    int lab[CI];
    float lsev[CI];
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) {
      const int t = g.tw0 + L.t(ci);
      lab[ci] = vload(labels, t, g.T);
      lsev[ci] = vload(lse, t, g.T);
    }
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) {
      const int label = lab[ci] - voff - g.fw0;
      const float Lse = lsev[ci];
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float v[8];
          acc8(acc, ri, ci, h, v);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float pr = fast_exp(v[e] - Lse);
            v[e] = (pr - (label == L.f(ri, h) + e ? 1.0f : 0.0f)) * scale;
          }
          stage.put(g, ci, ri, h, pack8(v));
        }
    }
    stage.flush<CI, NT>(g, d);
  }
};

// ---------------------------------------------------------------------------
// SwiGLU backward pair map 1 -> 2 (paper Fig. 7; notes sec. 3): acc = da_j,
// (g, v) = Pre[2j, 2j+1]; dPre = (da v s (1 + g (1 - s)), da g s);
// spart[t, pf] = sum (dPre_2j g + dPre_2j+1 v)  (RMSNorm statistic partial).
// ---------------------------------------------------------------------------
// LN: the two LayerNorm row statistics of the layer whose output pre is
// (the reading notes' "Eliminating the RMSNorm backward kernel", applied to
// LayerNorm): spart = sum dpre (pre - b) and apart = sum dpre c over the
// wave's columns, c = gamma^T Wgu, b = beta^T Wgu (b may be NULL).
template <bool HAS_SPART, bool LN = false>
struct EpiSwigluBwd {
  const uint16_t* pre;
  int ldp;
  uint16_t* dpre;
  int lddp;
  float* spart;
  int nparts;
  const float* cvec = nullptr;
  const float* bvec = nullptr;
  float* apart = nullptr;

  // The epilogue stages pre and dpre through the LDS the main loop has
  // released (32 KiB per wave, 128 KiB per workgroup); LN adds 2 KiB per wave
  // beyond them for the wave's 256 columns of c and b.
  static constexpr int LDS_BYTES = 4 * 32768 + (LN ? 4 * 2048 : 0);

  // Each wave works on its (32 CI)-token x 256-column pre/dpre tile in CI
  // phases of 32 tokens (16 KiB), double-buffered in its 32 KiB LDS slice:
  // LDS-DMA of whole 512-byte row segments; the pair map in the accumulator
  // layout, reading pre and writing dpre in place; then the rows read back
  // linearly and stored as whole row segments.  Phase p+2's DMA goes into
  // phase p's buffer once its rows are back in registers, before its stores,
  // so each phase's data arrives while the previous phase computes and
  // stores.  Row r keeps its 16-byte chunk c at position c ^ (r & 15): the
  // rows are 512 bytes apart, so every row starts at the same bank, and the
  // 16 rows that one 16-lane phase of an accumulator-layout access touches
  // (one chunk each) then cover all 16 bank groups of 16 bytes.
  //
  // Waits: vmcnt retires vector memory operations, loads and stores alike,
  // in issue order (the compiler's own waits on gfx950 rely on it: a load
  // followed by two stores is awaited with vmcnt(2)).  A phase's DMA is
  // complete once at most the operations issued after it are outstanding:
  // the next phase's DMA and the previous phases' row stores, which stay in
  // flight.  (The s-partial store, when there is one, only makes the wait
  // stricter.)
  template <int RI, int CI>
  __device__ __forceinline__ void apply(const f32x16 (&acc)[RI][CI], const Geom& g, char* smem) const {
    static_assert(CI >= 2, "at least two 32-token phases");
    constexpr int NI = 16;  // DMA / store instructions per phase (2 rows each)
    const Lane L(g);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    char* reg = smem + wave * 32768;
    const uint32_t lreg = lds_addr(reg);
    const int rlo = g.lane >> 5, pos = g.lane & 31;
    const TileView<2> po(dpre, lddp, g.tw0, 2 * g.fw0);
    const int cols = 2 * L.F;  // pre columns left from the wave tile origin
    auto fetch = [&](int p) {
      const uint16_t* base = pre + (size_t)(g.tw0 + 32 * p) * ldp + 2 * g.fw0;
      const uint32_t lbuf = lreg + (uint32_t)((p & 1) * 16384);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int r = 2 * i + rlo, c = pos ^ (r & 15);
        const bool ok = 32 * p + r < L.T && 8 * c < cols;
        dma16<true>(base, 0x7fffffffu, ok ? (uint32_t)(r * ldp + 8 * c) * 2u : OOB, lbuf + (uint32_t)(i * 1024));
      }
    };
    [[maybe_unused]] char* cb = smem + 4 * 32768 + wave * 2048;  // LN: c at [0, 1 KiB), b after it
    if constexpr (LN) {
      // The wave's 256 pre columns of c and b, 4 per lane, loaded before the
      // phase DMAs (so the wait below does not wait for those).
      const int col = 2 * g.fw0 + 4 * g.lane;
      const bool in = col < 2 * g.F;
      const f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
      const f32x4 cq = in ? *reinterpret_cast<const f32x4*>(cvec + col) : zero;
      const f32x4 bq = (in && bvec) ? *reinterpret_cast<const f32x4*>(bvec + col) : zero;
      fetch(0);
      fetch(1);
      st16(cb + 16 * g.lane, __builtin_bit_cast(u32x4, cq));
      st16(cb + 1024 + 16 * g.lane, __builtin_bit_cast(u32x4, bq));
    } else {
      fetch(0);
      fetch(1);
    }
#pragma unroll
    for (int p = 0; p < CI; ++p) {
      // Operations issued after phase p's DMA: p = 0: phase 1's DMA;
      // p = 1: phase 2's DMA (if any) and phase 0's stores; p >= 2 (its DMA
      // went out in phase p-2, before that phase's stores): phase p-2's and
      // p-1's stores and phase p+1's DMA (if any).
      const int later = p == 0 ? (CI > 1 ? NI : 0)
                      : p == 1 ? (CI > 2 ? NI : 0) + NI
                               : 2 * NI + (p + 1 < CI ? NI : 0);
      wait_vmcnt_le(later);
      char* buf = reg + (p & 1) * 16384;
      // dpre from pre and da in the accumulator layout, in place, in two
      // halves of the wave tile's features (ri pairs).  Each half's eight
      // pre chunks are read before any is written back: the writes go to the
      // same buffer, so the compiler keeps a read after an earlier write, and
      // reading chunk by chunk left one LDS round trip per chunk exposed
      // (one wave per SIMD, nothing else to run meanwhile).
      const int ci = p;
      const int r = g.lt;
      float ss = 0.0f, sa = 0.0f;
      static_assert(RI % 2 == 0, "feature halves of whole 32-row blocks");
#pragma unroll
      for (int r0 = 0; r0 < RI; r0 += 2) {
        u32x4 pv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int ri = r0 + (j >> 2), h = (j >> 1) & 1, c = j & 1;
          const int chunk = 8 * ri + 4 * h + 2 * g.hh + c;
          pv[j] = ld16(buf + r * 512 + ((chunk ^ (r & 15)) << 4));
        }
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int ri = r0 + (jj >> 1), h = jj & 1;
          const bool ok = L.ok(ci, ri, h);
          float dav[8];
          acc8(acc, ri, ci, h, dav);
#pragma unroll
          for (int c = 0; c < 2; ++c) {  // two 16-byte chunks = 4 pairs each
            const int chunk = 8 * ri + 4 * h + 2 * g.hh + c;
            char* a = buf + r * 512 + ((chunk ^ (r & 15)) << 4);
            float pvv[8], out[8];
            unpack8(pv[2 * jj + c], pvv);
            float cv[8], bv[8];
            if constexpr (LN) {
              unpack_f32x8(cb + 32 * chunk, cv);
              unpack_f32x8(cb + 1024 + 32 * chunk, bv);
            }
            float part = 0.0f, pa = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float da = dav[4 * c + q];
              const float gg = pvv[2 * q], uu = pvv[2 * q + 1];
              // With t = g sigma(g) (the SiLU): du = da t and
              // dg = da u (sigma + t (1 - sigma)), i.e. silu'(g) = sigma (1 + g (1 - sigma)).
              const float sg = sigmoidf_(gg);
              const float t = gg * sg;
              const float du = da * t;
              const float dg = (da * uu) * (fmaf(-t, sg, t) + sg);
              out[2 * q] = dg;
              out[2 * q + 1] = du;
              if constexpr (LN) {
                part = fmaf(dg, gg - bv[2 * q], fmaf(du, uu - bv[2 * q + 1], part));
                pa = fmaf(dg, cv[2 * q], fmaf(du, cv[2 * q + 1], pa));
              } else {
                part = fmaf(dg, gg, fmaf(du, uu, part));
              }
            }
            ss += ok ? part : 0.0f;
            if constexpr (LN) sa += ok ? pa : 0.0f;
            st16(a, pack8(out));
          }
        }
      }
      if constexpr (HAS_SPART) {
        ss = sum_halves(ss);
        if constexpr (LN) sa = sum_halves(sa);
        const bool w = g.hh == 0 && L.tok(ci) && L.F > 0;
        const int t = g.tw0 + L.t(ci);
        if (w) {
          spart[(size_t)t * nparts + g.pf] = ss;
          if constexpr (LN) apart[(size_t)t * nparts + g.pf] = sa;
        }
      }
      // Whole rows back out: instruction i stores rows 2i and 2i + 1.
      u32x4 sv[NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) sv[i] = ld16(buf + i * 1024 + 16 * g.lane);
      if (p + 2 < CI) {
        wait_lgkmcnt0();  // the buffer is read before the next DMA refills it
        fetch(p + 2);
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int rr = 2 * i + rlo, c = pos ^ (rr & 15);
        po.store16_nt(32 * p + rr, 8 * c, 32 * p + rr < L.T && 8 * c < cols, sv[i]);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// The same SwiGLU backward with the pair map of each tile run inside the next
// tile's k-loop: epilogue/MFMA overlap within one wave (the PingPong-style
// overlap of the epilogue with tensor-core work that the social thread "CODA
// reparameterizes memory-bound operations" names; paper Fig. 3).  A wave's
// 128 x 128 accumulator tile takes all 256 AGPRs, so a second accumulator set
// does not fit; instead the tile's epilogue (EpiSwigluBwdDump) stores da in
// fp32 where dpre will go: the 8 features f..f+7 of one token that a lane
// holds as one accumulator run are 32 bytes of fp32, exactly the 32 bytes of
// their 16 dpre values (columns 2f..2f+15).  The carry (SwigluBwdCarry) then
// runs that tile's pair map in 64 units per wave during the next tile's
// k-loop, U units per k-tile.  A unit is one 16-byte chunk (4 pairs) of one
// run: its da and pre loads go out one k-tile ahead (at the start of k-step
// 2, after the k-loop's wait for all memory operations, which covers the
// previous k-tile's loads), its pair map runs in 8 stages between the MFMA
// pairs of k-steps 2 and 3, and its dpre store and s partial come last.  Each
// lane reads back only what it stored itself, at the same addresses and in
// program order (as a register spill does).  Units beyond what the k-loop
// holds, and the last tile's, run after it.
// ---------------------------------------------------------------------------
struct EpiSwigluBwdDump {
  uint16_t* dpre;
  int lddp;

  template <int RI, int CI>
  __device__ __forceinline__ void apply(const f32x16 (&acc)[RI][CI], const Geom& g) const {
    const Lane L(g);
    const TileView<2> d(dpre, lddp, g.tw0, 2 * g.fw0);
#pragma unroll
    for (int ci = 0; ci < CI; ++ci)
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float v[8];
          acc8(acc, ri, ci, h, v);
          const bool ok = L.ok(ci, ri, h);
          const int col = 2 * L.f(ri, h);
          d.store16(L.t(ci), col, ok,
                    (u32x4){__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])});
          d.store16(L.t(ci), col + 8, ok,
                    (u32x4){__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])});
        }
  }
};

// The carry's arguments: the SwiGLU backward's pre, dpre and spart (nparts
// per token) over F features and T tokens.
struct SwigluBwdCarryArgs {
  const uint16_t* pre;
  int ldp;
  uint16_t* dpre;
  int lddp;
  float* spart;
  int nparts;
  int F, T;
};

template <int U, bool HAS_SPART>
struct SwigluBwdCarry {
  static_assert(U == 1 || U == 2, "units per k-tile");
  static constexpr bool kPersistent = true;
  static constexpr int kPrimeOps = 2 * U;
  // The dpre stores come last in a k-tile (k-step 3's last MFMA pair, after
  // its DMA); the next k-tile's wait need not wait for their completion.
  static constexpr int kTailOps = U;
  static constexpr int UNITS = 64;  // per wave and 256 x 256 tile: 4 x 4 runs x 2 halves x 2 chunks
  using Args = SwigluBwdCarryArgs;

  Args a;
  int lt, hh;
  bool pending;      // a tile's pair map is outstanding
  int tw0, fw0, pf;  // that tile's wave tile
  int lim;           // units the current k-loop carries (the rest: drain)
  __amdgpu_buffer_rsrc_t rp, rd;  // pre / dpre at its origin
  u32x4 bd[U], bp[U];              // the next k-tile's units, in flight: da (fp32), pre (bf16 pairs)
  // This k-tile's 4 U pairs, in flight through the pair map's stages.
  float xa[U][4], xg[U][4], xu[U][4], xs[U][4], xt[U][4], xw[U][4];
  uint32_t ow[U][4];               // dpre, packed
  float pp[U];                     // the units' shares of the s statistic
  float ss;                        // the s partial of the current token column

  __device__ __forceinline__ explicit SwigluBwdCarry(const Args& args) : a(args) {
    const int lane = (int)(threadIdx.x & 63);
    lt = lane & 31;
    hh = lane >> 5;
    pending = false;
    tw0 = fw0 = pf = 0;
    lim = 0;
    ss = 0.0f;
    rp = rd = __builtin_amdgcn_make_buffer_rsrc((void*)a.dpre, (short)0, 0, 0x00020000);
  }

  // Unit u: token column ci, run (ri, half), chunk c (u = 16 ci + 4 ri + 2 half + c).
  __device__ __forceinline__ bool unit(int u, int& t, int& col) const {
    const int ci = (u >> 4) & 3, ri = (u >> 2) & 3, half = (u >> 1) & 1, c = u & 1;
    t = ci * 32 + lt;
    const int f = ri * 32 + half * 16 + hh * 8;
    col = 2 * f + 8 * c;
    return (int)pending & (int)(u < UNITS) & (int)(t < a.T - tw0) & (int)(f < a.F - fw0);
  }
  // An empty asm that takes x and gives it back: the value is computed here
  // (the compiler would otherwise sink the whole pair map to its store, past
  // every MFMA of the k-tile) and later stages cannot move above it.
  __device__ __forceinline__ static void pin(float& x) { asm volatile("" : "+v"(x)); }
  __device__ __forceinline__ static void pin(uint32_t& x) { asm volatile("" : "+v"(x)); }
  // The loads of unit u (none, by out-of-range offsets, beyond `end`).
  __device__ __forceinline__ void load(int u, int end, u32x4& d, u32x4& q) const {
    int t, col;
    const bool ok = (int)unit(u, t, col) & (int)(u < end);
    d = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rd, ok ? (uint32_t)(t * a.lddp + col) * 2u : OOB, 0, 0));
    q = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rp, ok ? (uint32_t)(t * a.ldp + col) * 2u : OOB, 0, 2));
  }
  // Pair map stage k (0..7) of pair i of unit j, with (g, v) the pre pair,
  // da the accumulator value, s = sigmoid(g) and t = g s:
  //   du = da t,  dg = da v (s + t (1 - s)),  part += dg g + du v.
  // Each stage depends only on earlier ones, so stage k of all 4 U pairs are
  // independent instructions and one stage per MFMA pair keeps the wave's
  // in-order issue from waiting on a result.
  template <bool PIN = true>
  __device__ __forceinline__ void stage(int k, int j, int i, const u32x4& d, const u32x4& q) {
    switch (k) {
      case 0:
        xa[j][i] = __uint_as_float(d[i]);
        xg[j][i] = bf_lo(q[i]);
        xu[j][i] = bf_hi(q[i]);
        if (PIN) pin(xa[j][i]), pin(xg[j][i]), pin(xu[j][i]);
        break;
      case 1:
        xs[j][i] = fast_exp(-xg[j][i]);
        if (PIN) pin(xs[j][i]);
        break;
      case 2:
        xs[j][i] = __builtin_amdgcn_rcpf(1.0f + xs[j][i]);
        if (PIN) pin(xs[j][i]);
        break;
      case 3:
        xt[j][i] = xg[j][i] * xs[j][i];
        if (PIN) pin(xt[j][i]);
        break;
      case 4:
        xw[j][i] = fmaf(-xt[j][i], xs[j][i], xt[j][i]);
        if (PIN) pin(xw[j][i]);
        break;
      case 5:
        xw[j][i] += xs[j][i];
        xt[j][i] *= xa[j][i];  // du
        if (PIN) pin(xw[j][i]), pin(xt[j][i]);
        break;
      case 6:
        xw[j][i] *= xa[j][i] * xu[j][i];  // dg
        if (PIN) pin(xw[j][i]);
        break;
      default:
        ow[j][i] = pack_bf16x2(xw[j][i], xt[j][i]);
        pp[j] = fmaf(xw[j][i], xg[j][i], fmaf(xt[j][i], xu[j][i], i == 0 ? 0.0f : pp[j]));
        if (PIN) pin(ow[j][i]), pin(pp[j]);
        break;
    }
  }
  __device__ __forceinline__ void store(int u, const uint32_t (&o)[4], float part) {
    int t, col;
    const bool ok = unit(u, t, col);
    __builtin_amdgcn_raw_buffer_store_b128((u32x4){o[0], o[1], o[2], o[3]}, rd,
                                           ok ? (uint32_t)(t * a.lddp + col) * 2u : OOB, 0, 2);
    if constexpr (HAS_SPART) {
      ss += ok ? part : 0.0f;
      if ((u & 15) == 15) {  // the column's last unit (uniform)
        const float s2 = sum_halves(ss);
        ss = 0.0f;
        if (pending && u < UNITS && hh == 0 && t < a.T - tw0 && a.F - fw0 > 0)
          a.spart[(size_t)(tw0 + t) * a.nparts + pf] = s2;
      }
    }
  }

  // Units 0..U-1 in flight before k-tile 0.
  __device__ __forceinline__ void prime(int nk) {
    lim = nk * U < UNITS ? nk * U : UNITS;
#pragma unroll
    for (int j = 0; j < U; ++j) load(j, lim, bd[j], bp[j]);
  }
  // k-tile kt: at the start of k-step 2 (its loads have landed: the k-loop
  // waited for every memory operation) units kt U + j enter the pair map and
  // the next k-tile's go in flight; pair-map stage k runs at position 2 k of
  // the 16 MFMA pairs of k-steps 2 and 3, the stores at the last.
  __device__ __forceinline__ void slot(int kt, int step, int pr) {
    if (step < 2) return;
    const int pos = (step - 2) * 8 + pr;
    if (pos == 0) {
#pragma unroll
      for (int j = 0; j < U; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) stage(0, j, i, bd[j], bp[j]);
#pragma unroll
      for (int j = 0; j < U; ++j) load((kt + 1) * U + j, lim, bd[j], bp[j]);
    } else if ((pos & 1) == 0) {
#pragma unroll
      for (int j = 0; j < U; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) stage(pos >> 1, j, i, bd[j], bp[j]);
    } else if (pos == 15) {
#pragma unroll
      for (int j = 0; j < U; ++j) store(kt * U + j, ow[j], pp[j]);
    }
  }

  // Units u0 .. UNITS-1 of the pending tile, eight at a time.
  __device__ __forceinline__ void serial(int u0) {
    for (int u = u0; u < UNITS; u += 4 * U) {
      u32x4 d[4][U], q[4][U];
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int j = 0; j < U; ++j) load(u + b * U + j, UNITS, d[b][j], q[b][j]);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
          for (int j = 0; j < U; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) stage<false>(k, j, i, d[b][j], q[b][j]);
#pragma unroll
        for (int j = 0; j < U; ++j) store(u + b * U + j, ow[j], pp[j]);
      }
    }
  }
  __device__ __forceinline__ void drain(int nk) {
    const int done = nk * U < UNITS ? nk * U : UNITS;
    if (pending && done < UNITS) serial(done);
  }
  __device__ __forceinline__ void pend(const Geom& g) {
    pending = true;
    tw0 = g.tw0;
    fw0 = g.fw0;
    pf = g.pf;
    ss = 0.0f;
    rp = __builtin_amdgcn_make_buffer_rsrc((void*)(a.pre + (size_t)tw0 * a.ldp + 2 * fw0), (short)0, 0x7fffffff,
                                           0x00020000);
    rd = __builtin_amdgcn_make_buffer_rsrc((void*)(a.dpre + (size_t)tw0 * a.lddp + 2 * fw0), (short)0, 0x7fffffff,
                                           0x00020000);
  }
  __device__ __forceinline__ void finish() {
    if (pending) serial(0);
  }
};

// ---------------------------------------------------------------------------
// RMSNorm backward epilogue with the delayed statistic (notes sec. 3):
// acc = G = dY W1^T; dU = dRes + r (G * gamma) - r^2 s u; N2 = bf16(r u gamma);
// gpart[pt, f] = sum over the wave's tokens of r G u (dgamma column partials).
// ---------------------------------------------------------------------------
// LN: the LayerNorm backward in the same delayed form, with the row
// statistics a (mean of G * gamma) and s (mean of G * gamma * xhat):
// dU = dRes + r (G * gamma) - r a - r^2 s (u - mu); N2 = r (u - mu) gamma + beta;
// gpart sums r G (u - mu) (dgamma) and bgpart sums G (dbeta); beta may be NULL.
template <bool HAS_RES, bool HAS_N2, bool HAS_GPART, bool LN = false>
struct EpiRowscaleBwd {
  const uint16_t* u;
  int ldu;
  const uint16_t* gamma;
  const float* r;
  const float* s;
  const uint16_t* dres;
  int ldr;
  uint16_t* du;
  int lddu;
  uint16_t* n2;
  int ldn;
  float* gpart;
  int dcols;  // row stride of gpart (= d)
  const float* mu = nullptr;
  const float* a = nullptr;
  const uint16_t* beta = nullptr;
  float* bgpart = nullptr;

  template <int RI, int CI>
  __device__ __forceinline__ void apply(const f32x16 (&acc)[RI][CI], const Geom& g) const {
    if constexpr (LN)
      apply_ln(acc, g);
    else
      apply_rms(acc, g);
  }

  template <int RI, int CI>
  __device__ __forceinline__ void apply_rms(const f32x16 (&acc)[RI][CI], const Geom& g) const {
    static_assert(CI * 32 == WAVE_T, "column partials assume 128-token wave tiles");
    const Lane L(g);
    const TileView<2> ui(u, ldu, g.tw0, g.fw0);
    const TileView<2> ri_(dres, ldr, g.tw0, g.fw0);
    const TileView<2> duo(du, lddu, g.tw0, g.fw0);
    const TileView<2> n2o(n2, ldn, g.tw0, g.fw0);
    // Per-token factors of the four 32-token columns.
    float rt[CI], c2[CI];
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) {
      const int t = g.tw0 + L.t(ci);
      rt[ci] = L.tok(ci) ? vload(r, t, g.T) : 0.0f;
      c2[ci] = rt[ci] * rt[ci] * vload(s, t, g.T);
    }
    // Feature-block order (ri outer): the dgamma column sums of one 32-feature
    // block are finished and reduced over the tokens before the next block, so
    // only 16 of them are live at a time.
    float gsum[RI];
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) {
      u32x4 gv[2], uv[CI][2], rv[CI][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) gv[h] = vload16_bf16(gamma, g.fw0 + L.f(ri, h), g.F);
#pragma unroll
      for (int ci = 0; ci < CI; ++ci)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uv[ci][h] = ui.load16(L.t(ci), L.f(ri, h), L.ok(ci, ri, h));
          if constexpr (HAS_RES) rv[ci][h] = ri_.load16(L.t(ci), L.f(ri, h), L.ok(ci, ri, h));
        }
      float col[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) col[i] = 0.0f;
#pragma unroll
      for (int ci = 0; ci < CI; ++ci)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bool ok = L.ok(ci, ri, h);
          float uvv[8], o[8], gm[8], Gv[8];
          acc8(acc, ri, ci, h, Gv);
          unpack8(uv[ci][h], uvv);
          unpack8(gv[h], gm);
          if constexpr (HAS_RES) {
            unpack8(rv[ci][h], o);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = 0.0f;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float G = Gv[e];
            o[e] += rt[ci] * (G * gm[e]) - c2[ci] * uvv[e];
            col[h * 8 + e] += rt[ci] * G * uvv[e];  // rt = 0 and u = 0 outside the matrix
          }
          duo.store16(L.t(ci), L.f(ri, h), ok, pack8(o));
          if constexpr (HAS_N2) {
            float nv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) nv[e] = rt[ci] * uvv[e] * gm[e];
            n2o.store16(L.t(ci), L.f(ri, h), ok, pack8(nv));
          }
        }
      if constexpr (HAS_GPART) {
        // Transpose-reduce the 16 column sums over the 32 token lanes: halving
        // at lane distances 16, 8, 4, 2 leaves entry lt/2 (summed over 16
        // lanes) in lane lt; the last step adds the neighbour at distance 1.
#pragma unroll
        for (int step = 0; step < 4; ++step) {
          const int mask = 16 >> step;
          const int n = 16 >> step;
          const bool upper = (g.lt & mask) != 0;
#pragma unroll
          for (int i = 0; i < n / 2; ++i) {
            const float keep = upper ? col[i + n / 2] : col[i];
            const float send = upper ? col[i] : col[i + n / 2];
            col[i] = keep + __shfl_xor(send, mask);
          }
        }
        gsum[ri] = col[0] + __shfl_xor(col[0], 1);
      }
    }
    if constexpr (HAS_GPART) {
      // Lane lt (even) writes entry lt/2 = 8 half + e of each feature block.
      const int idx = g.lt >> 1;
      const TileView<4> gp(gpart, dcols, g.pt, g.fw0);
#pragma unroll
      for (int ri = 0; ri < RI; ++ri) {
        const int f = L.f(ri, idx >> 3) + (idx & 7);
        const bool ok = L.T > 0 && f < L.F && (g.lt & 1) == 0;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gsum[ri]), gp.rs, gp.off(0, f, ok), 0, 0);
      }
    }
  }
  // The LayerNorm form: the same walk over 32-feature blocks, with the mean
  // term and the dbeta column sums.
  template <int RI, int CI>
  __device__ __forceinline__ void apply_ln(const f32x16 (&acc)[RI][CI], const Geom& g) const {
    static_assert(CI * 32 == WAVE_T, "column partials assume 128-token wave tiles");
    const Lane L(g);
    const TileView<2> ui(u, ldu, g.tw0, g.fw0);
    const TileView<2> ri_(dres, ldr, g.tw0, g.fw0);
    const TileView<2> duo(du, lddu, g.tw0, g.fw0);
    const TileView<2> n2o(n2, ldn, g.tw0, g.fw0);
    float rt[CI], c2[CI], mus[CI], ra[CI];
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) {
      const int t = g.tw0 + L.t(ci);
      rt[ci] = L.tok(ci) ? vload(r, t, g.T) : 0.0f;
      c2[ci] = rt[ci] * rt[ci] * vload(s, t, g.T);
      mus[ci] = vload(mu, t, g.T);
      ra[ci] = rt[ci] * vload(a, t, g.T);
    }
    // beta may be NULL: read gamma in its place (always valid) and select 0
    const bool hb = beta != nullptr;
    const uint16_t* bsrc = hb ? beta : gamma;
    float gsum[RI], bsum[RI];
#pragma unroll
    for (int ri = 0; ri < RI; ++ri) {
      __builtin_amdgcn_sched_barrier(0);  // one 32-feature block's loads at a time
      u32x4 gv[2], bev[2], uv[CI][2], rv[CI][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        gv[h] = vload16_bf16(gamma, g.fw0 + L.f(ri, h), g.F);
        const u32x4 bq = vload16_bf16(bsrc, g.fw0 + L.f(ri, h), g.F);
        bev[h] = hb ? bq : (u32x4){0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int ci = 0; ci < CI; ++ci)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          uv[ci][h] = ui.load16(L.t(ci), L.f(ri, h), L.ok(ci, ri, h));
          if constexpr (HAS_RES) rv[ci][h] = ri_.load16(L.t(ci), L.f(ri, h), L.ok(ci, ri, h));
        }
      float col[16], bcol[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        col[i] = 0.0f;
        bcol[i] = 0.0f;
      }
#pragma unroll
      for (int ci = 0; ci < CI; ++ci)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bool ok = L.ok(ci, ri, h);
          float uvv[8], o[8], gm[8], Gv[8];
          acc8(acc, ri, ci, h, Gv);
          unpack8(uv[ci][h], uvv);
          unpack8(gv[h], gm);
          if constexpr (HAS_RES) {
            unpack8(rv[ci][h], o);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = 0.0f;
          }
          // rt = 0 outside the matrix, and G = 0 there (zero-filled operands)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float G = Gv[e], cu = uvv[e] - mus[ci];
            o[e] += rt[ci] * (G * gm[e]) - ra[ci] - c2[ci] * cu;
            col[h * 8 + e] += rt[ci] * G * cu;
            bcol[h * 8 + e] += G;
          }
          duo.store16(L.t(ci), L.f(ri, h), ok, pack8(o));
          if constexpr (HAS_N2) {
            float nv[8], bt[8];
            unpack8(bev[h], bt);
#pragma unroll
            for (int e = 0; e < 8; ++e) nv[e] = fmaf(rt[ci] * (uvv[e] - mus[ci]), gm[e], bt[e]);
            n2o.store16(L.t(ci), L.f(ri, h), ok, pack8(nv));
          }
        }
      if constexpr (HAS_GPART) {
        // the transpose-reduce of apply_rms, on both column sums
#pragma unroll
        for (int step = 0; step < 4; ++step) {
          const int mask = 16 >> step;
          const int n = 16 >> step;
          const bool upper = (g.lt & mask) != 0;
#pragma unroll
          for (int i = 0; i < n / 2; ++i) {
            const float keep = upper ? col[i + n / 2] : col[i];
            const float send = upper ? col[i] : col[i + n / 2];
            col[i] = keep + __shfl_xor(send, mask);
            const float bkeep = upper ? bcol[i + n / 2] : bcol[i];
            const float bsend = upper ? bcol[i] : bcol[i + n / 2];
            bcol[i] = bkeep + __shfl_xor(bsend, mask);
          }
        }
        gsum[ri] = col[0] + __shfl_xor(col[0], 1);
        bsum[ri] = bcol[0] + __shfl_xor(bcol[0], 1);
      }
    }
    if constexpr (HAS_GPART) {
      const int idx = g.lt >> 1;
      const TileView<4> gp(gpart, dcols, g.pt, g.fw0);
      const TileView<4> bp(bgpart, dcols, g.pt, g.fw0);
#pragma unroll
      for (int ri = 0; ri < RI; ++ri) {
        const int f = L.f(ri, idx >> 3) + (idx & 7);
        const bool ok = L.T > 0 && f < L.F && (g.lt & 1) == 0;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(gsum[ri]), gp.rs, gp.off(0, f, ok), 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(bsum[ri]), bp.rs, bp.off(0, f, ok), 0, 0);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// fp32 output (weight gradients): out (+)= acc.
// ---------------------------------------------------------------------------
template <bool ACCUM>
struct EpiF32 {
  float* out;
  int ld;

  // The plain store goes through the released LDS (fp32 rows of 512 bytes,
  // 64 rows per 32 KiB wave slice, so two passes of two 32-token columns)
  // and is non-temporal (weight gradients are written once, 0.1-1 GB);
  // the accumulating form keeps its register path.
  static constexpr int LDS_BYTES = ACCUM ? 0 : STAGE_LDS;

  template <int RI, int CI>
  __device__ __forceinline__ void apply(const f32x16 (&acc)[RI][CI], const Geom& g, char* smem = nullptr) const {
    const Lane L(g);
    const TileView<4> o(out, ld, g.tw0, g.fw0);
    if constexpr (!ACCUM) {
      static_assert(CI % 2 == 0, "passes of two 32-token columns");
      char* reg = smem + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) * 32768;
      const int rlo = g.lane >> 5, pos = g.lane & 31;
#pragma unroll
      for (int p = 0; p < CI / 2; ++p) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const int ci = 2 * p + cc, r = 32 * cc + g.lt;
#pragma unroll
          for (int ri = 0; ri < RI; ++ri)
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int c = 0; c < 2; ++c) {  // chunk = 4 consecutive features
                const f32x4 v = {acc[ri][ci][8 * h + 4 * c + 0], acc[ri][ci][8 * h + 4 * c + 1],
                                 acc[ri][ci][8 * h + 4 * c + 2], acc[ri][ci][8 * h + 4 * c + 3]};
                const int chunk = 8 * ri + 4 * h + 2 * g.hh + c;
                st16(reg + r * 512 + ((chunk ^ (r & 7)) << 4), __builtin_bit_cast(u32x4, v));
              }
        }
#pragma unroll
        for (int i0 = 0; i0 < 32; i0 += 8) {
          u32x4 sv[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) sv[i] = ld16(reg + (i0 + i) * 1024 + 16 * g.lane);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int r = 2 * (i0 + i) + rlo, c = pos ^ (r & 7);
            o.store16_nt(64 * p + r, 4 * c, 64 * p + r < L.T && 4 * c < L.F, sv[i]);
          }
        }
      }
      return;
    }
    u32x4 prev[2][RI][2][2];
    auto load_col = [&](int ci, u32x4 (&b)[RI][2][2]) {
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int c = 0; c < 2; ++c) b[ri][h][c] = o.load16(L.t(ci), L.f(ri, h) + 4 * c, L.ok(ci, ri, h));
    };
    if constexpr (ACCUM) load_col(0, prev[0]);
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) {
      if constexpr (ACCUM) {
        if (ci + 1 < CI) load_col(ci + 1, prev[(ci + 1) & 1]);
      }
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          float a[8];
          if constexpr (ACCUM) acc8(acc, ri, ci, h, a);
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            f32x4 v;
            if constexpr (ACCUM) {
              v = (f32x4){a[4 * c], a[4 * c + 1], a[4 * c + 2], a[4 * c + 3]} +
                  __builtin_bit_cast(f32x4, prev[ci & 1][ri][h][c]);
            } else {  // stored straight from the accumulator registers
              v = (f32x4){acc[ri][ci][8 * h + 4 * c + 0], acc[ri][ci][8 * h + 4 * c + 1],
                          acc[ri][ci][8 * h + 4 * c + 2], acc[ri][ci][8 * h + 4 * c + 3]};
            }
            o.store16(L.t(ci), L.f(ri, h) + 4 * c, L.ok(ci, ri, h), __builtin_bit_cast(u32x4, v));
          }
        }
    }
  }
};

}  // namespace coda
