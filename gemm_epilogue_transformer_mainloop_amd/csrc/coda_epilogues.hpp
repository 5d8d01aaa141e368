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
#pragma once

#include "coda_mainloop.hpp"

namespace coda {

constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * LOG2E); }
__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + fast_exp(-x)); }

// Sum over the two lanes (l, l^32) that hold the same token.
__device__ __forceinline__ float sum_halves(float v) { return v + __shfl_xor(v, 32); }

// ---------------------------------------------------------------------------
// Store-only / row-scale / residual epilogue:  Y = bf16( r_t * acc + res )
// (plain GEMM; GEMM2's delayed RMSNorm scale; data-gradient + residual)
// ---------------------------------------------------------------------------
template <bool HAS_R, bool HAS_RES>
struct EpiLinear {
  const float* r;
  const uint16_t* res;
  int ldres;
  uint16_t* Y;
  int ldy;

  template <int RI, int CI>
  __device__ __forceinline__ void apply(const f32x16 (&acc)[RI][CI], const Geom& g) const {
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) {
      const int t = tok_of(g, ci);
      if (t >= g.T) continue;
      const float rs = HAS_R ? r[t] : 1.0f;
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int f = feat_of(g, ri, half);
          if (f >= g.F) continue;
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = acc[ri][ci][8 * half + e] * rs;
          if constexpr (HAS_RES) {
            float z[8];
            unpack8(ld16(res + (size_t)t * ldres + f), z);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] += z[e];
          }
          st16(Y + (size_t)t * ldy + f, pack8(v));
        }
    }
  }
};

// ---------------------------------------------------------------------------
// GEMM1 of GEMM -> residual -> RMSNorm -> GEMM (notes sec. 2; paper Fig. 4,
// Listing 2): u = acc + z; U = bf16(u); H2 = bf16(u * gamma);
// part[t, pf] = sum over the wave's features of u^2 (unscaled, fp32).
// ---------------------------------------------------------------------------
template <bool HAS_Z, bool HAS_H2, bool HAS_PART>
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

  template <int RI, int CI>
  __device__ __forceinline__ void apply(const f32x16 (&acc)[RI][CI], const Geom& g) const {
    float gm[RI][2][8];
    if constexpr (HAS_H2) {
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int f = feat_of(g, ri, half);
          if (f < g.F)
            unpack8(ld16(gamma + f), gm[ri][half]);
          else
#pragma unroll
            for (int e = 0; e < 8; ++e) gm[ri][half][e] = 0.0f;
        }
    }
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) {
      const int t = tok_of(g, ci);
      const bool tok_ok = t < g.T;
      float ss = 0.0f;
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int f = feat_of(g, ri, half);
          if (!tok_ok || f >= g.F) continue;
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = acc[ri][ci][8 * half + e];
          if constexpr (HAS_Z) {
            float zz[8];
            unpack8(ld16(z + (size_t)t * ldz + f), zz);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] += zz[e];
          }
          st16(U + (size_t)t * ldu + f, pack8(v));
#pragma unroll
          for (int e = 0; e < 8; ++e) ss += v[e] * v[e];
          if constexpr (HAS_H2) {
            float h[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) h[e] = v[e] * gm[ri][half][e];
            st16(H2 + (size_t)t * ldh + f, pack8(h));
          }
        }
      if constexpr (HAS_PART) {
        ss = sum_halves(ss);
        if (g.hh == 0 && tok_ok && g.fw0 < g.F) part[(size_t)t * nparts + g.pf] = ss;
      }
    }
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

  template <int RI, int CI>
  __device__ __forceinline__ void apply(const f32x16 (&acc)[RI][CI], const Geom& g) const {
    // Per-lane frequencies in revolutions per position: theta^(-2k/hd) / (2 pi).
    constexpr float INV_2PI = 0.15915494309189535f;
    float fr[RI][2][4];
#pragma unroll
    for (int ri = 0; ri < RI; ++ri)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int f = feat_of(g, ri, half);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int k = ((f + 2 * q) % head_dim) >> 1;
          fr[ri][half][q] = exp2f(-(float)(2 * k) / (float)head_dim * log2_theta) * INV_2PI;
        }
      }
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) {
      const int t = tok_of(g, ci);
      if (t >= g.T) continue;
      const float rs = HAS_R ? r[t] : 1.0f;
      const float ps = (float)pos[t];
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int f = feat_of(g, ri, half);
          if (f >= g.F) continue;
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = acc[ri][ci][8 * half + e] * rs;
          if (f < n_rope) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              float rev = ps * fr[ri][half][q];
              rev -= floorf(rev);
              float sn = __builtin_amdgcn_sinf(rev), cs = __builtin_amdgcn_cosf(rev);
              if (INV) sn = -sn;
              const float a = v[2 * q], b = v[2 * q + 1];
              v[2 * q] = a * cs - b * sn;
              v[2 * q + 1] = a * sn + b * cs;
            }
          }
          st16(Y + (size_t)t * ldy + f, pack8(v));
        }
    }
  }
};

// ---------------------------------------------------------------------------
// SwiGLU pair map 2 -> 1 (paper Fig. 7): (g, v) = r * (acc_2j, acc_2j+1),
// a_j = g sigmoid(g) v; optional Pre = bf16(g, v) for the backward pass.
// The GEMM's feature space is the interleaved 2F columns.
// ---------------------------------------------------------------------------
template <bool HAS_R, bool HAS_PRE>
struct EpiSwiglu {
  const float* r;
  uint16_t* act;
  int ldact;
  uint16_t* pre;
  int ldp;

  template <int RI, int CI>
  __device__ __forceinline__ void apply(const f32x16 (&acc)[RI][CI], const Geom& g) const {
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) {
      const int t = tok_of(g, ci);
      if (t >= g.T) continue;
      const float rs = HAS_R ? r[t] : 1.0f;
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int f = feat_of(g, ri, half);
          if (f >= g.F) continue;
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = acc[ri][ci][8 * half + e] * rs;
          float a[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float gg = v[2 * q], uu = v[2 * q + 1];
            a[q] = gg * sigmoidf_(gg) * uu;
          }
          *reinterpret_cast<u32x2*>(act + (size_t)t * ldact + (f >> 1)) =
              (u32x2){pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
          if constexpr (HAS_PRE) st16(pre + (size_t)t * ldp + f, pack8(v));
        }
    }
  }
};

// ---------------------------------------------------------------------------
// LM-head cross-entropy statistics (notes sec. 2 "Cross-entropy loss"):
// per (token, wave feature tile) running max m and sum exp(l - m) of the fp32
// logits, plus the gathered target logit.  Logits are never stored.
// ---------------------------------------------------------------------------
struct EpiCE {
  const int32_t* labels;
  float* part_m;
  float* part_s;
  float* tgt;
  int nparts;

  template <int RI, int CI>
  __device__ __forceinline__ void apply(const f32x16 (&acc)[RI][CI], const Geom& g) const {
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) {
      const int t = tok_of(g, ci);
      const bool tok_ok = t < g.T;
      const int label = tok_ok ? labels[t] : -1;
      float m = -INFINITY;
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int f = feat_of(g, ri, half);
          if (f >= g.F) continue;
#pragma unroll
          for (int e = 0; e < 8; ++e) m = fmaxf(m, acc[ri][ci][8 * half + e]);
        }
      float s = 0.0f;
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int f = feat_of(g, ri, half);
          if (f >= g.F) continue;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float l = acc[ri][ci][8 * half + e];
            s += fast_exp(l - m);
            if (label == f + e) tgt[t] = l;
          }
        }
      // merge the two half-wave states of this token
      const float m2 = __shfl_xor(m, 32), s2 = __shfl_xor(s, 32);
      const float mm = fmaxf(m, m2);
      const float st = (m == -INFINITY ? 0.0f : s * fast_exp(m - mm)) +
                       (m2 == -INFINITY ? 0.0f : s2 * fast_exp(m2 - mm));
      if (g.hh == 0 && tok_ok && g.fw0 < g.F) {
        part_m[(size_t)t * nparts + g.pf] = mm;
        part_s[(size_t)t * nparts + g.pf] = st;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// dlogits of the LM-head cross-entropy backward (recomputed logits):
// D = (exp(l - lse_t) - [f == label_t]) * scale, bf16.
// ---------------------------------------------------------------------------
struct EpiCEBwd {
  const int32_t* labels;
  const float* lse;
  float scale;
  uint16_t* D;
  int ldd;

  template <int RI, int CI>
  __device__ __forceinline__ void apply(const f32x16 (&acc)[RI][CI], const Geom& g) const {
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) {
      const int t = tok_of(g, ci);
      if (t >= g.T) continue;
      const int label = labels[t];
      const float L = lse[t];
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int f = feat_of(g, ri, half);
          if (f >= g.F) continue;
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float pr = fast_exp(acc[ri][ci][8 * half + e] - L);
            v[e] = (pr - (label == f + e ? 1.0f : 0.0f)) * scale;
          }
          st16(D + (size_t)t * ldd + f, pack8(v));
        }
    }
  }
};

// ---------------------------------------------------------------------------
// SwiGLU backward pair map 1 -> 2 (paper Fig. 7; notes sec. 3): acc = da_j,
// (g, v) = Pre[2j, 2j+1]; dPre = (da v s (1 + g (1 - s)), da g s);
// spart[t, pf] = sum (dPre_2j g + dPre_2j+1 v)  (RMSNorm statistic partial).
// ---------------------------------------------------------------------------
template <bool HAS_SPART>
struct EpiSwigluBwd {
  const uint16_t* pre;
  int ldp;
  uint16_t* dpre;
  int lddp;
  float* spart;
  int nparts;

  template <int RI, int CI>
  __device__ __forceinline__ void apply(const f32x16 (&acc)[RI][CI], const Geom& g) const {
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) {
      const int t = tok_of(g, ci);
      const bool tok_ok = t < g.T;
      float ss = 0.0f;
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int f = feat_of(g, ri, half);
          if (!tok_ok || f >= g.F) continue;
#pragma unroll
          for (int c = 0; c < 2; ++c) {  // two 16-byte chunks = 4 pairs each
            float pv[8], out[8];
            unpack8(ld16(pre + (size_t)t * ldp + 2 * f + 8 * c), pv);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float da = acc[ri][ci][8 * half + 4 * c + q];
              const float gg = pv[2 * q], uu = pv[2 * q + 1];
              const float sg = sigmoidf_(gg);
              const float dg = da * uu * sg * (1.0f + gg * (1.0f - sg));
              const float du = da * gg * sg;
              out[2 * q] = dg;
              out[2 * q + 1] = du;
              ss += dg * gg + du * uu;
            }
            st16(dpre + (size_t)t * lddp + 2 * f + 8 * c, pack8(out));
          }
        }
      if constexpr (HAS_SPART) {
        ss = sum_halves(ss);
        if (g.hh == 0 && tok_ok && g.fw0 < g.F) spart[(size_t)t * nparts + g.pf] = ss;
      }
    }
  }
};

// ---------------------------------------------------------------------------
// RMSNorm backward epilogue with the delayed statistic (notes sec. 3):
// acc = G = dY W1^T; dU = dRes + r (G * gamma) - r^2 s u; N2 = bf16(r u gamma);
// gpart[pt, f] = sum over the wave's tokens of r G u (dgamma column partials).
// ---------------------------------------------------------------------------
template <bool HAS_RES, bool HAS_N2, bool HAS_GPART>
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

  template <int RI, int CI>
  __device__ __forceinline__ void apply(const f32x16 (&acc)[RI][CI], const Geom& g) const {
    static_assert(CI * 32 == WAVE_T, "column partials assume 128-token wave tiles");
    float gm[RI][2][8];
    float col[RI * 16];
#pragma unroll
    for (int i = 0; i < RI * 16; ++i) col[i] = 0.0f;
#pragma unroll
    for (int ri = 0; ri < RI; ++ri)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int f = feat_of(g, ri, half);
        if (f < g.F)
          unpack8(ld16(gamma + f), gm[ri][half]);
        else
#pragma unroll
          for (int e = 0; e < 8; ++e) gm[ri][half][e] = 0.0f;
      }
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) {
      const int t = tok_of(g, ci);
      if (t >= g.T) continue;
      const float rt = r[t], st = s[t];
      const float c2 = rt * rt * st;
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int f = feat_of(g, ri, half);
          if (f >= g.F) continue;
          float uv[8], o[8];
          unpack8(ld16(u + (size_t)t * ldu + f), uv);
          if constexpr (HAS_RES) {
            unpack8(ld16(dres + (size_t)t * ldr + f), o);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = 0.0f;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float G = acc[ri][ci][8 * half + e];
            o[e] += rt * (G * gm[ri][half][e]) - c2 * uv[e];
            col[ri * 16 + half * 8 + e] += rt * G * uv[e];
          }
          st16(du + (size_t)t * lddu + f, pack8(o));
          if constexpr (HAS_N2) {
            float nv[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) nv[e] = rt * uv[e] * gm[ri][half][e];
            st16(n2 + (size_t)t * ldn + f, pack8(nv));
          }
        }
    }
    if constexpr (HAS_GPART) {
      // Transpose-reduce the RI*16 column sums over the 32 token lanes: after
      // halving at lane distances 16, 8, 4, 2, 1 lane lt holds the sums of
      // entries 2*lt and 2*lt + 1.
      constexpr int N0 = RI * 16;
      static_assert(N0 == 64, "butterfly assumes 64 column sums per lane");
#pragma unroll
      for (int step = 0; step < 5; ++step) {
        const int mask = 16 >> step;
        const int n = N0 >> step;
        const bool upper = (g.lt & mask) != 0;
#pragma unroll
        for (int i = 0; i < n / 2; ++i) {
          const float keep = upper ? col[i + n / 2] : col[i];
          const float send = upper ? col[i] : col[i + n / 2];
          col[i] = keep + __shfl_xor(send, mask);
        }
      }
      if (g.tw0 >= g.T) return;  // no token of this wave tile exists
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int idx = 2 * g.lt + j;
        const int ri = idx >> 4, half = (idx >> 3) & 1, e = idx & 7;
        const int f = feat_of(g, ri, half) + e;
        if (f < g.F) gpart[(size_t)g.pt * dcols + f] = col[j];
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

  template <int RI, int CI>
  __device__ __forceinline__ void apply(const f32x16 (&acc)[RI][CI], const Geom& g) const {
#pragma unroll
    for (int ci = 0; ci < CI; ++ci) {
      const int t = tok_of(g, ci);
      if (t >= g.T) continue;
#pragma unroll
      for (int ri = 0; ri < RI; ++ri)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int f = feat_of(g, ri, half);
          if (f >= g.F) continue;
          float* o = out + (size_t)t * ld + f;
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            f32x4 v = {acc[ri][ci][8 * half + 4 * c + 0], acc[ri][ci][8 * half + 4 * c + 1],
                       acc[ri][ci][8 * half + 4 * c + 2], acc[ri][ci][8 * half + 4 * c + 3]};
            if constexpr (ACCUM) v += *reinterpret_cast<const f32x4*>(o + 4 * c);
            *reinterpret_cast<f32x4*>(o + 4 * c) = v;
          }
        }
    }
  }
};

}  // namespace coda
