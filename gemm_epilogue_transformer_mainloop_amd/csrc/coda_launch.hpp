// coda_launch.hpp - host-side launch of one fused GEMM (tile plan, grid
// shape and kernel choice), shared by the translation units of the C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "../../include/coda.h"
#include "coda_epilogues.hpp"
#include "coda_host.hpp"

namespace coda_launch {

using namespace coda;
using namespace coda_host;

// Epilogues that work on any wave-tile width (all but the dgamma column
// partials, which are laid out per 128-token wave tile).
template <class Epi>
struct AnyWaveWidth : std::true_type {};
template <bool A, bool B, bool C, bool D>
struct AnyWaveWidth<EpiRowscaleBwd<A, B, C, D>> : std::false_type {};

// Tile-count quantization.  One 256x256 tile per CU at a time: when the tile
// count leaves the last round of tiles partly empty (8192 x 3072 has 384
// tiles = 1.5 rounds on 256 CUs), the trailing feature range can instead be
// covered by 256-feature x 128-token tiles, two per big tile, each taking
// about 0.6 of a big tile's time (measured on 8192 x 3072 x 2048).  Returns
// the number of 256-wide feature tiles to keep in big tiles (the rest go to
// the half tiles), or 0 to keep every tile big.  Cost model in rounds: a big
// round is 1, a half-tile round 0.6; a split must save at least 0.2 rounds.
inline int quantization_split(int nTF, int nTT, int nTT_half, int cus) {
  if (cus <= 0 || nTF < 2) return 0;
  const double base = (double)cdiv(nTF * nTT, cus);
  double best = base - 0.2;
  int split = 0;
  for (int f1 = 1; f1 < nTF; ++f1) {
    const double c = (double)cdiv(f1 * nTT, cus) + 0.6 * (double)cdiv((nTF - f1) * nTT_half, cus);
    if (c < best) {
      best = c;
      split = f1;
    }
  }
  return split;
}

// Token split: when the feature split finds nothing, the trailing token
// range can be covered by 256 x 128 tiles instead (the weight gradient
// 14336 x 4096 over 8192 tokens has 56 x 16 = 896 tiles, 3.5 rounds: 48 token
// tiles x 16 = 768 big tiles are 3 rounds, the last 2048 tokens 256 half
// tiles, one round of 0.6).  Returns the number of 256-token tiles to keep
// big, or 0.  Same cost model as the feature split; of equal costs the one
// with the most big tiles.
inline int token_split(int nTF, int nTT, int T, int cus) {
  if (cus <= 0 || nTT < 2) return 0;
  const double base = (double)cdiv(nTF * nTT, cus);
  double best = base - 0.2;
  int split = 0;
  for (int tb = nTT - 1; tb >= 1; --tb) {
    const int nh = cdiv(T - 256 * tb, 128);
    const double c = (double)cdiv(nTF * tb, cus) + 0.6 * (double)cdiv(nTF * nh, cus);
    if (c < best) {
      best = c;
      split = tb;
    }
  }
  return split;
}

// The problem description of a launch over all of F x T.
inline Problem whole_problem(const uint16_t* W, int ldw, const uint16_t* X, int ldx, int F, int T, int K, int BT) {
  Problem p;
  p.W = W;
  p.X = X;
  p.ldw = ldw;
  p.ldx = ldx;
  p.F = F;
  p.T = T;
  p.K = K;
  p.nTF = cdiv(F, 256);
  p.nTT = cdiv(T, BT);
  p.f_base = 0;
  p.t_base = 0;
  p.tl = nullptr;
  p.tl_waves = 0;
  if constexpr (kTimeline) {
    std::lock_guard<std::mutex> lock(g_tl_mu);
    p.tl = g_tl_buf;
    p.tl_waves = g_tl_waves;
  }
  return p;
}

// Persistent launch (gemm_epi_kernel_persistent) of p's 256 x 256 tiles on
// the largest multiple of 8 workgroups not above the CU count, the carry
// built from `ca` in every workgroup.  The caller has checked the plan
// (coda_swiglu_bwd_units).
template <bool WK, bool XK, class Epi, class Carry>
coda_status launch_persistent(const Problem& p, const Epi& epi, const typename Carry::Args& ca, hipStream_t stream) {
  const int nb = p.nTF * p.nTT;
  const int g = (device_cus() / 8) * 8;
  if (nb == 0) return CODA_OK;
  if (g < 8) return CODA_ERR_UNSUPPORTED;
  hipLaunchKernelGGL((gemm_epi_kernel_persistent<WK, XK, Epi, Carry>), dim3(nb < g ? nb : g), dim3(NT), 0, stream,
                     p, epi, ca);
  return launched();
}

template <bool WK, bool XK, int BT = 256, class Epi>
coda_status launch_gemm(const uint16_t* W, int ldw, const uint16_t* X, int ldx, int F, int T, int K,
                        const Epi& epi, hipStream_t stream) {
  constexpr int BF = 256;
  Problem p = whole_problem(W, ldw, X, ldx, F, T, K, BT);
  const int nb = p.nTF * p.nTT;
  if (nb == 0) return CODA_OK;
  if constexpr (BT == 256 && AnyWaveWidth<Epi>::value) {
    const int cus = device_cus();
    const int split = coda_tile_split(F, T, cus);
    if (split > 0) {
      Problem big = p, half = p;
      big.nTF = split;
      half.f_base = split * BF;
      half.nTF = p.nTF - split;
      half.nTT = cdiv(T, 128);
      hipLaunchKernelGGL((gemm_epi_kernel_split<WK, XK, Epi>), dim3(big.nTF * big.nTT + half.nTF * half.nTT),
                         dim3(NT), 0, stream, big, half, epi);
      return launched();
    }
    // Under half a round of big tiles: 256 x 128 tiles run on twice as many
    // CUs in the same single round, so each CU's k-loop and epilogue (the
    // whole cost of a small GEMM) are about half as long.
    if (cus > 0 && 2 * nb <= cus && cdiv(T, 128) > p.nTT) {
      Problem none = p, half = p;
      none.nTF = 0;
      half.nTT = cdiv(T, 128);
      hipLaunchKernelGGL((gemm_epi_kernel_split<WK, XK, Epi>), dim3(half.nTF * half.nTT), dim3(NT), 0,
                         stream, none, half, epi);
      return launched();
    }
    const int tsplit = coda_tile_split_tokens(F, T, cus);
    if (tsplit > 0) {
      Problem big = p, half = p;
      big.nTT = tsplit;
      half.t_base = tsplit * 256;
      half.nTT = cdiv(T - half.t_base, 128);
      hipLaunchKernelGGL((gemm_epi_kernel_split<WK, XK, Epi>), dim3(big.nTF * big.nTT + half.nTF * half.nTT),
                         dim3(NT), 0, stream, big, half, epi);
      return launched();
    }
  }
  hipLaunchKernelGGL((gemm_epi_kernel<BF, BT, WK, XK, Epi>), dim3(nb), dim3(NT), 0, stream, p, epi);
  return launched();
}

}  // namespace coda_launch
