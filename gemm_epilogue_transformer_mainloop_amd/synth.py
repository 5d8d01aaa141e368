"""Seeded synthetic inputs for the CODA GEMM-epilogue path.

This module only draws random numbers and packs them into bfloat16 bit
patterns.  It contains none of the method's arithmetic, so both the HIP path
(via torch tensors built from the same bits) and the fp64 oracle (via the
exact fp64 widening of those bits) consume identical inputs.

Recipe (stated once, used everywhere):
  * ``numpy.random.default_rng(seed)`` (PCG64) draws float32 normals;
  * the float32 values are rounded to bfloat16 with round-to-nearest-even;
  * seed = 1000 * config_index + tensor_index, so every tensor of every
    workload is reproducible on its own.

The workloads follow the Llama-3-style layer shapes of the paper
"CODA: Rewriting Transformer Blocks as GEMM-Epilogue Programs" (its Figure 1
and Figure 6 name LLaMA-3 1B and 8B layers); no dataset or trained weight is
involved.
"""

from __future__ import annotations

import dataclasses
from typing import Dict, Tuple

import numpy as np

# --------------------------------------------------------------------------
# bfloat16 packing (data format, not method arithmetic)
# --------------------------------------------------------------------------


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return uint16 bits."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # u + 0x7FFF + lsb stays below 2^32 for every finite value and infinity
    # (the largest, 0xFF7FFFFF, becomes 0xFF807FFF); NaNs are set afterwards.
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bits to float64."""
    return bf16_bits_to_f32(b).astype(np.float64)


@dataclasses.dataclass
class Bf16:
    """A bfloat16 tensor held as its uint16 bit pattern."""

    bits: np.ndarray

    @property
    def shape(self) -> Tuple[int, ...]:
        return tuple(self.bits.shape)

    def f64(self) -> np.ndarray:
        return bf16_bits_to_f64(self.bits)

    def f32(self) -> np.ndarray:
        return bf16_bits_to_f32(self.bits)

    def torch(self, device="cpu"):
        """A torch.bfloat16 tensor with exactly these bits."""
        import torch

        t = torch.from_numpy(np.ascontiguousarray(self.bits).view(np.int16)).view(torch.bfloat16)
        return t.to(device)


def normal_bf16(seed: int, shape, std: float = 1.0, mean: float = 0.0) -> Bf16:
    """N(mean, std^2) drawn in float32 with PCG64(seed), rounded RNE to bfloat16."""
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    if mean != 0.0:
        a += np.float32(mean)
    return Bf16(f32_to_bf16_bits(a))


def int_bf16(seed: int, shape, lo: int, hi: int) -> Bf16:
    """Uniform integers in [lo, hi] stored as (exactly representable) bfloat16."""
    rng = np.random.default_rng(seed)
    a = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return Bf16(f32_to_bf16_bits(a))


def labels_int32(seed: int, m: int, vocab: int) -> np.ndarray:
    """Uniform int32 labels in [0, vocab)."""
    rng = np.random.default_rng(seed)
    return rng.integers(0, vocab, size=m, dtype=np.int64).astype(np.int32)


def positions_int32(m: int, seq_len: int) -> np.ndarray:
    """Token positions 0..seq_len-1 repeated per packed sequence."""
    return (np.arange(m, dtype=np.int64) % seq_len).astype(np.int32)


def seed_of(config: int, index: int) -> int:
    return 1000 * config + index


# --------------------------------------------------------------------------
# Workloads (shapes and distributions of the five synthetic configurations)
# --------------------------------------------------------------------------

EPS = 1e-6
ROPE_THETA = 500000.0
HEAD_DIM = 64
SEQ_LEN = 2048


def norm_block_inputs(config: int, M: int, d: int, K: int, N: int, n_rope_cols: int = 0) -> Dict[str, object]:
    """GEMM -> residual -> RMSNorm -> GEMM inputs.

    x[M,K] ~ N(0,1); W0[K,d] ~ N(0,1/K); z[M,d] ~ N(0,1); gamma[d] ~ N(1,0.1);
    W1[d,N] ~ N(0,1/d).  When ``n_rope_cols`` is set, a second (QKV-shaped)
    weight W1r[d, n_rope_cols] and positions i mod 2048 are added.
    """
    out: Dict[str, object] = {
        "x": normal_bf16(seed_of(config, 0), (M, K)),
        "W0": normal_bf16(seed_of(config, 1), (K, d), std=(1.0 / K) ** 0.5),
        "z": normal_bf16(seed_of(config, 2), (M, d)),
        "gamma": normal_bf16(seed_of(config, 3), (d,), std=0.1, mean=1.0),
        "W1": normal_bf16(seed_of(config, 4), (d, N), std=(1.0 / d) ** 0.5),
        "eps": EPS,
    }
    if n_rope_cols:
        out["W1r"] = normal_bf16(seed_of(config, 5), (d, n_rope_cols), std=(1.0 / d) ** 0.5)
        out["pos"] = positions_int32(M, SEQ_LEN)
    return out


def mlp_inputs(config: int, M: int, d: int, F: int) -> Dict[str, object]:
    """SwiGLU MLP with residual: x[M,d], Wgu[d,2F] (gate even / up odd columns), Wd[F,d], dY[M,d]."""
    return {
        "x": normal_bf16(seed_of(config, 0), (M, d)),
        "Wgu": normal_bf16(seed_of(config, 1), (d, 2 * F), std=(1.0 / d) ** 0.5),
        "Wd": normal_bf16(seed_of(config, 2), (F, d), std=(1.0 / F) ** 0.5),
        "dY": normal_bf16(seed_of(config, 3), (M, d)),
    }


def lmhead_inputs(config: int, M: int, d: int, V: int) -> Dict[str, object]:
    """LM head: h[M,d] ~ N(0,1), W[d,V] ~ N(0,1/d), labels uniform in [0,V)."""
    return {
        "h": normal_bf16(seed_of(config, 0), (M, d)),
        "W": normal_bf16(seed_of(config, 1), (d, V), std=(1.0 / d) ** 0.5),
        "labels": labels_int32(seed_of(config, 2), M, V),
    }


def block_inputs(config: int, M: int, d: int, F: int) -> Dict[str, object]:
    """Two stacked residual + RMSNorm + SwiGLU-MLP layers behind a d x d projection.

    x[M,d], z[M,d], dOut[M,d] ~ N(0,1); W0[d,d] ~ N(0,1/d); per layer l in {1,2}:
    gamma_l[d] ~ N(1,0.1), Wgu_l[d,2F] ~ N(0,1/d), Wd_l[F,d] ~ N(0,1/F).
    """
    s = (1.0 / d) ** 0.5
    sf = (1.0 / F) ** 0.5
    return {
        "x": normal_bf16(seed_of(config, 0), (M, d)),
        "z": normal_bf16(seed_of(config, 1), (M, d)),
        "W0": normal_bf16(seed_of(config, 2), (d, d), std=s),
        "gamma1": normal_bf16(seed_of(config, 3), (d,), std=0.1, mean=1.0),
        "Wgu1": normal_bf16(seed_of(config, 4), (d, 2 * F), std=s),
        "Wd1": normal_bf16(seed_of(config, 5), (F, d), std=sf),
        "gamma2": normal_bf16(seed_of(config, 6), (d,), std=0.1, mean=1.0),
        "Wgu2": normal_bf16(seed_of(config, 7), (d, 2 * F), std=s),
        "Wd2": normal_bf16(seed_of(config, 8), (F, d), std=sf),
        "dOut": normal_bf16(seed_of(config, 9), (M, d)),
        "eps": EPS,
    }


def ln_norm_block_inputs(config: int, M: int, d: int, K: int, N: int, z_mean: float = 0.5) -> Dict[str, object]:
    """GEMM -> residual -> LayerNorm -> GEMM inputs: those of norm_block_inputs
    with the residual z ~ N(z_mean, 1) (rows with a nonzero mean exercise the
    mean term) and a LayerNorm bias beta[d] ~ N(0, 0.1^2)."""
    out = norm_block_inputs(config, M, d, K, N)
    out["z"] = normal_bf16(seed_of(config, 2), (M, d), mean=z_mean)
    out["beta"] = normal_bf16(seed_of(config, 6), (d,), std=0.1)
    return out


def ln_block_inputs(config: int, M: int, d: int, F: int, z_mean: float = 0.5) -> Dict[str, object]:
    """block_inputs with LayerNorm biases beta_l[d] ~ N(0, 0.1^2) and the
    residual z ~ N(z_mean, 1)."""
    out = block_inputs(config, M, d, F)
    out["z"] = normal_bf16(seed_of(config, 1), (M, d), mean=z_mean)
    out["beta1"] = normal_bf16(seed_of(config, 10), (d,), std=0.1)
    out["beta2"] = normal_bf16(seed_of(config, 11), (d,), std=0.1)
    return out


# Full-size shapes of the five workloads (tokens, widths).
CONFIGS = {
    1: dict(kind="norm_block", M=256, d=512, K=512, N=1024),
    2: dict(kind="norm_block", M=8192, d=2048, K=2048, N=2048, n_rope_cols=3072),
    3: dict(kind="mlp", M=8192, d=2048, F=8192),
    4: dict(kind="lmhead", M=8192, d=2048, V=128256),
    5: dict(kind="block", M=8192, d=4096, F=14336),
}
