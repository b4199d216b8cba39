"""Algorithmic work counts, roofline peaks and timing statistics.

Work is counted the way the roofline argument of "Week 13. GPUs and
FlashAttention", Step 1, counts it: FLOPs the method needs and bytes it must
move at least, not what a kernel happens to execute.

* Prefill FLOPs: 4 d per visible (query, key) pair (2 d for the score, 2 d
  for the weighted value sum).  Pairs hidden by the causal mask are not
  counted ("Week 13", Step 2: blocks above the diagonal are skipped).
* Prefill bytes: Q, K, V read once, O and lse written once.
* Decode bytes: K and V of every cached token actually attended to, read
  once (tokens of a partly filled last page past the length do not count),
  plus q, o and lse.  Decode FLOPs: 4 d per (query head, token).
"""

from __future__ import annotations

import math

import numpy as np

# MI355X published peaks (AMD specification; dense, no sparsity).
MI355X_BF16_DENSE_FLOPS = 2.5e15
MI355X_FP8_DENSE_FLOPS = 5.0e15
MI355X_FP32_VECTOR_FLOPS = 157.3e12
MI355X_HBM_BYTES_PER_S = 8.0e12


def visible_pairs(Sq: int, Sk: int, causal: bool) -> int:
    """Number of (query, key) pairs a head attends to (bottom-right causal mask)."""
    if not causal:
        return Sq * Sk
    per_row = np.clip(np.arange(Sq, dtype=np.int64) + (Sk - Sq) + 1, 0, Sk)
    return int(per_row.sum())


def prefill_flops(B: int, Hq: int, Sq: int, Sk: int, d: int, causal: bool) -> int:
    return 4 * d * B * Hq * visible_pairs(Sq, Sk, causal)


def backward_flops(B: int, Hq: int, Sq: int, Sk: int, d: int, causal: bool) -> int:
    """Algorithmic FLOPs of the attention backward: five products of 2 d FLOP
    per visible (query, key) pair (S recomputed, dP = dO V^T, dV, dK, dQ)."""
    return 10 * d * B * Hq * visible_pairs(Sq, Sk, causal)


def prefill_min_bytes(B: int, Hq: int, Hkv: int, Sq: int, Sk: int, d: int,
                      in_bytes: int = 2, out_bytes: int = 2, with_lse: bool = True) -> int:
    reads = (B * Hq * Sq * d + 2 * B * Hkv * Sk * d) * in_bytes
    writes = B * Hq * Sq * d * out_bytes + (B * Hq * Sq * 4 if with_lse else 0)
    return reads + writes


def fp8_quantize_bytes(BH: int, S: int, d: int, block_rows: int) -> int:
    """Bytes a block quantizer must move: bf16 input read once, one code byte
    and one scale byte per block written."""
    return BH * S * d * 2 + BH * S * d + BH * (-(-S // block_rows))


def decode_kv_bytes(seqlens, Hkv: int, d: int, elem_bytes: int = 2) -> int:
    """K and V bytes of the tokens attended to (one read each)."""
    return int(np.asarray(seqlens, dtype=np.int64).sum()) * Hkv * 2 * d * elem_bytes


def decode_total_bytes(seqlens, Hq: int, Hkv: int, d: int, elem_bytes: int = 2) -> int:
    n = len(seqlens)
    return decode_kv_bytes(seqlens, Hkv, d, elem_bytes) + 2 * n * Hq * d * elem_bytes + n * Hq * 4


def decode_flops(seqlens, Hq: int, d: int) -> int:
    return int(np.asarray(seqlens, dtype=np.int64).sum()) * Hq * 4 * d


def mla_latent_bytes(seqlens, d_c: int, elem_bytes: int = 2) -> int:
    """Latent-cache bytes of the tokens attended to: one d_c-wide latent per
    token, read once (it serves as the key and the value of every head)."""
    return int(np.asarray(seqlens, dtype=np.int64).sum()) * d_c * elem_bytes


def mla_total_bytes(seqlens, H: int, d_h: int, d_c: int, elem_bytes: int = 2) -> int:
    """Minimum HBM bytes of one latent-cache decode step: the latents, both
    up-projections once, the queries and the outputs (with lse)."""
    n = len(seqlens)
    return (mla_latent_bytes(seqlens, d_c, elem_bytes) + 2 * H * d_c * d_h * elem_bytes
            + 2 * n * H * d_h * elem_bytes + n * H * 4)


def mla_flops(seqlens, H: int, d_h: int, d_c: int) -> int:
    """Algorithmic FLOPs of latent-cache decode in the absorbed form: per head
    the query and output projections (2 d_c d_h each per sequence) and, per
    attended token, the score and the weighted latent sum (2 d_c each)."""
    n = len(seqlens)
    return int(np.asarray(seqlens, dtype=np.int64).sum()) * H * 4 * d_c + n * H * 4 * d_c * d_h


def decode_intensity(Hq: int, Hkv: int, elem_bytes: int = 2) -> float:
    """FLOP per KV byte of single-token decode: 4 d (Hq/Hkv) over 2 d elem_bytes."""
    return 4.0 * (Hq / Hkv) / (2.0 * elem_bytes)


def score_matrix_entries(S: int) -> int:
    return S * S


def score_matrix_bytes(S: int, heads: int, elem_bytes: int) -> int:
    """Bytes of the S x S score matrices of all heads of one layer and example."""
    return S * S * heads * elem_bytes


def memory_saving(S: int, head_dim: int) -> float:
    """Size of the S x S score matrix over the S x head_dim output."""
    return S / head_dim


def ridge_point(peak_flops: float, bytes_per_s: float) -> float:
    """Arithmetic intensity (FLOP/byte) where compute and memory time are equal."""
    return peak_flops / bytes_per_s


def t_critical_95(n: int) -> float:
    """Two-sided 95% Student-t quantile for a mean of n measurements (n-1 dof)."""
    from scipy.stats import t
    return float(t.ppf(0.975, n - 1))


def summarize(samples) -> dict:
    """mean, std, p50, p95 and the 95% confidence half-width of the mean."""
    x = np.asarray(samples, dtype=np.float64)
    n = len(x)
    out = dict(n=n, mean=float(x.mean()), p50=float(np.percentile(x, 50)),
               p95=float(np.percentile(x, 95)), min=float(x.min()))
    out["std"] = float(x.std(ddof=1)) if n > 1 else 0.0
    out["ci95"] = t_critical_95(n) * out["std"] / math.sqrt(n) if n > 1 else float("nan")
    return out
