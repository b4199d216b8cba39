"""FP8 block quantization with incoherent processing, and attention of the
quantized inputs: fp64 reference (test infrastructure only).

"FlashAttention scaling, multi-GPU training and weight quantization",
section 1 (FP8 low-precision support): the FP8 forward keeps Q, K and V in an
8-bit float format; each small tile is scaled independently (block
quantization), and Q and K are first multiplied by a random orthogonal matrix
(incoherent processing), which leaves Q K^T unchanged while spreading an
outlier over the whole head dimension.  "Hardware Co-Design", section on
number formats: FP8 is an 8-bit floating-point format.

The pages name neither the 8-bit encoding nor the scale rule; the readings
taken here are:

* Encoding: OCP E4M3 (also called E4M3FN): 1 sign bit, 4 exponent bits with
  bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN, largest finite
  value 448, subnormals m/8 * 2^-6.  Rounding to nearest, ties to even.
* Scale of a block: the smallest power of two s with amax / s <= 448 (amax =
  largest magnitude in the block); an all-zero block has s = 1.  Code =
  round(x / s); the value a code stands for is its E4M3 value times s.  A
  power of two keeps x / s and the dequantisation exact.
* Block: ``block_rows`` consecutive rows of one (batch, head) slice.
* Rotation: every row vector x -> R x (the rows times R^T) with one d x d
  orthogonal matrix R for Q and K, so that (q R^T)(k R^T)^T = q k^T and the
  scores are unchanged; V is not rotated (that would change O).

Functions here quantize and dequantize from these definitions and compute the
attention of the dequantized tensors with :func:`oracle.sdpa`.
"""

from __future__ import annotations

import numpy as np

from .attention import sdpa

__all__ = [
    "E4M3_MAX",
    "e4m3_values",
    "e4m3_round",
    "e4m3_encode",
    "e4m3_decode",
    "block_scale_exponent",
    "quantize_blocks",
    "dequantize_blocks",
    "sdpa_fp8",
]

E4M3_MAX = 448.0


def _decode_one(code: int) -> float:
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    v = (m / 8.0) * 2.0 ** -6 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


def e4m3_values() -> np.ndarray:
    """The 256 code values (float64, index = code byte)."""
    return np.array([_decode_one(c) for c in range(256)], dtype=np.float64)


_TABLE = e4m3_values()


def e4m3_decode(codes) -> np.ndarray:
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_round(x) -> np.ndarray:
    """Round to the nearest E4M3 value, ties to even; |x| must not exceed the
    largest finite value (448) by half a step or more (no saturation: the
    block scale rule never produces such a value)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)                      # a = f 2^e, f in [0.5, 1)
    step_exp = np.maximum(e - 1, -6) - 3    # quantum 2^(E-3); subnormals share 2^-9
    step = np.ldexp(1.0, step_exp)
    r = np.rint(a / step) * step            # np.rint rounds half to even
    if np.any(r > E4M3_MAX):
        raise ValueError("value out of E4M3 range")
    return np.copysign(r, x)


def e4m3_encode(x) -> np.ndarray:
    """Code bytes of round-to-nearest-even E4M3 (sign kept, so -0 -> 0x80)."""
    r = e4m3_round(x)
    a = np.abs(r)
    _, e = np.frexp(a)
    normal = a >= 2.0 ** -6
    exp_field = np.where(normal, e - 1 + 7, 0)
    mant = np.where(normal, np.rint(a / np.ldexp(1.0, e - 1) * 8) - 8, np.rint(a / 2.0 ** -9))
    code = (exp_field.astype(np.int64) << 3) | mant.astype(np.int64)
    code = code | (np.signbit(r).astype(np.int64) << 7)
    return code.astype(np.uint8)


def block_scale_exponent(amax) -> np.ndarray:
    """e with 2^e the block scale: the smallest integer such that
    amax <= 448 * 2^e.  Integer logic on amax = M 2^E (M in [1, 2)):
    448 = 1.75 * 2^8, so e = E - 8, plus one when M > 1.75; e = 0 for 0.
    The scale is stored as an E8M0 byte, so e is clamped to [-127, 127]."""
    a = np.asarray(amax, dtype=np.float64)
    f, e2 = np.frexp(a)                     # a = f 2^e2, f in [0.5, 1): M = 2f, E = e2 - 1
    e = np.clip((e2 - 1) - 8 + (2.0 * f > 1.75), -127, 127)
    return np.where(a > 0, e, 0).astype(np.int64)


def quantize_blocks(x, block_rows: int, rot=None):
    """Quantize [..., S, d] per block of ``block_rows`` rows.

    ``rot`` (d x d, optional) rotates every row first (x -> rot x, i.e. the
    rows times rot^T).
    Returns (codes uint8 [..., S, d], scale exponents int64 [..., nblk]);
    the value of element (r, c) is e4m3(codes) * 2^exp[r // block_rows].
    """
    x = np.asarray(x, dtype=np.float64)
    if rot is not None:
        x = x @ np.asarray(rot, dtype=np.float64).T
    S = x.shape[-2]
    nblk = -(-S // block_rows)
    pad = nblk * block_rows - S
    xp = np.concatenate([x, np.zeros(x.shape[:-2] + (pad, x.shape[-1]))], axis=-2) if pad else x
    blocks = xp.reshape(x.shape[:-2] + (nblk, block_rows, x.shape[-1]))
    amax = np.abs(blocks).max(axis=(-2, -1))
    ex = block_scale_exponent(amax)
    scaled = blocks / np.ldexp(1.0, ex)[..., None, None]
    codes = e4m3_encode(scaled).reshape(xp.shape)[..., :S, :]
    return codes, ex


def dequantize_blocks(codes, exps, block_rows: int) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    S = codes.shape[-2]
    rows = np.arange(S) // block_rows
    s = np.ldexp(1.0, np.asarray(exps, dtype=np.int64))[..., rows]
    return e4m3_decode(codes) * s[..., None]


def sdpa_fp8(q8, q_exp, k8, k_exp, v8, v_exp, causal: bool, scale: float,
             q_rows: int = 128, kv_rows: int = 64):
    """Exact attention (fp64, :func:`oracle.sdpa`) of the dequantized
    tensors; q8 [B,Hq,Sq,d], k8 and v8 [B,Hkv,Sk,d] codes in the plain
    row-major layout, with their block scale exponents."""
    q = dequantize_blocks(q8, q_exp, q_rows)
    k = dequantize_blocks(k8, k_exp, kv_rows)
    v = dequantize_blocks(v8, v_exp, kv_rows)
    return sdpa(q, k, v, causal, scale)
