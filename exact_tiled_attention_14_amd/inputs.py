"""Seeded synthetic inputs for the attention workloads.

This module holds no attention arithmetic.  It draws random numbers, rounds
them to bfloat16 and lays out a paged cache; the fp64 oracle and the HIP
library both consume exactly what it returns, so the two sides see the same
bits.

Recipe (every stream comes from ``numpy.random.Generator(PCG64)`` seeded by
``SeedSequence(seed).spawn``; one child stream per tensor, so adding a tensor
never changes another one):

* Q, K, V: i.i.d. N(0, 1) drawn in fp32, then rounded to bf16 with
  round-to-nearest-even (bf16 workloads) or kept fp32 (fp32 workload).
* Outliers: ``round(frac * K.size)`` distinct scalar positions of K, chosen
  uniformly without replacement, multiplied by ``outlier_scale`` in fp32
  before the bf16 rounding.
* Checked-row subsets: per (batch, head), distinct rows chosen uniformly
  without replacement, sorted.
* Paged cache: sequence lengths uniform integers in [lo, hi]; a sequence of
  length n owns ceil(n / block_size) blocks; physical block ids are a random
  permutation of 0..num_blocks-1 handed out in (sequence, logical block)
  order; unused block-table entries hold -1; cache slots past a sequence's
  length hold N(0, 1) values (or NaN when ``poison_tail``).
"""

from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

__all__ = [
    "bf16_bits",
    "bf16_to_f32",
    "round_to_bf16",
    "PrefillCase",
    "DecodeCase",
    "make_prefill",
    "make_decode",
    "WORKLOADS",
    "workload",
]


# --- bfloat16 as uint16 bit patterns --------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16) with round-to-nearest-even.

    NaN stays a quiet NaN.  Finite values that round past the largest bf16
    become +-inf, as IEEE rounding prescribes.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    has_nan = bool(nan.any())
    # Non-NaN patterns are <= 0xFF800000, so the sum cannot wrap in uint32.
    t = np.right_shift(u, 16)
    np.bitwise_and(t, 1, out=t)
    t += 0x7FFF
    if has_nan:
        t[nan] = 0
    t += u
    t >>= 16
    out = t.astype(np.uint16)
    if has_nan:
        out[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit pattern (uint16) -> the exactly equal fp32 value."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16, returned as fp32."""
    return bf16_to_f32(bf16_bits(x))


_CHUNK = 1 << 22


def _round_bf16_inplace(x: np.ndarray) -> None:
    """Round a contiguous fp32 array to bf16 values in place, chunk by chunk.

    Same rounding as :func:`bf16_bits` (nearest, ties to even), without
    allocating a full-size temporary.
    """
    u = x.reshape(-1).view(np.uint32)
    tmp = np.empty(min(_CHUNK, u.size), dtype=np.uint32)
    for a in range(0, u.size, _CHUNK):
        c = u[a:a + _CHUNK]
        t = tmp[:c.size]
        nan = np.isnan(c.view(np.float32))
        np.right_shift(c, 16, out=t)
        np.bitwise_and(t, 1, out=t)
        t += 0x7FFF
        has_nan = bool(nan.any())
        if has_nan:
            t[nan] = 0
        t += c
        t &= 0xFFFF0000
        if has_nan:                    # NaN stays a quiet NaN
            t[nan] = (c[nan] | 0x00400000) & 0xFFFF0000
        c[...] = t


def _streams(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def _normal(rng, shape) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    flat = out.reshape(-1)
    for a in range(0, flat.size, _CHUNK):
        rng.standard_normal(dtype=np.float32, out=flat[a:a + _CHUNK])
    return out


# --- prefill ---------------------------------------------------------------

@dataclass
class PrefillCase:
    """One prefill workload: tensors as fp32 values (bf16-exact when bf16)."""
    q: np.ndarray            # [B, Hq, Sq, d] float32
    k: np.ndarray            # [B, Hkv, Sk, d] float32
    v: np.ndarray            # [B, Hkv, Sk, d] float32
    causal: bool
    scale: float
    dtype: str               # "bf16" or "f32"
    seed: int
    rows: np.ndarray | None = None   # [B, Hq, R] checked query rows, or None
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        B, Hq, Sq, d = self.q.shape
        return dict(B=B, Hq=Hq, Hkv=self.k.shape[1], Sq=Sq, Sk=self.k.shape[2], d=d)

    def bits(self, name: str) -> np.ndarray:
        """The bf16 bit patterns of tensor ``name`` (bf16 cases only)."""
        if self.dtype != "bf16":
            raise ValueError("bit patterns exist only for bf16 cases")
        return bf16_bits(getattr(self, name))


def make_prefill(B: int, Hq: int, Hkv: int, Sq: int, Sk: int, d: int, *, causal: bool,
                 dtype: str = "bf16", seed: int = 0, scale: float | None = None,
                 outlier_frac: float = 0.0, outlier_scale: float = 20.0,
                 check_rows: int | None = None) -> PrefillCase:
    """Seeded N(0,1) Q, K, V of the given shape (see the module recipe)."""
    if dtype not in ("bf16", "f32"):
        raise ValueError(dtype)
    rq, rk, rv, ro, rr = _streams(seed, 5)
    q = _normal(rq, (B, Hq, Sq, d))
    k = _normal(rk, (B, Hkv, Sk, d))
    v = _normal(rv, (B, Hkv, Sk, d))
    n_out = int(round(outlier_frac * k.size))
    if n_out:
        pos = ro.choice(k.size, size=n_out, replace=False)
        k.reshape(-1)[pos] *= np.float32(outlier_scale)
    if dtype == "bf16":
        for t in (q, k, v):
            _round_bf16_inplace(t)
    rows = None
    if check_rows is not None:
        R = min(check_rows, Sq)
        rows = np.stack([np.stack([np.sort(rr.choice(Sq, size=R, replace=False))
                                   for _ in range(Hq)]) for _ in range(B)])
    return PrefillCase(q=q, k=k, v=v, causal=causal,
                       scale=float(scale if scale is not None else 1.0 / math.sqrt(d)),
                       dtype=dtype, seed=seed, rows=rows,
                       meta=dict(outliers=n_out))


def make_rotation(d: int, *, seed: int = 0) -> np.ndarray:
    """A seeded random orthogonal d x d matrix (Haar distributed: QR of a
    Gaussian matrix with the signs of R's diagonal moved into Q), rounded to
    bf16 values (fp32 array).  The incoherent processing of the FP8 forward
    multiplies Q and K by it; it is an input like any other random draw."""
    (rr,) = _streams(seed + 0x51ED, 1)
    g = rr.standard_normal((d, d))
    qm, r = np.linalg.qr(g)
    qm = qm * np.sign(np.diag(r))[None, :]
    out = qm.astype(np.float32)
    _round_bf16_inplace(out)
    return out


# --- paged decode ----------------------------------------------------------

def make_grad_out(shape, *, seed: int = 0, dtype: str = "bf16") -> np.ndarray:
    """Seeded N(0,1) upstream gradient dO of the given shape (bf16-exact
    fp32 for dtype "bf16"), from its own stream: the backward workloads pair
    it with ``make_prefill`` inputs of the same seed."""
    (rg,) = _streams(seed + 0x9E3779B9, 1)
    g = _normal(rg, tuple(shape))
    if dtype == "bf16":
        _round_bf16_inplace(g)
    return g


@dataclass
class DecodeCase:
    """One paged decode step: one new query token per sequence, or Sq new
    tokens per sequence (``q`` [nseq, Sq, Hq, d]) for a multi-query step.

    The caches are kept as bf16 bit patterns (uint16) because they are large;
    :meth:`subset` extracts a few sequences with their pages as fp32 values.
    """
    q: np.ndarray            # [nseq, Hq, d] or [nseq, Sq, Hq, d] float32 (bf16-exact)
    kcache_bits: np.ndarray  # [num_blocks, Hkv, block_size, d] uint16 (bf16; NaN allowed in tails)
    vcache_bits: np.ndarray  # same
    block_table: np.ndarray  # [nseq, max_blocks] int32, -1 past a sequence's blocks
    seqlens: np.ndarray      # [nseq] int32
    scale: float
    seed: int

    @property
    def shape(self):
        if self.q.ndim == 4:
            nseq, Sq, Hq, d = self.q.shape
        else:
            (nseq, Hq, d), Sq = self.q.shape, 1
        nb, Hkv, bs, _ = self.kcache_bits.shape
        return dict(nseq=nseq, Sq=Sq, Hq=Hq, Hkv=Hkv, d=d, block_size=bs, num_blocks=nb,
                    max_blocks=self.block_table.shape[1])

    @property
    def kcache(self) -> np.ndarray:
        return bf16_to_f32(self.kcache_bits)

    @property
    def vcache(self) -> np.ndarray:
        return bf16_to_f32(self.vcache_bits)

    def bits(self, name: str) -> np.ndarray:
        if name in ("kcache", "vcache"):
            return getattr(self, name + "_bits")
        return bf16_bits(getattr(self, name))

    @property
    def kv_tokens(self) -> int:
        return int(self.seqlens.astype(np.int64).sum())

    def subset(self, seqs) -> "DecodeCase":
        """The listed sequences alone, their pages copied out and renumbered."""
        seqs = [int(s) for s in seqs]
        bs = self.kcache_bits.shape[2]
        ids = []
        table = np.full((len(seqs), self.block_table.shape[1]), -1, dtype=np.int32)
        for i, s in enumerate(seqs):
            n_pages = -(-int(self.seqlens[s]) // bs)
            table[i, :n_pages] = np.arange(len(ids), len(ids) + n_pages)
            ids.extend(int(x) for x in self.block_table[s, :n_pages])
        ids = np.asarray(ids, dtype=np.int64)
        return DecodeCase(q=self.q[seqs].copy(), kcache_bits=self.kcache_bits[ids],
                          vcache_bits=self.vcache_bits[ids], block_table=table,
                          seqlens=self.seqlens[seqs].copy(), scale=self.scale, seed=self.seed)


def _normal_bf16_bits(rng, shape) -> np.ndarray:
    """N(0,1) fp32 draws rounded to bf16, stored straight as bit patterns."""
    out = np.empty(shape, dtype=np.uint16).reshape(-1)
    buf = np.empty(min(_CHUNK, out.size), dtype=np.float32)
    for a in range(0, out.size, _CHUNK):
        c = buf[:min(_CHUNK, out.size - a)]
        rng.standard_normal(dtype=np.float32, out=c)
        _round_bf16_inplace(c)
        out[a:a + c.size] = c.view(np.uint32) >> 16
    return out.reshape(shape)


def make_decode(nseq: int, Hq: int, Hkv: int, d: int, *, len_lo: int, len_hi: int,
                block_size: int = 16, seed: int = 0, scale: float | None = None,
                max_blocks: int | None = None, poison_tail: bool = False,
                seqlens: np.ndarray | None = None, sq: int = 0) -> DecodeCase:
    """Seeded paged-cache decode inputs (see the module recipe).  ``sq`` > 0
    gives ``sq`` new query tokens per sequence (q [nseq, sq, Hq, d]); the
    cache holds them as the last ``sq`` tokens of each sequence."""
    rq, rl, rp, rk, rv = _streams(seed, 5)
    if seqlens is None:
        seqlens = rl.integers(len_lo, len_hi, size=nseq, endpoint=True)
    seqlens = np.asarray(seqlens, dtype=np.int32)
    pages = (seqlens.astype(np.int64) + block_size - 1) // block_size
    num_blocks = int(pages.sum())
    if max_blocks is None:
        max_blocks = max(1, -(-len_hi // block_size))
    if pages.max(initial=0) > max_blocks:
        raise ValueError("a sequence needs more blocks than max_blocks")
    perm = rp.permutation(num_blocks).astype(np.int32)
    table = np.full((nseq, max_blocks), -1, dtype=np.int32)
    cursor = 0
    for s in range(nseq):
        table[s, :pages[s]] = perm[cursor:cursor + pages[s]]
        cursor += pages[s]
    shape = (max(num_blocks, 1), Hkv, block_size, d)
    kc = _normal_bf16_bits(rk, shape)
    vc = _normal_bf16_bits(rv, shape)
    if poison_tail:
        nan_bits = np.uint16(0x7FC0)
        for s in range(nseq):
            n = int(seqlens[s])
            if n % block_size and pages[s]:
                last = table[s, pages[s] - 1]
                kc[last, :, n % block_size:, :] = nan_bits
                vc[last, :, n % block_size:, :] = nan_bits
    q = _normal(rq, (nseq, sq, Hq, d) if sq > 0 else (nseq, Hq, d))
    _round_bf16_inplace(q)
    return DecodeCase(q=q, kcache_bits=kc, vcache_bits=vc, block_table=table, seqlens=seqlens,
                      scale=float(scale if scale is not None else 1.0 / math.sqrt(d)), seed=seed)


@dataclass
class MLACase:
    """One latent-cache decode step: a query token per sequence, a paged
    cache of d_c-dimensional latents, and per-head up-projections."""
    q: np.ndarray            # [nseq, H, d_h] float32 (bf16-exact)
    w_uk: np.ndarray         # [H, d_c, d_h] float32 (bf16-exact): K = c W_uk[h]
    w_uv_t: np.ndarray       # [H, d_h, d_c] float32 (bf16-exact): V = c W_uv_t[h]^T
    cache: DecodeCase        # latent pages: kcache_bits [num_blocks, 1, block_size, d_c]
    scale: float

    @property
    def ccache(self) -> np.ndarray:
        return self.cache.kcache[:, 0]

    @property
    def ccache_bits(self) -> np.ndarray:
        return np.ascontiguousarray(self.cache.kcache_bits[:, 0])

    @property
    def shape(self):
        nseq, H, dh = self.q.shape
        cs = self.cache.shape
        return dict(nseq=nseq, H=H, d_h=dh, d_c=self.w_uk.shape[1], block_size=cs["block_size"],
                    num_blocks=cs["num_blocks"], max_blocks=cs["max_blocks"])

    def subset(self, seqs) -> "MLACase":
        """The listed sequences alone, their latent pages copied out and renumbered."""
        seqs = [int(s) for s in seqs]
        return MLACase(q=self.q[seqs].copy(), w_uk=self.w_uk, w_uv_t=self.w_uv_t, cache=self.cache.subset(seqs),
                       scale=self.scale)


def make_mla_decode(nseq: int, H: int, d_h: int, d_c: int, *, len_lo: int, len_hi: int, seed: int = 0,
                    seqlens: np.ndarray | None = None, poison_tail: bool = False) -> MLACase:
    """Seeded latent-cache decode inputs: the paged latent cache as in
    :func:`make_decode` (one "head" of width d_c), q ~ N(0,1), and
    up-projections ~ N(0, 1/d_c) so that reconstructed keys and values have
    unit variance; everything rounded to bf16."""
    cache = make_decode(nseq, 1, 1, d_c, len_lo=len_lo, len_hi=len_hi, seed=seed, seqlens=seqlens,
                        poison_tail=poison_tail)
    rq, rk, rv = _streams(seed + 0x4D4C41, 3)
    q = _normal(rq, (nseq, H, d_h))
    wk = _normal(rk, (H, d_c, d_h)) * np.float32(1.0 / math.sqrt(d_c))
    wv = _normal(rv, (H, d_h, d_c)) * np.float32(1.0 / math.sqrt(d_c))
    for t in (q, wk, wv):
        _round_bf16_inplace(t)
    return MLACase(q=q, w_uk=wk, w_uv_t=wv, cache=cache, scale=1.0 / math.sqrt(d_h))


# --- the five named workloads ---------------------------------------------

WORKLOADS = {
    "mha1_s128_d64_f32": dict(kind="prefill", seed=1, B=1, Hq=1, Hkv=1, Sq=128, Sk=128, d=64,
                              causal=False, dtype="f32"),
    "causal_mha_b2_h16_s2048_d128": dict(kind="prefill", seed=2, B=2, Hq=16, Hkv=16, Sq=2048,
                                         Sk=2048, d=128, causal=True, dtype="bf16"),
    "causal_gqa_h32kv8_s8192_d128_outliers": dict(kind="prefill", seed=3, B=1, Hq=32, Hkv=8,
                                                  Sq=8192, Sk=8192, d=128, causal=True,
                                                  dtype="bf16", outlier_frac=0.001,
                                                  outlier_scale=20.0),
    "causal_gqa_h32kv8_s32768_d128": dict(kind="prefill", seed=4, B=1, Hq=32, Hkv=8, Sq=32768,
                                          Sk=32768, d=128, causal=True, dtype="bf16",
                                          check_rows=512),
    "paged_decode_64seq_h32kv8_d128": dict(kind="decode", seed=5, nseq=64, Hq=32, Hkv=8, d=128,
                                           len_lo=1024, len_hi=8192, block_size=16),
    # multi-query verify step: the decode workload with 8 new tokens per
    # sequence (7 draft tokens + 1), so a K/V head's 4 query heads x 8 tokens
    # fill one 32-row matrix-core tile
    "paged_verify_64seq_q8_h32kv8_d128": dict(kind="decode", seed=6, nseq=64, Hq=32, Hkv=8, d=128,
                                              len_lo=1024, len_hi=8192, block_size=16, sq=8),
    # latent-cache decode: 64 sequences, 16 heads of 128 reading one
    # 512-wide latent per token (keys and values rebuilt by up-projection)
    "mla_decode_64seq_h16_dc512": dict(kind="mla", seed=7, nseq=64, H=16, d_h=128, d_c=512,
                                       len_lo=1024, len_hi=8192),
}


def workload(name: str, **overrides):
    """Build one of :data:`WORKLOADS` (keyword overrides allowed, e.g. ``seed``)."""
    spec = dict(WORKLOADS[name])
    spec.update(overrides)
    kind = spec.pop("kind")
    if kind == "prefill":
        return make_prefill(**spec)
    if kind == "mla":
        return make_mla_decode(**spec)
    return make_decode(**spec)
