"""GPU parity of latent-cache decode (fa_mla_decode) against the fp64 oracle
(oracle.mla_decode, which rebuilds every head's keys and values from the
latents).  Same bf16 tolerances as the other bf16 paths: max |dO| <= 2e-2,
rel-RMS <= 5e-3, lse within 1e-3 with -inf exactly where the oracle has -inf."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from exact_tiled_attention_14_amd import inputs as I  # noqa: E402

DEV = "cuda:0"
MAX_ABS, REL_RMS, LSE_TOL = 2e-2, 5e-3, 1e-3


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_tiled_attention_14_amd import binding
    binding.load()
    return binding


def _bf(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def _args(c, table=None):
    bt = c.cache.block_table if table is None else table
    return (_bf(I.bf16_bits(c.q)), _bf(I.bf16_bits(c.w_uk)), _bf(I.bf16_bits(c.w_uv_t)), _bf(c.ccache_bits),
            torch.from_numpy(np.ascontiguousarray(bt)).to(DEV), torch.from_numpy(c.cache.seqlens).to(DEV))


def run(Bm, c, table=None):
    o, lse = Bm.fa_mla_decode(*_args(c, table), c.scale)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def ref(c, table=None):
    bt = c.cache.block_table if table is None else table
    return oracle.mla_decode(c.q, c.w_uk, c.w_uv_t, c.ccache, bt, c.cache.seqlens, c.scale)


def check(o, lse, O, L, label):
    assert np.isfinite(o).all(), f"{label}: non-finite output"
    err = np.abs(o - O)
    ma = float(err.max())
    rr = float(np.sqrt((err ** 2).sum() / max((O ** 2).sum(), 1e-300)))
    print(f"{label}: max_abs={ma:.3e} rel_rms={rr:.3e}", flush=True)
    assert ma <= MAX_ABS and rr <= REL_RMS, label
    ninf = np.isneginf(L)
    assert (np.isneginf(lse) == ninf).all(), f"{label}: -inf pattern"
    if (~ninf).any():
        e = float(np.abs(lse[~ninf] - L[~ninf]).max())
        print(f"{label}: lse max_abs={e:.3e}", flush=True)
        assert e <= LSE_TOL, label


@pytest.mark.parametrize("H", [16, 1, 7, 32, 40, 128])
def test_head_counts(B, H):
    c = I.make_mla_decode(5 if H <= 40 else 3, H, 128, 512, len_lo=1, len_hi=700, seed=40 + H)
    o, lse = run(B, c)
    O, L = ref(c)
    check(o, lse, O, L, f"H{H}")


def test_ragged_lengths_and_nan_tails(B):
    lens = np.array([1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 511, 512, 513, 1000], dtype=np.int32)
    c = I.make_mla_decode(len(lens), 16, 128, 512, len_lo=1, len_hi=1024, seed=71, seqlens=lens, poison_tail=True)
    o, lse = run(B, c)
    O, L = ref(c)
    check(o, lse, O, L, "ragged + NaN tails")


@pytest.mark.parametrize("lens", [[512], [513, 4100], [8192, 2047, 6000], [70, 1025, 2090, 40]],
                         ids=["one-chunk", "two", "three", "partial-chunks"])
def test_long_sequences_split_in_chunks(B, lens):
    lens = np.array(lens, dtype=np.int32)
    c = I.make_mla_decode(len(lens), 16, 128, 512, len_lo=1, len_hi=8192, seed=int(lens.sum()) % 991, seqlens=lens)
    o, lse = run(B, c)
    O, L = ref(c)
    check(o, lse, O, L, f"chunks {lens.tolist()}")


def test_one_long_sequence_split_over_the_chip(B):
    """40,000 tokens of one sequence: the work split cuts it into hundreds of
    parts that the combine kernel merges."""
    c = I.make_mla_decode(1, 16, 128, 512, len_lo=1, len_hi=40000, seed=5, seqlens=np.array([40000], np.int32))
    o, lse = run(B, c)
    O, L = ref(c)
    check(o, lse, O, L, "one long sequence")


def test_more_sequences_than_resident_workgroups(B):
    """700 short sequences: one part each, more work items than stay resident."""
    c = I.make_mla_decode(700, 16, 128, 512, len_lo=0, len_hi=90, seed=6)
    o, lse = run(B, c)
    O, L = ref(c)
    check(o, lse, O, L, "700 sequences")


def test_empty_sequence_and_bad_block_ids(B):
    lens = np.array([0, 40, 600], dtype=np.int32)
    c = I.make_mla_decode(3, 16, 128, 512, len_lo=1, len_hi=600, seed=9, seqlens=lens)
    table = c.cache.block_table.copy()
    table[2, 1] = 10 ** 6                     # tokens 16..31 of sequence 2: no key
    table[2, 33] = -5                         # tokens 528..543 (second chunk): no key
    o, lse = run(B, c, table)
    O, L = ref(c)
    check(o[:2], lse[:2], O[:2], L[:2], "empty + valid")
    assert (o[0] == 0).all() and np.isneginf(lse[0]).all()
    # sequence 2 without the two pages, by the oracle over the remaining pages
    keep = [p for p in range(38) if p not in (1, 33)]
    pages = c.cache.block_table[2, keep]
    n = 16 * (len(keep) - 1) + (600 - 16 * 37)
    t2 = np.full((1, c.cache.block_table.shape[1]), -1, dtype=np.int32)
    t2[0, :len(keep)] = pages
    O2, L2 = oracle.mla_decode(c.q[2:3], c.w_uk, c.w_uv_t, c.ccache, t2, np.array([n], dtype=np.int32), c.scale)
    check(o[2:3], lse[2:3], O2, L2, "bad block ids")


def test_selecting_projections_match_paged_decode(B):
    """With w_uk[h] = [I; 0] and w_uv_t[h] = [0, I, 0, 0] the latent decode is
    multi-query decode (one K/V head) with K = c[:, :128], V = c[:, 128:256]:
    both library paths on the same cache must agree."""
    c = I.make_mla_decode(6, 8, 128, 512, len_lo=100, len_hi=3000, seed=23)     # 8 heads per K/V head
    eye = np.eye(128, dtype=np.float32)
    wk = np.zeros_like(c.w_uk)
    wk[:, :128, :] = eye
    wv = np.zeros_like(c.w_uv_t)
    wv[:, :, 128:256] = eye
    c2 = I.MLACase(q=c.q, w_uk=wk, w_uv_t=wv, cache=c.cache, scale=c.scale)
    o, lse = run(B, c2)
    cb = c.ccache_bits
    kc = np.ascontiguousarray(cb[:, None, :, :128])
    vc = np.ascontiguousarray(cb[:, None, :, 128:256])
    o1, l1 = B.fa_decode(_bf(I.bf16_bits(c.q)), _bf(kc), _bf(vc), torch.from_numpy(c.cache.block_table).to(DEV),
                         torch.from_numpy(c.cache.seqlens).to(DEV), c.scale)
    torch.cuda.synchronize()
    assert np.abs(o - o1.float().cpu().numpy()).max() <= MAX_ABS / 2
    assert np.abs(lse - l1.cpu().numpy()).max() <= LSE_TOL


def test_mla_workload_full(B):
    """The 64-sequence, 16-head, 512-latent workload in the benchmark's launch
    configuration, every sequence and every element."""
    c = I.workload("mla_decode_64seq_h16_dc512")
    o, lse = run(B, c)
    O, L = ref(c)
    check(o, lse, O, L, "mla workload (64 sequences)")


def test_binding_errors(B):
    c = I.make_mla_decode(2, 16, 128, 512, len_lo=10, len_hi=20, seed=1)
    q, wk, wv, cc, bt, sl = _args(c)
    with pytest.raises(B.FAError) as e:
        B.fa_mla_decode(q, wk, wv, cc, bt, sl, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    assert e.value.status == B.FA_ERR_WORKSPACE
    q129 = torch.zeros((2, 129, 128), dtype=torch.bfloat16, device=DEV)
    w129 = torch.zeros((129, 512, 128), dtype=torch.bfloat16, device=DEV)
    v129 = torch.zeros((129, 128, 512), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(B.FAError) as e:
        B.fa_mla_decode(q129, w129, v129, cc, bt, sl)
    assert e.value.status == B.FA_ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        B.fa_mla_decode(q, wv, wk, cc, bt, sl)
