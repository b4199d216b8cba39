"""The allocation-free decode entry point (fa_decode_noalloc) against the
workspace one (fa_decode), through the C ABI: same kernels, the scratch in
the library's fixed per-GPU array instead of a caller workspace.  Two calls
in a row, the second smaller (the array keeps the first call's contents),
and a size beyond the array's capacity is refused before any launch."""

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


def _dev_args(d):
    return (_bf(d.bits("q")), _bf(d.kcache_bits), _bf(d.vcache_bits), torch.from_numpy(d.block_table).to(DEV),
            torch.from_numpy(d.seqlens).to(DEV))


def _both(B, d):
    """(o, lse) of fa_decode and of fa_decode_noalloc on the same inputs."""
    args = _dev_args(d)
    o_ws, l_ws = B.fa_decode(*args, d.scale)
    o_na = torch.empty_like(o_ws)
    l_na = torch.empty_like(l_ws)
    B.fa_decode_noalloc(*args, d.scale, out=o_na, lse=l_na)
    torch.cuda.synchronize()
    return o_ws, l_ws, o_na, l_na


def _check(o_na, l_na, o_ws, l_ws, d, label):
    o = o_na.float().cpu().numpy().astype(np.float64)
    lse = l_na.cpu().numpy().astype(np.float64)
    # against the workspace entry point: the same kernels and split, so the same bits
    assert torch.equal(o_na.view(torch.int16), o_ws.view(torch.int16)), f"{label}: o differs from fa_decode"
    assert np.array_equal(lse, l_ws.cpu().numpy().astype(np.float64), equal_nan=True), f"{label}: lse differs"
    # and to the oracle, at the bf16 tolerances
    O, L = oracle.paged_decode(d.q, d.kcache, d.vcache, d.block_table, d.seqlens, d.scale)
    err = np.abs(o - O)
    ma, rr = float(err.max()), float(np.sqrt((err ** 2).sum() / (O ** 2).sum()))
    print(f"{label}: max_abs={ma:.3e} rel_rms={rr:.3e}", flush=True)
    assert ma <= MAX_ABS and rr <= REL_RMS
    fin = np.isfinite(L)
    assert (np.isneginf(lse) == np.isneginf(L)).all()
    assert float(np.abs(lse[fin] - L[fin]).max()) <= LSE_TOL


def test_noalloc_matches_workspace_decode_twice(B):
    big = I.workload("paged_decode_64seq_h32kv8_d128")
    assert B.fa_decode_workspace_size(64, 32, 8, 128, 16, big.block_table.shape[1]) <= \
        B.FA_DECODE_NOALLOC_SCRATCH_BYTES
    o_ws, l_ws, o_na, l_na = _both(B, big)
    _check(o_na, l_na, o_ws, l_ws, big, "decode workload")
    # second call, smaller: the array still holds the first call's partials
    small = I.make_decode(5, 8, 2, 128, len_lo=1, len_hi=900, seed=91, poison_tail=True)
    o_ws, l_ws, o_na, l_na = _both(B, small)
    _check(o_na, l_na, o_ws, l_ws, small, "smaller second call")


def test_noalloc_refuses_sizes_beyond_its_array(B):
    # 8 query heads per K/V head, 2000 sequences x 8 K/V heads: the decode needs
    # more scratch than the array holds
    nseq, Hq, Hkv = 2000, 64, 8
    need = B.fa_decode_workspace_size(nseq, Hq, Hkv, 128, 16, 4)
    assert need > B.FA_DECODE_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((nseq, Hq, 128), dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros((4, Hkv, 16, 128), dtype=torch.bfloat16, device=DEV)
    bt = torch.zeros((nseq, 4), dtype=torch.int32, device=DEV)
    sl = torch.ones((nseq,), dtype=torch.int32, device=DEV)
    o = torch.full_like(q, 7.0)
    lse = torch.full((nseq, Hq), 7.0, dtype=torch.float32, device=DEV)
    with pytest.raises(B.FAError) as e:
        B.fa_decode_noalloc(q, kc, kc, bt, sl, out=o, lse=lse)
    assert e.value.status == B.FA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((o == 7.0).all()) and bool((lse == 7.0).all())      # nothing was launched
