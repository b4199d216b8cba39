"""GPU parity of the attention backward (fa_bwd) against the fp64 oracle.

The kernel gets the oracle's forward outputs as its inputs (O rounded to bf16,
lse in fp32), so the test isolates the backward kernels.  Tolerance (derived
from the arithmetic, see the design notes): per gradient tensor,
||dX_gpu - dX_ref||_2 / ||dX_ref||_2 <= 1e-2 and max |dX_gpu - dX_ref| <=
2e-2 * max |dX_ref|.  The kernels round P and dS once to bf16 (relative
2^-9) as matrix-core operands, read O rounded to bf16 (which moves
D = rowsum(dO * O) by the same relative amount) and round each gradient once
to bf16 at the end; these independent relative errors of ~2^-9 give a
relative RMS error of a few 1e-3.
"""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
from exact_tiled_attention_14_amd import inputs as I  # noqa: E402

REL_RMS, MAX_REL = 1e-2, 2e-2
DEV = "cuda:0"


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_tiled_attention_14_amd import binding
    binding.load()
    return binding


def _bf(x):
    return torch.from_numpy(np.ascontiguousarray(I.bf16_bits(np.asarray(x, np.float32))).view(np.int16)) \
        .view(torch.bfloat16).to(DEV)


def _np(t):
    return t.float().cpu().numpy().astype(np.float64)


def check_grad(got, want, label):
    assert np.isfinite(got).all(), f"{label}: non-finite gradient"
    err = got - want
    ref = float(np.sqrt((want ** 2).sum()))
    rr = float(np.sqrt((err ** 2).sum())) / max(ref, 1e-300)
    scale = float(np.abs(want).max()) if want.size else 0.0
    ma = float(np.abs(err).max()) if err.size else 0.0
    print(f"{label}: rel_rms={rr:.3e} max_abs={ma:.3e} (max |ref| {scale:.3e})", flush=True)
    assert rr <= REL_RMS, f"{label}: rel_rms {rr:.3e}"
    assert ma <= MAX_REL * max(scale, 1e-30), f"{label}: max_abs {ma:.3e} vs max |ref| {scale:.3e}"


def run_bwd(Bm, c, do):
    """Oracle forward outputs -> fa_bwd; returns GPU (dq, dk, dv) and the oracle's."""
    O, L = oracle.sdpa(c.q, c.k, c.v, c.causal, c.scale)
    q, k, v = _bf(c.q), _bf(c.k), _bf(c.v)
    o, g = _bf(I.round_to_bf16(O.astype(np.float32))), _bf(do)
    lse = torch.from_numpy(L.astype(np.float32)).to(DEV)
    dq, dk, dv = Bm.fa_bwd(q, k, v, o, g, lse, c.causal, c.scale)
    torch.cuda.synchronize()
    ref = oracle.sdpa_backward(c.q, c.k, c.v, do, c.causal, c.scale)
    return (_np(dq), _np(dk), _np(dv)), ref


SHAPES = [
    (1, 2, 2, 150, 150, True),     # ragged Q and K blocks
    (2, 4, 2, 200, 333, True),     # GQA, Sq < Sk (bottom-right causal)
    (1, 4, 1, 333, 200, True),     # MQA, Sq > Sk: rows with no visible key
    (1, 2, 2, 100, 260, False),
    (1, 2, 2, 1, 77, True),        # a single query row
    (1, 8, 2, 640, 640, True),     # several full blocks, GQA; dQ pair grid with a middle block
    (1, 4, 4, 256, 256, True),     # dQ pair grid, two query blocks
    (2, 2, 1, 512, 512, True),     # dQ pair grid, MQA, four query blocks
    (1, 4, 2, 1024, 1024, True),   # dQ split-only grid (few pairs, 8 query blocks), GQA
    (1, 2, 1, 1152, 1152, True),   # dQ split-only grid, odd block count, MQA
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B{}Hq{}Hkv{}Sq{}Sk{}{}".format(*s[:5], "c" if s[5] else "n"))
def test_backward_small_shapes(B, shape):
    Bn, Hq, Hkv, Sq, Sk, causal = shape
    c = I.make_prefill(Bn, Hq, Hkv, Sq, Sk, 128, causal=causal, seed=40 + Sq + Sk)
    do = I.make_grad_out(c.q.shape, seed=40 + Sq + Sk)
    got, want = run_bwd(B, c, do)
    for name, x, y in zip(("dq", "dk", "dv"), got, want):
        check_grad(x, y, f"{name} {shape}")


def test_backward_causal_mha_b2_h16_s2048(B):
    """The headline prefill shape (the dQ kernel runs as a pair grid): every
    head compared in full against the oracle."""
    c = I.workload("causal_mha_b2_h16_s2048_d128")
    do = I.make_grad_out(c.q.shape, seed=2)
    # the kernel needs O and lse of every head: the oracle computes them all
    O_all, L_all = oracle.sdpa(c.q, c.k, c.v, True, c.scale)
    q, k, v = _bf(c.q), _bf(c.k), _bf(c.v)
    o, g = _bf(I.round_to_bf16(O_all.astype(np.float32))), _bf(do)
    lse = torch.from_numpy(L_all.astype(np.float32)).to(DEV)
    dq, dk, dv = B.fa_bwd(q, k, v, o, g, lse, True, c.scale)
    torch.cuda.synchronize()
    dq, dk, dv = _np(dq), _np(dk), _np(dv)
    for b, h in [(b, h) for b in range(2) for h in range(16)]:
        rq, rk, rv = oracle.sdpa_backward(c.q[b:b + 1, h:h + 1], c.k[b:b + 1, h:h + 1], c.v[b:b + 1, h:h + 1],
                                          do[b:b + 1, h:h + 1], True, c.scale)
        check_grad(dq[b:b + 1, h:h + 1], rq, f"dq b{b} h{h}")
        check_grad(dk[b:b + 1, h:h + 1], rk, f"dk b{b} h{h}")
        check_grad(dv[b:b + 1, h:h + 1], rv, f"dv b{b} h{h}")


def test_backward_constant_values(B):
    """Equal value rows: O does not depend on the scores, so dQ = dK = 0."""
    c = I.make_prefill(1, 2, 2, 300, 300, 128, causal=True, seed=60)
    c.v[:] = c.v[:, :, :1]
    do = I.make_grad_out(c.q.shape, seed=60)
    (dq, dk, dv), (rq, rk, rv) = run_bwd(B, c, do)
    assert np.abs(rq).max() < 1e-9 and np.abs(rk).max() < 1e-9
    # dP - D is a difference of equal fp32 sums (|dP| ~ 10): only their
    # rounding (~1e-5) reaches dS
    assert np.abs(dq).max() < 1e-2 and np.abs(dk).max() < 1e-2
    check_grad(dv, rv, "dv constant values")


def test_backward_key_gradients_sum_to_zero(B):
    """Softmax is unchanged by a common shift of all keys: the key gradients of
    every (batch, K/V head, dim) sum to zero up to the kernels' rounding."""
    c = I.make_prefill(1, 4, 2, 256, 256, 128, causal=True, seed=61)
    do = I.make_grad_out(c.q.shape, seed=61)
    (dq, dk, dv), _ = run_bwd(B, c, do)
    col = np.abs(dk).sum(axis=2)
    assert (np.abs(dk.sum(axis=2)) <= 2e-2 * col + 1e-3).all()


def test_backward_is_deterministic(B):
    c = I.make_prefill(1, 4, 2, 300, 300, 128, causal=True, seed=62)
    do = I.make_grad_out(c.q.shape, seed=62)
    O, L = oracle.sdpa(c.q, c.k, c.v, True, c.scale)
    args = [_bf(c.q), _bf(c.k), _bf(c.v), _bf(I.round_to_bf16(O.astype(np.float32))), _bf(do),
            torch.from_numpy(L.astype(np.float32)).to(DEV)]
    a = [t.clone() for t in B.fa_bwd(*args, True, c.scale)]
    b = B.fa_bwd(*args, True, c.scale)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_binding_errors(B):
    q = torch.zeros((1, 2, 8, 64), dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros((1, 2, 8), dtype=torch.float32, device=DEV)
    with pytest.raises(B.FAError) as e:
        B.fa_bwd(q, q, q, q, q, lse, True)
    assert e.value.status == B.FA_ERR_UNSUPPORTED
    q = torch.zeros((1, 2, 8, 128), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(B.FAError) as e:
        B.fa_bwd(q, q, q, q, q, lse, True, workspace=torch.empty(16, dtype=torch.uint8, device=DEV))
    assert e.value.status == B.FA_ERR_WORKSPACE


@pytest.mark.parametrize("shape", [(1, 4, 4, 512), (1, 4, 2, 1024)], ids=["pair", "split_only"])
def test_backward_pair_barrier_timeout_is_reported(B, shape):
    """The dQ pair grid's wave-group barriers with their poll bound forced to
    0 from the host: waits run out, the device count says so and the rows of
    the affected waves of dQ are NaN, never a plausible result.  Every wait is
    bounded, so the kernels still exit normally; the bound applies to that
    one call only, and the next call matches the oracle.  Covers the pair
    grid and the split-only grid (one query block halved between the groups)."""
    B.fa_sync_timeouts()
    b, hq, hkv, s = shape
    c = I.make_prefill(b, hq, hkv, s, s, 128, causal=True, seed=13)
    do = I.make_grad_out(c.q.shape, seed=13)
    O, L = oracle.sdpa(c.q, c.k, c.v, True, c.scale)
    q, k, v = _bf(c.q), _bf(c.k), _bf(c.v)
    o, g = _bf(I.round_to_bf16(O.astype(np.float32))), _bf(do)
    lse = torch.from_numpy(L.astype(np.float32)).to(DEV)
    B.fa_limit_next_sync_wait(0)
    dq, dk, dv = B.fa_bwd(q, k, v, o, g, lse, True, c.scale)
    torch.cuda.synchronize()
    n = B.fa_sync_timeouts()
    print(f"backward barrier timeouts with a zero poll bound: {n}", flush=True)
    assert n > 0
    assert bool(torch.isnan(dq.float()).any())
    dq, dk, dv = B.fa_bwd(q, k, v, o, g, lse, True, c.scale)
    torch.cuda.synchronize()
    assert B.fa_sync_timeouts() == 0
    ref = oracle.sdpa_backward(c.q, c.k, c.v, do, True, c.scale)
    for name, x, y in zip(("dq", "dk", "dv"), (_np(dq), _np(dk), _np(dv)), ref):
        check_grad(x, y, f"{name} after a timed-out call")
