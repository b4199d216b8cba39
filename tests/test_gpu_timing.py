"""The kernel-boundary timing hook (fa_time_next_call) on the GPU: it spans
the timed call's kernels, leaves results unchanged, and is used up by that
one call."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

from exact_tiled_attention_14_amd import inputs as I  # noqa: E402

DEV = "cuda:0"


@pytest.fixture(scope="module")
def B():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from exact_tiled_attention_14_amd import binding
    binding.load()
    return binding


def _bf(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def _marker():
    return torch.cuda.Event(enable_timing=True)


def _timed(B, call):
    """(kernel-boundary ms, stream-marker ms, result) of one call."""
    s = torch.cuda.current_stream()
    a, b = B.TimingEvent(), B.TimingEvent()
    ma, mb = _marker(), _marker()
    torch.cuda.synchronize()
    ma.record(s)
    B.fa_time_next_call(a, b)
    out = call()
    mb.record(s)
    torch.cuda.synchronize()
    return a.elapsed_ms(b), ma.elapsed_time(mb), out, (a, b)


def test_prefill_timing_spans_the_kernel(B):
    c = I.make_prefill(1, 8, 8, 1024, 1024, 128, causal=True, seed=90)
    q, k, v = _bf(c.bits("q")), _bf(c.bits("k")), _bf(c.bits("v"))
    o0, l0 = B.fa_fwd(q, k, v, True, c.scale)
    t_kernel, t_marker, (o1, l1), (a, b) = _timed(B, lambda: B.fa_fwd(q, k, v, True, c.scale))
    print(f"kernel-boundary {t_kernel * 1e3:.1f} us, stream markers {t_marker * 1e3:.1f} us", flush=True)
    assert 0.0 < t_kernel <= t_marker * 1.02 + 1e-3
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    # the hook was used up: an untimed call records neither event again
    B.fa_fwd(q, k, v, True, c.scale)
    torch.cuda.synchronize()
    assert a.elapsed_ms(b) == t_kernel


def test_decode_timing_spans_both_kernels(B):
    d = I.make_decode(16, 32, 8, 128, len_lo=500, len_hi=3000, seed=91)
    args = (_bf(d.bits("q")), _bf(d.kcache_bits), _bf(d.vcache_bits), torch.from_numpy(d.block_table).to(DEV),
            torch.from_numpy(d.seqlens).to(DEV), d.scale)
    o0, l0 = B.fa_decode(*args)
    t_kernel, t_marker, (o1, l1), _ = _timed(B, lambda: B.fa_decode(*args))
    print(f"kernel-boundary {t_kernel * 1e3:.1f} us, stream markers {t_marker * 1e3:.1f} us", flush=True)
    assert 0.0 < t_kernel <= t_marker * 1.02 + 1e-3
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_backward_timing_spans_three_kernels(B):
    c = I.make_prefill(1, 4, 2, 512, 512, 128, causal=True, seed=93)
    q, k, v = _bf(c.bits("q")), _bf(c.bits("k")), _bf(c.bits("v"))
    o, lse = B.fa_fwd(q, k, v, True, c.scale)
    g = _bf(I.bf16_bits(I.make_grad_out(c.q.shape, seed=93)))
    r0 = [t.clone() for t in B.fa_bwd(q, k, v, o, g, lse, True, c.scale)]
    t_kernel, t_marker, r1, _ = _timed(B, lambda: B.fa_bwd(q, k, v, o, g, lse, True, c.scale))
    print(f"kernel-boundary {t_kernel * 1e3:.1f} us, stream markers {t_marker * 1e3:.1f} us", flush=True)
    assert 0.0 < t_kernel <= t_marker * 1.02 + 1e-3
    assert all(torch.equal(x, y) for x, y in zip(r0, r1))


def test_fp8_timing_spans_each_call(B):
    """The one-launch quantizer, the FP8 forward on codes and the FP8 forward
    that quantizes Q itself, each timed on its own as the bench times them."""
    c = I.make_prefill(1, 8, 2, 1024, 1024, 128, causal=True, seed=94)
    q, k, v = _bf(c.bits("q")), _bf(c.bits("k")), _bf(c.bits("v"))
    R = _bf(I.bf16_bits(I.make_rotation(128, seed=94)))
    q8, qs, k8, ks, v8, vs = B.fa_quantize_fp8_qkv(q, k, v, rot=R)
    calls = {
        "quantize": lambda: B.fa_quantize_fp8_qkv(q, k, v, rot=R),
        "fp8": lambda: B.fa_fwd_fp8(q8, qs, k8, ks, v8, vs, True, c.scale),
        "fp8_qbf16": lambda: B.fa_fwd_fp8_qbf16(q, k8, ks, v8, vs, True, rot=R, scale=c.scale),
    }
    for name, call in calls.items():
        r0 = [t.clone() for t in call()]
        t_kernel, t_marker, r1, _ = _timed(B, call)
        print(f"{name}: kernel-boundary {t_kernel * 1e3:.1f} us, stream markers {t_marker * 1e3:.1f} us", flush=True)
        assert 0.0 < t_kernel <= t_marker * 1.02 + 1e-3, name
        assert all(torch.equal(x, y) for x, y in zip(r0, r1)), name


def test_rejected_call_clears_the_hook(B):
    c = I.make_prefill(1, 16, 16, 2048, 2048, 128, causal=False, seed=92)
    q, k, v = _bf(c.bits("q")), _bf(c.bits("k")), _bf(c.bits("v"))
    a, b = B.TimingEvent(), B.TimingEvent()
    a.record()
    b.record()
    B.fa_time_next_call(a, b)
    bad = torch.zeros((1, 2, 8, 96), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(B.FAError):
        B.fa_fwd(bad, bad, bad, True)
    B.fa_fwd(q, k, v, False, c.scale)   # ~100 us of work, must not be timed
    torch.cuda.synchronize()
    t = a.elapsed_ms(b)
    print(f"events after the rejected call: {t * 1e3:.1f} us apart", flush=True)
    assert t < 0.02
