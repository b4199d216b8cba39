"""Python binding of the C ABI in ``include/fa.h`` (argument marshalling only).

Every function here has the name of the C entry point it calls.  PyTorch
supplies device memory and the current stream; all arithmetic runs in the
HIP kernels of ``libfa.so``.  There is no fallback: if the library is
missing or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch  # must precede the library load: it brings up the HIP runtime libfa.so binds to

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = 0, -1, -2, -3, -4
FA_BF16, FA_F32 = 0, 1

_lib = None


class FAError(RuntimeError):
    """A non-zero fa_status returned by the library."""

    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {status} ({fa_status_string(status)})")
        self.status = status


_vp, _i, _f, _sz, _u8p = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p

# (argument types, result type) of every entry point of include/fa.h, in the
# header's order; a pointer of any type is passed as c_void_p.
SIGNATURES = {
    "fa_fwd": ([_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _i, _vp], _i),
    "fa_bwd_workspace_size": ([_i, _i, _i], _sz),
    "fa_bwd": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp], _i),
    "fa_decode_workspace_size": ([_i, _i, _i, _i, _i, _i], _sz),
    "fa_decode": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp], _i),
    "fa_decode_noalloc": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp], _i),
    "fa_decode_multi_workspace_size": ([_i, _i, _i, _i, _i, _i, _i], _sz),
    "fa_decode_multi": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp],
                        _i),
    "fa_mla_decode_workspace_size": ([_i, _i, _i, _i, _i, _i], _sz),
    "fa_mla_decode": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp, _sz, _vp], _i),
    "fa_quantize_fp8_bytes": ([_i, _i, _i, _i, _i], _sz),
    "fa_quantize_fp8": ([_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp], _i),
    "fa_quantize_fp8_qkv": ([_vp] * 10 + [_i] * 6 + [_vp], _i),
    "fa_fwd_fp8": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp], _i),
    "fa_fwd_fp8_qbf16": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _f, _vp], _i),
    "fa_time_next_call": ([_vp, _vp], _i),
    "fa_limit_next_sync_wait": ([_i], _i),
    "fa_sync_timeouts": ([_vp], _i),
    "fa_status_string": ([_i], ctypes.c_char_p),
}


def load() -> ctypes.CDLL:
    """Load ``libfa.so`` once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m exact_tiled_attention_14_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (args, res) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = list(args)
        fn.restype = res
    _lib = lib
    return lib


def fa_status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


_hip_rt = None


def _hip():
    """The HIP runtime already in the process (the one libfa.so is bound to)."""
    global _hip_rt
    if _hip_rt is None:
        load()
        lib = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD | os.RTLD_GLOBAL)
        vp = ctypes.c_void_p
        lib.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
        lib.hipEventRecord.argtypes = [vp, vp]
        lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        lib.hipEventDestroy.argtypes = [vp]
        for fn in ("hipEventCreateWithFlags", "hipEventRecord", "hipEventElapsedTime", "hipEventDestroy"):
            getattr(lib, fn).restype = ctypes.c_int
        _hip_rt = lib
    return _hip_rt


class TimingEvent:
    """A HIP timing event for fa_time_next_call.  It is created without the
    system-scope fence (hipEventDisableSystemFence), so that recording it
    does not write back and invalidate the caches between kernels: it is for
    measuring, not for making results visible to the host."""

    FLAGS = 0x20000000   # hipEventDisableSystemFence

    def __init__(self):
        self.handle = ctypes.c_void_p()
        st = _hip().hipEventCreateWithFlags(ctypes.byref(self.handle), self.FLAGS)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")

    def record(self, stream=None):
        """Record on a torch stream (default: the current one)."""
        s = stream if stream is not None else torch.cuda.current_stream()
        st = _hip().hipEventRecord(self.handle, ctypes.c_void_p(s.cuda_stream))
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed ({st})")

    def elapsed_ms(self, stop: "TimingEvent") -> float:
        """Milliseconds from this event to `stop`; both must have completed."""
        ms = ctypes.c_float()
        st = _hip().hipEventElapsedTime(ctypes.byref(ms), self.handle, stop.handle)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return float(ms.value)

    def __del__(self):
        if self.handle and _hip_rt is not None:
            _hip_rt.hipEventDestroy(self.handle)
            self.handle = ctypes.c_void_p()


def fa_time_next_call(start: TimingEvent | None = None, stop: TimingEvent | None = None) -> None:
    """Attach two TimingEvents to the kernels of the next fa_fwd / fa_bwd /
    fa_decode call on this thread: after it, ``start.elapsed_ms(stop)`` is
    the time from its first kernel's start to its last kernel's end.
    ``None, None`` clears."""
    if (start is None) != (stop is None):
        raise ValueError("fa_time_next_call takes two events or none")
    st = load().fa_time_next_call(None if start is None else start.handle, None if stop is None else stop.handle)
    if st != FA_OK:
        raise FAError("fa_time_next_call", st)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t, name, dtype, shape, device=None):
    """Type, dtype, rank (``shape`` an int) or exact shape (a tuple),
    contiguity and, with ``device``, the device of a tensor argument.  That
    the tensors live on a GPU is checked by :func:`_on_gpu` just before the
    launch, so every shape error is raised first."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if isinstance(shape, int):
        if t.dim() != shape:
            raise ValueError(f"{name} must have {shape} dimensions (got {tuple(t.shape)})")
    elif tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(*tensors):
    for t in tensors:
        if t is not None and t.device.type != "cuda":
            raise ValueError(f"tensor arguments must be GPU tensors (got {t.device})")


def fa_fwd(q, k, v, causal: bool, scale: float | None = None, out=None, lse=None,
           return_lse: bool = True):
    """Attention forward: q [B,Hq,Sq,d], k/v [B,Hkv,Sk,d] (bf16 or fp32).

    Returns ``(o, lse)``; ``lse`` is [B,Hq,Sq] fp32 (None if not requested).
    """
    lib = load()
    dtype = q.dtype
    if dtype == torch.bfloat16:
        code = FA_BF16
    elif dtype == torch.float32:
        code = FA_F32
    else:
        raise TypeError(f"unsupported dtype {dtype}")
    _check(q, "q", dtype, 4)
    _check(k, "k", dtype, 4, q.device)
    _check(v, "v", dtype, 4, q.device)
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Sk, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch q={tuple(q.shape)} k={tuple(k.shape)} v={tuple(v.shape)}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", dtype, tuple(q.shape), q.device)
    if lse is None and return_lse:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    elif lse is not None:
        _check(lse, "lse", torch.float32, (B, Hq, Sq), q.device)
    _on_gpu(q, k, v, out, lse)
    st = lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, Hq, Hkv, Sq, Sk, d,
                    int(bool(causal)), float(scale), code, _stream(q.device))
    if st != FA_OK:
        raise FAError("fa_fwd", st)
    return out, lse


FA_FP8_ROWS, FA_FP8_VBLOCKS = 0, 1


def fa_quantize_fp8(x, block_rows: int, layout: int = FA_FP8_ROWS, rot=None):
    """FP8 (E4M3) block quantization of a bf16 [B,H,S,d] tensor.

    ``layout`` FA_FP8_ROWS gives codes [B,H,S,d]; FA_FP8_VBLOCKS (for V,
    block_rows 64, no rotation) gives [B,H,ceil(S/64),d,64], each 64-key block
    d-major with the key order include/fa.h states.  ``rot`` is a bf16 [d,d]
    orthogonal matrix R; each row x becomes R x first.  Returns ``(codes, scales)``,
    scales [B,H,ceil(S/block_rows)] uint8 E8M0 bytes.
    """
    lib = load()
    _check(x, "x", torch.bfloat16, 4)
    B, H, S, d = x.shape
    if rot is not None:
        _check(rot, "rot", torch.bfloat16, 2, x.device)
        if tuple(rot.shape) != (d, d):
            raise ValueError("rot must be [d, d]")
    nbytes = int(lib.fa_quantize_fp8_bytes(B, H, S, d, int(layout)))
    if nbytes == 0:
        raise FAError("fa_quantize_fp8_bytes", FA_ERR_UNSUPPORTED)
    nblk = -(-S // block_rows)
    if layout == FA_FP8_VBLOCKS:
        codes = torch.empty((B, H, -(-S // 64), d, 64), dtype=torch.uint8, device=x.device)
    else:
        codes = torch.empty((B, H, S, d), dtype=torch.uint8, device=x.device)
    assert codes.numel() == nbytes
    scales = torch.empty((B, H, nblk), dtype=torch.uint8, device=x.device)
    _on_gpu(x, rot, codes, scales)
    st = lib.fa_quantize_fp8(_ptr(x), _ptr(rot), _ptr(codes), _ptr(scales), B, H, S, d, int(block_rows),
                             int(layout), _stream(x.device))
    if st != FA_OK:
        raise FAError("fa_quantize_fp8", st)
    return codes, scales


def fa_quantize_fp8_qkv(q, k, v, rot=None):
    """Q (128-row blocks), K (64-row blocks), both times ``rot`` if given, and
    V (FA_FP8_VBLOCKS) quantized in one launch.  Returns
    ``(q8, q_scales, k8, k_scales, v8, v_scales)``, laid out as the three
    :func:`fa_quantize_fp8` calls would return them."""
    lib = load()
    _check(q, "q", torch.bfloat16, 4)
    _check(k, "k", torch.bfloat16, 4, q.device)
    _check(v, "v", torch.bfloat16, 4, q.device)
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Sk, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch q={tuple(q.shape)} k={tuple(k.shape)} v={tuple(v.shape)}")
    if rot is not None:
        _check(rot, "rot", torch.bfloat16, 2, q.device)
        if tuple(rot.shape) != (d, d):
            raise ValueError("rot must be [d, d]")
    if d != 128:
        raise FAError("fa_quantize_fp8_qkv", FA_ERR_UNSUPPORTED)
    u8, dev = torch.uint8, q.device
    nk = -(-Sk // 64)
    q8 = torch.empty((B, Hq, Sq, d), dtype=u8, device=dev)
    qs = torch.empty((B, Hq, -(-Sq // 128)), dtype=u8, device=dev)
    k8 = torch.empty((B, Hkv, Sk, d), dtype=u8, device=dev)
    ks = torch.empty((B, Hkv, nk), dtype=u8, device=dev)
    v8 = torch.empty((B, Hkv, nk, d, 64), dtype=u8, device=dev)
    vs = torch.empty((B, Hkv, nk), dtype=u8, device=dev)
    _on_gpu(q, k, v, rot, q8, qs, k8, ks, v8, vs)
    st = lib.fa_quantize_fp8_qkv(_ptr(q), _ptr(k), _ptr(v), _ptr(rot), _ptr(q8), _ptr(qs), _ptr(k8), _ptr(ks),
                                 _ptr(v8), _ptr(vs), B, Hq, Hkv, Sq, Sk, d, _stream(dev))
    if st != FA_OK:
        raise FAError("fa_quantize_fp8_qkv", st)
    return q8, qs, k8, ks, v8, vs


def fa_fwd_fp8(q8, q_scale, k8, k_scale, v8, v_scale, causal: bool, scale: float | None = None, out=None,
               lse=None):
    """Attention forward on FP8 inputs from fa_quantize_fp8: q8 [B,Hq,Sq,d]
    (128-row scale blocks), k8 [B,Hkv,Sk,d] (64-row blocks), v8 in
    FA_FP8_VBLOCKS layout.  Returns ``(o bf16 [B,Hq,Sq,d], lse fp32 [B,Hq,Sq])``."""
    lib = load()
    u8 = torch.uint8
    _check(q8, "q8", u8, 4)
    _check(k8, "k8", u8, 4, q8.device)
    _check(v8, "v8", u8, 5, q8.device)
    B, Hq, Sq, d = q8.shape
    Hkv, Sk = k8.shape[1], k8.shape[2]
    nk = -(-Sk // 64)
    if tuple(k8.shape) != (B, Hkv, Sk, d) or tuple(v8.shape) != (B, Hkv, nk, d, 64):
        raise ValueError(f"shape mismatch q8={tuple(q8.shape)} k8={tuple(k8.shape)} v8={tuple(v8.shape)}")
    for t, n, shp in ((q_scale, "q_scale", (B, Hq, -(-Sq // 128))), (k_scale, "k_scale", (B, Hkv, nk)),
                      (v_scale, "v_scale", (B, Hkv, nk))):
        _check(t, n, u8, 3, q8.device)
        if tuple(t.shape) != shp:
            raise ValueError(f"{n} must be {shp}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, Sq, d), dtype=torch.bfloat16, device=q8.device)
    else:
        _check(out, "out", torch.bfloat16, (B, Hq, Sq, d), q8.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q8.device)
    else:
        _check(lse, "lse", torch.float32, (B, Hq, Sq), q8.device)
    _on_gpu(q8, k8, v8, q_scale, k_scale, v_scale, out, lse)
    st = lib.fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scale), _ptr(k_scale), _ptr(v_scale), _ptr(out),
                        _ptr(lse), B, Hq, Hkv, Sq, Sk, d, int(bool(causal)), float(scale), _stream(q8.device))
    if st != FA_OK:
        raise FAError("fa_fwd_fp8", st)
    return out, lse


def fa_fwd_fp8_qbf16(q, k8, k_scale, v8, v_scale, causal: bool, rot=None, scale: float | None = None, out=None,
                     lse=None):
    """FP8 forward with Q given in bf16 [B,Hq,Sq,d] and quantized inside the
    kernel (128-row blocks, times ``rot`` if given: the rotation K was
    quantized with); k8/k_scale and v8/v_scale as for :func:`fa_fwd_fp8`.
    Bit-identical to ``fa_fwd_fp8(*fa_quantize_fp8(q, 128, rot=rot), ...)``.
    Returns ``(o bf16 [B,Hq,Sq,d], lse fp32 [B,Hq,Sq])``."""
    lib = load()
    u8 = torch.uint8
    _check(q, "q", torch.bfloat16, 4)
    _check(k8, "k8", u8, 4, q.device)
    _check(v8, "v8", u8, 5, q.device)
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k8.shape[1], k8.shape[2]
    nk = -(-Sk // 64)
    if tuple(k8.shape) != (B, Hkv, Sk, d) or tuple(v8.shape) != (B, Hkv, nk, d, 64):
        raise ValueError(f"shape mismatch q={tuple(q.shape)} k8={tuple(k8.shape)} v8={tuple(v8.shape)}")
    for t, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
        _check(t, n, u8, 3, q.device)
        if tuple(t.shape) != (B, Hkv, nk):
            raise ValueError(f"{n} must be {(B, Hkv, nk)}")
    if rot is not None:
        _check(rot, "rot", torch.bfloat16, 2, q.device)
        if tuple(rot.shape) != (d, d):
            raise ValueError("rot must be [d, d]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, Sq, d), dtype=torch.bfloat16, device=q.device)
    else:
        _check(out, "out", torch.bfloat16, (B, Hq, Sq, d), q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    else:
        _check(lse, "lse", torch.float32, (B, Hq, Sq), q.device)
    _on_gpu(q, rot, k8, v8, k_scale, v_scale, out, lse)
    st = lib.fa_fwd_fp8_qbf16(_ptr(q), _ptr(rot), _ptr(k8), _ptr(v8), _ptr(k_scale), _ptr(v_scale), _ptr(out),
                              _ptr(lse), B, Hq, Hkv, Sq, Sk, d, int(bool(causal)), float(scale), _stream(q.device))
    if st != FA_OK:
        raise FAError("fa_fwd_fp8_qbf16", st)
    return out, lse


def fa_bwd_workspace_size(B: int, Hq: int, Sq: int) -> int:
    return int(load().fa_bwd_workspace_size(B, Hq, Sq))


def fa_bwd(q, k, v, o, dout, lse, causal: bool, scale: float | None = None, dq=None, dk=None, dv=None,
           workspace=None):
    """Attention backward (bf16): gradients of sum(dout * o) for o = fa_fwd(q, k, v).

    q, o, dout [B,Hq,Sq,d]; k, v [B,Hkv,Sk,d]; lse [B,Hq,Sq] fp32 from the forward.
    Returns ``(dq, dk, dv)`` in bf16.
    """
    lib = load()
    dt = torch.bfloat16
    _check(q, "q", dt, 4)
    for t, n in ((k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _check(t, n, dt, 4, q.device)
    _check(lse, "lse", torch.float32, 3, q.device)
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    if tuple(k.shape) != (B, Hkv, Sk, d) or tuple(v.shape) != tuple(k.shape):
        raise ValueError(f"shape mismatch q={tuple(q.shape)} k={tuple(k.shape)} v={tuple(v.shape)}")
    if o.shape != q.shape or dout.shape != q.shape or tuple(lse.shape) != (B, Hq, Sq):
        raise ValueError("o and dout must have q's shape, lse must be [B, Hq, Sq]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    outs = []
    for t, ref, n in ((dq, q, "dq"), (dk, k, "dk"), (dv, v, "dv")):
        if t is None:
            t = torch.empty_like(ref)
        else:
            _check(t, n, dt, 4, q.device)
            if t.shape != ref.shape:
                raise ValueError(f"{n} must have the shape of {'q' if n == 'dq' else 'k'}")
        outs.append(t)
    dq, dk, dv = outs
    need = fa_bwd_workspace_size(B, Hq, Sq)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device:
        raise ValueError("workspace must be on q's device")
    _on_gpu(q, k, v, o, dout, lse, dq, dk, dv, workspace)
    st = lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
                    B, Hq, Hkv, Sq, Sk, d, int(bool(causal)), float(scale), _ptr(workspace),
                    workspace.numel() * workspace.element_size(), _stream(q.device))
    if st != FA_OK:
        raise FAError("fa_bwd", st)
    return dq, dk, dv


def fa_decode_workspace_size(nseq: int, Hq: int, Hkv: int, d: int, block_size: int,
                             max_blocks_per_seq: int) -> int:
    return int(load().fa_decode_workspace_size(nseq, Hq, Hkv, d, block_size, max_blocks_per_seq))


def fa_decode(q, kcache, vcache, block_table, seqlens, scale: float | None = None, out=None,
              lse=None, workspace=None, return_lse: bool = True):
    """Single-token decode over a paged cache.

    q [nseq,Hq,d] bf16; kcache/vcache [num_blocks,Hkv,block_size,d] bf16;
    block_table [nseq,max_blocks] int32; seqlens [nseq] int32.
    Returns ``(o [nseq,Hq,d] bf16, lse [nseq,Hq] fp32 or None)``.
    """
    lib = load()
    _check(q, "q", torch.bfloat16, 3)
    dev = q.device
    _check(kcache, "kcache", torch.bfloat16, 4, dev)
    _check(vcache, "vcache", torch.bfloat16, 4, dev)
    _check(block_table, "block_table", torch.int32, 2, dev)
    _check(seqlens, "seqlens", torch.int32, 1, dev)
    nseq, Hq, d = q.shape
    num_blocks, Hkv, bs, d2 = kcache.shape
    if vcache.shape != kcache.shape or d2 != d:
        raise ValueError("cache shape mismatch")
    if block_table.shape[0] != nseq or seqlens.shape[0] != nseq:
        raise ValueError("block_table / seqlens must have nseq rows")
    max_blocks = block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_decode_workspace_size(nseq, Hq, Hkv, d, bs, max_blocks)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.device != dev:
        raise ValueError("workspace must be on q's device")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", torch.bfloat16, (nseq, Hq, d), dev)
    if lse is None and return_lse:
        lse = torch.empty((nseq, Hq), dtype=torch.float32, device=dev)
    elif lse is not None:
        _check(lse, "lse", torch.float32, (nseq, Hq), dev)
    _on_gpu(q, kcache, vcache, block_table, seqlens, out, lse, workspace)
    st = lib.fa_decode(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(block_table), _ptr(seqlens),
                       _ptr(out), _ptr(lse), nseq, Hq, Hkv, d, bs, max_blocks, num_blocks,
                       float(scale), _ptr(workspace), workspace.numel() * workspace.element_size(),
                       _stream(dev))
    if st != FA_OK:
        raise FAError("fa_decode", st)
    return out, lse


FA_DECODE_NOALLOC_SCRATCH_BYTES = 32 << 20


def fa_decode_noalloc(q, kcache, vcache, block_table, seqlens, scale: float | None = None, out=None, lse=None):
    """fa_decode without a workspace: the library's fixed per-GPU scratch
    array (FA_DECODE_NOALLOC_SCRATCH_BYTES) serves instead, so the C call
    allocates nothing.  ``out`` and ``lse`` must be given (this wrapper does
    not allocate them either).  Returns ``(out, lse)``."""
    lib = load()
    _check(q, "q", torch.bfloat16, 3)
    dev = q.device
    _check(kcache, "kcache", torch.bfloat16, 4, dev)
    _check(vcache, "vcache", torch.bfloat16, 4, dev)
    _check(block_table, "block_table", torch.int32, 2, dev)
    _check(seqlens, "seqlens", torch.int32, 1, dev)
    nseq, Hq, d = q.shape
    num_blocks, Hkv, bs, d2 = kcache.shape
    if vcache.shape != kcache.shape or d2 != d:
        raise ValueError("cache shape mismatch")
    if block_table.shape[0] != nseq or seqlens.shape[0] != nseq:
        raise ValueError("block_table / seqlens must have nseq rows")
    if out is None or lse is None:
        raise ValueError("fa_decode_noalloc writes into caller-given out and lse")
    _check(out, "out", torch.bfloat16, (nseq, Hq, d), dev)
    _check(lse, "lse", torch.float32, (nseq, Hq), dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _on_gpu(q, kcache, vcache, block_table, seqlens, out, lse)
    st = lib.fa_decode_noalloc(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(block_table), _ptr(seqlens), _ptr(out),
                               _ptr(lse), nseq, Hq, Hkv, d, bs, block_table.shape[1], num_blocks, float(scale),
                               _stream(dev))
    if st != FA_OK:
        raise FAError("fa_decode_noalloc", st)
    return out, lse


def fa_decode_multi_workspace_size(nseq: int, Sq: int, Hq: int, Hkv: int, d: int, block_size: int,
                                   max_blocks_per_seq: int) -> int:
    return int(load().fa_decode_multi_workspace_size(nseq, Sq, Hq, Hkv, d, block_size, max_blocks_per_seq))


def fa_decode_multi(q, kcache, vcache, block_table, seqlens, scale: float | None = None, out=None, lse=None,
                    workspace=None):
    """Sq new tokens per sequence against a paged cache (verify step).

    q [nseq,Sq,Hq,d] bf16 (token t of sequence s at position seqlens[s]-Sq+t,
    causal); caches, block_table and seqlens as for fa_decode.
    Returns ``(o [nseq,Sq,Hq,d] bf16, lse [nseq,Sq,Hq] fp32)``.
    """
    lib = load()
    _check(q, "q", torch.bfloat16, 4)
    dev = q.device
    _check(kcache, "kcache", torch.bfloat16, 4, dev)
    _check(vcache, "vcache", torch.bfloat16, 4, dev)
    _check(block_table, "block_table", torch.int32, 2, dev)
    _check(seqlens, "seqlens", torch.int32, 1, dev)
    nseq, Sq, Hq, d = q.shape
    num_blocks, Hkv, bs, d2 = kcache.shape
    if vcache.shape != kcache.shape or d2 != d:
        raise ValueError("cache shape mismatch")
    if block_table.shape[0] != nseq or seqlens.shape[0] != nseq:
        raise ValueError("block_table / seqlens must have nseq rows")
    max_blocks = block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = fa_decode_multi_workspace_size(nseq, Sq, Hq, Hkv, d, bs, max_blocks)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.device != dev:
        raise ValueError("workspace must be on q's device")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", torch.bfloat16, (nseq, Sq, Hq, d), dev)
    if lse is None:
        lse = torch.empty((nseq, Sq, Hq), dtype=torch.float32, device=dev)
    else:
        _check(lse, "lse", torch.float32, (nseq, Sq, Hq), dev)
    _on_gpu(q, kcache, vcache, block_table, seqlens, out, lse, workspace)
    st = lib.fa_decode_multi(_ptr(q), _ptr(kcache), _ptr(vcache), _ptr(block_table), _ptr(seqlens), _ptr(out),
                             _ptr(lse), nseq, Sq, Hq, Hkv, d, bs, max_blocks, num_blocks, float(scale),
                             _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev))
    if st != FA_OK:
        raise FAError("fa_decode_multi", st)
    return out, lse


def fa_mla_decode_workspace_size(nseq: int, H: int, d_h: int, d_c: int, block_size: int,
                                 max_blocks_per_seq: int) -> int:
    return int(load().fa_mla_decode_workspace_size(nseq, H, d_h, d_c, block_size, max_blocks_per_seq))


def fa_mla_decode(q, w_uk, w_uv_t, ccache, block_table, seqlens, scale: float | None = None, out=None, lse=None,
                  workspace=None):
    """One new token per sequence against a paged latent cache (MLA).

    q [nseq,H,d_h], w_uk [H,d_c,d_h], w_uv_t [H,d_h,d_c], ccache
    [num_blocks,block_size,d_c], all bf16; block_table, seqlens as for
    fa_decode.  Returns ``(o [nseq,H,d_h] bf16, lse [nseq,H] fp32)``.
    """
    lib = load()
    _check(q, "q", torch.bfloat16, 3)
    dev = q.device
    _check(w_uk, "w_uk", torch.bfloat16, 3, dev)
    _check(w_uv_t, "w_uv_t", torch.bfloat16, 3, dev)
    _check(ccache, "ccache", torch.bfloat16, 3, dev)
    _check(block_table, "block_table", torch.int32, 2, dev)
    _check(seqlens, "seqlens", torch.int32, 1, dev)
    nseq, H, dh = q.shape
    num_blocks, bs, dc = ccache.shape
    if tuple(w_uk.shape) != (H, dc, dh) or tuple(w_uv_t.shape) != (H, dh, dc):
        raise ValueError("projection shapes must be w_uk [H,d_c,d_h] and w_uv_t [H,d_h,d_c]")
    if block_table.shape[0] != nseq or seqlens.shape[0] != nseq:
        raise ValueError("block_table / seqlens must have nseq rows")
    max_blocks = block_table.shape[1]
    if scale is None:
        scale = 1.0 / math.sqrt(dh)
    need = fa_mla_decode_workspace_size(nseq, H, dh, dc, bs, max_blocks)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    elif workspace.device != dev:
        raise ValueError("workspace must be on q's device")
    if out is None:
        out = torch.empty_like(q)
    else:
        _check(out, "out", torch.bfloat16, (nseq, H, dh), dev)
    if lse is None:
        lse = torch.empty((nseq, H), dtype=torch.float32, device=dev)
    else:
        _check(lse, "lse", torch.float32, (nseq, H), dev)
    _on_gpu(q, w_uk, w_uv_t, ccache, block_table, seqlens, out, lse, workspace)
    st = lib.fa_mla_decode(_ptr(q), _ptr(w_uk), _ptr(w_uv_t), _ptr(ccache), _ptr(block_table), _ptr(seqlens),
                           _ptr(out), _ptr(lse), nseq, H, dh, dc, bs, max_blocks, num_blocks, float(scale),
                           _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(dev))
    if st != FA_OK:
        raise FAError("fa_mla_decode", st)
    return out, lse


def fa_limit_next_sync_wait(spins: int) -> None:
    """Bound the wave-group barriers of the next fa_fwd, fa_fwd_fp8 or fa_bwd
    call on this thread to ``spins`` polls (a test hook; the default bound is restored after that
    call).  A barrier that runs out counts one timeout (see fa_sync_timeouts)
    and the rows of the waves it affected come out as NaN."""
    st = load().fa_limit_next_sync_wait(int(spins))
    if st != FA_OK:
        raise FAError("fa_limit_next_sync_wait", st)


def fa_sync_timeouts() -> int:
    """Number of wave-group barrier timeouts on the current device since the
    last read; the count is cleared.  Synchronises the device."""
    n = ctypes.c_uint(0)
    st = load().fa_sync_timeouts(ctypes.byref(n))
    if st != FA_OK:
        raise FAError("fa_sync_timeouts", st)
    return int(n.value)
