#!/usr/bin/env python3
"""Benchmark of the exact tiled attention hot path on one MI355X.

One step runs the whole path once on resident synthetic inputs:

  * fp32 prefill, B=1 H=1 S=128 d=64, non-causal (correctness-sized; launch bound)
  * bf16 causal prefill, B=2 H=16 S=2048 d=128 (the headline workload)
  * bf16 paged decode, 64 sequences x 1 token, Hq=32 Hkv=8 d=128, 16-token
    pages, lengths uniform in [1024, 8192]

Each call is timed with HIP events that its own kernel launches record
(fa_time_next_call: the first kernel's start to the last kernel's end, on the
stream the kernels run on; the events skip the system-scope cache fence), the
interval a kernel trace reports.  A spin kernel queued ahead of each timed
loop lets the host enqueue every timed launch before the GPU gets there (the
JSON's `host_lead` says whether it did).  The
headline `value` is the algorithmic TFLOP/s of the causal prefill (4 d FLOP per
visible query-key pair) over the prefill launch time; decode reports the
algorithmic KV bytes (each attended token's K and V once) over the decode
launch time.  Before each decode launch a 512 MiB buffer is read so that
neither L2 nor the 256 MB Infinity Cache holds cache lines from the last step
(outside the decode's own events); the prefill, which follows the previous
step's decode, also starts from cold caches.  The flush reads rather than
writes: a write leaves the caches full of dirty lines whose write-back would
be charged to the next timed kernel.  `traffic` is the HBM bytes per
launch that the rocprofv3 counter passes summarised under profiles/ measured,
reported only while the kernel source is the one they measured.  The fp64 CPU
oracle is timed on the whole prefill workload, repeated until at least 10 s
of oracle work, as a reported baseline.

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "prefill attn TFLOP/s (% bf16 MFMA peak); decode KV GB/s (% HBM peak)"
PREFILL = "causal_mha_b2_h16_s2048_d128"
DECODE = "paged_decode_64seq_h32kv8_d128"
FP32 = "mha1_s128_d64_f32"
EXTRA = ["causal_gqa_h32kv8_s8192_d128_outliers", "causal_gqa_h32kv8_s32768_d128"]
# rocprofv3 summaries whose FETCH_SIZE / WRITE_SIZE passes give the HBM traffic
# per launch; used only while the kernel source still has the recorded hash
PROFILE_PREFILL = os.path.join(ROOT, "profiles", "fwd_bf16_causal_mha_b2_h16_s2048_d128.md")
PROFILE_DECODE = os.path.join(ROOT, "profiles", "decode_paged_64seq_h32kv8_d128.md")
PROFILE_FP8 = os.path.join(ROOT, "profiles", "fwd_fp8_causal_mha_b2_h16_s2048_d128.md")
PROFILE_VERIFY = os.path.join(ROOT, "profiles", "decode_multi_paged_64seq_q8_h32kv8_d128.md")
VERIFY = "paged_verify_64seq_q8_h32kv8_d128"
PROFILE_MLA = os.path.join(ROOT, "profiles", "mla_decode_64seq_h16_dc512.md")
MLA = "mla_decode_64seq_h16_dc512"
CPU_MIN_SECONDS = 10.0


def gpu_lead(stream, ms):
    """Queue a spin of about `ms` milliseconds on the stream (assuming a shader
    clock near 2.4 GHz) so that the host enqueues the timed launches before the
    GPU reaches them: the events then time the kernels, not the host's Python
    and argument checks between launches.  Returns (start, end) events around
    the spin."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    torch.cuda._sleep(int(ms * 2.4e6))
    b.record(stream)
    return a, b


def lead_report(lead, host_s):
    """Whether the host finished enqueueing before the GPU finished the spin."""
    spin_ms = lead[0].elapsed_time(lead[1])
    return {"spin_ms": round(spin_ms, 3), "host_enqueue_ms": round(host_s * 1e3, 3),
            "host_ahead": bool(host_s * 1e3 < spin_ms)}


class GfxClock:
    """Samples the shader (GFX) clock and the socket power with amdsmi while
    the GPU works through a queued loop.  Fractions of peak are quoted against
    the 2.4 GHz peak clock; under sustained matrix-core load the clock and power
    limits say how far the chip actually ran from it.  Every method returns
    None / [] when amdsmi is not usable on the machine."""

    def __init__(self):
        self.h = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            hs = amdsmi.amdsmi_get_processor_handles()
            if hs:
                self.h, self.smi = hs[0], amdsmi
        except Exception:
            self.h = None

    @staticmethod
    def _num(x):
        if isinstance(x, (list, tuple)):
            v = [float(e) for e in x if isinstance(e, (int, float))]
            return sorted(v)[len(v) // 2] if v else None
        return float(x) if isinstance(x, (int, float)) else None

    def read(self):
        """{name: value} of this instant (MHz, W), values that the driver does not report left out."""
        if self.h is None:
            return {}
        out = {}
        try:
            m = self.smi.amdsmi_get_gpu_metrics_info(self.h)
            for key, name in (("current_gfxclks", "current_gfxclk_mhz"), ("current_gfxclk", "current_gfxclk_mhz"),
                              ("average_gfxclk_frequency", "average_gfxclk_mhz"),
                              ("average_socket_power", "socket_power_w")):
                v = self._num(m.get(key))
                if v is not None and name not in out:
                    out[name] = v
        except Exception:
            pass
        if "current_gfxclk_mhz" not in out:
            try:
                out["current_gfxclk_mhz"] = float(
                    self.smi.amdsmi_get_clock_info(self.h, self.smi.AmdSmiClkType.GFX)["clk"])
            except Exception:
                pass
        return out

    def sample_until(self, done, start=None, period_s=0.0005, max_s=10.0):
        """Samples from the completion of the torch event `start` (if given)
        until the completion of `done`."""
        out, t0 = [], time.perf_counter()
        while start is not None and not start.query() and time.perf_counter() - t0 < max_s:
            time.sleep(period_s)
        while self.h is not None and not done.query() and time.perf_counter() - t0 < max_s:
            v = self.read()
            if v:
                out.append(v)
            time.sleep(period_s)
        return out


def clock_report(samples):
    """Medians (and the sample count) of each quantity; None without samples."""
    if not samples:
        return None
    rep = {"samples": len(samples)}
    for name in sorted({k for s in samples for k in s}):
        x = sorted(s[name] for s in samples if name in s)
        rep[name] = x[len(x) // 2]
    return rep


def kernel_events(n):
    """n (start, stop) pairs of timing events for fa_time_next_call."""
    from exact_tiled_attention_14_amd import binding
    return [(binding.TimingEvent(), binding.TimingEvent()) for _ in range(n)]


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-extra", action="store_true", help="skip the 8k/32k GQA prefill timings")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward timing")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 forward timing")
    ap.add_argument("--no-verify", action="store_true", help="skip the multi-query (verify) decode timing")
    ap.add_argument("--no-mla", action="store_true", help="skip the latent-cache (MLA) decode timing")
    ap.add_argument("--cpu-heads", type=int, default=4, help="heads per oracle call when timing the CPU baseline")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this path has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1:
        sys.exit("--steps must be >= 1")

    import numpy as np
    import torch

    from exact_tiled_attention_14_amd import binding, inputs, metrics, profiling

    if not torch.cuda.is_available():
        sys.exit("no GPU visible")
    dev = torch.device("cuda:0")
    binding.load()

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    # ---- inputs, built on the host by the seeded generator, copied once ----
    log("generating inputs")
    cf = inputs.workload(FP32)
    f_q, f_k, f_v = (torch.from_numpy(getattr(cf, n)).to(dev) for n in "qkv")
    f_o, f_l = torch.empty_like(f_q), torch.empty(cf.q.shape[:3], dtype=torch.float32, device=dev)

    cp = inputs.workload(PREFILL)
    shp = cp.shape
    p_q, p_k, p_v = to_dev(cp.bits("q")), to_dev(cp.bits("k")), to_dev(cp.bits("v"))
    p_o = torch.empty_like(p_q)
    p_l = torch.empty((shp["B"], shp["Hq"], shp["Sq"]), dtype=torch.float32, device=dev)
    log("prefill inputs ready")

    cd = inputs.workload(DECODE)
    dshp = cd.shape
    d_q = to_dev(cd.bits("q"))
    d_kc, d_vc = to_dev(cd.kcache_bits), to_dev(cd.vcache_bits)
    d_bt = torch.from_numpy(cd.block_table).to(dev)
    d_sl = torch.from_numpy(cd.seqlens).to(dev)
    d_o = torch.empty_like(d_q)
    d_l = torch.empty((dshp["nseq"], dshp["Hq"]), dtype=torch.float32, device=dev)
    ws_bytes = binding.fa_decode_workspace_size(dshp["nseq"], dshp["Hq"], dshp["Hkv"], dshp["d"],
                                                dshp["block_size"], dshp["max_blocks"])
    d_ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    # Between timed calls the caches are flushed by READING a 512 MiB buffer:
    # L2 and the 256 MB Infinity Cache then hold only clean lines of an
    # unrelated buffer.  Writing the buffer instead would leave them full of
    # dirty lines whose write-back the next kernel pays for (the prefill took
    # 65-69 us after a 512 MiB fill against 57-60 us after a 512 MiB read and
    # 55 us warm; the decode was the same after either).
    flush_buf = torch.ones(128 << 20, dtype=torch.float32, device=dev)

    def flush_caches():
        flush_buf.sum()

    log("decode inputs ready")

    def run_f32():
        binding.fa_fwd(f_q, f_k, f_v, cf.causal, cf.scale, out=f_o, lse=f_l)

    def run_prefill():
        binding.fa_fwd(p_q, p_k, p_v, True, cp.scale, out=p_o, lse=p_l)

    def run_decode():
        binding.fa_decode(d_q, d_kc, d_vc, d_bt, d_sl, cd.scale, out=d_o, lse=d_l, workspace=d_ws)

    stream = torch.cuda.current_stream(dev)
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        run_f32()
        run_prefill()
        flush_caches()
        run_decode()
    torch.cuda.synchronize()

    K = args.steps
    e_f, e_p, e_d = kernel_events(K), kernel_events(K), kernel_events(K)
    t_start, t_end = ev(), ev()
    log(f"timing {K} steps")
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    lead = gpu_lead(stream, 2.0 + 0.6 * K)
    host0 = time.perf_counter()
    t_start.record(stream)
    for i in range(K):
        binding.fa_time_next_call(*e_f[i])
        run_f32()
        binding.fa_time_next_call(*e_p[i])
        run_prefill()
        flush_caches()
        binding.fa_time_next_call(*e_d[i])
        run_decode()
    t_end.record(stream)
    host_s = time.perf_counter() - host0
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = t_start.elapsed_time(t_end) / K
    lead_main = lead_report(lead, host_s)
    log(f"host lead: {lead_main}")

    ms_f = [a.elapsed_ms(b) for a, b in e_f]
    ms_p = [a.elapsed_ms(b) for a, b in e_p]
    ms_d = [a.elapsed_ms(b) for a, b in e_d]
    sp, sd, sf = metrics.summarize(ms_p), metrics.summarize(ms_d), metrics.summarize(ms_f)

    flops_p = metrics.prefill_flops(shp["B"], shp["Hq"], shp["Sq"], shp["Sk"], shp["d"], True)
    tflops_p = flops_p / (sp["mean"] * 1e-3) / 1e12
    kv_bytes = metrics.decode_kv_bytes(cd.seqlens, dshp["Hkv"], dshp["d"])
    gbs_d = kv_bytes / (sd["mean"] * 1e-3) / 1e9
    peak_tf = metrics.MI355X_BF16_DENSE_FLOPS / 1e12
    peak_gb = metrics.MI355X_HBM_BYTES_PER_S / 1e9
    log(f"prefill {sp['mean']*1e3:.1f} us -> {tflops_p:.1f} TFLOP/s; decode {sd['mean']*1e3:.1f} us -> "
        f"{gbs_d:.0f} GB/s; fp32 {sf['mean']*1e3:.1f} us; step {ms_step:.3f} ms")

    result = {
        "metric": METRIC,
        "value": round(tflops_p, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), bf16-rounded; paged cache with seeded lengths and block permutation)",
        "config": {
            "workload": PREFILL, "B": shp["B"], "Hq": shp["Hq"], "Hkv": shp["Hkv"], "S": shp["Sq"],
            "d": shp["d"], "causal": True,
            "step_also_runs": [FP32, DECODE],
        },
        "roofline": {
            "kernel": "fwd_bf16_kernel<128,causal,pair>",
            "bound": "mfma",
            "achieved": round(tflops_p, 2),
            "peak": peak_tf,
            "unit": "TFLOP/s",
            "frac": round(tflops_p / peak_tf, 4),
            "traffic": profiling.current_traffic(PROFILE_PREFILL),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_flops_per_launch": flops_p,
            "launch_us": {k: round(v * 1e3, 2) for k, v in sp.items() if k != "n"},
            "launch_timing": "HIP events recorded by the kernel launch itself (hipExtLaunchKernel; "
                             "no system-scope fence), first kernel start to last kernel end",
        },
        "decode": {
            "workload": DECODE,
            "kernels": "decode_partial_kernel<4> + decode_combine_kernel<4>",
            "bound": "hbm",
            "achieved": round(gbs_d, 1),
            "peak": peak_gb,
            "unit": "GB/s",
            "frac": round(gbs_d / peak_gb, 4),
            "traffic": profiling.current_traffic(PROFILE_DECODE),
            "traffic_unit": "HBM bytes per launch of decode_partial_kernel (rocprofv3, copy-calibrated)",
            "algorithmic_kv_bytes_per_launch": kv_bytes,
            "kv_tokens": cd.kv_tokens,
            "launch_us": {k: round(v * 1e3, 2) for k, v in sd.items() if k != "n"},
        },
        "fp32_prefill_us": round(sf["mean"] * 1e3, 2),
        "wall_s_timed_region": round(wall, 4),
        "host_lead": lead_main,
    }

    # ---- attention backward on the headline shape, timed on its own ----
    if not args.no_backward:
        log("backward: inputs")
        g_do = to_dev(inputs.bf16_bits(inputs.make_grad_out(cp.q.shape, seed=2)))
        binding.fa_fwd(p_q, p_k, p_v, True, cp.scale, out=p_o, lse=p_l)
        b_dq, b_dk, b_dv = torch.empty_like(p_q), torch.empty_like(p_k), torch.empty_like(p_v)
        b_ws = torch.empty(binding.fa_bwd_workspace_size(shp["B"], shp["Hq"], shp["Sq"]), dtype=torch.uint8,
                           device=dev)

        def run_bwd():
            binding.fa_bwd(p_q, p_k, p_v, p_o, g_do, p_l, True, cp.scale, dq=b_dq, dk=b_dk, dv=b_dv, workspace=b_ws)

        for _ in range(2):
            run_bwd()
        reps = max(5, min(K, 20))
        evs = kernel_events(reps)
        torch.cuda.synchronize()
        lead = gpu_lead(stream, 2.0 + 0.3 * reps)
        host0 = time.perf_counter()
        for a, b in evs:
            binding.fa_time_next_call(a, b)
            run_bwd()
        host_s = time.perf_counter() - host0
        torch.cuda.synchronize()
        lead_bwd = lead_report(lead, host_s)
        st = metrics.summarize([a.elapsed_ms(b) for a, b in evs])
        fl = metrics.backward_flops(shp["B"], shp["Hq"], shp["Sq"], shp["Sk"], shp["d"], True)
        tf = fl / (st["mean"] * 1e-3) / 1e12
        result["backward"] = {
            "workload": PREFILL, "kernels": "bwd_delta_kernel + bwd_dq_kernel<causal> + bwd_dkdv_kernel<causal>",
            "bound": "mfma", "achieved": round(tf, 1), "peak": peak_tf, "unit": "TFLOP/s",
            "frac": round(tf / peak_tf, 4), "algorithmic_flops_per_launch": fl,
            "note": "algorithmic = 5 products of 2d FLOP per visible pair; the kernels execute 7 (S and dP are "
                    "recomputed in both the dQ and the dK/dV kernel)",
            "launch_us": {k: round(v * 1e3, 2) for k, v in st.items() if k != "n"},
            "host_lead": lead_bwd,
        }
        log(f"backward: {st['mean']*1e3:.1f} us -> {tf:.1f} TFLOP/s")
        del g_do, b_dq, b_dk, b_dv, b_ws

    # ---- FP8 forward on the headline shape: quantize (rotated Q, K; V blocks), then attend ----
    if not args.no_fp8:
        log("fp8: quantize + forward")
        rot = to_dev(inputs.bf16_bits(inputs.make_rotation(shp["d"], seed=2)))

        def run_fp8(evs=None):
            names = ("quant_q", "quant_k", "quant_v", "fwd_fp8")
            calls = (lambda: binding.fa_quantize_fp8(p_q, 128, rot=rot),
                     lambda: binding.fa_quantize_fp8(p_k, 64, rot=rot),
                     lambda: binding.fa_quantize_fp8(p_v, 64, layout=binding.FA_FP8_VBLOCKS))
            outs = []
            for n, fn in zip(names[:3], calls):
                if evs is not None:
                    binding.fa_time_next_call(*evs[n])
                outs.append(fn())
            (q8, qs), (k8, ks), (v8, vs) = outs
            if evs is not None:
                binding.fa_time_next_call(*evs["fwd_fp8"])
            binding.fa_fwd_fp8(q8, qs, k8, ks, v8, vs, True, cp.scale, out=p_o, lse=p_l)

        for _ in range(2):
            run_fp8()
        reps = max(5, min(K, 20))
        names = ("quant_q", "quant_k", "quant_v", "fwd_fp8")
        evs = [{n: (binding.TimingEvent(), binding.TimingEvent()) for n in names} for _ in range(reps)]
        torch.cuda.synchronize()
        lead = gpu_lead(stream, 2.0 + 0.5 * reps)
        host0 = time.perf_counter()
        for i in range(reps):
            flush_caches()        # cold caches, as in the step
            run_fp8(evs[i])
        host_s = time.perf_counter() - host0
        torch.cuda.synchronize()
        st = {n: metrics.summarize([e[n][0].elapsed_ms(e[n][1]) for e in evs]) for n in names}
        tf8 = flops_p / (st["fwd_fp8"]["mean"] * 1e-3) / 1e12
        peak8 = metrics.MI355X_FP8_DENSE_FLOPS / 1e12
        bh_q, bh_kv = shp["B"] * shp["Hq"], shp["B"] * shp["Hkv"]
        qbytes = {"quant_q": metrics.fp8_quantize_bytes(bh_q, shp["Sq"], shp["d"], 128),
                  "quant_k": metrics.fp8_quantize_bytes(bh_kv, shp["Sk"], shp["d"], 64),
                  "quant_v": metrics.fp8_quantize_bytes(bh_kv, shp["Sk"], shp["d"], 64)}
        result["fp8"] = {
            "workload": PREFILL, "kernel": "fwd_fp8_kernel<causal>", "bound": "mfma",
            "achieved": round(tf8, 1), "peak": peak8, "unit": "TFLOP/s", "frac": round(tf8 / peak8, 4),
            "vs_bf16_kernel": round(sp["mean"] / st["fwd_fp8"]["mean"], 3),
            "traffic": profiling.current_traffic(PROFILE_FP8),
            "algorithmic_flops_per_launch": flops_p,
            "launch_us": {k: round(v * 1e3, 2) for k, v in st["fwd_fp8"].items() if k != "n"},
            "quantize": {n: {"us": round(st[n]["mean"] * 1e3, 2), "bytes": qbytes[n],
                             "GB/s": round(qbytes[n] / (st[n]["mean"] * 1e-3) / 1e9, 1)} for n in qbytes},
            "note": "E4M3 Q, K (rotated by a seeded orthogonal matrix) and V with power-of-two block scales; "
                    "caches flushed before each quantize + forward sequence",
            "host_lead": lead_report(lead, host_s),
        }
        log(f"fp8: forward {st['fwd_fp8']['mean']*1e3:.1f} us -> {tf8:.1f} TFLOP/s; quantize q/k/v "
            f"{st['quant_q']['mean']*1e3:.1f}/{st['quant_k']['mean']*1e3:.1f}/{st['quant_v']['mean']*1e3:.1f} us")

    # ---- multi-query paged attention (verify step, 8 new tokens per sequence) ----
    if not args.no_verify:
        log("verify: inputs")
        cv = inputs.workload(VERIFY)
        vshp = cv.shape
        v_q = to_dev(cv.bits("q"))
        v_kc, v_vc = to_dev(cv.kcache_bits), to_dev(cv.vcache_bits)
        v_bt = torch.from_numpy(cv.block_table).to(dev)
        v_sl = torch.from_numpy(cv.seqlens).to(dev)
        v_o = torch.empty_like(v_q)
        v_l = torch.empty((vshp["nseq"], vshp["Sq"], vshp["Hq"]), dtype=torch.float32, device=dev)
        v_ws = torch.empty(binding.fa_decode_multi_workspace_size(vshp["nseq"], vshp["Sq"], vshp["Hq"], vshp["Hkv"],
                                                                  vshp["d"], vshp["block_size"], vshp["max_blocks"]),
                           dtype=torch.uint8, device=dev)

        def run_verify():
            binding.fa_decode_multi(v_q, v_kc, v_vc, v_bt, v_sl, cv.scale, out=v_o, lse=v_l, workspace=v_ws)

        for _ in range(2):
            run_verify()
        reps = max(5, min(K, 20))
        evs = kernel_events(reps)
        torch.cuda.synchronize()
        lead = gpu_lead(stream, 2.0 + 0.3 * reps)
        host0 = time.perf_counter()
        for i, (a, b) in enumerate(evs):
            flush_caches()
            binding.fa_time_next_call(a, b)
            run_verify()
        host_s = time.perf_counter() - host0
        torch.cuda.synchronize()
        st = metrics.summarize([a.elapsed_ms(b) for a, b in evs])
        vbytes = metrics.decode_kv_bytes(cv.seqlens, vshp["Hkv"], vshp["d"])
        gbs_v = vbytes / (st["mean"] * 1e-3) / 1e9
        result["verify"] = {
            "workload": VERIFY, "kernels": "mq_partial_kernel<4> + mq_combine_kernel<4>", "bound": "hbm",
            "achieved": round(gbs_v, 1), "peak": peak_gb, "unit": "GB/s", "frac": round(gbs_v / peak_gb, 4),
            "traffic": profiling.current_traffic(PROFILE_VERIFY),
            "algorithmic_kv_bytes_per_launch": vbytes, "kv_tokens": cv.kv_tokens,
            "flops_per_launch": metrics.decode_flops(cv.seqlens, vshp["Hq"], vshp["d"]) * vshp["Sq"],
            "launch_us": {k: round(v * 1e3, 2) for k, v in st.items() if k != "n"},
            "note": "caches flushed (512 MiB read) before each launch, outside its events",
            "host_lead": lead_report(lead, host_s),
        }
        log(f"verify: {st['mean']*1e3:.1f} us -> {gbs_v:.0f} GB/s")
        del v_q, v_kc, v_vc, v_o, v_ws
        torch.cuda.empty_cache()

    # ---- latent-cache (MLA) decode: 16 heads over one 512-wide latent per token ----
    if not args.no_mla:
        log("mla: inputs")
        cm = inputs.workload(MLA)
        msh = cm.shape
        m_q, m_wk, m_wv = to_dev(inputs.bf16_bits(cm.q)), to_dev(inputs.bf16_bits(cm.w_uk)), \
            to_dev(inputs.bf16_bits(cm.w_uv_t))
        m_cc = to_dev(cm.ccache_bits)
        m_bt = torch.from_numpy(cm.cache.block_table).to(dev)
        m_sl = torch.from_numpy(cm.cache.seqlens).to(dev)
        m_o = torch.empty_like(m_q)
        m_l = torch.empty((msh["nseq"], msh["H"]), dtype=torch.float32, device=dev)
        m_ws = torch.empty(binding.fa_mla_decode_workspace_size(msh["nseq"], msh["H"], msh["d_h"], msh["d_c"],
                                                                msh["block_size"], msh["max_blocks"]),
                           dtype=torch.uint8, device=dev)

        def run_mla():
            binding.fa_mla_decode(m_q, m_wk, m_wv, m_cc, m_bt, m_sl, cm.scale, out=m_o, lse=m_l, workspace=m_ws)

        for _ in range(2):
            run_mla()
        reps = max(5, min(K, 20))
        evs = kernel_events(reps)
        torch.cuda.synchronize()
        lead = gpu_lead(stream, 2.0 + 0.3 * reps)
        host0 = time.perf_counter()
        for i, (a, b) in enumerate(evs):
            flush_caches()
            binding.fa_time_next_call(a, b)
            run_mla()
        host_s = time.perf_counter() - host0
        torch.cuda.synchronize()
        st = metrics.summarize([a.elapsed_ms(b) for a, b in evs])
        lat_bytes = metrics.mla_latent_bytes(cm.cache.seqlens, msh["d_c"])
        gbs_m = lat_bytes / (st["mean"] * 1e-3) / 1e9
        result["mla"] = {
            "workload": MLA, "bound": "hbm",
            "kernels": "mla_absorb_kernel + mla_partial_kernel + mla_combine_kernel + mla_upproj_kernel",
            "achieved": round(gbs_m, 1), "peak": peak_gb, "unit": "GB/s", "frac": round(gbs_m / peak_gb, 4),
            "traffic": profiling.current_traffic(PROFILE_MLA),
            "algorithmic_latent_bytes_per_launch": lat_bytes,
            "min_bytes_per_launch": metrics.mla_total_bytes(cm.cache.seqlens, msh["H"], msh["d_h"], msh["d_c"]),
            "kv_tokens": cm.cache.kv_tokens,
            "flops_per_launch": metrics.mla_flops(cm.cache.seqlens, msh["H"], msh["d_h"], msh["d_c"]),
            "materialized_kv_bytes_equivalent": metrics.decode_kv_bytes(cm.cache.seqlens, msh["H"], msh["d_h"]),
            "launch_us": {k: round(v * 1e3, 2) for k, v in st.items() if k != "n"},
            "note": "achieved = latent bytes over the whole call (4 kernels); caches flushed (512 MiB read) "
                    "before each call, outside its events",
            "host_lead": lead_report(lead, host_s),
        }
        log(f"mla: {st['mean']*1e3:.1f} us -> {gbs_m:.0f} GB/s of latents")
        del m_q, m_wk, m_wv, m_cc, m_o, m_ws, cm
        torch.cuda.empty_cache()

    # ---- larger prefill workloads, timed on their own ----
    clock = GfxClock()
    # ---- shader clock under the headline prefill, repeated back to back ----
    if clock.h is not None:
        for _ in range(3):
            run_prefill()
        torch.cuda.synchronize()
        lead = gpu_lead(stream, 40.0)           # the host enqueues every prefill before the GPU starts them
        for _ in range(400):
            run_prefill()
        done = torch.cuda.Event()
        done.record(stream)
        samples = clock.sample_until(done, start=lead[1])
        torch.cuda.synchronize()
        # (the first quarter of the samples is dropped: the clock settles under the new load)
        result["roofline"]["gfx_clock_under_load"] = clock_report(samples[len(samples) // 4:])

    if not args.no_extra:
        extra = {}
        for name in EXTRA:
            spec = dict(inputs.WORKLOADS[name])
            log(f"generating {name}")
            c = inputs.workload(name)
            s = c.shape
            q, k, v = to_dev(c.bits("q")), to_dev(c.bits("k")), to_dev(c.bits("v"))
            del c
            o = torch.empty_like(q)
            lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
            scale = 1.0 / math.sqrt(s["d"])
            for _ in range(2):
                binding.fa_fwd(q, k, v, True, scale, out=o, lse=lse)
            # at least 50 timed launches of the 8k workload, 20 of the 32k one (with the default --steps)
            reps = max(3, min(K, 20 if s["Sq"] > 8192 else 50))
            evs = kernel_events(reps)
            torch.cuda.synchronize()
            lead = gpu_lead(stream, 2.0 + 0.3 * reps)
            host0 = time.perf_counter()
            for a, b in evs:
                binding.fa_time_next_call(a, b)
                binding.fa_fwd(q, k, v, True, scale, out=o, lse=lse)
            host_s = time.perf_counter() - host0
            done = torch.cuda.Event()
            done.record(stream)
            samples = clock.sample_until(done, start=lead[1])
            torch.cuda.synchronize()
            st = metrics.summarize([a.elapsed_ms(b) for a, b in evs])
            fl = metrics.prefill_flops(s["B"], s["Hq"], s["Sq"], s["Sk"], s["d"], True)
            tf = fl / (st["mean"] * 1e-3) / 1e12
            extra[name] = {"us": round(st["mean"] * 1e3, 1), "TFLOP/s": round(tf, 1),
                           "frac_bf16_peak": round(tf / peak_tf, 4), "reps": reps, "causal": spec["causal"],
                           "host_lead": lead_report(lead, host_s),
                           "gfx_clock_under_load": clock_report(samples[len(samples) // 4:])}
            log(f"{name}: {st['mean']*1e3:.1f} us -> {tf:.1f} TFLOP/s")
            del q, k, v, o, lse
            torch.cuda.empty_cache()
        result["extra_prefill"] = extra

    # ---- the fp64 oracle on the host, a bounded sample of the prefill workload ----
    if not args.no_cpu_baseline:
        import oracle
        try:
            from threadpoolctl import threadpool_info
            threads = max((p.get("num_threads", 1) for p in threadpool_info()
                           if p.get("user_api") == "blas"), default=1)
        except Exception:  # threadpoolctl missing or no BLAS reported
            threads = os.cpu_count() or 1
        # the whole prefill workload, one batch entry at a time, repeated
        # until at least CPU_MIN_SECONDS of oracle work has been timed
        h = max(1, min(args.cpu_heads, shp["Hq"]))
        log(f"timing the fp64 oracle on the prefill workload ({h} heads per call)")
        reps, dt = 0, 0.0
        while dt < CPU_MIN_SECONDS:
            for b_ in range(shp["B"]):
                for h0 in range(0, shp["Hq"], h):
                    t0 = time.perf_counter()
                    oracle.sdpa(cp.q[b_:b_ + 1, h0:h0 + h], cp.k[b_:b_ + 1, h0:h0 + h], cp.v[b_:b_ + 1, h0:h0 + h],
                                True, cp.scale)
                    dt += time.perf_counter() - t0
            reps += 1
        fl = reps * flops_p
        result["cpu_baseline"] = {
            "value": round(fl / dt / 1e12, 6),
            "unit": "TFLOP/s",
            "cores": int(threads),
            "kind": "oracle",
            "sample": f"the whole {PREFILL} workload ({shp['B']}x{shp['Hq']} heads, all {shp['Sq']} rows), "
                      f"{h} heads per oracle call, {reps} pass(es), {dt:.1f} s of fp64 NumPy; algorithmic "
                      f"causal FLOPs over oracle time",
            "host_cpus": os.cpu_count(),
        }
        log(f"oracle: {dt:.2f} s for {reps} pass(es)")

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
