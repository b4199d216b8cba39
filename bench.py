#!/usr/bin/env python3
"""Benchmark of the exact tiled attention hot path on one MI355X.

One step runs the whole path once on resident synthetic inputs:

  * fp32 prefill, B=1 H=1 S=128 d=64, non-causal (correctness-sized; launch bound)
  * bf16 causal GQA prefill, B=1 Hq=32 Hkv=8 S=32768 d=128 (the headline
    workload: the largest of the five, on one GPU)
  * bf16 paged decode, 64 sequences x 1 token, Hq=32 Hkv=8 d=128, 16-token
    pages, lengths uniform in [1024, 8192]

Each call is timed with HIP events that its own kernel launches record
(fa_time_next_call: the first kernel's start to the last kernel's end, on the
stream the kernels run on; the events skip the system-scope cache fence), the
interval a kernel trace reports.  A spin kernel queued ahead of each timed
loop lets the host enqueue every timed launch before the GPU gets there (the
JSON's `host_lead` says whether it did).  The headline `value` is the
algorithmic TFLOP/s of the 32k causal prefill (4 d FLOP per visible query-key
pair) over its launch time; decode reports the algorithmic KV bytes (each
attended token's K and V once) over the decode launch time.  Before each
decode launch, and before every launch of the other prefill workloads, a
512 MiB buffer is read so that neither L2 nor the 256 MB Infinity Cache holds
lines of the previous call (outside the call's own events).  The flush reads
rather than writes: a write leaves the caches full of dirty lines whose
write-back would be charged to the next timed kernel.  `traffic` is the HBM
bytes per launch that the rocprofv3 counter passes summarised under profiles/
measured, and `mfma_busy` the matrix-core busy fraction of the same runs,
both reported only while the kernel source is the one they measured.

`per_config` holds every workload: the 2k and 8k prefills with their own
roofline blocks, the fp32 and decode figures of the step.  The fp64 CPU
oracle is timed on the same workloads on the host (`cpu_baseline`: the 32k
workload's 512 checked rows per head at the top level, the others in full
under `per_config`), as a reported baseline.

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
HEADLINE = "causal_gqa_h32kv8_s32768_d128"
DECODE = "paged_decode_64seq_h32kv8_d128"
FP32 = "mha1_s128_d64_f32"
PREFILL2K = "causal_mha_b2_h16_s2048_d128"
PREFILL8K = "causal_gqa_h32kv8_s8192_d128_outliers"
VERIFY = "paged_verify_64seq_q8_h32kv8_d128"
MLA = "mla_decode_64seq_h16_dc512"


def _profile(name):
    return os.path.join(ROOT, "profiles", name + ".md")


# rocprofv3 summaries whose FETCH_SIZE / WRITE_SIZE and MFMA passes give the
# HBM traffic and busy fraction per launch; used only while the kernel source
# still has the recorded hash
PROFILES = {
    HEADLINE: _profile("fwd_bf16_causal_gqa_h32kv8_s32768_d128"),
    PREFILL8K: _profile("fwd_bf16_causal_gqa_h32kv8_s8192_d128_outliers"),
    PREFILL2K: _profile("fwd_bf16_causal_mha_b2_h16_s2048_d128"),
    DECODE: _profile("decode_paged_64seq_h32kv8_d128"),
    "fp8": _profile("fwd_fp8_causal_mha_b2_h16_s2048_d128"),
    "fp8q": _profile("fwd_fp8_qbf16_causal_mha_b2_h16_s2048_d128"),
    ("fp8", PREFILL8K): _profile("fwd_fp8_causal_gqa_h32kv8_s8192_d128_outliers"),
    ("fp8", HEADLINE): _profile("fwd_fp8_causal_gqa_h32kv8_s32768_d128"),
    "quant": _profile("quant_fp8_qkv_b2_h16_s2048_d128"),
    VERIFY: _profile("decode_multi_paged_64seq_q8_h32kv8_d128"),
    MLA: _profile("mla_decode_64seq_h16_dc512"),
}
CPU_MIN_SECONDS = 0.5     # small oracle runs are repeated until they take this long


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


def kernel_events(n):
    """n (start, stop) pairs of timing events for fa_time_next_call."""
    from exact_tiled_attention_14_amd import binding
    return [(binding.TimingEvent(), binding.TimingEvent()) for _ in range(n)]


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-extra", action="store_true", help="skip the 2k/8k prefill timings")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward timing")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 forward timing")
    ap.add_argument("--no-verify", action="store_true", help="skip the multi-query (verify) decode timing")
    ap.add_argument("--no-mla", action="store_true", help="skip the latent-cache (MLA) decode timing")
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
    peak_tf = metrics.MI355X_BF16_DENSE_FLOPS / 1e12
    peak_gb = metrics.MI355X_HBM_BYTES_PER_S / 1e9

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def us(st):
        return {k: round(v * 1e3, 2) for k, v in st.items() if k != "n"}

    # ---- inputs, built on the host by the seeded generator, copied once ----
    log("generating inputs")
    cf = inputs.workload(FP32)
    f_q, f_k, f_v = (torch.from_numpy(getattr(cf, n)).to(dev) for n in "qkv")
    f_o, f_l = torch.empty_like(f_q), torch.empty(cf.q.shape[:3], dtype=torch.float32, device=dev)

    ch = inputs.workload(HEADLINE)
    shp = ch.shape
    p_q, p_k, p_v = to_dev(ch.bits("q")), to_dev(ch.bits("k")), to_dev(ch.bits("v"))
    p_o = torch.empty_like(p_q)
    p_l = torch.empty((shp["B"], shp["Hq"], shp["Sq"]), dtype=torch.float32, device=dev)
    log("headline prefill inputs ready")

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
    # dirty lines whose write-back the next kernel pays for.
    flush_buf = torch.ones(128 << 20, dtype=torch.float32, device=dev)

    def flush_caches():
        flush_buf.sum()

    log("decode inputs ready")

    def run_f32():
        binding.fa_fwd(f_q, f_k, f_v, cf.causal, cf.scale, out=f_o, lse=f_l)

    def run_prefill():
        binding.fa_fwd(p_q, p_k, p_v, True, ch.scale, out=p_o, lse=p_l)

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

    sp = metrics.summarize([a.elapsed_ms(b) for a, b in e_p])
    sd = metrics.summarize([a.elapsed_ms(b) for a, b in e_d])
    sf = metrics.summarize([a.elapsed_ms(b) for a, b in e_f])

    flops_p = metrics.prefill_flops(shp["B"], shp["Hq"], shp["Sq"], shp["Sk"], shp["d"], True)
    tflops_p = flops_p / (sp["mean"] * 1e-3) / 1e12
    kv_bytes = metrics.decode_kv_bytes(cd.seqlens, dshp["Hkv"], dshp["d"])
    gbs_d = kv_bytes / (sd["mean"] * 1e-3) / 1e9
    log(f"prefill {sp['mean']*1e3:.1f} us -> {tflops_p:.1f} TFLOP/s; decode {sd['mean']*1e3:.1f} us -> "
        f"{gbs_d:.0f} GB/s; fp32 {sf['mean']*1e3:.1f} us; step {ms_step:.3f} ms")

    def prefill_roofline(kernel, flops, st, prof, note):
        pr = profiling.current_profile(prof)
        tf = flops / (st["mean"] * 1e-3) / 1e12
        # the shader clock the kernel ran at under the profiler: its active
        # cycles per XCD over its mean duration (counter and trace passes)
        sclk = (pr["active_cycles"] / pr["kernel_avg_us"]
                if pr["active_cycles"] and pr["kernel_avg_us"] else None)
        return {
            "kernel": kernel, "bound": "mfma", "achieved": round(tf, 2), "peak": peak_tf, "unit": "TFLOP/s",
            "frac": round(tf / peak_tf, 4), "traffic": pr["traffic"],
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "effective_sclk_mhz": round(sclk, 0) if sclk else None,
            "frac_of_peak_at_effective_sclk": round(tf / (peak_tf * sclk / 2400.0), 4) if sclk else None,
            "mfma_busy": pr["mfma_busy"], "profile": pr["profile"], "profile_kernel_avg_us": pr["kernel_avg_us"],
            "algorithmic_flops_per_launch": flops, "launch_us": us(st), "caches": note,
            "launch_timing": "HIP events recorded by the kernel launch itself (hipExtLaunchKernel; "
                             "no system-scope fence), first kernel start to last kernel end",
        }

    headline_roof = prefill_roofline("fwd_bf16_kernel<128,causal,grid>", flops_p, sp, PROFILES[HEADLINE],
                                     "runs after the previous step's decode; 8 ms per launch, so the "
                                     "caches' start state matters little")
    decode_block = {
        "workload": DECODE,
        "kernels": "decode_partial_kernel<4> + decode_combine_kernel<4>",
        "bound": "hbm",
        "achieved": round(gbs_d, 1),
        "peak": peak_gb,
        "unit": "GB/s",
        "frac": round(gbs_d / peak_gb, 4),
        "traffic": profiling.current_profile(PROFILES[DECODE])["traffic"],
        "traffic_unit": "HBM bytes per launch of decode_partial_kernel (rocprofv3, copy-calibrated)",
        "algorithmic_kv_bytes_per_launch": kv_bytes,
        "kv_tokens": cd.kv_tokens,
        "launch_us": us(sd),
        "caches": "flushed (512 MiB read) before each launch, outside its events",
    }
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
            "workload": HEADLINE, "B": shp["B"], "Hq": shp["Hq"], "Hkv": shp["Hkv"], "S": shp["Sq"],
            "d": shp["d"], "causal": True,
            "step_also_runs": [FP32, DECODE],
        },
        "roofline": headline_roof,
        "decode": decode_block,
        "per_config": {
            FP32: {"launch_us": us(sf), "bound": "launch", "note": "correctness-sized (4.2 MFLOP)"},
            HEADLINE: {"see": "roofline"},
            DECODE: {"see": "decode"},
        },
        "wall_s_timed_region": round(wall, 4),
        "host_lead": lead_main,
    }

    def time_calls(fn, reps, flush, lead_ms_per_rep):
        """Launch statistics of `reps` calls of fn, each preceded by a cache flush
        (outside its events) when `flush`."""
        for _ in range(2):
            fn()
        evs = kernel_events(reps)
        torch.cuda.synchronize()
        lead = gpu_lead(stream, 2.0 + lead_ms_per_rep * reps)
        host0 = time.perf_counter()
        for a, b in evs:
            if flush:
                flush_caches()
            binding.fa_time_next_call(a, b)
            fn()
        host_s = time.perf_counter() - host0
        torch.cuda.synchronize()
        st = metrics.summarize([a.elapsed_ms(b) for a, b in evs])
        return st, lead_report(lead, host_s)

    # ---- the fp32 workload on its own (the step times it once per step) ----
    if not args.no_extra:
        st_f, _ = time_calls(lambda: binding.fa_fwd(f_q, f_k, f_v, cf.causal, cf.scale, out=f_o, lse=f_l),
                             max(5, min(K * 3, 60)), False, 0.05)
        result["per_config"][FP32]["launch_us_alone"] = us(st_f)
        result["per_config"][FP32]["reps_alone"] = max(5, min(K * 3, 60))

    # ---- FP8 forward at a long workload (the multi-round grid): rotated Q and
    # K, V in 64-key blocks; the one-launch quantizer, the forward on the codes
    # and the forward that quantizes Q itself, each timed on its own ----
    fp8_long = {}

    def fp8_at(name, q, k, v, scale, fl, bf16_us, reps):
        rot = to_dev(inputs.bf16_bits(inputs.make_rotation(q.shape[-1], seed=2)))
        q8, qs, k8, ks, v8, vs = binding.fa_quantize_fp8_qkv(q, k, v, rot=rot)
        o8 = torch.empty_like(q)
        l8 = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        st_q, _ = time_calls(lambda: binding.fa_quantize_fp8_qkv(q, k, v, rot=rot), reps, True, 0.1)
        st_8, _ = time_calls(lambda: binding.fa_fwd_fp8(q8, qs, k8, ks, v8, vs, True, scale, out=o8, lse=l8),
                             reps, True, 0.1)
        st_f, _ = time_calls(lambda: binding.fa_fwd_fp8_qbf16(q, k8, ks, v8, vs, True, rot=rot, scale=scale,
                                                              out=o8, lse=l8), reps, True, 0.1)
        peak8 = metrics.MI355X_FP8_DENSE_FLOPS / 1e12
        t8, tf, tq = st_8["mean"] * 1e3, st_f["mean"] * 1e3, st_q["mean"] * 1e3
        a8, af = fl / (t8 * 1e-6) / 1e12, fl / (tf * 1e-6) / 1e12
        out = {
            "workload": name, "kernel": "fwd_fp8_kernel<causal,grid>", "bound": "mfma", "achieved": round(a8, 1),
            "peak": peak8, "unit": "TFLOP/s", "frac": round(a8 / peak8, 4), "launch_us": us(st_8), "reps": reps,
            "traffic": profiling.current_profile(PROFILES[("fp8", name)])["traffic"],
            "forward_q_bf16": {"entry_point": "fa_fwd_fp8_qbf16", "us": round(tf, 2), "achieved": round(af, 1),
                               "frac": round(af / peak8, 4), "launch_us": us(st_f)},
            "quantize_qkv_us": round(tq, 2), "bf16_forward_us": round(bf16_us, 2),
            "vs_bf16_forward": {"codes": round(bf16_us / t8, 3), "q_bf16": round(bf16_us / tf, 3),
                                "quantize_qkv_plus_forward": round(bf16_us / (tq + t8), 3)},
            "note": "codes of rotated Q and K and of V from one quantizer launch; caches flushed (512 MiB read) "
                    "before each launch, outside its events",
        }
        del q8, qs, k8, ks, v8, vs, o8, l8
        torch.cuda.empty_cache()
        log(f"fp8 {name}: {t8:.1f} us ({a8 / peak8:.3f} of FP8 peak), Q quantized inside {tf:.1f} us, "
            f"quantize {tq:.1f} us; bf16 {bf16_us:.1f} us")
        return out

    if not args.no_fp8:
        fp8_long[HEADLINE] = fp8_at(HEADLINE, p_q, p_k, p_v, ch.scale, flops_p, sp["mean"] * 1e3,
                                    max(3, min(K, 10)))

    # ---- the 2k and 8k prefill workloads, each on its own, cold caches ----
    if not args.no_extra:
        for name, reps in ((PREFILL2K, max(5, min(K * 3, 60))), (PREFILL8K, max(5, min(K * 3, 60)))):
            log(f"generating {name}")
            c = inputs.workload(name)
            s = c.shape
            q, k, v = to_dev(c.bits("q")), to_dev(c.bits("k")), to_dev(c.bits("v"))
            del c
            o = torch.empty_like(q)
            lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
            scale = 1.0 / math.sqrt(s["d"])
            st, lead_x = time_calls(lambda: binding.fa_fwd(q, k, v, True, scale, out=o, lse=lse), reps, True,
                                         0.3)
            fl = metrics.prefill_flops(s["B"], s["Hq"], s["Sq"], s["Sk"], s["d"], True)
            # (the launch's choice: a causal square problem whose heavy/light query-block
            # pairs fit one 8-wave workgroup per CU runs as the pair grid)
            pair = (s["Sq"] == s["Sk"] and s["Sq"] % 128 == 0 and s["Sq"] >= 256
                    and s["B"] * s["Hq"] * ((s["Sq"] // 128 + 1) // 2) <= torch.cuda.get_device_properties(dev).multi_processor_count)
            roof = prefill_roofline("fwd_bf16_kernel<128,causal,%s>" % ("pair" if pair else "grid"), fl, st,
                                    PROFILES[name], "flushed (512 MiB read) before each launch, outside its events")
            roof.update({"reps": reps, "host_lead": lead_x, "shape": {k_: s[k_] for k_ in ("B", "Hq", "Hkv", "Sq", "Sk", "d")}})
            result["per_config"][name] = roof
            log(f"{name}: {st['mean']*1e3:.1f} us -> {roof['achieved']:.1f} TFLOP/s ({roof['frac']:.3f} of peak)")
            if name == PREFILL8K and not args.no_fp8:
                fp8_long[name] = fp8_at(name, q, k, v, scale, fl, st["mean"] * 1e3, max(5, min(K, 20)))
            del q, k, v, o, lse
            torch.cuda.empty_cache()

    # ---- attention backward and FP8 forward on the 2k workload, each timed on its own ----
    if not (args.no_backward and args.no_fp8):
        log("backward / fp8: inputs")
        cb = inputs.workload(PREFILL2K)
        bs_ = cb.shape
        b_q, b_k, b_v = to_dev(cb.bits("q")), to_dev(cb.bits("k")), to_dev(cb.bits("v"))
        b_o, b_l = torch.empty_like(b_q), torch.empty(b_q.shape[:3], dtype=torch.float32, device=dev)
        g_do = to_dev(inputs.bf16_bits(inputs.make_grad_out(cb.q.shape, seed=2)))
        binding.fa_fwd(b_q, b_k, b_v, True, cb.scale, out=b_o, lse=b_l)
        b_dq, b_dk, b_dv = torch.empty_like(b_q), torch.empty_like(b_k), torch.empty_like(b_v)
        b_ws = torch.empty(binding.fa_bwd_workspace_size(bs_["B"], bs_["Hq"], bs_["Sq"]), dtype=torch.uint8,
                           device=dev)

        def run_bwd():
            binding.fa_bwd(b_q, b_k, b_v, b_o, g_do, b_l, True, cb.scale, dq=b_dq, dk=b_dk, dv=b_dv, workspace=b_ws)

        if not args.no_backward:
            st, lead_b = time_calls(run_bwd, max(5, min(K, 20)), True, 0.4)
            fl = metrics.backward_flops(bs_["B"], bs_["Hq"], bs_["Sq"], bs_["Sk"], bs_["d"], True)
            tf = fl / (st["mean"] * 1e-3) / 1e12
            result["backward"] = {
                "workload": PREFILL2K, "kernels": "bwd_dq_kernel<causal> (also forms D) + bwd_dkdv_kernel<causal>",
                "bound": "mfma", "achieved": round(tf, 1), "peak": peak_tf, "unit": "TFLOP/s",
                "frac": round(tf / peak_tf, 4), "algorithmic_flops_per_launch": fl,
                "note": "algorithmic = 5 products of 2d FLOP per visible pair",
                "launch_us": us(st), "caches": "flushed (512 MiB read) before each call, outside its events",
                "host_lead": lead_b,
            }
            log(f"backward: {st['mean']*1e3:.1f} us -> {tf:.1f} TFLOP/s")

        # ---- FP8 forward on the 2k workload: quantize (rotated Q, K; V blocks), then attend ----
        if not args.no_fp8:
            log("fp8: quantize + forward")
            rot = to_dev(inputs.bf16_bits(inputs.make_rotation(bs_["d"], seed=2)))
            names = ("quantize", "fwd_fp8")

            def run_fp8(evs=None):
                if evs is not None:
                    binding.fa_time_next_call(*evs["quantize"])
                q8, qs, k8, ks, v8, vs = binding.fa_quantize_fp8_qkv(b_q, b_k, b_v, rot=rot)
                if evs is not None:
                    binding.fa_time_next_call(*evs["fwd_fp8"])
                binding.fa_fwd_fp8(q8, qs, k8, ks, v8, vs, True, cb.scale, out=b_o, lse=b_l)

            for _ in range(2):
                run_fp8()
            reps = max(5, min(K, 20))
            evs = [{n: (binding.TimingEvent(), binding.TimingEvent()) for n in names} for _ in range(reps)]
            torch.cuda.synchronize()
            lead = gpu_lead(stream, 2.0 + 0.5 * reps)
            host0 = time.perf_counter()
            for i in range(reps):
                flush_caches()
                run_fp8(evs[i])
            host_s = time.perf_counter() - host0
            torch.cuda.synchronize()
            st = {n: metrics.summarize([e[n][0].elapsed_ms(e[n][1]) for e in evs]) for n in names}
            fl2k = metrics.prefill_flops(bs_["B"], bs_["Hq"], bs_["Sq"], bs_["Sk"], bs_["d"], True)
            tf8 = fl2k / (st["fwd_fp8"]["mean"] * 1e-3) / 1e12
            peak8 = metrics.MI355X_FP8_DENSE_FLOPS / 1e12
            bh_q, bh_kv = bs_["B"] * bs_["Hq"], bs_["B"] * bs_["Hkv"]
            qbytes = (metrics.fp8_quantize_bytes(bh_q, bs_["Sq"], bs_["d"], 128)
                      + 2 * metrics.fp8_quantize_bytes(bh_kv, bs_["Sk"], bs_["d"], 64))
            total_us = sum(st[n]["mean"] for n in names) * 1e3
            bf16_2k = result["per_config"].get(PREFILL2K, {}).get("launch_us", {}).get("mean")
            result["fp8"] = {
                "workload": PREFILL2K, "kernel": "fwd_fp8_kernel<causal,pair>", "bound": "mfma",
                "achieved": round(tf8, 1), "peak": peak8, "unit": "TFLOP/s", "frac": round(tf8 / peak8, 4),
                "traffic": profiling.current_profile(PROFILES["fp8"])["traffic"],
                "algorithmic_flops_per_launch": fl2k,
                "launch_us": us(st["fwd_fp8"]),
                "quantize": {"kernel": "quant_kernel (Q, K and V in one launch)", "us": round(st["quantize"]["mean"] * 1e3, 2),
                             "bytes": qbytes, "GB/s": round(qbytes / (st["quantize"]["mean"] * 1e-3) / 1e9, 1),
                             "frac": round(qbytes / (st["quantize"]["mean"] * 1e-3) / 1e9 / peak_gb, 4),
                             "traffic": profiling.current_profile(PROFILES["quant"])["traffic"]},
                "quantize_plus_forward_us": round(total_us, 2),
                "bf16_forward_us": bf16_2k,
                "note": "E4M3 Q, K (rotated by a seeded orthogonal matrix) and V with power-of-two block scales; "
                        "caches flushed before each quantize + forward sequence",
                "host_lead": lead_report(lead, host_s),
            }
            log(f"fp8: forward {st['fwd_fp8']['mean']*1e3:.1f} us -> {tf8:.1f} TFLOP/s; quantize q+k+v "
                f"{st['quantize']['mean']*1e3:.1f} us")
            # With K and V already held in FP8 (quantized once, as a quantized
            # cache keeps them), a call quantizes only Q: its own timing.
            st_q, _ = time_calls(lambda: binding.fa_quantize_fp8(b_q, 128, rot=rot), reps, True, 0.1)
            q_us = st_q["mean"] * 1e3
            result["fp8"]["quantize_q_only"] = {
                "us": round(q_us, 2), "bytes": metrics.fp8_quantize_bytes(bh_q, bs_["Sq"], bs_["d"], 128),
                "plus_forward_us": round(q_us + st["fwd_fp8"]["mean"] * 1e3, 2),
                "note": "Q alone (rotated), K and V held in FP8 from an earlier quantization",
            }
            log(f"fp8: quantize q alone {q_us:.1f} us")
            # The same with Q quantized inside the forward (fa_fwd_fp8_qbf16):
            # one launch, Q read once in bf16, its codes never written.
            k8h, ksh, v8h, vsh = binding.fa_quantize_fp8_qkv(b_q, b_k, b_v, rot=rot)[2:]
            st_f, _ = time_calls(lambda: binding.fa_fwd_fp8_qbf16(b_q, k8h, ksh, v8h, vsh, True, rot=rot,
                                                                  scale=cb.scale, out=b_o, lse=b_l),
                                 reps, True, 0.1)
            f_us = st_f["mean"] * 1e3
            result["fp8"]["forward_q_bf16"] = {
                "entry_point": "fa_fwd_fp8_qbf16", "kernel": "fwd_fp8_kernel<causal,pair,qbf16>",
                "us": round(f_us, 2), "TFLOP/s": round(fl2k / (f_us * 1e-6) / 1e12, 1),
                "traffic": profiling.current_profile(PROFILES["fp8q"])["traffic"],
                "vs_bf16_forward": round(bf16_2k / f_us, 3) if bf16_2k else None,
                "launch_us": us(st_f),
                "note": "Q in bf16, rotated and quantized inside the forward (bit-identical to quantize + "
                        "fa_fwd_fp8); K and V held in FP8 from an earlier quantization; caches flushed",
            }
            log(f"fp8: forward with Q quantized inside {f_us:.1f} us")
            result["fp8"]["per_config"] = fp8_long
            del k8h, ksh, v8h, vsh
        del b_q, b_k, b_v, b_o, b_l, g_do, b_dq, b_dk, b_dv, b_ws
        torch.cuda.empty_cache()

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
        st, lead_v = time_calls(lambda: binding.fa_decode_multi(v_q, v_kc, v_vc, v_bt, v_sl, cv.scale, out=v_o,
                                                                   lse=v_l, workspace=v_ws),
                                   max(5, min(K, 20)), True, 0.4)
        vbytes = metrics.decode_kv_bytes(cv.seqlens, vshp["Hkv"], vshp["d"])
        gbs_v = vbytes / (st["mean"] * 1e-3) / 1e9
        result["verify"] = {
            "workload": VERIFY, "kernels": "mq_partial_kernel<4> + mq_combine_kernel<4>", "bound": "hbm",
            "achieved": round(gbs_v, 1), "peak": peak_gb, "unit": "GB/s", "frac": round(gbs_v / peak_gb, 4),
            "traffic": profiling.current_profile(PROFILES[VERIFY])["traffic"],
            "algorithmic_kv_bytes_per_launch": vbytes, "kv_tokens": cv.kv_tokens,
            "flops_per_launch": metrics.decode_flops(cv.seqlens, vshp["Hq"], vshp["d"]) * vshp["Sq"],
            "launch_us": us(st),
            "note": "caches flushed (512 MiB read) before each launch, outside its events",
            "host_lead": lead_v,
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
        st, lead_m = time_calls(lambda: binding.fa_mla_decode(m_q, m_wk, m_wv, m_cc, m_bt, m_sl, cm.scale, out=m_o,
                                                                 lse=m_l, workspace=m_ws),
                                   max(5, min(K, 20)), True, 0.4)
        lat_bytes = metrics.mla_latent_bytes(cm.cache.seqlens, msh["d_c"])
        gbs_m = lat_bytes / (st["mean"] * 1e-3) / 1e9
        result["mla"] = {
            "workload": MLA, "bound": "hbm",
            "kernels": "mla_absorb_kernel + mla_partial_kernel + mla_merge_upproj_kernel",
            "achieved": round(gbs_m, 1), "peak": peak_gb, "unit": "GB/s", "frac": round(gbs_m / peak_gb, 4),
            "traffic": profiling.current_profile(PROFILES[MLA])["traffic"],
            "algorithmic_latent_bytes_per_launch": lat_bytes,
            "min_bytes_per_launch": metrics.mla_total_bytes(cm.cache.seqlens, msh["H"], msh["d_h"], msh["d_c"]),
            "kv_tokens": cm.cache.kv_tokens,
            "flops_per_launch": metrics.mla_flops(cm.cache.seqlens, msh["H"], msh["d_h"], msh["d_c"]),
            "materialized_kv_bytes_equivalent": metrics.decode_kv_bytes(cm.cache.seqlens, msh["H"], msh["d_h"]),
            "launch_us": us(st),
            "note": "achieved = latent bytes over the whole call; caches flushed (512 MiB read) before each call, "
                    "outside its events",
            "host_lead": lead_m,
        }
        log(f"mla: {st['mean']*1e3:.1f} us -> {gbs_m:.0f} GB/s of latents")
        del m_q, m_wk, m_wv, m_cc, m_o, m_ws, cm
        torch.cuda.empty_cache()

    # ---- the fp64 oracle on the host: the same workloads ----
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(ch, cf, cd, metrics)

    print(json.dumps(result), flush=True)


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"), default=1)
    except Exception:  # threadpoolctl missing or no BLAS reported
        return os.cpu_count() or 1


def cpu_baseline(ch, cf, cd, metrics):
    """The fp64 oracle, as it stands, timed on the host with time.perf_counter.

    Top level: the 32k workload's checked rows (512 per head, plus the first
    and last row), per-row time and algorithmic TFLOP/s of those rows.
    ``per_config``: the fp32 workload (repeated to at least 0.5 s), the 2k and
    8k workloads in full (one pass, per head group) and the 64-sequence decode
    in full.  ``materialized`` rates count the work the oracle actually does
    (every (query, key) pair, 4 d FLOP each, masked ones included)."""
    import numpy as np

    import oracle
    from exact_tiled_attention_14_amd import inputs

    threads = int(_blas_threads())
    base = {"kind": "oracle", "cores": threads, "host_cpus": os.cpu_count(), "blas_threads": threads}
    per = {}

    # fp32 workload: tiny; repeated
    log("oracle: fp32 workload")
    reps, dt = 0, 0.0
    while dt < CPU_MIN_SECONDS:
        t0 = time.perf_counter()
        oracle.sdpa(cf.q, cf.k, cf.v, cf.causal, cf.scale)
        dt += time.perf_counter() - t0
        reps += 1
    s1 = cf.shape
    fl1 = metrics.prefill_flops(s1["B"], s1["Hq"], s1["Sq"], s1["Sk"], s1["d"], cf.causal)
    per[FP32] = {"value": round(fl1 * reps / dt / 1e12, 6), "unit": "TFLOP/s", "seconds_per_call": dt / reps,
                 "sample": f"the whole workload, {reps} calls"}

    # 2k and 8k prefills in full, 4 / 8 query heads per oracle call
    for name, hpc in ((PREFILL2K, 4), (PREFILL8K, 8)):
        log(f"oracle: {name} in full")
        c = inputs.workload(name)
        s = c.shape
        g = s["Hq"] // s["Hkv"]
        t0 = time.perf_counter()
        for b in range(s["B"]):
            for h0 in range(0, s["Hq"], hpc):
                oracle.sdpa(c.q[b:b + 1, h0:h0 + hpc], c.k[b:b + 1, h0 // g:(h0 + hpc) // g],
                            c.v[b:b + 1, h0 // g:(h0 + hpc) // g], True, c.scale)
        dt = time.perf_counter() - t0
        fl = metrics.prefill_flops(s["B"], s["Hq"], s["Sq"], s["Sk"], s["d"], True)
        mat = 4.0 * s["B"] * s["Hq"] * s["Sq"] * s["Sk"] * s["d"]
        per[name] = {"value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "seconds": round(dt, 2),
                     "materialized_TFLOP/s": round(mat / dt / 1e12, 6),
                     "sample": f"the whole workload, one pass, {hpc} query heads per oracle call"}
        log(f"oracle: {name} {dt:.1f} s")
        del c

    # decode in full
    log("oracle: decode workload in full")
    t0 = time.perf_counter()
    oracle.paged_decode(cd.q, cd.kcache, cd.vcache, cd.block_table, cd.seqlens, cd.scale)
    dt = time.perf_counter() - t0
    kv_bytes = metrics.decode_kv_bytes(cd.seqlens, cd.shape["Hkv"], cd.shape["d"])
    per[DECODE] = {"value": round(kv_bytes / dt / 1e9, 3), "unit": "GB/s", "seconds": round(dt, 2),
                   "sample": "all 64 sequences (pages gathered, one query row per head)"}

    # headline: the 32k workload's checked rows
    log("oracle: 32k workload, checked rows")
    s = ch.shape
    rows = np.concatenate([ch.rows, np.broadcast_to(np.array([0, s["Sq"] - 1]), (s["B"], s["Hq"], 2))], axis=2)
    g = s["Hq"] // s["Hkv"]
    t0 = time.perf_counter()
    for h0 in range(0, s["Hq"], g):
        oracle.sdpa_rows(ch.q[:, h0:h0 + g], ch.k[:, h0 // g:h0 // g + 1], ch.v[:, h0 // g:h0 // g + 1],
                         rows[:, h0:h0 + g], True, ch.scale)
    dt = time.perf_counter() - t0
    n_rows = rows.size
    fl = float(4 * s["d"] * (rows.astype(np.int64) + 1 + (s["Sk"] - s["Sq"])).sum())   # visible pairs of those rows
    mat = 4.0 * s["d"] * s["Sk"] * n_rows
    out = dict(base)
    out.update({
        "value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s",
        "sample": f"{HEADLINE}: {rows.shape[2]} checked rows in each of the {s['Hq']} heads ({n_rows} rows), "
                  f"one oracle call per K/V head group; algorithmic causal FLOPs of those rows over the oracle time",
        "seconds": round(dt, 2), "ms_per_row": round(dt / n_rows * 1e3, 4),
        "materialized_TFLOP/s": round(mat / dt / 1e12, 6),
        "per_config": per,
    })
    log(f"oracle: 32k rows {dt:.1f} s")
    return out



if __name__ == "__main__":
    main()
