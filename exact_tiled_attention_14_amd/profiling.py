"""Driver and summariser for the rocprofv3 runs whose summaries live in profiles/.

`run` launches one workload a few times through the C ABI, each launch
followed by a device synchronisation, and then a plain device-to-device copy
of a known size.  Under `rocprofv3 --pmc FETCH_SIZE` (or `WRITE_SIZE`) the
copy is the calibration: the counter's reading for it, divided into the bytes
it must move, is the factor applied to the attention kernels' readings.

`summarize` turns rocprofv3 CSV output (kernel stats, and optionally the
FETCH_SIZE / WRITE_SIZE and MFMA counter passes) into a short markdown file.
Its last section holds `key: value` lines that bench.py reads back: the HBM
bytes per launch of a kernel, valid only while the sha256 of the kernel's
source file is unchanged.

Examples (from the repository root):

    python -m exact_tiled_attention_14_amd.profiling run --workload prefill --reps 5
    python -m exact_tiled_attention_14_amd.profiling summarize --stats DIR/p_kernel_stats.csv \\
        --fetch DIR_F/p_counter_collection.csv --write DIR_W/p_counter_collection.csv \\
        --kernel fwd_bf16_kernel --source exact_tiled_attention_14_amd/csrc/fwd_bf16.hip \\
        --title "..." --command "..." --out profiles/NAME.md
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import math
import os
import re
import sys
from collections import defaultdict

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

COPY_KERNEL_HINT = "copyBuffer|elementwise|copy|fill"   # what the plain copy (and its source fill) show up as
PREFILL = "causal_mha_b2_h16_s2048_d128"
DECODE = "paged_decode_64seq_h32kv8_d128"
VERIFY = "paged_verify_64seq_q8_h32kv8_d128"
MLA = "mla_decode_64seq_h16_dc512"
GQA8K = "causal_gqa_h32kv8_s8192_d128_outliers"
GQA32K = "causal_gqa_h32kv8_s32768_d128"


def source_sha256(path: str) -> str:
    with open(os.path.join(ROOT, path) if not os.path.isabs(path) else path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


# --------------------------------------------------------------------------- run

def _run(args) -> None:
    import numpy as np
    import torch

    from . import binding, inputs

    if not torch.cuda.is_available():
        sys.exit("no GPU visible")
    dev = torch.device("cuda:0")
    binding.load()

    def to_dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    launches = []
    if args.workload in ("prefill", "all"):
        c = inputs.workload(PREFILL)
        q, k, v = to_dev(c.bits("q")), to_dev(c.bits("k")), to_dev(c.bits("v"))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        launches.append(("prefill", lambda: binding.fa_fwd(q, k, v, True, c.scale, out=o, lse=lse)))
    for wl, name in (("gqa8k", GQA8K), ("gqa32k", GQA32K)):
        # long-sequence GQA prefills: run on their own (same kernel as the headline prefill)
        if args.workload == wl:
            c = inputs.workload(name)
            gq, gk, gv = to_dev(c.bits("q")), to_dev(c.bits("k")), to_dev(c.bits("v"))
            go = torch.empty_like(gq)
            gl = torch.empty(gq.shape[:3], dtype=torch.float32, device=dev)
            launches.append((wl, lambda: binding.fa_fwd(gq, gk, gv, True, c.scale, out=go, lse=gl)))
    for wl, name in (("fp8_8k", GQA8K), ("fp8_32k", GQA32K)):
        # the FP8 forward on the same long workloads (codes of rotated Q and K, and V, quantized once)
        if args.workload == wl:
            c = inputs.workload(name)
            gq, gk, gv = to_dev(c.bits("q")), to_dev(c.bits("k")), to_dev(c.bits("v"))
            rot = to_dev(inputs.bf16_bits(inputs.make_rotation(c.q.shape[-1], seed=2)))
            q8l, qsl, k8l, ksl, v8l, vsl = binding.fa_quantize_fp8_qkv(gq, gk, gv, rot=rot)
            del gk, gv
            go = torch.empty_like(gq)
            gl = torch.empty(gq.shape[:3], dtype=torch.float32, device=dev)
            torch.cuda.synchronize()
            launches.append((wl, lambda: binding.fa_fwd_fp8(q8l, qsl, k8l, ksl, v8l, vsl, True, c.scale, out=go,
                                                            lse=gl)))
    if args.workload in ("backward", "all"):
        c = inputs.workload(PREFILL)
        bq, bk, bv = to_dev(c.bits("q")), to_dev(c.bits("k")), to_dev(c.bits("v"))
        bo = torch.empty_like(bq)
        bl = torch.empty(bq.shape[:3], dtype=torch.float32, device=dev)
        binding.fa_fwd(bq, bk, bv, True, c.scale, out=bo, lse=bl)
        bg = to_dev(inputs.bf16_bits(inputs.make_grad_out(c.q.shape, seed=2)))
        grads = (torch.empty_like(bq), torch.empty_like(bk), torch.empty_like(bv))
        bws = torch.empty(binding.fa_bwd_workspace_size(*bq.shape[:3]), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        launches.append(("backward", lambda: binding.fa_bwd(bq, bk, bv, bo, bg, bl, True, c.scale, dq=grads[0],
                                                            dk=grads[1], dv=grads[2], workspace=bws)))
    if args.workload in ("fp8", "all"):
        c = inputs.workload(PREFILL)
        fq, fk, fv = to_dev(c.bits("q")), to_dev(c.bits("k")), to_dev(c.bits("v"))
        rot = to_dev(inputs.bf16_bits(inputs.make_rotation(c.q.shape[-1], seed=2)))
        q8, qs, k8, ks, v8, vs = binding.fa_quantize_fp8_qkv(fq, fk, fv, rot=rot)
        fo = torch.empty_like(fq)
        fl = torch.empty(fq.shape[:3], dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        launches.append(("fp8_quantize_qkv", lambda: binding.fa_quantize_fp8_qkv(fq, fk, fv, rot=rot)))
        launches.append(("fp8_forward", lambda: binding.fa_fwd_fp8(q8, qs, k8, ks, v8, vs, True, c.scale, out=fo,
                                                                   lse=fl)))
        launches.append(("fp8_forward_qbf16", lambda: binding.fa_fwd_fp8_qbf16(fq, k8, ks, v8, vs, True, rot=rot,
                                                                               scale=c.scale, out=fo, lse=fl)))
    if args.workload in ("verify", "all"):
        cv = inputs.workload(VERIFY)
        vsh = cv.shape
        vq, vkc, vvc = to_dev(cv.bits("q")), to_dev(cv.kcache_bits), to_dev(cv.vcache_bits)
        vbt = torch.from_numpy(cv.block_table).to(dev)
        vsl = torch.from_numpy(cv.seqlens).to(dev)
        vo = torch.empty_like(vq)
        vl = torch.empty((vsh["nseq"], vsh["Sq"], vsh["Hq"]), dtype=torch.float32, device=dev)
        vws = torch.empty(binding.fa_decode_multi_workspace_size(vsh["nseq"], vsh["Sq"], vsh["Hq"], vsh["Hkv"], vsh["d"],
                                                                 vsh["block_size"], vsh["max_blocks"]),
                          dtype=torch.uint8, device=dev)
        launches.append(("verify", lambda: binding.fa_decode_multi(vq, vkc, vvc, vbt, vsl, cv.scale, out=vo, lse=vl,
                                                                   workspace=vws)))
    if args.workload in ("mla", "all"):
        cm = inputs.workload(MLA)
        msh = cm.shape
        mq, mwk, mwv = (to_dev(inputs.bf16_bits(x)) for x in (cm.q, cm.w_uk, cm.w_uv_t))
        mcc = to_dev(cm.ccache_bits)
        mbt = torch.from_numpy(cm.cache.block_table).to(dev)
        msl = torch.from_numpy(cm.cache.seqlens).to(dev)
        mo = torch.empty_like(mq)
        ml = torch.empty((msh["nseq"], msh["H"]), dtype=torch.float32, device=dev)
        mws = torch.empty(binding.fa_mla_decode_workspace_size(msh["nseq"], msh["H"], msh["d_h"], msh["d_c"],
                                                               msh["block_size"], msh["max_blocks"]),
                          dtype=torch.uint8, device=dev)
        launches.append(("mla", lambda: binding.fa_mla_decode(mq, mwk, mwv, mcc, mbt, msl, cm.scale, out=mo, lse=ml,
                                                              workspace=mws)))
    if args.workload in ("decode", "all"):
        d = inputs.workload(DECODE)
        s = d.shape
        dq, kc, vc = to_dev(d.bits("q")), to_dev(d.kcache_bits), to_dev(d.vcache_bits)
        bt = torch.from_numpy(d.block_table).to(dev)
        sl = torch.from_numpy(d.seqlens).to(dev)
        do = torch.empty_like(dq)
        dl = torch.empty((s["nseq"], s["Hq"]), dtype=torch.float32, device=dev)
        ws = torch.empty(binding.fa_decode_workspace_size(s["nseq"], s["Hq"], s["Hkv"], s["d"], s["block_size"],
                                                          s["max_blocks"]), dtype=torch.uint8, device=dev)
        launches.append(("decode", lambda: binding.fa_decode(dq, kc, vc, bt, sl, d.scale, out=do, lse=dl,
                                                             workspace=ws)))
    for name, fn in launches:
        for i in range(args.reps):
            fn()
            torch.cuda.synchronize()
        print(f"{name}: {args.reps} launches done", flush=True)
    if args.copy_mib > 0:
        n = args.copy_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(args.reps):
            dst.copy_(src)
            torch.cuda.synchronize()
        print(f"copy: {args.reps} x {args.copy_mib} MiB done", flush=True)


# --------------------------------------------------------------------- summarize

def _read_stats(path):
    rows = list(csv.DictReader(open(path)))
    return [{"name": r["Name"], "calls": int(r["Calls"]), "avg_us": float(r["AverageNs"]) / 1e3,
             "min_us": float(r["MinNs"]) / 1e3, "max_us": float(r["MaxNs"]) / 1e3,
             "pct": float(r["Percentage"])} for r in rows]


def _read_counters(path):
    """Per dispatch: {dispatch_id: (kernel name, {counter: value})}."""
    out = {}
    for r in csv.DictReader(open(path)):
        did = int(r["Dispatch_Id"])
        name, vals = out.setdefault(did, (r["Kernel_Name"], {}))
        vals[r["Counter_Name"]] = vals.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def _mean_counter(disp, pattern, counter, at_least=None):
    xs = [v[counter] for (name, v) in disp.values() if re.search(pattern, name) and counter in v
          and (at_least is None or v[counter] >= at_least)]
    return (sum(xs) / len(xs), len(xs)) if xs else (None, 0)


def _summarize(args) -> None:
    stats = _read_stats(args.stats)
    lines = [f"# {args.title}", "", "Command (from the repository root, one MI355X):", "", "```", args.command, "```", ""]
    if args.note:
        lines += [args.note, ""]
    lines += ["| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{r['name'][:90]}` | {r['calls']} | {r['avg_us']:.2f} | {r['min_us']:.2f} | "
                     f"{r['max_us']:.2f} | {r['pct']:.2f} |")
    lines.append("")
    kv = {}
    sel = [r for r in stats if re.search(args.kernel, r["name"])]
    if args.trace and args.min_us is not None:
        # one kernel serving two calls of different size: keep the longer dispatches
        durs = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in csv.DictReader(open(args.trace))
                if re.search(args.kernel, r["Kernel_Name"])]
        kept = [d for d in durs if d >= args.min_us]
        if kept:
            kv["kernel_avg_us"] = f"{sum(kept) / len(kept):.3f}"
            lines += [f"`kernel_avg_us` below averages the {len(kept)} dispatches of `{args.kernel}` that took at "
                      f"least {args.min_us:g} us (of {len(durs)} in the trace).", ""]
    elif sel:
        kv["kernel_avg_us"] = f"{sum(r['avg_us'] * r['calls'] for r in sel) / sum(r['calls'] for r in sel):.3f}"
    counter_rows = []
    for label, path, counter in (("read", args.fetch, "FETCH_SIZE"), ("written", args.write, "WRITE_SIZE")):
        if not path:
            continue
        disp = _read_counters(path)
        k_kib, k_n = _mean_counter(disp, args.kernel, counter)
        # the calibration dispatches: copy-like kernels that moved at least half
        # the copy's size (input uploads and small fills are excluded)
        c_kib, c_n = _mean_counter(disp, COPY_KERNEL_HINT, counter, at_least=args.copy_mib * 1024 / 2)
        if k_kib is None or c_kib is None or c_kib <= 0:
            continue
        factor = (args.copy_mib * 1024.0) / c_kib       # copy moves copy_mib MiB each way
        k_bytes = k_kib * 1024.0 * factor
        counter_rows.append(f"| {counter} | {k_kib:.0f} KiB ({k_n} dispatches) | {c_kib:.0f} KiB | "
                            f"{factor:.4f} | {k_bytes / 1e6:.2f} MB |")
        kv[f"hbm_bytes_{label}_per_launch"] = f"{k_bytes:.0f}"
        kv[f"{counter.lower()}_calibration_factor"] = f"{factor:.5f}"
    if counter_rows:
        lines += [f"HBM traffic of `{args.kernel}` per launch.  Each counter pass also profiles a plain "
                  f"{args.copy_mib} MiB device copy; the copy must read and write exactly that much, so "
                  f"its reading gives the scale factor.", "",
                  "| counter | kernel, mean per dispatch | copy, mean | factor | kernel bytes per launch |",
                  "|---|---|---|---|---|"] + counter_rows + [""]
        if "hbm_bytes_read_per_launch" in kv and "hbm_bytes_written_per_launch" in kv:
            kv["hbm_bytes_per_launch"] = f"{float(kv['hbm_bytes_read_per_launch']) + float(kv['hbm_bytes_written_per_launch']):.0f}"
    if args.mfma:
        disp = _read_counters(args.mfma)
        busy, n = _mean_counter(disp, args.kernel, "SQ_VALU_MFMA_BUSY_CYCLES")
        gui, _ = _mean_counter(disp, args.kernel, "GRBM_GUI_ACTIVE")
        insts, _ = _mean_counter(disp, args.kernel, "SQ_INSTS_MFMA")
        if busy is not None and gui:
            simds = args.cus * 4
            cycles = gui / args.xcds          # GRBM_GUI_ACTIVE is summed over the XCDs
            frac = busy / (cycles * simds)
            lines += [f"MFMA counters of `{args.kernel}` (mean of {n} dispatches): SQ_VALU_MFMA_BUSY_CYCLES "
                      f"{busy:.4g}, GRBM_GUI_ACTIVE {gui:.4g} (summed over {args.xcds} XCDs: {cycles:.4g} cycles), "
                      f"SQ_INSTS_MFMA {insts:.4g}.  Busy fraction = MFMA busy cycles / (active cycles x {simds} "
                      f"SIMDs) = {frac:.3f}.", ""]
            kv["mfma_busy_fraction"] = f"{frac:.4f}"
            kv["gui_active_cycles_per_xcd"] = f"{cycles:.0f}"
    if args.source:
        kv["source"] = args.source
        kv["source_sha256"] = source_sha256(args.source)
    kv["kernel"] = args.kernel
    lines += ["## values read by bench.py", "", "```"] + [f"{k}: {v}" for k, v in kv.items()] + ["```", ""]
    os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
    with open(args.out, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {args.out}")


def read_profile_values(path: str) -> dict:
    """The `key: value` block at the end of a summary written by `summarize`."""
    vals, inside = {}, False
    try:
        with open(path) as f:
            for ln in f:
                if ln.startswith("## values read by bench.py"):
                    inside = True
                elif inside and ":" in ln and not ln.startswith("```"):
                    k, v = ln.split(":", 1)
                    vals[k.strip()] = v.strip()
    except OSError:
        return {}
    return vals


def current_profile(path: str) -> dict:
    """The figures of a summary that still describe the current kernel source:
    ``traffic`` (HBM bytes per launch), ``mfma_busy`` (busy fraction),
    ``kernel_avg_us`` (rocprofv3's mean duration) and ``active_cycles``
    (GRBM_GUI_ACTIVE per XCD per launch), each None when missing or when the
    kernel source has changed since the profile was taken."""
    vals = read_profile_values(path)
    out = {"traffic": None, "mfma_busy": None, "kernel_avg_us": None, "active_cycles": None,
           "profile": os.path.relpath(path, ROOT)}
    try:
        fresh = "source" in vals and source_sha256(vals["source"]) == vals.get("source_sha256")
    except OSError:
        fresh = False
    if not fresh:
        return out
    for key, name in (("hbm_bytes_per_launch", "traffic"), ("mfma_busy_fraction", "mfma_busy"),
                      ("kernel_avg_us", "kernel_avg_us"), ("gui_active_cycles_per_xcd", "active_cycles")):
        if key in vals:
            out[name] = float(vals[key])
    return out


def current_traffic(path: str):
    """HBM bytes per launch from a summary, or None when it is missing or its
    kernel source has changed since the counters were taken."""
    vals = read_profile_values(path)
    if "hbm_bytes_per_launch" not in vals or "source" not in vals:
        return None
    try:
        if source_sha256(vals["source"]) != vals.get("source_sha256"):
            return None
    except OSError:
        return None
    return float(vals["hbm_bytes_per_launch"])


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--workload", choices=["prefill", "decode", "backward", "fp8", "verify", "mla", "gqa8k", "gqa32k",
                                          "fp8_8k", "fp8_32k", "all"], default="all")
    r.add_argument("--reps", type=int, default=5)
    r.add_argument("--copy-mib", type=int, default=1024)
    s = sub.add_parser("summarize")
    s.add_argument("--stats", required=True)
    s.add_argument("--fetch")
    s.add_argument("--write")
    s.add_argument("--mfma")
    s.add_argument("--kernel", required=True, help="regex selecting the kernel of interest")
    s.add_argument("--source", help="kernel source file whose hash the traffic figure is tied to")
    s.add_argument("--copy-mib", type=int, default=1024)
    s.add_argument("--cus", type=int, default=256)
    s.add_argument("--xcds", type=int, default=8)
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--note", default="")
    s.add_argument("--out", required=True)
    s.add_argument("--trace", help="kernel trace CSV; with --min-us, kernel_avg_us averages only the matching "
                                   "dispatches of at least that duration")
    s.add_argument("--min-us", type=float, default=None)
    a = ap.parse_args(argv)
    if a.cmd == "run":
        _run(a)
    else:
        _summarize(a)


if __name__ == "__main__":
    main()
