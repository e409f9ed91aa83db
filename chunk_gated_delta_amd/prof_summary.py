"""Turn rocprofv3 CSV output into the short text summaries kept with the project.

    python -m chunk_gated_delta_amd.prof_summary stats KERNEL_STATS_CSV --title T --command C [--bench-json J]
                                                   [--trace KERNEL_TRACE_CSV] --out F
    python -m chunk_gated_delta_amd.prof_summary traffic FETCH_CSV WRITE_CSV --copy-mib N --title T
                                                   --command-fetch C1 --command-write C2 --out F

    python -m chunk_gated_delta_amd.prof_summary mfma COUNTER_CSV --stats-csv KERNEL_STATS_CSV --simds N
                                                   --title T --command C --command-stats C2 --out F
    python -m chunk_gated_delta_amd.prof_summary lds COUNTER_CSV --title T --command C --out F

`stats` tabulates a --kernel-trace --stats run.  `mfma` takes one --pmc run of the MFMA
counters (SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE, the derived MfmaUtil, and the
bf16 / fp32 MFMA op counts SQ_INSTS_VALU_MFMA_MOPS_*, each 512 flops) and the kernel
statistics of a trace run of the same program, and writes per kernel the fraction of
SIMD cycles the matrix cores were busy and the MFMA flops per launch and per second,
again with a machine-readable line for bench.py.  `traffic` takes one --pmc FETCH_SIZE
run and one --pmc WRITE_SIZE run of `python -m chunk_gated_delta_amd.profile_step
--copy-mib N` and scales each counter (KiB per dispatch) by what it reads for the
reference kernel, which reads N MiB and writes N MiB; the per-kernel HBM bytes per
launch are also written as a machine-readable line (with the digest of the kernel
sources they were measured on) that bench.py reports while the sources are unchanged.
"""
import argparse
import csv
import json
import statistics
import sys

TRAFFIC_TAG = "<!-- hbm-traffic: "
MFMA_TAG = "<!-- mfma: "


def short_name(mangled):
    for key in ("bwd_chunk_kernel", "bwd_state_kernel", "fwd_prep_kernel", "fwd_state_kernel",
                "fwd_content_kernel", "fwd_affine_kernel", "seg_scan_kernel", "decode_kernel",
                "content_gate_bwd_kernel", "content_gates_kernel", "add_grad_mean_kernel",
                "init_grad_mean_kernel", "sum_over_batch_kernel", "logit_grads_kernel", "sum_heads_kernel",
                "copy_or_zero_kernel", "stream_copy_kernel"):
        if key in mangled:
            return key
    return mangled[:48]


def stats(args):
    rows = list(csv.DictReader(open(args.csv)))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    out = [f"# {args.title}", "", "Command (from /tmp with TMPDIR=/tmp; repository at $R, PYTHONPATH=$R):", "",
           "    " + args.command, "", "Durations in microseconds (rocprofv3 kernel statistics).", "",
           "| kernel | mangled name | calls | average us | min us | max us | share % |", "|---|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        out.append(f"| {short_name(r['Name'])} | `{r['Name'][:90]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {100 * float(r['TotalDurationNs']) / total:.1f} |")
    if args.trace:
        # the same kernel can run at several launch shapes (the training step's chunk-gradient
        # launch covers every chunk, the content-aware backward's one chunk per head): split
        # the trace by (kernel, grid) so each shape's average stands on its own
        groups = {}
        for r in csv.DictReader(open(args.trace)):
            key = (r["Kernel_Name"], int(r["Grid_Size_X"]), int(r["Grid_Size_Y"]), int(r["Workgroup_Size_X"]))
            groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        gtot = sum(sum(v) for v in groups.values())
        out += ["", "Per launch shape (the same run's kernel trace; workgroups = grid / workgroup size):", "",
                "| kernel | workgroups (x, y) | threads | calls | average us | min us | max us | share % |",
                "|---|---|---|---|---|---|---|---|"]
        for (name, gx, gy, wx), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            if 100 * sum(d) / gtot < 0.1:
                continue
            out.append(f"| {short_name(name)} | ({gx // max(wx, 1)}, {gy}) | {wx} | {len(d)} | "
                       f"{statistics.mean(d):.1f} | {min(d):.1f} | {max(d):.1f} | {100 * sum(d) / gtot:.1f} |")
    if args.bench_json:
        line = [ln for ln in open(args.bench_json) if ln.startswith("{")][-1]
        b = json.loads(line)
        out += ["", "The same run's bench line (HIP events on the launch stream, mean per launch):", ""]
        for k_, v_ in b["extra"]["stage_ms"].items():
            out.append(f"* {k_}: {1e3 * v_:.1f} us")
        out.append(f"* step: {1e3 * b['ms_per_step']:.1f} us; roofline kernel {b['roofline']['kernel']}, "
                   f"launch {1e3 * b['roofline']['launch_ms']:.1f} us")
    open(args.out, "w").write("\n".join(out) + "\n")


def _per_kernel(path, counter):
    vals = {}
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != counter:
            continue
        vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return vals


def traffic(args):
    from chunk_gated_delta_amd.build import source_digest
    fetch = _per_kernel(args.fetch_csv, "FETCH_SIZE")
    write = _per_kernel(args.write_csv, "WRITE_SIZE")
    ref_kib = args.copy_mib * 1024.0
    # reference kernel: the dispatches that read (torch.neg); the fill that precedes them reads nothing
    ref_f = [v for k_, vs in fetch.items() if "carve" not in k_ for v in vs if v > 0.25 * ref_kib]
    ref_w = [v for k_, vs in write.items() if "carve" not in k_ for v in vs if v > 0.25 * ref_kib]
    f_scale = ref_kib / statistics.median(ref_f)
    w_scale = ref_kib / statistics.median(ref_w)
    out = [f"# {args.title}", "", "Commands (from /tmp with TMPDIR=/tmp; repository at $R, PYTHONPATH=$R):", "",
           "    " + args.command_fetch, "    " + args.command_write, "",
           f"Reference kernel (torch.neg, {args.copy_mib} MiB read + {args.copy_mib} MiB written): FETCH_SIZE reads "
           f"{statistics.median(ref_f):.0f} KiB, WRITE_SIZE {statistics.median(ref_w):.0f} KiB per dispatch, so the "
           f"counters are scaled by {f_scale:.3f} (fetch) and {w_scale:.3f} (write).", "",
           "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM read MB | HBM written MB | total MB |",
           "|---|---|---|---|---|---|---|"]
    record = {"source_digest": source_digest(), "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4),
              "bytes_per_launch": {}}
    for name in fetch:
        if "carve" not in name:
            continue
        fk = statistics.median(fetch[name])
        wk = statistics.median(write.get(name, [0.0]))
        rd, wr = fk * f_scale * 1024, wk * w_scale * 1024
        out.append(f"| {short_name(name)} `{name[:70]}` | {len(fetch[name])} | {fk:.0f} | {wk:.0f} | "
                   f"{rd / 1e6:.1f} | {wr / 1e6:.1f} | {(rd + wr) / 1e6:.1f} |")
        record["bytes_per_launch"][short_name(name)] = {"read": round(rd), "write": round(wr)}
    out += ["", "Kernel sources digest at measurement: `" + record["source_digest"] + "`", "",
            TRAFFIC_TAG + json.dumps(record) + " -->"]
    open(args.out, "w").write("\n".join(out) + "\n")


def _counters(path):
    per = {}
    for r in csv.DictReader(open(path)):
        per.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return per


def mfma(args):
    from chunk_gated_delta_amd.build import source_digest
    per = _counters(args.csv)
    avg_ns = {r["Name"]: float(r["AverageNs"]) for r in csv.DictReader(open(args.stats_csv))}
    out = [f"# {args.title}", "", "Commands (from /tmp with TMPDIR=/tmp; repository at $R, PYTHONPATH=$R):", "",
           "    " + args.command, "    " + args.command_stats, "",
           "MFMA busy = the share of SIMD cycles in which the matrix core was busy during the dispatch "
           f"(rocprofv3's MfmaUtil: summed SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE x {args.simds} SIMDs; "
           f"the last column recomputes it from the raw counters, the CSV's GRBM_GUI_ACTIVE being the sum over "
           f"{args.xcc} XCDs). MFMA flops = "
           "SQ_INSTS_VALU_MFMA_MOPS_* x 512 per dispatch; TFLOP/s divides them by the kernel's average duration "
           "in the trace run. Medians over dispatches.", "",
           "| kernel | dispatches | average us | MFMA busy % | bf16 MFMA GFLOP | fp32 MFMA GFLOP | MFMA TFLOP/s | "
           "busy / (GUI x SIMDs) % |", "|---|---|---|---|---|---|---|---|"]
    record = {"source_digest": source_digest(), "simds": args.simds, "kernels": {}}
    for name, c in per.items():
        if "carve" not in name:
            continue
        med = {k_: statistics.median(v_) for k_, v_ in c.items()}
        n = max(len(v_) for v_ in c.values())
        util = med.get("MfmaUtil")
        raw = None
        if med.get("GRBM_GUI_ACTIVE"):
            # the CSV sums GRBM_GUI_ACTIVE over the XCDs, each of which counts the dispatch's cycles
            raw = med.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (med["GRBM_GUI_ACTIVE"] / args.xcc * args.simds)
        busy = util / 100.0 if util is not None else raw
        fb = med.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) * 512
        ff = med.get("SQ_INSTS_VALU_MFMA_MOPS_F32", 0.0) * 512
        ns = avg_ns.get(name)
        tf = (fb + ff) / (ns * 1e-9) / 1e12 if ns else None
        out.append(f"| {short_name(name)} | {n} | {ns / 1e3 if ns else float('nan'):.1f} | "
                   f"{100 * busy if busy is not None else float('nan'):.1f} | {fb / 1e9:.2f} | {ff / 1e9:.2f} | "
                   f"{tf if tf is not None else float('nan'):.1f} | {100 * raw if raw is not None else float('nan'):.1f} |")
        record["kernels"][short_name(name)] = {
            "busy_frac": None if busy is None else round(busy, 4), "bf16_flops": fb, "f32_flops": ff,
            "tflops": None if tf is None else round(tf, 2), "avg_us": None if not ns else round(ns / 1e3, 1)}
    out += ["", "Kernel sources digest at measurement: `" + record["source_digest"] + "`", "",
            MFMA_TAG + json.dumps(record) + " -->"]
    open(args.out, "w").write("\n".join(out) + "\n")


def lds(args):
    """LDS counters (SQ_INSTS_LDS, SQ_LDS_IDX_ACTIVE, SQ_LDS_BANK_CONFLICT) averaged per kernel."""
    from chunk_gated_delta_amd.build import source_digest
    per = _counters(args.csv)
    out = [f"# {args.title}", "", "Command (from /tmp with TMPDIR=/tmp; repository at $R, PYTHONPATH=$R):", "",
           "    " + args.command, "",
           "Counter values averaged over the dispatches of each kernel (cycles summed over the chip as the SQ "
           "counters report them).", "",
           "| kernel | dispatches | SQ_INSTS_LDS | SQ_LDS_IDX_ACTIVE | SQ_LDS_BANK_CONFLICT | conflict / active |",
           "|---|---|---|---|---|---|"]
    for name, c in per.items():
        if "carve" not in name:
            continue
        mean = {k_: statistics.mean(v_) for k_, v_ in c.items()}
        act = mean.get("SQ_LDS_IDX_ACTIVE", 0.0)
        con = mean.get("SQ_LDS_BANK_CONFLICT", 0.0)
        out.append(f"| {short_name(name)} `{name[:70]}` | {len(c.get('SQ_LDS_IDX_ACTIVE', []))} | "
                   f"{mean.get('SQ_INSTS_LDS', 0.0):.0f} | {act:.0f} | {con:.0f} | {con / act if act else 0.0:.2f} |")
    out += ["", "Kernel sources digest at measurement: `" + source_digest() + "`"]
    open(args.out, "w").write("\n".join(out) + "\n")


def _read_tagged(path, tag):
    try:
        for line in open(path):
            if line.startswith(tag):
                return json.loads(line[len(tag):].rsplit(" -->", 1)[0])
    except OSError:
        return None
    return None


def read_mfma(path):
    """The machine-readable record of an MFMA counter summary, or None."""
    return _read_tagged(path, MFMA_TAG)


def read_traffic(path):
    """The machine-readable record of a traffic summary, or None."""
    return _read_tagged(path, TRAFFIC_TAG)


def main(argv=None):
    p = argparse.ArgumentParser()
    sub = p.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--bench-json")
    s.add_argument("--trace", help="kernel trace CSV of the same run: adds per-launch-shape statistics")
    s.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("fetch_csv")
    t.add_argument("write_csv")
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--title", required=True)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    t.add_argument("--out", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("csv")
    m.add_argument("--stats-csv", required=True)
    m.add_argument("--simds", type=int, default=1024, help="SIMDs of the device (compute units x 4)")
    m.add_argument("--xcc", type=int, default=8, help="XCDs of the device")
    m.add_argument("--title", required=True)
    m.add_argument("--command", required=True)
    m.add_argument("--command-stats", required=True)
    m.add_argument("--out", required=True)
    d = sub.add_parser("lds")
    d.add_argument("csv")
    d.add_argument("--title", required=True)
    d.add_argument("--command", required=True)
    d.add_argument("--out", required=True)
    a = p.parse_args(argv)
    {"stats": stats, "traffic": traffic, "mfma": mfma, "lds": lds}[a.cmd](a)
    return 0


if __name__ == "__main__":
    sys.exit(main())
