"""Benchmark of the CARVE key-axis gated delta rule on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--pass fwd+bwd|fwd] [--no-cpu-baseline]

One step = one pass of the hot path over one batch of the 1.3B-head-shape
workload (B4 H16 T4096 d128 L64, bf16 q/k/v, fp32 gates and state): the
token-only training forward (chunk prep + state pass, keeping the chunk factors
and chunk-entry states for the backward) followed by the backward (reverse
state pass, chunk gradients).  Inputs are synthetic and seeded, already
resident in HBM when the timed region starts.  Prints ONE JSON line.  The plain
(inference) forward and the content-aware forward of the same shape are timed
separately and reported under "extra".

Roofline: every stage is bracketed with HIP events on the stream it runs on
(carve_fwd_ex / carve_bwd_ex) inside the timed region; the stage with the
largest mean duration is the dominant kernel, and its achieved bandwidth is
its algorithmic bytes (inputs it must read plus outputs it must write, per
token-head, times the token-heads of one launch) over that mean duration.
That figure is set against the published 8 TB/s and against the copy bandwidth
measured in the same run (the library's streaming copy kernel and torch's copy
over 1 GiB); the MFMA-busy fraction and MFMA flop rate of the dominant kernel
come from the committed rocprofv3 counter summary while the kernel sources are
unchanged since it was taken.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--pass", dest="passes", default="fwd+bwd", choices=["fwd+bwd", "fwd"])
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-heads", type=int, default=64,
                   help="(batch, head) sequences of the workload the CPU oracle runs (full length)")
    p.add_argument("--no-content", action="store_true")
    p.add_argument("--no-long", action="store_true", help="skip the long-context forward")
    p.add_argument("--no-decode", action="store_true", help="skip the recurrent decode step")
    p.add_argument("--no-logits", action="store_true", help="skip the gate pre-activation entry points")
    return p.parse_args()


def hbm_frac(bytes_per_token_head, wl, ms, extra_bytes=0):
    """Algorithmic bytes of a whole call (per token-head figure x B*H*T, plus fixed extras such
    as S_T) over its time, as a fraction of the HBM peak."""
    total = bytes_per_token_head * wl.B * wl.H * wl.T + extra_bytes
    return round(total / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)


def algorithmic(wl, with_bwd):
    """Algorithmic bytes and flops per token-head (inputs read once, outputs written once;
    triangle-aware flop count, 2 per multiply-add)."""
    d, L = wl.Dk, wl.L
    es = 2 if wl.dtype == "bf16" else 4
    gates = 4 * d * (2 if wl.erase in ("sigmoid", "ones") else 1) + 4       # log_g (+ b) + w
    fwd_in = 3 * es * d + gates                                                # q, k, v, gates
    fwd_out = es * d                                                           # o
    flops_fwd = 2 * ((L - 1) / 2 * (2 * d + d) + (L + 1) / 2 * (d + d) + 3 * d * d + L * L / 6)
    out = {"fwd_in": fwd_in, "fwd_out": fwd_out, "fwd": fwd_in + fwd_out, "flops_fwd": flops_fwd}
    if with_bwd:
        bwd_in = fwd_in + es * d                                               # inputs again + dO
        bwd_out = 3 * es * d + gates                                           # dq dk dv + dlog_g (+ db) + dw
        out.update(bwd_in=bwd_in, bwd_out=bwd_out, bwd=bwd_in + bwd_out, flops_bwd=2 * flops_fwd)
    return out


TRAFFIC_SUMMARY = os.path.join(HERE, "profiles", "head1p3b_fwd_bwd_hbm_traffic.md")
MFMA_SUMMARY = os.path.join(HERE, "profiles", "head1p3b_fwd_bwd_mfma.md")
STAGE_KERNEL = {"fwd_prep": "fwd_prep_kernel", "fwd_state": "fwd_state_kernel",
                "bwd_state_rev": "bwd_state_kernel", "bwd_chunk_grads": "bwd_chunk_kernel"}


def measured_traffic(stage):
    """HBM bytes per launch of a training-step kernel from the committed rocprofv3 counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by a reference copy kernel), or None when
    the kernel sources changed after the counters were taken."""
    from chunk_gated_delta_amd.build import source_digest
    from chunk_gated_delta_amd.prof_summary import read_traffic
    rec = read_traffic(TRAFFIC_SUMMARY)
    if not rec or rec.get("source_digest") != source_digest():
        return None
    b = rec["bytes_per_launch"].get(STAGE_KERNEL.get(stage, ""))
    return None if b is None else int(b["read"] + b["write"])


def measured_mfma(stage):
    """MFMA-busy fraction and MFMA flops of a training-step kernel from the committed rocprofv3
    counter summary, or None when the kernel sources changed after the counters were taken."""
    from chunk_gated_delta_amd.build import source_digest
    from chunk_gated_delta_amd.prof_summary import read_mfma
    rec = read_mfma(MFMA_SUMMARY)
    if not rec or rec.get("source_digest") != source_digest():
        return None
    return rec["kernels"].get(STAGE_KERNEL.get(stage, ""))


def copy_bandwidth(dev, mib=1024, nrep=10):
    """Achievable device copy bandwidth (GB/s, bytes read + written over time), measured live
    with the library's streaming copy kernel and with torch's copy on a `mib` MiB buffer."""
    import torch
    from chunk_gated_delta_amd import carve
    src = torch.empty(mib << 18, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    nbytes = 2 * src.numel() * 4
    out = {}
    for name, fn in (("stream_copy", lambda: carve.stream_copy(dst, src)), ("torch_copy", lambda: dst.copy_(src))):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(nrep):
            fn()
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(nbytes / (e0.elapsed_time(e1) / nrep * 1e-3) / 1e9, 1)
    del src, dst
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the CARVE kernels run on a single MI355X "
              f"(--gpus {args.gpus} is not supported; (batch, head) sequences are independent, so they "
              f"would shard across GPUs with no communication).", file=sys.stderr)
        sys.exit(2)

    import torch
    from chunk_gated_delta_amd import carve
    from chunk_gated_delta_amd.synth import WORKLOADS, make_inputs

    wl = WORKLOADS["head1p3b_fwd"]
    with_bwd = args.passes == "fwd+bwd"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = make_inputs(wl, with_dO=True)

    def t_bf16(key):
        return torch.from_numpy(np.ascontiguousarray(inp[key + "_bits"]).view(np.int16)).to(dev).view(torch.bfloat16)

    def t_f32(key):
        return torch.from_numpy(np.ascontiguousarray(inp[key], dtype=np.float32)).to(dev)

    q, k, v, dO = t_bf16("q"), t_bf16("k"), t_bf16("v"), t_bf16("dO")
    log_g, b, w = t_f32("log_g"), t_f32("b"), t_f32("w")
    B, H, T, D = wl.B, wl.H, wl.T, wl.Dk
    o = torch.empty_like(v)
    S_T = torch.empty((B, H, D, D), dtype=torch.float32, device=dev)
    ws_f = torch.empty(max(1, carve.fwd_workspace_bytes(q, v, wl.L)), dtype=torch.uint8, device=dev)
    lib = carve.load_library()
    shape = carve.make_shape(q, v, wl.L)
    import ctypes
    saved = torch.empty(max(1, lib.carve_saved_size(ctypes.byref(shape))), dtype=torch.uint8, device=dev)
    ws_b = torch.empty(max(1, lib.carve_bwd_saved_workspace_size(ctypes.byref(shape))), dtype=torch.uint8,
                       device=dev)
    grads = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
             "dlog_g": torch.empty_like(log_g), "db": torch.empty_like(b), "dw": torch.empty_like(w), "dS0": None}

    fwd_names = ["fwd_prep", "fwd_state"]
    bwd_names = ["bwd_state_rev", "bwd_chunk_grads"]

    def new_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        for e in evs:
            e.record()          # materialise the underlying hipEvent_t
        return evs

    def step(fe, be):
        if with_bwd:
            carve.fwd_save(q, k, v, log_g, w, b=b, L=wl.L, o=o, S_T=S_T, saved=saved,
                           profile=carve.make_profile(fe) if fe is not None else None)
            carve.bwd_saved(q, k, v, log_g, w, dO, saved, b=b, L=wl.L, want_dS0=False, workspace=ws_b, out=grads,
                            profile=carve.make_profile(be) if be is not None else None)
        else:
            carve.fwd(q, k, v, log_g, w, b=b, L=wl.L, o=o, S_T=S_T, workspace=ws_f,
                      profile=carve.make_profile(fe) if fe is not None else None)

    for _ in range(args.warmup):
        step(None, None)
    torch.cuda.synchronize()

    stage_evs = [(new_events(len(fwd_names)), new_events(len(bwd_names)) if with_bwd else None)
                 for _ in range(args.steps)]
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        step(*stage_evs[i])
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / args.steps

    stage_ms = {}
    for fe, be in stage_evs:
        for j, name in enumerate(fwd_names):
            stage_ms.setdefault(name, []).append(fe[j].elapsed_time(fe[j + 1]))
        if be is not None:
            for j, name in enumerate(bwd_names):
                stage_ms.setdefault(name, []).append(be[j].elapsed_time(be[j + 1]))
    stage_mean = {k_: float(np.mean(v_)) for k_, v_ in stage_ms.items()}

    # plain (inference) forward: the fwd part of the metric
    pf = [new_events(len(fwd_names)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    f0.record()
    for i in range(args.steps):
        carve.fwd(q, k, v, log_g, w, b=b, L=wl.L, o=o, S_T=S_T, workspace=ws_f, profile=carve.make_profile(pf[i]))
    f1.record()
    torch.cuda.synchronize()
    fwd_ms = f0.elapsed_time(f1) / args.steps
    fwd_stage = {name: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in pf])) for j, name in enumerate(fwd_names)}

    # per-step times, hot (back to back) and cold: before each cold step a 512 MiB buffer is
    # overwritten so the 256 MB last-level cache holds none of the step's inputs
    def per_step(nrep, flush):
        times = []
        for _ in range(nrep):
            if flush is not None:
                flush.add_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            step(None, None)
            e1.record()
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return times
    nrep = min(args.steps, 10)
    hot = per_step(nrep, None)
    flush = torch.zeros(512 * (1 << 20) // 4, dtype=torch.float32, device=dev)
    cold = per_step(nrep, flush)
    del flush

    extra = {"stage_ms": {k_: round(v_, 4) for k_, v_ in stage_mean.items()},
             "step_ms_hot": {"median": round(float(np.median(hot)), 4), "min": round(float(np.min(hot)), 4)},
             "step_ms_cold": {"median": round(float(np.median(cold)), 4), "min": round(float(np.min(cold)), 4)},
             "tokens_per_s_cold_median": B * T / (float(np.median(cold)) * 1e-3),
             "fwd_ms": round(fwd_ms, 4), "fwd_stage_ms": {k_: round(v_, 4) for k_, v_ in fwd_stage.items()},
             "fwd_tokens_per_s": B * T / (fwd_ms * 1e-3),
             # each workload's algorithmic bytes over its time, against 8 TB/s (the training step's
             # is path_hbm_frac below)
             "hbm_frac": {"fwd": hbm_frac(algorithmic(wl, False)["fwd"], wl, fwd_ms)}}

    # long-context forward (B1 H16 T32768 d128 L64): sixteen heads of 512 chunks, whose state
    # pass runs as segments chained by a scan of their affine maps
    if not args.no_long:
        wlc = WORKLOADS["long_ctx_fwd"]
        lin = make_inputs(wlc)
        lq, lk, lv = (torch.from_numpy(np.ascontiguousarray(lin[key + "_bits"]).view(np.int16)).to(dev)
                      .view(torch.bfloat16) for key in ("q", "k", "v"))
        lg_, lw_ = (torch.from_numpy(np.ascontiguousarray(lin[key], dtype=np.float32)).to(dev) for key in ("log_g", "w"))
        lb_ = torch.from_numpy(np.ascontiguousarray(lin["b"], dtype=np.float32)).to(dev) if "b" in lin else None
        for _ in range(2):
            carve.fwd(lq, lk, lv, lg_, lw_, b=lb_, L=wlc.L)
        torch.cuda.synchronize()
        le0, le1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        le0.record()
        for _ in range(5):
            carve.fwd(lq, lk, lv, lg_, lw_, b=lb_, L=wlc.L)
        le1.record()
        torch.cuda.synchronize()
        lms = le0.elapsed_time(le1) / 5
        extra["long_ctx_fwd_ms"] = round(lms, 4)
        extra["long_ctx_fwd_tokens_per_s"] = wlc.B * wlc.T / (lms * 1e-3)
        # inputs (no erase tensor) and o, plus the final state S_T
        extra.setdefault("hbm_frac", {})["long_ctx_fwd"] = hbm_frac(
            algorithmic(wlc, False)["fwd"], wlc, lms, extra_bytes=wlc.B * wlc.H * wlc.Dv * wlc.Dk * 4)
        # the training pair at the same shape: both state passes run as segments
        ldO = torch.from_numpy(np.ascontiguousarray(make_inputs(wlc, with_dO=True)["dO_bits"]).view(np.int16)).to(
            dev).view(torch.bfloat16)
        lsaved = carve.fwd_save(lq, lk, lv, lg_, lw_, b=lb_, L=wlc.L)[2]

        def long_pair():
            carve.fwd_save(lq, lk, lv, lg_, lw_, b=lb_, L=wlc.L, saved=lsaved)
            carve.bwd_saved(lq, lk, lv, lg_, lw_, ldO, lsaved, b=lb_, L=wlc.L, want_dS0=False)
        for _ in range(2):
            long_pair()
        torch.cuda.synchronize()
        le0.record()
        for _ in range(3):
            long_pair()
        le1.record()
        torch.cuda.synchronize()
        ltms = le0.elapsed_time(le1) / 3
        extra["long_ctx_train_ms"] = round(ltms, 4)
        extra["long_ctx_train_tokens_per_s"] = wlc.B * wlc.T / (ltms * 1e-3)
        del lq, lk, lv, lg_, lw_, lb_, ldO, lsaved

    # content-aware forward of the same shape (separate timing, not part of the step)
    if not args.no_content:
        wc = WORKLOADS["content_fwd"]
        cin = make_inputs(wc)
        cq = torch.from_numpy(np.ascontiguousarray(cin["q_bits"]).view(np.int16)).to(dev).view(torch.bfloat16)
        ck = torch.from_numpy(np.ascontiguousarray(cin["k_bits"]).view(np.int16)).to(dev).view(torch.bfloat16)
        cv = torch.from_numpy(np.ascontiguousarray(cin["v_bits"]).view(np.int16)).to(dev).view(torch.bfloat16)
        cf = {key: torch.from_numpy(np.ascontiguousarray(cin[key], dtype=np.float32)).to(dev)
              for key in ("log_g", "w", "b_x", "U1", "U2")}
        cont = {"b_x": cf["b_x"], "U1": cf["U1"], "U2": cf["U2"]}
        ws_c = torch.empty(max(1, carve.fwd_workspace_bytes(cq, cv, wc.L, content=True)), dtype=torch.uint8,
                           device=dev)
        co = torch.empty_like(cv)
        for _ in range(2):
            carve.fwd(cq, ck, cv, cf["log_g"], cf["w"], L=wc.L, content=cont, o=co, workspace=ws_c)
        torch.cuda.synchronize()
        ce0, ce1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nrep = 5
        ce0.record()
        for _ in range(nrep):
            carve.fwd(cq, ck, cv, cf["log_g"], cf["w"], L=wc.L, content=cont, o=co, workspace=ws_c)
        ce1.record()
        torch.cuda.synchronize()
        cms = ce0.elapsed_time(ce1) / nrep
        extra["content_fwd_ms"] = round(cms, 4)
        extra["content_fwd_tokens_per_s"] = wc.B * wc.T / (cms * 1e-3)
        # inputs with b_x in place of b (4 Dk bytes), and o
        cfb = algorithmic(wc, False)["fwd"] + 4 * wc.Dk
        extra.setdefault("hbm_frac", {})["content_fwd"] = hbm_frac(cfb, wc, cms)
        # its backward (gradients of q, k, v, log g, b_x, w, U1, U2): a reverse sweep over the
        # content periods, each a few launches over all heads
        cdo = torch.from_numpy(np.ascontiguousarray(make_inputs(wc, with_dO=True)["dO_bits"]).view(np.int16)).to(
            dev).view(torch.bfloat16)
        ws_cb = torch.empty(carve.bwd_content_workspace_bytes(cq, cv, wc.L, R=cf["U1"].shape[1]), dtype=torch.uint8,
                            device=dev)
        # as in training: the forward records each period's signal and mean, the backward reads
        # them; the backward that re-runs the content-aware forward instead is timed beside it
        zr, mr = carve.content_records(wc.B, wc.H, wc.T, wc.Dk, wc.Dv, wc.L, dev)
        carve.fwd(cq, ck, cv, cf["log_g"], cf["w"], L=wc.L, content=dict(cont, z_rec=zr, m_rec=mr), o=co,
                  workspace=ws_c)
        crec = dict(cont, z_rec=zr, m_rec=mr)

        def time_bwd(c_):
            for _ in range(2):
                carve.bwd_content(cq, ck, cv, cf["log_g"], cf["w"], cdo, c_, L=wc.L, workspace=ws_cb)
            torch.cuda.synchronize()
            ce0.record()
            for _ in range(3):
                carve.bwd_content(cq, ck, cv, cf["log_g"], cf["w"], cdo, c_, L=wc.L, workspace=ws_cb)
            ce1.record()
            torch.cuda.synchronize()
            return ce0.elapsed_time(ce1) / 3

        cbms = time_bwd(crec)
        extra["content_bwd_ms"] = round(cbms, 4)
        extra["content_bwd_tokens_per_s"] = wc.B * wc.T / (cbms * 1e-3)
        extra["content_bwd_recompute_ms"] = round(time_bwd(cont), 4)
        # the inputs again with dO, and dq, dk, dv, dlog g, db_x, dw (as the plain backward with b)
        extra["hbm_frac"]["content_bwd"] = hbm_frac(cfb + (algorithmic(wl, True)["bwd"] - algorithmic(wl, False)["fwd"]),
                                                     wc, cbms)
        del cq, ck, cv, cf, cont, crec, zr, mr, ws_c, co, cdo, ws_cb

    # gates given as pre-activations (activated inside the kernels), same shape; the plain
    # backward that recomputes the forward is timed beside it
    if not args.no_logits:
        extra["logits"] = logits_bench(q, k, v, dO, wl, dev)
        # f, b_x, w_hat take the places of log g, b, w: the same bytes as the plain pair
        alg_l = algorithmic(wl, True)
        extra.setdefault("hbm_frac", {})["fwd_logits"] = hbm_frac(alg_l["fwd"], wl, extra["logits"]["fwd_logits_ms"])
        extra["hbm_frac"]["bwd_logits"] = hbm_frac(alg_l["fwd"] + alg_l["bwd"], wl, extra["logits"]["bwd_logits_ms"])

    # recurrent decode step (one token per sequence and head, state updated in place)
    if not args.no_decode:
        extra["decode"] = {f"B{db}_H{H}": decode_bench(db, H, D, dev) for db in (B, 256)}

    # roofline of the dominant stage
    alg = algorithmic(wl, with_bwd)
    units = B * H * T
    stage_bytes = {
        "fwd_prep": alg["fwd_in"], "fwd_state": alg["fwd_out"],
        "bwd_state_rev": es_do(wl),
        "bwd_chunk_grads": alg.get("bwd_in", 0) + alg.get("bwd_out", 0),
    }
    dom = max(stage_mean, key=stage_mean.get)
    dom_ms = stage_mean[dom]
    ach = stage_bytes[dom] * units / (dom_ms * 1e-3) / 1e9
    path_bytes = alg["fwd"] + (alg["bwd"] if with_bwd else 0)
    path_flops = alg["flops_fwd"] + (alg["flops_bwd"] if with_bwd else 0)
    extra["path_hbm_frac"] = path_bytes * units / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS
    extra["path_mfma_frac"] = path_flops * units / (ms_step * 1e-3) / 1e12 / BF16_PEAK_TFLOPS
    extra["algorithmic_bytes_per_token_head"] = path_bytes
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None,
                "bytes_per_token_head": stage_bytes[dom], "launch_ms": round(dom_ms, 4)}
    copy_gbs = copy_bandwidth(dev)
    measured_peak = max(copy_gbs.values())
    roofline["measured_copy_GBs"] = copy_gbs
    roofline["measured_peak"] = measured_peak
    roofline["frac_of_measured"] = round(ach / measured_peak, 4)
    mf = measured_mfma(dom) if with_bwd else None
    if mf is not None:
        roofline["mfma_busy_frac"] = mf["busy_frac"]
        roofline["mfma_tflops"] = mf["tflops"]
        roofline["mfma_frac_of_bf16_peak"] = None if mf["tflops"] is None else round(mf["tflops"] / BF16_PEAK_TFLOPS, 4)
    traffic = measured_traffic(dom) if with_bwd else None
    if traffic is not None:
        roofline["traffic"] = traffic
        roofline["traffic_unit"] = "HBM bytes per launch (read + written)"
        roofline["traffic_over_algorithmic"] = round(traffic / (stage_bytes[dom] * units), 3)

    # every stage against the same roofline: its algorithmic bytes, and (while the counter
    # summary matches the kernel sources) its measured HBM traffic, per launch time
    stage_rl = {}
    for st_name, st_ms in stage_mean.items():
        rec = {"launch_ms": round(st_ms, 4), "bytes_per_token_head": stage_bytes.get(st_name),
               "algorithmic_GBs": round(stage_bytes.get(st_name, 0) * units / (st_ms * 1e-3) / 1e9, 1)}
        tr = measured_traffic(st_name) if with_bwd else None
        if tr is not None:
            rec["traffic_GBs"] = round(tr / (st_ms * 1e-3) / 1e9, 1)
            rec["traffic_frac_of_measured_copy"] = round(tr / (st_ms * 1e-3) / 1e9 / measured_peak, 3)
        stage_rl[st_name] = rec
    extra["stage_roofline"] = stage_rl

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, wl, args.cpu_sample_heads, with_bwd)

    tokens = B * T
    line = {
        "metric": "tokens/s (fwd, fwd+bwd) at B4 H16 T4096 d128 L64; % MFMA peak",
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "head1p3b_" + args.passes.replace("+", "_"), "B": B, "H": H, "T": T, "d": D,
                   "L": wl.L, "pass": args.passes, "parallelism": "single-gpu"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line))


def logits_bench(q, k, v, dO, wl, dev, nrep=5):
    """Time fwd_logits / bwd_logits and the plain recomputing backward at the workload shape."""
    import torch
    from chunk_gated_delta_amd import carve
    B, H, T, D = wl.B, wl.H, wl.T, wl.Dk
    gen = torch.Generator(device=dev).manual_seed(1007)
    f = torch.randn((B, H, T, D), generator=gen, device=dev)
    A = torch.rand((H, D), generator=gen, device=dev) * 0.2 + 0.02
    tau = torch.randn((H, D), generator=gen, device=dev) * 0.5
    w_hat = torch.randn((B, H, T), generator=gen, device=dev)
    b_x = torch.randn((B, H, T, D), generator=gen, device=dev) + 2.0
    ws_f = torch.empty(max(1, carve.fwd_workspace_bytes(q, v, wl.L)), dtype=torch.uint8, device=dev)
    log_g = (-A[None, :, None, :] * torch.nn.functional.softplus(f + tau[None, :, None, :])).contiguous()
    b, w = torch.sigmoid(b_x).contiguous(), torch.sigmoid(w_hat).contiguous()

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(nrep):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return round(e0.elapsed_time(e1) / nrep, 4)
    saved = carve.fwd_logits_save(q, k, v, f, A, tau, w_hat, b_x=b_x, L=wl.L)[2]
    out = {"fwd_logits_ms": timed(lambda: carve.fwd_logits(q, k, v, f, A, tau, w_hat, b_x=b_x, L=wl.L,
                                                           workspace=ws_f)),
           "bwd_logits_ms": timed(lambda: carve.bwd_logits(q, k, v, f, A, tau, w_hat, dO, b_x=b_x, L=wl.L)),
           "bwd_plain_ms": timed(lambda: carve.bwd(q, k, v, log_g, w, dO, b=b, L=wl.L)),
           # the training pair: the forward keeps its factors, the backward does not recompute it
           "fwd_logits_save_ms": timed(lambda: carve.fwd_logits_save(q, k, v, f, A, tau, w_hat, b_x=b_x, L=wl.L,
                                                                     saved=saved)),
           "bwd_logits_saved_ms": timed(lambda: carve.bwd_logits_saved(q, k, v, f, A, tau, w_hat, dO, saved,
                                                                       b_x=b_x, L=wl.L))}
    out["train_pair_ms"] = round(out["fwd_logits_save_ms"] + out["bwd_logits_saved_ms"], 4)
    return out


def decode_bench(B, H, D, dev, nrep=200):
    """Time carve.decode_step at batch B (bf16 q/k/v, fp32 gates and state, d = D): per step,
    one token for each of B sequences; the state (B*H*D*D fp32) is read and written once."""
    import torch
    from chunk_gated_delta_amd import carve
    from chunk_gated_delta_amd.synth import random_inputs
    inp = random_inputs(B, H, 1, D, D, dtype="bf16", seed=1006, erase="sigmoid", dists="softplus_decay")

    def t_(key, bf):
        if bf:
            x = torch.from_numpy(np.ascontiguousarray(inp[key + "_bits"]).view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            x = torch.from_numpy(np.ascontiguousarray(inp[key], dtype=np.float32)).to(dev)
        return x[:, :, 0].contiguous()
    q, k, v = t_("q", True), t_("k", True), t_("v", True)
    lg, b = t_("log_g", False), t_("b", False)
    w = torch.from_numpy(np.ascontiguousarray(inp["w"][:, :, 0], dtype=np.float32)).to(dev)
    S = torch.zeros((B, H, D, D), dtype=torch.float32, device=dev)
    o = torch.empty_like(v)
    for _ in range(10):
        carve.decode_step(q, k, v, lg, w, S, b=b, o=o)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(nrep):
        carve.decode_step(q, k, v, lg, w, S, b=b, o=o)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / nrep
    state_bytes = 2 * 4 * B * H * D * D            # the state read and written once per step
    return {"us_per_step": round(us, 3), "tokens_per_s": B / (us * 1e-6),
            "state_GB_per_s": round(state_bytes / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(state_bytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def es_do(wl):
    """dO bytes per token-head read by the reverse state pass."""
    return (2 if wl.dtype == "bf16" else 4) * wl.Dv


def cpu_baseline(inp, wl, n_heads, with_bwd):
    """The float64 reference timed on the host: the first n_heads (batch, head) sequences of
    the workload over the full sequence length, split over a pool of host processes (one per
    core this process may use, at most 16), scaled to the workload's tokens."""
    from oracle.head_pool import HeadPool, cpu_model, host_workers
    BH = wl.B * wl.H
    n_heads = max(1, min(n_heads, BH))
    sl = {k_: v_.reshape((1, BH) + v_.shape[2:])[:, :n_heads]
          for k_, v_ in inp.items() if not k_.endswith("_bits") and np.ndim(v_) >= 3}
    kw = dict(q=sl["q"], k=sl["k"], v=sl["v"], log_g=sl["log_g"], w=sl["w"], b=sl.get("b"))
    workers = host_workers()
    with HeadPool(workers) as pool:
        t0 = time.perf_counter()
        pool.run("forward", 1, n_heads, groups=workers, L=wl.L, **kw)
        if with_bwd:
            pool.run("backward", 1, n_heads, groups=workers, dO=sl["dO"], **kw)
        dt = time.perf_counter() - t0
    return {"value": wl.B * wl.T * (n_heads / BH) / dt, "unit": "tokens/s", "cores": workers, "kind": "oracle",
            "sample": f"{n_heads} of the {wl.B}x{wl.H} (batch, head) sequences, all {wl.T} tokens, "
                      f"{'forward+backward' if with_bwd else 'forward'}, float64 numpy, {workers} processes "
                      f"of one thread; tokens/s scaled by {n_heads}/{BH} of the workload",
            "seconds": round(dt, 2), "cpu": cpu_model(), "numpy": np.__version__}


if __name__ == "__main__":
    main()
