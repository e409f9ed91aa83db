"""Drive the CARVE kernels for an external profiler (rocprofv3).

    python -m chunk_gated_delta_amd.profile_step [--steps 5] [--warmup 2]
                                                  [--pass fwd+bwd|fwd|long|content|content_bwd|decode]
                                                  [--copy-mib 0]
                                                  [--decode-batch 256]

Runs the 1.3B-head-shape workload (B4 H16 T4096 d128 L64, bf16 q/k/v, fp32 gates;
synthetic seeded inputs) through the same entry points as bench.py: the training step
(fwd_save + bwd_saved), the plain forward, the content-aware forward or its backward (given the forward's
per-period records), the
long-context forward (B1 H16 T32768, --pass long), or recurrent decode
steps (one token per sequence and head at batch --decode-batch).  With
--copy-mib N it also runs a plain elementwise kernel that reads N MiB and writes N MiB
(torch.neg), the reference against which HBM byte counters are scaled.  Prints one
progress line per phase.
"""
import argparse
import sys
import time


def main(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--pass", dest="passes", default="fwd+bwd",
                   choices=["fwd+bwd", "fwd", "long", "content", "content_bwd", "decode"])
    p.add_argument("--decode-batch", type=int, default=256)
    p.add_argument("--copy-mib", type=int, default=0)
    args = p.parse_args(argv)

    import numpy as np
    import torch
    from chunk_gated_delta_amd import carve
    from chunk_gated_delta_amd.synth import WORKLOADS, make_inputs

    dev = torch.device("cuda:0")
    wl = WORKLOADS["content_fwd" if args.passes in ("content", "content_bwd")
                   else "long_ctx_fwd" if args.passes == "long" else "head1p3b_fwd"]
    if args.passes == "decode":
        return decode(args, wl, dev)
    inp = make_inputs(wl, with_dO=args.passes in ("fwd+bwd", "content_bwd"))

    def bf16(name):
        return torch.from_numpy(np.ascontiguousarray(inp[name + "_bits"]).view(np.int16)).to(dev).view(torch.bfloat16)

    def f32(name):
        return torch.from_numpy(np.ascontiguousarray(inp[name], dtype=np.float32)).to(dev)

    q, k, v = bf16("q"), bf16("k"), bf16("v")
    log_g, w = f32("log_g"), f32("w")
    b = f32("b") if "b" in inp else None
    dO = bf16("dO") if args.passes in ("fwd+bwd", "content_bwd") else None
    content = None
    if args.passes in ("content", "content_bwd"):
        content = {"b_x": f32("b_x"), "U1": f32("U1"), "U2": f32("U2")}
    if args.passes == "content_bwd":
        # the forward's per-period records, as a training step would keep them
        zr, mr = carve.content_records(wl.B, wl.H, wl.T, wl.Dk, wl.Dv, wl.L, dev)
        carve.fwd(q, k, v, log_g, w, L=wl.L, content=dict(content, z_rec=zr, m_rec=mr))
        content = dict(content, z_rec=zr, m_rec=mr)
    print(f"[profile_step] inputs ready: {wl.name} B{wl.B} H{wl.H} T{wl.T} d{wl.Dk} L{wl.L}", flush=True)

    def step():
        if args.passes == "fwd+bwd":
            o, _, saved = carve.fwd_save(q, k, v, log_g, w, b=b, L=wl.L)
            carve.bwd_saved(q, k, v, log_g, w, dO, saved, b=b, L=wl.L)
        elif args.passes in ("fwd", "long"):
            carve.fwd(q, k, v, log_g, w, b=b, L=wl.L)
        elif args.passes == "content_bwd":
            carve.bwd_content(q, k, v, log_g, w, dO, content, L=wl.L)
        else:
            carve.fwd(q, k, v, log_g, w, L=wl.L, content=content)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / max(args.steps, 1)
    print(f"[profile_step] {args.passes}: {args.warmup} warm-up + {args.steps} steps, {ms:.3f} ms/step", flush=True)

    if args.copy_mib > 0:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(f"[profile_step] reference kernel: torch.neg over {args.copy_mib} MiB in, "
              f"{args.copy_mib} MiB out, 3 calls", flush=True)
    return 0


def decode(args, wl, dev):
    """Recurrent decode steps at batch --decode-batch (heads and width of the workload)."""
    import numpy as np
    import torch
    from chunk_gated_delta_amd import carve
    from chunk_gated_delta_amd.synth import random_inputs
    B, H, D = args.decode_batch, wl.H, wl.Dk
    inp = random_inputs(B, H, 1, D, D, dtype="bf16", seed=1006, erase="sigmoid", dists="softplus_decay")

    def bf16(name):
        x = torch.from_numpy(np.ascontiguousarray(inp[name + "_bits"]).view(np.int16)).to(dev).view(torch.bfloat16)
        return x[:, :, 0].contiguous()

    def f32(name):
        return torch.from_numpy(np.ascontiguousarray(inp[name], dtype=np.float32)).to(dev)[:, :, 0].contiguous()

    q, k, v = bf16("q"), bf16("k"), bf16("v")
    lg, b = f32("log_g"), f32("b")
    w = torch.from_numpy(np.ascontiguousarray(inp["w"][:, :, 0], dtype=np.float32)).to(dev)
    S = torch.zeros((B, H, D, D), dtype=torch.float32, device=dev)
    print(f"[profile_step] decode inputs ready: B{B} H{H} d{D}", flush=True)
    for _ in range(args.warmup + args.steps):
        carve.decode_step(q, k, v, lg, w, S, b=b)
    torch.cuda.synchronize()
    print(f"[profile_step] decode: {args.warmup} warm-up + {args.steps} steps", flush=True)
    if args.copy_mib > 0:
        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(f"[profile_step] reference kernel: torch.neg over {args.copy_mib} MiB in, "
              f"{args.copy_mib} MiB out, 3 calls", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
