"""Full-size workloads compared with the float64 oracle on EVERY (batch, head) sequence
(needs an MI355X).  The oracle runs over groups of heads in a pool of host processes
(oracle/head_pool.py); each output and gradient is compared per head, normalised by that
head's own largest reference magnitude, so a slip that touches only some heads (the state
passes map value slices and heads to workgroups) cannot hide behind the others.

Workloads (shapes and distributions of chunk_gated_delta_amd/synth.py):
  head1p3b_fwd   B4 H16 T4096 d128 L64 bf16, b = sigmoid(N(2,1)): the plain forward and the
                 training pair fwd_save + bwd_saved, exactly as the benchmark launches them
  long_ctx_fwd   B1 H16 T32768 d128 L64 bf16: o and the final state S_T
  content_fwd    B4 H16 T4096 d128 L64 bf16, rank-16 content projection: o, S_T, m_out,
                 and the content backward
  train_fwd_bwd  B8 H16 T2048 d128 L64 bf16, b = 1: forward and the recomputing backward
"""
import numpy as np
import pytest
import torch

from chunk_gated_delta_amd import carve
from chunk_gated_delta_amd.synth import WORKLOADS, make_inputs
from oracle.head_pool import HeadPool
from tests.helpers import per_head_rel, to_device, to_np

pytestmark = pytest.mark.gpu

TOL = 2e-2          # bf16 inputs


def announce(name):
    print(f"\n[case] {name}", flush=True)


def progress(label):
    def cb(done, total):
        if done == total or done % 8 == 0:
            print(f"  oracle {label}: {done}/{total} head groups", flush=True)
    return cb


def check_all(label, pairs):
    """pairs: name -> (gpu array, reference array), both [B, H, ...]."""
    bad = {}
    for name, (g, r) in pairs.items():
        e = per_head_rel(g, r)
        b, h = np.unravel_index(int(np.argmax(e)), e.shape)
        print(f"  {label} {name}: worst head ({b},{h}) {e.max():.2e}, median {np.median(e):.2e}", flush=True)
        if e.max() > TOL:
            bad[name] = (float(e.max()), int(b), int(h), int(np.sum(e > TOL)))
    assert not bad, bad


def token_kwargs(inp):
    return dict(q=inp["q"], k=inp["k"], v=inp["v"], log_g=inp["log_g"], w=inp["w"], b=inp.get("b"))


def test_head1p3b_every_head_fwd_and_training_pair():
    """The benchmark's launch: plain forward, then fwd_save + bwd_saved; o, S_T and every
    gradient (dq, dk, dv, dlog_g, db, dw) of all 64 heads against the oracle."""
    wl = WORKLOADS["head1p3b_fwd"]
    announce(wl.name + " every head: fwd, fwd_save + bwd_saved")
    inp = make_inputs(wl, with_dO=True)
    d = to_device(inp, wl.dtype)
    o1, s1, _ = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d["b"], L=wl.L)
    o2, s2, saved = carve.fwd_save(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d["b"], L=wl.L)
    g = carve.bwd_saved(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], saved, b=d["b"], L=wl.L)
    torch.cuda.synchronize()
    gpu = {"o(fwd)": to_np(o1), "S_T(fwd)": to_np(s1), "o(fwd_save)": to_np(o2), "S_T(fwd_save)": to_np(s2)}
    gpu.update({key: to_np(g[key]) for key in ("dq", "dk", "dv", "dlog_g", "db", "dw")})
    del d, o1, s1, o2, s2, saved, g
    with HeadPool() as pool:
        ro, rS, _ = pool.run("forward", wl.B, wl.H, L=wl.L, progress=progress("forward"), **token_kwargs(inp))
        ref = pool.run("backward", wl.B, wl.H, dO=inp["dO"], progress=progress("backward"), **token_kwargs(inp))
    pairs = {"o(fwd)": (gpu["o(fwd)"], ro), "S_T(fwd)": (gpu["S_T(fwd)"], rS),
             "o(fwd_save)": (gpu["o(fwd_save)"], ro), "S_T(fwd_save)": (gpu["S_T(fwd_save)"], rS)}
    pairs.update({key: (gpu[key], ref[key]) for key in ("dq", "dk", "dv", "dlog_g", "db", "dw")})
    check_all(wl.name, pairs)


def test_long_ctx_every_head():
    """B1 H16 T32768: o and S_T of all 16 heads (512 chunks each; the state pass runs as
    segments chained by a scan of their affine maps)."""
    wl = WORKLOADS["long_ctx_fwd"]
    announce(wl.name + " every head")
    inp = make_inputs(wl)
    d = to_device(inp, wl.dtype)
    o, S_T, _ = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d.get("b"), L=wl.L)
    torch.cuda.synchronize()
    o, S_T = to_np(o), to_np(S_T)
    del d
    with HeadPool() as pool:
        ro, rS, _ = pool.run("forward", wl.B, wl.H, groups=wl.B * wl.H, L=wl.L, progress=progress("forward"),
                             **token_kwargs(inp))
    check_all(wl.name, {"o": (o, ro), "S_T": (S_T, rS)})


def test_content_every_head_fwd_and_bwd():
    """Content-aware erase at B4 H16 T4096: o, S_T, m_out and the content backward's
    dq, dk, dv, dlog_g, db_x, dw, dm0, dS0 of all 64 heads; dU1 / dU2 (sums over the batch)
    per head index."""
    wl = WORKLOADS["content_fwd"]
    announce(wl.name + " every head: content fwd + bwd")
    inp = make_inputs(wl, with_dO=True)
    d = to_device(inp, wl.dtype)
    cont = {"b_x": d["b_x"], "U1": d["U1"], "U2": d["U2"]}
    o, S_T, m = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], L=wl.L, content=cont)
    g = carve.bwd_content(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], cont, L=wl.L)
    torch.cuda.synchronize()
    names = ("dq", "dk", "dv", "dlog_g", "db_x", "dw", "dm0", "dS0")
    gpu = {"o": to_np(o), "S_T": to_np(S_T), "m_out": to_np(m)}
    gpu.update({key: to_np(g[key]) for key in names + ("dU1", "dU2")})
    del d, o, S_T, m, g
    rc = {"b_x": inp["b_x"], "U1": inp["U1"], "U2": inp["U2"]}
    kw = dict(q=inp["q"], k=inp["k"], v=inp["v"], log_g=inp["log_g"], w=inp["w"], L=wl.L, content=rc)
    with HeadPool() as pool:
        ro, rS, rm = pool.run("forward", wl.B, wl.H, progress=progress("content forward"), **kw)
        ref = pool.run("backward_content", wl.B, wl.H, dO=inp["dO"], progress=progress("content backward"), **kw)
    pairs = {"o": (gpu["o"], ro), "S_T": (gpu["S_T"], rS), "m_out": (gpu["m_out"], rm)}
    pairs.update({key: (gpu[key], ref[key]) for key in names})
    # [H, ...] sums over the batch: compare per head index (as a batch of one)
    pairs.update({key: (gpu[key][None], ref[key][None]) for key in ("dU1", "dU2")})
    check_all(wl.name, pairs)


def test_train_every_head_fwd_and_bwd():
    """Training workload B8 H16 T2048, b = 1: o, S_T and every gradient of all 128 heads
    through the backward that recomputes the forward."""
    wl = WORKLOADS["train_fwd_bwd"]
    announce(wl.name + " every head: fwd + bwd")
    inp = make_inputs(wl)
    d = to_device(inp, wl.dtype)
    o, S_T, _ = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d["b"], L=wl.L)
    g = carve.bwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], b=d["b"], L=wl.L)
    torch.cuda.synchronize()
    names = ("dq", "dk", "dv", "dlog_g", "db", "dw")
    gpu = {"o": to_np(o), "S_T": to_np(S_T)}
    gpu.update({key: to_np(g[key]) for key in names})
    del d, o, S_T, g
    with HeadPool() as pool:
        ro, rS, _ = pool.run("forward", wl.B, wl.H, L=wl.L, progress=progress("forward"), **token_kwargs(inp))
        ref = pool.run("backward", wl.B, wl.H, dO=inp["dO"], progress=progress("backward"), **token_kwargs(inp))
    pairs = {"o": (gpu["o"], ro), "S_T": (gpu["S_T"], rS)}
    pairs.update({key: (gpu[key], ref[key]) for key in names})
    check_all(wl.name, pairs)
