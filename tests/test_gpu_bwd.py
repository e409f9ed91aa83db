"""GPU backward parity against the float64 reverse-mode reference (needs an MI355X).

Error metric: per gradient tensor, max|gpu - ref| / max|ref|; bars 1e-4 (float32
inputs) and 2e-2 (bfloat16 inputs).  The reference backward is itself pinned by
finite differences in the CPU suite.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from chunk_gated_delta_amd import carve
from chunk_gated_delta_amd.synth import random_inputs
from tests.helpers import max_rel, per_head_rel, to_device, to_np

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}
NAMES = ("dq", "dk", "dv", "dlog_g", "db", "dw", "dS0")


def announce(name):
    print(f"\n[case] {name}", flush=True)


def gpu_bwd(inp, dtype, L, S0=None, dS_T=None):
    d = to_device(inp, dtype)
    S0d = None if S0 is None else torch.from_numpy(np.asarray(S0, np.float32)).cuda()
    dSd = None if dS_T is None else torch.from_numpy(np.asarray(dS_T, np.float32)).cuda()
    g = carve.bwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], b=d.get("b"), S0=S0d, dS_T=dSd, L=L)
    torch.cuda.synchronize()
    return {k_: (None if v_ is None else to_np(v_)) for k_, v_ in g.items()}


CASES = [
    # name, B, H, T, D, dtype, L, erase, dists, with_state
    ("bf16_d128_ragged", 1, 2, 200, 128, "bf16", 64, "sigmoid", "softplus_decay", True),
    ("bf16_d128_no_b", 2, 1, 128, 128, "bf16", 64, "none", "uniform_decay", False),
    ("bf16_d128_L32", 1, 2, 96, 128, "bf16", 32, "ones", "uniform_decay", True),
    ("bf16_d64", 2, 2, 150, 64, "bf16", 64, "sigmoid", "softplus_decay", True),
    ("f32_d64", 1, 2, 100, 64, "f32", 64, "sigmoid", "softplus_decay", True),
    ("f32_d128", 1, 1, 70, 128, "f32", 64, "none", "uniform_decay", True),
    ("bf16_T1", 1, 1, 1, 128, "bf16", 64, "sigmoid", "softplus_decay", True),
]


@pytest.mark.parametrize("name,B,H,T,D,dtype,L,erase,dists,with_state", CASES, ids=[c[0] for c in CASES])
def test_bwd_parity(name, B, H, T, D, dtype, L, erase, dists, with_state):
    announce(name)
    inp = random_inputs(B, H, T, D, D, dtype=dtype, seed=zlib.crc32(name.encode()) % 1000, erase=erase,
                        dists=dists, with_dO=True)
    rng = np.random.default_rng(9)
    S0 = dS_T = None
    if with_state:
        S0 = np.asarray(rng.standard_normal((B, H, D, D)) * 0.3, np.float32).astype(np.float64)
        dS_T = np.asarray(rng.standard_normal((B, H, D, D)) * 0.3, np.float32).astype(np.float64)
    g = gpu_bwd(inp, dtype, L, S0=S0, dS_T=dS_T)
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], inp["dO"], b=inp.get("b"),
                          S0=S0, dS_T=dS_T)
    errs = {}
    for key in NAMES:
        if ref[key] is None:
            assert g[key] is None
            continue
        errs[key] = max_rel(g[key], ref[key])
    print("  " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
    assert all(v_ <= TOL[dtype] for v_ in errs.values()), errs


def test_bwd_determinism():
    announce("bwd determinism")
    inp = random_inputs(2, 2, 256, 128, 128, dtype="bf16", seed=61, erase="sigmoid", dists="softplus_decay",
                        with_dO=True)
    g1 = gpu_bwd(inp, "bf16", 64)
    g2 = gpu_bwd(inp, "bf16", 64)
    for key in NAMES:
        if g1[key] is not None:
            assert np.array_equal(g1[key], g2[key]), key


def test_bwd_empty():
    announce("bwd empty")
    q = torch.zeros((1, 2, 0, 64), dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros((1, 2, 0, 64), dtype=torch.float32, device="cuda")
    w = torch.zeros((1, 2, 0), dtype=torch.float32, device="cuda")
    dS_T = torch.randn((1, 2, 64, 64), device="cuda")
    g = carve.bwd(q, q, q, lg, w, q, dS_T=dS_T)
    torch.cuda.synchronize()
    assert torch.equal(g["dS0"], dS_T)


def test_saved_pair_matches_recompute_bitwise():
    """fwd_save gives the same o and S_T as fwd, and bwd_saved the same gradients as bwd
    (the same arithmetic, only the forward is not recomputed)."""
    announce("fwd_save / bwd_saved vs fwd / bwd")
    for (D, dtype, T, erase) in [(128, "bf16", 200, "sigmoid"), (64, "f32", 100, "none")]:
        inp = random_inputs(2, 2, T, D, D, dtype=dtype, seed=71 + D, erase=erase, dists="softplus_decay",
                            with_dO=True)
        d = to_device(inp, dtype)
        S0 = torch.randn((2, 2, D, D), device="cuda") * 0.3
        dS_T = torch.randn((2, 2, D, D), device="cuda") * 0.3
        o1, s1, _ = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d.get("b"), S0=S0)
        o2, s2, saved = carve.fwd_save(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d.get("b"), S0=S0)
        g1 = carve.bwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], b=d.get("b"), S0=S0, dS_T=dS_T)
        g2 = carve.bwd_saved(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], saved, b=d.get("b"), dS_T=dS_T)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(s1, s2)
        for key in NAMES:
            if g1[key] is not None:
                assert torch.equal(g1[key], g2[key]), (D, key)


@pytest.mark.parametrize("B,H", [(8, 8), (8, 16)], ids=["slice32", "slice64"])
def test_wide_value_slices_every_head(B, H):
    """Enough heads that the state passes split D=128 into 32- and 64-row value slices
    (whose state copies and outputs leave through LDS), with a ragged tail, S0 and dS_T;
    forward and gradients of every head against the reference, normalised per head."""
    announce(f"wide value slices B{B} H{H}")
    T, D = 100, 128
    inp = random_inputs(B, H, T, D, D, dtype="bf16", seed=300 + H, erase="sigmoid", dists="softplus_decay",
                        with_dO=True)
    rng = np.random.default_rng(11)
    S0 = np.asarray(rng.standard_normal((B, H, D, D)) * 0.3, np.float32).astype(np.float64)
    dS_T = np.asarray(rng.standard_normal((B, H, D, D)) * 0.3, np.float32).astype(np.float64)
    d = to_device(inp, "bf16")
    S0d = torch.from_numpy(np.asarray(S0, np.float32)).cuda()
    dSd = torch.from_numpy(np.asarray(dS_T, np.float32)).cuda()
    o, S_T, _ = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d["b"], S0=S0d)
    g = carve.bwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], b=d["b"], S0=S0d, dS_T=dSd)
    torch.cuda.synchronize()
    o_ref, sT_ref, _ = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], b=inp["b"], S0=S0)
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], inp["dO"], b=inp["b"],
                          S0=S0, dS_T=dS_T)
    errs = {"o": per_head_rel(to_np(o), o_ref).max(), "S_T": per_head_rel(to_np(S_T), sT_ref).max()}
    errs.update({key: per_head_rel(to_np(g[key]), ref[key]).max() for key in NAMES})
    print("  worst head " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
    assert all(v_ <= 2e-2 for v_ in errs.values()), errs
