"""GPU parity of the backward through the content-aware erase (needs an MI355X).

Compared with the float64 reverse-mode reference (itself pinned by finite
differences in the CPU suite).  Error metric: per gradient tensor,
max|gpu - ref| / max|ref|; bars 1e-4 (float32 inputs) and 2e-2 (bfloat16 inputs).
"""
import numpy as np
import pytest
import torch

import oracle
from chunk_gated_delta_amd import carve
from chunk_gated_delta_amd.synth import random_inputs
from tests.helpers import max_rel, to_device, to_np

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}
NAMES = ("dq", "dk", "dv", "dlog_g", "db_x", "dw", "dU1", "dU2", "dm0", "dS0")


def announce(name):
    print(f"\n[case] {name}", flush=True)


def f32(x):
    return torch.from_numpy(np.asarray(x, np.float32)).cuda()


def content_case(B, H, T, D, dtype, seed, scale=8.0):
    inp = random_inputs(B, H, T, D, D, dtype=dtype, seed=seed, erase="content", dists="softplus_decay",
                        with_dO=True)
    inp["U1"] = inp["U1"] * scale
    inp["U2"] = inp["U2"] * scale
    rng = np.random.default_rng(seed + 1)
    extra = {
        "m0": np.asarray(rng.standard_normal((B, H, D)) * 0.5, np.float32).astype(np.float64),
        "S0": np.asarray(rng.standard_normal((B, H, D, D)) * 0.3, np.float32).astype(np.float64),
        "dS_T": np.asarray(rng.standard_normal((B, H, D, D)) * 0.3, np.float32).astype(np.float64),
        "dm_out": np.asarray(rng.standard_normal((B, H, D)), np.float32).astype(np.float64),
    }
    return inp, extra


def run_both(inp, ex, dtype, L, proj=True):
    d = to_device(inp, dtype)
    U1 = d["U1"] if proj else None
    U2 = d["U2"] if proj else None
    g = carve.bwd_content(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"],
                          {"b_x": d["b_x"], "U1": U1, "U2": U2, "m0": f32(ex["m0"])},
                          S0=f32(ex["S0"]), dS_T=f32(ex["dS_T"]), dm_out=f32(ex["dm_out"]), L=L)
    torch.cuda.synchronize()
    g = {k_: (None if v_ is None else to_np(v_)) for k_, v_ in g.items()}
    ref = oracle.backward_content(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], inp["dO"],
                                  {"b_x": inp["b_x"], "U1": inp["U1"] if proj else None,
                                   "U2": inp["U2"] if proj else None, "m0": ex["m0"]},
                                  S0=ex["S0"], dS_T=ex["dS_T"], dm_out=ex["dm_out"], L=L)
    return g, ref


def check(g, ref, tol):
    errs = {}
    for key in NAMES:
        if ref[key] is None:
            assert g[key] is None, key
            continue
        errs[key] = max_rel(g[key], ref[key])
    print("  " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
    assert all(v_ <= tol for v_ in errs.values()), errs


CASES = [
    # dtype, B, H, T, D, L
    ("f32", 1, 2, 200, 64, 64),
    ("bf16", 2, 2, 256, 128, 64),
    ("bf16", 1, 2, 320, 128, 128),
    ("bf16", 2, 1, 100, 64, 32),
    ("f32", 1, 1, 96, 128, 32),
    # periods longer than the gate kernel's 64-token batch: a partial second batch, and
    # three batches with a short last period
    ("f32", 1, 2, 200, 64, 96),
    ("bf16", 1, 1, 400, 128, 192),
]


@pytest.mark.parametrize("dtype,B,H,T,D,L", CASES, ids=[f"{c[0]}_T{c[3]}_d{c[4]}_L{c[5]}" for c in CASES])
def test_content_bwd_parity(dtype, B, H, T, D, L):
    announce(f"content bwd {dtype} B{B} H{H} T{T} d{D} L{L}")
    inp, ex = content_case(B, H, T, D, dtype, seed=200 + T + D + L)
    g, ref = run_both(inp, ex, dtype, L)
    check(g, ref, TOL[dtype])
    # the chain through the mean outputs must matter here (else it pins nothing)
    ref0 = oracle.backward_content(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], inp["dO"],
                                   {"b_x": inp["b_x"], "U1": None, "U2": None, "m0": ex["m0"]},
                                   S0=ex["S0"], dS_T=ex["dS_T"], dm_out=ex["dm_out"], L=L)
    assert max_rel(ref0["dk"], ref["dk"]) > 0.02


def test_content_bwd_rank64():
    """The largest projection rank (64) at width 64, over several periods, with the
    projection scaled by 64: sigma(b_x + z) then reaches hard erase on many channels,
    so tiles of tokens take the range-safe path as well as the fast one."""
    announce("content bwd rank 64 d64")
    B, H, T, D, L = 2, 2, 150, 64, 32
    inp = random_inputs(B, H, T, D, D, dtype="bf16", seed=321, erase="content", dists="softplus_decay",
                        with_dO=True, rank=64)
    inp["U1"] = inp["U1"] * 64.0
    inp["U2"] = inp["U2"] * 64.0
    rng = np.random.default_rng(322)
    ex = {"m0": np.asarray(rng.standard_normal((B, H, D)) * 0.5, np.float32).astype(np.float64),
          "S0": np.asarray(rng.standard_normal((B, H, D, D)) * 0.3, np.float32).astype(np.float64),
          "dS_T": np.asarray(rng.standard_normal((B, H, D, D)) * 0.3, np.float32).astype(np.float64),
          "dm_out": np.asarray(rng.standard_normal((B, H, D)), np.float32).astype(np.float64)}
    g, ref = run_both(inp, ex, "bf16", L)
    check(g, ref, TOL["bf16"])


def test_content_bwd_no_projection():
    announce("content bwd without projection")
    inp, ex = content_case(2, 2, 150, 128, "bf16", seed=301)
    g, ref = run_both(inp, ex, "bf16", 64, proj=False)
    check(g, ref, TOL["bf16"])
    assert np.all(g["dm0"] == 0)


def test_content_bwd_zero_projection_bit_exact():
    """U_b = 0 gives the same gradients as U_b absent, bit for bit, and zero
    gradients for the projection and the carried-in mean."""
    announce("content bwd zero projection bit exact")
    inp, ex = content_case(2, 2, 192, 128, "bf16", seed=302)
    d = to_device(inp, "bf16")
    outs = []
    for U1, U2 in ((torch.zeros_like(d["U1"]), torch.zeros_like(d["U2"])), (None, None)):
        g = carve.bwd_content(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"],
                              {"b_x": d["b_x"], "U1": U1, "U2": U2, "m0": f32(ex["m0"])},
                              S0=f32(ex["S0"]), dS_T=f32(ex["dS_T"]), L=64)
        torch.cuda.synchronize()
        outs.append(g)
    for key in ("dq", "dk", "dv", "dlog_g", "db_x", "dw", "dm0", "dS0"):
        assert torch.equal(outs[0][key], outs[1][key]), key
    assert torch.count_nonzero(outs[0]["dU1"]) == 0 and torch.count_nonzero(outs[0]["dU2"]) == 0


@pytest.mark.parametrize("T,L,R", [(1, 64, 16), (59, 64, 1), (64, 64, 4)])
def test_content_bwd_short_sequences(T, L, R):
    """One token, one partial chunk, exactly one chunk (only m0 feeds a gate)."""
    announce(f"content bwd short T{T} L{L} R{R}")
    B, H, D = 2, 2, 128
    inp = random_inputs(B, H, T, D, D, dtype="bf16", seed=400 + T, erase="content", dists="softplus_decay",
                        with_dO=True, rank=R)
    inp["U1"] = inp["U1"] * 8.0
    inp["U2"] = inp["U2"] * 8.0
    rng = np.random.default_rng(401)
    ex = {"m0": np.asarray(rng.standard_normal((B, H, D)), np.float32).astype(np.float64),
          "S0": np.asarray(rng.standard_normal((B, H, D, D)) * 0.3, np.float32).astype(np.float64),
          "dS_T": np.asarray(rng.standard_normal((B, H, D, D)) * 0.3, np.float32).astype(np.float64),
          "dm_out": np.asarray(rng.standard_normal((B, H, D)), np.float32).astype(np.float64)}
    g, ref = run_both(inp, ex, "bf16", L)
    check(g, ref, TOL["bf16"])


def test_content_bwd_empty_sequence():
    """T = 0: S_T = S0 and m_out = m0, so their gradients pass through; the rest is zero."""
    announce("content bwd empty")
    B, H, D = 1, 2, 64
    z = torch.zeros((B, H, 0, D), dtype=torch.bfloat16, device="cuda")
    zf = torch.zeros((B, H, 0, D), dtype=torch.float32, device="cuda")
    dS_T = torch.randn((B, H, D, D), device="cuda")
    dm_out = torch.randn((B, H, D), device="cuda")
    U1 = torch.randn((H, 4, D), device="cuda")
    U2 = torch.randn((H, D, 4), device="cuda")
    g = carve.bwd_content(z, z, z, zf, torch.zeros((B, H, 0), device="cuda"), z, {"b_x": zf, "U1": U1, "U2": U2},
                          dS_T=dS_T, dm_out=dm_out, L=64)
    torch.cuda.synchronize()
    assert torch.equal(g["dS0"], dS_T) and torch.equal(g["dm0"], dm_out)
    assert torch.count_nonzero(g["dU1"]) == 0 and torch.count_nonzero(g["dU2"]) == 0


def test_forward_records_match_reference():
    """The forward's per-period records: m_rec[p] is the mean output of period p-1 (m0 for
    the first), z_rec[p] = U2 U1 m_rec[p]; checked against the reference forward's outputs."""
    announce("content forward records")
    B, H, T, D, L = 2, 2, 200, 128, 64
    inp, ex = content_case(B, H, T, D, "bf16", seed=131)
    d = to_device(inp, "bf16")
    zr, mr = carve.content_records(B, H, T, D, D, L, "cuda")
    carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], L=L,
              content={"b_x": d["b_x"], "U1": d["U1"], "U2": d["U2"], "m0": f32(ex["m0"]), "z_rec": zr, "m_rec": mr})
    torch.cuda.synchronize()
    ro, _, _ = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], L=L,
                              content={"b_x": inp["b_x"], "U1": inp["U1"], "U2": inp["U2"], "m0": ex["m0"]})
    P = (T + L - 1) // L
    m_ref = np.empty((B, H, P, D))
    m_ref[:, :, 0] = ex["m0"]
    for p_ in range(1, P):
        m_ref[:, :, p_] = ro[:, :, (p_ - 1) * L:p_ * L].mean(axis=2)
    z_ref = np.einsum("hkr,bhpr->bhpk", inp["U2"], np.einsum("hrv,bhpv->bhpr", inp["U1"], m_ref))
    em, ez = max_rel(to_np(mr), m_ref), max_rel(to_np(zr), z_ref)
    print(f"  err m_rec={em:.2e} z_rec={ez:.2e}", flush=True)
    assert em <= TOL["bf16"] and ez <= TOL["bf16"]


@pytest.mark.parametrize("dtype,D,T,L", [("bf16", 128, 200, 64), ("f32", 64, 130, 32)])
def test_backward_with_records_is_bit_identical(dtype, D, T, L):
    """Passing the forward's records skips the re-run of the content-aware forward and gives
    the same gradients, bit for bit."""
    announce(f"content backward with records {dtype} d{D} T{T} L{L}")
    B, H = 2, 2
    inp, ex = content_case(B, H, T, D, dtype, seed=141 + D)
    d = to_device(inp, dtype)
    cont = {"b_x": d["b_x"], "U1": d["U1"], "U2": d["U2"], "m0": f32(ex["m0"])}
    zr, mr = carve.content_records(B, H, T, D, D, L, "cuda")
    carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], S0=f32(ex["S0"]), L=L,
              content=dict(cont, z_rec=zr, m_rec=mr))
    kw = dict(S0=f32(ex["S0"]), dS_T=f32(ex["dS_T"]), dm_out=f32(ex["dm_out"]), L=L)
    g0 = carve.bwd_content(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], cont, **kw)
    g1 = carve.bwd_content(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], dict(cont, z_rec=zr, m_rec=mr), **kw)
    torch.cuda.synchronize()
    for key in NAMES:
        assert torch.equal(g0[key], g1[key]), key
