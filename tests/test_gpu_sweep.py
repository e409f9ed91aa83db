"""Token counts at and around every tile boundary (needs an MI355X).  The kernels tile tokens
in 16-token blocks inside 32- or 64-token chunks, and the state passes walk whole chunks;
each count below sits on, just before or just after one of those edges.  For each: the
forward (o, S_T), the recomputing backward (every gradient and dS0) and the training pair
(the same bits as the recomputing calls) against the float64 oracle, float32 and bfloat16,
both head widths and one unequal pair; and the content-aware forward and backward at
counts around the content period."""
import numpy as np
import pytest
import torch

import oracle
from chunk_gated_delta_amd import carve
from chunk_gated_delta_amd.synth import random_inputs
from tests.helpers import max_rel, to_device, to_np

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}
NAMES = ("dq", "dk", "dv", "dlog_g", "db", "dw", "dS0")
TS = (1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 191)


def f32(x):
    return torch.from_numpy(np.asarray(x, np.float32)).cuda()


@pytest.mark.parametrize("dtype,Dk,Dv", [("bf16", 128, 128), ("f32", 64, 64), ("bf16", 64, 128), ("f32", 128, 128)])
def test_token_count_sweep(dtype, Dk, Dv):
    print(f"\n[case] token sweep {dtype} Dk{Dk} Dv{Dv}", flush=True)
    B, H = 1, 2
    worst = {}
    for T in TS:
        inp = random_inputs(B, H, T, Dk, Dv, dtype=dtype, seed=1000 + T + Dk, erase="sigmoid",
                            dists="softplus_decay", with_dO=True)
        rng = np.random.default_rng(2000 + T)
        S0 = np.asarray(rng.standard_normal((B, H, Dv, Dk)) * 0.3, np.float32).astype(np.float64)
        dS_T = np.asarray(rng.standard_normal((B, H, Dv, Dk)) * 0.3, np.float32).astype(np.float64)
        d = to_device(inp, dtype)
        S0d, dSd = f32(S0), f32(dS_T)
        o, S_T, _ = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d["b"], S0=S0d)
        g = carve.bwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], b=d["b"], S0=S0d, dS_T=dSd)
        o2, S_T2, saved = carve.fwd_save(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d["b"], S0=S0d)
        g2 = carve.bwd_saved(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], saved, b=d["b"], dS_T=dSd)
        torch.cuda.synchronize()
        ro, rS, _ = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], b=inp["b"], S0=S0)
        ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], inp["dO"], b=inp["b"], S0=S0,
                              dS_T=dS_T)
        errs = {"o": max_rel(to_np(o), ro), "S_T": max_rel(to_np(S_T), rS)}
        errs.update({k_: max_rel(to_np(g[k_]), ref[k_]) for k_ in NAMES})
        bad = {k_: v_ for k_, v_ in errs.items() if not v_ <= TOL[dtype]}
        assert not bad, (T, bad)
        assert torch.equal(o2, o) and torch.equal(S_T2, S_T), T
        for k_ in NAMES:
            assert torch.equal(g2[k_], g[k_]), (T, k_)
        for k_, v_ in errs.items():
            worst[k_] = max(worst.get(k_, 0.0), v_)
    print("  worst over T: " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in worst.items()), flush=True)


@pytest.mark.parametrize("dtype,D,L", [("bf16", 128, 64), ("f32", 64, 32)])
def test_content_token_count_sweep(dtype, D, L):
    """Content-aware forward and backward with T on, just before and just after the first
    and second period ends (the mean of a ragged last period is over its own tokens)."""
    print(f"\n[case] content token sweep {dtype} D{D} L{L}", flush=True)
    B, H = 1, 2
    worst = {}
    for T in (1, L - 1, L, L + 1, 2 * L - 1, 2 * L, 2 * L + 1):
        inp = random_inputs(B, H, T, D, D, dtype=dtype, seed=3000 + T, erase="content", dists="softplus_decay",
                            with_dO=True)
        inp["U1"] = inp["U1"] * 8.0
        inp["U2"] = inp["U2"] * 8.0
        rng = np.random.default_rng(3100 + T)
        m0 = np.asarray(rng.standard_normal((B, H, D)) * 0.5, np.float32).astype(np.float64)
        dm_out = np.asarray(rng.standard_normal((B, H, D)), np.float32).astype(np.float64)
        d = to_device(inp, dtype)
        cont = {"b_x": d["b_x"], "U1": d["U1"], "U2": d["U2"], "m0": f32(m0)}
        o, S_T, m_out = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], L=L, content=cont)
        g = carve.bwd_content(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], cont, dm_out=f32(dm_out), L=L)
        torch.cuda.synchronize()
        rc = {"b_x": inp["b_x"], "U1": inp["U1"], "U2": inp["U2"], "m0": m0}
        ro, rS, rm = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], L=L, content=rc)
        ref = oracle.backward_content(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], inp["dO"], rc,
                                      dm_out=dm_out, L=L)
        errs = {"o": max_rel(to_np(o), ro), "S_T": max_rel(to_np(S_T), rS), "m_out": max_rel(to_np(m_out), rm)}
        errs.update({k_: max_rel(to_np(g[k_]), ref[k_])
                     for k_ in ("dq", "dk", "dv", "dlog_g", "db_x", "dw", "dU1", "dU2", "dm0")})
        bad = {k_: v_ for k_, v_ in errs.items() if not v_ <= TOL[dtype]}
        assert not bad, (T, bad)
        for k_, v_ in errs.items():
            worst[k_] = max(worst.get(k_, 0.0), v_)
    print("  worst over T: " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in worst.items()), flush=True)
