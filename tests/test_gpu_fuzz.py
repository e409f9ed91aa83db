"""Seeded random configurations against the float64 oracle (needs an MI355X).  Each case
draws batch, heads, token count, both head widths, dtype, chunk length, erase mode, gate
distribution, an initial state and the call pair at random, so combinations that no
hand-written case names (a ragged tail with unequal widths and L = 16, a one-token
sequence with a content projection of rank 64, ...) meet the same bars: 1e-4 for float32
inputs, 2e-2 for bfloat16, max-normalised per tensor.  The configurations are printed
before each call."""
import numpy as np
import pytest
import torch

import oracle
from chunk_gated_delta_amd import carve
from chunk_gated_delta_amd.synth import random_inputs
from tests.helpers import hard_runs, max_rel, to_device, to_np

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}


def f32(x):
    return None if x is None else torch.from_numpy(np.asarray(x, np.float32)).cuda()


def draw_case(rng):
    c = dict(B=int(rng.integers(1, 4)), H=int(rng.integers(1, 4)), T=int(rng.integers(1, 301)),
             Dk=int(rng.choice([64, 128])), Dv=int(rng.choice([64, 128])), dtype=str(rng.choice(["bf16", "f32"])),
             L=int(rng.choice([16, 32, 64, 128])), erase=str(rng.choice(["none", "ones", "sigmoid"])),
             dists=str(rng.choice(["softplus_decay", "uniform_decay"])), state=bool(rng.integers(0, 2)),
             pair=str(rng.choice(["recompute", "saved"])))
    return c


@pytest.mark.parametrize("seed", range(4))
def test_random_token_configs(seed):
    rng = np.random.default_rng(5000 + seed)
    for i in range(10):
        c = draw_case(rng)
        print(f"\n[case] seed {seed} #{i}: {c}", flush=True)
        B, H, T, Dk, Dv, dtype = c["B"], c["H"], c["T"], c["Dk"], c["Dv"], c["dtype"]
        inp = random_inputs(B, H, T, Dk, Dv, dtype=dtype, seed=int(rng.integers(1 << 30)), erase=c["erase"],
                            dists=c["dists"], with_dO=True)
        S0 = dS_T = None
        if c["state"]:
            S0 = np.asarray(rng.standard_normal((B, H, Dv, Dk)) * 0.3, np.float32).astype(np.float64)
            dS_T = np.asarray(rng.standard_normal((B, H, Dv, Dk)) * 0.3, np.float32).astype(np.float64)
        d = to_device(inp, dtype)
        b = d.get("b")
        if c["pair"] == "saved":
            o, S_T, saved = carve.fwd_save(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=b, S0=f32(S0), L=c["L"])
            g = carve.bwd_saved(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], saved, b=b, dS_T=f32(dS_T),
                                L=c["L"])
        else:
            o, S_T, _ = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=b, S0=f32(S0), L=c["L"])
            g = carve.bwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], b=b, S0=f32(S0), dS_T=f32(dS_T),
                          L=c["L"])
        torch.cuda.synchronize()
        ro, rS, _ = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], b=inp.get("b"), S0=S0)
        ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], inp["dO"], b=inp.get("b"),
                              S0=S0, dS_T=dS_T)
        errs = {"o": max_rel(to_np(o), ro), "S_T": max_rel(to_np(S_T), rS)}
        for key in ("dq", "dk", "dv", "dlog_g", "db", "dw", "dS0"):
            if ref[key] is None or g[key] is None:
                assert (ref[key] is None) == (g[key] is None), key
                continue
            errs[key] = max_rel(to_np(g[key]), ref[key])
        print("  " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
        assert all(v_ <= TOL[dtype] for v_ in errs.values()), (c, errs)


@pytest.mark.parametrize("seed", range(2))
def test_random_content_configs(seed):
    rng = np.random.default_rng(6000 + seed)
    for i in range(8):
        dtype = str(rng.choice(["bf16", "f32"]))
        L = int(rng.choice([32, 64, 128]))
        c = dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 3)), T=int(rng.integers(1, 301)),
                 Dk=int(rng.choice([64, 128])), Dv=int(rng.choice([64, 128])), dtype=dtype, L=L,
                 R=int(rng.choice([1, 16, 64])), proj=bool(rng.integers(0, 4) > 0), m0=bool(rng.integers(0, 2)))
        print(f"\n[case] content seed {seed} #{i}: {c}", flush=True)
        B, H, T, Dk, Dv = c["B"], c["H"], c["T"], c["Dk"], c["Dv"]
        inp = random_inputs(B, H, T, Dk, Dv, dtype=dtype, seed=int(rng.integers(1 << 30)), erase="content",
                            dists="softplus_decay", with_dO=True, rank=c["R"])
        inp["U1"] = inp["U1"] * 8.0
        inp["U2"] = inp["U2"] * 8.0
        m0 = np.asarray(rng.standard_normal((B, H, Dv)) * 0.5, np.float32).astype(np.float64) if c["m0"] else None
        dm_out = np.asarray(rng.standard_normal((B, H, Dv)), np.float32).astype(np.float64)
        d = to_device(inp, dtype)
        U1, U2 = (d["U1"], d["U2"]) if c["proj"] else (None, None)
        cont = {"b_x": d["b_x"], "U1": U1, "U2": U2, "m0": f32(m0)}
        o, S_T, m_out = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], L=L, content=cont)
        g = carve.bwd_content(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], cont, dm_out=f32(dm_out), L=L)
        torch.cuda.synchronize()
        rc = {"b_x": inp["b_x"], "U1": inp["U1"] if c["proj"] else None, "U2": inp["U2"] if c["proj"] else None,
              "m0": m0}
        ro, rS, rm = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], L=L, content=rc)
        ref = oracle.backward_content(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], inp["dO"], rc,
                                      dm_out=dm_out, L=L)
        errs = {"o": max_rel(to_np(o), ro), "S_T": max_rel(to_np(S_T), rS), "m_out": max_rel(to_np(m_out), rm)}
        for key in ("dq", "dk", "dv", "dlog_g", "db_x", "dw", "dU1", "dU2", "dm0"):
            if ref.get(key) is None or g.get(key) is None:
                continue
            errs[key] = max_rel(to_np(g[key]), ref[key])
        print("  " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
        assert all(v_ <= TOL[dtype] for v_ in errs.values()), (c, errs)


@pytest.mark.parametrize("seed", range(2))
def test_random_hard_range_configs(seed):
    """Random shapes over the whole retention range: runs of hard erase (b down to 1e-6) and
    bursts of strong decay (log g down to -40 per token) on a random share of key channels,
    so tiles take the range-safe path and blocks beyond -64 the exact fix-up.  The erase
    gradient is compared where b >= 0.25 (it is ill-conditioned below), d/dlog g everywhere."""
    rng = np.random.default_rng(7000 + seed)
    for i in range(8):
        c = dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 3)), T=int(rng.integers(20, 301)),
                 Dk=int(rng.choice([64, 128])), Dv=int(rng.choice([64, 128])), dtype=str(rng.choice(["bf16", "f32"])),
                 L=int(rng.choice([32, 64])), frac=float(rng.uniform(0.05, 0.5)),
                 pair=str(rng.choice(["recompute", "saved"])))
        print(f"\n[case] hard seed {seed} #{i}: {c}", flush=True)
        B, H, T, Dk, Dv, dtype = c["B"], c["H"], c["T"], c["Dk"], c["Dv"], c["dtype"]
        inp = random_inputs(B, H, T, Dk, Dv, dtype=dtype, seed=int(rng.integers(1 << 30)), erase="sigmoid",
                            dists="softplus_decay", with_dO=True)
        m1, burst = hard_runs(rng, B, H, T, Dk, c["frac"], 2.0, 40.0)
        m2, tiny = hard_runs(rng, B, H, T, Dk, c["frac"], 1e-6, 1e-2)
        inp["log_g"] = np.asarray(np.where(m1, -burst, inp["log_g"]), np.float32).astype(np.float64)
        inp["b"] = np.asarray(np.where(m2, tiny, inp["b"]), np.float32).astype(np.float64)
        S0 = np.asarray(rng.standard_normal((B, H, Dv, Dk)) * 0.3, np.float32).astype(np.float64)
        dS_T = np.asarray(rng.standard_normal((B, H, Dv, Dk)) * 0.3, np.float32).astype(np.float64)
        d = to_device(inp, dtype)
        if c["pair"] == "saved":
            o, S_T, saved = carve.fwd_save(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d["b"], S0=f32(S0), L=c["L"])
            g = carve.bwd_saved(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], saved, b=d["b"],
                                dS_T=f32(dS_T), L=c["L"])
        else:
            o, S_T, _ = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d["b"], S0=f32(S0), L=c["L"])
            g = carve.bwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], b=d["b"], S0=f32(S0),
                          dS_T=f32(dS_T), L=c["L"])
        torch.cuda.synchronize()
        ro, rS, _ = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], b=inp["b"], S0=S0)
        ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], inp["dO"], b=inp["b"], S0=S0,
                              dS_T=dS_T)
        errs = {"o": max_rel(to_np(o), ro), "S_T": max_rel(to_np(S_T), rS)}
        errs.update({key: max_rel(to_np(g[key]), ref[key]) for key in ("dq", "dk", "dv", "dlog_g", "dw", "dS0")})
        sel = inp["b"] >= 0.25
        errs["db(b>=0.25)"] = max_rel(to_np(g["db"])[sel], ref["db"][sel])
        print("  " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
        for key in ("dq", "dk", "dv", "dlog_g", "db", "dw"):
            assert torch.isfinite(g[key]).all().item(), key
        assert all(v_ <= TOL[dtype] for v_ in errs.values()), (c, errs)


@pytest.mark.parametrize("seed", range(2))
def test_random_logit_configs(seed):
    """Gates given as pre-activations: random shapes, widths, dtype, chunk length, amplitudes up
    to 10 (strong decay included), with and without b_x, recomputing or saved pair."""
    rng = np.random.default_rng(8000 + seed)
    for i in range(6):
        c = dict(B=int(rng.integers(1, 3)), H=int(rng.integers(1, 3)), T=int(rng.integers(1, 301)),
                 Dk=int(rng.choice([64, 128])), Dv=int(rng.choice([64, 128])), dtype=str(rng.choice(["bf16", "f32"])),
                 L=int(rng.choice([16, 32, 64, 128])), bx=bool(rng.integers(0, 2)),
                 pair=str(rng.choice(["recompute", "saved"])))
        print(f"\n[case] logits seed {seed} #{i}: {c}", flush=True)
        B, H, T, Dk, Dv, dtype = c["B"], c["H"], c["T"], c["Dk"], c["Dv"], c["dtype"]
        inp = random_inputs(B, H, T, Dk, Dv, dtype=dtype, seed=int(rng.integers(1 << 30)), erase="none",
                            with_dO=True)
        r64 = lambda x: np.asarray(x, np.float32).astype(np.float64)
        gl = {"f": r64(rng.standard_normal((B, H, T, Dk))), "A": r64(rng.uniform(0.05, 10.0, (H, Dk))),
              "tau": r64(rng.standard_normal((H, Dk)) * 0.5), "w_hat": r64(rng.standard_normal((B, H, T))),
              "b_x": r64(rng.normal(2.0, 1.0, (B, H, T, Dk))) if c["bx"] else None}
        S0 = r64(rng.standard_normal((B, H, Dv, Dk)) * 0.3)
        dS_T = r64(rng.standard_normal((B, H, Dv, Dk)) * 0.3)
        d = to_device(inp, dtype)
        args = (d["q"], d["k"], d["v"], f32(gl["f"]), f32(gl["A"]), f32(gl["tau"]), f32(gl["w_hat"]))
        if c["pair"] == "saved":
            o, S_T, saved = carve.fwd_logits_save(*args, b_x=f32(gl["b_x"]), S0=f32(S0), L=c["L"])
            g = carve.bwd_logits_saved(*args, d["dO"], saved, b_x=f32(gl["b_x"]), dS_T=f32(dS_T), L=c["L"])
        else:
            o, S_T = carve.fwd_logits(*args, b_x=f32(gl["b_x"]), S0=f32(S0), L=c["L"])
            g = carve.bwd_logits(*args, d["dO"], b_x=f32(gl["b_x"]), S0=f32(S0), dS_T=f32(dS_T), L=c["L"])
        torch.cuda.synchronize()
        ro, rS = oracle.forward_logits(inp["q"], inp["k"], inp["v"], gl["f"], gl["A"], gl["tau"], gl["w_hat"],
                                       b_x=gl["b_x"], S0=S0)
        ref = oracle.backward_logits(inp["q"], inp["k"], inp["v"], gl["f"], gl["A"], gl["tau"], gl["w_hat"],
                                     inp["dO"], b_x=gl["b_x"], S0=S0, dS_T=dS_T)
        errs = {"o": max_rel(to_np(o), ro), "S_T": max_rel(to_np(S_T), rS)}
        for key in ("dq", "dk", "dv", "df", "dA", "dtau", "db_x", "dw_hat", "dS0"):
            if ref[key] is None or g[key] is None:
                assert (ref[key] is None) == (g[key] is None), key
                continue
            errs[key] = max_rel(to_np(g[key]), ref[key])
        print("  " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
        assert all(v_ <= TOL[dtype] for v_ in errs.values()), (c, errs)


@pytest.mark.parametrize("seed", range(2))
def test_random_decode_configs(seed):
    """The recurrent decode step: random shapes and widths, token-only (with or without b) or
    content-aware (random rank and period, starting mid-chunk from a carried mean), a run of
    decode calls against the oracle forward over the same tokens."""
    rng = np.random.default_rng(9000 + seed)
    for i in range(6):
        content = bool(rng.integers(0, 2))
        c = dict(B=int(rng.integers(1, 4)), H=int(rng.integers(1, 4)), T=int(rng.integers(1, 40)),
                 Dk=int(rng.choice([64, 128])), Dv=int(rng.choice([64, 128])), dtype=str(rng.choice(["bf16", "f32"])),
                 content=content, L=int(rng.choice([4, 8, 16])), R=int(rng.choice([1, 16, 64])),
                 erase=str(rng.choice(["none", "sigmoid"])))
        print(f"\n[case] decode seed {seed} #{i}: {c}", flush=True)
        B, H, T, Dk, Dv, dtype, L = c["B"], c["H"], c["T"], c["Dk"], c["Dv"], c["dtype"], c["L"]
        inp = random_inputs(B, H, T, Dk, Dv, dtype=dtype, seed=int(rng.integers(1 << 30)),
                            erase="content" if content else c["erase"], dists="softplus_decay", rank=c["R"])
        if content:
            inp["U1"] = inp["U1"] * 8.0
            inp["U2"] = inp["U2"] * 8.0
        d = to_device(inp, dtype)
        S0 = np.asarray(rng.standard_normal((B, H, Dv, Dk)) * 0.3, np.float32).astype(np.float64)
        S = f32(S0)
        m0 = np.asarray(rng.standard_normal((B, H, Dv)) * 0.5, np.float32).astype(np.float64)
        carry = {"U1": d["U1"], "U2": d["U2"], "m_in": f32(m0),
                 "csum": torch.zeros((B, H, Dv), dtype=torch.float32, device="cuda"), "pos": 0} if content else None
        outs = []
        for t in range(T):
            tok = {key: d[key][:, :, t].contiguous() for key in ("q", "k", "v", "log_g", "w")}
            cont = dict(carry, b_x=d["b_x"][:, :, t].contiguous()) if content else None
            b = d["b"][:, :, t].contiguous() if (not content and "b" in d) else None
            o_t, m_out = carve.decode_step(tok["q"], tok["k"], tok["v"], tok["log_g"], tok["w"], S, b=b, L=L,
                                           content=cont)
            outs.append(o_t)
            if content:
                carry["m_in"] = m_out
                carry["pos"] = (carry["pos"] + 1) % L
        torch.cuda.synchronize()
        o = torch.stack(outs, dim=2)
        rc = {"b_x": inp["b_x"], "U1": inp["U1"], "U2": inp["U2"], "m0": m0} if content else None
        ro, rS, _ = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], b=inp.get("b"), S0=S0,
                                   L=L, content=rc)
        errs = {"o": max_rel(to_np(o), ro), "S": max_rel(to_np(S), rS)}
        print("  " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
        assert all(v_ <= TOL[dtype] for v_ in errs.values()), (c, errs)
