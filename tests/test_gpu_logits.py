"""GPU parity of the forward and backward with gates given as pre-activations
(needs an MI355X): log g = -A softplus(f + tau), b = sigmoid(b_x), w = sigmoid(w_hat)
activated inside the kernels, compared with the float64 reference (itself pinned by
finite differences).  Error metric: max|gpu - ref| / max|ref| per tensor; bars 1e-4
(float32 inputs) and 2e-2 (bfloat16 inputs)."""
import numpy as np
import pytest
import torch

import oracle
from chunk_gated_delta_amd import carve
from chunk_gated_delta_amd.synth import random_inputs
from tests.helpers import max_rel, to_device, to_np

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}


def announce(name):
    print(f"\n[case] {name}", flush=True)


def f32np(x):
    return np.asarray(x, np.float32).astype(np.float64)


def logit_case(B, H, T, D, dtype, seed, with_bx=True):
    inp = random_inputs(B, H, T, D, D, dtype=dtype, seed=seed, erase="none", with_dO=True)
    rng = np.random.default_rng(seed + 7)
    inp["f"] = f32np(rng.standard_normal((B, H, T, D)))
    inp["A"] = f32np(rng.uniform(0.05, 10.0, (H, D)))   # amplitudes up to 10: strong decay included
    inp["tau"] = f32np(rng.standard_normal((H, D)) * 0.5)
    inp["w_hat"] = f32np(rng.standard_normal((B, H, T)))
    inp["b_x"] = f32np(rng.normal(2.0, 1.0, (B, H, T, D))) if with_bx else None
    inp["S0"] = f32np(rng.standard_normal((B, H, D, D)) * 0.3)
    inp["dS_T"] = f32np(rng.standard_normal((B, H, D, D)) * 0.3)
    return inp


def dev(x):
    return None if x is None else torch.from_numpy(np.asarray(x, np.float32)).cuda()


CASES = [("f32", 1, 2, 100, 64, True), ("bf16", 2, 2, 200, 128, True), ("bf16", 1, 2, 130, 128, False),
         ("f32", 2, 1, 64, 128, False)]
IDS = [f"{c[0]}_T{c[3]}_d{c[4]}_{'bx' if c[5] else 'nob'}" for c in CASES]


@pytest.mark.parametrize("dtype,B,H,T,D,with_bx", CASES, ids=IDS)
def test_fwd_logits_parity(dtype, B, H, T, D, with_bx):
    announce(f"fwd logits {dtype} T{T} d{D} b_x={with_bx}")
    inp = logit_case(B, H, T, D, dtype, seed=500 + T + D, with_bx=with_bx)
    d = to_device(inp, dtype)
    o, S_T = carve.fwd_logits(d["q"], d["k"], d["v"], dev(inp["f"]), dev(inp["A"]), dev(inp["tau"]),
                              dev(inp["w_hat"]), b_x=dev(inp["b_x"]), S0=dev(inp["S0"]))
    torch.cuda.synchronize()
    ro, rS = oracle.forward_logits(inp["q"], inp["k"], inp["v"], inp["f"], inp["A"], inp["tau"], inp["w_hat"],
                                   b_x=inp["b_x"], S0=inp["S0"])
    eo, es = max_rel(to_np(o), ro), max_rel(to_np(S_T), rS)
    print(f"  err o={eo:.2e} S_T={es:.2e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("dtype,B,H,T,D,with_bx", CASES, ids=IDS)
def test_bwd_logits_parity(dtype, B, H, T, D, with_bx):
    announce(f"bwd logits {dtype} T{T} d{D} b_x={with_bx}")
    inp = logit_case(B, H, T, D, dtype, seed=600 + T + D, with_bx=with_bx)
    d = to_device(inp, dtype)
    g = carve.bwd_logits(d["q"], d["k"], d["v"], dev(inp["f"]), dev(inp["A"]), dev(inp["tau"]), dev(inp["w_hat"]),
                         d["dO"], b_x=dev(inp["b_x"]), S0=dev(inp["S0"]), dS_T=dev(inp["dS_T"]))
    torch.cuda.synchronize()
    ref = oracle.backward_logits(inp["q"], inp["k"], inp["v"], inp["f"], inp["A"], inp["tau"], inp["w_hat"],
                                 inp["dO"], b_x=inp["b_x"], S0=inp["S0"], dS_T=inp["dS_T"])
    errs = {}
    for key in ("dq", "dk", "dv", "df", "dA", "dtau", "db_x", "dw_hat", "dS0"):
        if ref[key] is None:
            assert g[key] is None
            continue
        errs[key] = max_rel(to_np(g[key]), ref[key])
    print("  " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
    assert all(v_ <= TOL[dtype] for v_ in errs.values()), errs


def test_fwd_logits_segmented_long_memory():
    """Few heads, many chunks: the gate pre-activation forward runs the segmented state
    pass too.  Slow decay (A small, f + tau very negative) and a small write gate keep
    the carried state alive across segments."""
    announce("fwd logits segmented, long memory")
    B, H, T, D = 1, 2, 64 * 80 + 3, 128
    inp = logit_case(B, H, T, D, "bf16", seed=901, with_bx=False)
    rng = np.random.default_rng(902)
    inp["A"] = f32np(rng.uniform(0.001, 0.01, (H, D)))
    inp["tau"] = f32np(np.full((H, D), -3.0))
    inp["w_hat"] = f32np(rng.normal(-4.0, 0.5, (B, H, T)))
    d = to_device(inp, "bf16")
    o, S_T = carve.fwd_logits(d["q"], d["k"], d["v"], dev(inp["f"]), dev(inp["A"]), dev(inp["tau"]),
                              dev(inp["w_hat"]), S0=dev(inp["S0"]))
    torch.cuda.synchronize()
    ro, rS = oracle.forward_logits(inp["q"], inp["k"], inp["v"], inp["f"], inp["A"], inp["tau"], inp["w_hat"],
                                   S0=inp["S0"])
    ro0, _ = oracle.forward_logits(inp["q"], inp["k"], inp["v"], inp["f"], inp["A"], inp["tau"], inp["w_hat"])
    carried = max_rel(ro0[:, :, -64:], ro[:, :, -64:])
    eo, es = max_rel(to_np(o), ro), max_rel(to_np(S_T), rS)
    print(f"  err o={eo:.2e} S_T={es:.2e}; S0's share of the last chunk's outputs {carried:.2e}", flush=True)
    assert carried > 0.1
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]


def test_logits_match_activated_gates():
    """The fused activation agrees with passing the activated gates (computed in
    float32 on the device) to the plain entry points, within the bf16 bar."""
    announce("logits vs activated gates")
    inp = logit_case(2, 2, 256, 128, "bf16", seed=700)
    d = to_device(inp, "bf16")
    f, A, tau, wh, bx = (dev(inp[k_]) for k_ in ("f", "A", "tau", "w_hat", "b_x"))
    log_g = -A[None, :, None, :] * torch.nn.functional.softplus(f + tau[None, :, None, :])
    b, w = torch.sigmoid(bx), torch.sigmoid(wh)
    o1, S1 = carve.fwd_logits(d["q"], d["k"], d["v"], f, A, tau, wh, b_x=bx)
    o2, S2, _ = carve.fwd(d["q"], d["k"], d["v"], log_g.contiguous(), w.contiguous(), b=b.contiguous())
    torch.cuda.synchronize()
    assert max_rel(to_np(o1), to_np(o2)) <= 2e-2 and max_rel(to_np(S1), to_np(S2)) <= 2e-2


def test_logits_single_token_and_empty():
    announce("logits T1 and T0")
    inp = logit_case(1, 2, 1, 128, "bf16", seed=801)
    d = to_device(inp, "bf16")
    g = carve.bwd_logits(d["q"], d["k"], d["v"], dev(inp["f"]), dev(inp["A"]), dev(inp["tau"]), dev(inp["w_hat"]),
                         d["dO"], b_x=dev(inp["b_x"]), S0=dev(inp["S0"]), dS_T=dev(inp["dS_T"]))
    torch.cuda.synchronize()
    ref = oracle.backward_logits(inp["q"], inp["k"], inp["v"], inp["f"], inp["A"], inp["tau"], inp["w_hat"],
                                 inp["dO"], b_x=inp["b_x"], S0=inp["S0"], dS_T=inp["dS_T"])
    for key in ("dq", "dk", "dv", "df", "dA", "dtau", "db_x", "dw_hat", "dS0"):
        assert max_rel(to_np(g[key]), ref[key]) <= TOL["bf16"], key
    # no tokens: S_T = S0, and the amplitude / bias gradients are zero
    z = torch.zeros((1, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    zf = torch.zeros((1, 2, 0, 128), dtype=torch.float32, device="cuda")
    S0 = dev(inp["S0"])
    o, S_T = carve.fwd_logits(z, z, z, zf, dev(inp["A"]), dev(inp["tau"]), torch.zeros((1, 2, 0), device="cuda"),
                              S0=S0)
    torch.cuda.synchronize()
    assert torch.equal(S_T, S0)


# ---------------------------------------------------------------- training pair
def saved_pair(d, inp):
    o, S_T, saved = carve.fwd_logits_save(d["q"], d["k"], d["v"], dev(inp["f"]), dev(inp["A"]), dev(inp["tau"]),
                                          dev(inp["w_hat"]), b_x=dev(inp["b_x"]), S0=dev(inp["S0"]))
    g = carve.bwd_logits_saved(d["q"], d["k"], d["v"], dev(inp["f"]), dev(inp["A"]), dev(inp["tau"]),
                               dev(inp["w_hat"]), d["dO"], saved, b_x=dev(inp["b_x"]), dS_T=dev(inp["dS_T"]))
    return o, S_T, g


GRADS = ("dq", "dk", "dv", "df", "dA", "dtau", "db_x", "dw_hat", "dS0")


@pytest.mark.parametrize("dtype,B,H,T,D,with_bx", CASES, ids=IDS)
def test_logits_saved_pair_matches_recompute_bitwise(dtype, B, H, T, D, with_bx):
    """fwd_logits_save gives the bits of fwd_logits, and bwd_logits_saved those of
    bwd_logits (the same arithmetic; only the forward is not recomputed)."""
    announce(f"logits saved pair vs recompute {dtype} T{T} d{D} b_x={with_bx}")
    inp = logit_case(B, H, T, D, dtype, seed=700 + T + D, with_bx=with_bx)
    d = to_device(inp, dtype)
    o1, s1 = carve.fwd_logits(d["q"], d["k"], d["v"], dev(inp["f"]), dev(inp["A"]), dev(inp["tau"]),
                              dev(inp["w_hat"]), b_x=dev(inp["b_x"]), S0=dev(inp["S0"]))
    g1 = carve.bwd_logits(d["q"], d["k"], d["v"], dev(inp["f"]), dev(inp["A"]), dev(inp["tau"]), dev(inp["w_hat"]),
                          d["dO"], b_x=dev(inp["b_x"]), S0=dev(inp["S0"]), dS_T=dev(inp["dS_T"]))
    o2, s2, g2 = saved_pair(d, inp)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    for key in GRADS:
        if g1[key] is None:
            assert g2[key] is None
            continue
        assert torch.equal(g1[key], g2[key]), key


def test_logits_saved_pair_segmented_parity():
    """Few heads, 40 chunks: the saved pair runs its forward and reverse state passes as
    segments; every output and gradient against the reference."""
    announce("logits saved pair, segmented, bf16 B1 H2 T2560 d128")
    inp = logit_case(1, 2, 64 * 40, 128, "bf16", seed=720, with_bx=True)
    d = to_device(inp, "bf16")
    o, S_T, g = saved_pair(d, inp)
    torch.cuda.synchronize()
    ro, rS = oracle.forward_logits(inp["q"], inp["k"], inp["v"], inp["f"], inp["A"], inp["tau"], inp["w_hat"],
                                   b_x=inp["b_x"], S0=inp["S0"])
    ref = oracle.backward_logits(inp["q"], inp["k"], inp["v"], inp["f"], inp["A"], inp["tau"], inp["w_hat"],
                                 inp["dO"], b_x=inp["b_x"], S0=inp["S0"], dS_T=inp["dS_T"])
    errs = {"o": max_rel(to_np(o), ro), "S_T": max_rel(to_np(S_T), rS)}
    errs.update({key: max_rel(to_np(g[key]), ref[key]) for key in GRADS})
    print("  " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
    assert all(v_ <= TOL["bf16"] for v_ in errs.values()), errs
