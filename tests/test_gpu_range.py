"""GPU parity over the whole retention range (needs an MI355X).

The gates of these cases reach far beyond the workloads' mild decay: hard erase
(b down to 1e-6 held over runs of tokens), bursts of strong decay (log g down to -40
per token) and gate pre-activations with amplitudes up to 10, so that a key channel's
log-retention over one 64-token tile falls to about -500 and below.  The pages put no
floor on the decay (log g <= 0) and define the erase as a factor in (0, 1] (CARVE
notes, section 2.1 CARVE-update legend, section 2.3 decay legend).  Every path is
compared element-wise with the float64 reference: forward, backward, the training
pair, the content-aware forward and backward, and the gates as pre-activations.
Bars 2e-2 (bfloat16 inputs) and 1e-4 (float32 inputs), max|gpu - ref| / max|ref| per
tensor.

The erase gradient d/db = d/dlog g / b is ill-conditioned where b is small: it carries
the absolute error of d/dlog g divided by b.  It is compared where b >= 0.25; d/dlog g
(which equals b * d/db) is compared everywhere, and so are the well-conditioned
pre-activation gradients d/db_x = d/dlog g (1 - b) of the content and logit paths.
"""
import numpy as np
import pytest
import torch

import oracle
from chunk_gated_delta_amd import carve
from chunk_gated_delta_amd.synth import random_inputs
from tests.helpers import hard_runs, max_rel, to_device, to_np

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}


def announce(name):
    print(f"\n[case] {name}", flush=True)


def f32np(x):
    return np.asarray(x, np.float32).astype(np.float64)


def dev(x):
    return None if x is None else torch.from_numpy(np.asarray(x, np.float32)).cuda()


def hard_case(B, H, T, D, dtype, seed, erase=True):
    """Workload-shaped inputs with runs of hard erase and bursts of strong decay."""
    inp = random_inputs(B, H, T, D, D, dtype=dtype, seed=seed, erase="sigmoid" if erase else "none",
                        dists="softplus_decay", with_dO=True)
    rng = np.random.default_rng(seed + 11)
    m1, burst = hard_runs(rng, B, H, T, D, 0.3, 2.0, 40.0)
    inp["log_g"] = f32np(np.where(m1, -burst, inp["log_g"]))
    if erase:
        m2, tiny = hard_runs(rng, B, H, T, D, 0.3, 1e-6, 1e-2)
        inp["b"] = f32np(np.where(m2, tiny, inp["b"]))
    la = inp["log_g"] + (np.log(inp["b"]) if erase else 0.0)
    ntile = T // 64
    if ntile:
        per_tile = la[:, :, :64 * ntile].reshape(B, H, ntile, 64, D).sum(axis=3)
        assert per_tile.min() < -500, per_tile.min()      # the range these cases are for
    S0 = f32np(rng.standard_normal((B, H, D, D)) * 0.3)
    dS_T = f32np(rng.standard_normal((B, H, D, D)) * 0.3)
    return inp, S0, dS_T


CASES = [
    # dtype, B, H, T, D, L, erase
    ("bf16", 1, 2, 300, 128, 64, True),
    ("bf16", 2, 1, 200, 64, 64, True),
    ("bf16", 1, 2, 256, 128, 32, False),
    ("f32", 1, 2, 150, 64, 64, True),
    ("f32", 1, 1, 130, 128, 64, True),
]
IDS = [f"{c[0]}_T{c[3]}_d{c[4]}_L{c[5]}_{'b' if c[6] else 'nob'}" for c in CASES]


@pytest.mark.parametrize("dtype,B,H,T,D,L,erase", CASES, ids=IDS)
def test_fwd_hard_range(dtype, B, H, T, D, L, erase):
    announce(f"fwd hard range {dtype} B{B} H{H} T{T} d{D} L{L} erase={erase}")
    inp, S0, _ = hard_case(B, H, T, D, dtype, seed=1200 + T + D, erase=erase)
    d = to_device(inp, dtype)
    o, S_T, _ = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d.get("b"), S0=dev(S0), L=L)
    torch.cuda.synchronize()
    ro, rS, _ = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], b=inp.get("b"), S0=S0)
    eo, es = max_rel(to_np(o), ro), max_rel(to_np(S_T), rS)
    print(f"  err o={eo:.2e} S_T={es:.2e}", flush=True)
    assert np.all(np.isfinite(to_np(o)))
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def check_grads(g, ref, b, tol):
    errs = {}
    for key in ("dq", "dk", "dv", "dlog_g", "dw", "dS0"):
        errs[key] = max_rel(g[key], ref[key])
    if b is not None:
        sel = b >= 0.25
        errs["db(b>=0.25)"] = max_rel(g["db"][sel], ref["db"][sel])
    print("  " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
    for key in g:
        if g[key] is not None:
            assert np.all(np.isfinite(g[key])), key
    assert all(v_ <= tol for v_ in errs.values()), errs


@pytest.mark.parametrize("dtype,B,H,T,D,L,erase", CASES, ids=IDS)
def test_bwd_hard_range(dtype, B, H, T, D, L, erase):
    announce(f"bwd hard range {dtype} B{B} H{H} T{T} d{D} L{L} erase={erase}")
    inp, S0, dS_T = hard_case(B, H, T, D, dtype, seed=1300 + T + D, erase=erase)
    d = to_device(inp, dtype)
    g = carve.bwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], b=d.get("b"), S0=dev(S0), dS_T=dev(dS_T),
                  L=L)
    torch.cuda.synchronize()
    g = {k_: (None if v_ is None else to_np(v_)) for k_, v_ in g.items()}
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], inp["dO"], b=inp.get("b"),
                          S0=S0, dS_T=dS_T)
    check_grads(g, ref, inp.get("b"), TOL[dtype])


def test_training_pair_hard_range():
    """fwd_save + bwd_saved (the benchmarked pair) over the hard range."""
    announce("training pair hard range bf16 B2 H2 T320 d128")
    B, H, T, D = 2, 2, 320, 128
    inp, S0, dS_T = hard_case(B, H, T, D, "bf16", seed=1401)
    d = to_device(inp, "bf16")
    o, S_T, saved = carve.fwd_save(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d["b"], S0=dev(S0))
    g = carve.bwd_saved(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], saved, b=d["b"], dS_T=dev(dS_T))
    torch.cuda.synchronize()
    ro, rS, _ = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], b=inp["b"], S0=S0)
    assert max_rel(to_np(o), ro) <= TOL["bf16"] and max_rel(to_np(S_T), rS) <= TOL["bf16"]
    g = {k_: (None if v_ is None else to_np(v_)) for k_, v_ in g.items()}
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], inp["dO"], b=inp["b"], S0=S0,
                          dS_T=dS_T)
    check_grads(g, ref, inp["b"], TOL["bf16"])


def test_mild_blocks_unchanged_by_hard_chunks():
    """A head whose gates are mild gives the same outputs and gradients whether or not
    another head of the same call needs the exact within-block terms."""
    announce("mild head beside a hard head")
    B, H, T, D = 1, 2, 192, 128
    inp, S0, dS_T = hard_case(B, H, T, D, "bf16", seed=1501)
    mild = random_inputs(B, H, T, D, D, dtype="bf16", seed=1502, erase="sigmoid", dists="softplus_decay",
                         with_dO=True)
    for key in ("log_g", "b"):
        inp[key][:, 1] = mild[key][:, 1]
    d = to_device(inp, "bf16")
    g = carve.bwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], b=d["b"], S0=dev(S0), dS_T=dev(dS_T))
    d1 = {k_: v_[:, 1:2].contiguous() for k_, v_ in d.items()}
    g1 = carve.bwd(d1["q"], d1["k"], d1["v"], d1["log_g"], d1["w"], d1["dO"], b=d1["b"], S0=dev(S0[:, 1:2]),
                   dS_T=dev(dS_T[:, 1:2]))
    torch.cuda.synchronize()
    for key in ("dq", "dk", "dv", "dlog_g", "db", "dw"):
        assert torch.equal(g[key][:, 1:2], g1[key]), key


def content_hard(B, H, T, D, dtype, seed, scale):
    inp = random_inputs(B, H, T, D, D, dtype=dtype, seed=seed, erase="content", dists="softplus_decay",
                        with_dO=True)
    rng = np.random.default_rng(seed + 3)
    m, tiny = hard_runs(rng, B, H, T, D, 0.3, 1e-6, 1e-2)
    inp["b_x"] = f32np(np.where(m, np.log(tiny), inp["b_x"]))   # sigmoid(log b) ~ b for small b
    inp["U1"] = inp["U1"] * scale
    inp["U2"] = inp["U2"] * scale
    ex = {"m0": f32np(rng.standard_normal((B, H, D)) * 0.5),
          "S0": f32np(rng.standard_normal((B, H, D, D)) * 0.3),
          "dS_T": f32np(rng.standard_normal((B, H, D, D)) * 0.3),
          "dm_out": f32np(rng.standard_normal((B, H, D)))}
    return inp, ex


CONTENT_CASES = [("bf16", 2, 2, 256, 128, 64, 64.0), ("f32", 1, 2, 160, 64, 32, 64.0), ("bf16", 1, 2, 200, 64, 64, 64.0),
                 ("f32", 1, 2, 200, 64, 64, 200.0)]


@pytest.mark.parametrize("dtype,B,H,T,D,L,scale", CONTENT_CASES,
                         ids=[f"{c[0]}_T{c[3]}_d{c[4]}_L{c[5]}_s{int(c[6])}" for c in CONTENT_CASES])
def test_content_hard_range(dtype, B, H, T, D, L, scale):
    announce(f"content hard range {dtype} B{B} H{H} T{T} d{D} L{L} projection x{scale}")
    inp, ex = content_hard(B, H, T, D, dtype, seed=1600 + T + D, scale=scale)
    d = to_device(inp, dtype)
    content = {"b_x": d["b_x"], "U1": d["U1"], "U2": d["U2"], "m0": dev(ex["m0"])}
    o, S_T, m_out = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], S0=dev(ex["S0"]), L=L, content=content)
    g = carve.bwd_content(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], content, S0=dev(ex["S0"]),
                          dS_T=dev(ex["dS_T"]), dm_out=dev(ex["dm_out"]), L=L)
    torch.cuda.synchronize()
    rc = {"b_x": inp["b_x"], "U1": inp["U1"], "U2": inp["U2"], "m0": ex["m0"]}
    ro, rS, rm = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], S0=ex["S0"], L=L, content=rc)
    errs = {"o": max_rel(to_np(o), ro), "S_T": max_rel(to_np(S_T), rS), "m_out": max_rel(to_np(m_out), rm)}
    ref = oracle.backward_content(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], inp["dO"], rc,
                                  S0=ex["S0"], dS_T=ex["dS_T"], dm_out=ex["dm_out"], L=L)
    for key in ("dq", "dk", "dv", "dlog_g", "db_x", "dw", "dU1", "dU2", "dm0", "dS0"):
        errs[key] = max_rel(to_np(g[key]), ref[key])
    print("  " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
    assert all(v_ <= TOL[dtype] for v_ in errs.values()), errs


LOGIT_CASES = [("bf16", 2, 2, 256, 128, True), ("f32", 1, 2, 130, 64, True), ("bf16", 1, 2, 200, 128, False)]


@pytest.mark.parametrize("dtype,B,H,T,D,with_bx", LOGIT_CASES,
                         ids=[f"{c[0]}_T{c[3]}_d{c[4]}_{'bx' if c[5] else 'nob'}" for c in LOGIT_CASES])
def test_logits_hard_range(dtype, B, H, T, D, with_bx):
    """Amplitudes up to 10 and wide logits: per-token log-retention down to about -40."""
    announce(f"logits hard range {dtype} B{B} H{H} T{T} d{D} b_x={with_bx}")
    inp = random_inputs(B, H, T, D, D, dtype=dtype, seed=1700 + T + D, erase="none", with_dO=True)
    rng = np.random.default_rng(1701 + T)
    inp["f"] = f32np(rng.normal(0.0, 2.0, (B, H, T, D)))
    inp["A"] = f32np(rng.uniform(0.05, 10.0, (H, D)))
    inp["tau"] = f32np(rng.standard_normal((H, D)))
    inp["w_hat"] = f32np(rng.standard_normal((B, H, T)))
    inp["b_x"] = f32np(rng.normal(0.0, 4.0, (B, H, T, D))) if with_bx else None
    S0 = f32np(rng.standard_normal((B, H, D, D)) * 0.3)
    dS_T = f32np(rng.standard_normal((B, H, D, D)) * 0.3)
    d = to_device(inp, dtype)
    o, S_T = carve.fwd_logits(d["q"], d["k"], d["v"], dev(inp["f"]), dev(inp["A"]), dev(inp["tau"]),
                              dev(inp["w_hat"]), b_x=dev(inp["b_x"]), S0=dev(S0))
    g = carve.bwd_logits(d["q"], d["k"], d["v"], dev(inp["f"]), dev(inp["A"]), dev(inp["tau"]), dev(inp["w_hat"]),
                         d["dO"], b_x=dev(inp["b_x"]), S0=dev(S0), dS_T=dev(dS_T))
    torch.cuda.synchronize()
    ro, rS = oracle.forward_logits(inp["q"], inp["k"], inp["v"], inp["f"], inp["A"], inp["tau"], inp["w_hat"],
                                   b_x=inp["b_x"], S0=S0)
    ref = oracle.backward_logits(inp["q"], inp["k"], inp["v"], inp["f"], inp["A"], inp["tau"], inp["w_hat"],
                                 inp["dO"], b_x=inp["b_x"], S0=S0, dS_T=dS_T)
    errs = {"o": max_rel(to_np(o), ro), "S_T": max_rel(to_np(S_T), rS)}
    for key in ("dq", "dk", "dv", "df", "dA", "dtau", "db_x", "dw_hat", "dS0"):
        if ref[key] is None:
            assert g[key] is None
            continue
        errs[key] = max_rel(to_np(g[key]), ref[key])
    print("  " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
    assert all(v_ <= TOL[dtype] for v_ in errs.values()), errs
