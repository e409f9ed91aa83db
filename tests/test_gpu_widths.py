"""Unequal key and value widths (needs an MI355X).  The state is d_v x d_k with independent
widths; the library runs such calls at the wider width on padded copies (the decode step
takes both widths directly).  Checked against the float64 oracle, which computes at the
true widths: forward outputs and final state, every gradient of the recomputing backward
and of the training pair (which must also match the recomputing backward bit for bit, as
at equal widths), the gates as pre-activations (both pairs), the content-aware forward
with its per-period records and its backward (with and without the records), the no-allocation forward (bit for bit against carve_fwd),
and the decode step, token-only and content-aware.  Ragged token counts, both orders of the
widths, float32 and bfloat16; and at full length (T = 4096) the training pair on every
head, each head normalised by its own reference."""
import numpy as np
import pytest
import torch

import oracle
from chunk_gated_delta_amd import carve
from chunk_gated_delta_amd.synth import random_inputs
from oracle.head_pool import HeadPool
from tests.helpers import max_rel, per_head_rel, to_device, to_np

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}
NAMES = ("dq", "dk", "dv", "dlog_g", "db", "dw", "dS0")


def announce(name):
    print(f"\n[case] {name}", flush=True)


def f32(x):
    return torch.from_numpy(np.asarray(x, np.float32)).cuda()


CASES = [
    # dtype, B, H, T, Dk, Dv: several tiles and a ragged tail (bf16: 64-token tiles, f32: 32)
    ("bf16", 2, 2, 64 * 3 + 17, 64, 128),
    ("bf16", 1, 3, 64 * 2 + 40, 128, 64),
    ("f32", 1, 2, 32 * 4 + 9, 64, 128),
    ("f32", 2, 1, 32 * 3 + 21, 128, 64),
]
IDS = [f"{c[0]}_k{c[4]}_v{c[5]}_T{c[3]}" for c in CASES]


def setup(dtype, B, H, T, Dk, Dv, seed):
    inp = random_inputs(B, H, T, Dk, Dv, dtype=dtype, seed=seed, erase="sigmoid", dists="softplus_decay",
                        with_dO=True)
    rng = np.random.default_rng(seed + 1)
    S0 = np.asarray(rng.standard_normal((B, H, Dv, Dk)) * 0.3, np.float32).astype(np.float64)
    dS_T = np.asarray(rng.standard_normal((B, H, Dv, Dk)) * 0.3, np.float32).astype(np.float64)
    return inp, S0, dS_T


@pytest.mark.parametrize("dtype,B,H,T,Dk,Dv", CASES, ids=IDS)
def test_unequal_widths_forward_and_backward(dtype, B, H, T, Dk, Dv):
    announce(f"unequal widths {dtype} B{B} H{H} T{T} Dk{Dk} Dv{Dv}")
    inp, S0, dS_T = setup(dtype, B, H, T, Dk, Dv, seed=300 + Dk + T)
    d = to_device(inp, dtype)
    S0d, dSd = f32(S0), f32(dS_T)
    o, S_T, _ = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d["b"], S0=S0d)
    g = carve.bwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], b=d["b"], S0=S0d, dS_T=dSd)
    o2, S_T2, saved = carve.fwd_save(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d["b"], S0=S0d)
    g2 = carve.bwd_saved(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], saved, b=d["b"], dS_T=dSd)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (B, H, T, Dv) and tuple(S_T.shape) == (B, H, Dv, Dk)
    ro, rS, _ = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], b=inp["b"], S0=S0)
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], inp["dO"], b=inp["b"], S0=S0,
                          dS_T=dS_T)
    errs = {"o": max_rel(to_np(o), ro), "S_T": max_rel(to_np(S_T), rS)}
    errs.update({k_: max_rel(to_np(g[k_]), ref[k_]) for k_ in NAMES})
    print("  " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
    assert all(v_ <= TOL[dtype] for v_ in errs.values()), errs
    # the training pair runs the same arithmetic as the recomputing calls
    assert torch.equal(o2, o) and torch.equal(S_T2, S_T)
    for k_ in NAMES:
        assert torch.equal(g2[k_], g[k_]), k_


def test_unequal_widths_noalloc_and_empty():
    announce("unequal widths: no-allocation forward, empty inputs")
    dtype, B, H, T, Dk, Dv = "bf16", 2, 2, 100, 64, 128
    inp, S0, _ = setup(dtype, B, H, T, Dk, Dv, seed=321)
    d = to_device(inp, dtype)
    S0d = f32(S0)
    for _ in range(2):   # twice in a row: the scratch holds the previous call's contents
        o, S_T, _ = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d["b"], S0=S0d)
        on, S_Tn, _ = carve.fwd_noalloc(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d["b"], S0=S0d)
        torch.cuda.synchronize()
        assert torch.equal(on, o) and torch.equal(S_Tn, S_T)
    # T = 0: the final state is the initial one, the state gradient passes through
    e = {k_: v_[:, :, :0].contiguous() for k_, v_ in d.items() if v_.dim() >= 3}
    o0, S_T0, _ = carve.fwd(e["q"], e["k"], e["v"], e["log_g"], e["w"], b=e["b"], S0=S0d)
    dS_T = torch.randn((B, H, Dv, Dk), device="cuda")
    g0 = carve.bwd(e["q"], e["k"], e["v"], e["log_g"], e["w"], e["dO"], b=e["b"], S0=S0d, dS_T=dS_T)
    torch.cuda.synchronize()
    assert o0.numel() == 0 and torch.equal(S_T0, S0d) and torch.equal(g0["dS0"], dS_T)


def decode_tokens(d, T, S, L, b=True, content=None):
    outs = []
    for t in range(T):
        tok = {k_: d[k_][:, :, t].contiguous() for k_ in ("q", "k", "v", "log_g", "w") if k_ in d}
        cont = None
        if content is not None:
            cont = dict(content, b_x=d["b_x"][:, :, t].contiguous())
        o, m_out = carve.decode_step(tok["q"], tok["k"], tok["v"], tok["log_g"], tok["w"], S,
                                     b=d["b"][:, :, t].contiguous() if b else None, L=L, content=cont)
        outs.append(o)
        if content is not None:
            content["m_in"] = m_out
            content["pos"] = (content["pos"] + 1) % L
    torch.cuda.synchronize()
    return torch.stack(outs, dim=2)


@pytest.mark.parametrize("dtype,Dk,Dv", [("bf16", 64, 128), ("f32", 128, 64)])
def test_unequal_widths_decode(dtype, Dk, Dv):
    announce(f"unequal widths decode {dtype} Dk{Dk} Dv{Dv}")
    B, H, T = 2, 2, 37
    inp, S0, _ = setup(dtype, B, H, T, Dk, Dv, seed=340 + Dk)
    d = to_device(inp, dtype)
    S = f32(S0)
    o = decode_tokens(d, T, S, L=64)
    ro, rS, _ = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], b=inp["b"], S0=S0)
    eo, es = max_rel(to_np(o), ro), max_rel(to_np(S), rS)
    print(f"  err o={eo:.2e} S={es:.2e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("dtype,Dk,Dv", [("f32", 64, 128), ("bf16", 128, 64)])
def test_unequal_widths_content_decode(dtype, Dk, Dv):
    """Content-aware decode across chunk boundaries: U1 is [H, R, Dv], U2 [H, Dk, R]."""
    announce(f"unequal widths content decode {dtype} Dk{Dk} Dv{Dv}")
    B, H, T, L = 2, 2, 41, 16
    inp = random_inputs(B, H, T, Dk, Dv, dtype=dtype, seed=360 + Dk, erase="content", dists="softplus_decay")
    inp["U1"] = inp["U1"] * 8.0
    inp["U2"] = inp["U2"] * 8.0
    d = to_device(inp, dtype)
    S = torch.zeros((B, H, Dv, Dk), dtype=torch.float32, device="cuda")
    carry = {"U1": d["U1"], "U2": d["U2"], "m_in": None,
             "csum": torch.zeros((B, H, Dv), dtype=torch.float32, device="cuda"), "pos": 0}
    o = decode_tokens(d, T, S, L=L, b=False, content=carry)
    ro, rS, _ = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], L=L,
                               content={"b_x": inp["b_x"], "U1": inp["U1"], "U2": inp["U2"]})
    eo, es = max_rel(to_np(o), ro), max_rel(to_np(S), rS)
    print(f"  err o={eo:.2e} S={es:.2e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("dtype,Dk,Dv,T,L", [("bf16", 64, 128, 64 * 3 + 30, 64), ("f32", 128, 64, 32 * 5 + 7, 32)])
def test_unequal_widths_content_forward(dtype, Dk, Dv, T, L):
    """Content-aware erase at unequal widths: U1 [H, R, Dv] reads the mean output, U2 [H, Dk, R]
    feeds the key-axis gate.  Outputs, final state, the last chunk's mean, and the per-period
    records z [B, H, P, Dk] and m [B, H, P, Dv]; the no-allocation forward gives the same bits."""
    announce(f"unequal widths content forward {dtype} Dk{Dk} Dv{Dv} T{T} L{L}")
    B, H = 2, 2
    inp = random_inputs(B, H, T, Dk, Dv, dtype=dtype, seed=380 + Dk, erase="content", dists="softplus_decay")
    inp["U1"] = inp["U1"] * 8.0
    inp["U2"] = inp["U2"] * 8.0
    d = to_device(inp, dtype)
    m0 = np.asarray(np.random.default_rng(381).standard_normal((B, H, Dv)) * 0.5, np.float32)
    cont = {"b_x": d["b_x"], "U1": d["U1"], "U2": d["U2"], "m0": f32(m0)}
    zr, mr = carve.content_records(B, H, T, Dk, Dv, L, torch.device("cuda"))
    o, S_T, m_out = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], L=L, content=dict(cont, z_rec=zr, m_rec=mr))
    on, S_Tn, m_outn = carve.fwd_noalloc(d["q"], d["k"], d["v"], d["log_g"], d["w"], L=L, content=cont)
    torch.cuda.synchronize()
    assert torch.equal(on, o) and torch.equal(S_Tn, S_T) and torch.equal(m_outn, m_out)
    ro, rS, rm = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], L=L,
                                content={"b_x": inp["b_x"], "U1": inp["U1"], "U2": inp["U2"],
                                         "m0": m0.astype(np.float64)})
    errs = {"o": max_rel(to_np(o), ro), "S_T": max_rel(to_np(S_T), rS), "m_out": max_rel(to_np(m_out), rm)}
    # records: period p's z is U2 U1 m_{p-1}, with m_{p-1} the previous period's mean (m0 first)
    P = zr.shape[2]
    ref_m = np.concatenate([m0.astype(np.float64)[:, :, None],
                            np.stack([ro[:, :, L * j:min(L * (j + 1), T)].mean(axis=2) for j in range(P - 1)], 2)
                            if P > 1 else np.zeros((B, H, 0, Dv))], axis=2)
    ref_z = np.einsum("hkr,hrv,bhpv->bhpk", inp["U2"], inp["U1"], ref_m)
    errs["m_rec"] = max_rel(to_np(mr), ref_m)
    errs["z_rec"] = max_rel(to_np(zr), ref_z)
    print("  " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
    assert all(v_ <= TOL[dtype] for v_ in errs.values()), errs
    ro0, _, _ = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], L=L,
                               content={"b_x": inp["b_x"], "U1": None, "U2": None})
    assert max_rel(ro0, ro) > 0.02       # the content signal matters at this scale


LOGIT_GRADS = ("dq", "dk", "dv", "df", "dA", "dtau", "db_x", "dw_hat", "dS0")


@pytest.mark.parametrize("dtype,B,H,T,Dk,Dv", [CASES[0], CASES[3]], ids=[IDS[0], IDS[3]])
def test_unequal_widths_gate_logits(dtype, B, H, T, Dk, Dv):
    """Gates given as pre-activations at unequal widths (A and tau per head and key channel):
    the recomputing pair against the oracle, and the saved pair bit for bit against it."""
    announce(f"unequal widths gate logits {dtype} B{B} H{H} T{T} Dk{Dk} Dv{Dv}")
    inp, S0, dS_T = setup(dtype, B, H, T, Dk, Dv, seed=400 + Dk + T)
    rng = np.random.default_rng(401)
    f64 = lambda x: np.asarray(x, np.float32).astype(np.float64)
    gl = {"f": f64(rng.standard_normal((B, H, T, Dk))), "A": f64(rng.uniform(0.05, 10.0, (H, Dk))),
          "tau": f64(rng.standard_normal((H, Dk)) * 0.5), "w_hat": f64(rng.standard_normal((B, H, T))),
          "b_x": f64(rng.normal(2.0, 1.0, (B, H, T, Dk)))}
    d = to_device(inp, dtype)
    gd = {k_: f32(v_) for k_, v_ in gl.items()}
    S0d, dSd = f32(S0), f32(dS_T)
    args = (d["q"], d["k"], d["v"], gd["f"], gd["A"], gd["tau"], gd["w_hat"])
    o, S_T = carve.fwd_logits(*args, b_x=gd["b_x"], S0=S0d)
    g = carve.bwd_logits(*args, d["dO"], b_x=gd["b_x"], S0=S0d, dS_T=dSd)
    o2, S_T2, saved = carve.fwd_logits_save(*args, b_x=gd["b_x"], S0=S0d)
    g2 = carve.bwd_logits_saved(*args, d["dO"], saved, b_x=gd["b_x"], dS_T=dSd)
    torch.cuda.synchronize()
    ro, rS = oracle.forward_logits(inp["q"], inp["k"], inp["v"], gl["f"], gl["A"], gl["tau"], gl["w_hat"],
                                   b_x=gl["b_x"], S0=S0)
    ref = oracle.backward_logits(inp["q"], inp["k"], inp["v"], gl["f"], gl["A"], gl["tau"], gl["w_hat"], inp["dO"],
                                 b_x=gl["b_x"], S0=S0, dS_T=dS_T)
    errs = {"o": max_rel(to_np(o), ro), "S_T": max_rel(to_np(S_T), rS)}
    errs.update({k_: max_rel(to_np(g[k_]), ref[k_]) for k_ in LOGIT_GRADS})
    print("  " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
    assert all(v_ <= TOL[dtype] for v_ in errs.values()), errs
    assert torch.equal(o2, o) and torch.equal(S_T2, S_T)
    for k_ in LOGIT_GRADS:
        assert torch.equal(g2[k_], g[k_]), k_


CONTENT_GRADS = ("dq", "dk", "dv", "dlog_g", "db_x", "dw", "dU1", "dU2", "dm0", "dS0")


@pytest.mark.parametrize("dtype,Dk,Dv,T,L", [("bf16", 64, 128, 64 * 3 + 30, 64), ("f32", 128, 64, 32 * 5 + 7, 32)])
def test_unequal_widths_content_backward(dtype, Dk, Dv, T, L):
    """Backward through the content-aware erase at unequal widths: every gradient (dU1
    [H, R, Dv], dU2 [H, Dk, R], dm0 [B, H, Dv]) against the oracle; given the forward's
    records, the same bits without re-running the forward."""
    announce(f"unequal widths content backward {dtype} Dk{Dk} Dv{Dv} T{T} L{L}")
    B, H = 2, 2
    inp = random_inputs(B, H, T, Dk, Dv, dtype=dtype, seed=420 + Dk, erase="content", dists="softplus_decay",
                        with_dO=True)
    inp["U1"] = inp["U1"] * 8.0
    inp["U2"] = inp["U2"] * 8.0
    rng = np.random.default_rng(421)
    f64 = lambda x: np.asarray(x, np.float32).astype(np.float64)
    m0, S0 = f64(rng.standard_normal((B, H, Dv)) * 0.5), f64(rng.standard_normal((B, H, Dv, Dk)) * 0.3)
    dS_T, dm_out = f64(rng.standard_normal((B, H, Dv, Dk)) * 0.3), f64(rng.standard_normal((B, H, Dv)))
    d = to_device(inp, dtype)
    cont = {"b_x": d["b_x"], "U1": d["U1"], "U2": d["U2"], "m0": f32(m0)}
    kw = dict(S0=f32(S0), dS_T=f32(dS_T), dm_out=f32(dm_out), L=L)
    g = carve.bwd_content(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], cont, **kw)
    zr, mr = carve.content_records(B, H, T, Dk, Dv, L, torch.device("cuda"))
    carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], S0=f32(S0), L=L, content=dict(cont, z_rec=zr, m_rec=mr))
    g1 = carve.bwd_content(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], dict(cont, z_rec=zr, m_rec=mr),
                           **kw)
    torch.cuda.synchronize()
    ref = oracle.backward_content(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], inp["dO"],
                                  {"b_x": inp["b_x"], "U1": inp["U1"], "U2": inp["U2"], "m0": m0},
                                  S0=S0, dS_T=dS_T, dm_out=dm_out, L=L)
    errs = {k_: max_rel(to_np(g[k_]), ref[k_]) for k_ in CONTENT_GRADS}
    print("  " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
    assert all(v_ <= TOL[dtype] for v_ in errs.values()), errs
    for k_ in CONTENT_GRADS:
        assert torch.equal(g1[k_], g[k_]), k_


@pytest.mark.parametrize("Dk,Dv", [(64, 128), (128, 64)])
def test_unequal_widths_full_length_every_head(Dk, Dv):
    """B2 H16 T4096 bf16 with the benchmark's gate distributions: fwd_save + bwd_saved,
    o, S_T and every gradient of all 32 heads against the oracle, per head."""
    B, H, T = 2, 16, 4096
    announce(f"unequal widths full length every head Dk{Dk} Dv{Dv}")
    inp = random_inputs(B, H, T, Dk, Dv, dtype="bf16", seed=440 + Dk, erase="sigmoid", dists="softplus_decay",
                        with_dO=True)
    d = to_device(inp, "bf16")
    o, S_T, saved = carve.fwd_save(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d["b"])
    g = carve.bwd_saved(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], saved, b=d["b"], want_dS0=False)
    torch.cuda.synchronize()
    gpu = {"o": to_np(o), "S_T": to_np(S_T)}
    gpu.update({k_: to_np(g[k_]) for k_ in ("dq", "dk", "dv", "dlog_g", "db", "dw")})
    del d, o, S_T, saved, g
    kw = dict(q=inp["q"], k=inp["k"], v=inp["v"], log_g=inp["log_g"], w=inp["w"], b=inp["b"])
    with HeadPool() as pool:
        ro, rS, _ = pool.run("forward", B, H, **kw)
        ref = pool.run("backward", B, H, dO=inp["dO"], **kw)
    ref.update(o=ro, S_T=rS)
    bad = {}
    for k_, x in gpu.items():
        e = per_head_rel(x, ref[k_])
        print(f"  {k_}: worst head {e.max():.2e}, median {np.median(e):.2e}", flush=True)
        if e.max() > TOL["bf16"]:
            bad[k_] = float(e.max())
    assert not bad, bad
