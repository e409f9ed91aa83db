"""The torch.autograd functions over the training pairs (needs an MI355X): a backward
through them gives the bits the library's backward gives for the same upstream gradients
(the wrappers only marshal), and unused outputs get zero gradients."""
import numpy as np
import pytest
import torch

from chunk_gated_delta_amd import carve
from chunk_gated_delta_amd.autograd import carve_attention, carve_attention_content, carve_attention_logits
from chunk_gated_delta_amd.synth import random_inputs
from tests.helpers import to_device

pytestmark = pytest.mark.gpu


def leaf(t):
    return None if t is None else t.detach().clone().requires_grad_(True)


@pytest.mark.parametrize("dtype,Dk,Dv", [("bf16", 128, 128), ("f32", 64, 128)])
def test_token_pair_autograd_matches_library(dtype, Dk, Dv):
    print(f"\n[case] autograd token pair {dtype} Dk{Dk} Dv{Dv}", flush=True)
    B, H, T = 2, 2, 150
    inp = random_inputs(B, H, T, Dk, Dv, dtype=dtype, seed=41, erase="sigmoid", dists="softplus_decay", with_dO=True)
    d = to_device(inp, dtype)
    S0 = torch.randn((B, H, Dv, Dk), device="cuda") * 0.3
    dS_T = torch.randn((B, H, Dv, Dk), device="cuda") * 0.3
    xs = {key: leaf(d[key]) for key in ("q", "k", "v", "log_g", "w", "b")}
    s0 = leaf(S0)
    o, S_T = carve_attention(xs["q"], xs["k"], xs["v"], xs["log_g"], xs["w"], b=xs["b"], S0=s0)
    (o.float() * d["dO"].float()).sum().add_((S_T * dS_T).sum()).backward()
    _, _, saved = carve.fwd_save(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d["b"], S0=S0)
    g = carve.bwd_saved(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], saved, b=d["b"], dS_T=dS_T)
    torch.cuda.synchronize()
    for key, name in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("log_g", "dlog_g"), ("w", "dw"), ("b", "db")):
        assert torch.equal(xs[key].grad, g[name]), key
    assert torch.equal(s0.grad, g["dS0"])
    # only o used: the final-state gradient is zero
    xs2 = {key: leaf(d[key]) for key in ("q", "k", "v", "log_g", "w")}
    o2, _ = carve_attention(xs2["q"], xs2["k"], xs2["v"], xs2["log_g"], xs2["w"])
    (o2.float() * d["dO"].float()).sum().backward()
    g2 = carve.bwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"])
    torch.cuda.synchronize()
    assert torch.equal(xs2["q"].grad, g2["dq"]) and torch.equal(xs2["log_g"].grad, g2["dlog_g"])


def test_logit_pair_autograd_matches_library():
    print("\n[case] autograd logit pair bf16", flush=True)
    B, H, T, D = 1, 2, 200, 128
    inp = random_inputs(B, H, T, D, D, dtype="bf16", seed=42, erase="none", with_dO=True)
    d = to_device(inp, "bf16")
    rng = np.random.default_rng(43)
    t32 = lambda x: torch.from_numpy(np.asarray(x, np.float32)).cuda()
    gl = {"f": t32(rng.standard_normal((B, H, T, D))), "A": t32(rng.uniform(0.05, 3.0, (H, D))),
          "tau": t32(rng.standard_normal((H, D)) * 0.5), "w_hat": t32(rng.standard_normal((B, H, T))),
          "b_x": t32(rng.normal(2.0, 1.0, (B, H, T, D)))}
    xs = {key: leaf(val) for key, val in dict(d, **gl).items() if key in ("q", "k", "v", *gl)}
    o, S_T = carve_attention_logits(xs["q"], xs["k"], xs["v"], xs["f"], xs["A"], xs["tau"], xs["w_hat"],
                                    b_x=xs["b_x"])
    (o.float() * d["dO"].float()).sum().backward()
    args = (d["q"], d["k"], d["v"], gl["f"], gl["A"], gl["tau"], gl["w_hat"])
    _, _, saved = carve.fwd_logits_save(*args, b_x=gl["b_x"])
    g = carve.bwd_logits_saved(*args, d["dO"], saved, b_x=gl["b_x"], want_dS0=False)
    torch.cuda.synchronize()
    for key, name in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("f", "df"), ("A", "dA"), ("tau", "dtau"),
                      ("w_hat", "dw_hat"), ("b_x", "db_x")):
        assert torch.equal(xs[key].grad, g[name]), key


def test_content_pair_autograd_matches_library():
    print("\n[case] autograd content pair bf16", flush=True)
    B, H, T, D, L = 2, 2, 200, 128, 64
    inp = random_inputs(B, H, T, D, D, dtype="bf16", seed=44, erase="content", dists="softplus_decay",
                        with_dO=True)
    inp["U1"] = inp["U1"] * 8.0
    inp["U2"] = inp["U2"] * 8.0
    d = to_device(inp, "bf16")
    m0 = torch.randn((B, H, D), device="cuda") * 0.5
    dm = torch.randn((B, H, D), device="cuda")
    xs = {key: leaf(d[key]) for key in ("q", "k", "v", "log_g", "w", "b_x", "U1", "U2")}
    m0l = leaf(m0)
    o, S_T, m_out = carve_attention_content(xs["q"], xs["k"], xs["v"], xs["log_g"], xs["w"], xs["b_x"], xs["U1"],
                                            xs["U2"], m0=m0l, L=L)
    (o.float() * d["dO"].float()).sum().add_((m_out * dm).sum()).backward()
    cont = {"b_x": d["b_x"], "U1": d["U1"], "U2": d["U2"], "m0": m0}
    g = carve.bwd_content(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], cont, dm_out=dm, L=L)
    torch.cuda.synchronize()
    for key, name in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("log_g", "dlog_g"), ("w", "dw"), ("b_x", "db_x"),
                      ("U1", "dU1"), ("U2", "dU2")):
        assert torch.equal(xs[key].grad, g[name]), key
    assert torch.equal(m0l.grad, g["dm0"])
