"""GPU parity of the recurrent decode step against the float64 reference (needs an MI355X).

The decode step is the token recurrence itself, so a run of T decode calls must
reproduce the reference forward over the same T tokens: every output o_t, the
final state, and on the content path the chunk means.  Error metric and bars as
for the forward: max|gpu - ref| / max|ref| per tensor, 1e-4 for float32 inputs,
2e-2 for bfloat16 inputs.
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


def announce(name):
    print(f"\n[case] {name}", flush=True)


def token(d, key, t):
    return d[key][:, :, t].contiguous()


def decode_run(d, T, S, L=64, b=True, content=None, t0=0):
    """Decode tokens t0 .. t0+T-1 of the device inputs d, updating S in place.
    content: None or dict(U1, U2, m_in, csum, pos) carried across the calls."""
    outs = []
    for t in range(t0, t0 + T):
        cont = None
        if content is not None:
            cont = {"b_x": token(d, "b_x", t), "U1": content["U1"], "U2": content["U2"],
                    "m_in": content["m_in"], "csum": content["csum"], "pos": content["pos"]}
        o, m_out = carve.decode_step(token(d, "q", t), token(d, "k", t), token(d, "v", t), token(d, "log_g", t),
                                     d["w"][:, :, t].contiguous(), S, b=token(d, "b", t) if b else None, L=L,
                                     content=cont)
        outs.append(o)
        if content is not None:
            content["m_in"] = m_out
            content["pos"] = (content["pos"] + 1) % L
    torch.cuda.synchronize()
    return torch.stack(outs, dim=2)


@pytest.mark.parametrize("dtype,D,erase,T", [("f32", 64, "sigmoid", 40), ("bf16", 128, "sigmoid", 48),
                                             ("bf16", 128, "none", 33), ("f32", 128, "none", 20),
                                             ("bf16", 64, "ones", 25)])
def test_decode_matches_reference(dtype, D, erase, T):
    announce(f"decode {dtype} D{D} {erase} T{T}")
    B, H = 2, 3
    inp = random_inputs(B, H, T, D, D, dtype=dtype, seed=70 + D + T, erase=erase, dists="softplus_decay")
    d = to_device(inp, dtype)
    S0 = np.asarray(np.random.default_rng(3).standard_normal((B, H, D, D)) * 0.3, np.float32)
    S = torch.from_numpy(S0).cuda()
    o = decode_run(d, T, S, b=erase != "none")
    ro, rS, _ = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], b=inp.get("b"),
                               S0=S0.astype(np.float64))
    eo, es = max_rel(to_np(o), ro), max_rel(to_np(S), rS)
    print(f"  err o={eo:.2e} S={es:.2e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_then_decode(dtype):
    """S_T of a chunked forward continues the sequence token by token."""
    announce(f"prefill + decode {dtype}")
    B, H, D, T1, T2 = 2, 2, 128, 200, 24
    inp = random_inputs(B, H, T1 + T2, D, D, dtype=dtype, seed=81, erase="sigmoid", dists="softplus_decay")
    d = to_device(inp, dtype)
    pre = {k_: v_[:, :, :T1].contiguous() for k_, v_ in d.items()}
    o1, S, _ = carve.fwd(pre["q"], pre["k"], pre["v"], pre["log_g"], pre["w"], b=pre["b"], L=64)
    o2 = decode_run(d, T2, S, t0=T1)
    ro, rS, _ = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], b=inp["b"])
    e1 = max_rel(to_np(o1), ro[:, :, :T1])
    e2 = max_rel(to_np(o2), ro[:, :, T1:])
    es = max_rel(to_np(S), rS)
    print(f"  err prefill o={e1:.2e} decode o={e2:.2e} S={es:.2e}", flush=True)
    assert max(e1, e2, es) <= TOL[dtype]


def content_setup(dtype, B, H, T, D, seed, scale=8.0):
    inp = random_inputs(B, H, T, D, D, dtype=dtype, seed=seed, erase="content", dists="softplus_decay")
    inp["U1"] = inp["U1"] * scale
    inp["U2"] = inp["U2"] * scale
    return inp, to_device(inp, dtype)


@pytest.mark.parametrize("dtype,D,L,T", [("f32", 64, 8, 27), ("bf16", 128, 16, 50)])
def test_decode_content_matches_reference(dtype, D, L, T):
    """Content-aware decode across several chunk boundaries, from a carried-in mean."""
    announce(f"decode content {dtype} D{D} L{L} T{T}")
    B, H = 2, 2
    inp, d = content_setup(dtype, B, H, T, D, seed=90 + D)
    m0 = np.asarray(np.random.default_rng(2).standard_normal((B, H, D)) * 0.5, np.float32)
    S = torch.zeros((B, H, D, D), dtype=torch.float32, device="cuda")
    carry = {"U1": d["U1"], "U2": d["U2"], "m_in": torch.from_numpy(m0).cuda(),
             "csum": torch.zeros((B, H, D), dtype=torch.float32, device="cuda"), "pos": 0}
    o = decode_run(d, T, S, L=L, b=False, content=carry)
    ro, rS, rm = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], L=L,
                                content={"b_x": inp["b_x"], "U1": inp["U1"], "U2": inp["U2"],
                                         "m0": m0.astype(np.float64)})
    # the reference's m_out is the mean of the last (ragged) chunk: csum / pos on the decode side
    npos = carry["pos"]
    m = to_np(carry["csum"]) / npos if npos > 0 else to_np(carry["m_in"])
    errs = (max_rel(to_np(o), ro), max_rel(to_np(S), rS), max_rel(m, rm))
    print(f"  err o={errs[0]:.2e} S={errs[1]:.2e} m={errs[2]:.2e}", flush=True)
    assert max(errs) <= TOL[dtype]
    ro0, _, _ = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], L=L,
                               content={"b_x": inp["b_x"], "U1": None, "U2": None})
    assert max_rel(ro0, ro) > 0.02       # the content signal matters at this scale


def test_content_prefill_then_decode():
    """A content-aware prefill of whole chunks hands over through m_out (pos = 0)."""
    announce("content prefill + decode")
    B, H, D, L, T1, T2 = 2, 2, 128, 64, 128, 40
    inp, d = content_setup("bf16", B, H, T1 + T2, D, seed=97)
    pre = {k_: (v_[:, :, :T1].contiguous() if v_.dim() == 4 else v_) for k_, v_ in d.items()}
    pre["w"] = d["w"][:, :, :T1].contiguous()
    o1, S, m1 = carve.fwd(pre["q"], pre["k"], pre["v"], pre["log_g"], pre["w"], L=L,
                          content={"b_x": pre["b_x"], "U1": d["U1"], "U2": d["U2"]})
    carry = {"U1": d["U1"], "U2": d["U2"], "m_in": m1,
             "csum": torch.zeros((B, H, D), dtype=torch.float32, device="cuda"), "pos": 0}
    o2 = decode_run(d, T2, S, L=L, b=False, content=carry, t0=T1)
    ro, rS, _ = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], L=L,
                               content={"b_x": inp["b_x"], "U1": inp["U1"], "U2": inp["U2"]})
    e1 = max_rel(to_np(o1), ro[:, :, :T1])
    e2 = max_rel(to_np(o2), ro[:, :, T1:])
    es = max_rel(to_np(S), rS)
    print(f"  err prefill o={e1:.2e} decode o={e2:.2e} S={es:.2e}", flush=True)
    assert max(e1, e2, es) <= 2e-2


def test_decode_zero_projection_bit_exact():
    """U_b = 0 gives the same bits as U_b absent in the decode step too."""
    announce("decode zero projection bit exact")
    B, H, D, L, T = 2, 3, 128, 4, 10
    inp, d = content_setup("bf16", B, H, T, D, seed=99)
    m0 = torch.from_numpy(np.asarray(np.random.default_rng(4).standard_normal((B, H, D)), np.float32)).cuda()
    res = []
    for U1, U2 in ((torch.zeros_like(d["U1"]), torch.zeros_like(d["U2"])), (None, None)):
        S = torch.zeros((B, H, D, D), dtype=torch.float32, device="cuda")
        carry = {"U1": U1, "U2": U2, "m_in": m0.clone(),
                 "csum": torch.zeros((B, H, D), dtype=torch.float32, device="cuda"), "pos": 0}
        o = decode_run(d, T, S, L=L, b=False, content=carry)
        res.append((o, S, carry["m_in"], carry["csum"]))
    for x, y in zip(*res):
        assert torch.equal(x, y)


def test_decode_content_rank64_d64():
    """Largest projection rank (64) at key width 64, across a chunk boundary."""
    announce("decode content rank 64 d64")
    B, H, D, L, T, R = 2, 2, 64, 4, 9, 64
    inp = random_inputs(B, H, T, D, D, dtype="bf16", seed=111, erase="content", dists="softplus_decay", rank=R)
    inp["U1"] = inp["U1"] * 6.0
    inp["U2"] = inp["U2"] * 6.0
    d = to_device(inp, "bf16")
    S = torch.zeros((B, H, D, D), dtype=torch.float32, device="cuda")
    carry = {"U1": d["U1"], "U2": d["U2"], "m_in": None,
             "csum": torch.zeros((B, H, D), dtype=torch.float32, device="cuda"), "pos": 0}
    o = decode_run(d, T, S, L=L, b=False, content=carry)
    ro, rS, _ = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], L=L,
                               content={"b_x": inp["b_x"], "U1": inp["U1"], "U2": inp["U2"]})
    eo, es = max_rel(to_np(o), ro), max_rel(to_np(S), rS)
    print(f"  err o={eo:.2e} S={es:.2e}", flush=True)
    assert eo <= TOL["bf16"] and es <= TOL["bf16"]
