"""The largest accepted head count (needs an MI355X): B*H = 65535 sequences, the launch
grids' limit, with one full and one ragged 64-token tile each (T = 65, d = 64, bf16).  The
training pair fwd_save + bwd_saved and the plain forward run over every head; sampled
heads (the first, the last and a spread between) are compared element-wise with the
float64 oracle, and every head through the identity <dq, q> = <dO, o> (o is linear in q).
Also the longest sequence tested, one head of 2^20 tokens (below).  Inputs are drawn on
the device from a seeded generator with the bench workload's distributions; the oracle
takes exactly the device values of its heads."""
import numpy as np
import pytest
import torch

import oracle
from chunk_gated_delta_amd import carve
from tests.helpers import max_rel, to_np

pytestmark = pytest.mark.gpu

B, H, T, D = 5, 13107, 65, 64
TOL = 2e-2


def draw():
    g = torch.Generator(device="cuda").manual_seed(65535)
    n = lambda *shape: torch.randn(shape, generator=g, device="cuda")
    q = torch.nn.functional.normalize(n(B, H, T, D), dim=-1).to(torch.bfloat16)
    k = torch.nn.functional.normalize(n(B, H, T, D), dim=-1).to(torch.bfloat16)
    v = n(B, H, T, D).to(torch.bfloat16)
    dO = n(B, H, T, D).to(torch.bfloat16)
    log_g = (-0.1 * torch.nn.functional.softplus(n(B, H, T, D))).contiguous()
    b = torch.sigmoid(n(B, H, T, D) + 2.0).contiguous()
    w = torch.sigmoid(n(B, H, T)).contiguous()
    return dict(q=q, k=k, v=v, dO=dO, log_g=log_g, b=b, w=w)


def test_max_head_count_training_pair_and_forward():
    print(f"\n[case] B{B} H{H} (B*H = {B * H}) T{T} d{D} bf16", flush=True)
    d = draw()
    o, S_T, saved = carve.fwd_save(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d["b"])
    g = carve.bwd_saved(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], saved, b=d["b"], want_dS0=False)
    o2, S2, _ = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d["b"])
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(S_T, S2)
    # every head: <dq, q> = <dO, o>
    lhs = (g["dq"].float() * d["q"].float()).sum(dim=(2, 3))
    rhs = (d["dO"].float() * o.float()).sum(dim=(2, 3))
    rel = ((lhs - rhs).abs().max() / rhs.abs().max()).item()
    print(f"  <dq,q> vs <dO,o> over {B * H} heads: {rel:.2e}", flush=True)
    assert rel <= TOL
    assert all(torch.isfinite(g[key]).all().item() for key in ("dq", "dk", "dv", "dlog_g", "db", "dw"))
    # sampled heads element-wise
    rng = np.random.default_rng(7)
    flat = sorted({0, B * H - 1, *rng.integers(0, B * H, 22).tolist()})
    for i in flat:
        bi, hi = divmod(i, H)
        host = {key: to_np(val[bi:bi + 1, hi:hi + 1]) for key, val in d.items()}
        ro, rS, _ = oracle.forward(host["q"], host["k"], host["v"], host["log_g"], host["w"], b=host["b"])
        ref = oracle.backward(host["q"], host["k"], host["v"], host["log_g"], host["w"], host["dO"], b=host["b"])
        errs = {"o": max_rel(to_np(o[bi:bi + 1, hi:hi + 1]), ro), "S_T": max_rel(to_np(S_T[bi:bi + 1, hi:hi + 1]), rS)}
        errs.update({key: max_rel(to_np(g[key][bi:bi + 1, hi:hi + 1]), ref[key])
                     for key in ("dq", "dk", "dv", "dlog_g", "db", "dw")})
        assert all(v_ <= TOL for v_ in errs.values()), (i, errs)
    print(f"  {len(flat)} sampled heads within {TOL}", flush=True)


def test_longest_sequence():
    """One head of 2^20 tokens (16,384 chunks; the state passes run as segments chained by
    the scan of their affine maps).  Checked where the oracle can follow: the first 4,096
    tokens' outputs from the zero state; the last 4,096 tokens' outputs, the final state
    and their gradients (which depend only on those tokens, the state entering them and the
    final-state gradient) against the oracle continued from the state a split run carries
    to that point; and over the whole sequence <dq, q> = <dO, o>."""
    TL, DL, tail = 1 << 20, 128, 4096
    print(f"\n[case] B1 H1 T{TL} d{DL} bf16", flush=True)
    g_ = torch.Generator(device="cuda").manual_seed(1 << 20)
    n = lambda *shape: torch.randn(shape, generator=g_, device="cuda")
    d = dict(q=torch.nn.functional.normalize(n(1, 1, TL, DL), dim=-1).to(torch.bfloat16),
             k=torch.nn.functional.normalize(n(1, 1, TL, DL), dim=-1).to(torch.bfloat16),
             v=n(1, 1, TL, DL).to(torch.bfloat16), dO=n(1, 1, TL, DL).to(torch.bfloat16),
             log_g=(-0.1 * torch.nn.functional.softplus(n(1, 1, TL, DL))).contiguous(),
             b=torch.sigmoid(n(1, 1, TL, DL) + 2.0).contiguous(), w=torch.sigmoid(n(1, 1, TL)).contiguous())
    part = lambda a_, b_: {key: val[:, :, a_:b_].contiguous() for key, val in d.items()}
    o, S_T, saved = carve.fwd_save(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d["b"])
    g = carve.bwd_saved(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], saved, b=d["b"], want_dS0=False)
    del saved
    head = part(0, TL - tail)
    _, S_a, _ = carve.fwd(head["q"], head["k"], head["v"], head["log_g"], head["w"], b=head["b"])
    del head
    torch.cuda.synchronize()
    print("  GPU runs done", flush=True)
    lhs = (g["dq"].float() * d["q"].float()).sum().item()
    rhs = (d["dO"].float() * o.float()).sum().item()
    print(f"  <dq,q> = {lhs:.6e}, <dO,o> = {rhs:.6e}", flush=True)
    assert abs(lhs - rhs) <= TOL * abs(rhs)
    first = {key: to_np(val) for key, val in part(0, tail).items()}
    ro, _, _ = oracle.forward(first["q"], first["k"], first["v"], first["log_g"], first["w"], b=first["b"])
    e_first = max_rel(to_np(o[:, :, :tail]), ro)
    last = {key: to_np(val) for key, val in part(TL - tail, TL).items()}
    S_in = to_np(S_a)
    ro, rS, _ = oracle.forward(last["q"], last["k"], last["v"], last["log_g"], last["w"], b=last["b"], S0=S_in)
    ref = oracle.backward(last["q"], last["k"], last["v"], last["log_g"], last["w"], last["dO"], b=last["b"], S0=S_in)
    errs = {"o(first)": e_first, "o(last)": max_rel(to_np(o[:, :, TL - tail:]), ro), "S_T": max_rel(to_np(S_T), rS)}
    errs.update({key: max_rel(to_np(g[key][:, :, TL - tail:]), ref[key]) for key in ("dq", "dk", "dv", "dlog_g", "db", "dw")})
    print("  " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
    assert all(v_ <= TOL for v_ in errs.values()), errs
