"""The largest accepted head count (needs an MI355X): B*H = 65535 sequences, the launch
grids' limit, with one full and one ragged 64-token tile each (T = 65, d = 64, bf16).  The
training pair fwd_save + bwd_saved and the plain forward run over every head; sampled
heads (the first, the last and a spread between) are compared element-wise with the
float64 oracle, and every head through the identity <dq, q> = <dO, o> (o is linear in q).
Inputs are drawn on the device from a seeded generator with the bench workload's
distributions; the oracle takes exactly the device values of its heads."""
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
