"""GPU test of carve_fwd_noalloc, the forward for callers that cannot allocate device
memory (needs an MI355X).  Its outputs are compared with carve_fwd's on the same inputs,
over two calls in a row whose second input is smaller, for token-only and content-aware
gates, and a shape whose workspace exceeds the library's scratch is rejected on the host
before any launch.  The two entry points run the same kernels, so the outputs must agree
bit for bit (stricter than the bf16 / fp32 bars of the parity tests)."""
import numpy as np
import pytest
import torch

from chunk_gated_delta_amd import carve
from chunk_gated_delta_amd.synth import random_inputs
from tests.helpers import to_device

pytestmark = pytest.mark.gpu


def announce(name):
    print(f"\n[case] {name}", flush=True)


def f32(x):
    return torch.from_numpy(np.asarray(x, np.float32)).cuda()


def compare(B, H, T, D, dtype, seed, content):
    inp = random_inputs(B, H, T, D, D, dtype=dtype, seed=seed, erase="content" if content else "sigmoid",
                        dists="softplus_decay")
    d = to_device(inp, dtype)
    S0 = f32(np.random.default_rng(seed).standard_normal((B, H, D, D)) * 0.3)
    cont = None
    b = d.get("b")
    if content:
        cont = {"b_x": d["b_x"], "U1": d["U1"], "U2": d["U2"],
                "m0": f32(np.random.default_rng(seed + 1).standard_normal((B, H, D)) * 0.5)}
    o1, S1, m1 = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=b, S0=S0, L=64, content=cont)
    o2, S2, m2 = carve.fwd_noalloc(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=b, S0=S0, L=64, content=cont)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(S1, S2)
    if content:
        assert torch.equal(m1, m2)


def test_noalloc_two_calls_token_only():
    announce("noalloc token-only: B2 H4 T512 d128, then B1 H2 T200 d64")
    compare(2, 4, 512, 128, "bf16", seed=2001, content=False)
    compare(1, 2, 200, 64, "bf16", seed=2002, content=False)


def test_noalloc_two_calls_content():
    announce("noalloc content-aware: B2 H4 T384 d128, then B1 H1 T130 d64 (f32)")
    compare(2, 4, 384, 128, "bf16", seed=2003, content=True)
    compare(1, 1, 130, 64, "f32", seed=2004, content=True)


def test_noalloc_rejects_beyond_scratch():
    announce("noalloc rejects a workspace beyond the scratch")
    B, H, T, D = 2, 16, 2048, 128
    q = torch.zeros((B, H, T, D), dtype=torch.bfloat16, device="cuda")
    lg = torch.zeros((B, H, T, D), dtype=torch.float32, device="cuda")
    w = torch.zeros((B, H, T), dtype=torch.float32, device="cuda")
    assert carve.fwd_workspace_bytes(q, q, 64) > 64 << 20
    with pytest.raises(RuntimeError, match="CARVE_ERR_WORKSPACE"):
        carve.fwd_noalloc(q, q, q, lg, w, L=64)
