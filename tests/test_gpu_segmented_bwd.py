"""The training pair with segmented state passes (needs an MI355X).  With few heads and a
long sequence the forward and the reverse state passes cut each head's chunk chain into
segments: the reverse pass forms each segment's affine map of the state gradient, chains
the maps with a reverse scan from dS_T, and then runs every segment from its own entering
gradient.  Checked against the float64 oracle with slow decay and small writes, so the
gradient carried through the chain of segment maps matters, and against the sequential
reverse pass the same heads take inside a batch large enough to fill the GPU."""
import numpy as np
import pytest
import torch

import oracle
from chunk_gated_delta_amd import carve
from chunk_gated_delta_amd.synth import random_inputs
from tests.helpers import max_rel, to_device, to_np

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f32": 1e-4}
NAMES = ("dq", "dk", "dv", "dlog_g", "dw", "dS0")


def announce(name):
    print(f"\n[case] {name}", flush=True)


def f32(x):
    return torch.from_numpy(np.asarray(x, np.float32)).cuda()


def long_memory_inputs(B, H, T, D, dtype, seed):
    """Slow key-axis decay (a in [0.9995, 1]) and a small write gate (w in [0, 0.05]): most of
    the state gradient entering a segment survives it, so the segments' maps carry weight."""
    inp = random_inputs(B, H, T, D, D, dtype=dtype, seed=seed, erase="none", dists="uniform_decay", with_dO=True)
    rng = np.random.default_rng(seed + 1)
    inp["log_g"] = rng.uniform(np.log(0.9995), 0.0, (B, H, T, D)).astype(np.float32).astype(np.float64)
    inp["w"] = rng.uniform(0.0, 0.05, (B, H, T)).astype(np.float32).astype(np.float64)
    inp.pop("b", None)
    return inp


def run_pair(inp, dtype, S0, dS_T, saved_pair=True):
    d = to_device(inp, dtype)
    S0d, dSd = f32(S0), f32(dS_T)
    if saved_pair:
        o, S_T, saved = carve.fwd_save(d["q"], d["k"], d["v"], d["log_g"], d["w"], S0=S0d)
        g = carve.bwd_saved(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], saved, dS_T=dSd, want_dS0=True)
    else:
        o, S_T, _ = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], S0=S0d)
        g = carve.bwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], d["dO"], S0=S0d, dS_T=dSd, want_dS0=True)
    torch.cuda.synchronize()
    out = {"o": to_np(o), "S_T": to_np(S_T)}
    out.update({k_: to_np(g[k_]) for k_ in NAMES})
    return out


def reference(inp, S0, dS_T):
    ro, rS, _ = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], S0=S0)
    ref = oracle.backward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], inp["dO"], S0=S0, dS_T=dS_T)
    ref.update(o=ro, S_T=rS)
    return ref


SEG_CASES = [
    # dtype, B, H, T, D: 6 segments of 17 chunks (64-token tiles) / 4 of 18 (32-token tiles),
    # a partial chunk in the last segment
    ("bf16", 1, 2, 64 * 100 + 5, 128),
    ("f32", 2, 1, 32 * 70 + 9, 64),
]


@pytest.mark.parametrize("saved_pair", [True, False], ids=["saved_pair", "recompute"])
@pytest.mark.parametrize("dtype,B,H,T,D", SEG_CASES, ids=[f"{c[0]}_d{c[4]}_T{c[3]}" for c in SEG_CASES])
def test_segmented_training_pair_long_memory(dtype, B, H, T, D, saved_pair):
    announce(f"segmented training pair {dtype} B{B} H{H} T{T} d{D} {'saved' if saved_pair else 'recompute'}")
    inp = long_memory_inputs(B, H, T, D, dtype, seed=500 + D)
    rng = np.random.default_rng(501)
    S0 = np.asarray(rng.standard_normal((B, H, D, D)), np.float32).astype(np.float64)
    dS_T = np.asarray(rng.standard_normal((B, H, D, D)), np.float32).astype(np.float64)
    got = run_pair(inp, dtype, S0, dS_T, saved_pair)
    ref = reference(inp, S0, dS_T)
    errs = {k_: max_rel(got[k_], ref[k_]) for k_ in ("o", "S_T") + NAMES}
    print("  " + " ".join(f"{k_}={v_:.2e}" for k_, v_ in errs.items()), flush=True)
    assert all(v_ <= TOL[dtype] for v_ in errs.values()), errs


@pytest.mark.parametrize("dtype,B,H,T,D", SEG_CASES, ids=[f"{c[0]}_d{c[4]}_T{c[3]}" for c in SEG_CASES])
def test_segmented_reverse_carries_late_output_gradient(dtype, B, H, T, D):
    """dO is zero except on the last 64 tokens and dS_T = 0: every gradient of the first
    segment's tokens and dS0 arrive only through the reverse scan of the segment maps."""
    announce(f"segmented reverse carry {dtype} T{T} d{D}")
    inp = long_memory_inputs(B, H, T, D, dtype, seed=520 + D)
    inp["dO"] = inp["dO"].copy()
    inp["dO"][:, :, :-64] = 0.0
    if dtype == "bf16":
        bits = inp["dO_bits"].copy()
        bits[:, :, :-64] = 0
        inp["dO_bits"] = bits
    S0 = np.asarray(np.random.default_rng(521).standard_normal((B, H, D, D)), np.float32).astype(np.float64)
    dS_T = np.zeros((B, H, D, D))
    got = run_pair(inp, dtype, S0, dS_T, True)
    ref = reference(inp, S0, dS_T)
    first = T // 4       # tokens of the first segment(s)
    # dq_t = S_t^T dO_t is local: exactly zero where dO is
    assert np.all(ref["dq"][:, :, :first] == 0) and np.all(got["dq"][:, :, :first] == 0)
    for key in ("dk", "dv", "dlog_g"):
        r = ref[key][:, :, :first]
        assert np.max(np.abs(r)) > 1e-3 * np.max(np.abs(ref[key])), key     # carried, not vanishing
        e = max_rel(got[key][:, :, :first], r)
        print(f"  {key} first {first} tokens: err {e:.2e}", flush=True)
        assert e <= TOL[dtype], (key, e)
    e = max_rel(got["dS0"], ref["dS0"])
    print(f"  dS0 err {e:.2e}", flush=True)
    assert e <= TOL[dtype]


def test_segmented_reverse_matches_sequential():
    """The same two heads run segmented (alone: B1 H2) and sequentially (inside a batch of
    32 heads, which fills the compute units without segments) agree to rounding, through
    fwd_save + bwd_saved."""
    announce("segmented vs sequential reverse pass")
    D, T = 128, 64 * 64 + 30
    inp = random_inputs(16, 2, T, D, D, dtype="bf16", seed=78, erase="sigmoid", dists="softplus_decay",
                        with_dO=True)
    d = to_device(inp, "bf16")
    dS_T = torch.randn((16, 2, D, D), device="cuda") * 0.3

    def pair(x, dst):
        o, S_T, saved = carve.fwd_save(x["q"], x["k"], x["v"], x["log_g"], x["w"], b=x["b"])
        return carve.bwd_saved(x["q"], x["k"], x["v"], x["log_g"], x["w"], x["dO"], saved, b=x["b"], dS_T=dst,
                               want_dS0=True)

    g_all = pair(d, dS_T)
    sub = {k_: v_[5:6].contiguous() for k_, v_ in d.items()}
    g_one = pair(sub, dS_T[5:6].contiguous())
    torch.cuda.synchronize()
    for key in ("dq", "dk", "dv", "dlog_g", "db", "dw", "dS0"):
        e = max_rel(to_np(g_one[key]), to_np(g_all[key][5:6]))
        print(f"  {key} diff {e:.2e}", flush=True)
        assert e <= 1e-2, (key, e)
