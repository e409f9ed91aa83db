"""GPU forward parity against the float64 reference (needs an MI355X).

Error metric: per tensor, max|gpu - ref| / max|ref|.  Bars: 1e-4 for float32
inputs, 2e-2 for bfloat16 inputs.  Both sides consume the same (already
rounded) input values, so input quantisation is not counted.
"""
import zlib

import numpy as np
import pytest
import torch

import oracle
from chunk_gated_delta_amd import carve
from chunk_gated_delta_amd.synth import WORKLOADS, make_inputs, random_inputs
from tests.helpers import max_rel, to_device, to_np

pytestmark = pytest.mark.gpu
TOL = {"f32": 1e-4, "bf16": 2e-2}


def announce(name):
    print(f"\n[case] {name}", flush=True)


def run_gpu(inp, dtype, L, S0=None, content=None):
    d = to_device(inp, dtype)
    S0d = None if S0 is None else torch.from_numpy(np.asarray(S0, np.float32)).cuda()
    cont = None
    if content is not None:
        cont = {"b_x": d["b_x"], "U1": content.get("U1"), "U2": content.get("U2"), "m0": content.get("m0")}
    o, S_T, m = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d.get("b"), S0=S0d, L=L, content=cont)
    torch.cuda.synchronize()
    return to_np(o), to_np(S_T), (None if m is None else to_np(m))


def run_ref(inp, L, S0=None, content=None):
    return oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"], b=inp.get("b"), S0=S0, L=L,
                          content=content)


CASES = [
    # name, B, H, T, D, dtype, L, erase, dists
    ("tiny_f32_full", 1, 2, 256, 64, "f32", 64, "none", "uniform_decay"),
    ("f32_d64_ragged", 2, 1, 77, 64, "f32", 64, "sigmoid", "softplus_decay"),
    ("f32_d128_tile32", 1, 2, 100, 128, "f32", 64, "sigmoid", "softplus_decay"),
    ("bf16_d128_ragged", 2, 2, 200, 128, "bf16", 64, "sigmoid", "softplus_decay"),
    ("bf16_d128_L32", 1, 3, 160, 128, "bf16", 32, "none", "uniform_decay"),
    ("bf16_d64", 2, 2, 300, 64, "bf16", 64, "ones", "uniform_decay"),
    ("bf16_d64_L16", 1, 2, 50, 64, "bf16", 16, "sigmoid", "softplus_decay"),
    ("f32_T1", 1, 1, 1, 64, "f32", 64, "sigmoid", "uniform_decay"),
]


@pytest.mark.parametrize("name,B,H,T,D,dtype,L,erase,dists", CASES, ids=[c[0] for c in CASES])
def test_fwd_parity(name, B, H, T, D, dtype, L, erase, dists):
    announce(name)
    inp = random_inputs(B, H, T, D, D, dtype=dtype, seed=zlib.crc32(name.encode()) % 1000, erase=erase, dists=dists)
    rng = np.random.default_rng(5)
    S0 = np.asarray(rng.standard_normal((B, H, D, D)) * 0.3, np.float32).astype(np.float64)
    o, S_T, _ = run_gpu(inp, dtype, L, S0=S0)
    ro, rS, _ = run_ref(inp, L, S0=S0)
    eo, es = max_rel(o, ro), max_rel(S_T, rS)
    print(f"  err o={eo:.2e} S_T={es:.2e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


# Few heads and many chunks: the state pass runs as segments whose affine maps are
# chained by a scan (B*H*Dk/16 < 256 compute units' worth of 16-row slices, at least
# 32 chunks).  Ragged lengths put a partial chunk in the last segment.
SEG_CASES = [
    # name, B, H, T, D, dtype
    ("seg_bf16_d128", 1, 2, 64 * 100 + 5, 128, "bf16"),
    ("seg_f32_d64", 2, 1, 32 * 70 + 9, 64, "f32"),
    ("seg_bf16_d64_exact", 1, 3, 64 * 48, 64, "bf16"),
]


@pytest.mark.parametrize("name,B,H,T,D,dtype", SEG_CASES, ids=[c[0] for c in SEG_CASES])
def test_segmented_state_pass_parity(name, B, H, T, D, dtype):
    announce(f"segmented {name} T{T}")
    inp = random_inputs(B, H, T, D, D, dtype=dtype, seed=zlib.crc32(name.encode()) % 1000, erase="sigmoid",
                        dists="softplus_decay")
    S0 = np.asarray(np.random.default_rng(6).standard_normal((B, H, D, D)) * 0.3, np.float32).astype(np.float64)
    o, S_T, _ = run_gpu(inp, dtype, 64, S0=S0)
    ro, rS, _ = run_ref(inp, 64, S0=S0)
    eo, es = max_rel(o, ro), max_rel(S_T, rS)
    print(f"  err o={eo:.2e} S_T={es:.2e}", flush=True)
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_segmented_matches_sequential_pass():
    """The same two heads run segmented (alone) and sequentially (inside a batch of
    32 heads, which fills the compute units without segments) agree to rounding."""
    announce("segmented vs sequential state pass")
    D, T = 128, 64 * 64 + 30
    inp = random_inputs(16, 2, T, D, D, dtype="bf16", seed=77, erase="sigmoid", dists="softplus_decay")
    d = to_device(inp, "bf16")
    o_all, S_all, _ = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d["b"], L=64)
    sub = {k_: v_[3:4].contiguous() for k_, v_ in d.items()}
    o_one, S_one, _ = carve.fwd(sub["q"], sub["k"], sub["v"], sub["log_g"], sub["w"], b=sub["b"], L=64)
    torch.cuda.synchronize()
    eo = max_rel(to_np(o_one), to_np(o_all[3:4]))
    es = max_rel(to_np(S_one), to_np(S_all[3:4]))
    print(f"  diff o={eo:.2e} S_T={es:.2e}", flush=True)
    assert eo <= 1e-2 and es <= 1e-2


def long_memory_inputs(B, H, T, D, dtype, seed):
    """Slow key-axis decay (a in [0.9995, 1]) and a small write gate (w in [0, 0.05]):
    most of the state entering a segment survives it, so the segments' maps Pi carry
    real weight (with the workload decays they underflow to nothing over a segment)."""
    inp = random_inputs(B, H, T, D, D, dtype=dtype, seed=seed, erase="none", dists="uniform_decay")
    rng = np.random.default_rng(seed + 1)
    inp["log_g"] = rng.uniform(np.log(0.9995), 0.0, (B, H, T, D)).astype(np.float32).astype(np.float64)
    inp["w"] = rng.uniform(0.0, 0.05, (B, H, T)).astype(np.float32).astype(np.float64)
    inp.pop("b", None)
    return inp


LONG_MEMORY_CASES = [("bf16", 128, 64 * 100 + 5), ("f32", 64, 32 * 70 + 9)]


@pytest.mark.parametrize("dtype,D,T", LONG_MEMORY_CASES, ids=[f"{c[0]}_d{c[1]}" for c in LONG_MEMORY_CASES])
def test_segmented_long_memory_parity(dtype, D, T):
    announce(f"segmented long memory {dtype} d{D} T{T}")
    B, H = 1, 2
    inp = long_memory_inputs(B, H, T, D, dtype, seed=90 + D)
    S0 = np.asarray(np.random.default_rng(8).standard_normal((B, H, D, D)), np.float32).astype(np.float64)
    o, S_T, _ = run_gpu(inp, dtype, 64, S0=S0)
    ro, rS, _ = run_ref(inp, 64, S0=S0)
    eo, es = max_rel(o, ro), max_rel(S_T, rS)
    # S0 still shapes the last outputs: the carry through every segment map matters
    ro0, _, _ = run_ref(inp, 64, S0=None)
    carried = max_rel(ro0[:, :, -64:], ro[:, :, -64:])
    print(f"  err o={eo:.2e} S_T={es:.2e}; S0's share of the last chunk's outputs {carried:.2e}", flush=True)
    assert carried > 0.1
    assert eo <= TOL[dtype] and es <= TOL[dtype]


def test_segmented_long_memory_matches_sequential():
    announce("segmented vs sequential, long memory")
    D, T = 128, 64 * 64 + 30
    inp = long_memory_inputs(16, 2, T, D, "bf16", seed=78)
    d = to_device(inp, "bf16")
    S0 = torch.from_numpy(np.asarray(np.random.default_rng(9).standard_normal((16, 2, D, D)), np.float32)).cuda()
    o_all, S_all, _ = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], S0=S0, L=64)
    sub = {k_: v_[5:6].contiguous() for k_, v_ in d.items()}
    o_one, S_one, _ = carve.fwd(sub["q"], sub["k"], sub["v"], sub["log_g"], sub["w"], S0=S0[5:6].contiguous(), L=64)
    torch.cuda.synchronize()
    eo = max_rel(to_np(o_one), to_np(o_all[5:6]))
    es = max_rel(to_np(S_one), to_np(S_all[5:6]))
    print(f"  diff o={eo:.2e} S_T={es:.2e}", flush=True)
    assert eo <= 1e-2 and es <= 1e-2


def test_tiny_f32_workload_zero_state():
    wl = WORKLOADS["tiny_f32"]
    announce(wl.name)
    inp = make_inputs(wl)
    o, S_T, _ = run_gpu(inp, "f32", wl.L)
    ro, rS, _ = run_ref(inp, wl.L)
    assert max_rel(o, ro) <= 1e-4 and max_rel(S_T, rS) <= 1e-4


def test_chunk_size_independence():
    """Token-only gates: the result does not depend on L (16, 32, 64, 128 use different tilings)."""
    announce("chunk_size_independence")
    inp = random_inputs(1, 2, 256, 128, 128, dtype="bf16", seed=31, erase="sigmoid", dists="softplus_decay")
    ro, rS, _ = run_ref(inp, 64)
    outs = {}
    for L in (16, 32, 64, 128):
        o, S_T, _ = run_gpu(inp, "bf16", L)
        assert max_rel(o, ro) <= 2e-2 and max_rel(S_T, rS) <= 2e-2, L
        outs[L] = o
    assert max_rel(outs[16], outs[32]) == 0.0          # same 32-token tiling
    assert max_rel(outs[64], outs[128]) == 0.0         # same 64-token tiling
    assert max_rel(outs[32], outs[64]) <= 2e-2


def test_state_carry_split():
    """One call over T equals two calls over T/2 with the state carried."""
    announce("state_carry_split")
    inp = random_inputs(2, 2, 256, 128, 128, dtype="bf16", seed=32, erase="sigmoid", dists="softplus_decay")
    d = to_device(inp, "bf16")
    o_full, S_full, _ = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], b=d["b"], L=64)
    h = 128
    sl = lambda t: t[:, :, :h].contiguous()
    sr = lambda t: t[:, :, h:].contiguous()
    o1, S1, _ = carve.fwd(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["log_g"]), sl(d["w"]), b=sl(d["b"]), L=64)
    o2, S2, _ = carve.fwd(sr(d["q"]), sr(d["k"]), sr(d["v"]), sr(d["log_g"]), sr(d["w"]), b=sr(d["b"]), S0=S1,
                          L=64)
    torch.cuda.synchronize()
    # the split at a tile boundary performs the same arithmetic: bit-identical
    assert torch.equal(torch.cat([o1, o2], 2), o_full)
    assert torch.equal(S2, S_full)


def test_determinism():
    announce("determinism")
    inp = random_inputs(2, 4, 512, 128, 128, dtype="bf16", seed=33, erase="sigmoid", dists="softplus_decay")
    a = run_gpu(inp, "bf16", 64)
    b = run_gpu(inp, "bf16", 64)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_empty_inputs():
    announce("empty_inputs")
    for (B, H, T) in [(1, 2, 0), (0, 2, 16)]:
        q = torch.zeros((B, H, T, 64), dtype=torch.bfloat16, device="cuda")
        lg = torch.zeros((B, H, T, 64), dtype=torch.float32, device="cuda")
        w = torch.zeros((B, H, T), dtype=torch.float32, device="cuda")
        S0 = torch.randn((B, H, 64, 64), device="cuda")
        o, S_T, _ = carve.fwd(q, q, q, lg, w, S0=S0)
        torch.cuda.synchronize()
        assert o.shape == (B, H, T, 64)
        assert torch.equal(S_T, S0)


# ----------------------------------------------------------- content-aware erase

def content_inputs(B, H, T, D, dtype, seed, scale=1.0, R=16):
    inp = random_inputs(B, H, T, D, D, dtype=dtype, seed=seed, erase="content", dists="softplus_decay", rank=R)
    inp["U1"] = inp["U1"] * scale
    inp["U2"] = inp["U2"] * scale
    return inp


@pytest.mark.parametrize("dtype,D,L,T,scale", [("f32", 64, 64, 200, 8.0), ("bf16", 128, 64, 256, 8.0),
                                               ("bf16", 128, 128, 320, 8.0), ("bf16", 64, 32, 100, 8.0)])
def test_content_parity(dtype, D, L, T, scale):
    announce(f"content {dtype} D{D} L{L} T{T}")
    inp = content_inputs(2, 2, T, D, dtype, seed=40 + D + L, scale=scale)
    d = to_device(inp, dtype)
    m0 = np.random.default_rng(1).standard_normal((2, 2, D)) * 0.5
    m0 = np.asarray(m0, np.float32).astype(np.float64)
    cont_gpu = {"U1": d["U1"], "U2": d["U2"], "m0": torch.from_numpy(m0.astype(np.float32)).cuda()}
    o, S_T, m = run_gpu(inp, dtype, L, content=cont_gpu)
    ro, rS, rm = run_ref(inp, L, content={"b_x": inp["b_x"], "U1": inp["U1"], "U2": inp["U2"], "m0": m0})
    errs = (max_rel(o, ro), max_rel(S_T, rS), max_rel(m, rm))
    print(f"  err o={errs[0]:.2e} S_T={errs[1]:.2e} m={errs[2]:.2e}", flush=True)
    assert max(errs) <= TOL[dtype]
    # the content signal must matter at this scale (else the test pins nothing)
    ro0, _, _ = run_ref(inp, L, content={"b_x": inp["b_x"], "U1": None, "U2": None})
    print(f"  content effect on o: {max_rel(ro0, ro):.2e}", flush=True)
    assert max_rel(ro0, ro) > 0.02


@pytest.mark.parametrize("dtype,D,L,R", [("bf16", 64, 64, 64), ("f32", 128, 32, 40)])
def test_content_parity_high_rank(dtype, D, L, R):
    """Projection ranks above 16 (up to the largest, 64): the signal's first product runs in
    several passes over the rows of U1."""
    announce(f"content {dtype} D{D} L{L} rank {R}")
    T = 3 * L + 11
    inp = content_inputs(2, 2, T, D, dtype, seed=60 + D + R, scale=32.0, R=R)
    d = to_device(inp, dtype)
    o, S_T, m = run_gpu(inp, dtype, L, content={"U1": d["U1"], "U2": d["U2"]})
    ro, rS, rm = run_ref(inp, L, content={"b_x": inp["b_x"], "U1": inp["U1"], "U2": inp["U2"]})
    errs = (max_rel(o, ro), max_rel(S_T, rS), max_rel(m, rm))
    ro0, _, _ = run_ref(inp, L, content={"b_x": inp["b_x"], "U1": None, "U2": None})
    print(f"  err o={errs[0]:.2e} S_T={errs[1]:.2e} m={errs[2]:.2e}; content effect {max_rel(ro0, ro):.2e}", flush=True)
    assert max(errs) <= TOL[dtype]
    assert max_rel(ro0, ro) > 0.02


def test_content_zero_projection_bit_exact():
    """U_b = 0 reproduces the U_b-absent path bit for bit (o, S_T and m_out)."""
    announce("content_zero_projection_bit_exact")
    inp = content_inputs(2, 3, 256, 128, "bf16", seed=50)
    d = to_device(inp, "bf16")
    z1 = torch.zeros_like(d["U1"])
    z2 = torch.zeros_like(d["U2"])
    oz, sz, mz = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], L=64,
                           content={"b_x": d["b_x"], "U1": z1, "U2": z2})
    oa, sa, ma = carve.fwd(d["q"], d["k"], d["v"], d["log_g"], d["w"], L=64,
                           content={"b_x": d["b_x"], "U1": None, "U2": None})
    torch.cuda.synchronize()
    assert torch.equal(oz, oa) and torch.equal(sz, sa) and torch.equal(mz, ma)
    # and both match the token-only reference fed b = sigmoid(b_x)
    ro, rS, _ = oracle.forward(inp["q"], inp["k"], inp["v"], inp["log_g"], inp["w"],
                               b=1 / (1 + np.exp(-inp["b_x"])))
    assert max_rel(to_np(oz), ro) <= 2e-2 and max_rel(to_np(sz), rS) <= 2e-2
