"""Seeded synthetic inputs for the CARVE key-axis gated delta rule.

This module only draws random numbers and rounds them to the dtypes the
kernels receive; it holds none of the operation's arithmetic, so both the HIP
path and the float64 reference can consume its output.

Every workload draws from numpy's PCG64 generator, seeded per workload, in a
fixed order: q, k, v, log_g, b (or b_x), w, dO, U1, U2.  q and k are drawn
N(0, 1) and L2-normalised per token in float64 (the caller-side normalisation
the pages assume, since the operation itself applies no query/key scaling),
then rounded once (round-to-nearest-even) to the workload's dtype.  Both sides
then see exactly the same values, so input quantisation is not counted as
kernel error.  Gates and states are float32 on the device; they are rounded
to float32 here for the same reason.

The distributions follow the workload descriptions: the tiny float32 case
and the long-context / training cases use log a ~ U(log 0.9, 0), b = 1 and
w = sigmoid(N(0, 1)); the 1.3B-head-shape case uses log g = -0.1 softplus(N(0,1)),
b = sigmoid(N(2, 1)); the content-erase case adds b_x ~ N(2, 1) and a rank-16
projection with entries N(0, 0.02^2) (0.02 read as a standard deviation).
"""

from dataclasses import dataclass, field
import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    Dk: int
    Dv: int
    L: int
    dtype: str              # "f32" or "bf16": dtype of q, k, v, o (and dO, dq, dk, dv)
    dists: str              # "uniform_decay" or "softplus_decay"
    erase: str              # "none" (b = NULL), "ones" (b = 1 tensor), "sigmoid" (b = sigmoid(N(2,1))), "content"
    backward: bool = False
    rank: int = 16
    seed: int = 0
    note: str = field(default="", compare=False)


WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", 1, 2, 256, 64, 64, 64, "f32", "uniform_decay", "none", seed=1001,
                         note="B1 H2 T256 d64 L64, fp32 inputs"),
    "head1p3b_fwd": Workload("head1p3b_fwd", 4, 16, 4096, 128, 128, 64, "bf16", "softplus_decay", "sigmoid",
                             seed=1002, note="B4 H16 T4096 d128 L64, bf16"),
    "long_ctx_fwd": Workload("long_ctx_fwd", 1, 16, 32768, 128, 128, 64, "bf16", "uniform_decay", "none",
                             seed=1003, note="B1 H16 T32768 d128 L64, bf16, S_T compared"),
    "content_fwd": Workload("content_fwd", 4, 16, 4096, 128, 128, 64, "bf16", "softplus_decay", "content",
                            seed=1004, note="B4 H16 T4096 d128 L64, content-aware erase, rank 16"),
    "train_fwd_bwd": Workload("train_fwd_bwd", 8, 16, 2048, 128, 128, 64, "bf16", "uniform_decay", "ones",
                              backward=True, seed=1005, note="B8 H16 T2048 d128 L64, fwd+bwd"),
}


def round_bf16_bits(x):
    """Round float64 values to bfloat16 (via float32, round-to-nearest-even).

    Returns (bits as uint16, the rounded values as float64)."""
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x32.view(np.uint32).astype(np.uint64)
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    back = (rounded.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return rounded, back


def round_f32(x):
    return np.asarray(x, dtype=np.float32).astype(np.float64)


def _l2norm(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x):
    return np.logaddexp(0.0, x)


class Inputs(dict):
    """dict of float64 arrays (the exact values both sides consume) plus, for
    bf16 workloads, the raw bf16 bit patterns under '<name>_bits'."""


def make_inputs(wl, B=None, H=None, T=None, seed=None, with_dO=None):
    """Draw the inputs of workload `wl` (optionally overriding B, H, T, seed).

    Keys: q, k, v, log_g, w, and b (erase "sigmoid"/"ones"), or b_x, U1, U2
    (erase "content"), and dO when the workload has a backward pass or
    with_dO is set.  Float tensors of dtype bf16 also carry '<key>_bits'."""
    B = wl.B if B is None else B
    H = wl.H if H is None else H
    T = wl.T if T is None else T
    seed = wl.seed if seed is None else seed
    with_dO = wl.backward if with_dO is None else with_dO
    rng = np.random.Generator(np.random.PCG64(seed))
    Dk, Dv = wl.Dk, wl.Dv
    out = Inputs()

    def act(name, x):
        if wl.dtype == "bf16":
            bits, vals = round_bf16_bits(x)
            out[name] = vals
            out[name + "_bits"] = bits
        else:
            out[name] = round_f32(x)

    act("q", _l2norm(rng.standard_normal((B, H, T, Dk))))
    act("k", _l2norm(rng.standard_normal((B, H, T, Dk))))
    act("v", rng.standard_normal((B, H, T, Dv)))
    if wl.dists == "uniform_decay":
        out["log_g"] = round_f32(rng.uniform(np.log(0.9), 0.0, (B, H, T, Dk)))
    else:
        out["log_g"] = round_f32(-0.1 * _softplus(rng.standard_normal((B, H, T, Dk))))
    if wl.erase == "sigmoid":
        out["b"] = round_f32(_sigmoid(rng.normal(2.0, 1.0, (B, H, T, Dk))))
    elif wl.erase == "ones":
        out["b"] = np.ones((B, H, T, Dk))
    elif wl.erase == "content":
        out["b_x"] = round_f32(rng.normal(2.0, 1.0, (B, H, T, Dk)))
    out["w"] = round_f32(_sigmoid(rng.standard_normal((B, H, T))))
    if with_dO:
        act("dO", rng.standard_normal((B, H, T, Dv)))
    if wl.erase == "content":
        out["U1"] = round_f32(rng.normal(0.0, 0.02, (H, wl.rank, Dv)))
        out["U2"] = round_f32(rng.normal(0.0, 0.02, (H, Dk, wl.rank)))
    return out


def random_inputs(B, H, T, Dk, Dv, dtype="f32", seed=0, erase="none", dists="uniform_decay",
                  with_dO=False, rank=16):
    """Inputs of an arbitrary shape with one of the workload recipes."""
    wl = Workload("custom", B, H, T, Dk, Dv, 64, dtype, dists, erase, backward=with_dO, rank=rank, seed=seed)
    return make_inputs(wl)
