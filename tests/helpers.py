"""Shared test helpers: move seeded synthetic inputs to the device, compare, and draw hard
gate runs (strong decay, hard erase) for the range tests."""
import numpy as np
import torch


def dev_tensor(inp, key, device, dtype):
    """Device tensor holding exactly the values the reference sees."""
    if dtype == "bf16" and key + "_bits" in inp:
        bits = np.ascontiguousarray(inp[key + "_bits"]).view(np.int16)
        return torch.from_numpy(bits).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(inp[key], dtype=np.float32)).to(device)


def to_device(inp, dtype, device="cuda"):
    out = {}
    for key in ("q", "k", "v", "dO"):
        if key in inp:
            out[key] = dev_tensor(inp, key, device, dtype)
    for key in ("log_g", "b", "w", "b_x", "U1", "U2"):
        if key in inp:
            out[key] = torch.from_numpy(np.ascontiguousarray(inp[key], dtype=np.float32)).to(device)
    return out


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_rel(gpu, ref):
    """max |gpu - ref| / max |ref| over the whole tensor (max-normalised error)."""
    ref = np.asarray(ref, np.float64)
    gpu = np.asarray(gpu, np.float64)
    den = np.max(np.abs(ref))
    return float(np.max(np.abs(gpu - ref)) / (den if den > 0 else 1.0))


def per_head_rel(gpu, ref):
    """[B, H] array: max |gpu - ref| / max |ref| within each (batch, head) sequence."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    ax = tuple(range(2, ref.ndim))
    den = np.max(np.abs(ref), axis=ax) if ax else np.abs(ref)
    num = np.max(np.abs(gpu - ref), axis=ax) if ax else np.abs(gpu - ref)
    return num / np.where(den > 0, den, 1.0)


def hard_runs(rng, B, H, T, D, frac, lo, hi, run=(4, 24)):
    """Mask of runs of tokens (lengths in `run`) on a random fraction of key channels,
    and log-uniform values in [lo, hi] for them."""
    mask = np.zeros((B, H, T, D), bool)
    for b in range(B):
        for h in range(H):
            chans = rng.choice(D, int(frac * D), replace=False)
            for c in chans:
                t = int(rng.integers(0, max(T // 8, 1)))
                while t < T:
                    n = int(rng.integers(run[0], run[1] + 1))
                    mask[b, h, t:t + n, c] = True
                    t += n + int(rng.integers(8, 64))
    vals = np.exp(rng.uniform(np.log(lo), np.log(hi), (B, H, T, D)))
    return mask, vals
