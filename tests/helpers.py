"""Shared test helpers: move seeded synthetic inputs to the device and compare."""
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
