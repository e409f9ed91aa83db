"""Python binding of libcarve.so (ctypes).

Argument marshalling only: every step of the operation runs in the HIP
kernels behind the C ABI (include/carve.h).  PyTorch supplies device memory
(outputs and workspace are allocated with torch on the inputs' device) and
the current HIP stream.  There is no CPU fallback: if the library is missing
or a call is rejected, a RuntimeError is raised.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcarve.so")

CARVE_F32 = 0
CARVE_BF16 = 1


class carve_shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("T", ctypes.c_int),
                ("Dk", ctypes.c_int), ("Dv", ctypes.c_int), ("L", ctypes.c_int), ("dtype", ctypes.c_int)]


class carve_content(ctypes.Structure):
    _fields_ = [("b_x", ctypes.c_void_p), ("U1", ctypes.c_void_p), ("U2", ctypes.c_void_p),
                ("R", ctypes.c_int), ("m0", ctypes.c_void_p), ("m_out", ctypes.c_void_p),
                ("z_rec", ctypes.c_void_p), ("m_rec", ctypes.c_void_p)]


def content_records(B, H, T, Dk, Dv, L, device):
    """Per-period record buffers (z_rec [B,H,P,Dk], m_rec [B,H,P,Dv], P = ceil(T / L)) for the
    content dict of fwd (which fills them) and bwd_content (which then skips re-running the
    content-aware forward)."""
    P = (T + L - 1) // L
    return (torch.empty((B, H, P, Dk), dtype=torch.float32, device=device),
            torch.empty((B, H, P, Dv), dtype=torch.float32, device=device))


def _records(content, B, H, T, Dk, Dv, L, dev):
    """Pointers of the content dict's record tensors (both or neither)."""
    zr, mr = content.get("z_rec"), content.get("m_rec")
    if (zr is None) != (mr is None):
        raise ValueError("z_rec and m_rec are given together")
    if zr is None:
        return None, None
    P = (T + L - 1) // L
    _check(zr, "z_rec", (B, H, P, Dk), torch.float32, dev)
    _check(mr, "m_rec", (B, H, P, Dv), torch.float32, dev)
    return zr.data_ptr(), mr.data_ptr()


class carve_gate_logits(ctypes.Structure):
    _fields_ = [("f", ctypes.c_void_p), ("A", ctypes.c_void_p), ("tau", ctypes.c_void_p), ("b_x", ctypes.c_void_p),
                ("w_hat", ctypes.c_void_p)]


class carve_decode_content(ctypes.Structure):
    _fields_ = [("b_x", ctypes.c_void_p), ("U1", ctypes.c_void_p), ("U2", ctypes.c_void_p),
                ("R", ctypes.c_int), ("m_in", ctypes.c_void_p), ("m_out", ctypes.c_void_p),
                ("csum", ctypes.c_void_p), ("pos", ctypes.c_int)]


class carve_profile(ctypes.Structure):
    _fields_ = [("events", ctypes.c_void_p * 9), ("n_events", ctypes.c_int)]


def make_profile(events):
    """carve_profile from torch.cuda.Event objects (each recorded once so its handle exists)."""
    prof = carve_profile()
    for i, ev in enumerate(events):
        prof.events[i] = ev.cuda_event
    prof.n_events = len(events)
    return prof


_lib = None


def load_library():
    """Load libcarve.so (built in-tree by chunk_gated_delta_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m chunk_gated_delta_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    sp = ctypes.POINTER(carve_shape)
    cp = ctypes.POINTER(carve_content)
    lib.carve_fwd_workspace_size.argtypes = [sp, cp]
    lib.carve_fwd_workspace_size.restype = sz
    lib.carve_bwd_workspace_size.argtypes = [sp]
    lib.carve_bwd_workspace_size.restype = sz
    lib.carve_fwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, cp, vp, vp, vp, sz, vp]
    lib.carve_fwd.restype = i
    pp = ctypes.POINTER(carve_profile)
    lib.carve_fwd_ex.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, cp, vp, vp, vp, sz, vp, pp]
    lib.carve_fwd_ex.restype = i
    lib.carve_fwd_noalloc.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, cp, vp, vp, vp]
    lib.carve_fwd_noalloc.restype = i
    lib.carve_bwd_ex.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, pp]
    lib.carve_bwd_ex.restype = i
    lib.carve_bwd.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.carve_bwd.restype = i
    lib.carve_saved_size.argtypes = [sp]
    lib.carve_saved_size.restype = sz
    lib.carve_bwd_saved_workspace_size.argtypes = [sp]
    lib.carve_bwd_saved_workspace_size.restype = sz
    lib.carve_fwd_save.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, pp]
    lib.carve_fwd_save.restype = i
    lib.carve_bwd_saved.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                    vp, pp]
    lib.carve_bwd_saved.restype = i
    glp = ctypes.POINTER(carve_gate_logits)
    lib.carve_fwd_logits.argtypes = [sp, vp, vp, vp, glp, vp, vp, vp, vp, sz, vp]
    lib.carve_fwd_logits.restype = i
    lib.carve_bwd_logits_workspace_size.argtypes = [sp]
    lib.carve_bwd_logits_workspace_size.restype = sz
    lib.carve_bwd_logits.argtypes = [sp, vp, vp, vp, glp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.carve_bwd_logits.restype = i
    lib.carve_bwd_logits_saved_workspace_size.argtypes = [sp]
    lib.carve_bwd_logits_saved_workspace_size.restype = sz
    lib.carve_fwd_logits_save.argtypes = [sp, vp, vp, vp, glp, vp, vp, vp, vp, sz, vp, pp]
    lib.carve_fwd_logits_save.restype = i
    lib.carve_bwd_logits_saved.argtypes = [sp, vp, vp, vp, glp, vp, vp, vp, sz, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                           vp, sz, vp, pp]
    lib.carve_bwd_logits_saved.restype = i
    lib.carve_bwd_content_workspace_size.argtypes = [sp, cp]
    lib.carve_bwd_content_workspace_size.restype = sz
    lib.carve_bwd_content.argtypes = [sp, vp, vp, vp, vp, vp, vp, cp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                      vp, vp, vp, sz, vp]
    lib.carve_bwd_content.restype = i
    dcp = ctypes.POINTER(carve_decode_content)
    lib.carve_decode_step.argtypes = [sp, vp, vp, vp, vp, vp, vp, vp, dcp, vp, vp]
    lib.carve_decode_step.restype = i
    lib.carve_stream_copy.argtypes = [vp, vp, sz, vp]
    lib.carve_stream_copy.restype = i
    lib.carve_status_string.argtypes = [i]
    lib.carve_status_string.restype = ctypes.c_char_p
    lib.carve_abi_version.argtypes = []
    lib.carve_abi_version.restype = i
    _lib = lib
    return lib


def status_string(code):
    return load_library().carve_status_string(code).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return CARVE_BF16
    if t.dtype == torch.float32:
        return CARVE_F32
    raise TypeError(f"q/k/v must be float32 or bfloat16, got {t.dtype}")


def _check(t, name, shape, dtype, device):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _raise(code, what):
    if code != 0:
        raise RuntimeError(f"{what}: {status_string(code)}")


def make_shape(q, v, L):
    B, H, T, Dk = q.shape
    return carve_shape(B, H, T, Dk, v.shape[-1], L, _dtype_code(q))


def fwd_workspace_bytes(q, v, L=64, content=False):
    lib = load_library()
    s = make_shape(q, v, L)
    c = carve_content() if content else None
    return lib.carve_fwd_workspace_size(ctypes.byref(s), ctypes.byref(c) if c is not None else None)


def _fwd_args(q, k, v, log_g, w, b, S0, L, content, o, S_T, want_state):
    """Checks and marshalling shared by fwd and fwd_noalloc: (lib, shape, content struct or
    None, o, S_T, m_out, objects to keep alive during the call)."""
    lib = load_library()
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    dt = q.dtype
    _check(k, "k", (B, H, T, Dk), dt, dev)
    _check(v, "v", (B, H, T, Dv), dt, dev)
    _check(log_g, "log_g", (B, H, T, Dk), torch.float32, dev)
    _check(b, "b", (B, H, T, Dk), torch.float32, dev)
    _check(w, "w", (B, H, T), torch.float32, dev)
    _check(S0, "S0", (B, H, Dv, Dk), torch.float32, dev)
    s = make_shape(q, v, L)
    cs = None
    m_out = None
    keep = []
    if content is not None:
        bx = content["b_x"]
        U1 = content.get("U1")
        U2 = content.get("U2")
        m0 = content.get("m0")
        _check(bx, "b_x", (B, H, T, Dk), torch.float32, dev)
        R = 0
        if U1 is not None:
            R = U1.shape[1]
            _check(U1, "U1", (H, R, Dv), torch.float32, dev)
            _check(U2, "U2", (H, Dk, R), torch.float32, dev)
        _check(m0, "m0", (B, H, Dv), torch.float32, dev)
        m_out = torch.empty((B, H, Dv), dtype=torch.float32, device=dev)
        zr, mr = _records(content, B, H, T, Dk, Dv, L, dev)
        cs = carve_content(bx.data_ptr(), None if U1 is None else U1.data_ptr(),
                           None if U2 is None else U2.data_ptr(), R,
                           None if m0 is None else m0.data_ptr(), m_out.data_ptr(), zr, mr)
        keep.append(cs)
    if o is None:
        o = torch.empty((B, H, T, Dv), dtype=dt, device=dev)
    if S_T is None and want_state:
        S_T = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev)
    return lib, s, cs, o, S_T, m_out, keep


def fwd(q, k, v, log_g, w, b=None, S0=None, L=64, content=None, o=None, S_T=None, workspace=None,
        want_state=True, profile=None):
    """o, S_T, m_out = fwd(...).

    q, k [B,H,T,Dk], v [B,H,T,Dv] (float32 or bfloat16, one dtype); log_g, b [B,H,T,Dk]
    float32; w [B,H,T] float32; S0 [B,H,Dv,Dk] float32 or None.  content is None or a dict
    with b_x [B,H,T,Dk], U1 [H,R,Dv] / U2 [H,Dk,R] (or None), m0 [B,H,Dv] (or None), and
    optionally z_rec / m_rec (content_records), which the forward fills.
    Outputs may be passed preallocated (o, S_T, workspace)."""
    lib, s, cs, o, S_T, m_out, keep = _fwd_args(q, k, v, log_g, w, b, S0, L, content, o, S_T, want_state)
    dev = q.device
    need = lib.carve_fwd_workspace_size(ctypes.byref(s), ctypes.byref(cs) if cs is not None else None)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    code = lib.carve_fwd_ex(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(b), _ptr(w), _ptr(S0),
                            ctypes.byref(cs) if cs is not None else None, _ptr(o), _ptr(S_T),
                            _ptr(workspace), workspace.numel(), _stream(dev),
                            ctypes.byref(profile) if profile is not None else None)
    _raise(code, "carve_fwd")
    return o, S_T, m_out


def fwd_noalloc(q, k, v, log_g, w, b=None, S0=None, L=64, content=None, o=None, S_T=None, want_state=True):
    """fwd() through carve_fwd_noalloc: no workspace, the library's fixed device scratch
    instead (outputs may be passed preallocated; the C entry point itself allocates
    nothing).  Raises RuntimeError (CARVE_ERR_WORKSPACE) for shapes beyond the scratch."""
    lib, s, cs, o, S_T, m_out, keep = _fwd_args(q, k, v, log_g, w, b, S0, L, content, o, S_T, want_state)
    code = lib.carve_fwd_noalloc(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(b), _ptr(w),
                                 _ptr(S0), ctypes.byref(cs) if cs is not None else None, _ptr(o), _ptr(S_T),
                                 _stream(q.device))
    _raise(code, "carve_fwd_noalloc")
    return o, S_T, m_out


def bwd(q, k, v, log_g, w, dO, b=None, S0=None, dS_T=None, L=64, want_dS0=True, workspace=None, out=None,
        profile=None):
    """Gradients of the token-only forward: dict with dq, dk, dv, dlog_g, db (None if b is None),
    dw and dS0 (None unless want_dS0)."""
    lib = load_library()
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    dt = q.dtype
    _check(k, "k", (B, H, T, Dk), dt, dev)
    _check(v, "v", (B, H, T, Dv), dt, dev)
    _check(dO, "dO", (B, H, T, Dv), dt, dev)
    _check(log_g, "log_g", (B, H, T, Dk), torch.float32, dev)
    _check(b, "b", (B, H, T, Dk), torch.float32, dev)
    _check(w, "w", (B, H, T), torch.float32, dev)
    _check(S0, "S0", (B, H, Dv, Dk), torch.float32, dev)
    _check(dS_T, "dS_T", (B, H, Dv, Dk), torch.float32, dev)
    s = make_shape(q, v, L)
    g = out if out is not None else {}
    if out is None:
        g["dq"] = torch.empty_like(q)
        g["dk"] = torch.empty_like(k)
        g["dv"] = torch.empty_like(v)
        g["dlog_g"] = torch.empty_like(log_g)
        g["db"] = None if b is None else torch.empty_like(b)
        g["dw"] = torch.empty_like(w)
        g["dS0"] = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev) if want_dS0 else None
    need = lib.carve_bwd_workspace_size(ctypes.byref(s))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    code = lib.carve_bwd_ex(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(b), _ptr(w), _ptr(S0),
                            _ptr(dO), _ptr(dS_T), _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dlog_g"]),
                            _ptr(g["db"]), _ptr(g["dw"]), _ptr(g["dS0"]), _ptr(workspace), workspace.numel(),
                            _stream(dev), ctypes.byref(profile) if profile is not None else None)
    _raise(code, "carve_bwd")
    return g


def fwd_save(q, k, v, log_g, w, b=None, S0=None, L=64, o=None, S_T=None, saved=None, profile=None):
    """Forward (token-only gates) that also keeps what bwd_saved needs.

    Returns (o, S_T, saved); `saved` is a uint8 device buffer for bwd_saved."""
    lib = load_library()
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    dt = q.dtype
    _check(k, "k", (B, H, T, Dk), dt, dev)
    _check(v, "v", (B, H, T, Dv), dt, dev)
    _check(log_g, "log_g", (B, H, T, Dk), torch.float32, dev)
    _check(b, "b", (B, H, T, Dk), torch.float32, dev)
    _check(w, "w", (B, H, T), torch.float32, dev)
    _check(S0, "S0", (B, H, Dv, Dk), torch.float32, dev)
    s = make_shape(q, v, L)
    if o is None:
        o = torch.empty((B, H, T, Dv), dtype=dt, device=dev)
    if S_T is None:
        S_T = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev)
    need = lib.carve_saved_size(ctypes.byref(s))
    if saved is None or saved.numel() < need:
        saved = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    code = lib.carve_fwd_save(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(b), _ptr(w), _ptr(S0),
                              _ptr(o), _ptr(S_T), _ptr(saved), saved.numel(), _stream(dev),
                              ctypes.byref(profile) if profile is not None else None)
    _raise(code, "carve_fwd_save")
    return o, S_T, saved


def bwd_saved(q, k, v, log_g, w, dO, saved, b=None, dS_T=None, L=64, want_dS0=True, workspace=None, out=None,
              profile=None):
    """Backward from the buffer of fwd_save (same inputs): dict as bwd()."""
    lib = load_library()
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    dt = q.dtype
    _check(k, "k", (B, H, T, Dk), dt, dev)
    _check(v, "v", (B, H, T, Dv), dt, dev)
    _check(dO, "dO", (B, H, T, Dv), dt, dev)
    _check(log_g, "log_g", (B, H, T, Dk), torch.float32, dev)
    _check(b, "b", (B, H, T, Dk), torch.float32, dev)
    _check(w, "w", (B, H, T), torch.float32, dev)
    _check(dS_T, "dS_T", (B, H, Dv, Dk), torch.float32, dev)
    s = make_shape(q, v, L)
    g = out if out is not None else {}
    if out is None:
        g["dq"] = torch.empty_like(q)
        g["dk"] = torch.empty_like(k)
        g["dv"] = torch.empty_like(v)
        g["dlog_g"] = torch.empty_like(log_g)
        g["db"] = None if b is None else torch.empty_like(b)
        g["dw"] = torch.empty_like(w)
        g["dS0"] = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev) if want_dS0 else None
    need = lib.carve_bwd_saved_workspace_size(ctypes.byref(s))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    code = lib.carve_bwd_saved(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(b), _ptr(w), _ptr(dO),
                               _ptr(dS_T), _ptr(saved), saved.numel(), _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]),
                               _ptr(g["dlog_g"]), _ptr(g["db"]), _ptr(g["dw"]), _ptr(g["dS0"]), _ptr(workspace),
                               workspace.numel(), _stream(dev),
                               ctypes.byref(profile) if profile is not None else None)
    _raise(code, "carve_bwd_saved")
    return g


def _gate_logits(q, f, A, tau, w_hat, b_x):
    B, H, T, Dk = q.shape
    dev = q.device
    _check(f, "f", (B, H, T, Dk), torch.float32, dev)
    _check(A, "A", (H, Dk), torch.float32, dev)
    _check(tau, "tau", (H, Dk), torch.float32, dev)
    _check(w_hat, "w_hat", (B, H, T), torch.float32, dev)
    _check(b_x, "b_x", (B, H, T, Dk), torch.float32, dev)
    return carve_gate_logits(f.data_ptr(), A.data_ptr(), tau.data_ptr(), None if b_x is None else b_x.data_ptr(),
                             w_hat.data_ptr())


def fwd_logits(q, k, v, f, A, tau, w_hat, b_x=None, S0=None, L=64, o=None, S_T=None, workspace=None):
    """o, S_T with the gates given as pre-activations: log g = -A softplus(f + tau),
    b = sigmoid(b_x) (None: b = 1), w = sigmoid(w_hat); f, b_x [B,H,T,Dk], A, tau [H,Dk],
    w_hat [B,H,T], all float32."""
    lib = load_library()
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    _check(k, "k", (B, H, T, Dk), q.dtype, dev)
    _check(v, "v", (B, H, T, Dv), q.dtype, dev)
    _check(S0, "S0", (B, H, Dv, Dk), torch.float32, dev)
    g = _gate_logits(q, f, A, tau, w_hat, b_x)
    s = make_shape(q, v, L)
    if o is None:
        o = torch.empty((B, H, T, Dv), dtype=q.dtype, device=dev)
    if S_T is None:
        S_T = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev)
    need = lib.carve_fwd_workspace_size(ctypes.byref(s), None)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    code = lib.carve_fwd_logits(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(g), _ptr(S0), _ptr(o),
                                _ptr(S_T), _ptr(workspace), workspace.numel(), _stream(dev))
    _raise(code, "carve_fwd_logits")
    return o, S_T


def bwd_logits(q, k, v, f, A, tau, w_hat, dO, b_x=None, S0=None, dS_T=None, L=64, want_dS0=True, workspace=None):
    """Gradients of fwd_logits: dict with dq, dk, dv, df, dA, dtau, db_x (None without
    b_x), dw_hat and dS0 (None unless want_dS0)."""
    lib = load_library()
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    _check(k, "k", (B, H, T, Dk), q.dtype, dev)
    _check(v, "v", (B, H, T, Dv), q.dtype, dev)
    _check(dO, "dO", (B, H, T, Dv), q.dtype, dev)
    _check(S0, "S0", (B, H, Dv, Dk), torch.float32, dev)
    _check(dS_T, "dS_T", (B, H, Dv, Dk), torch.float32, dev)
    g = _gate_logits(q, f, A, tau, w_hat, b_x)
    s = make_shape(q, v, L)
    out = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v), "df": torch.empty_like(f),
           "dA": torch.empty_like(A), "dtau": torch.empty_like(tau),
           "db_x": None if b_x is None else torch.empty_like(b_x), "dw_hat": torch.empty_like(w_hat),
           "dS0": torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev) if want_dS0 else None}
    need = lib.carve_bwd_logits_workspace_size(ctypes.byref(s))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    code = lib.carve_bwd_logits(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(g), _ptr(S0), _ptr(dO),
                                _ptr(dS_T), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["df"]),
                                _ptr(out["dA"]), _ptr(out["dtau"]), _ptr(out["db_x"]), _ptr(out["dw_hat"]),
                                _ptr(out["dS0"]), _ptr(workspace), workspace.numel(), _stream(dev))
    _raise(code, "carve_bwd_logits")
    return out


def fwd_logits_save(q, k, v, f, A, tau, w_hat, b_x=None, S0=None, L=64, o=None, S_T=None, saved=None, profile=None):
    """fwd_logits that also keeps what bwd_logits_saved needs: (o, S_T, saved)."""
    lib = load_library()
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    _check(k, "k", (B, H, T, Dk), q.dtype, dev)
    _check(v, "v", (B, H, T, Dv), q.dtype, dev)
    _check(S0, "S0", (B, H, Dv, Dk), torch.float32, dev)
    g = _gate_logits(q, f, A, tau, w_hat, b_x)
    s = make_shape(q, v, L)
    if o is None:
        o = torch.empty((B, H, T, Dv), dtype=q.dtype, device=dev)
    if S_T is None:
        S_T = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev)
    need = lib.carve_saved_size(ctypes.byref(s))
    if saved is None or saved.numel() < need:
        saved = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    code = lib.carve_fwd_logits_save(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(g), _ptr(S0), _ptr(o),
                                     _ptr(S_T), _ptr(saved), saved.numel(), _stream(dev),
                                     ctypes.byref(profile) if profile is not None else None)
    _raise(code, "carve_fwd_logits_save")
    return o, S_T, saved


def bwd_logits_saved(q, k, v, f, A, tau, w_hat, dO, saved, b_x=None, dS_T=None, L=64, want_dS0=True,
                     workspace=None, out=None, profile=None):
    """Backward from the buffer of fwd_logits_save (same inputs): dict as bwd_logits()."""
    lib = load_library()
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    _check(k, "k", (B, H, T, Dk), q.dtype, dev)
    _check(v, "v", (B, H, T, Dv), q.dtype, dev)
    _check(dO, "dO", (B, H, T, Dv), q.dtype, dev)
    _check(dS_T, "dS_T", (B, H, Dv, Dk), torch.float32, dev)
    g = _gate_logits(q, f, A, tau, w_hat, b_x)
    s = make_shape(q, v, L)
    res = out if out is not None else {
        "dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v), "df": torch.empty_like(f),
        "dA": torch.empty_like(A), "dtau": torch.empty_like(tau),
        "db_x": None if b_x is None else torch.empty_like(b_x), "dw_hat": torch.empty_like(w_hat),
        "dS0": torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev) if want_dS0 else None}
    need = lib.carve_bwd_logits_saved_workspace_size(ctypes.byref(s))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    code = lib.carve_bwd_logits_saved(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), ctypes.byref(g), _ptr(dO),
                                      _ptr(dS_T), _ptr(saved), saved.numel(), _ptr(res["dq"]), _ptr(res["dk"]),
                                      _ptr(res["dv"]), _ptr(res["df"]), _ptr(res["dA"]), _ptr(res["dtau"]),
                                      _ptr(res["db_x"]), _ptr(res["dw_hat"]), _ptr(res["dS0"]), _ptr(workspace),
                                      workspace.numel(), _stream(dev),
                                      ctypes.byref(profile) if profile is not None else None)
    _raise(code, "carve_bwd_logits_saved")
    return res


def bwd_content_workspace_bytes(q, v, L=64, R=0, records=False):
    """Workspace bytes of bwd_content for this shape (R: projection rank, 0 = none;
    records: the forward's per-period records are passed, so it is not re-run)."""
    lib = load_library()
    s = make_shape(q, v, L)
    c = carve_content(None, 1 if R else None, 1 if R else None, R, None, None,
                      16 if records else None, 16 if records else None)
    return lib.carve_bwd_content_workspace_size(ctypes.byref(s), ctypes.byref(c))


def bwd_content(q, k, v, log_g, w, dO, content, S0=None, dS_T=None, dm_out=None, L=64, want_dS0=True,
                want_dm0=True, workspace=None):
    """Gradients of the content-aware forward: dict with dq, dk, dv, dlog_g, db_x, dw,
    dU1 / dU2 (None without projection), dm0 and dS0 (None unless asked for).
    content: dict with b_x, U1, U2 (or None) and m0 (or None), as for fwd(), and optionally
    the records z_rec / m_rec that fwd() filled for the same inputs (then the content-aware
    forward is not run again)."""
    lib = load_library()
    B, H, T, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    dt = q.dtype
    _check(k, "k", (B, H, T, Dk), dt, dev)
    _check(v, "v", (B, H, T, Dv), dt, dev)
    _check(dO, "dO", (B, H, T, Dv), dt, dev)
    _check(log_g, "log_g", (B, H, T, Dk), torch.float32, dev)
    _check(w, "w", (B, H, T), torch.float32, dev)
    _check(S0, "S0", (B, H, Dv, Dk), torch.float32, dev)
    _check(dS_T, "dS_T", (B, H, Dv, Dk), torch.float32, dev)
    _check(dm_out, "dm_out", (B, H, Dv), torch.float32, dev)
    bx, U1, U2, m0 = content["b_x"], content.get("U1"), content.get("U2"), content.get("m0")
    _check(bx, "b_x", (B, H, T, Dk), torch.float32, dev)
    R = 0
    if U1 is not None:
        R = U1.shape[1]
        _check(U1, "U1", (H, R, Dv), torch.float32, dev)
        _check(U2, "U2", (H, Dk, R), torch.float32, dev)
    _check(m0, "m0", (B, H, Dv), torch.float32, dev)
    zr, mr = _records(content, B, H, T, Dk, Dv, L, dev)
    cs = carve_content(bx.data_ptr(), None if U1 is None else U1.data_ptr(), None if U2 is None else U2.data_ptr(),
                       R, None if m0 is None else m0.data_ptr(), None, zr, mr)
    s = make_shape(q, v, L)
    g = {"dq": torch.empty_like(q), "dk": torch.empty_like(k), "dv": torch.empty_like(v),
         "dlog_g": torch.empty_like(log_g), "db_x": torch.empty_like(bx), "dw": torch.empty_like(w),
         "dU1": None if U1 is None else torch.empty_like(U1), "dU2": None if U2 is None else torch.empty_like(U2),
         "dm0": torch.empty((B, H, Dv), dtype=torch.float32, device=dev) if want_dm0 else None,
         "dS0": torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=dev) if want_dS0 else None}
    need = lib.carve_bwd_content_workspace_size(ctypes.byref(s), ctypes.byref(cs))
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    code = lib.carve_bwd_content(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(w), _ptr(S0),
                                 ctypes.byref(cs), _ptr(dO), _ptr(dS_T), _ptr(dm_out), _ptr(g["dq"]), _ptr(g["dk"]),
                                 _ptr(g["dv"]), _ptr(g["dlog_g"]), _ptr(g["db_x"]), _ptr(g["dw"]), _ptr(g["dU1"]),
                                 _ptr(g["dU2"]), _ptr(g["dm0"]), _ptr(g["dS0"]), _ptr(workspace), workspace.numel(),
                                 _stream(dev))
    _raise(code, "carve_bwd_content")
    return g


def decode_step(q, k, v, log_g, w, S, b=None, L=64, content=None, o=None):
    """One recurrent decode token per (batch, head); S [B,H,Dv,Dk] float32 is updated in place.

    q, k [B,H,Dk], v [B,H,Dv] (float32 or bfloat16); log_g, b [B,H,Dk] float32; w [B,H]
    float32.  content is None or a dict with b_x [B,H,Dk], U1 [H,R,Dv] / U2 [H,Dk,R] (or None),
    m_in [B,H,Dv] (or None), csum [B,H,Dv] (updated in place) and pos (tokens of the current
    chunk of L before this one).  Returns (o [B,H,Dv], m_out [B,H,Dv] or None)."""
    lib = load_library()
    B, H, Dk = q.shape
    Dv = v.shape[-1]
    dev = q.device
    dt = q.dtype
    _check(k, "k", (B, H, Dk), dt, dev)
    _check(v, "v", (B, H, Dv), dt, dev)
    _check(log_g, "log_g", (B, H, Dk), torch.float32, dev)
    _check(b, "b", (B, H, Dk), torch.float32, dev)
    _check(w, "w", (B, H), torch.float32, dev)
    _check(S, "S", (B, H, Dv, Dk), torch.float32, dev)
    s = carve_shape(B, H, 1, Dk, Dv, L, _dtype_code(q))
    cs = None
    m_out = None
    if content is not None:
        bx, U1, U2 = content["b_x"], content.get("U1"), content.get("U2")
        m_in, csum = content.get("m_in"), content["csum"]
        _check(bx, "b_x", (B, H, Dk), torch.float32, dev)
        R = 0
        if U1 is not None:
            R = U1.shape[1]
            _check(U1, "U1", (H, R, Dv), torch.float32, dev)
            _check(U2, "U2", (H, Dk, R), torch.float32, dev)
        _check(m_in, "m_in", (B, H, Dv), torch.float32, dev)
        _check(csum, "csum", (B, H, Dv), torch.float32, dev)
        m_out = content.get("m_out")
        if m_out is None:
            m_out = torch.empty((B, H, Dv), dtype=torch.float32, device=dev)
        _check(m_out, "m_out", (B, H, Dv), torch.float32, dev)
        cs = carve_decode_content(bx.data_ptr(), None if U1 is None else U1.data_ptr(),
                                  None if U2 is None else U2.data_ptr(), R,
                                  None if m_in is None else m_in.data_ptr(), m_out.data_ptr(),
                                  csum.data_ptr(), int(content.get("pos", 0)))
    if o is None:
        o = torch.empty((B, H, Dv), dtype=dt, device=dev)
    code = lib.carve_decode_step(ctypes.byref(s), _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(b), _ptr(w),
                                 _ptr(S), ctypes.byref(cs) if cs is not None else None, _ptr(o), _stream(dev))
    _raise(code, "carve_decode_step")
    return o, m_out


def stream_copy(dst, src):
    """Copy src into dst (same number of bytes, contiguous device tensors) with the library's
    streaming copy kernel on the current stream; a measurement helper for the achievable
    copy bandwidth, not part of the CARVE operation."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("stream_copy: dst and src differ in size")
    if not (dst.is_contiguous() and src.is_contiguous()) or dst.device != src.device:
        raise ValueError("stream_copy: contiguous tensors on one device required")
    code = load_library().carve_stream_copy(_ptr(dst), _ptr(src), nbytes, _stream(src.device))
    _raise(code, "carve_stream_copy")
    return dst
