"""torch.autograd functions over the training pairs of the C ABI.

Argument marshalling only: each forward calls the library's forward that keeps what its
backward needs (carve_fwd_save, carve_fwd_logits_save, or the content-aware carve_fwd
with its per-period records) and holds that buffer on the autograd context; the backward
calls the matching library backward (carve_bwd_saved, carve_bwd_logits_saved,
carve_bwd_content) with the incoming gradients.  Every step of both passes runs in the
HIP kernels; there is no CPU fallback.

    from chunk_gated_delta_amd.autograd import carve_attention
    o, S_T = carve_attention(q, k, v, log_g, w, b=b)          # token-only gates
    loss = f(o); loss.backward()                                 # grads of q, k, v, log_g, w, b
"""
import torch

from . import carve


def _c(t):
    """A contiguous view of an incoming gradient (autograd may hand over expanded zeros)."""
    return None if t is None else t.contiguous()


class _TokenPair(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, log_g, w, b, S0, L):
        o, S_T, saved = carve.fwd_save(q, k, v, log_g, w, b=b, S0=S0, L=L)
        ctx.L, ctx.has_b, ctx.has_S0 = L, b is not None, S0 is not None
        ctx.save_for_backward(q, k, v, log_g, w, b, saved)
        return o, S_T

    @staticmethod
    def backward(ctx, dO, dS_T):
        q, k, v, log_g, w, b, saved = ctx.saved_tensors
        g = carve.bwd_saved(q, k, v, log_g, w, _c(dO), saved, b=b, dS_T=_c(dS_T), L=ctx.L, want_dS0=ctx.has_S0)
        return g["dq"], g["dk"], g["dv"], g["dlog_g"], g["dw"], g["db"], g["dS0"], None


class _LogitPair(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, f, A, tau, w_hat, b_x, S0, L):
        o, S_T, saved = carve.fwd_logits_save(q, k, v, f, A, tau, w_hat, b_x=b_x, S0=S0, L=L)
        ctx.L, ctx.has_S0 = L, S0 is not None
        ctx.save_for_backward(q, k, v, f, A, tau, w_hat, b_x, saved)
        return o, S_T

    @staticmethod
    def backward(ctx, dO, dS_T):
        q, k, v, f, A, tau, w_hat, b_x, saved = ctx.saved_tensors
        g = carve.bwd_logits_saved(q, k, v, f, A, tau, w_hat, _c(dO), saved, b_x=b_x, dS_T=_c(dS_T), L=ctx.L,
                                   want_dS0=ctx.has_S0)
        return g["dq"], g["dk"], g["dv"], g["df"], g["dA"], g["dtau"], g["dw_hat"], g["db_x"], g["dS0"], None


class _ContentPair(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, log_g, w, b_x, U1, U2, m0, S0, L):
        B, H, T, Dk = q.shape
        z_rec, m_rec = carve.content_records(B, H, T, Dk, v.shape[-1], L, q.device)
        content = {"b_x": b_x, "U1": U1, "U2": U2, "m0": m0, "z_rec": z_rec, "m_rec": m_rec}
        o, S_T, m_out = carve.fwd(q, k, v, log_g, w, S0=S0, L=L, content=content)
        ctx.L, ctx.has_S0, ctx.has_m0 = L, S0 is not None, m0 is not None
        ctx.save_for_backward(q, k, v, log_g, w, b_x, U1, U2, m0, S0, z_rec, m_rec)
        return o, S_T, m_out

    @staticmethod
    def backward(ctx, dO, dS_T, dm_out):
        q, k, v, log_g, w, b_x, U1, U2, m0, S0, z_rec, m_rec = ctx.saved_tensors
        content = {"b_x": b_x, "U1": U1, "U2": U2, "m0": m0, "z_rec": z_rec, "m_rec": m_rec}
        g = carve.bwd_content(q, k, v, log_g, w, _c(dO), content, S0=S0, dS_T=_c(dS_T), dm_out=_c(dm_out), L=ctx.L,
                              want_dS0=ctx.has_S0, want_dm0=ctx.has_m0)
        return (g["dq"], g["dk"], g["dv"], g["dlog_g"], g["dw"], g["db_x"], g["dU1"], g["dU2"], g["dm0"], g["dS0"],
                None)


def carve_attention(q, k, v, log_g, w, b=None, S0=None, L=64):
    """(o, S_T) of the token-only forward, differentiable in q, k, v, log_g, w, b and S0
    (the training pair carve_fwd_save / carve_bwd_saved)."""
    return _TokenPair.apply(q, k, v, log_g, w, b, S0, L)


def carve_attention_logits(q, k, v, f, A, tau, w_hat, b_x=None, S0=None, L=64):
    """(o, S_T) with the gates given as pre-activations (log g = -A softplus(f + tau),
    b = sigmoid(b_x), w = sigmoid(w_hat)), differentiable in every input (the training pair
    carve_fwd_logits_save / carve_bwd_logits_saved)."""
    return _LogitPair.apply(q, k, v, f, A, tau, w_hat, b_x, S0, L)


def carve_attention_content(q, k, v, log_g, w, b_x, U1=None, U2=None, m0=None, S0=None, L=64):
    """(o, S_T, m_out) with the content-aware erase b = sigmoid(b_x + U2 U1 m), differentiable
    in q, k, v, log_g, w, b_x, U1, U2, m0 and S0 (carve_fwd with records, carve_bwd_content)."""
    return _ContentPair.apply(q, k, v, log_g, w, b_x, U1, U2, m0, S0, L)
