"""Float64, token-serial CPU reference for the CARVE key-axis gated delta rule.

TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.  Only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import this module.  It shares
no code with the HIP library and does not import it.

Sources (the CARVE pages; equations there were lost in text extraction, so
each step below is the plainest reading of the surviving symbol legends):

* liuzhao09.github.io CARVE notes, section 2.1 (delta-rule legend): the state
  is a fixed d_v x d_k matrix; the old state predicts the value of the current
  key, S_{t-1} k_t, and only the prediction error v_t - S_{t-1} k_t is written
  as a rank-1 correction along k_t.
* same page, section 2.1 (CARVE update legend): the key-axis decay g and the
  key-axis erase b both act by right-multiplying a diagonal matrix onto the
  old state; the write strength w is one scalar per head broadcast over d_v.
  Reading taken here: a_t = exp(log g_t) * b_t forms ONE diagonal that is
  applied to S_{t-1} before both the prediction and the retention, i.e.
      P_t = S_{t-1} Diag(a_t)
      S_t = P_t + w_t (v_t - P_t k_t) k_t^T
* same page, section 2.2: the readout is o_t = S_t q_t (post-update state).
  (The gist.science technical summary writes S_{t-1} q_t; the reading taken
  is the blog's S_t q_t.)
* same page, section 2.2 (content-aware erase legend) and the gist.science
  technical summary, section 2.1: the content signal is the mean of the
  previous chunk's outputs, m = (1/L) sum o_t, passed through a zero-initialised
  low-rank projection U_b = U2 U1 into the key axis; the erase gate of chunk c
  is b_{c,t} = sigmoid(b_{x,t} + U_b m_{c-1}).  Both pages say sequences shorter
  than two chunks get no content signal; reading: m_{-1} = m0 (0 if absent).
  A ragged final chunk averages over the tokens it actually holds.
* same page, section 2.3: log g <= 0, exp(log g) is the retention factor.

No query scaling and no normalisation happen inside the operation; the
caller L2-normalises q and k.

Arrays are numpy float64 with leading [B, H] axes; the loops run over tokens
and are vectorised over (B*H) heads only.

Functions: forward (token-serial forward, token-only or content-aware gates),
backward (reverse mode of the token-only forward), backward_content (reverse
mode of the content-aware forward, including the projection and the carried-in
mean), and gates_from_logits / forward_logits / backward_logits (the gates given
as pre-activations, computed inside the operation).
"""

import numpy as np


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _as64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def forward(q, k, v, log_g, w, b=None, S0=None, L=64, content=None, return_states=False):
    """Token-serial forward pass.

    q, k   : [B, H, T, Dk]      v : [B, H, T, Dv]
    log_g  : [B, H, T, Dk] (<= 0, log of the key-axis retention)
    w      : [B, H, T]     (scalar write strength per head and token)
    b      : [B, H, T, Dk] erase gate in (0, 1]; None means b = 1.  Must be
             None when `content` is given (then b comes from the content gate).
    S0     : [B, H, Dv, Dk] initial state; None means zero.
    L      : chunk length; only matters for the content path (it fixes which
             tokens are averaged into m).
    content: None, or a dict with
             'b_x' [B, H, T, Dk] erase pre-activation,
             'U1' [H, R, Dv] and 'U2' [H, Dk, R] (both None: no projection),
             'm0' [B, H, Dv] carried-in previous-chunk mean (None: zero).
    Returns (o [B,H,T,Dv], S_T [B,H,Dv,Dk], m_out [B,H,Dv] or None); with
    return_states=True also the list of S_t, t = 0..T (S_0 = initial state).
    """
    q, k, v, log_g, w = map(_as64, (q, k, v, log_g, w))
    B, H, T, Dk = k.shape
    Dv = v.shape[-1]
    BH = B * H
    qf = q.reshape(BH, T, Dk)
    kf = k.reshape(BH, T, Dk)
    vf = v.reshape(BH, T, Dv)
    gf = log_g.reshape(BH, T, Dk)
    wf = w.reshape(BH, T)
    if content is not None and b is not None:
        raise ValueError("b must be None when the content gate is used")
    bf = None if b is None else _as64(b).reshape(BH, T, Dk)
    S = np.zeros((BH, Dv, Dk)) if S0 is None else _as64(S0).reshape(BH, Dv, Dk).copy()
    o = np.zeros((BH, T, Dv))
    states = [S.copy()] if return_states else None

    if content is not None:
        bx = _as64(content["b_x"]).reshape(BH, T, Dk)
        U1 = content.get("U1")
        U2 = content.get("U2")
        if (U1 is None) != (U2 is None):
            raise ValueError("U1 and U2 must both be given or both be None")
        if U1 is not None:
            # per-head projections, broadcast over the batch axis
            U1h = np.broadcast_to(_as64(U1)[None], (B,) + np.shape(U1)).reshape(BH, *np.shape(U1)[1:])
            U2h = np.broadcast_to(_as64(U2)[None], (B,) + np.shape(U2)).reshape(BH, *np.shape(U2)[1:])
        m0 = content.get("m0")
        m_prev = np.zeros((BH, Dv)) if m0 is None else _as64(m0).reshape(BH, Dv).copy()
        csum = np.zeros((BH, Dv))
        z = np.zeros((BH, Dk))
        count = 0

    for t in range(T):
        if content is not None:
            if t % L == 0:
                # content signal of this chunk: low-rank projection of the
                # previous chunk's mean output (zero when U_b is absent)
                if U1 is not None:
                    r = np.einsum("nrv,nv->nr", U1h, m_prev)
                    z = np.einsum("nkr,nr->nk", U2h, r)
                else:
                    z = np.zeros((BH, Dk))
                csum = np.zeros((BH, Dv))
                count = 0
            bt = _sigmoid(bx[:, t] + z)
        else:
            bt = 1.0 if bf is None else bf[:, t]
        a = np.exp(gf[:, t]) * bt                       # key-axis retention times erase
        P = S * a[:, None, :]                           # S_{t-1} Diag(a_t)
        e = vf[:, t] - np.einsum("nvk,nk->nv", P, kf[:, t])   # prediction error
        S = P + wf[:, t][:, None, None] * e[:, :, None] * kf[:, t][:, None, :]
        o[:, t] = np.einsum("nvk,nk->nv", S, qf[:, t])  # post-update readout
        if return_states:
            states.append(S.copy())
        if content is not None:
            csum += o[:, t]
            count += 1
            if (t + 1) % L == 0 or t == T - 1:
                m_prev = csum / count

    o = o.reshape(B, H, T, Dv)
    S_T = S.reshape(B, H, Dv, Dk)
    m_out = None
    if content is not None:
        m_out = m_prev.reshape(B, H, Dv)
    if return_states:
        return o, S_T, m_out, [s.reshape(B, H, Dv, Dk) for s in states]
    return o, S_T, m_out


def backward(q, k, v, log_g, w, dO, b=None, S0=None, dS_T=None, segment=64):
    """Reverse-mode gradients of the token-only forward pass (no content gate).

    Given dO = dLoss/do [B,H,T,Dv] and dS_T = dLoss/dS_T (None: zero), returns a
    dict with dq, dk, dv, dlog_g, db (None when b is None), dw and dS0.  The
    gradients are taken in the parameterisation of the inputs: dlog_g is the
    derivative w.r.t. log g, db w.r.t. the erase probability b, dw w.r.t. the
    write strength w.

    States are checkpointed every `segment` tokens and each segment is re-run
    forward before its reverse sweep, so memory stays O(segment * Dv * Dk).
    """
    q, k, v, log_g, w, dO = map(_as64, (q, k, v, log_g, w, dO))
    B, H, T, Dk = k.shape
    Dv = v.shape[-1]
    BH = B * H
    qf = q.reshape(BH, T, Dk)
    kf = k.reshape(BH, T, Dk)
    vf = v.reshape(BH, T, Dv)
    gf = log_g.reshape(BH, T, Dk)
    wf = w.reshape(BH, T)
    dOf = dO.reshape(BH, T, Dv)
    bf = None if b is None else _as64(b).reshape(BH, T, Dk)

    def retention(t):
        g = np.exp(gf[:, t])
        return g, (g if bf is None else g * bf[:, t])

    def step(S, t):
        _, a = retention(t)
        P = S * a[:, None, :]
        e = vf[:, t] - np.einsum("nvk,nk->nv", P, kf[:, t])
        return P + wf[:, t][:, None, None] * e[:, :, None] * kf[:, t][:, None, :]

    S = np.zeros((BH, Dv, Dk)) if S0 is None else _as64(S0).reshape(BH, Dv, Dk).copy()
    checkpoints = {}
    for t in range(T):
        if t % segment == 0:
            checkpoints[t] = S.copy()
        S = step(S, t)

    dq = np.zeros((BH, T, Dk))
    dk = np.zeros((BH, T, Dk))
    dv = np.zeros((BH, T, Dv))
    dlog_g = np.zeros((BH, T, Dk))
    db = None if bf is None else np.zeros((BH, T, Dk))
    dw = np.zeros((BH, T))
    dS = np.zeros((BH, Dv, Dk)) if dS_T is None else _as64(dS_T).reshape(BH, Dv, Dk).copy()

    for start in sorted(checkpoints, reverse=True):
        stop = min(start + segment, T)
        # seg_states[i] is the state before token start+i (after token start+i-1)
        seg_states = [checkpoints[start]]
        for t in range(start, stop):
            seg_states.append(step(seg_states[-1], t))
        for t in range(stop - 1, start - 1, -1):
            S_prev = seg_states[t - start]         # state before token t
            S_t = seg_states[t - start + 1]        # state after token t
            g, a = retention(t)
            kt, vt, qt, wt = kf[:, t], vf[:, t], qf[:, t], wf[:, t]
            P = S_prev * a[:, None, :]
            e = vt - np.einsum("nvk,nk->nv", P, kt)
            # o_t = S_t q_t
            dS = dS + dOf[:, t][:, :, None] * qt[:, None, :]
            dq[:, t] = np.einsum("nvk,nv->nk", S_t, dOf[:, t])
            # S_t = P + w e k^T with e = v - P k
            r = np.einsum("nvk,nk->nv", dS, kt)
            dv[:, t] = wt[:, None] * r
            dw[:, t] = np.einsum("nv,nv->n", e, r)
            dk[:, t] = wt[:, None] * (np.einsum("nvk,nv->nk", dS, e) - np.einsum("nvk,nv->nk", P, r))
            dP = dS - wt[:, None, None] * r[:, :, None] * kt[:, None, :]
            # P = S_{t-1} Diag(a), a = exp(log g) * b
            da = np.einsum("nvk,nvk->nk", S_prev, dP)
            dlog_g[:, t] = a * da
            if db is not None:
                db[:, t] = g * da
            dS = dP * a[:, None, :]

    out = {
        "dq": dq.reshape(B, H, T, Dk),
        "dk": dk.reshape(B, H, T, Dk),
        "dv": dv.reshape(B, H, T, Dv),
        "dlog_g": dlog_g.reshape(B, H, T, Dk),
        "db": None if db is None else db.reshape(B, H, T, Dk),
        "dw": dw.reshape(B, H, T),
        "dS0": dS.reshape(B, H, Dv, Dk),
    }
    return out


def backward_content(q, k, v, log_g, w, dO, content, S0=None, dS_T=None, dm_out=None, L=64):
    """Reverse-mode gradients of the content-aware forward pass.

    content: dict with 'b_x' [B,H,T,Dk], 'U1' [H,R,Dv] / 'U2' [H,Dk,R] (both None:
    no projection) and 'm0' [B,H,Dv] (None: zero), as for forward().  The loss is
    <dO, o> + <dS_T, S_T> + <dm_out, m_out> (dS_T, dm_out None: zero).  Returns a
    dict with dq, dk, dv, dlog_g, db_x, dw, dU1 [H,R,Dv], dU2 [H,Dk,R] (None
    without projection; summed over the batch), dm0 [B,H,Dv] and dS0.

    The chain, in the order of the pages' content-aware erase (notes section 2.2):
    chunk c's gate is b = sigmoid(x), x = b_x + z_c, z_c = U2 r_c, r_c = U1 m_{c-1},
    and m_{c-1} is the mean of chunk c-1's outputs.  So, going backwards, chunk c's
    gate gradient dx_t = db_t b_t (1 - b_t) gives dz_c = sum_t dx_t, then
    dU2 += dz_c r_c^T, dr_c = U2^T dz_c, dU1 += dr_c m_{c-1}^T and dm_{c-1} = U1^T dr_c,
    which reaches every output of chunk c-1 as dm_{c-1} / (its token count) before
    that chunk is swept (chunk 0's goes to m0).  Inside a chunk the per-token
    steps are those of backward() with b_t in place of the erase input.
    """
    q, k, v, log_g, w, dO = map(_as64, (q, k, v, log_g, w, dO))
    B, H, T, Dk = k.shape
    Dv = v.shape[-1]
    BH = B * H
    qf, kf, vf = q.reshape(BH, T, Dk), k.reshape(BH, T, Dk), v.reshape(BH, T, Dv)
    gf, wf, dOf = log_g.reshape(BH, T, Dk), w.reshape(BH, T), dO.reshape(BH, T, Dv)
    bx = _as64(content["b_x"]).reshape(BH, T, Dk)
    U1, U2 = content.get("U1"), content.get("U2")
    if (U1 is None) != (U2 is None):
        raise ValueError("U1 and U2 must both be given or both be None")
    proj = U1 is not None
    if proj:
        R = np.shape(U1)[1]
        U1h = np.broadcast_to(_as64(U1)[None], (B,) + np.shape(U1)).reshape(BH, R, Dv)
        U2h = np.broadcast_to(_as64(U2)[None], (B,) + np.shape(U2)).reshape(BH, Dk, R)
    m0 = content.get("m0")
    m_prev = np.zeros((BH, Dv)) if m0 is None else _as64(m0).reshape(BH, Dv).copy()

    # forward sweep: the state entering every chunk, each chunk's gates and the mean
    # output m_{c-1} its gate was formed from
    NCh = (T + L - 1) // L
    S = np.zeros((BH, Dv, Dk)) if S0 is None else _as64(S0).reshape(BH, Dv, Dk).copy()
    S_in, m_in, bgate = [], [], np.zeros((BH, T, Dk))
    for c in range(NCh):
        t0, t1 = c * L, min((c + 1) * L, T)
        S_in.append(S.copy())
        m_in.append(m_prev.copy())
        z = np.einsum("nkr,nr->nk", U2h, np.einsum("nrv,nv->nr", U1h, m_prev)) if proj else np.zeros((BH, Dk))
        csum = np.zeros((BH, Dv))
        for t in range(t0, t1):
            bgate[:, t] = _sigmoid(bx[:, t] + z)
            a = np.exp(gf[:, t]) * bgate[:, t]
            P = S * a[:, None, :]
            e = vf[:, t] - np.einsum("nvk,nk->nv", P, kf[:, t])
            S = P + wf[:, t][:, None, None] * e[:, :, None] * kf[:, t][:, None, :]
            csum += np.einsum("nvk,nk->nv", S, qf[:, t])
        m_prev = csum / (t1 - t0)

    dq, dk, dv = np.zeros((BH, T, Dk)), np.zeros((BH, T, Dk)), np.zeros((BH, T, Dv))
    dlog_g, dbx, dw = np.zeros((BH, T, Dk)), np.zeros((BH, T, Dk)), np.zeros((BH, T))
    dU1 = np.zeros((BH, R, Dv)) if proj else None
    dU2 = np.zeros((BH, Dk, R)) if proj else None
    dS = np.zeros((BH, Dv, Dk)) if dS_T is None else _as64(dS_T).reshape(BH, Dv, Dk).copy()
    # gradient w.r.t. the mean output of the chunk being swept (the last one: dm_out)
    dm = np.zeros((BH, Dv)) if dm_out is None else _as64(dm_out).reshape(BH, Dv).copy()

    for c in range(NCh - 1, -1, -1):
        t0, t1 = c * L, min((c + 1) * L, T)
        dOc = dOf[:, t0:t1] + (dm / (t1 - t0))[:, None, :]     # m_c's gradient reaches each output
        # states before every token of the chunk
        states = [S_in[c]]
        for t in range(t0, t1):
            a = np.exp(gf[:, t]) * bgate[:, t]
            P = states[-1] * a[:, None, :]
            e = vf[:, t] - np.einsum("nvk,nk->nv", P, kf[:, t])
            states.append(P + wf[:, t][:, None, None] * e[:, :, None] * kf[:, t][:, None, :])
        dz = np.zeros((BH, Dk))
        for t in range(t1 - 1, t0 - 1, -1):
            S_prev, S_t = states[t - t0], states[t - t0 + 1]
            g = np.exp(gf[:, t])
            bt = bgate[:, t]
            a = g * bt
            kt, vt, qt, wt, dot = kf[:, t], vf[:, t], qf[:, t], wf[:, t], dOc[:, t - t0]
            P = S_prev * a[:, None, :]
            e = vt - np.einsum("nvk,nk->nv", P, kt)
            dS = dS + dot[:, :, None] * qt[:, None, :]
            dq[:, t] = np.einsum("nvk,nv->nk", S_t, dot)
            r = np.einsum("nvk,nk->nv", dS, kt)
            dv[:, t] = wt[:, None] * r
            dw[:, t] = np.einsum("nv,nv->n", e, r)
            dk[:, t] = wt[:, None] * (np.einsum("nvk,nv->nk", dS, e) - np.einsum("nvk,nv->nk", P, r))
            dP = dS - wt[:, None, None] * r[:, :, None] * kt[:, None, :]
            da = np.einsum("nvk,nvk->nk", S_prev, dP)
            dlog_g[:, t] = a * da
            dx = g * da * bt * (1.0 - bt)                  # through b = sigmoid(b_x + z_c)
            dbx[:, t] = dx
            dz += dx
            dS = dP * a[:, None, :]
        # z_c = U2 U1 m_{c-1}
        if proj:
            rc = np.einsum("nrv,nv->nr", U1h, m_in[c])
            dU2 += np.einsum("nk,nr->nkr", dz, rc)
            dr = np.einsum("nkr,nk->nr", U2h, dz)
            dU1 += np.einsum("nr,nv->nrv", dr, m_in[c])
            dm = np.einsum("nrv,nr->nv", U1h, dr)
        else:
            dm = np.zeros((BH, Dv))

    out = {
        "dq": dq.reshape(B, H, T, Dk), "dk": dk.reshape(B, H, T, Dk), "dv": dv.reshape(B, H, T, Dv),
        "dlog_g": dlog_g.reshape(B, H, T, Dk), "db_x": dbx.reshape(B, H, T, Dk), "dw": dw.reshape(B, H, T),
        "dU1": None if not proj else dU1.reshape(B, H, R, Dv).sum(axis=0),
        "dU2": None if not proj else dU2.reshape(B, H, Dk, R).sum(axis=0),
        "dm0": dm.reshape(B, H, Dv), "dS0": dS.reshape(B, H, Dv, Dk),
    }
    return out


def _softplus(x):
    return np.logaddexp(0.0, x)


def gates_from_logits(f, A, tau, w_hat, b_x=None):
    """Gates from their pre-activations, the reading taken of the pages' fused
    gate (notes section 2.3 legends: A the log-decay amplitude, f the decay
    logits, tau a bias, the output log g <= 0; scalar write pre-activation w_hat):
        log g = -A softplus(f + tau)   (A, tau per head and key channel, [H, Dk])
        b = sigmoid(b_x)               (None: b = 1)
        w = sigmoid(w_hat)
    Returns (log_g, b, w)."""
    f, A, tau, w_hat = map(_as64, (f, A, tau, w_hat))
    log_g = -A[None, :, None, :] * _softplus(f + tau[None, :, None, :])
    b = None if b_x is None else _sigmoid(_as64(b_x))
    return log_g, b, _sigmoid(w_hat)


def forward_logits(q, k, v, f, A, tau, w_hat, b_x=None, S0=None):
    """Token-only forward pass with the gates given as pre-activations (see
    gates_from_logits).  Returns (o, S_T)."""
    log_g, b, w = gates_from_logits(f, A, tau, w_hat, b_x)
    o, S_T, _ = forward(q, k, v, log_g, w, b=b, S0=S0)
    return o, S_T


def backward_logits(q, k, v, f, A, tau, w_hat, dO, b_x=None, S0=None, dS_T=None):
    """Gradients of forward_logits: dict with dq, dk, dv, df, dA, dtau ([H, Dk],
    summed over batch and tokens), db_x (None without b_x), dw_hat and dS0.
    The chain rule through the three activations:
        d f = d(log g) * (-A sigmoid(f + tau)),  d tau = sum d f,
        d A = sum d(log g) * (-softplus(f + tau)),
        d b_x = d b * b (1 - b),  d w_hat = d w * w (1 - w)."""
    log_g, b, w = gates_from_logits(f, A, tau, w_hat, b_x)
    g = backward(q, k, v, log_g, w, dO, b=b, S0=S0, dS_T=dS_T)
    f, A, tau = map(_as64, (f, A, tau))
    y = f + tau[None, :, None, :]
    df = g["dlog_g"] * (-A[None, :, None, :] * _sigmoid(y))
    out = {key: g[key] for key in ("dq", "dk", "dv", "dS0")}
    out["df"] = df
    out["dtau"] = df.sum(axis=(0, 2))
    out["dA"] = (g["dlog_g"] * (-_softplus(y))).sum(axis=(0, 2))
    out["db_x"] = None if b is None else g["db"] * b * (1.0 - b)
    out["dw_hat"] = g["dw"] * w * (1.0 - w)
    return out
