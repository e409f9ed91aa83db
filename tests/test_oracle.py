"""Pins for the float64 reference (CPU only).

Each test checks the reference against something other than its own loop:
hand-worked values, closed forms of special cases, exact identities of the
recurrence, or finite differences.  The pins are chosen so that a plausible
slip (decay applied after the write instead of before, pre-update readout,
decay on the value axis instead of the key axis, a transposed product, an
off-by-one chunk mean, a dropped gradient term) fails at least one of them.
"""

import json
import os

import numpy as np
import pytest

from oracle import forward, backward, backward_content, backward_logits, forward_logits, gates_from_logits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_case(rng, B=1, H=2, T=12, Dk=5, Dv=4, unit_keys=True, with_b=True):
    q = rng.standard_normal((B, H, T, Dk))
    k = rng.standard_normal((B, H, T, Dk))
    if unit_keys:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, T, Dv))
    log_g = rng.uniform(np.log(0.5), 0.0, (B, H, T, Dk))
    b = rng.uniform(0.3, 1.0, (B, H, T, Dk)) if with_b else None
    w = rng.uniform(0.05, 0.95, (B, H, T))
    S0 = rng.standard_normal((B, H, Dv, Dk))
    return dict(q=q, k=k, v=v, log_g=log_g, b=b, w=w, S0=S0)


# ---------------------------------------------------------------- forward pins

def test_golden_two_tokens():
    """Hand-worked two-token example (fixture cites the update and readout legends)."""
    with open(os.path.join(GOLDEN, "worked_two_tokens.json")) as f:
        g = json.load(f)
    inp = g["inputs"]
    k = np.array(inp["k"], float)[None, None]
    v = np.array(inp["v"], float)[None, None]
    q = np.array(inp["q"], float)[None, None]
    log_g = np.log(np.array(inp["a"], float))[None, None]
    w = np.array(inp["w"], float)[None, None]
    S0 = np.array(inp["S0"], float)[None, None]
    o, S_T, _ = forward(q, k, v, log_g, w, S0=S0)
    np.testing.assert_allclose(o[0, 0], np.array(g["expected"]["o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(S_T[0, 0], np.array(g["expected"]["S_T"]), rtol=0, atol=1e-14)


def test_readout_is_post_update():
    """T=1 from a zero state: o_0 = w_0 v_0 (k_0 . q_0); a pre-update readout would give 0."""
    rng = np.random.default_rng(1)
    c = rand_case(rng, T=1)
    o, _, _ = forward(c["q"], c["k"], c["v"], c["log_g"], c["w"], b=c["b"])
    kq = np.einsum("bhtk,bhtk->bht", c["k"], c["q"])
    np.testing.assert_allclose(o, c["w"][..., None] * c["v"] * kq[..., None], rtol=1e-13, atol=1e-15)


def test_unrolled_product():
    """S_T = S0 M_1...M_T + sum_t w_t v_t k_t^T M_{t+1}...M_T with M_t = Diag(a_t)(I - w_t k_t k_t^T),
    and o_t = S_t q_t, computed with explicit d_k x d_k matrix products."""
    rng = np.random.default_rng(2)
    c = rand_case(rng, B=2, H=2, T=9, Dk=5, Dv=3)
    o, S_T, _ = forward(c["q"], c["k"], c["v"], c["log_g"], c["w"], b=c["b"], S0=c["S0"])
    B, H, T, Dk = c["k"].shape
    for bi in range(B):
        for hi in range(H):
            a = np.exp(c["log_g"][bi, hi]) * c["b"][bi, hi]
            M = [np.diag(a[t]) @ (np.eye(Dk) - c["w"][bi, hi, t] * np.outer(c["k"][bi, hi, t], c["k"][bi, hi, t]))
                 for t in range(T)]
            for t_end in range(1, T + 1):
                prod = np.eye(Dk)
                for t in range(t_end):
                    prod = prod @ M[t]
                S = c["S0"][bi, hi] @ prod
                for t in range(t_end):
                    tail = np.eye(Dk)
                    for s in range(t + 1, t_end):
                        tail = tail @ M[s]
                    S = S + c["w"][bi, hi, t] * np.outer(c["v"][bi, hi, t], c["k"][bi, hi, t]) @ tail
                np.testing.assert_allclose(o[bi, hi, t_end - 1], S @ c["q"][bi, hi, t_end - 1], rtol=1e-11, atol=1e-12)
            np.testing.assert_allclose(S_T[bi, hi], S, rtol=1e-11, atol=1e-12)


def test_one_hot_keys_decouple_columns():
    """k_t = e_{i_t}: column j != i_t only decays (col_j <- a_j col_j); column i_t becomes
    (1 - w) a_i col_i + w v_t.  Decay on the value axis or a transposed state fails this."""
    rng = np.random.default_rng(3)
    B, H, T, Dk, Dv = 1, 3, 20, 4, 3
    idx = rng.integers(0, Dk, (B, H, T))
    k = np.zeros((B, H, T, Dk))
    np.put_along_axis(k, idx[..., None], 1.0, axis=-1)
    q = rng.standard_normal((B, H, T, Dk))
    v = rng.standard_normal((B, H, T, Dv))
    log_g = rng.uniform(-0.7, 0.0, (B, H, T, Dk))
    b = rng.uniform(0.2, 1.0, (B, H, T, Dk))
    w = rng.uniform(0, 1, (B, H, T))
    S0 = rng.standard_normal((B, H, Dv, Dk))
    o, S_T, _ = forward(q, k, v, log_g, w, b=b, S0=S0)
    for h in range(H):
        cols = S0[0, h].copy()  # [Dv, Dk]
        for t in range(T):
            a = np.exp(log_g[0, h, t]) * b[0, h, t]
            i = idx[0, h, t]
            new = cols * a[None, :]
            new[:, i] = (1 - w[0, h, t]) * a[i] * cols[:, i] + w[0, h, t] * v[0, h, t]
            cols = new
            np.testing.assert_allclose(o[0, h, t], cols @ q[0, h, t], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(S_T[0, h], cols, rtol=1e-12, atol=1e-13)


def test_orthonormal_keys_no_decay_is_linear_attention():
    """a = 1 and orthonormal keys: S_T = S0 (I - sum w_t k_t k_t^T) + sum w_t v_t k_t^T;
    with S0 = 0 and w = 1 the outputs are causal linear attention o_t = sum_{s<=t} v_s (k_s . q_t)."""
    rng = np.random.default_rng(4)
    B, H, T, D = 1, 2, 6, 8
    Qm, _ = np.linalg.qr(rng.standard_normal((D, D)))
    k = np.broadcast_to(Qm[:T][None, None], (B, H, T, D)).copy()
    q = rng.standard_normal((B, H, T, D))
    v = rng.standard_normal((B, H, T, D))
    zero = np.zeros((B, H, T, D))
    w = rng.uniform(0.1, 0.9, (B, H, T))
    S0 = rng.standard_normal((B, H, D, D))
    _, S_T, _ = forward(q, k, v, zero, w, S0=S0)
    for h in range(H):
        proj = sum(w[0, h, t] * np.outer(k[0, h, t], k[0, h, t]) for t in range(T))
        write = sum(w[0, h, t] * np.outer(v[0, h, t], k[0, h, t]) for t in range(T))
        np.testing.assert_allclose(S_T[0, h], S0[0, h] @ (np.eye(D) - proj) + write, rtol=1e-12, atol=1e-12)
    o, _, _ = forward(q, k, v, zero, np.ones((B, H, T)))
    scores = np.einsum("bhsk,bhtk->bhts", k, q)
    causal = np.tril(np.ones((T, T)))
    np.testing.assert_allclose(o, np.einsum("bhts,bhsv->bhtv", scores * causal, v), rtol=1e-12, atol=1e-12)


def test_no_write_is_pure_key_axis_decay():
    """w = 0: S_t = S0 Diag(prod_{s<=t} a_s) (inclusive product), o_t = S_t q_t."""
    rng = np.random.default_rng(5)
    c = rand_case(rng, B=2, H=1, T=10)
    w0 = np.zeros_like(c["w"])
    o, S_T, _ = forward(c["q"], c["k"], c["v"], c["log_g"], w0, b=c["b"], S0=c["S0"])
    cum = np.cumprod(np.exp(c["log_g"]) * c["b"], axis=2)  # [B,H,T,Dk]
    St = c["S0"][:, :, None] * cum[:, :, :, None, :]        # [B,H,T,Dv,Dk]
    np.testing.assert_allclose(o, np.einsum("bhtvk,bhtk->bhtv", St, c["q"]), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S_T, St[:, :, -1], rtol=1e-12, atol=1e-14)


def test_delta_rule_retrieval_identity():
    """After each update S_t k_t = (1 - w_t|k_t|^2) P_t k_t + w_t |k_t|^2 v_t with P_t = S_{t-1}Diag(a_t);
    with w = 1 and unit keys the state maps k_t exactly to v_t (the delta rule's defining property)."""
    rng = np.random.default_rng(6)
    c = rand_case(rng, B=1, H=2, T=15, unit_keys=False)
    _, _, _, states = forward(c["q"], c["k"], c["v"], c["log_g"], c["w"], b=c["b"], S0=c["S0"], return_states=True)
    a = np.exp(c["log_g"]) * c["b"]
    for t in range(c["k"].shape[2]):
        kt = c["k"][:, :, t]
        P = states[t] * a[:, :, t][:, :, None, :]
        nk = np.sum(kt * kt, axis=-1)
        lhs = np.einsum("bhvk,bhk->bhv", states[t + 1], kt)
        Pk = np.einsum("bhvk,bhk->bhv", P, kt)
        wt = c["w"][:, :, t]
        rhs = (1 - wt * nk)[..., None] * Pk + (wt * nk)[..., None] * c["v"][:, :, t]
        np.testing.assert_allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    c2 = rand_case(rng, B=1, H=2, T=15, unit_keys=True)
    _, _, _, states = forward(c2["q"], c2["k"], c2["v"], c2["log_g"], np.ones_like(c2["w"]), b=c2["b"],
                              S0=c2["S0"], return_states=True)
    for t in range(15):
        np.testing.assert_allclose(np.einsum("bhvk,bhk->bhv", states[t + 1], c2["k"][:, :, t]), c2["v"][:, :, t],
                                   rtol=1e-12, atol=1e-12)


def test_scalar_decay_reduces_to_rescaled_delta_rule():
    """b = 1 and a_t = alpha_t 1 (one decay per head): with S0 = 0 the decayed run equals
    (prod_{s<=t} alpha_s) times an undecayed delta-rule run on values v_t / prod_{s<=t} alpha_s."""
    rng = np.random.default_rng(7)
    c = rand_case(rng, B=1, H=2, T=14, with_b=False)
    alpha = rng.uniform(0.6, 1.0, (1, 2, 14))
    log_g = np.broadcast_to(np.log(alpha)[..., None], c["k"].shape).copy()
    o, S_T, _ = forward(c["q"], c["k"], c["v"], log_g, c["w"])
    cum = np.cumprod(alpha, axis=-1)
    o_hat, S_hat, _ = forward(c["q"], c["k"], c["v"] / cum[..., None], np.zeros_like(log_g), c["w"])
    np.testing.assert_allclose(o, cum[..., None] * o_hat, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(S_T, cum[..., -1][..., None, None] * S_hat, rtol=1e-11, atol=1e-13)


def test_frobenius_bound():
    """|S_t|_F <= max_i a_{t,i} |S_{t-1}|_F + w_t |v_t| |k_t| whenever w_t |k_t|^2 <= 2 (stability)."""
    rng = np.random.default_rng(8)
    c = rand_case(rng, B=2, H=2, T=64, Dk=16, Dv=16, unit_keys=False)
    c["k"] /= np.linalg.norm(c["k"], axis=-1, keepdims=True)
    c["k"] *= rng.uniform(0.5, 1.4, c["k"].shape[:-1])[..., None]  # w |k|^2 <= 0.95 * 1.96 < 2
    _, _, _, states = forward(c["q"], c["k"], c["v"], c["log_g"], c["w"], b=c["b"], S0=c["S0"], return_states=True)
    a = np.exp(c["log_g"]) * c["b"]
    for t in range(64):
        assert np.all(c["w"][:, :, t] * np.sum(c["k"][:, :, t] ** 2, -1) <= 2)
        lhs = np.linalg.norm(states[t + 1], axis=(-2, -1))
        rhs = (a[:, :, t].max(-1) * np.linalg.norm(states[t], axis=(-2, -1))
               + c["w"][:, :, t] * np.linalg.norm(c["v"][:, :, t], axis=-1) * np.linalg.norm(c["k"][:, :, t], axis=-1))
        assert np.all(lhs <= rhs * (1 + 1e-12))


def test_linear_in_values_and_initial_state():
    """o and S_T are jointly linear in (v, S0)."""
    rng = np.random.default_rng(9)
    c1 = rand_case(rng, T=11)
    v2 = rng.standard_normal(c1["v"].shape)
    S02 = rng.standard_normal(c1["S0"].shape)
    args = (c1["q"], c1["k"])
    o1, s1, _ = forward(*args, c1["v"], c1["log_g"], c1["w"], b=c1["b"], S0=c1["S0"])
    o2, s2, _ = forward(*args, v2, c1["log_g"], c1["w"], b=c1["b"], S0=S02)
    o3, s3, _ = forward(*args, 2 * c1["v"] - 3 * v2, c1["log_g"], c1["w"], b=c1["b"], S0=2 * c1["S0"] - 3 * S02)
    np.testing.assert_allclose(o3, 2 * o1 - 3 * o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s3, 2 * s1 - 3 * s2, rtol=1e-11, atol=1e-12)


def test_causality_and_state_carry():
    rng = np.random.default_rng(10)
    c = rand_case(rng, B=1, H=2, T=20)
    o, S_T, _ = forward(c["q"], c["k"], c["v"], c["log_g"], c["w"], b=c["b"], S0=c["S0"])
    c2 = {k_: (None if x is None else x.copy()) for k_, x in c.items()}
    for key in ("q", "k", "v", "log_g", "b"):
        c2[key][:, :, 13:] = rng.standard_normal(c2[key][:, :, 13:].shape) * 0.1 + (1 if key == "b" else 0)
    c2["w"][:, :, 13:] = 0.3
    o2, _, _ = forward(c2["q"], c2["k"], c2["v"], c2["log_g"], c2["w"], b=c2["b"], S0=c2["S0"])
    assert np.array_equal(o[:, :, :13], o2[:, :, :13])
    sl = lambda x, a_, b_: x[:, :, a_:b_]
    oa, Sa, _ = forward(*(sl(c[n], 0, 7) for n in ("q", "k", "v", "log_g", "w")), b=sl(c["b"], 0, 7), S0=c["S0"])
    ob, Sb, _ = forward(*(sl(c[n], 7, 20) for n in ("q", "k", "v", "log_g", "w")), b=sl(c["b"], 7, 20), S0=Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=2), o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(Sb, S_T, rtol=1e-13, atol=1e-14)


# ------------------------------------------------------------ content-path pins

def content_case(rng, B=1, H=2, T=12, D=3, R=2):
    c = rand_case(rng, B=B, H=H, T=T, Dk=D, Dv=D, with_b=False)
    c["b_x"] = rng.normal(1.0, 1.0, (B, H, T, D))
    c["U1"] = rng.normal(0, 0.5, (H, R, D))
    c["U2"] = rng.normal(0, 0.5, (H, D, R))
    return c


def _sig(x):
    return 1 / (1 + np.exp(-x))


def test_content_zero_projection_is_token_only():
    """U_b = 0 gives b = sigmoid(b_x) everywhere: bit-identical to U_b absent, and equal to the
    token-only path fed b = sigmoid(b_x) (zero-initialised projection reproduces the baseline)."""
    rng = np.random.default_rng(11)
    c = content_case(rng, T=12)
    base = (c["q"], c["k"], c["v"], c["log_g"], c["w"])
    zero = dict(b_x=c["b_x"], U1=np.zeros_like(c["U1"]), U2=np.zeros_like(c["U2"]))
    absent = dict(b_x=c["b_x"], U1=None, U2=None)
    oz, sz, mz = forward(*base, S0=c["S0"], L=4, content=zero)
    oa, sa, ma = forward(*base, S0=c["S0"], L=4, content=absent)
    assert np.array_equal(oz, oa) and np.array_equal(sz, sa) and np.array_equal(mz, ma)
    ot, st, _ = forward(*base, b=_sig(c["b_x"]), S0=c["S0"])
    assert np.array_equal(oz, ot) and np.array_equal(sz, st)


def test_content_chunk_composition():
    """Two chunks of L=3: chunk 0 is the token-only run with b = sigmoid(b_x); chunk 1 is the token-only
    run from the carried state with b = sigmoid(b_x + U2 U1 m_0), m_0 the mean of chunk 0's outputs;
    m_out is the mean of chunk 1's outputs.  An off-by-one in the averaged window or in the chunk that
    receives the signal fails this."""
    rng = np.random.default_rng(12)
    L = 3
    c = content_case(rng, T=2 * L)
    cont = dict(b_x=c["b_x"], U1=c["U1"], U2=c["U2"])
    o, S_T, m_out = forward(c["q"], c["k"], c["v"], c["log_g"], c["w"], S0=c["S0"], L=L, content=cont)
    s0 = lambda x: x[:, :, :L]
    s1 = lambda x: x[:, :, L:]
    names = ("q", "k", "v", "log_g", "w")
    o0, S1, _ = forward(*(s0(c[n]) for n in names), b=_sig(s0(c["b_x"])), S0=c["S0"])
    m0 = o0.mean(axis=2)                                          # [B,H,Dv]
    z = np.einsum("hkr,hrv,bhv->bhk", c["U2"], c["U1"], m0)
    o1, S2, _ = forward(*(s1(c[n]) for n in names), b=_sig(s1(c["b_x"]) + z[:, :, None, :]), S0=S1)
    np.testing.assert_allclose(o, np.concatenate([o0, o1], axis=2), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(S_T, S2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(m_out, o1.mean(axis=2), rtol=1e-13, atol=1e-14)


def test_content_first_chunk_has_no_signal_and_carry():
    rng = np.random.default_rng(13)
    L = 4
    c = content_case(rng, T=3 * L)
    names = ("q", "k", "v", "log_g", "w")
    cont = dict(b_x=c["b_x"], U1=c["U1"], U2=c["U2"])
    o, S_T, m_out = forward(*(c[n] for n in names), S0=c["S0"], L=L, content=cont)
    cont2 = dict(cont, U1=3 * c["U1"] + 1.0, U2=c["U2"] - 0.5)
    o2, _, _ = forward(*(c[n] for n in names), S0=c["S0"], L=L, content=cont2)
    assert np.array_equal(o[:, :, :L], o2[:, :, :L])
    assert not np.allclose(o[:, :, L:], o2[:, :, L:])
    # split at a chunk boundary, carrying both S and m
    cut = 2 * L
    sl = lambda x, a_, b_: x[:, :, a_:b_]
    oa, Sa, ma = forward(*(sl(c[n], 0, cut) for n in names), S0=c["S0"], L=L,
                         content=dict(cont, b_x=sl(c["b_x"], 0, cut)))
    ob, Sb, mb = forward(*(sl(c[n], cut, 3 * L) for n in names), S0=Sa, L=L,
                         content=dict(cont, b_x=sl(c["b_x"], cut, 3 * L), m0=ma))
    np.testing.assert_allclose(np.concatenate([oa, ob], 2), o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(Sb, S_T, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(mb, m_out, rtol=1e-13, atol=1e-14)


def test_content_ragged_tail_mean():
    """A final partial chunk averages over the tokens it holds."""
    rng = np.random.default_rng(14)
    L = 4
    c = content_case(rng, T=10)
    names = ("q", "k", "v", "log_g", "w")
    o, _, m_out = forward(*(c[n] for n in names), S0=c["S0"], L=L, content=dict(b_x=c["b_x"], U1=c["U1"], U2=c["U2"]))
    np.testing.assert_allclose(m_out, o[:, :, 8:10].mean(axis=2), rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------- backward pins

def _loss(c, dO, dS_T, b_key="b"):
    o, S_T, _ = forward(c["q"], c["k"], c["v"], c["log_g"], c["w"], b=c.get(b_key), S0=c["S0"])
    return np.sum(o * dO) + np.sum(S_T * dS_T)


@pytest.mark.parametrize("seed", [20, 21])
def test_backward_matches_finite_differences(seed):
    rng = np.random.default_rng(seed)
    c = rand_case(rng, B=1, H=2, T=7, Dk=3, Dv=2, unit_keys=False)
    dO = rng.standard_normal(c["v"].shape)
    dS_T = rng.standard_normal(c["S0"].shape)
    g = backward(c["q"], c["k"], c["v"], c["log_g"], c["w"], dO, b=c["b"], S0=c["S0"], dS_T=dS_T, segment=3)
    eps = 1e-6
    for name, gname in [("q", "dq"), ("k", "dk"), ("v", "dv"), ("log_g", "dlog_g"), ("b", "db"),
                        ("w", "dw"), ("S0", "dS0")]:
        x = c[name]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = x[i]
            x[i] = old + eps
            lp = _loss(c, dO, dS_T)
            x[i] = old - eps
            lm = _loss(c, dO, dS_T)
            x[i] = old
            fd[i] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g[gname], fd, rtol=1e-6, atol=1e-7, err_msg=gname)


def test_backward_directional_derivative_larger():
    """Directional finite differences at T=64, d=16 (several random directions)."""
    rng = np.random.default_rng(22)
    c = rand_case(rng, B=1, H=2, T=64, Dk=16, Dv=16)
    dO = rng.standard_normal(c["v"].shape)
    dS_T = rng.standard_normal(c["S0"].shape)
    g = backward(c["q"], c["k"], c["v"], c["log_g"], c["w"], dO, b=c["b"], S0=c["S0"], dS_T=dS_T, segment=16)
    names = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("log_g", "dlog_g"), ("b", "db"), ("w", "dw"), ("S0", "dS0")]
    for trial in range(6):
        dirs = {n: rng.standard_normal(c[n].shape) for n, _ in names}
        eps = 1e-5
        cp = {n: (c[n] + eps * dirs[n] if n in dirs else c[n]) for n in c}
        cm = {n: (c[n] - eps * dirs[n] if n in dirs else c[n]) for n in c}
        fd = (_loss(cp, dO, dS_T) - _loss(cm, dO, dS_T)) / (2 * eps)
        an = sum(np.sum(g[gn] * dirs[n]) for n, gn in names)
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (trial, fd, an)


def test_backward_homogeneity_identities():
    """o is linear in q: <dq,q> = <dO,o>.  (o, S_T) are jointly linear in (v, S0):
    <dv,v> + <dS0,S0> = <dO,o> + <dS_T,S_T>.  log a = log g + log b: dlog_g = b * db."""
    rng = np.random.default_rng(23)
    c = rand_case(rng, B=2, H=2, T=40, Dk=8, Dv=6)
    dO = rng.standard_normal(c["v"].shape)
    dS_T = rng.standard_normal(c["S0"].shape)
    o, S_T, _ = forward(c["q"], c["k"], c["v"], c["log_g"], c["w"], b=c["b"], S0=c["S0"])
    g = backward(c["q"], c["k"], c["v"], c["log_g"], c["w"], dO, b=c["b"], S0=c["S0"], dS_T=dS_T, segment=8)
    lo = np.sum(dO * o)
    ls = np.sum(dS_T * S_T)
    assert abs(np.sum(g["dq"] * c["q"]) - lo) <= 1e-11 * max(1, abs(lo))
    assert abs(np.sum(g["dv"] * c["v"]) + np.sum(g["dS0"] * c["S0"]) - lo - ls) <= 1e-11 * max(1, abs(lo + ls))
    np.testing.assert_allclose(g["dlog_g"], c["b"] * g["db"], rtol=1e-12, atol=1e-14)


def test_backward_segmenting_is_invisible():
    rng = np.random.default_rng(24)
    c = rand_case(rng, B=1, H=2, T=23, Dk=4, Dv=3)
    dO = rng.standard_normal(c["v"].shape)
    g1 = backward(c["q"], c["k"], c["v"], c["log_g"], c["w"], dO, b=c["b"], S0=c["S0"], segment=5)
    g2 = backward(c["q"], c["k"], c["v"], c["log_g"], c["w"], dO, b=c["b"], S0=c["S0"], segment=64)
    for key in g1:
        np.testing.assert_allclose(g1[key], g2[key], rtol=1e-13, atol=1e-14)


# ------------------------------------------------- content-aware backward pins

def content_case(rng, B=1, H=2, T=11, D=4, R=3, uscale=0.8):
    c = rand_case(rng, B=B, H=H, T=T, Dk=D, Dv=D, unit_keys=False, with_b=False)
    c["b_x"] = rng.normal(1.0, 1.0, (B, H, T, D))
    c["U1"] = rng.standard_normal((H, R, D)) * uscale
    c["U2"] = rng.standard_normal((H, D, R)) * uscale
    c["m0"] = rng.standard_normal((B, H, D))
    return c


def _content_loss(c, dO, dS_T, dm_out, L):
    cont = {"b_x": c["b_x"], "U1": c["U1"], "U2": c["U2"], "m0": c["m0"]}
    o, S_T, m = forward(c["q"], c["k"], c["v"], c["log_g"], c["w"], S0=c["S0"], L=L, content=cont)
    return np.sum(o * dO) + np.sum(S_T * dS_T) + np.sum(m * dm_out)


@pytest.mark.parametrize("seed,T,L", [(30, 11, 4), (31, 9, 3), (32, 6, 8)])
def test_content_backward_matches_finite_differences(seed, T, L):
    """Every input, including the projection, the carried-in mean and S0, against
    central differences of <dO,o> + <dS_T,S_T> + <dm_out,m_out> (ragged last chunk,
    several chunks, and a single chunk)."""
    rng = np.random.default_rng(seed)
    c = content_case(rng, T=T)
    dO = rng.standard_normal(c["v"].shape)
    dS_T = rng.standard_normal(c["S0"].shape)
    dm_out = rng.standard_normal(c["m0"].shape)
    g = backward_content(c["q"], c["k"], c["v"], c["log_g"], c["w"], dO,
                         {"b_x": c["b_x"], "U1": c["U1"], "U2": c["U2"], "m0": c["m0"]},
                         S0=c["S0"], dS_T=dS_T, dm_out=dm_out, L=L)
    eps = 1e-6
    for name, gname in [("q", "dq"), ("k", "dk"), ("v", "dv"), ("log_g", "dlog_g"), ("b_x", "db_x"), ("w", "dw"),
                        ("U1", "dU1"), ("U2", "dU2"), ("m0", "dm0"), ("S0", "dS0")]:
        x = c[name]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = x[i]
            x[i] = old + eps
            lp = _content_loss(c, dO, dS_T, dm_out, L)
            x[i] = old - eps
            lm = _content_loss(c, dO, dS_T, dm_out, L)
            x[i] = old
            fd[i] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g[gname], fd, rtol=1e-6, atol=1e-7, err_msg=gname)


def test_content_backward_zero_projection_is_token_only():
    """With U1 = U2 = 0 the gate is b = sigmoid(b_x) in every chunk: the gradients are
    the token-only backward's with that b, db_x = db * b (1 - b), and nothing flows into
    the projection or the carried-in mean."""
    rng = np.random.default_rng(33)
    c = content_case(rng, B=2, H=2, T=21, D=5)
    dO = rng.standard_normal(c["v"].shape)
    dS_T = rng.standard_normal(c["S0"].shape)
    bz = 1.0 / (1.0 + np.exp(-c["b_x"]))
    ref = backward(c["q"], c["k"], c["v"], c["log_g"], c["w"], dO, b=bz, S0=c["S0"], dS_T=dS_T)
    for U1, U2 in ((np.zeros_like(c["U1"]), np.zeros_like(c["U2"])), (None, None)):
        g = backward_content(c["q"], c["k"], c["v"], c["log_g"], c["w"], dO,
                             {"b_x": c["b_x"], "U1": U1, "U2": U2, "m0": c["m0"]}, S0=c["S0"], dS_T=dS_T, L=4)
        for key in ("dq", "dk", "dv", "dlog_g", "dw", "dS0"):
            np.testing.assert_allclose(g[key], ref[key], rtol=1e-12, atol=1e-13, err_msg=key)
        np.testing.assert_allclose(g["db_x"], ref["db"] * bz * (1 - bz), rtol=1e-12, atol=1e-13)
        assert np.all(g["dm0"] == 0)
        if U1 is not None:
            assert np.all(g["dU1"] == 0) and np.all(g["dU2"] == 0)


def test_content_backward_first_chunk_gradient_of_m0():
    """In a single chunk, m0 enters only through z = U2 U1 m0, so
    dm0 = U1^T U2^T sum_t db_x,t exactly (per head, no batch sum)."""
    rng = np.random.default_rng(34)
    c = content_case(rng, B=2, H=2, T=5, D=4)
    dO = rng.standard_normal(c["v"].shape)
    g = backward_content(c["q"], c["k"], c["v"], c["log_g"], c["w"], dO,
                         {"b_x": c["b_x"], "U1": c["U1"], "U2": c["U2"], "m0": c["m0"]}, S0=c["S0"], L=8)
    dz = g["db_x"].sum(axis=2)                                   # [B,H,Dk]
    want = np.einsum("hrv,hkr,bhk->bhv", c["U1"], c["U2"], dz)
    np.testing.assert_allclose(g["dm0"], want, rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------ gate pre-activations

def logit_case(rng, B=1, H=2, T=9, D=3, with_bx=True):
    c = rand_case(rng, B=B, H=H, T=T, Dk=D, Dv=D, unit_keys=False, with_b=False)
    c["f"] = rng.standard_normal((B, H, T, D))
    c["A"] = rng.uniform(0.05, 0.6, (H, D))
    c["tau"] = rng.standard_normal((H, D)) * 0.5
    c["w_hat"] = rng.standard_normal((B, H, T))
    c["b_x"] = rng.normal(1.0, 1.0, (B, H, T, D)) if with_bx else None
    return c


def test_gates_from_logits_values():
    """The activations themselves: softplus(0) = log 2, sigmoid(0) = 1/2, and log g <= 0."""
    f = np.zeros((1, 1, 1, 2))
    log_g, b, w = gates_from_logits(f, np.array([[1.0, 2.0]]), np.zeros((1, 2)), np.zeros((1, 1, 1)), b_x=f)
    np.testing.assert_allclose(log_g[0, 0, 0], [-np.log(2.0), -2 * np.log(2.0)], rtol=1e-15)
    assert np.all(b == 0.5) and np.all(w == 0.5)
    rng = np.random.default_rng(40)
    lg, _, _ = gates_from_logits(rng.standard_normal((2, 3, 5, 4)) * 30, rng.uniform(0, 2, (3, 4)),
                                 rng.standard_normal((3, 4)), rng.standard_normal((2, 3, 5)))
    assert np.all(lg <= 0) and np.all(np.isfinite(lg))


def test_gates_from_logits_bias_inside_softplus():
    """Nonzero logits and bias, per head and key channel (notes section 2.3, fused-gate legend:
    the bias shifts the decay logit before the softplus).  f = 1, tau = -1 gives softplus(0) =
    log 2; f = 2, tau = log(e - 1) - 2 gives softplus(log(e - 1)) = 1; f = -1, tau = 1 + log 3
    gives log 4.  A misplaced bias (softplus(f) + tau) or a head/channel mix-up of A or tau
    changes every one of these.  b_x = log 3 gives b = 3/4; w_hat = -log 3 gives w = 1/4."""
    A = np.array([[0.7, 1.9, 3.0], [5.0, 0.25, 10.0]])                 # [H=2, Dk=3]
    tau = np.array([[-1.0, np.log(np.e - 1.0) - 2.0, 1.0 + np.log(3.0)],
                    [1.0 + np.log(3.0), -1.0, np.log(np.e - 1.0) - 2.0]])
    f = np.empty((1, 2, 2, 3))
    f[0, 0, :] = [1.0, 2.0, -1.0]
    f[0, 1, :] = [-1.0, 1.0, 2.0]
    b_x = np.full((1, 2, 2, 3), np.log(3.0))
    w_hat = np.full((1, 2, 2), -np.log(3.0))
    log_g, b, w = gates_from_logits(f, A, tau, w_hat, b_x=b_x)
    sp = np.array([[np.log(2.0), 1.0, np.log(4.0)], [np.log(4.0), np.log(2.0), 1.0]])
    for t in range(2):
        np.testing.assert_allclose(log_g[0, :, t], -A * sp, rtol=1e-14)
    np.testing.assert_allclose(b, 0.75, rtol=1e-15)
    np.testing.assert_allclose(w, 0.25, rtol=1e-15)


@pytest.mark.parametrize("with_bx", [True, False])
def test_logit_backward_matches_finite_differences(with_bx):
    rng = np.random.default_rng(41 + with_bx)
    c = logit_case(rng, with_bx=with_bx)
    dO = rng.standard_normal(c["v"].shape)
    dS_T = rng.standard_normal(c["S0"].shape)

    def loss():
        o, S_T = forward_logits(c["q"], c["k"], c["v"], c["f"], c["A"], c["tau"], c["w_hat"], b_x=c["b_x"],
                                S0=c["S0"])
        return np.sum(o * dO) + np.sum(S_T * dS_T)

    g = backward_logits(c["q"], c["k"], c["v"], c["f"], c["A"], c["tau"], c["w_hat"], dO, b_x=c["b_x"],
                        S0=c["S0"], dS_T=dS_T)
    eps = 1e-6
    names = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("f", "df"), ("A", "dA"), ("tau", "dtau"),
             ("w_hat", "dw_hat"), ("S0", "dS0")] + ([("b_x", "db_x")] if with_bx else [])
    for name, gname in names:
        x = c[name]
        fd = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = x[i]
            x[i] = old + eps
            lp = loss()
            x[i] = old - eps
            lm = loss()
            x[i] = old
            fd[i] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(g[gname], fd, rtol=1e-6, atol=1e-7, err_msg=gname)
    if not with_bx:
        assert g["db_x"] is None


@pytest.mark.parametrize("Dk,Dv", [(6, 3), (3, 6)])
def test_unequal_widths_reduce_to_padded_equal_widths(Dk, Dv):
    """The state is d_v x d_k with independent widths (notes section 1).  Each value row of
    the recurrence evolves on its own, and a key channel with k = q = 0 and a = 1 neither
    feeds nor is fed by the others, so zero-padding the narrower axis to the wider one
    reproduces the unequal-width result on the true rows and columns: forward outputs, the
    final state and every gradient."""
    rng = np.random.default_rng(90 + Dk)
    c = rand_case(rng, B=1, H=2, T=11, Dk=Dk, Dv=Dv)
    dO = rng.standard_normal(c["v"].shape)
    dS_T = rng.standard_normal(c["S0"].shape)
    D = max(Dk, Dv)

    def pad(x, axis_len, fill=0.0):
        out = np.full(x.shape[:-1] + (axis_len,), fill)
        out[..., :x.shape[-1]] = x
        return out

    p = dict(c)
    p["q"], p["k"] = pad(c["q"], D), pad(c["k"], D)
    p["log_g"], p["b"] = pad(c["log_g"], D, 0.0), pad(c["b"], D, 1.0)
    p["v"] = pad(c["v"], D)
    p["S0"] = np.zeros(c["S0"].shape[:2] + (D, D))
    p["S0"][..., :Dv, :Dk] = c["S0"]
    pdS = np.zeros_like(p["S0"])
    pdS[..., :Dv, :Dk] = dS_T
    o, S_T, _ = forward(c["q"], c["k"], c["v"], c["log_g"], c["w"], b=c["b"], S0=c["S0"])
    po, pS, _ = forward(p["q"], p["k"], p["v"], p["log_g"], p["w"], b=p["b"], S0=p["S0"])
    np.testing.assert_allclose(po[..., :Dv], o, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(pS[..., :Dv, :Dk], S_T, rtol=1e-12, atol=1e-12)
    assert np.all(po[..., Dv:] == 0) and np.all(pS[..., Dv:, :] == 0) and np.all(pS[..., :, Dk:] == 0)
    g = backward(c["q"], c["k"], c["v"], c["log_g"], c["w"], dO, b=c["b"], S0=c["S0"], dS_T=dS_T)
    pg = backward(p["q"], p["k"], p["v"], p["log_g"], p["w"], pad(dO, D), b=p["b"], S0=p["S0"], dS_T=pdS)
    for key, width in (("dq", Dk), ("dk", Dk), ("dlog_g", Dk), ("db", Dk), ("dv", Dv)):
        np.testing.assert_allclose(pg[key][..., :width], g[key], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(pg["dw"], g["dw"], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(pg["dS0"][..., :Dv, :Dk], g["dS0"], rtol=1e-10, atol=1e-12)
