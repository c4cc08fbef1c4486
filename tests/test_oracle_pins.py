"""Pins for the float64 oracle: facts fixed by the pages and by the mathematics.

Every check here compares the oracle with something other than itself:
a worked example derived by hand, closed forms, textbook special cases
(the plain delta rule, gated DeltaNet, gated linear attention), brute-force
dense unrolling with explicit transition matrices, and invariants (content
boundary, chunk-length independence without a content projection, state
chaining). The pages print no numeric example of their own.
"""
import json
import os

import numpy as np
import pytest

from oracle import (carve_backward, carve_forward, carve_step, decay_from_logits, l2_normalize,
                    l2_normalize_backward, sigmoid)

HERE = os.path.dirname(os.path.abspath(__file__))


def rand_inputs(rng, B, T, H, dk, dv, rank=0, ub_std=0.3):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    x = rng.standard_normal((B, T, H, dk))
    g = -(np.maximum(x, 0) + np.log1p(np.exp(-np.abs(x))))
    bx = rng.standard_normal((B, T, H, dk))
    w = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    Ud = Uu = None
    if rank:
        Ud = ub_std * rng.standard_normal((H, rank, dv))
        Uu = ub_std * rng.standard_normal((H, dk, rank))
    return q, k, v, g, bx, w, Ud, Uu


# ---------------------------------------------------------------- worked example

def test_hand_worked_example():
    """Gist.science summary §2.1-2.3: a 4-token pass worked by hand (tests/golden)."""
    fx = json.load(open(os.path.join(HERE, "golden", "hand_worked_content_gate.json")))
    tb = lambda key: np.transpose(np.array(fx[key], dtype=np.float64), (1, 0, 2, 3))
    q, k, v = tb("q"), tb("k"), tb("v")
    g = np.log(tb("g_exp"))
    p = tb("bx_sigmoid")
    bx = np.log(p / (1 - p))
    w = np.transpose(np.array(fx["w"]), (1, 0, 2))
    Ud = np.array(fx["U_down"])
    Uu = np.log(np.array(fx["U_up_exp"]))
    o, S, m = carve_forward(q, k, v, g, bx, w, fx["L"], Ud, Uu,
                            state_in=np.array(fx["state_in"]))
    np.testing.assert_allclose(o, tb("expected_o"), rtol=0, atol=1e-12)
    np.testing.assert_allclose(S, np.array(fx["expected_state_out"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(m, np.array(fx["expected_mean_out"]), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- closed forms

def test_single_token_closed_form():
    """T=1: o_1 = S_in q_1 and S_1 = S_in D (I - (b k) k^T) + w v k^T with b from mean_in."""
    rng = np.random.default_rng(1)
    B, H, dk, dv, r = 2, 3, 5, 4, 2
    q, k, v, g, bx, w, Ud, Uu = rand_inputs(rng, B, 1, H, dk, dv, rank=r)
    S_in = rng.standard_normal((B, H, dv, dk))
    m_in = rng.standard_normal((B, H, dv))
    o, S, m = carve_forward(q, k, v, g, bx, w, 1, Ud, Uu, state_in=S_in, mean_in=m_in)
    for b_ in range(B):
        for h in range(H):
            z = Uu[h] @ (Ud[h] @ m_in[b_, h])
            bb = 1 / (1 + np.exp(-(bx[b_, 0, h] + z)))
            kk = k[b_, 0, h]
            D = np.diag(np.exp(g[b_, 0, h]))
            S1 = S_in[b_, h] @ D @ (np.eye(dk) - np.outer(bb * kk, kk)) + w[b_, 0, h] * np.outer(v[b_, 0, h], kk)
            np.testing.assert_allclose(o[b_, 0, h], S_in[b_, h] @ q[b_, 0, h], atol=1e-13)
            np.testing.assert_allclose(S[b_, h], S1, atol=1e-13)
            np.testing.assert_allclose(m[b_, h], S_in[b_, h] @ q[b_, 0, h], atol=1e-13)


def test_zero_state_first_token():
    """With S_in = 0 the first readout is 0 and S_1 = w v k^T."""
    rng = np.random.default_rng(2)
    q, k, v, g, bx, w, _, _ = rand_inputs(rng, 1, 1, 2, 6, 3)
    o, S, _ = carve_forward(q, k, v, g, bx, w, 1)
    assert np.all(o == 0)
    np.testing.assert_allclose(S[0], w[0, 0, :, None, None] * v[0, 0][:, :, None] * k[0, 0][:, None, :], atol=1e-15)


def test_plain_delta_rule_exact_retrieval():
    """b=1, g=0, w=1 is the delta rule: with unit keys S_t k_t = v_t exactly,
    so a query equal to the last key reads back the last value."""
    rng = np.random.default_rng(3)
    B, T, H, dk, dv = 1, 12, 2, 8, 5
    q, k, v, _, _, _, _, _ = rand_inputs(rng, B, T, H, dk, dv)
    q[:, 1:] = k[:, :-1]                   # query t+1 = key t
    g = np.zeros_like(k)
    bx = np.full_like(k, 40.0)             # sigmoid(40) == 1.0 exactly in float64
    assert sigmoid(40.0) == 1.0
    w = np.ones((B, T, H))
    o, S, _ = carve_forward(q, k, v, g, bx, w, 4)
    np.testing.assert_allclose(o[:, 1:], v[:, :-1], atol=1e-12)
    np.testing.assert_allclose(np.einsum("bhed,bhd->bhe", S, k[:, -1]), v[:, -1], atol=1e-12)


def test_plain_delta_rule_orthonormal_keys():
    """Delta rule with orthonormal keys and T <= d_k: S_T = sum_t v_t k_t^T."""
    rng = np.random.default_rng(4)
    dk, dv, T = 8, 3, 6
    Q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Q[:, :T].T[None, :, None, :]
    v = rng.standard_normal((1, T, 1, dv))
    q = rng.standard_normal((1, T, 1, dk))
    o, S, _ = carve_forward(q, k, v, np.zeros_like(k), np.full_like(k, 40.0), np.ones((1, T, 1)), T)
    np.testing.assert_allclose(S[0, 0], sum(np.outer(v[0, t, 0], k[0, t, 0]) for t in range(T)), atol=1e-12)


def test_gated_deltanet_special_case():
    """Theorem 1 (subsumption): scalar decay alpha and scalar erase=write beta give
    gated DeltaNet, S_t = alpha_t S_{t-1} (I - beta_t k k^T) + beta_t v k^T."""
    rng = np.random.default_rng(5)
    B, T, H, dk, dv = 2, 10, 2, 6, 4
    q, k, v, _, _, _, _, _ = rand_inputs(rng, B, T, H, dk, dv)
    alpha = rng.uniform(0.3, 1.0, (B, T, H))
    beta = rng.uniform(0.05, 0.95, (B, T, H))
    g = np.repeat(np.log(alpha)[..., None], dk, axis=-1)
    bx = np.repeat(np.log(beta / (1 - beta))[..., None], dk, axis=-1)
    o, S, _ = carve_forward(q, k, v, g, bx, beta, 5)
    for b_ in range(B):
        for h in range(H):
            St = np.zeros((dv, dk))
            for t in range(T):
                np.testing.assert_allclose(o[b_, t, h], St @ q[b_, t, h], atol=1e-12)
                kk = k[b_, t, h]
                St = alpha[b_, t, h] * St @ (np.eye(dk) - beta[b_, t, h] * np.outer(kk, kk)) \
                    + beta[b_, t, h] * np.outer(v[b_, t, h], kk)
            np.testing.assert_allclose(S[b_, h], St, atol=1e-12)


def test_no_erase_is_gated_linear_attention():
    """b = 0 leaves decay and write only: o_t = S_in (e^{G_{t-1}} q_t)
    + sum_{j<t} w_j v_j <k_j e^{G_{t-1} - G_j}, q_t> (G inclusive, G_{-1} = 0).
    Pins the key-axis decay direction and the exclusive readout index."""
    rng = np.random.default_rng(6)
    B, T, H, dk, dv = 1, 9, 2, 5, 3
    q, k, v, g, _, w, _, _ = rand_inputs(rng, B, T, H, dk, dv)
    bx = np.full_like(k, -800.0)           # sigmoid(-800) underflows to 0.0
    assert sigmoid(-800.0) == 0.0
    S_in = rng.standard_normal((B, H, dv, dk))
    o, _, _ = carve_forward(q, k, v, g, bx, w, 3, state_in=S_in)
    G = np.cumsum(g, axis=1)
    for h in range(H):
        for t in range(T):
            Gp = G[0, t - 1, h] if t > 0 else np.zeros(dk)
            ref = S_in[0, h] @ (np.exp(Gp) * q[0, t, h])
            for j in range(t):
                ref = ref + w[0, j, h] * v[0, j, h] * np.dot(k[0, j, h] * np.exp(Gp - G[0, j, h]), q[0, t, h])
            np.testing.assert_allclose(o[0, t, h], ref, atol=1e-12)


def test_hard_decay_is_memoryless():
    """alpha = 0 (g = -1e4): every step wipes the state, so o_{t+1} = w_t v_t <k_t, q_{t+1}>."""
    rng = np.random.default_rng(7)
    B, T, H, dk, dv = 1, 8, 2, 6, 4
    q, k, v, _, bx, w, _, _ = rand_inputs(rng, B, T, H, dk, dv)
    g = np.full_like(k, -1e4)
    S_in = rng.standard_normal((B, H, dv, dk))
    o, S, _ = carve_forward(q, k, v, g, bx, w, 4, state_in=S_in)
    ref = w[:, :-1, :, None] * v[:, :-1] * np.sum(k[:, :-1] * q[:, 1:], axis=-1, keepdims=True)
    np.testing.assert_allclose(o[:, 1:], ref, atol=1e-13)
    np.testing.assert_allclose(o[0, 0], np.einsum("hed,hd->he", S_in[0], q[0, 0]), atol=1e-13)
    np.testing.assert_allclose(S[0], w[0, -1, :, None, None] * v[0, -1][:, :, None] * k[0, -1][:, None, :], atol=1e-13)


# ---------------------------------------------------------------- brute force

def brute_force(q, k, v, g, bx, w, L, Ud, Uu, S_in):
    """Dense unrolling with explicit d_k x d_k transitions M_t = D_t (I - (b_t k_t) k_t^T):
    S_t = S_in prod_{s<=t} M_s + sum_{j<=t} w_j v_j k_j^T prod_{j<s<=t} M_s,
    each S_t rebuilt from scratch; the content gate is recomputed from the
    previous chunk's outputs."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    o = np.zeros((B, T, H, dv))
    S_T = np.zeros((B, H, dv, dk))
    for b_ in range(B):
        for h in range(H):
            M, W = [], []
            prev_mean = np.zeros(dv)
            for t in range(T):
                c = t // L
                if t % L == 0 and c > 0:
                    prev_mean = o[b_, (c - 1) * L:c * L, h].mean(axis=0)
                z = Uu[h] @ (Ud[h] @ prev_mean) if Ud is not None else 0.0
                bb = 1 / (1 + np.exp(-(bx[b_, t, h] + z)))
                kk = k[b_, t, h]
                M.append(np.diag(np.exp(g[b_, t, h])) @ (np.eye(dk) - np.outer(bb * kk, kk)))
                W.append(w[b_, t, h] * np.outer(v[b_, t, h], kk))

                def state_after(n):          # state after n tokens, from scratch
                    P = np.eye(dk)
                    for s in range(n):
                        P = P @ M[s]
                    acc = S_in[b_, h] @ P
                    for j in range(n):
                        P = np.eye(dk)
                        for s in range(j + 1, n):
                            P = P @ M[s]
                        acc = acc + W[j] @ P
                    return acc
                o[b_, t, h] = state_after(t) @ q[b_, t, h]
            S_T[b_, h] = state_after(T)
    return o, S_T


@pytest.mark.parametrize("L,T", [(1, 12), (2, 12), (3, 12), (4, 12), (4, 11), (5, 12)])
def test_brute_force_unrolling(L, T):
    rng = np.random.default_rng(10 + L + T)
    B, H, dk, dv = 1, 2, 5, 3
    q, k, v, g, bx, w, Ud, Uu = rand_inputs(rng, B, T, H, dk, dv, rank=2, ub_std=1.5)
    S_in = rng.standard_normal((B, H, dv, dk))
    o, S, _ = carve_forward(q, k, v, g, bx, w, L, Ud, Uu, state_in=S_in)
    o_ref, S_ref = brute_force(q, k, v, g, bx, w, L, Ud, Uu, S_in)
    np.testing.assert_allclose(o, o_ref, atol=1e-12)
    np.testing.assert_allclose(S, S_ref, atol=1e-12)


# ---------------------------------------------------------------- content path

def test_content_gate_closed_form():
    """Gist.science summary §2.1: chunk 1 is gated by the mean of chunk 0's outputs.
    With k = 0 and g = 0 in chunk 0, S stays S_in, so m_0 = S_in mean(q_0..q_{L-1})
    and the second token of chunk 1 reads S_in D (I - (b k) k^T) + w v k^T with
    b = sigmoid(bx + U_up U_down m_0)."""
    rng = np.random.default_rng(20)
    B, L, H, dk, dv, r = 1, 4, 2, 5, 3, 2
    T = 2 * L
    q, k, v, g, bx, w, Ud, Uu = rand_inputs(rng, B, T, H, dk, dv, rank=r, ub_std=2.0)
    k[:, :L] = 0.0
    g[:, :L] = 0.0
    S_in = rng.standard_normal((B, H, dv, dk))
    o, _, _ = carve_forward(q, k, v, g, bx, w, L, Ud, Uu, state_in=S_in)
    for h in range(H):
        m0 = S_in[0, h] @ q[0, :L, h].mean(axis=0)
        b = 1 / (1 + np.exp(-(bx[0, L, h] + Uu[h] @ (Ud[h] @ m0))))
        kk = k[0, L, h]
        S1 = S_in[0, h] @ np.diag(np.exp(g[0, L, h])) @ (np.eye(dk) - np.outer(b * kk, kk)) \
            + w[0, L, h] * np.outer(v[0, L, h], kk)
        np.testing.assert_allclose(o[0, :L + 1, h], q[0, :L + 1, h] @ S_in[0, h].T, atol=1e-13)
        np.testing.assert_allclose(o[0, L + 1, h], S1 @ q[0, L + 1, h], atol=1e-13)


def test_short_sequence_gets_no_content_signal():
    """Limitations paragraph: a sequence no longer than one chunk gets no content
    signal, so with mean_in = 0 the output does not depend on U_b at all."""
    rng = np.random.default_rng(21)
    q, k, v, g, bx, w, Ud, Uu = rand_inputs(rng, 2, 8, 2, 6, 4, rank=3, ub_std=3.0)
    o0, S0, _ = carve_forward(q, k, v, g, bx, w, 8)
    o1, S1, _ = carve_forward(q, k, v, g, bx, w, 8, Ud, Uu)
    assert np.array_equal(o0, o1) and np.array_equal(S0, S1)
    o2, _, _ = carve_forward(q, k, v, g, bx, w, 4, Ud, Uu)     # two chunks: the signal exists
    assert np.abs(o2 - o0).max() > 1e-3


def test_zero_projection_is_memory_blind_key_axis_rule():
    """U_b = 0 gives the memory-blind key-axis gated delta rule: b = sigmoid(bx),
    S_t = S_{t-1} D_t (I - (b_t k_t) k_t^T) + w_t v_t k_t^T, written here with
    explicit matrices. A zero-filled projection equals an absent one bitwise,
    and the output does not depend on L."""
    rng = np.random.default_rng(22)
    B, T, H, dk, dv, r = 1, 16, 2, 6, 4, 3
    q, k, v, g, bx, w, Ud, Uu = rand_inputs(rng, B, T, H, dk, dv, rank=r)
    S_in = rng.standard_normal((B, H, dv, dk))
    o, S, _ = carve_forward(q, k, v, g, bx, w, 4, state_in=S_in)
    oz, Sz, _ = carve_forward(q, k, v, g, bx, w, 4, np.zeros_like(Ud), np.zeros_like(Uu), state_in=S_in)
    assert np.array_equal(o, oz) and np.array_equal(S, Sz)
    for L in (1, 2, 8, 16):
        oL, SL, _ = carve_forward(q, k, v, g, bx, w, L, state_in=S_in)
        assert np.array_equal(oL, o) and np.array_equal(SL, S)
    for h in range(H):
        St = S_in[0, h].copy()
        for t in range(T):
            np.testing.assert_allclose(o[0, t, h], St @ q[0, t, h], atol=1e-12)
            bb = 1 / (1 + np.exp(-bx[0, t, h]))
            kk = k[0, t, h]
            St = St @ np.diag(np.exp(g[0, t, h])) @ (np.eye(dk) - np.outer(bb * kk, kk)) \
                + w[0, t, h] * np.outer(v[0, t, h], kk)
        np.testing.assert_allclose(S[0, h], St, atol=1e-12)


def test_state_and_mean_chaining():
    """Running [0, T) equals [0, T/2) then [T/2, T) with S and m carried over."""
    rng = np.random.default_rng(23)
    B, T, H, dk, dv, L = 2, 24, 2, 5, 4, 4
    q, k, v, g, bx, w, Ud, Uu = rand_inputs(rng, B, T, H, dk, dv, rank=2, ub_std=2.0)
    o, S, m = carve_forward(q, k, v, g, bx, w, L, Ud, Uu)
    h = T // 2
    oa, Sa, ma = carve_forward(q[:, :h], k[:, :h], v[:, :h], g[:, :h], bx[:, :h], w[:, :h], L, Ud, Uu)
    ob, Sb, mb = carve_forward(q[:, h:], k[:, h:], v[:, h:], g[:, h:], bx[:, h:], w[:, h:], L, Ud, Uu,
                               state_in=Sa, mean_in=ma)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=1), o, atol=1e-13)
    np.testing.assert_allclose(Sb, S, atol=1e-13)
    np.testing.assert_allclose(mb, m, atol=1e-13)


def test_state_stays_bounded():
    """Theorem 4 (Lyapunov): with decay and erase the state norm stays bounded."""
    rng = np.random.default_rng(24)
    q, k, v, g, bx, w, Ud, Uu = rand_inputs(rng, 1, 2048, 2, 16, 16, rank=4, ub_std=0.05)
    o, S, m = carve_forward(q, k, v, g, bx, w, 64, Ud, Uu)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(S))
    assert np.abs(S).max() < 10.0


def test_ragged_length_is_causal_prefix():
    """A partial last chunk (reading R6): outputs are causal, so a ragged run is
    the prefix of a longer run, and mean_out is the mean of its partial chunk."""
    rng = np.random.default_rng(25)
    q, k, v, g, bx, w, Ud, Uu = rand_inputs(rng, 2, 16, 2, 5, 4, rank=2, ub_std=2.0)
    o16, _, _ = carve_forward(q, k, v, g, bx, w, 4, Ud, Uu)
    sl = slice(0, 11)
    o11, S11, m11 = carve_forward(q[:, sl], k[:, sl], v[:, sl], g[:, sl], bx[:, sl], w[:, sl], 4, Ud, Uu)
    np.testing.assert_array_equal(o11, o16[:, :11])
    np.testing.assert_allclose(m11, o11[:, 8:11].mean(axis=1), atol=1e-14)


def test_empty_sequence_passes_state_through():
    rng = np.random.default_rng(26)
    q, k, v, g, bx, w, Ud, Uu = rand_inputs(rng, 1, 0, 2, 4, 3, rank=2)
    S_in = rng.standard_normal((1, 2, 3, 4))
    m_in = rng.standard_normal((1, 2, 3))
    o, S, m = carve_forward(q, k, v, g, bx, w, 4, Ud, Uu, state_in=S_in, mean_in=m_in)
    assert o.shape == (1, 0, 2, 3)
    np.testing.assert_array_equal(S, S_in)
    np.testing.assert_array_equal(m, m_in)


# ---------------------------------------------------------------- decode step

def test_step_hand_worked_example():
    """The 4-token hand-worked pass (tests/golden), taken one decode step at a
    time: every output, the final state and both chunk means."""
    fx = json.load(open(os.path.join(HERE, "golden", "hand_worked_content_gate.json")))
    tok = lambda key, t: np.array(fx[key][t], dtype=np.float64)   # [B, H, d]
    Ud = np.array(fx["U_down"])
    Uu = np.log(np.array(fx["U_up_exp"]))
    L = fx["L"]
    S = np.array(fx["state_in"], dtype=np.float64)
    m = np.zeros((1, 1, 1))
    acc = np.zeros((1, 1, 1))
    means = []
    for t in range(4):
        p = tok("bx_sigmoid", t)
        o, S, m, acc = carve_step(S, m, acc, t % L, tok("q", t), tok("k", t), tok("v", t),
                                  np.log(tok("g_exp", t)), np.log(p / (1 - p)), np.array(fx["w"][t]), L, Ud, Uu)
        np.testing.assert_allclose(o, tok("expected_o", t), rtol=0, atol=1e-12)
        if t % L == L - 1:
            means.append(float(m[0, 0, 0]))
            assert not acc.any()
    np.testing.assert_allclose(S, np.array(fx["expected_state_out"]), rtol=0, atol=1e-12)
    # m0 = (4 + 1) / 2 (derivation in the fixture), m1 = the fixture's mean_out
    np.testing.assert_allclose(means, [2.5, np.array(fx["expected_mean_out"]).item()], rtol=0, atol=1e-12)


@pytest.mark.parametrize("T,L", [(10, 4), (8, 4), (7, 1), (5, 8)])
def test_step_sequence_equals_forward(T, L):
    """Stepping t = 0 .. T-1 with pos = t mod L from (state_in, mean_in, 0)
    gives the forward pass's outputs and state; after the last whole chunk the
    carried mean is that chunk's mean, and a partial last chunk's mean is the
    carried sum over its tokens."""
    rng = np.random.default_rng(T * 10 + L)
    B, H, dk, dv, r = 2, 3, 5, 4, 3
    q, k, v, g, bx, w, Ud, Uu = rand_inputs(rng, B, T, H, dk, dv, rank=r)
    S_in = rng.standard_normal((B, H, dv, dk))
    m_in = rng.standard_normal((B, H, dv))
    o_ref, S_ref, m_ref = carve_forward(q, k, v, g, bx, w, L, Ud, Uu, state_in=S_in, mean_in=m_in)
    S, m, acc = S_in.copy(), m_in.copy(), np.zeros((B, H, dv))
    for t in range(T):
        o, S, m, acc = carve_step(S, m, acc, t % L, q[:, t], k[:, t], v[:, t], g[:, t], bx[:, t], w[:, t],
                                  L, Ud, Uu)
        np.testing.assert_allclose(o, o_ref[:, t], rtol=0, atol=1e-13)
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=1e-13)
    tail = T % L
    if tail == 0:
        np.testing.assert_allclose(m, m_ref, rtol=0, atol=1e-13)
    else:
        np.testing.assert_allclose(acc / tail, m_ref, rtol=0, atol=1e-13)


def test_step_rejects_position_outside_chunk():
    rng = np.random.default_rng(3)
    q, k, v, g, bx, w, _, _ = rand_inputs(rng, 1, 1, 1, 2, 2)
    with pytest.raises(ValueError):
        carve_step(np.zeros((1, 1, 2, 2)), np.zeros((1, 1, 2)), np.zeros((1, 1, 2)), 4,
                   q[:, 0], k[:, 0], v[:, 0], g[:, 0], bx[:, 0], w[:, 0], 4)


# ---------------------------------------------------------------- decay activation

def test_decay_from_logits_closed_forms():
    """g = -softplus(a): g(0) = -ln 2; a = ln 3 gives exp(g) = 1/4 exactly in
    closed form; exp(g(a)) = 1 / (1 + e^a), so the decay factor falls as the
    logit rises; g(a) - g(-a) = -a; and d g / d a = -1 / (1 + e^{-a})."""
    assert decay_from_logits(0.0) == pytest.approx(-np.log(2.0), rel=1e-15)
    assert np.exp(decay_from_logits(np.log(3.0))) == pytest.approx(0.25, rel=1e-15)
    a = np.linspace(-30.0, 30.0, 121)
    np.testing.assert_allclose(np.exp(decay_from_logits(a)), 1.0 / (1.0 + np.exp(a)), rtol=1e-13, atol=0)
    np.testing.assert_allclose(decay_from_logits(a) - decay_from_logits(-a), -a, rtol=0, atol=1e-13)
    h = 1e-6
    fd = (decay_from_logits(a + h) - decay_from_logits(a - h)) / (2 * h)
    np.testing.assert_allclose(fd, -1.0 / (1.0 + np.exp(-a)), rtol=0, atol=1e-8)
    assert np.all(decay_from_logits(a) < 0)


def test_decay_from_logits_extremes():
    """Neither end overflows or loses its leading term: g(800) = -800 (the
    decay is e^-800), and g(-50) = -e^-50 (1 - e^-50 / 2 + ...), a decay within
    1e-22 of one that must not round to zero."""
    assert decay_from_logits(800.0) == -800.0
    assert decay_from_logits(1e4) == -1e4
    assert decay_from_logits(-50.0) == pytest.approx(-np.exp(-50.0), rel=1e-15, abs=0)
    assert decay_from_logits(-700.0) == pytest.approx(-np.exp(-700.0), rel=1e-15, abs=0)   # e^-700 is still normal


def test_decay_logits_in_the_layer():
    """The activation composed with the layer: logits of +1e4 are the hard
    decay (every token wipes the state), and logits of -50 leave the state
    undecayed to within 1e-21, so the layer is the ungated rule on those."""
    rng = np.random.default_rng(17)
    B, T, H, dk, dv = 1, 8, 2, 6, 4
    q, k, v, _, bx, w, _, _ = rand_inputs(rng, B, T, H, dk, dv)
    o_hard, _, _ = carve_forward(q, k, v, decay_from_logits(np.full_like(k, 1e4)), bx, w, 4)
    ref = w[:, :-1, :, None] * v[:, :-1] * np.sum(k[:, :-1] * q[:, 1:], axis=-1, keepdims=True)
    np.testing.assert_allclose(o_hard[:, 1:], ref, atol=1e-13)
    o_none, S_none, _ = carve_forward(q, k, v, decay_from_logits(np.full_like(k, -50.0)), bx, w, 4)
    o_zero, S_zero, _ = carve_forward(q, k, v, np.zeros_like(k), bx, w, 4)
    np.testing.assert_allclose(o_none, o_zero, atol=1e-18)
    np.testing.assert_allclose(S_none, S_zero, atol=1e-18)


# ---------------------------------------------------------------- gradients

GRAD_OF = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "bx": "dbx", "w": "dw", "U_down": "dU_down",
           "U_up": "dU_up", "state_in": "dstate_in", "mean_in": "dmean_in"}


def fd_gradients(args, L, do, dSo, dmo, h=1e-6):
    """Central differences of J = <do, o> + <dSo, state_out> + <dmo, mean_out>
    with respect to every element of every input: the derivative of the
    forward pass itself, independent of the adjoint's formulas."""
    def J(a):
        o, S, m = carve_forward(a["q"], a["k"], a["v"], a["g"], a["bx"], a["w"], L, a["U_down"], a["U_up"],
                                state_in=a["state_in"], mean_in=a["mean_in"])
        return np.sum(o * do) + np.sum(S * dSo) + np.sum(m * dmo)
    out = {}
    for name in GRAD_OF:
        x = args[name]
        if x is None:
            continue
        fd = np.zeros_like(x)
        for i in np.ndindex(x.shape):
            a = dict(args)
            xp = x.copy(); xp[i] += h; a[name] = xp
            jp = J(a)
            xm = x.copy(); xm[i] -= h; a[name] = xm
            fd[i] = (jp - J(a)) / (2 * h)
        out[name] = fd
    return out


@pytest.mark.parametrize("T,L,rank", [(7, 3, 2), (6, 3, 0), (5, 8, 2), (9, 2, 1), (4, 1, 2)])
def test_backward_matches_finite_differences(T, L, rank):
    """Every gradient the oracle's adjoint returns (inputs, gates, projection
    factors, incoming state and mean) equals the finite-difference derivative
    of the pinned forward pass: whole and ragged last chunks, with and without
    a content projection, a single chunk (T < L) and L = 1."""
    rng = np.random.default_rng(100 * T + 10 * L + rank)
    B, H, dk, dv = 1, 2, 3, 2
    q, k, v, g, bx, w, Ud, Uu = rand_inputs(rng, B, T, H, dk, dv, rank=rank, ub_std=0.8)
    args = dict(q=q, k=k, v=v, g=g, bx=bx, w=w, U_down=Ud, U_up=Uu,
                state_in=rng.standard_normal((B, H, dv, dk)), mean_in=rng.standard_normal((B, H, dv)))
    do = rng.standard_normal((B, T, H, dv))
    dSo = rng.standard_normal((B, H, dv, dk))
    dmo = rng.standard_normal((B, H, dv))
    got = carve_backward(q, k, v, g, bx, w, L, do, Ud, Uu, args["state_in"], args["mean_in"], dSo, dmo)
    fd = fd_gradients(args, L, do, dSo, dmo)
    for name, ref in fd.items():
        x = got[GRAD_OF[name]]
        err = np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-12)
        assert err < 1e-7, f"{name}: relative error {err:.2e}"
    if rank == 0:
        assert got["dU_down"] is None and got["dU_up"] is None
    if T <= L and rank:
        # one chunk from a zero incoming mean: the gate never sees a content
        # signal, so the projection gets no gradient
        zero_mean = carve_backward(q, k, v, g, bx, w, L, do, Ud, Uu, args["state_in"], None, dSo, dmo)
        assert not zero_mean["dU_down"].any() and not zero_mean["dU_up"].any()


def test_backward_without_state_and_mean_gradients():
    """Absent dstate_out and dmean_out count as zeros: with rank 0 the incoming
    mean then gets no gradient, and doubling do doubles every gradient."""
    rng = np.random.default_rng(5)
    q, k, v, g, bx, w, _, _ = rand_inputs(rng, 2, 6, 1, 3, 2)
    do = rng.standard_normal((2, 6, 1, 2))
    a = carve_backward(q, k, v, g, bx, w, 4, do)
    b = carve_backward(q, k, v, g, bx, w, 4, 2 * do)
    assert not a["dmean_in"].any()
    for n in ("dq", "dk", "dv", "dg", "dbx", "dw", "dstate_in"):
        np.testing.assert_allclose(b[n], 2 * a[n], rtol=1e-13, atol=1e-15)


def test_backward_empty_sequence_passes_gradients_through():
    rng = np.random.default_rng(6)
    B, H, dk, dv = 2, 1, 3, 2
    z = np.zeros((B, 0, H, dk))
    dSo, dmo = rng.standard_normal((B, H, dv, dk)), rng.standard_normal((B, H, dv))
    got = carve_backward(z, z, np.zeros((B, 0, H, dv)), z, z, np.zeros((B, 0, H)), 4,
                         np.zeros((B, 0, H, dv)), dstate_out=dSo, dmean_out=dmo)
    np.testing.assert_array_equal(got["dstate_in"], dSo)
    np.testing.assert_array_equal(got["dmean_in"], dmo)


# ---------------------------------------------------------------- q, k normalisation

def test_l2_normalize_closed_forms():
    """Unit norm per token; a positive scale of a token changes nothing; a
    vector along an axis maps to that axis; the zero vector stays zero."""
    rng = np.random.default_rng(21)
    x = rng.standard_normal((2, 5, 3, 6))
    y = l2_normalize(x)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), 1.0, rtol=1e-14)
    c = rng.uniform(0.01, 50.0, size=(2, 5, 3, 1))
    np.testing.assert_allclose(l2_normalize(c * x), y, rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(l2_normalize(np.array([0.0, -3.0, 0.0])), np.array([0.0, -1.0, 0.0]))
    np.testing.assert_array_equal(l2_normalize(np.zeros(4)), np.zeros(4))


def test_l2_normalize_backward_matches_finite_differences():
    """The chain rule through the normalisation equals central differences of
    <dy, l2_normalize(x)>, and it has no radial part: <x, dx> = 0 (a scale of
    x does not change the output)."""
    rng = np.random.default_rng(22)
    x = rng.standard_normal((3, 7))
    dy = rng.standard_normal((3, 7))
    got = l2_normalize_backward(x, dy)
    h, fd = 1e-6, np.zeros_like(x)
    for i in np.ndindex(x.shape):
        xp, xm = x.copy(), x.copy()
        xp[i] += h
        xm[i] -= h
        fd[i] = (np.sum(dy * l2_normalize(xp)) - np.sum(dy * l2_normalize(xm))) / (2 * h)
    np.testing.assert_allclose(got, fd, rtol=0, atol=1e-8)
    np.testing.assert_allclose(np.sum(got * x, axis=-1), 0.0, atol=1e-12)


def test_normalised_layer_is_scale_invariant_and_its_gradients_compose():
    """The layer on normalised q, k does not see a per-token scale of q or k,
    and the composed backward (the layer's gradients of q, k taken through the
    normalisation) equals central differences of the composed forward."""
    rng = np.random.default_rng(23)
    B, T, H, dk, dv, L = 1, 6, 2, 3, 2, 3
    q, k, v, g, bx, w, Ud, Uu = rand_inputs(rng, B, T, H, dk, dv, rank=2, ub_std=0.8)
    q = q * rng.uniform(0.2, 5.0, size=(B, T, H, 1))        # raw, not unit-norm
    k = k * rng.uniform(0.2, 5.0, size=(B, T, H, 1))
    fwd = lambda qq, kk: carve_forward(l2_normalize(qq), l2_normalize(kk), v, g, bx, w, L, Ud, Uu)
    o1, S1, m1 = fwd(q, k)
    o2, S2, m2 = fwd(3.0 * q, 0.5 * k)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(S2, S1, rtol=1e-12, atol=1e-14)
    do = rng.standard_normal((B, T, H, dv))
    gr = carve_backward(l2_normalize(q), l2_normalize(k), v, g, bx, w, L, do, Ud, Uu)
    dq = l2_normalize_backward(q, gr["dq"])
    dk_ = l2_normalize_backward(k, gr["dk"])
    J = lambda qq, kk: np.sum(fwd(qq, kk)[0] * do)
    h = 1e-6
    for x, got, which in ((q, dq, 0), (k, dk_, 1)):
        fd = np.zeros_like(x)
        for i in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[i] += h
            xm[i] -= h
            fd[i] = ((J(xp, k) - J(xm, k)) if which == 0 else (J(q, xp) - J(q, xm))) / (2 * h)
        np.testing.assert_allclose(got, fd, rtol=0, atol=1e-7 * max(1.0, np.abs(fd).max()))


def test_detached_mean_gradients_are_those_of_the_frozen_gate_layer():
    """With detach_mean, the gradients equal central differences of the layer
    whose gate means are frozen at their values (stepped with carve_step, the
    mean of each chunk replaced by the original run's): the projection still
    gets its gradient, mean_in gets none, and they differ from the full
    gradients."""
    rng = np.random.default_rng(31)
    B, T, H, dk, dv, L, r = 1, 7, 2, 3, 2, 3, 2
    q, k, v, g, bx, w, Ud, Uu = rand_inputs(rng, B, T, H, dk, dv, rank=r, ub_std=0.8)
    S_in = rng.standard_normal((B, H, dv, dk))
    m_in = rng.standard_normal((B, H, dv))
    do = rng.standard_normal((B, T, H, dv))
    # the gate means of the original run: mean_in, then each whole chunk's mean
    o0, _, _ = carve_forward(q, k, v, g, bx, w, L, Ud, Uu, state_in=S_in, mean_in=m_in)
    means = [m_in] + [o0[:, c * L:(c + 1) * L].mean(axis=1) for c in range((T - 1) // L)]

    def J(a):
        S, acc = S_in.copy(), np.zeros((B, H, dv))
        total = 0.0
        for t in range(T):
            o, S, _, acc = carve_step(S, means[t // L], acc, t % L, a["q"][:, t], a["k"][:, t], v[:, t], a["g"][:, t],
                                      a["bx"][:, t], w[:, t], L, a["U_down"], a["U_up"])
            total += np.sum(o * do[:, t])
        return total
    args = dict(q=q, k=k, g=g, bx=bx, U_down=Ud, U_up=Uu)
    got = carve_backward(q, k, v, g, bx, w, L, do, Ud, Uu, S_in, m_in, detach_mean=True)
    full = carve_backward(q, k, v, g, bx, w, L, do, Ud, Uu, S_in, m_in)
    h = 1e-6
    for name, gname in (("q", "dq"), ("k", "dk"), ("g", "dg"), ("bx", "dbx"), ("U_down", "dU_down"),
                        ("U_up", "dU_up")):
        x = args[name]
        fd = np.zeros_like(x)
        for i in np.ndindex(x.shape):
            a = dict(args)
            xp = x.copy(); xp[i] += h; a[name] = xp
            jp = J(a)
            xm = x.copy(); xm[i] -= h; a[name] = xm
            fd[i] = (jp - J(a)) / (2 * h)
        err = np.abs(got[gname] - fd).max() / max(np.abs(fd).max(), 1e-12)
        assert err < 1e-7, f"{name}: {err:.2e}"
    assert not got["dmean_in"].any()
    assert np.abs(full["dq"] - got["dq"]).max() > 1e-3       # the mean path does carry gradient
