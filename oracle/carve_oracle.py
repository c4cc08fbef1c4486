"""Float64 CPU oracle for the CARVE layer's forward pass.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or run
this module: only the test suite, the smoke check and the benchmark's CPU
baseline leg use it. It shares no code with the HIP library.

The layer is defined token by token; the WY chunk solver is a way to reach the
same numbers (the chunkability theorem, Theorem 11 in §3 of the gist.science
technical summaries). So the oracle is the plain token recurrence in float64,
vectorised only across independent (batch, head) pairs.

Sources (the five pages about arXiv 2606.27229, "CARVE: Content-Aware
Recurrent with Value Efficiency for Chunk-Parallel Linear Attention"):
  [S1] gist.science technical summary (German and Dutch editions), §1
       "Problemstellung": per head the memory is a matrix S_t of shape
       d_v x d_k.
  [S2] same, §2 "Methodik": every gate acts on the key axis only.
  [S3] same, §2.1 "Content-Aware Erase via Output Reuse": the readout is
       o_t = S_{t-1} q_t; the chunk mean m_c = (1/L) sum of o_t over the chunk;
       the erase gate is sigmoid(b_x + U_b m); U_b is low-rank and starts at
       zero; the signal lags by one chunk.
  [S4] same, §2.2 "Scalar Value Write Gate": one scalar w per head and token,
       broadcast over all value channels.
  [S5] same, §2.3 "Key-Axis Decay und Fusion": exponential decay on the key
       axis only.
  [S5'] same, §2.3: the decay activation may be applied inside the kernel
       ("gate-in-kernel"), so the activated tensor is never stored.
  [S6] same, closing "Limitations" paragraph: sequences shorter than two
       chunks receive no content signal.
  [S7] aisea.builders paper card, "Key figure": the chunk mean of the previous
       chunk's outputs goes through zero-initialised low-rank projections.

Readings where the pages leave a step open (each listed in the design notes):
  R1  The erase vector b scales the retrieval key: the transition is
      S <- S D (I - (b*k) k^T) + w v k^T. (The pages give no update equation;
      this is the key-axis-only form that keeps one triangular system per
      chunk.)
  R2  Decay is applied first, then erase acts on the decayed state.
  R3  The gate of chunk c uses m_{c-1}; m_{-1} is mean_in (default zero).
  R4  U_b = U_up @ U_down per head, U_down [r, d_v], U_up [d_k, r].
  R5  No 1/sqrt(d_k) scale on q.
  R6  T need not be a multiple of L: the last chunk may be partial, and its
      mean is taken over the tokens it holds (it can only reach mean_out).
  R9  The decay activation (not named on the pages) is g = -softplus(a) of a
      raw decay logit a: it maps every real a to a log-decay below zero, so
      exp(g) = sigmoid(-a) lies in (0, 1).
  R10 Gradients (the pages train the layer but give no backward pass) are
      the exact derivatives of the forward pass as defined here, through every
      path it has: the stale chunk mean m_{c-1} passes gradient back to the
      previous chunk's outputs and to mean_in, and U_down, U_up receive theirs
      through the gate.
  R11 In-kernel normalisation of q and k (the workload recipes L2-normalise
      them per token) is q / max(|q|, 1e-12) over d_k for each (batch, token,
      head), applied before anything else reads them.
"""
from __future__ import annotations

import numpy as np

__all__ = ["sigmoid", "decay_from_logits", "l2_normalize", "l2_normalize_backward", "carve_forward",
           "carve_step", "carve_backward", "content_gate_bias"]

NORM_EPS = 1e-12


def sigmoid(x: np.ndarray) -> np.ndarray:
    """Logistic function, written so no intermediate overflows for large |x|."""
    x = np.asarray(x, dtype=np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def decay_from_logits(a: np.ndarray) -> np.ndarray:
    """Log-decay g = -softplus(a) = -log(1 + e^a) from raw decay logits a, in
    float64 ([S5], [S5'], reading R9). Evaluated as -(max(a, 0) + log1p(e^{-|a|}))
    so no intermediate overflows and tiny decays keep their relative accuracy."""
    a = np.asarray(a, dtype=np.float64)
    return -(np.maximum(a, 0.0) + np.log1p(np.exp(-np.abs(a))))


def l2_normalize(x: np.ndarray) -> np.ndarray:
    """x / max(|x|, 1e-12) over the last axis, in float64 (reading R11)."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / np.maximum(n, NORM_EPS)


def l2_normalize_backward(x: np.ndarray, dxhat: np.ndarray) -> np.ndarray:
    """Gradient with respect to x of l2_normalize(x), given the gradient of
    its output: (dxhat - xhat <xhat, dxhat>) / |x| where |x| > 1e-12 (the
    projection that removes the radial part), dxhat / 1e-12 below it."""
    x = np.asarray(x, dtype=np.float64)
    dxhat = np.asarray(dxhat, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    xhat = x / np.maximum(n, NORM_EPS)
    radial = xhat * np.sum(xhat * dxhat, axis=-1, keepdims=True)
    return np.where(n > NORM_EPS, (dxhat - radial) / np.maximum(n, NORM_EPS), dxhat / NORM_EPS)


def content_gate_bias(m: np.ndarray, U_down: np.ndarray | None,
                      U_up: np.ndarray | None) -> np.ndarray:
    """z = U_b m with U_b = U_up U_down, per head ([S3], [S7], reading R4).

    m: [B, H, d_v] -> z: [B, H, d_k]. Without a projection z is zero.
    """
    B, H, _ = m.shape
    if U_down is None or U_up is None or U_down.shape[1] == 0:
        return None
    y = np.einsum("hre,bhe->bhr", U_down, m)        # U_down m: [B, H, r]
    return np.einsum("hdr,bhr->bhd", U_up, y)       # U_up (U_down m): [B, H, d_k]


def _token(S, q, k, v, g, bx, w, z):
    """One token of the recurrence for every (batch, head), in float64.

    S [B, H, d_v, d_k]; q, k, g, bx [B, H, d_k]; v [B, H, d_v]; w [B, H];
    z [B, H, d_k] or None. Returns (o_t, S_t):
      b   = sigmoid(bx + z)                       [S3], key axis only [S2]
      o_t = S q                                   readout before the update [S3]
      S   = S diag(exp(g))                        key-axis decay [S5], R2
      S   = S - (S (b*k)) k^T + w v k^T           erase then write [S4], R1
    """
    b = sigmoid(bx if z is None else bx + z)                     # [B, H, dk]
    ot = np.einsum("bhed,bhd->bhe", S, q)                        # o_t = S_{t-1} q_t
    S = S * np.exp(g)[:, :, None, :]                             # decay columns (key axis)
    r = np.einsum("bhed,bhd->bhe", S, b * k)                     # erase-weighted retrieval
    delta = w[:, :, None] * v - r                                # [B, H, dv]
    S = S + delta[:, :, :, None] * k[:, :, None, :]
    return ot, S


def carve_forward(q, k, v, g, bx, w, L, U_down=None, U_up=None,
                  state_in=None, mean_in=None):
    """Token-by-token CARVE forward pass in float64.

    Arguments (any float dtype; upcast to float64):
      q, k, g, bx : [B, T, H, d_k]   query, key, log-decay (<= 0), erase logit
      v           : [B, T, H, d_v]   value
      w           : [B, T, H]        scalar write gate
      L           : chunk length of the content signal (T need not be a multiple)
      U_down      : [H, r, d_v] or None;  U_up: [H, d_k, r] or None
      state_in    : [B, H, d_v, d_k] or None (zeros)
      mean_in     : [B, H, d_v] or None (zeros): the mean that feeds chunk 0
    Returns (o [B, T, H, d_v], state_out [B, H, d_v, d_k], mean_out [B, H, d_v]).

    Per chunk c (reading R3): z = U_b m_{c-1}; then for each token t
      b   = sigmoid(bx_t + z)                     [S3], key axis only [S2]
      o_t = S q_t                                 readout before the update [S3]
      S   = S diag(exp(g_t))                      key-axis decay [S5], R2
      S   = S - (S (b*k_t)) k_t^T + w_t v_t k_t^T erase then write [S4], R1
    and m_c is the mean of o_t over the chunk [S3].
    """
    f = lambda x: np.asarray(x, dtype=np.float64)
    q, k, v, g, bx, w = map(f, (q, k, v, g, bx, w))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if L < 1:
        raise ValueError("L must be positive")
    Ud = None if U_down is None else f(U_down)
    Uu = None if U_up is None else f(U_up)

    S = np.zeros((B, H, dv, dk)) if state_in is None else f(state_in).copy()
    m = np.zeros((B, H, dv)) if mean_in is None else f(mean_in).copy()
    o = np.empty((B, T, H, dv))

    for c in range((T + L - 1) // L):
        z = content_gate_bias(m, Ud, Uu)
        acc = np.zeros((B, H, dv))
        t_end = min(T, (c + 1) * L)                              # reading R6
        for t in range(c * L, t_end):
            ot, S = _token(S, q[:, t], k[:, t], v[:, t], g[:, t], bx[:, t], w[:, t], z)
            o[:, t] = ot
            acc += ot
        m = acc / (t_end - c * L)
    return o, S, m


def carve_step(state, mean_prev, chunk_acc, pos, q, k, v, g, bx, w, L,
               U_down=None, U_up=None):
    """One decode step: token `pos` (0 <= pos < L) of its chunk, for every
    (batch, head), in float64.

    Arguments (any float dtype; upcast to float64):
      state      : [B, H, d_v, d_k]  the state before this token
      mean_prev  : [B, H, d_v]       mean of the previous chunk's outputs (R3)
      chunk_acc  : [B, H, d_v]       sum of this chunk's outputs before this token
      q, k, g, bx: [B, H, d_k];  v: [B, H, d_v];  w: [B, H]
      U_down, U_up as in carve_forward.
    Returns (o [B, H, d_v], state, mean_prev, chunk_acc) after the token. At
    the chunk's last position (pos == L - 1) the chunk's mean replaces
    mean_prev and the sum restarts from zero. Stepping tokens 0 .. T-1 with
    pos = t mod L from (state_in, mean_in, 0) reproduces carve_forward's o and
    state; after a whole chunk, mean_prev is its m_c.
    """
    f = lambda x: np.asarray(x, dtype=np.float64)
    if not 0 <= pos < L:
        raise ValueError("pos must lie in [0, L)")
    Ud = None if U_down is None else f(U_down)
    Uu = None if U_up is None else f(U_up)
    m = f(mean_prev)
    z = content_gate_bias(m, Ud, Uu)                              # gate of this chunk (R3)
    ot, S = _token(f(state), f(q), f(k), f(v), f(g), f(bx), f(w), z)
    acc = f(chunk_acc) + ot
    if pos == L - 1:
        m, acc = acc / L, np.zeros_like(acc)
    return ot, S, m, acc


def carve_backward(q, k, v, g, bx, w, L, do, U_down=None, U_up=None,
                   state_in=None, mean_in=None, dstate_out=None, dmean_out=None, detach_mean=False):
    """Gradients of carve_forward in float64 (reading R10), by the adjoint of
    the token recurrence taken backwards through the sequence.

    Arguments as for carve_forward, plus the gradients of a scalar loss with
    respect to its outputs: do [B, T, H, d_v], and optionally dstate_out
    [B, H, d_v, d_k] and dmean_out [B, H, d_v] (zeros when None).
    Returns a dict with dq, dk, dg, dbx [B, T, H, d_k], dv [B, T, H, d_v],
    dw [B, T, H], dU_down [H, r, d_v] and dU_up [H, d_k, r] (None without a
    projection), dstate_in [B, H, d_v, d_k] and dmean_in [B, H, d_v].

    With S' = S diag(e^g), r = S' (b*k), delta = w v - r and S_t = S' + delta k^T,
    the adjoint of one token, given dS (of S_t) and the token's total output
    gradient do_t, is
      d delta = dS k          dk  = dS^T delta + (S'^T dr) * b,   dr = -d delta
      dv = w d delta          dw  = <d delta, v>
      dS' = dS + dr (b*k)^T   dg  = sum over rows of dS' * S'
      db  = (S'^T dr) * k     dbx = db * b (1 - b)
      dq  = S_{t-1}^T do_t    dS_{t-1} = dS' diag(e^g) + do_t q^T.
    The output gradient of token t in chunk c adds dm_c / n_c, where n_c is
    the chunk's token count and dm_c collects dmean_out (last chunk) and the
    gradient that chunk c + 1's gate sends back through z = U_up (U_down m_c).
    With detach_mean the gate means are taken as constants: the gates still
    pass gradient to U_down and U_up, but none reaches earlier outputs or
    mean_in through them (the other reading of R10).
    """
    f = lambda x: np.asarray(x, dtype=np.float64)
    q, k, v, g, bx, w, do = map(f, (q, k, v, g, bx, w, do))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if L < 1:
        raise ValueError("L must be positive")
    Ud = None if U_down is None else f(U_down)
    Uu = None if U_up is None else f(U_up)
    content = Ud is not None and Uu is not None and Ud.shape[1] > 0

    # forward pass, keeping each token's state before it and each chunk's gate input
    S = np.zeros((B, H, dv, dk)) if state_in is None else f(state_in).copy()
    m = np.zeros((B, H, dv)) if mean_in is None else f(mean_in).copy()
    nc = (T + L - 1) // L
    S_before = np.empty((B, T, H, dv, dk))
    b_all = np.empty((B, T, H, dk))
    gate_mean = []                                   # m_{c-1} for each chunk c
    for c in range(nc):
        gate_mean.append(m)
        z = content_gate_bias(m, Ud, Uu)
        acc = np.zeros((B, H, dv))
        t_end = min(T, (c + 1) * L)
        for t in range(c * L, t_end):
            S_before[:, t] = S
            b_all[:, t] = sigmoid(bx[:, t] if z is None else bx[:, t] + z)
            ot, S = _token(S, q[:, t], k[:, t], v[:, t], g[:, t], bx[:, t], w[:, t], z)
            acc += ot
        m = acc / (t_end - c * L)

    dS = np.zeros((B, H, dv, dk)) if dstate_out is None else f(dstate_out).copy()
    dmo = np.zeros((B, H, dv)) if dmean_out is None else f(dmean_out)
    grads = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("dbx", bx),
                                               ("dw", w))}
    dUd = None if Ud is None else np.zeros_like(Ud)
    dUu = None if Uu is None else np.zeros_like(Uu)
    dm = np.zeros((B, H, dv))                        # gradient of m_c from chunk c + 1's gate
    for c in reversed(range(nc)):
        t0, t1 = c * L, min(T, (c + 1) * L)
        dmc = dm + (dmo if c == nc - 1 else 0.0)
        dz = np.zeros((B, H, dk))
        for t in reversed(range(t0, t1)):
            Sp, b = S_before[:, t], b_all[:, t]
            qt, kt, vt, gt, wt = q[:, t], k[:, t], v[:, t], g[:, t], w[:, t]
            dec = np.exp(gt)
            Sd = Sp * dec[:, :, None, :]                                  # S'
            bk = b * kt
            delta = wt[:, :, None] * vt - np.einsum("bhed,bhd->bhe", Sd, bk)
            dot = do[:, t] + dmc / (t1 - t0)
            ddelta = np.einsum("bhed,bhd->bhe", dS, kt)
            dr = -ddelta
            sdr = np.einsum("bhed,bhe->bhd", Sd, dr)                       # S'^T dr
            dSd = dS + dr[:, :, :, None] * bk[:, :, None, :]
            grads["dk"][:, t] = np.einsum("bhed,bhe->bhd", dS, delta) + sdr * b
            grads["dv"][:, t] = wt[:, :, None] * ddelta
            grads["dw"][:, t] = np.sum(ddelta * vt, axis=-1)
            grads["dg"][:, t] = np.sum(dSd * Sd, axis=-2)
            grads["dbx"][:, t] = sdr * kt * b * (1.0 - b)
            grads["dq"][:, t] = np.einsum("bhed,bhe->bhd", Sp, dot)
            dz += grads["dbx"][:, t]
            dS = dSd * dec[:, :, None, :] + dot[:, :, :, None] * qt[:, :, None, :]
        if content:                                   # z = U_up y, y = U_down m_{c-1}
            mp = gate_mean[c]
            y = np.einsum("hre,bhe->bhr", Ud, mp)
            dUu += np.einsum("bhd,bhr->hdr", dz, y)
            dy = np.einsum("hdr,bhd->bhr", Uu, dz)
            dUd += np.einsum("bhr,bhe->hre", dy, mp)
            dm = np.zeros((B, H, dv)) if detach_mean else np.einsum("hre,bhr->bhe", Ud, dy)
        else:
            dm = np.zeros((B, H, dv))
    grads.update(dU_down=dUd, dU_up=dUu, dstate_in=dS, dmean_in=dm if nc else dmo.copy())
    return grads
