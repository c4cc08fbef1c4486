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
"""
from __future__ import annotations

import numpy as np

__all__ = ["sigmoid", "decay_from_logits", "carve_forward", "carve_step", "content_gate_bias"]


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
