"""fp64 CPU oracle: four gate variants, three evaluation forms each, and two decode steps.

TEST INFRASTRUCTURE ONLY (see the package docstring): plain numpy in float64,
shared with nothing on the GPU side.

Conventions, all fixed by "Scrivere meglio nella memoria: gate e delta rule",
section "Superiore" of the introduction and section "Dimenticare: i gate":

* the memory is ``S`` of shape ``[d_v, d_k]``, written as a sum of outer
  products ``v k^T`` (rows = value channels, columns = key channels);
* it is read *after* the write of token t: ``o_t = S_t q_t`` (the page defines
  ``S_t`` as the memory after the first t tokens; the worked example of the
  RetNet page starts its running totals at the first score, 6);
* gates and the delta transition multiply ``S`` from the right, so each key
  channel (column) decays at its own rate.

Array layout (the same one the C ABI uses): ``q, k`` are ``[B, H, T, d_k]``,
``v`` and the output ``o`` are ``[B, H, T, d_v]``, states are
``[B, H, d_v, d_k]``. Every function returns ``(o, S_T)`` where ``S_T`` is the
memory after the last token (equal to ``s0`` - or zeros - when T = 0).

Variants (the transition table of section "Le ricorrenze come regressione
online" of the same page):

* retention (RetNet row, fixed per-head decay): ``S_t = g_h S_{t-1} + v_t k_t^T``
  with ``g_h = exp(log_gamma[h])``;
* scalar data-dependent decay (the Mamba-2 half of the "Mamba-2 / RetNet" row):
  ``S_t = alpha_t S_{t-1} + v_t k_t^T``, one ``alpha_t = exp(log_alpha[..., t])``
  per token and head;
* GLA (diagonal data-dependent gate, one per key channel):
  ``S_t = S_{t-1} Diag(alpha_t) + v_t k_t^T``, ``alpha_t = exp(log_alpha[..., t, :])``;
* gated delta rule (Gated DeltaNet row):
  ``S_t = S_{t-1} [alpha_t (I - beta_t k_t k_t^T)] + beta_t v_t k_t^T`` with a
  scalar ``alpha_t = exp(log_alpha[..., t])`` and write strength ``beta_t``.

Forms (RetNet page, section "RetNet: la retention e le sue tre forme", Fig.
16.5): the recurrent form is the definition; the parallel ("quadratic") form
and the chunkwise form must give the same numbers up to rounding.

Also here: the reverse-mode gradients of the fixed and scalar decays, and
variational linear attention (VLA summary page, "Riepilogo Tecnico: Attenzione
Lineare Variazionale (VLA)", section 2.3) in its recurrent form, which returns
``(o, S_T, A_T, n_T)`` with the inverse penalty ``A`` and the readout's denominator
vector ``n`` beside the memory.
"""

import numpy as np

__all__ = [
    "retention_recurrent",
    "retention_quadratic",
    "retention_chunkwise",
    "scalar_recurrent",
    "scalar_quadratic",
    "scalar_chunkwise",
    "gla_recurrent",
    "gla_quadratic",
    "gla_chunkwise",
    "gdelta_recurrent",
    "gdelta_quadratic",
    "gdelta_chunkwise",
    "decode_step",
    "gdelta_decode_step",
    "silu_l2",
    "rms_norm",
    "layer_norm",
    "scalar_backward",
    "gdelta_backward",
    "retention_backward",
    "forward_substitution",
    "gla_backward",
    "vla_recurrent",
    "vla_decode_step",
    "elu1",
]


# --------------------------------------------------------------------------- helpers

def _f64(*arrays):
    return [None if a is None else np.asarray(a, dtype=np.float64) for a in arrays]


def _init_state(q, v, s0):
    """Zero memory (pure accumulation starts empty) unless a state is handed over."""
    lead = q.shape[:-2]
    dk, dv = q.shape[-1], v.shape[-1]
    if s0 is None:
        return np.zeros(lead + (dv, dk))
    return np.array(s0, dtype=np.float64, copy=True)


def _outer(v_t, k_t):
    """The write ``v k^T`` of one token, batched over the leading axes."""
    return v_t[..., :, None] * k_t[..., None, :]


def _read(S, q_t):
    """The readout ``S q`` of one token, batched over the leading axes."""
    return np.einsum("...mc,...c->...m", S, q_t)


def forward_substitution(L, R):
    """Solve ``(I + L) X = R`` for X, with ``L`` strictly lower triangular.

    Textbook forward substitution, one row at a time: every equation uses only
    the solutions of the previous ones ("Scrivere meglio nella memoria",
    section "Correggere: la delta rule", the triangular system of the WY
    representation). ``L`` is ``[..., n, n]``, ``R`` is ``[..., n, m]``.
    """
    L = np.asarray(L, dtype=np.float64)
    X = np.array(R, dtype=np.float64, copy=True)
    n = L.shape[-1]
    for i in range(n):
        if i:
            X[..., i, :] -= np.einsum("...j,...jm->...m", L[..., i, :i], X[..., :i, :])
    return X


# --------------------------------------------------------------------------- retention

def _gamma_per_head(log_gamma, lead):
    """Broadcast the per-head decay ``[H]`` against the leading axes ``[B, H]``."""
    lg = np.asarray(log_gamma, dtype=np.float64)
    return np.broadcast_to(lg, lead)


def retention_recurrent(q, k, v, log_gamma, s0=None):
    """Recurrent form (the definition): ``S_t = g S_{t-1} + v_t k_t^T``, ``o_t = S_t q_t``.

    "Scrivere meglio nella memoria", section "Dimenticare: i gate", scalar
    decay equation with the RetNet choice alpha_t = gamma fixed per head; the
    RetNet page, section on retention, recurrent form (cost O(d^2) per token).
    """
    q, k, v = _f64(q, k, v)
    S = _init_state(q, v, s0)
    g = np.exp(_gamma_per_head(log_gamma, q.shape[:-2]))[..., None, None]
    T = q.shape[-2]
    o = np.zeros(v.shape)
    for t in range(T):
        S = g * S + _outer(v[..., t, :], k[..., t, :])
        o[..., t, :] = _read(S, q[..., t, :])
    return o, S


def retention_quadratic(q, k, v, log_gamma, s0=None):
    """Parallel form ``O = (Q K^T (.) D) V`` with ``D_ij = g^(i-j)`` for ``i >= j`` and 0 above.

    The RetNet page, section on retention, parallel (training) form: D is a
    causal mask whose entry for the pair (i, j) is g^(i-j). A handed-over
    state adds its decayed readout ``g^(i+1) S_0 q_i`` (unrolling the
    recurrence from ``S_0``); the final memory is the unrolled sum
    ``S_T = g^T S_0 + sum_j g^(T-1-j) v_j k_j^T``.
    """
    q, k, v = _f64(q, k, v)
    lead = q.shape[:-2]
    T = q.shape[-2]
    lg = _gamma_per_head(log_gamma, lead)[..., None, None]
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    dist = (i - j).astype(np.float64)
    D = np.where(i >= j, np.exp(lg * np.maximum(dist, 0.0)), 0.0)
    scores = np.einsum("...ic,...jc->...ij", q, k)
    o = np.einsum("...ij,...jm->...im", scores * D, v)
    S0 = _init_state(q, v, s0)
    steps = np.arange(1, T + 1, dtype=np.float64)
    lg1 = lg[..., 0, 0]
    o += np.exp(lg1[..., None] * steps)[..., :, None] * np.einsum("...mc,...ic->...im", S0, q)
    w_last = np.exp(lg1[..., None] * (T - 1 - np.arange(T, dtype=np.float64)))
    S = np.exp(lg1 * T)[..., None, None] * S0 + np.einsum("...j,...jm,...jc->...mc", w_last, v, k)
    return o, S


def retention_chunkwise(q, k, v, log_gamma, chunk, s0=None):
    """Chunkwise form: the parallel form inside each block of ``chunk`` tokens, the
    recurrent form from one block to the next (the RetNet page, section on
    retention, chunkwise form; Fig. 16.5 right panel). The last block may be
    shorter (the worked example uses blocks of two over three scores).

    Per block of n tokens with incoming memory ``S_in`` and local index i, j:
    ``o_i = sum_{j<=i} g^(i-j) (q_i . k_j) v_j + g^(i+1) S_in q_i`` and
    ``S_out = g^n S_in + sum_j g^(n-1-j) v_j k_j^T``.
    """
    q, k, v = _f64(q, k, v)
    lead = q.shape[:-2]
    T = q.shape[-2]
    lg = _gamma_per_head(log_gamma, lead)
    S = _init_state(q, v, s0)
    o = np.zeros(v.shape)
    for t0 in range(0, T, chunk):
        n = min(chunk, T - t0)
        Q, K, V = q[..., t0:t0 + n, :], k[..., t0:t0 + n, :], v[..., t0:t0 + n, :]
        i = np.arange(n)[:, None]
        j = np.arange(n)[None, :]
        D = np.where(i >= j, np.exp(lg[..., None, None] * np.maximum(i - j, 0)), 0.0)
        P = np.einsum("...ic,...jc->...ij", Q, K) * D
        inner = np.exp(lg[..., None] * np.arange(1, n + 1))  # g^(i+1)
        o[..., t0:t0 + n, :] = (np.einsum("...ij,...jm->...im", P, V)
                                + inner[..., :, None] * np.einsum("...mc,...ic->...im", S, Q))
        w = np.exp(lg[..., None] * (n - 1 - np.arange(n)))    # g^(n-1-j)
        S = (np.exp(lg * n)[..., None, None] * S
             + np.einsum("...j,...jm,...jc->...mc", w, V, K))
    return o, S


# --------------------------------------------------------------------------- scalar decay

def scalar_recurrent(q, k, v, log_alpha, s0=None):
    """Recurrent form (the definition): ``S_t = alpha_t S_{t-1} + v_t k_t^T``, ``o_t = S_t q_t``.

    "Scrivere meglio nella memoria", section "Dimenticare: i gate", scalar
    decay equation with the gate produced from the input at every step (the
    Mamba-2 reading of the same equation; one number per token and head).
    ``log_alpha`` is ``[B, H, T]``.
    """
    q, k, v, la = _f64(q, k, v, log_alpha)
    S = _init_state(q, v, s0)
    T = q.shape[-2]
    o = np.zeros(v.shape)
    for t in range(T):
        S = np.exp(la[..., t])[..., None, None] * S + _outer(v[..., t, :], k[..., t, :])
        o[..., t, :] = _read(S, q[..., t, :])
    return o, S


def scalar_quadratic(q, k, v, log_alpha, s0=None):
    """Parallel form, the recurrence unrolled over the whole sequence.

    Same section: what is written at step j reaches step t weighted by the
    product of the gates of steps j+1 .. t. With ``G_t = sum_{r<=t} log alpha_r``
    that weight is ``exp(G_t - G_j)``, so
    ``o_t = sum_{j<=t} exp(G_t - G_j) (q_t . k_j) v_j + exp(G_t) S_0 q_t`` and
    ``S_T = exp(G_{T-1}) S_0 + sum_j exp(G_{T-1} - G_j) v_j k_j^T``.
    """
    q, k, v, la = _f64(q, k, v, log_alpha)
    T = q.shape[-2]
    G = np.cumsum(la, axis=-1)                                      # [..., T]
    causal = np.arange(T)[:, None] >= np.arange(T)[None, :]
    diff = G[..., :, None] - G[..., None, :]
    D = np.where(causal, np.exp(np.where(causal, diff, 0.0)), 0.0)
    scores = np.einsum("...ic,...jc->...ij", q, k)
    o = np.einsum("...ij,...jm->...im", scores * D, v)
    S0 = _init_state(q, v, s0)
    o += np.exp(G)[..., :, None] * np.einsum("...mc,...ic->...im", S0, q)
    if T == 0:
        return o, S0
    last = G[..., -1]
    S = np.exp(last)[..., None, None] * S0 + np.einsum(
        "...j,...jm,...jc->...mc", np.exp(last[..., None] - G), v, k)
    return o, S


def scalar_chunkwise(q, k, v, log_alpha, chunk, s0=None):
    """Chunkwise form: the parallel form inside each block, the memory carried between
    blocks (the RetNet page, section on retention, chunkwise form, with the decay
    now read from the gates). With local inclusive cumulative log-gates ``G_i``:
    ``o_i = sum_{j<=i} exp(G_i - G_j) (q_i . k_j) v_j + exp(G_i) S_in q_i``,
    ``S_out = exp(G_{n-1}) S_in + sum_j exp(G_{n-1} - G_j) v_j k_j^T``.
    """
    q, k, v, la = _f64(q, k, v, log_alpha)
    T = q.shape[-2]
    S = _init_state(q, v, s0)
    o = np.zeros(v.shape)
    for t0 in range(0, T, chunk):
        n = min(chunk, T - t0)
        Q, K, V = q[..., t0:t0 + n, :], k[..., t0:t0 + n, :], v[..., t0:t0 + n, :]
        G = np.cumsum(la[..., t0:t0 + n], axis=-1)
        causal = np.arange(n)[:, None] >= np.arange(n)[None, :]
        diff = G[..., :, None] - G[..., None, :]
        D = np.where(causal, np.exp(np.where(causal, diff, 0.0)), 0.0)
        P = np.einsum("...ic,...jc->...ij", Q, K) * D
        o[..., t0:t0 + n, :] = (np.einsum("...ij,...jm->...im", P, V)
                                + np.exp(G)[..., :, None] * np.einsum("...mc,...ic->...im", S, Q))
        last = G[..., -1]
        S = (np.exp(last)[..., None, None] * S
             + np.einsum("...j,...jm,...jc->...mc", np.exp(last[..., None] - G), V, K))
    return o, S


# --------------------------------------------------------------------------- GLA

def gla_recurrent(q, k, v, log_alpha, s0=None):
    """Recurrent form (the definition): ``S_t = S_{t-1} Diag(alpha_t) + v_t k_t^T``.

    "Scrivere meglio nella memoria", section "Dimenticare: i gate", the
    diagonal-gate equation of Gated Linear Attention: one gate per key channel,
    multiplying from the right so that column c decays at rate alpha_{t,c}.
    """
    q, k, v, la = _f64(q, k, v, log_alpha)
    S = _init_state(q, v, s0)
    T = q.shape[-2]
    o = np.zeros(v.shape)
    for t in range(T):
        S = S * np.exp(la[..., t, :])[..., None, :] + _outer(v[..., t, :], k[..., t, :])
        o[..., t, :] = _read(S, q[..., t, :])
    return o, S


def gla_quadratic(q, k, v, log_alpha, s0=None):
    """Parallel form of GLA, the recurrence unrolled over the whole sequence.

    Unrolling the diagonal-gate recurrence ("Dimenticare: i gate": what is
    written at step j reaches step t weighted by the product of the gates in
    between) gives, per key channel c with ``B_t = sum_{r<=t} log alpha_r``:
    ``o_t = sum_{j<=t} [sum_c q_tc k_jc exp(B_tc - B_jc)] v_j + S_0 (q_t (.) exp(B_t))``
    and ``S_T = S_0 Diag(exp(B_{T-1})) + sum_j v_j (k_j (.) exp(B_{T-1} - B_j))^T``.
    O(T^2 d) memory and time: for small T only.
    """
    q, k, v, la = _f64(q, k, v, log_alpha)
    T = q.shape[-2]
    Bc = np.cumsum(la, axis=-2)                                   # [..., T, dk]
    diff = Bc[..., :, None, :] - Bc[..., None, :, :]              # [..., t, j, dk]
    causal = (np.arange(T)[:, None] >= np.arange(T)[None, :])[..., None]
    W = np.where(causal, np.exp(np.where(causal, diff, 0.0)), 0.0)
    P = np.einsum("...tc,...jc,...tjc->...tj", q, k, W)
    o = np.einsum("...tj,...jm->...tm", P, v)
    S0 = _init_state(q, v, s0)
    o += np.einsum("...mc,...tc->...tm", S0, q * np.exp(Bc))
    if T == 0:
        return o, S0
    last = Bc[..., -1, :]
    S = S0 * np.exp(last)[..., None, :] + np.einsum(
        "...jm,...jc->...mc", v, k * np.exp(last[..., None, :] - Bc))
    return o, S


def gla_chunkwise(q, k, v, log_alpha, chunk, s0=None):
    """Chunkwise GLA: parallel inside each block, the memory carried between blocks.

    With local inclusive cumulative log-gates ``b_i`` (restarting at each block)
    and the incoming memory ``S_in``:
    ``o_i = sum_{j<=i} [sum_c q_ic k_jc exp(b_ic - b_jc)] v_j + S_in (q_i (.) exp(b_i))``,
    ``S_out = S_in Diag(exp(b_{n-1})) + sum_j v_j (k_j (.) exp(b_{n-1} - b_j))^T``.
    Every exponent used is <= 0 when the gates are <= 1.
    """
    q, k, v, la = _f64(q, k, v, log_alpha)
    T = q.shape[-2]
    S = _init_state(q, v, s0)
    o = np.zeros(v.shape)
    for t0 in range(0, T, chunk):
        n = min(chunk, T - t0)
        Q, K, V = q[..., t0:t0 + n, :], k[..., t0:t0 + n, :], v[..., t0:t0 + n, :]
        b = np.cumsum(la[..., t0:t0 + n, :], axis=-2)
        diff = b[..., :, None, :] - b[..., None, :, :]
        causal = (np.arange(n)[:, None] >= np.arange(n)[None, :])[..., None]
        W = np.where(causal, np.exp(np.where(causal, diff, 0.0)), 0.0)
        P = np.einsum("...ic,...jc,...ijc->...ij", Q, K, W)
        o[..., t0:t0 + n, :] = (np.einsum("...ij,...jm->...im", P, V)
                                + np.einsum("...mc,...ic->...im", S, Q * np.exp(b)))
        last = b[..., -1, :]
        S = S * np.exp(last)[..., None, :] + np.einsum(
            "...jm,...jc->...mc", V, K * np.exp(last[..., None, :] - b))
    return o, S


# --------------------------------------------------------------------------- gated delta rule

def gdelta_recurrent(q, k, v, log_alpha, beta, s0=None):
    """Recurrent form (the definition) of Gated DeltaNet.

    "Scrivere meglio nella memoria", section "Unire oblio e correzione: Gated
    DeltaNet": ``S_t = S_{t-1} [alpha_t (I - beta_t k_t k_t^T)] + beta_t v_t k_t^T``.
    Written the way section "Correggere: la delta rule" reads it: first the
    memory fades, ``S' = alpha_t S_{t-1}``; then it is queried with the current
    key, ``v_bar = S' k_t``, and only the error is written:
    ``S_t = S' + beta_t (v_t - v_bar) k_t^T``.
    """
    q, k, v, la, be = _f64(q, k, v, log_alpha, beta)
    S = _init_state(q, v, s0)
    T = q.shape[-2]
    o = np.zeros(v.shape)
    for t in range(T):
        Sp = np.exp(la[..., t])[..., None, None] * S
        v_bar = _read(Sp, k[..., t, :])
        S = Sp + be[..., t][..., None, None] * _outer(v[..., t, :] - v_bar, k[..., t, :])
        o[..., t, :] = _read(S, q[..., t, :])
    return o, S


def _gdelta_block(Q, K, V, la, be, S):
    """One block of the gated delta rule in WY / pseudo-value form.

    Section "Correggere: la delta rule" writes the DeltaNet memory as a sum of
    outer products of pseudo-values, ``S_t = sum_{i<=t} u_i k_i^T`` with
    ``u_t = beta_t (v_t - sum_{i<t} u_i (k_i^T k_t))``: one triangular system per
    block, only the end-of-block memory passing on. Section "Unire oblio e
    correzione" says Gated DeltaNet extends the same representation; with the
    local cumulative log-decay ``G_i = sum_{r<=i} log alpha_r`` the extension is

      S_i = e^{G_i} S_in + sum_{j<=i} e^{G_i - G_j} u_j k_j^T,
      u_i = beta_i (v_i - e^{G_i} S_in k_i - sum_{j<i} e^{G_i - G_j} (k_j . k_i) u_j),

    i.e. ``(I + A) U = diag(beta) (V - diag(e^G) K S_in^T)`` with
    ``A = strictly_lower(diag(beta) (K K^T (.) Gamma))``, ``Gamma_ij = e^{G_i - G_j}``;
    then ``o_i = e^{G_i} S_in q_i + sum_{j<=i} Gamma_ij (q_i . k_j) u_j`` and
    ``S_out = e^{G_{n-1}} S_in + sum_j e^{G_{n-1} - G_j} u_j k_j^T``.
    """
    n = Q.shape[-2]
    G = np.cumsum(la, axis=-1)                                     # [..., n]
    idx = np.arange(n)
    lower_strict = idx[:, None] > idx[None, :]
    lower = idx[:, None] >= idx[None, :]
    gdiff = G[..., :, None] - G[..., None, :]
    Gamma = np.where(lower, np.exp(np.where(lower, gdiff, 0.0)), 0.0)
    KK = np.einsum("...ic,...jc->...ij", K, K)
    A = np.where(lower_strict, be[..., :, None] * KK * Gamma, 0.0)
    eG = np.exp(G)
    R = be[..., :, None] * (V - eG[..., :, None] * np.einsum("...mc,...ic->...im", S, K))
    U = forward_substitution(A, R)
    QK = np.einsum("...ic,...jc->...ij", Q, K)
    O = eG[..., :, None] * np.einsum("...mc,...ic->...im", S, Q) + np.einsum(
        "...ij,...jm->...im", QK * Gamma, U)
    w = np.exp(G[..., -1:] - G)                                    # e^{G_{n-1} - G_j}
    S_out = eG[..., -1][..., None, None] * S + np.einsum("...j,...jm,...jc->...mc", w, U, K)
    return O, S_out


def gdelta_quadratic(q, k, v, log_alpha, beta, s0=None):
    """Parallel form of the gated delta rule: the WY block taken over the whole sequence.

    One triangular system of size T (O(T^2 d)); for small T only.
    """
    q, k, v, la, be = _f64(q, k, v, log_alpha, beta)
    S = _init_state(q, v, s0)
    if q.shape[-2] == 0:
        return np.zeros(v.shape), S
    return _gdelta_block(q, k, v, la, be, S)


def gdelta_chunkwise(q, k, v, log_alpha, beta, chunk, s0=None):
    """Chunkwise gated delta rule: one WY block per ``chunk`` tokens, the end-of-block
    memory handed to the next block ("Correggere: la delta rule": only the
    memory at the end of a block passes to the following one)."""
    q, k, v, la, be = _f64(q, k, v, log_alpha, beta)
    T = q.shape[-2]
    S = _init_state(q, v, s0)
    o = np.zeros(v.shape)
    for t0 in range(0, T, chunk):
        sl = slice(t0, min(T, t0 + chunk))
        O, S = _gdelta_block(q[..., sl, :], k[..., sl, :], v[..., sl, :],
                             la[..., sl], be[..., sl], S)
        o[..., sl, :] = O
    return o, S


# --------------------------------------------------------------------------- decode

def decode_step(q, k, v, alpha, s):
    """One token of generation with a per-key-channel gate (GLA row; a scalar decay is
    the constant gate): ``S <- S Diag(alpha)``, ``S <- S + v k^T``, ``o = S q``.

    The RetNet page, section on retention, recurrent form: generation costs the
    same two gestures for every token, at constant memory. ``q, k, alpha`` are
    ``[N, H, d_k]``, ``v`` is ``[N, H, d_v]``, ``s`` is ``[N, H, d_v, d_k]``.
    Returns ``(o, s_new)``; the input state is not modified.
    """
    q, k, v, a, s = _f64(q, k, v, alpha, s)
    S = s * a[..., None, :] + _outer(v, k)
    return _read(S, q), S


def gdelta_decode_step(q, k, v, alpha, beta, s):
    """One token of generation under the gated delta rule ("Scrivere meglio nella
    memoria", section "Unire oblio e correzione: Gated DeltaNet"):
    ``S <- S [alpha (I - beta k k^T)] + beta v k^T``, then ``o = S q``.

    The transition is applied as written, as a d_k x d_k matrix multiplying the
    memory from the right. ``q, k`` are ``[N, H, d_k]``, ``v`` is ``[N, H, d_v]``,
    ``alpha`` and ``beta`` are ``[N, H]`` (one gate and one write strength per
    sequence and head), ``s`` is ``[N, H, d_v, d_k]``. Returns ``(o, s_new)``; the
    input state is not modified.
    """
    q, k, v, a, b, s = _f64(q, k, v, alpha, beta, s)
    dk = k.shape[-1]
    eye = np.eye(dk)
    M = a[..., None, None] * (eye - b[..., None, None] * k[..., :, None] * k[..., None, :])
    S = np.einsum("...mc,...cd->...md", s, M) + b[..., None, None] * _outer(v, k)
    return _read(S, q), S


# --------------------------------------------------------------------------- feature map and output norm

def silu_l2(x):
    """DeltaNet's feature map on a query or key ("Scrivere meglio nella memoria", section
    "Superiore" of the introduction, and section "Correggere: la delta rule"): a SiLU,
    ``x * sigmoid(x)``, followed by L2 normalisation over the channel axis, so that
    ``beta ||k||^2 <= 1`` keeps the transition's eigenvalues in [0, 1]. A zero row stays
    zero (its norm is 0; nothing is divided)."""
    x = np.asarray(x, dtype=np.float64)
    y = x / (1.0 + np.exp(-x))
    n = np.sqrt(np.sum(y * y, axis=-1, keepdims=True))
    return np.where(n > 0.0, y / np.where(n > 0.0, n, 1.0), 0.0)


def rms_norm(o, weight, eps):
    """The output normalisation the pages name for DeltaNet (same page, on stabilising the
    readout without the normaliser z_t): each output row divided by its root mean square
    over the value channels, ``o / sqrt(mean(o^2) + eps)``, times a per-channel weight."""
    o = np.asarray(o, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    return o / np.sqrt(np.mean(o * o, axis=-1, keepdims=True) + eps) * w


def layer_norm(o, weight, bias, eps):
    """The output normalisation the gates page names for GLA (section "Correggere: la delta
    rule", beside DeltaNet's RMS norm): each output row centred on its mean over the value
    channels and divided by its standard deviation, ``(o - mean) / sqrt(var + eps)``, with
    ``var`` the mean squared deviation (the population variance), then scaled and shifted
    per channel by ``weight`` and ``bias`` (``bias=None``: no shift)."""
    o = np.asarray(o, dtype=np.float64)
    mean = np.mean(o, axis=-1, keepdims=True)
    dev = o - mean
    var = np.mean(dev * dev, axis=-1, keepdims=True)
    y = dev / np.sqrt(var + eps) * np.asarray(weight, dtype=np.float64)
    return y if bias is None else y + np.asarray(bias, dtype=np.float64)


# --------------------------------------------------------------------------- backward (reverse mode)

def scalar_backward(q, k, v, log_alpha, do, dS_T=None, s0=None):
    """Gradients of the scalar-decay recurrence by reverse-mode differentiation of its
    recurrent form (the definition: "Dimenticare: i gate", scalar decay equation), token by
    token. With D_t the gradient of the loss with respect to S_t:
    ``D_{T-1} = dS_T + do_{T-1} q_{T-1}^T``, ``D_t = a_{t+1} D_{t+1} + do_t q_t^T``, and
    ``dq_t = S_t^T do_t``, ``dk_t = D_t^T v_t``, ``dv_t = D_t k_t``,
    ``d log a_t = a_t <D_t, S_{t-1}>`` (Frobenius), ``dS_0 = a_0 D_0``.
    Returns ``(dq, dk, dv, dlog_alpha, ds0)``; ``do`` is ``[B, H, T, d_v]``."""
    q, k, v, la, do = _f64(q, k, v, log_alpha, do)
    S0 = _init_state(q, v, s0)
    T = q.shape[-2]
    a = np.exp(la)
    states = [S0]
    S = S0
    for t in range(T):
        S = a[..., t][..., None, None] * S + _outer(v[..., t, :], k[..., t, :])
        states.append(S)
    D = np.zeros_like(S0) if dS_T is None else np.asarray(dS_T, dtype=np.float64).copy()
    dq = np.zeros(q.shape); dk = np.zeros(k.shape); dv = np.zeros(v.shape); dla = np.zeros(la.shape)
    for t in range(T - 1, -1, -1):
        D = D + _outer(do[..., t, :], q[..., t, :])                 # now the gradient w.r.t. S_t
        dq[..., t, :] = np.einsum("...mc,...m->...c", states[t + 1], do[..., t, :])
        dk[..., t, :] = np.einsum("...mc,...m->...c", D, v[..., t, :])
        dv[..., t, :] = np.einsum("...mc,...c->...m", D, k[..., t, :])
        dla[..., t] = a[..., t] * np.einsum("...mc,...mc->...", D, states[t])
        D = a[..., t][..., None, None] * D                            # through S_t = a_t S_{t-1} + ...
    return dq, dk, dv, dla, D


def gdelta_backward(q, k, v, log_alpha, beta, do, dS_T=None, s0=None):
    """Gradients of the gated delta rule by reverse-mode differentiation of its recurrent
    form (the definition: "Scrivere meglio nella memoria", section "Unire oblio e
    correzione: Gated DeltaNet"), token by token. Forward, per token: the fade
    ``S' = a_t S_{t-1}``, the prediction ``e_t = S' k_t``, the write
    ``u_t = beta_t (v_t - e_t)``, ``S_t = S' + u_t k_t^T`` and the readout ``o_t = S_t q_t``.
    Backward, with D the gradient of the loss with respect to S_t (``dS_T`` after the last
    token), each step taken in reverse order:
    ``D += do_t q_t^T``, ``dq_t = S_t^T do_t``; through the write ``du_t = D k_t``,
    ``dk_t = D^T u_t``; through ``u_t``: ``dbeta_t = du_t . (v_t - e_t)``,
    ``dv_t = beta_t du_t``, ``de_t = -beta_t du_t``; through the prediction
    ``dk_t += S'^T de_t`` and ``D' = D + de_t k_t^T`` (the gradient w.r.t. S'); through the
    fade ``d log a_t = <D', S'>`` (Frobenius) and ``D = a_t D'`` for S_{t-1}.
    Returns ``(dq, dk, dv, dlog_alpha, dbeta, ds0)``; ``do`` is ``[B, H, T, d_v]``."""
    q, k, v, la, be, do = _f64(q, k, v, log_alpha, beta, do)
    S0 = _init_state(q, v, s0)
    T = q.shape[-2]
    a = np.exp(la)
    states = [S0]
    S = S0
    for t in range(T):
        Sp = a[..., t][..., None, None] * S
        u = be[..., t][..., None] * (v[..., t, :] - _read(Sp, k[..., t, :]))
        S = Sp + _outer(u, k[..., t, :])
        states.append(S)
    D = np.zeros_like(S0) if dS_T is None else np.asarray(dS_T, dtype=np.float64).copy()
    dq = np.zeros(q.shape); dk = np.zeros(k.shape); dv = np.zeros(v.shape)
    dla = np.zeros(la.shape); dbe = np.zeros(be.shape)
    for t in range(T - 1, -1, -1):
        kt, vt, qt = k[..., t, :], v[..., t, :], q[..., t, :]
        Sp = a[..., t][..., None, None] * states[t]
        e = _read(Sp, kt)
        u = be[..., t][..., None] * (vt - e)
        D = D + _outer(do[..., t, :], qt)                            # now the gradient w.r.t. S_t
        dq[..., t, :] = np.einsum("...mc,...m->...c", states[t + 1], do[..., t, :])
        du = _read(D, kt)
        dkt = np.einsum("...mc,...m->...c", D, u)
        dbe[..., t] = np.sum(du * (vt - e), axis=-1)
        dv[..., t, :] = be[..., t][..., None] * du
        de = -be[..., t][..., None] * du
        dkt = dkt + np.einsum("...mc,...m->...c", Sp, de)
        dk[..., t, :] = dkt
        D = D + _outer(de, kt)                                        # the gradient w.r.t. S'
        dla[..., t] = np.einsum("...mc,...mc->...", D, Sp)
        D = a[..., t][..., None, None] * D                            # through S' = a_t S_{t-1}
    return dq, dk, dv, dla, dbe, D


def gla_backward(q, k, v, log_alpha, do, dS_T=None, s0=None):
    """Gradients of the diagonal-gate (GLA) recurrence by reverse-mode differentiation of its
    recurrent form ("Dimenticare: i gate", diagonal-gate equation), token by token. With D_t
    the gradient of the loss with respect to S_t: ``D_{T-1} = dS_T + do_{T-1} q_{T-1}^T``,
    ``D_t = D_{t+1} Diag(a_{t+1}) + do_t q_t^T``, and ``dq_t = S_t^T do_t``,
    ``dk_t = D_t^T v_t``, ``dv_t = D_t k_t``, ``d log a_t[c] = a_t[c] sum_m D_t[m, c]
    S_{t-1}[m, c]``, ``dS_0 = D_0 Diag(a_0)``. Returns ``(dq, dk, dv, dlog_alpha, ds0)`` with
    ``dlog_alpha`` shaped like ``log_alpha`` ``[B, H, T, d_k]``."""
    q, k, v, la, do = _f64(q, k, v, log_alpha, do)
    S0 = _init_state(q, v, s0)
    T = q.shape[-2]
    a = np.exp(la)
    states = [S0]
    S = S0
    for t in range(T):
        S = S * a[..., t, :][..., None, :] + _outer(v[..., t, :], k[..., t, :])
        states.append(S)
    D = np.zeros_like(S0) if dS_T is None else np.asarray(dS_T, dtype=np.float64).copy()
    dq = np.zeros(q.shape); dk = np.zeros(k.shape); dv = np.zeros(v.shape); dla = np.zeros(la.shape)
    for t in range(T - 1, -1, -1):
        D = D + _outer(do[..., t, :], q[..., t, :])                 # now the gradient w.r.t. S_t
        dq[..., t, :] = np.einsum("...mc,...m->...c", states[t + 1], do[..., t, :])
        dk[..., t, :] = np.einsum("...mc,...m->...c", D, v[..., t, :])
        dv[..., t, :] = np.einsum("...mc,...c->...m", D, k[..., t, :])
        dla[..., t, :] = a[..., t, :] * np.einsum("...mc,...mc->...c", D, states[t])
        D = D * a[..., t, :][..., None, :]                           # through S_t = S_{t-1} Diag(a_t) + ...
    return dq, dk, dv, dla, D


def retention_backward(q, k, v, log_gamma, do, dS_T=None, s0=None):
    """Retention is the scalar decay with the same gate at every step of head h, so its
    gradients are scalar_backward's, with the gate gradient summed over the batch and the
    tokens of each head. Returns ``(dq, dk, dv, dlog_gamma [H], ds0)``."""
    q = np.asarray(q)
    B, H, T = q.shape[:3]
    la = np.broadcast_to(np.asarray(log_gamma, dtype=np.float64)[None, :, None], (B, H, T))
    dq, dk, dv, dla, ds0 = scalar_backward(q, k, v, la, do, dS_T=dS_T, s0=s0)
    return dq, dk, dv, dla.sum(axis=(0, 2)), ds0


# --------------------------------------------------------------------------- variational linear attention

def elu1(x):
    """The ELU+1 feature map named by the VLA summary page for its output (section 2.3, last
    paragraph): ``x + 1`` for ``x > 0``, ``e^x`` otherwise; positive everywhere."""
    x = np.asarray(x, dtype=np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def _vla_step(S, A, n, q_t, k_t, v_t, u_t, readout):
    """One token of VLA, the three steps of the recursive update in the order the VLA
    summary page gives them ("Riepilogo Tecnico: Attenzione Lineare Variazionale (VLA)",
    section 2.3; the penalty geometry of section 2.2):

    1. Sherman-Morrison on the inverse penalty: ``M_t = M_{t-1} + u_t u_t^T`` gives
       ``A_t = A_{t-1} - z_t z_t^T / (1 + u_t^T z_t)`` with ``z_t = A_{t-1} u_t``;
    2. the gating vector from the *updated* inverse: ``a_t = A_t k^_t / |A_t k^_t|``,
       with the key normalised to unit length (section 2.1);
    3. the memory: ``S_t = S_{t-1} + (v_t - S_{t-1} k^_t) a_t^T``.

    Readout, read after the write. ``"ratio"`` (the page's output: a ratio of recurrences
    as in standard linear attention, with the ELU+1 feature map phi): keys and queries pass
    through phi, ``k^_t = phi(k_t) / |phi(k_t)|``, and the denominator vector ``n`` obeys the
    same update driven by the constant value 1, ``n_t = n_{t-1} + (1 - n_{t-1}.k^_t) a_t``;
    ``o_t = S_t phi(q_t) / (n_t . phi(q_t))``. ``"linear"``: no feature map and no
    normaliser, ``k^_t = k_t / |k_t|``, ``o_t = S_t q_t``; ``n`` is not used.
    Shapes: S ``[..., d_v, d_k]``, A ``[..., d_k, d_k]``, n and vectors ``[..., d]``."""
    z = np.einsum("...mc,...c->...m", A, u_t)
    den = 1.0 + np.sum(u_t * z, axis=-1)
    A = A - z[..., :, None] * z[..., None, :] / den[..., None, None]
    kf = elu1(k_t) if readout == "ratio" else k_t
    kh = kf / np.linalg.norm(kf, axis=-1, keepdims=True)
    y = np.einsum("...mc,...c->...m", A, kh)
    a = y / np.linalg.norm(y, axis=-1, keepdims=True)
    resid = v_t - np.einsum("...mc,...c->...m", S, kh)
    S = S + resid[..., :, None] * a[..., None, :]
    if readout == "linear":
        return _read(S, q_t), S, A, n
    n = n + (1.0 - np.sum(n * kh, axis=-1))[..., None] * a
    fq = elu1(q_t)
    return _read(S, fq) / np.sum(n * fq, axis=-1)[..., None], S, A, n


def _vla_init_penalty(k, a0, lambda0):
    dk = k.shape[-1]
    if a0 is not None:
        return np.array(a0, dtype=np.float64)
    return np.broadcast_to(np.eye(dk) / float(lambda0), k.shape[:-2] + (dk, dk)).copy()


def _vla_readout(readout):
    if readout not in ("ratio", "linear"):
        raise ValueError(f"readout must be 'ratio' or 'linear', got {readout!r}")
    return readout


def vla_recurrent(q, k, v, u, lambda0=1.0, s0=None, a0=None, n0=None, readout="ratio"):
    """Variational linear attention over whole sequences, token by token (the
    definition: section 2.3 of the VLA summary page; see ``_vla_step``).

    ``q, k, u`` are ``[B, H, T, d_k]`` (``u_t`` the penalty direction added to M at
    token t), ``v`` is ``[B, H, T, d_v]``. The inverse penalty starts at
    ``A_0 = M_0^{-1} = I / lambda0`` unless ``a0 [B, H, d_k, d_k]`` is given; the
    memory at ``s0`` or zeros; with the ratio readout the denominator vector at
    ``n0 [B, H, d_k]`` or zeros. Returns ``(o, S_T, A_T, n_T)`` (``n_T`` None with the
    linear readout)."""
    readout = _vla_readout(readout)
    q, k, v, u, n0 = _f64(q, k, v, u, n0)
    S = _init_state(q, v, s0)
    A = _vla_init_penalty(k, a0, lambda0)
    n = None
    if readout == "ratio":
        n = np.zeros(k.shape[:-2] + (k.shape[-1],)) if n0 is None else n0.copy()
    T = q.shape[-2]
    o = np.zeros(v.shape)
    for t in range(T):
        o[..., t, :], S, A, n = _vla_step(S, A, n, q[..., t, :], k[..., t, :], v[..., t, :], u[..., t, :], readout)
    return o, S, A, n


def vla_decode_step(q, k, v, u, s, a, n=None, readout="ratio"):
    """One VLA token for N sequences: ``q, k, u [N, H, d_k]``, ``v [N, H, d_v]``, the
    memory ``s [N, H, d_v, d_k]``, inverse penalty ``a [N, H, d_k, d_k]`` and, with the ratio
    readout, the denominator vector ``n [N, H, d_k]``. Returns ``(o, s_new, a_new, n_new)``;
    the inputs are not modified."""
    readout = _vla_readout(readout)
    q, k, v, u, s, a, n = _f64(q, k, v, u, s, a, n)
    if readout == "ratio" and n is None:
        raise ValueError("the ratio readout carries the denominator vector n")
    return _vla_step(s, a, n, q, k, v, u, readout)
