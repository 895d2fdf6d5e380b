"""Pins of the oracle's variational linear attention (VLA summary page, "Riepilogo
Tecnico: Attenzione Lineare Variazionale (VLA)", sections 2.1-2.3 and 3.1).

Each test checks the oracle against something other than itself: three-token examples
worked by hand from the update rule (one per readout), the closed form of the inverse
penalty, steps rebuilt from a directly inverted penalty matrix, the delta rule it reduces
to when no penalty is added, the exact read-back of the ratio readout, and the Jacobian by
finite differences.

Two readouts: ``"ratio"`` is the page's output (section 2.3, last paragraph: a ratio of
recurrences as in standard linear attention, with the ELU+1 feature map phi on keys and
queries; the denominator vector n follows the same update driven by the value 1);
``"linear"`` is ``o = S q`` with the key only normalised."""

from math import log, sqrt

import numpy as np
import pytest

import oracle as orc


def _hand_inputs():
    # d_k = 2, d_v = 1, lambda0 = 1, three tokens
    q = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    k = np.array([[1.0, 1.0], [0.0, 3.0], [1.0, 0.0]])
    v = np.array([[2.0], [1.0], [0.0]])
    u = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    return [x[None, None] for x in (q, k, v, u)]


def test_hand_example_linear():
    """Worked by hand from the three steps of section 2.3 with A_0 = I, S_0 = 0:
    t=1: z = (1,0), A_1 = diag(1/2, 1), A_1 k^ ~ (1/2, 1) so a = (1,2)/sqrt5, S_1 = 2a^T,
         o_1 = 2/sqrt5;
    t=2: z = (0,1), A_2 = I/2, k^ = (0,1) = a, S_2 = (2/sqrt5, 1), o_2 = 1;
    t=3: z = (1/2,1/2), den = 2, A_3 = [[3/8,-1/8],[-1/8,3/8]], a = (3,-1)/sqrt10,
         residual -2/sqrt5, S_3 = (2/sqrt5 - 3sqrt2/5, 1 + sqrt2/5), o_3 = S_3 . (1,1).
    Using A_{t-1} for the gating vector, the opposite sign in the Sherman-Morrison step,
    an unnormalised key or the write without the residual all change o_1, o_2 or o_3."""
    q, k, v, u = _hand_inputs()
    o, S, A, n = orc.vla_recurrent(q, k, v, u, lambda0=1.0, readout="linear")
    assert n is None
    r5, r2 = np.sqrt(5.0), np.sqrt(2.0)
    s3 = np.array([2 / r5 - 3 * r2 / 5, 1 + r2 / 5])
    np.testing.assert_allclose(o[0, 0, :, 0], [2 / r5, 1.0, s3.sum()], rtol=0, atol=1e-14)
    np.testing.assert_allclose(S[0, 0], s3[None, :], rtol=0, atol=1e-14)
    np.testing.assert_allclose(A[0, 0], [[3 / 8, -1 / 8], [-1 / 8, 3 / 8]], rtol=0, atol=1e-15)


def test_hand_example_ratio():
    """The ratio readout worked by hand, d_k = 2, d_v = 1, A_0 = I, S_0 = 0, n_0 = 0, with
    phi(x) = x + 1 (x > 0) or e^x:
    t=1: k = (0,0), phi(k) = (1,1), k^ = (1,1)/sqrt2, u = 0 so a = k^; v = 2:
         S_1 = sqrt2 (1,1), n_1 = (1,1)/sqrt2; q = (1, -ln2), phi(q) = (2, 1/2):
         o_1 = 2.5 sqrt2 / (2.5/sqrt2) = 2;
    t=2: k = (2,3), phi(k) = (3,4), k^ = a = (0.6, 0.8); v = 1, q = 0, phi(q) = (1,1):
         S_2 = (0.6 + 0.16 sqrt2, 0.8 - 0.12 sqrt2), n_2 = (0.6 + 0.08 sqrt2, 0.8 - 0.06 sqrt2),
         o_2 = (1.4 + 0.04 sqrt2) / (1.4 + 0.02 sqrt2);
    t=3: u = (1,0): A_3 = diag(1/2, 1); k = (1,1), k^ = (1,1)/sqrt2, a = (1,2)/sqrt5; v = 0,
         q = 0: S_3 = S_2 - (S_2.k^) a, n_3 = n_2 + (1 - n_2.k^) a,
         o_3 = (1.4 + 0.04 sqrt2)(1 - 3/sqrt10) / ((1.4 + 0.02 sqrt2) + (1 - (1.4 + 0.02 sqrt2)/sqrt2) 3/sqrt5).
    phi on the query only (k^ = k/|k| = 0/0 at t=1), ELU without the +1 (phi(k_1) = 0), a
    denominator driven by v instead of 1, or n left out of the update change o_1, o_2 or o_3."""
    r2 = sqrt(2.0)
    q = np.array([[1.0, -log(2.0)], [0.0, 0.0], [0.0, 0.0]])
    k = np.array([[0.0, 0.0], [2.0, 3.0], [1.0, 1.0]])
    v = np.array([[2.0], [1.0], [0.0]])
    u = np.array([[0.0, 0.0], [0.0, 0.0], [1.0, 0.0]])
    o, S, A, n = orc.vla_recurrent(*(x[None, None] for x in (q, k, v, u)), lambda0=1.0)
    o2 = (1.4 + 0.04 * r2) / (1.4 + 0.02 * r2)
    o3 = (1.4 + 0.04 * r2) * (1 - 3 / sqrt(10.0)) / ((1.4 + 0.02 * r2) + (1 - (1.4 + 0.02 * r2) / r2) * 3 / sqrt(5.0))
    np.testing.assert_allclose(o[0, 0, :, 0], [2.0, o2, o3], rtol=0, atol=1e-14)
    s2 = np.array([0.6 + 0.16 * r2, 0.8 - 0.12 * r2])
    n2 = np.array([0.6 + 0.08 * r2, 0.8 - 0.06 * r2])
    a3 = np.array([1.0, 2.0]) / sqrt(5.0)
    np.testing.assert_allclose(S[0, 0, 0], s2 - s2.sum() / r2 * a3, rtol=0, atol=1e-14)
    np.testing.assert_allclose(n[0, 0], n2 + (1 - n2.sum() / r2) * a3, rtol=0, atol=1e-14)
    np.testing.assert_allclose(A[0, 0], [[0.5, 0.0], [0.0, 1.0]], rtol=0, atol=1e-15)


def test_elu1_values():
    """phi = ELU + 1: x + 1 above zero, e^x at and below zero (continuous at 0, positive)."""
    x = np.array([-50.0, -1.0, 0.0, 0.5, 3.0])
    np.testing.assert_allclose(orc.elu1(x), [np.exp(-50.0), np.exp(-1.0), 1.0, 1.5, 4.0], rtol=1e-15)


def _rand(rng, B, H, T, dk, dv):
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv))
    u = rng.standard_normal((B, H, T, dk)) / np.sqrt(dk)
    return q, k, v, u


@pytest.mark.parametrize("readout", ["ratio", "linear"])
def test_inverse_penalty_closed_form(readout):
    """Section 2.2: A_t = M_t^{-1} exactly, with M_t = M_0 + sum_s u_s u_s^T; checked with a
    direct inverse, from M_0 = lambda0 I and from a handed-over A_0 (whatever the readout)."""
    rng = np.random.default_rng(50)
    B, H, T, dk, dv = 2, 2, 20, 6, 3
    q, k, v, u = _rand(rng, B, H, T, dk, dv)
    _, _, A, _ = orc.vla_recurrent(q, k, v, u, lambda0=0.7, readout=readout)
    M = 0.7 * np.eye(dk) + np.einsum("bhtc,bhtd->bhcd", u, u)
    np.testing.assert_allclose(A, np.linalg.inv(M), rtol=1e-10, atol=1e-12)
    G = rng.standard_normal((B, H, dk, dk))
    M0 = G @ np.swapaxes(G, -1, -2) + np.eye(dk)
    _, _, A, _ = orc.vla_recurrent(q, k, v, u, a0=np.linalg.inv(M0), readout=readout)
    np.testing.assert_allclose(A, np.linalg.inv(M0 + np.einsum("bhtc,bhtd->bhcd", u, u)), rtol=1e-9, atol=1e-11)


@pytest.mark.parametrize("readout", ["ratio", "linear"])
def test_step_rebuilt_from_direct_inverse(readout):
    """The whole recurrence rebuilt with A_t = inv(M_t) taken directly at every token
    (no Sherman-Morrison), the gating vector, the write and the readout as written in
    section 2.3 (ratio: phi on k and q, the denominator vector written with the value 1)."""
    rng = np.random.default_rng(51)
    B, H, T, dk, dv = 1, 3, 12, 5, 4
    q, k, v, u = _rand(rng, B, H, T, dk, dv)
    s0 = rng.standard_normal((B, H, dv, dk))
    n0 = rng.uniform(0.5, 1.5, (B, H, dk))
    o, S, _, n = orc.vla_recurrent(q, k, v, u, lambda0=2.0, s0=s0, n0=n0, readout=readout)
    phi = (lambda x: np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))) if readout == "ratio" else (lambda x: x)
    for h in range(H):
        M = 2.0 * np.eye(dk)
        Sh = s0[0, h].copy()
        nh = n0[0, h].copy()
        for t in range(T):
            M = M + np.outer(u[0, h, t], u[0, h, t])
            kf = phi(k[0, h, t])
            kh = kf / np.linalg.norm(kf)
            y = np.linalg.solve(M, kh)
            a = y / np.linalg.norm(y)
            Sh = Sh + np.outer(v[0, h, t] - Sh @ kh, a)
            nh = nh + (1.0 - nh @ kh) * a
            fq = phi(q[0, h, t])
            want = Sh @ fq / (nh @ fq) if readout == "ratio" else Sh @ fq
            np.testing.assert_allclose(o[0, h, t], want, rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(S[0, h], Sh, rtol=1e-10, atol=1e-12)
        if readout == "ratio":
            np.testing.assert_allclose(n[0, h], nh, rtol=1e-10, atol=1e-12)


def test_no_penalty_is_the_delta_rule():
    """With u = 0 the inverse penalty stays I / lambda0 and the gating vector is the
    normalised key: the write is the delta rule with beta = 1 on unit keys, so the memory
    reads back exactly v_t under k^_t after every token, and the outputs are the gated
    delta rule's (its own pins elsewhere) with alpha = beta = 1."""
    rng = np.random.default_rng(52)
    B, H, T, dk, dv = 2, 1, 9, 4, 3
    q, k, v, _ = _rand(rng, B, H, T, dk, dv)
    u = np.zeros_like(k)
    o, S, A, _ = orc.vla_recurrent(q, k, v, u, lambda0=3.0, readout="linear")
    np.testing.assert_allclose(A, np.broadcast_to(np.eye(dk) / 3.0, A.shape), atol=1e-15)
    kh = k / np.linalg.norm(k, axis=-1, keepdims=True)
    s = np.zeros((B, H, dv, dk))
    a = np.broadcast_to(np.eye(dk) / 3.0, (B, H, dk, dk))
    for t in range(T):
        _, s, a, _ = orc.vla_decode_step(q[:, :, t], k[:, :, t], v[:, :, t], u[:, :, t], s, a, readout="linear")
        np.testing.assert_allclose(np.einsum("bhmc,bhc->bhm", s, kh[:, :, t]), v[:, :, t], atol=1e-12)
    o_d, S_d = orc.gdelta_recurrent(q, kh, v, np.zeros((B, H, T)), np.ones((B, H, T)))
    np.testing.assert_allclose(o, o_d, atol=1e-12)
    np.testing.assert_allclose(S, S_d, atol=1e-12)


def test_ratio_reads_back_the_value():
    """With u = 0 (a = k^) and the query equal to the key, the ratio readout returns the value
    just written, exactly: S_t k^_t = v_t and n_t . k^_t = 1 after the write, and phi(q_t) is
    a positive multiple of k^_t. Fails if phi is left off either side, if the denominator
    is written with anything but 1, or if numerator and denominator use different keys."""
    rng = np.random.default_rng(56)
    B, H, T, dk, dv = 2, 2, 15, 8, 5
    _, k, v, _ = _rand(rng, B, H, T, dk, dv)
    s0 = rng.standard_normal((B, H, dv, dk))
    n0 = rng.uniform(0.5, 1.5, (B, H, dk))
    o, _, _, _ = orc.vla_recurrent(k, k, v, np.zeros_like(k), lambda0=0.4, s0=s0, n0=n0)
    np.testing.assert_allclose(o, v, rtol=1e-11, atol=1e-12)


def test_ratio_is_an_extra_memory_row():
    """The denominator vector is one more row of the memory with value 1: the linear readout
    run on phi(k), phi(q) with v extended by a constant 1 gives the numerator in its first
    d_v outputs and the denominator in the last."""
    rng = np.random.default_rng(57)
    B, H, T, dk, dv = 1, 2, 17, 6, 3
    q, k, v, u = _rand(rng, B, H, T, dk, dv)
    s0 = rng.standard_normal((B, H, dv, dk)) * 0.1
    n0 = rng.uniform(0.5, 1.5, (B, H, dk))
    o, S, A, n = orc.vla_recurrent(q, k, v, u, lambda0=1.3, s0=s0, n0=n0)
    v_ext = np.concatenate([v, np.ones((B, H, T, 1))], axis=-1)
    s_ext = np.concatenate([s0, n0[:, :, None, :]], axis=-2)
    o_lin, S_lin, A_lin, _ = orc.vla_recurrent(orc.elu1(q), orc.elu1(k), v_ext, u, lambda0=1.3, s0=s_ext,
                                               readout="linear")
    np.testing.assert_allclose(o, o_lin[..., :dv] / o_lin[..., dv:], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S, S_lin[..., :dv, :], atol=1e-12)
    np.testing.assert_allclose(n, S_lin[..., dv, :], atol=1e-12)
    np.testing.assert_allclose(A, A_lin, atol=1e-13)


def test_key_scale_invariance():
    """Linear readout: only the direction of k enters (section 2.3: the key is normalised);
    the penalty direction u is not normalised, so scaling it changes the result."""
    rng = np.random.default_rng(53)
    B, H, T, dk, dv = 1, 2, 8, 4, 4
    q, k, v, u = _rand(rng, B, H, T, dk, dv)
    scale = rng.uniform(0.1, 10.0, (B, H, T, 1))
    o1, S1, A1, _ = orc.vla_recurrent(q, k, v, u, readout="linear")
    o2, S2, A2, _ = orc.vla_recurrent(q, k * scale, v, u, readout="linear")
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(S2, S1, atol=1e-12)
    o3, _, _, _ = orc.vla_recurrent(q, k, v, u * 3.0, readout="linear")
    assert np.max(np.abs(o3 - o1)) > 1e-3


def test_jacobian():
    """Section 3.1: dS_t / dS_{t-1} is S -> S (I - k^ a^T). Checked by central differences of
    one step against that map, with a built from a directly inverted penalty. Its spectral
    norm is 1 when a = k^ (u = 0, a projector); for a != k^ it exceeds 1 (the linear hand
    example's third token), so the page's unit-norm statement is read as the case a = k^."""
    rng = np.random.default_rng(54)
    dk, dv = 4, 3
    S0 = rng.standard_normal((dv, dk)); A0 = np.eye(dk)
    q = rng.standard_normal(dk); k = rng.standard_normal(dk); v = rng.standard_normal(dv)
    u = rng.standard_normal(dk) / 2
    kh = k / np.linalg.norm(k)
    y = np.linalg.solve(np.eye(dk) + np.outer(u, u), kh)
    a = y / np.linalg.norm(y)
    P = np.eye(dk) - np.outer(kh, a)
    eps = 1e-6
    for idx in np.ndindex(S0.shape):
        dS = np.zeros_like(S0); dS[idx] = eps
        _, Sp, _, _ = orc.vla_decode_step(q, k, v, u, S0 + dS, A0, readout="linear")
        _, Sm, _, _ = orc.vla_decode_step(q, k, v, u, S0 - dS, A0, readout="linear")
        np.testing.assert_allclose((Sp - Sm) / (2 * eps), dS / eps @ P, atol=1e-8)
    assert abs(np.linalg.norm(np.eye(dk) - np.outer(kh, kh), 2) - 1.0) < 1e-12
    k3 = np.array([1.0, 0.0]); a3 = np.array([3.0, -1.0]) / np.sqrt(10.0)
    assert np.linalg.norm(np.eye(2) - np.outer(k3, a3), 2) > 1.0 + 1e-3


@pytest.mark.parametrize("readout", ["ratio", "linear"])
@pytest.mark.parametrize("split", [0, 1, 5, 9])
def test_decode_and_resume(split, readout):
    """Decode steps one token at a time, and two calls joined at ``split`` with the memory,
    the inverse penalty and (ratio) the denominator vector handed over, equal one call."""
    rng = np.random.default_rng(55)
    B, H, T, dk, dv = 2, 2, 9, 4, 3
    q, k, v, u = _rand(rng, B, H, T, dk, dv)
    o, S, A, n = orc.vla_recurrent(q, k, v, u, lambda0=0.5, readout=readout)
    o1, S1, A1, n1 = orc.vla_recurrent(q[:, :, :split], k[:, :, :split], v[:, :, :split], u[:, :, :split],
                                       lambda0=0.5, readout=readout)
    o2, S2, A2, n2 = orc.vla_recurrent(q[:, :, split:], k[:, :, split:], v[:, :, split:], u[:, :, split:], s0=S1,
                                       a0=A1, n0=n1, readout=readout)
    np.testing.assert_allclose(np.concatenate([o1, o2], axis=2), o, atol=1e-12)
    np.testing.assert_allclose(S2, S, atol=1e-12)
    np.testing.assert_allclose(A2, A, atol=1e-12)
    if readout == "ratio":
        np.testing.assert_allclose(n2, n, atol=1e-12)
    s, a = np.zeros((B, H, dv, dk)), np.broadcast_to(np.eye(dk) / 0.5, (B, H, dk, dk))
    nn = np.zeros((B, H, dk)) if readout == "ratio" else None
    for t in range(T):
        ot, s, a, nn = orc.vla_decode_step(q[:, :, t], k[:, :, t], v[:, :, t], u[:, :, t], s, a, nn, readout=readout)
        np.testing.assert_allclose(ot, o[:, :, t], atol=1e-12)
