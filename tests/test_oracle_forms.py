"""The oracle's three forms agree, and agree with brute force on tiny inputs.

The RetNet page (section on retention, Fig. 16.5) states that the parallel,
recurrent and chunkwise forms give exactly the same result; the recurrent form
is the definition. Brute force here means the recurrence unrolled by hand:
explicit double sums over (t, j) with the product of the gates in between for
retention and GLA, and the explicit product of transition matrices (the
transition column of the table in "Le ricorrenze come regressione online") for
the gated delta rule, all in plain Python loops.
"""

import numpy as np
import pytest

import oracle as orc


def _rand(seed, B, H, T, dk, dv, state=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, dk)) / np.sqrt(dk)
    k = rng.standard_normal((B, H, T, dk)) / np.sqrt(dk)
    v = rng.standard_normal((B, H, T, dv))
    s0 = rng.standard_normal((B, H, dv, dk)) if state else None
    return rng, q, k, v, s0


SHAPES = [(1, 1, 1, 4, 3), (2, 3, 23, 8, 6), (1, 2, 64, 16, 16), (2, 1, 50, 5, 7)]
CHUNKS = [1, 3, 16, 64]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("chunk", CHUNKS)
@pytest.mark.parametrize("state", [False, True])
def test_retention_forms_agree(shape, chunk, state):
    rng, q, k, v, s0 = _rand(1, *shape, state=state)
    lg = np.log(rng.uniform(0.5, 0.999, shape[1]))
    o_r, S_r = orc.retention_recurrent(q, k, v, lg, s0=s0)
    o_q, S_q = orc.retention_quadratic(q, k, v, lg, s0=s0)
    o_c, S_c = orc.retention_chunkwise(q, k, v, lg, chunk, s0=s0)
    for o, S in ((o_q, S_q), (o_c, S_c)):
        np.testing.assert_allclose(o, o_r, atol=1e-12, rtol=0)
        np.testing.assert_allclose(S, S_r, atol=1e-12, rtol=0)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("chunk", CHUNKS)
@pytest.mark.parametrize("state", [False, True])
def test_gla_forms_agree(shape, chunk, state):
    rng, q, k, v, s0 = _rand(2, *shape, state=state)
    B, H, T, dk, dv = shape
    la = -np.logaddexp(0.0, -rng.standard_normal((B, H, T, dk))) / 4.0
    o_r, S_r = orc.gla_recurrent(q, k, v, la, s0=s0)
    o_q, S_q = orc.gla_quadratic(q, k, v, la, s0=s0)
    o_c, S_c = orc.gla_chunkwise(q, k, v, la, chunk, s0=s0)
    for o, S in ((o_q, S_q), (o_c, S_c)):
        np.testing.assert_allclose(o, o_r, atol=1e-12, rtol=0)
        np.testing.assert_allclose(S, S_r, atol=1e-12, rtol=0)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("chunk", CHUNKS)
@pytest.mark.parametrize("state", [False, True])
def test_scalar_forms_agree(shape, chunk, state):
    rng, q, k, v, s0 = _rand(5, *shape, state=state)
    B, H, T, dk, dv = shape
    la = -np.logaddexp(0.0, -rng.standard_normal((B, H, T))) / 2.0
    o_r, S_r = orc.scalar_recurrent(q, k, v, la, s0=s0)
    o_q, S_q = orc.scalar_quadratic(q, k, v, la, s0=s0)
    o_c, S_c = orc.scalar_chunkwise(q, k, v, la, chunk, s0=s0)
    for o, S in ((o_q, S_q), (o_c, S_c)):
        np.testing.assert_allclose(o, o_r, atol=1e-12, rtol=0)
        np.testing.assert_allclose(S, S_r, atol=1e-12, rtol=0)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("chunk", CHUNKS)
@pytest.mark.parametrize("state", [False, True])
def test_gdelta_forms_agree(shape, chunk, state):
    rng, q, k, v, s0 = _rand(3, *shape, state=state)
    B, H, T, dk, dv = shape
    k = k / np.linalg.norm(k, axis=-1, keepdims=True)
    la = -np.logaddexp(0.0, rng.standard_normal((B, H, T))) / 8.0
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, H, T))))
    o_r, S_r = orc.gdelta_recurrent(q, k, v, la, beta, s0=s0)
    o_q, S_q = orc.gdelta_quadratic(q, k, v, la, beta, s0=s0)
    o_c, S_c = orc.gdelta_chunkwise(q, k, v, la, beta, chunk, s0=s0)
    for o, S in ((o_q, S_q), (o_c, S_c)):
        np.testing.assert_allclose(o, o_r, atol=1e-11, rtol=0)
        np.testing.assert_allclose(S, S_r, atol=1e-11, rtol=0)


def test_empty_sequence_passes_state_through():
    """T = 0: no output rows, and the final memory is the handed-over one (or zeros)."""
    rng, q, k, v, s0 = _rand(4, 2, 2, 0, 8, 4)
    la_d = np.zeros((2, 2, 0, 8)); la_s = np.zeros((2, 2, 0))
    lg = np.log([0.9, 0.8])
    for fn in (lambda s: orc.retention_recurrent(q, k, v, lg, s0=s),
               lambda s: orc.retention_quadratic(q, k, v, lg, s0=s),
               lambda s: orc.retention_chunkwise(q, k, v, lg, 4, s0=s),
               lambda s: orc.gla_recurrent(q, k, v, la_d, s0=s),
               lambda s: orc.gla_quadratic(q, k, v, la_d, s0=s),
               lambda s: orc.gla_chunkwise(q, k, v, la_d, 4, s0=s),
               lambda s: orc.scalar_recurrent(q, k, v, la_s, s0=s),
               lambda s: orc.scalar_quadratic(q, k, v, la_s, s0=s),
               lambda s: orc.scalar_chunkwise(q, k, v, la_s, 4, s0=s),
               lambda s: orc.gdelta_recurrent(q, k, v, la_s, la_s, s0=s),
               lambda s: orc.gdelta_quadratic(q, k, v, la_s, la_s, s0=s),
               lambda s: orc.gdelta_chunkwise(q, k, v, la_s, la_s, 4, s0=s)):
        o, S = fn(s0)
        assert o.shape == (2, 2, 0, 4)
        np.testing.assert_array_equal(S, s0)
        o, S = fn(None)
        np.testing.assert_array_equal(S, np.zeros((2, 2, 4, 8)))


# ----------------------------------------------------------------------------- brute force

def test_retention_and_gla_brute_force_double_sum():
    """o_t = sum_{j<=t} (prod_{r=j+1..t} alpha_r) (q_t . k_j) v_j per key channel, plus the
    handed-over memory decayed over t+1 steps, in pure Python loops (T <= 6)."""
    rng = np.random.default_rng(20)
    T, dk, dv = 6, 3, 2
    q = rng.standard_normal((T, dk)); k = rng.standard_normal((T, dk)); v = rng.standard_normal((T, dv))
    s0 = rng.standard_normal((dv, dk))
    a = rng.uniform(0.3, 0.95, (T, dk))
    want = np.zeros((T, dv))
    for t in range(T):
        for m in range(dv):
            tot = 0.0
            for c in range(dk):
                dec0 = 1.0
                for r in range(0, t + 1):
                    dec0 *= a[r, c]
                tot += s0[m, c] * dec0 * q[t, c]
                for j in range(t + 1):
                    dec = 1.0
                    for r in range(j + 1, t + 1):
                        dec *= a[r, c]
                    tot += q[t, c] * k[j, c] * dec * v[j, m]
            want[t, m] = tot
    a4 = lambda x: x[None, None]
    for o, _ in (orc.gla_recurrent(a4(q), a4(k), a4(v), a4(np.log(a)), s0=s0[None, None]),
                 orc.gla_quadratic(a4(q), a4(k), a4(v), a4(np.log(a)), s0=s0[None, None]),
                 orc.gla_chunkwise(a4(q), a4(k), a4(v), a4(np.log(a)), 4, s0=s0[None, None])):
        np.testing.assert_allclose(o[0, 0], want, atol=1e-13)
    # retention: the same double sum with one gate for every channel and step
    g = 0.8
    want = np.zeros((T, dv))
    for t in range(T):
        for m in range(dv):
            tot = sum(g ** (t + 1) * s0[m, c] * q[t, c] for c in range(dk))
            for j in range(t + 1):
                tot += g ** (t - j) * sum(q[t, c] * k[j, c] for c in range(dk)) * v[j, m]
            want[t, m] = tot
    lg = np.array([np.log(g)])
    for o, _ in (orc.retention_recurrent(a4(q), a4(k), a4(v), lg, s0=s0[None, None]),
                 orc.retention_quadratic(a4(q), a4(k), a4(v), lg, s0=s0[None, None]),
                 orc.retention_chunkwise(a4(q), a4(k), a4(v), lg, 4, s0=s0[None, None])):
        np.testing.assert_allclose(o[0, 0], want, atol=1e-13)


def test_scalar_brute_force_gate_products():
    """Scalar data-dependent decay: what is written at step j reaches step t weighted by
    alpha_{j+1} ... alpha_t (one number per step for the whole memory), and the handed-over
    memory by alpha_1 ... alpha_t; explicit products in pure Python loops (T <= 7)."""
    rng = np.random.default_rng(23)
    T, dk, dv = 7, 3, 2
    q = rng.standard_normal((T, dk)); k = rng.standard_normal((T, dk)); v = rng.standard_normal((T, dv))
    s0 = rng.standard_normal((dv, dk))
    a = rng.uniform(0.2, 0.99, T)
    want = np.zeros((T, dv))
    want_S = np.zeros((dv, dk))
    for t in range(T):
        dec0 = 1.0
        for r in range(t + 1):
            dec0 *= a[r]
        for m in range(dv):
            tot = sum(dec0 * s0[m, c] * q[t, c] for c in range(dk))
            for j in range(t + 1):
                dec = 1.0
                for r in range(j + 1, t + 1):
                    dec *= a[r]
                tot += dec * sum(q[t, c] * k[j, c] for c in range(dk)) * v[j, m]
            want[t, m] = tot
    for m in range(dv):
        for c in range(dk):
            dec0 = 1.0
            for r in range(T):
                dec0 *= a[r]
            tot = dec0 * s0[m, c]
            for j in range(T):
                dec = 1.0
                for r in range(j + 1, T):
                    dec *= a[r]
                tot += dec * v[j, m] * k[j, c]
            want_S[m, c] = tot
    a4 = lambda x: x[None, None]
    la = np.log(a)
    for o, S in (orc.scalar_recurrent(a4(q), a4(k), a4(v), a4(la), s0=s0[None, None]),
                 orc.scalar_quadratic(a4(q), a4(k), a4(v), a4(la), s0=s0[None, None]),
                 orc.scalar_chunkwise(a4(q), a4(k), a4(v), a4(la), 3, s0=s0[None, None])):
        np.testing.assert_allclose(o[0, 0], want, atol=1e-13)
        np.testing.assert_allclose(S[0, 0], want_S, atol=1e-13)


def test_gdelta_brute_force_transition_products():
    """S_t = S_0 M_1 ... M_t + sum_j beta_j v_j k_j^T M_{j+1} ... M_t with
    M_r = alpha_r (I - beta_r k_r k_r^T), the table's transition for Gated DeltaNet."""
    rng = np.random.default_rng(21)
    T, dk, dv = 6, 4, 3
    q = rng.standard_normal((T, dk)); k = rng.standard_normal((T, dk)) / 2
    v = rng.standard_normal((T, dv)); s0 = rng.standard_normal((dv, dk))
    alpha = rng.uniform(0.5, 1.0, T); beta = rng.uniform(0.0, 1.0, T)
    M = [alpha[r] * (np.eye(dk) - beta[r] * np.outer(k[r], k[r])) for r in range(T)]
    want_o = np.zeros((T, dv))
    for t in range(T):
        S = s0.copy()
        for r in range(t + 1):
            S = S @ M[r]
        for j in range(t + 1):
            W = beta[j] * np.outer(v[j], k[j])
            for r in range(j + 1, t + 1):
                W = W @ M[r]
            S = S + W
        want_o[t] = S @ q[t]
    a4 = lambda x: x[None, None]
    la = np.log(alpha)
    for o, _ in (orc.gdelta_recurrent(a4(q), a4(k), a4(v), a4(la), a4(beta), s0=s0[None, None]),
                 orc.gdelta_quadratic(a4(q), a4(k), a4(v), a4(la), a4(beta), s0=s0[None, None]),
                 orc.gdelta_chunkwise(a4(q), a4(k), a4(v), a4(la), a4(beta), 4, s0=s0[None, None])):
        np.testing.assert_allclose(o[0, 0], want_o, atol=1e-13)


def test_decode_step_brute_force():
    """One decode step by hand: S[m, c] * alpha[c] + v[m] k[c], then o[m] = sum_c S[m, c] q[c]."""
    rng = np.random.default_rng(22)
    N, H, dk, dv = 2, 3, 4, 5
    q = rng.standard_normal((N, H, dk)); k = rng.standard_normal((N, H, dk))
    v = rng.standard_normal((N, H, dv)); a = rng.uniform(0.1, 1.0, (N, H, dk))
    s = rng.standard_normal((N, H, dv, dk))
    o, S = orc.decode_step(q, k, v, a, s)
    for n in range(N):
        for h in range(H):
            for m in range(dv):
                row = [s[n, h, m, c] * a[n, h, c] + v[n, h, m] * k[n, h, c] for c in range(dk)]
                assert o[n, h, m] == pytest.approx(sum(row[c] * q[n, h, c] for c in range(dk)), abs=1e-13)
                np.testing.assert_allclose(S[n, h, m], row, atol=1e-15)


def test_gdelta_decode_step_brute_force():
    """One gated-delta decode step by hand: e = sum_c S[m, c] k[c] (what the memory reads
    under k), S_new[m, c] = alpha (S[m, c] - beta e k[c]) + beta v[m] k[c], o[m] = sum_c
    S_new[m, c] q[c]."""
    rng = np.random.default_rng(24)
    N, H, dk, dv = 2, 2, 4, 3
    q = rng.standard_normal((N, H, dk)); k = rng.standard_normal((N, H, dk))
    v = rng.standard_normal((N, H, dv)); a = rng.uniform(0.1, 1.0, (N, H)); b = rng.uniform(0.0, 1.0, (N, H))
    s = rng.standard_normal((N, H, dv, dk))
    o, S = orc.gdelta_decode_step(q, k, v, a, b, s)
    for n in range(N):
        for h in range(H):
            for m in range(dv):
                e = sum(s[n, h, m, c] * k[n, h, c] for c in range(dk))
                row = [a[n, h] * (s[n, h, m, c] - b[n, h] * e * k[n, h, c]) + b[n, h] * v[n, h, m] * k[n, h, c]
                       for c in range(dk)]
                np.testing.assert_allclose(S[n, h, m], row, atol=1e-14)
                assert o[n, h, m] == pytest.approx(sum(row[c] * q[n, h, c] for c in range(dk)), abs=1e-13)


# ----------------------------------------------------------------------------- resume

@pytest.mark.parametrize("split", [0, 1, 7, 16, 33, 40])
def test_resume_from_handed_over_state(split):
    """Only the end-of-block memory passes on: running [0, split) then [split, T) from the
    handed-over state equals one run over [0, T), for every variant."""
    rng, q, k, v, s0 = _rand(30, 2, 2, 40, 8, 6)
    lg = np.log([0.95, 0.7])
    la_d = -np.logaddexp(0.0, -rng.standard_normal(q.shape)) / 4.0
    la_s = -np.logaddexp(0.0, rng.standard_normal(q.shape[:-1])) / 8.0
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal(q.shape[:-1])))
    runs = {
        "scalar": lambda sl, s: orc.scalar_chunkwise(q[..., sl, :], k[..., sl, :], v[..., sl, :], la_s[..., sl], 16,
                                                     s0=s),
        "retention": lambda sl, s: orc.retention_chunkwise(q[..., sl, :], k[..., sl, :], v[..., sl, :], lg, 16, s0=s),
        "gla": lambda sl, s: orc.gla_chunkwise(q[..., sl, :], k[..., sl, :], v[..., sl, :], la_d[..., sl, :], 16, s0=s),
        "gdelta": lambda sl, s: orc.gdelta_chunkwise(q[..., sl, :], k[..., sl, :], v[..., sl, :],
                                                     la_s[..., sl], beta[..., sl], 16, s0=s),
    }
    for name, run in runs.items():
        o_full, S_full = run(slice(0, 40), s0)
        o_a, S_a = run(slice(0, split), s0)
        o_b, S_b = run(slice(split, 40), S_a)
        np.testing.assert_allclose(np.concatenate([o_a, o_b], axis=-2), o_full, atol=1e-12, err_msg=name)
        np.testing.assert_allclose(S_b, S_full, atol=1e-12, err_msg=name)


# ----------------------------------------------------------------------------- backward

def _loss(o, S, W_o, W_s):
    """A fixed random linear functional of the outputs and the final memory: its gradients
    with respect to o and S_T are W_o and W_s."""
    return np.sum(o * W_o) + np.sum(S * W_s)


@pytest.mark.parametrize("kind", ["scalar", "retention", "gla"])
def test_backward_matches_finite_differences(kind):
    """Central differences of L = <W_o, o> + <W_s, S_T> through the recurrent form, against
    the reverse-mode gradients, for every input element (tiny sizes, fp64)."""
    rng = np.random.default_rng(40)
    B, H, T, dk, dv = 1, 2, 5, 3, 2
    q = rng.standard_normal((B, H, T, dk)); k = rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv)); s0 = rng.standard_normal((B, H, dv, dk))
    W_o = rng.standard_normal((B, H, T, dv)); W_s = rng.standard_normal((B, H, dv, dk))
    if kind == "scalar":
        gate = -np.logaddexp(0.0, -rng.standard_normal((B, H, T)))
        fwd = lambda q, k, v, g, s: orc.scalar_recurrent(q, k, v, g, s0=s)
        grads = orc.scalar_backward(q, k, v, gate, W_o, dS_T=W_s, s0=s0)
    elif kind == "gla":
        gate = -np.logaddexp(0.0, -rng.standard_normal((B, H, T, dk)))
        fwd = lambda q, k, v, g, s: orc.gla_recurrent(q, k, v, g, s0=s)
        grads = orc.gla_backward(q, k, v, gate, W_o, dS_T=W_s, s0=s0)
    else:
        gate = np.log(rng.uniform(0.5, 0.95, H))
        fwd = lambda q, k, v, g, s: orc.retention_recurrent(q, k, v, g, s0=s)
        grads = orc.retention_backward(q, k, v, gate, W_o, dS_T=W_s, s0=s0)
    args = [q, k, v, gate, s0]
    eps = 1e-6
    for which, g in zip(range(5), grads):
        x = args[which]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            plus = [a.copy() for a in args]; minus = [a.copy() for a in args]
            plus[which][idx] += eps; minus[which][idx] -= eps
            num[idx] = (_loss(*fwd(*plus), W_o, W_s) - _loss(*fwd(*minus), W_o, W_s)) / (2 * eps)
        np.testing.assert_allclose(g, num, atol=1e-7, rtol=1e-6, err_msg=f"{kind} input {which}")


def test_gdelta_backward_matches_finite_differences():
    """Central differences of L = <W_o, o> + <W_s, S_T> through the gated delta rule's
    recurrent form, against the reverse-mode gradients, for every element of q, k, v, log
    alpha, beta and S_0 (tiny sizes, fp64; keys not normalised, so every term of the
    transition is exercised)."""
    rng = np.random.default_rng(43)
    B, H, T, dk, dv = 1, 2, 5, 3, 2
    q = rng.standard_normal((B, H, T, dk)); k = rng.standard_normal((B, H, T, dk)) * 0.7
    v = rng.standard_normal((B, H, T, dv)); s0 = rng.standard_normal((B, H, dv, dk))
    la = -np.logaddexp(0.0, -rng.standard_normal((B, H, T)))
    be = rng.uniform(0.2, 0.9, (B, H, T))
    W_o = rng.standard_normal((B, H, T, dv)); W_s = rng.standard_normal((B, H, dv, dk))
    grads = orc.gdelta_backward(q, k, v, la, be, W_o, dS_T=W_s, s0=s0)
    args = [q, k, v, la, be, s0]
    fwd = lambda q, k, v, la, be, s: orc.gdelta_recurrent(q, k, v, la, be, s0=s)
    eps = 1e-6
    for which, g in enumerate(grads):
        x = args[which]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            plus = [a.copy() for a in args]; minus = [a.copy() for a in args]
            plus[which][idx] += eps; minus[which][idx] -= eps
            num[idx] = (_loss(*fwd(*plus), W_o, W_s) - _loss(*fwd(*minus), W_o, W_s)) / (2 * eps)
        np.testing.assert_allclose(g, num, atol=1e-7, rtol=1e-6, err_msg=f"gdelta input {which}")


def test_gdelta_backward_without_writes_is_the_scalar_fade():
    """beta = 0: nothing is written (S_t = a_t S_{t-1}), which is the scalar decay with v = 0;
    dq, d log a and dS_0 equal the scalar-decay gradients at v = 0, and dk, dv are zero."""
    rng = np.random.default_rng(44)
    B, H, T, dk, dv = 2, 2, 9, 4, 3
    q = rng.standard_normal((B, H, T, dk)); k = rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv)); s0 = rng.standard_normal((B, H, dv, dk))
    la = -np.logaddexp(0.0, -rng.standard_normal((B, H, T)))
    do = rng.standard_normal((B, H, T, dv)); dS = rng.standard_normal((B, H, dv, dk))
    gd = orc.gdelta_backward(q, k, v, la, np.zeros((B, H, T)), do, dS_T=dS, s0=s0)
    sc = orc.scalar_backward(q, k, np.zeros_like(v), la, do, dS_T=dS, s0=s0)
    np.testing.assert_allclose(gd[0], sc[0], atol=1e-12)      # dq
    np.testing.assert_allclose(gd[3], sc[3], atol=1e-12)      # d log a
    np.testing.assert_allclose(gd[5], sc[4], atol=1e-12)      # dS_0
    np.testing.assert_array_equal(gd[1], 0.0)
    np.testing.assert_array_equal(gd[2], 0.0)


def test_gdelta_backward_gate_gradient_identity():
    """S_0 enters the recurrence only through the first fade a_0 S_0, so scaling S_0 by e^eps
    and shifting log a_0 by eps change the loss alike: d log a_0 = <dS_0, S_0> (Frobenius),
    for any beta."""
    rng = np.random.default_rng(45)
    B, H, T, dk, dv = 1, 1, 6, 3, 2
    q = rng.standard_normal((B, H, T, dk)); k = rng.standard_normal((B, H, T, dk)) * 0.6
    v = rng.standard_normal((B, H, T, dv)); s0 = rng.standard_normal((B, H, dv, dk))
    la = -np.logaddexp(0.0, -rng.standard_normal((B, H, T))); be = rng.uniform(0.1, 0.9, (B, H, T))
    do = rng.standard_normal((B, H, T, dv))
    grads = orc.gdelta_backward(q, k, v, la, be, do, s0=s0)
    # at t = 0: scaling S_0 by e^eps is the same as shifting log a_0 by eps
    np.testing.assert_allclose(grads[3][..., 0], np.sum(grads[5] * s0, axis=(-2, -1)), rtol=1e-10, atol=1e-12)


def test_gate_gradient_identity():
    """The gate gradient from the rescaling argument: every term of o_t carries e^(B_t) and
    every term written at j carries e^(-B_j), so dL/dB_t = q_t . dq_t - k_t . dk_t (plus
    <dS_T, S_T> at the last token), and d log a_r = sum_{t >= r} dL/dB_t."""
    rng = np.random.default_rng(41)
    B, H, T, dk, dv = 2, 2, 9, 4, 3
    q = rng.standard_normal((B, H, T, dk)); k = rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv)); s0 = rng.standard_normal((B, H, dv, dk))
    la = -np.logaddexp(0.0, -rng.standard_normal((B, H, T)))
    do = rng.standard_normal((B, H, T, dv)); dS = rng.standard_normal((B, H, dv, dk))
    dq, dk_, dv_, dla, _ = orc.scalar_backward(q, k, v, la, do, dS_T=dS, s0=s0)
    _, S_T = orc.scalar_recurrent(q, k, v, la, s0=s0)
    per_t = np.sum(q * dq, axis=-1) - np.sum(k * dk_, axis=-1)
    want = np.flip(np.cumsum(np.flip(per_t, -1), -1), -1) + np.sum(dS * S_T, axis=(-2, -1))[..., None]
    np.testing.assert_allclose(dla, want, atol=1e-10)


def test_gla_gate_gradient_identity():
    """Per key channel the same rescaling argument holds: a shift of log a_r[c] equals scaling
    channel c of q_s by e^eps and of k_s by e^-eps for s >= r, and column c of S_T by e^eps, so
    d log a_r[c] = sum_{t >= r} (q_t[c] dq_t[c] - k_t[c] dk_t[c]) + sum_m dS_T[m, c] S_T[m, c]."""
    rng = np.random.default_rng(42)
    B, H, T, dk, dv = 2, 1, 8, 5, 3
    q = rng.standard_normal((B, H, T, dk)); k = rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv)); s0 = rng.standard_normal((B, H, dv, dk))
    la = -np.logaddexp(0.0, -rng.standard_normal((B, H, T, dk)))
    do = rng.standard_normal((B, H, T, dv)); dS = rng.standard_normal((B, H, dv, dk))
    dq, dk_, dv_, dla, _ = orc.gla_backward(q, k, v, la, do, dS_T=dS, s0=s0)
    _, S_T = orc.gla_recurrent(q, k, v, la, s0=s0)
    per_t = q * dq - k * dk_
    want = np.flip(np.cumsum(np.flip(per_t, 2), 2), 2) + np.sum(dS * S_T, axis=-2)[..., None, :]
    np.testing.assert_allclose(dla, want, atol=1e-10)


def test_gla_backward_with_shared_gate_is_scalar_backward():
    """A per-channel gate that is the same on every channel is the scalar decay: the GLA
    gradients equal the scalar-decay ones, and the channel gate gradients sum to the scalar
    gate gradient."""
    rng = np.random.default_rng(43)
    B, H, T, dk, dv = 1, 2, 7, 4, 3
    q = rng.standard_normal((B, H, T, dk)); k = rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv)); s0 = rng.standard_normal((B, H, dv, dk))
    la = -np.logaddexp(0.0, -rng.standard_normal((B, H, T)))
    do = rng.standard_normal((B, H, T, dv)); dS = rng.standard_normal((B, H, dv, dk))
    g = orc.gla_backward(q, k, v, np.repeat(la[..., None], dk, axis=-1), do, dS_T=dS, s0=s0)
    s = orc.scalar_backward(q, k, v, la, do, dS_T=dS, s0=s0)
    for a, b in zip(g[:3], s[:3]):
        np.testing.assert_allclose(a, b, atol=1e-12)
    np.testing.assert_allclose(g[3].sum(axis=-1), s[3], atol=1e-12)
    np.testing.assert_allclose(g[4], s[4], atol=1e-12)
