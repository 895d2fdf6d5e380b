"""Pins of the fp64 oracle against what the pages and the mathematics fix.

Each test ties an oracle function to something other than itself: numbers the
pages print (golden fixtures, cited there), closed forms of special cases,
invariants the pages state, or an independent derivation written out here.
A plausible slip in the oracle (a dropped decay, a gate on the wrong side,
reading before writing, a sign in the delta correction, a wrong triangular
solve) fails at least one of them.
"""

import json
import os

import numpy as np
import pytest

import oracle as orc


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _scalar_seq(values):
    """Shape [1, 1, T, 1] arrays for the one-channel examples."""
    return np.asarray(values, dtype=np.float64).reshape(1, 1, -1, 1)


# ----------------------------------------------------------------------------- worked example

def test_worked_example_three_forms(golden_dir):
    """RetNet page, Fig. 16.5: scores 6, 7, 8 with the total halved at each step give the
    running totals 6, 10, 13 in the parallel, recurrent and block-of-two forms."""
    g = _load(golden_dir, "retention_worked_example.json")
    v = _scalar_seq(g["scores"])
    ones = np.ones_like(v)
    lg = np.array([np.log(g["decay"])])
    want = np.array(g["running_totals"], dtype=np.float64)
    o_rec, _ = orc.retention_recurrent(ones, ones, v, lg)
    o_par, _ = orc.retention_quadratic(ones, ones, v, lg)
    o_chk, _ = orc.retention_chunkwise(ones, ones, v, lg, chunk=g["block"])
    for o in (o_rec, o_par, o_chk):
        np.testing.assert_allclose(o.reshape(-1), want, rtol=0, atol=1e-12)


def test_worked_example_gla_and_decode(golden_dir):
    """The same example through the diagonal gate (one channel, gate 1/2 every step) in all
    three GLA forms, and through three single-token decode steps."""
    g = _load(golden_dir, "retention_worked_example.json")
    v = _scalar_seq(g["scores"])
    ones = np.ones_like(v)
    la = np.full_like(v, np.log(g["decay"]))
    want = np.array(g["running_totals"], dtype=np.float64)
    for o, _ in (orc.gla_recurrent(ones, ones, v, la),
                 orc.gla_quadratic(ones, ones, v, la),
                 orc.gla_chunkwise(ones, ones, v, la, chunk=g["block"])):
        np.testing.assert_allclose(o.reshape(-1), want, atol=1e-12)
    S = np.zeros((1, 1, 1, 1))
    got = []
    for t, score in enumerate(g["scores"]):
        one = np.ones((1, 1, 1))
        o, S = orc.decode_step(one, one, np.full((1, 1, 1), score), np.full((1, 1, 1), g["decay"]), S)
        got.append(o.item())
    np.testing.assert_allclose(got, want, atol=1e-12)


# ----------------------------------------------------------------------------- decay powers

@pytest.mark.parametrize("form", ["recurrent", "quadratic", "chunkwise"])
def test_decay_powers(golden_dir, form):
    """An impulse written at step 0 reads back gamma^t at step t: 0.9^10 ~ 0.35,
    0.9^50 ~ 0.005, 0.9^100 ~ 2.7e-5 (to the printed digits), and the halving
    filter taps 1, 0.5, 0.25, 0.125."""
    g = _load(golden_dir, "decay_powers.json")
    T = 101
    k = np.zeros((1, 1, T, 1)); k[0, 0, 0, 0] = 1.0
    v = k.copy()
    q = np.ones((1, 1, T, 1))

    def run(gamma):
        lg = np.array([np.log(gamma)])
        if form == "recurrent":
            return orc.retention_recurrent(q, k, v, lg)[0].reshape(-1)
        if form == "quadratic":
            return orc.retention_quadratic(q, k, v, lg)[0].reshape(-1)
        return orc.retention_chunkwise(q, k, v, lg, chunk=16)[0].reshape(-1)

    o = run(0.9)
    assert round(o[10], g["printed_digits"]["10"]) == g["gamma_0_9"]["10"]
    assert round(o[50], g["printed_digits"]["50"]) == g["gamma_0_9"]["50"]
    assert float(f"{o[100]:.1e}") == g["gamma_0_9"]["100"]
    o = run(0.5)
    np.testing.assert_allclose(o[:4], g["halving_taps"], atol=1e-15)


# ----------------------------------------------------------------------------- recall table

def _recall_experiment(N, d, trials, seed):
    """The pages' recall experiment, the memory written and updated by the oracle.

    Accumulation is retention with no decay (gamma = 1); the delta rule is the gated
    delta rule with no decay (alpha = 1) and full write strength (beta = 1)."""
    rng = np.random.default_rng(seed)
    Ks = np.empty((trials, N, d)); Vs = np.empty((trials, N, d)); vn = np.empty((trials, d))
    for t in range(trials):
        K = rng.standard_normal((N, d))
        Ks[t] = K / np.linalg.norm(K, axis=1, keepdims=True)
        Vs[t] = rng.standard_normal((N, d))
        vn[t] = rng.standard_normal(d)
    q = np.zeros((trials, 1, N, d))
    K4, V4 = Ks[:, None], Vs[:, None]
    zeros_t = np.zeros((trials, 1, N))
    ones_t = np.ones((trials, 1, N))
    out = {}
    for rule in ("sum", "delta"):
        if rule == "sum":
            _, S = orc.retention_recurrent(q, K4, V4, np.zeros(1))
        else:
            _, S = orc.gdelta_recurrent(q, K4, V4, zeros_t, ones_t)
        S = S[:, 0]                                           # [trials, d, d]
        read = np.einsum("tmc,tnc->tnm", S, Ks)               # S k_i for every key
        recall = (np.linalg.norm(read - Vs, axis=2) / np.linalg.norm(Vs, axis=2)).mean(axis=1)
        k0 = Ks[:, None, None, 0, :]                          # [trials,1,1,d]
        v_new = vn[:, None, None, :]
        s0 = S[:, None]
        if rule == "sum":
            o, _ = orc.retention_recurrent(k0, k0, v_new, np.zeros(1), s0=s0)
        else:
            o, _ = orc.gdelta_recurrent(k0, k0, v_new, np.zeros((trials, 1, 1)),
                                        np.ones((trials, 1, 1)), s0=s0)
        rewrite = np.linalg.norm(o[:, 0, 0] - vn, axis=1) / np.linalg.norm(vn, axis=1)
        out[rule] = (recall.mean(), rewrite.mean())
    return out


def test_recall_error_table(golden_dir):
    """The recall / rewrite errors printed under the pages' experiment (d = 32, 2000
    trials, seed 0) come out of the oracle's accumulation and delta steps to the
    printed two decimals."""
    g = _load(golden_dir, "recall_error_table.json")
    s = g["setup"]
    for row in g["rows"]:
        r = _recall_experiment(row["N"], s["d"], s["trials"], s["seed"])
        assert round(r["sum"][0], 2) == row["recall_sum"], (row, r)
        assert round(r["delta"][0], 2) == row["recall_delta"], (row, r)
        assert round(r["sum"][1], 2) == row["rewrite_sum"], (row, r)
        assert round(r["delta"][1], 2) == row["rewrite_delta"], (row, r)


# ----------------------------------------------------------------------------- delta rule

def _one_delta_step(read_before, target, beta, key):
    """A one-channel memory that currently reads ``read_before`` under ``key``: write
    ``target`` with strength ``beta``; return what it reads afterwards."""
    s0 = np.full((1, 1, 1, 1), read_before / key)
    kk = np.full((1, 1, 1, 1), key)
    o, S = orc.gdelta_recurrent(kk, kk, np.full((1, 1, 1, 1), target),
                                np.zeros((1, 1, 1)), np.full((1, 1, 1), beta), s0=s0)
    return o.item(), S


def test_mario_ledger():
    """"Correggere: la delta rule", the ledger: it reads 7 where 10 is right. Half dose
    gives 8.5 (also as erasing half of 7 and writing half of 10), full dose 10, zero
    dose 7; a key of double weight (beta |k|^2 = 2) swings 7 -> 13 -> 7 for ever."""
    assert _one_delta_step(7.0, 10.0, 0.5, 1.0)[0] == pytest.approx(8.5, abs=1e-14)
    assert 0.5 * 7.0 + 0.5 * 10.0 == 8.5
    assert _one_delta_step(7.0, 10.0, 1.0, 1.0)[0] == pytest.approx(10.0, abs=1e-14)
    assert _one_delta_step(7.0, 10.0, 0.0, 1.0)[0] == pytest.approx(7.0, abs=1e-14)
    read = 7.0
    seen = []
    for _ in range(4):
        read, _ = _one_delta_step(read, 10.0, 1.0, np.sqrt(2.0))
        seen.append(read)
    np.testing.assert_allclose(seen, [13.0, 7.0, 13.0, 7.0], atol=1e-12)


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("form", ["recurrent", "quadratic", "chunkwise"])
def test_delta_overwrite_reads_back_value(form, gated):
    """With beta = 1 and unit keys the entry under k_t is overwritten: S_t k_t = v_t
    ("Correggere: la delta rule"); the decay does not change it, since
    alpha S (I - k k^T) k = 0. Reading with q_t = k_t therefore returns v_t exactly."""
    rng = np.random.default_rng(11)
    B, H, T, d = 2, 2, 37, 16
    k = rng.standard_normal((B, H, T, d)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, H, T, d))
    la = (np.log(rng.uniform(0.5, 1.0, (B, H, T))) if gated else np.zeros((B, H, T)))
    beta = np.ones((B, H, T))
    s0 = rng.standard_normal((B, H, d, d))
    if form == "recurrent":
        o, S = orc.gdelta_recurrent(k, k, v, la, beta, s0=s0)
    elif form == "quadratic":
        o, S = orc.gdelta_quadratic(k, k, v, la, beta, s0=s0)
    else:
        o, S = orc.gdelta_chunkwise(k, k, v, la, beta, chunk=8, s0=s0)
    np.testing.assert_allclose(o, v, atol=1e-11)
    np.testing.assert_allclose(np.einsum("bhmc,bhc->bhm", S, k[:, :, -1]), v[:, :, -1], atol=1e-11)


def test_gdelta_decode_step_pins():
    """The gated-delta decode step: (a) with beta = 1 and a unit key, the entry under k is
    overwritten whatever the gate, S_new k = v ("Correggere: la delta rule"); (b) beta = 0
    only fades the memory, S_new = alpha S ("Unire oblio e correzione"); (c) alpha = 1 and
    beta = 1/2 with a unit key halves the error under k; (d) T steps of it give the
    recurrent form of the chunked variant, token by token."""
    rng = np.random.default_rng(16)
    N, H, dk, dv = 3, 2, 8, 5
    s = rng.standard_normal((N, H, dv, dk))
    k = rng.standard_normal((N, H, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q = rng.standard_normal((N, H, dk)); v = rng.standard_normal((N, H, dv))
    a = rng.uniform(0.3, 1.0, (N, H))
    o, S = orc.gdelta_decode_step(q, k, v, a, np.ones((N, H)), s)
    np.testing.assert_allclose(np.einsum("nhmc,nhc->nhm", S, k), v, atol=1e-12)
    np.testing.assert_allclose(o, np.einsum("nhmc,nhc->nhm", S, q), atol=1e-12)
    _, S = orc.gdelta_decode_step(q, k, v, a, np.zeros((N, H)), s)
    np.testing.assert_allclose(S, a[..., None, None] * s, atol=1e-12)
    _, S = orc.gdelta_decode_step(q, k, v, np.ones((N, H)), np.full((N, H), 0.5), s)
    err_old = v - np.einsum("nhmc,nhc->nhm", s, k)
    err_new = v - np.einsum("nhmc,nhc->nhm", S, k)
    np.testing.assert_allclose(err_new, 0.5 * err_old, atol=1e-12)
    T = 6
    qs = rng.standard_normal((1, 1, T, dk)); ks = rng.standard_normal((1, 1, T, dk)) / 2
    vs = rng.standard_normal((1, 1, T, dv))
    la = np.log(rng.uniform(0.4, 1.0, (1, 1, T))); be = rng.uniform(0.0, 1.0, (1, 1, T))
    s0 = rng.standard_normal((1, 1, dv, dk))
    o_rec, S_rec = orc.gdelta_recurrent(qs, ks, vs, la, be, s0=s0)
    S = s0[:, :, None].repeat(1, axis=2)[:, :, 0]
    for t in range(T):
        o_t, S = orc.gdelta_decode_step(qs[:, :, t], ks[:, :, t], vs[:, :, t], np.exp(la[:, :, t]),
                                        be[:, :, t], S)
        np.testing.assert_allclose(o_t, o_rec[:, :, t], atol=1e-12)
    np.testing.assert_allclose(S, S_rec, atol=1e-12)


def test_silu_l2_and_rms_norm():
    """The feature map and the output norm against their definitions at points where the
    answer is known: SiLU(0) = 0, SiLU(x) -> x for large x and -> 0 for very negative x,
    SiLU(1) = 1 / (1 + 1/e); every mapped row has unit L2 norm and keeps the direction of
    SiLU(x); a row that SiLU sends to zero stays zero. RMS norm: unit root mean square
    with unit weight, invariant to scaling the row, the weight multiplies channel by
    channel, and eps only matters for tiny rows."""
    x = np.array([[0.0, 30.0, -30.0, 1.0]])
    y = orc.silu_l2(x)
    silu = np.array([0.0, 30.0, -30.0 * np.exp(-30.0) / (1.0 + np.exp(-30.0)), 1.0 / (1.0 + np.exp(-1.0))])
    np.testing.assert_allclose(y[0], silu / np.linalg.norm(silu), rtol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(y), 1.0, rtol=1e-14)
    rng = np.random.default_rng(17)
    x = rng.standard_normal((3, 5, 16))
    y = orc.silu_l2(x)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), 1.0, rtol=1e-13)
    s = x / (1.0 + np.exp(-x))
    cos = np.sum(y * s, axis=-1) / np.linalg.norm(s, axis=-1)
    np.testing.assert_allclose(cos, 1.0, rtol=1e-13)
    np.testing.assert_array_equal(orc.silu_l2(np.zeros((2, 8))), 0.0)
    o = rng.standard_normal((4, 7, 32)) * 3.0
    r = orc.rms_norm(o, np.ones(32), 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean(r * r, axis=-1)), 1.0, rtol=1e-13)
    np.testing.assert_allclose(orc.rms_norm(5.0 * o, np.ones(32), 0.0), r, rtol=1e-13)
    w = rng.uniform(0.5, 2.0, 32)
    np.testing.assert_allclose(orc.rms_norm(o, w, 0.0), r * w, rtol=1e-13)
    np.testing.assert_allclose(orc.rms_norm(o, np.ones(32), 1e-12), r, rtol=1e-9)
    tiny = np.full((1, 32), 1e-4)
    np.testing.assert_allclose(orc.rms_norm(tiny, np.ones(32), 1e-6), tiny / np.sqrt(1e-8 + 1e-6), rtol=1e-13)


def test_layer_norm():
    """GLA's output norm against its definition: a hand-worked row (x = 1, 2, 3, 4: mean 2.5,
    population variance 1.25, so the normalised row is (x - 2.5) / sqrt(1.25)); with unit
    weight, zero bias and eps = 0 every row has mean 0 and mean square 1; adding a constant
    or multiplying by a positive factor leaves the row unchanged; a negative factor flips
    its sign; weight and bias act channel by channel after the normalisation; a constant
    row becomes the bias (its deviation is 0); eps enters as sqrt(var + eps)."""
    y = orc.layer_norm(np.array([[1.0, 2.0, 3.0, 4.0]]), np.ones(4), None, 0.0)
    np.testing.assert_allclose(y[0], np.array([-1.5, -0.5, 0.5, 1.5]) / np.sqrt(1.25), rtol=1e-14)
    np.testing.assert_allclose(y[0], [-1.3416407864998738, -0.4472135954999579, 0.4472135954999579,
                                      1.3416407864998738], rtol=1e-14)
    rng = np.random.default_rng(18)
    o = rng.standard_normal((4, 7, 64)) * 3.0 + 1.5
    r = orc.layer_norm(o, np.ones(64), np.zeros(64), 0.0)
    np.testing.assert_allclose(np.mean(r, axis=-1), 0.0, atol=1e-13)
    np.testing.assert_allclose(np.mean(r * r, axis=-1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(orc.layer_norm(o + 7.0, np.ones(64), None, 0.0), r, atol=1e-12)
    np.testing.assert_allclose(orc.layer_norm(0.25 * o, np.ones(64), None, 0.0), r, atol=1e-12)
    np.testing.assert_allclose(orc.layer_norm(-2.0 * o, np.ones(64), None, 0.0), -r, atol=1e-12)
    w, b = rng.uniform(0.5, 2.0, 64), rng.standard_normal(64)
    np.testing.assert_allclose(orc.layer_norm(o, w, b, 0.0), r * w + b, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(orc.layer_norm(np.full((2, 64), 3.0), w, b, 1e-5), np.broadcast_to(b, (2, 64)),
                               atol=1e-15)
    x = np.array([[0.0, 2.0]])   # mean 1, variance 1
    np.testing.assert_allclose(orc.layer_norm(x, np.ones(2), None, 3.0)[0], np.array([-1.0, 1.0]) / 2.0, rtol=1e-14)


def test_transition_eigenvalues_and_norm():
    """The transition I - beta k k^T has eigenvalues 1 (d-1 times) and 1 - beta |k|^2; its
    spectral norm is exactly 1 when 0 <= beta |k|^2 <= 2; Gated DeltaNet scales it by
    alpha. Obtained from the oracle as the memory one step after S_0 = I with v = 0."""
    rng = np.random.default_rng(5)
    d = 12
    for alpha, beta, knorm in [(1.0, 0.7, 1.0), (1.0, 1.0, 1.0), (0.8, 0.35, 1.3), (1.0, 0.5, 1.9)]:
        k = rng.standard_normal(d); k *= knorm / np.linalg.norm(k)
        kk = k.reshape(1, 1, 1, d)
        M = orc.gdelta_recurrent(np.zeros((1, 1, 1, d)), kk, np.zeros((1, 1, 1, d)),
                                 np.full((1, 1, 1), np.log(alpha)), np.full((1, 1, 1), beta),
                                 s0=np.eye(d).reshape(1, 1, d, d))[1][0, 0]
        ev = np.sort(np.linalg.eigvalsh((M + M.T) / 2))
        want = np.sort(np.r_[np.full(d - 1, alpha), alpha * (1 - beta * knorm ** 2)])
        np.testing.assert_allclose(ev, want, atol=1e-13)
        if alpha == 1.0 and beta * knorm ** 2 <= 2:
            assert np.linalg.norm(M, 2) == pytest.approx(1.0, abs=1e-13)


def test_transitions_multiply_from_the_right():
    """Gate and delta transition act on key channels (columns): one step from S_0 = M with
    no write gives M Diag(alpha) for GLA and M alpha (I - beta k k^T) for the gated delta
    rule, not the left products ("Dimenticare: i gate", on the side of the product)."""
    rng = np.random.default_rng(6)
    dv, dk = 5, 7
    M = rng.standard_normal((dv, dk))
    a = rng.uniform(0.2, 0.9, dk)
    _, S = orc.gla_recurrent(np.zeros((1, 1, 1, dk)), np.zeros((1, 1, 1, dk)), np.zeros((1, 1, 1, dv)),
                             np.log(a).reshape(1, 1, 1, dk), s0=M.reshape(1, 1, dv, dk))
    np.testing.assert_allclose(S[0, 0], M @ np.diag(a), atol=1e-15)
    k = rng.standard_normal(dk)
    alpha, beta = 0.9, 0.6
    _, S = orc.gdelta_recurrent(np.zeros((1, 1, 1, dk)), k.reshape(1, 1, 1, dk), np.zeros((1, 1, 1, dv)),
                                np.full((1, 1, 1), np.log(alpha)), np.full((1, 1, 1), beta),
                                s0=M.reshape(1, 1, dv, dk))
    np.testing.assert_allclose(S[0, 0], M @ (alpha * (np.eye(dk) - beta * np.outer(k, k))), atol=1e-14)


def test_gla_gate_extremes_per_column():
    """alpha_{t,c} -> 1 keeps column c (pure accumulation there), alpha_{t,c} -> 0 clears it
    before the write ("Dimenticare: i gate"). The zero gate is taken as e^-60, the limit
    the sigmoid never reaches."""
    rng = np.random.default_rng(7)
    T, d = 9, 6
    q = rng.standard_normal((1, 1, T, d)); k = rng.standard_normal((1, 1, T, d))
    v = rng.standard_normal((1, 1, T, d))
    la = np.log(rng.uniform(0.3, 0.9, (1, 1, T, d)))
    la[..., 1] = 0.0          # gate 1 on channel 1
    la[..., 4] = -60.0        # gate e^-60 ~ 1e-26 on channel 4: numerically zero
    for fn in (lambda: orc.gla_recurrent(q, k, v, la),
               lambda: orc.gla_chunkwise(q, k, v, la, chunk=4)):
        _, S = fn()
        np.testing.assert_allclose(S[0, 0, :, 1], (v[0, 0].T @ k[0, 0, :, 1]), atol=1e-13)
        np.testing.assert_allclose(S[0, 0, :, 4], v[0, 0, -1] * k[0, 0, -1, 4], atol=1e-13)


def test_beta_zero_only_fades():
    """beta -> 0 switches the write off together with the correction: S_t = alpha_t S_{t-1},
    not the scalar-decay-plus-write row ("Unire oblio e correzione")."""
    rng = np.random.default_rng(8)
    B, H, T, d = 1, 2, 13, 8
    q = rng.standard_normal((B, H, T, d)); k = rng.standard_normal((B, H, T, d))
    v = rng.standard_normal((B, H, T, d))
    la = np.log(rng.uniform(0.6, 1.0, (B, H, T)))
    s0 = rng.standard_normal((B, H, d, d))
    G = np.cumsum(la, axis=-1)
    want_o = np.exp(G)[..., None] * np.einsum("bhmc,bhtc->bhtm", s0, q)
    for o, S in (orc.gdelta_recurrent(q, k, v, la, np.zeros((B, H, T)), s0=s0),
                 orc.gdelta_chunkwise(q, k, v, la, np.zeros((B, H, T)), chunk=4, s0=s0)):
        np.testing.assert_allclose(o, want_o, atol=1e-12)
        np.testing.assert_allclose(S, np.exp(G[..., -1])[..., None, None] * s0, atol=1e-12)


def test_alpha_one_is_deltanet_pseudo_values():
    """alpha -> 1 recovers DeltaNet, whose memory the pages write as a sum of pseudo-values
    S_t = sum_{i<=t} u_i k_i^T with u_t = beta_t (v_t - sum_{i<t} u_i (k_i . k_t))
    ("Correggere: la delta rule"); that recursion is written out here independently."""
    rng = np.random.default_rng(9)
    T, dk, dv = 21, 8, 5
    q = rng.standard_normal((T, dk)); k = rng.standard_normal((T, dk)) / np.sqrt(dk)
    v = rng.standard_normal((T, dv)); beta = rng.uniform(0.1, 0.9, T)
    u = np.zeros((T, dv))
    for t in range(T):
        acc = v[t].copy()
        for i in range(t):
            acc -= u[i] * (k[i] @ k[t])
        u[t] = beta[t] * acc
    want_o = np.array([sum(u[i] * (k[i] @ q[t]) for i in range(t + 1)) for t in range(T)])
    want_S = sum(np.outer(u[i], k[i]) for i in range(T))
    a = lambda x: x[None, None]
    for o, S in (orc.gdelta_recurrent(a(q), a(k), a(v), np.zeros((1, 1, T)), a(beta)),
                 orc.gdelta_quadratic(a(q), a(k), a(v), np.zeros((1, 1, T)), a(beta)),
                 orc.gdelta_chunkwise(a(q), a(k), a(v), np.zeros((1, 1, T)), a(beta), chunk=6)):
        np.testing.assert_allclose(o[0, 0], want_o, atol=1e-12)
        np.testing.assert_allclose(S[0, 0], want_S, atol=1e-12)


def test_delta_step_is_gradient_step():
    """One delta-rule step is one gradient step of l(S) = 1/2 |S k - v|^2 with learning rate
    beta ("Le ricorrenze come regressione online"); the gradient here is taken by central
    finite differences, independently of the closed form."""
    rng = np.random.default_rng(10)
    dv, dk = 4, 6
    S0 = rng.standard_normal((dv, dk)); k = rng.standard_normal(dk); v = rng.standard_normal(dv)
    beta = 0.37
    loss = lambda S: 0.5 * np.sum((S @ k - v) ** 2)
    h = 1e-6
    grad = np.zeros_like(S0)
    for m in range(dv):
        for c in range(dk):
            E = np.zeros_like(S0); E[m, c] = h
            grad[m, c] = (loss(S0 + E) - loss(S0 - E)) / (2 * h)
    want = S0 - beta * grad
    _, S = orc.gdelta_recurrent(np.zeros((1, 1, 1, dk)), k.reshape(1, 1, 1, dk), v.reshape(1, 1, 1, dv),
                                np.zeros((1, 1, 1)), np.full((1, 1, 1), beta), s0=S0.reshape(1, 1, dv, dk))
    np.testing.assert_allclose(S[0, 0], want, atol=1e-8)


def test_accumulation_vs_delta_orthonormal_keys():
    """Accumulation equals the delta step only when S_{t-1} k_t = 0 and beta = 1: with
    orthonormal keys from an empty memory the two agree at beta = 1 and differ by a
    factor of two already at the first token at beta = 0.5."""
    rng = np.random.default_rng(12)
    d = 8
    K, _ = np.linalg.qr(rng.standard_normal((d, d)))
    K = K.T.reshape(1, 1, d, d)                    # rows are orthonormal keys
    V = rng.standard_normal((1, 1, d, d)); Q = rng.standard_normal((1, 1, d, d))
    o_sum, S_sum = orc.retention_recurrent(Q, K, V, np.zeros(1))
    o_del, S_del = orc.gdelta_recurrent(Q, K, V, np.zeros((1, 1, d)), np.ones((1, 1, d)))
    np.testing.assert_allclose(o_del, o_sum, atol=1e-13)
    np.testing.assert_allclose(S_del, S_sum, atol=1e-13)
    _, S1_sum = orc.retention_recurrent(Q[..., :1, :], K[..., :1, :], V[..., :1, :], np.zeros(1))
    _, S1_del = orc.gdelta_recurrent(Q[..., :1, :], K[..., :1, :], V[..., :1, :],
                                     np.zeros((1, 1, 1)), np.full((1, 1, 1), 0.5))
    np.testing.assert_allclose(S1_sum, 2.0 * S1_del, atol=1e-14)


def test_gla_constant_gate_is_retention():
    """A diagonal gate with every channel at gamma is the scalar decay (GLA's hierarchy:
    fixed scalar -> data-dependent scalar -> diagonal)."""
    rng = np.random.default_rng(13)
    B, H, T, dk, dv = 2, 3, 19, 5, 4
    q = rng.standard_normal((B, H, T, dk)); k = rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv))
    lg = np.log(np.array([0.5, 0.9, 0.99]))
    la = np.broadcast_to(lg[None, :, None, None], (B, H, T, dk))
    o_r, S_r = orc.retention_recurrent(q, k, v, lg)
    o_g, S_g = orc.gla_recurrent(q, k, v, la)
    np.testing.assert_allclose(o_g, o_r, atol=1e-12)
    np.testing.assert_allclose(S_g, S_r, atol=1e-12)


def test_scalar_gate_special_cases(golden_dir):
    """The scalar data-dependent decay against the rows it sits between in the pages'
    hierarchy (fixed scalar -> data-dependent scalar -> diagonal): a gate that is the
    same at every step is retention; the same gate copied into every key channel is GLA;
    alpha = 1 is pure accumulation, S_T = S_0 + sum_j v_j k_j^T; and the worked example of
    the RetNet page (scores 6, 7, 8, total halved each step) gives 6, 10, 13."""
    rng = np.random.default_rng(15)
    B, H, T, dk, dv = 2, 3, 21, 5, 4
    q = rng.standard_normal((B, H, T, dk)); k = rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv)); s0 = rng.standard_normal((B, H, dv, dk))
    lg = np.log(np.array([0.5, 0.9, 0.99]))
    la_const = np.broadcast_to(lg[None, :, None], (B, H, T))
    o_r, S_r = orc.retention_recurrent(q, k, v, lg, s0=s0)
    for fn in (orc.scalar_recurrent, orc.scalar_quadratic):
        o_s, S_s = fn(q, k, v, la_const, s0=s0)
        np.testing.assert_allclose(o_s, o_r, atol=1e-12)
        np.testing.assert_allclose(S_s, S_r, atol=1e-12)
    la = -np.logaddexp(0.0, -rng.standard_normal((B, H, T)))
    o_g, S_g = orc.gla_recurrent(q, k, v, np.broadcast_to(la[..., None], (B, H, T, dk)), s0=s0)
    o_s, S_s = orc.scalar_chunkwise(q, k, v, la, 8, s0=s0)
    np.testing.assert_allclose(o_s, o_g, atol=1e-12)
    np.testing.assert_allclose(S_s, S_g, atol=1e-12)
    _, S_acc = orc.scalar_chunkwise(q, k, v, np.zeros((B, H, T)), 8, s0=s0)
    np.testing.assert_allclose(S_acc, s0 + np.einsum("bhtm,bhtc->bhmc", v, k), atol=1e-12)
    g = _load(golden_dir, "retention_worked_example.json")
    sv = _scalar_seq(g["scores"])
    ones = np.ones_like(sv)
    la_w = np.full(sv.shape[:-1], np.log(g["decay"]))
    for o, _ in (orc.scalar_recurrent(ones, ones, sv, la_w),
                 orc.scalar_quadratic(ones, ones, sv, la_w),
                 orc.scalar_chunkwise(ones, ones, sv, la_w, chunk=g["block"])):
        np.testing.assert_allclose(o.reshape(-1), g["running_totals"], atol=1e-12)


def test_forward_substitution_matches_library_solve():
    """The oracle's triangular solve agrees with LAPACK's general solver."""
    rng = np.random.default_rng(14)
    n, m = 17, 5
    L = np.tril(rng.standard_normal((3, n, n)), -1) * 0.3
    R = rng.standard_normal((3, n, m))
    X = orc.forward_substitution(L, R)
    want = np.linalg.solve(np.eye(n) + L, R)
    np.testing.assert_allclose(X, want, atol=1e-12)
