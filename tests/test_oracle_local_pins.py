"""Pins of the oracle's local scoring ("What the released code actually
does", step 4: attention internals have no direct path to the loss, so a
jitter earns c_s = -<g_s, Delta o_s>, the inner product of the output's
change with an error estimate of that output; keys, values and gates add
later tokens' scores with decay gamma = 0.98, queries use their own token's
score only).

Reading pinned here: the jittered output is the layer's own, so draw i's
score at token t is -<e_t, s_i sigma a_t^(n(i))> against a supplied error
estimate e_t, and the score then runs through the same centring, credit,
reweighting and outer product as the loss reduction.  Each test compares the
oracle with something other than itself: the quadratic-loss estimator
(pinned by finite differences and closed forms in test_oracle_pins.py), exact
identities that follow from the linearity of the score, and the expectation
law.
"""
import numpy as np
import pytest

from token_activation_perturbation_amd import synth


def _inputs(T=12, d_in=5, d_out=7, seed=3):
    inp = synth.random_inputs(T, d_in, d_out, "f32", seed)
    rng = np.random.default_rng(seed + 100)
    E = rng.standard_normal((T, d_out)).astype(np.float32)
    return inp["X"], E


def _noise(oracle_mod, seed, K_n, T, d_out):
    _, g = oracle_mod.noise_fill(seed, 0, K_n, 0, T, d_out, words=False, gauss=True)
    return g  # [n][t][c]


@pytest.mark.parametrize("gamma,sigma", [(0.0, 1e-2), (0.98, 1e-2), (0.98, 0.4), (1.0, 0.2)])
def test_local_antithetic_exact_identity(oracle_mod, gamma, sigma):
    """With a linear score the pair's scores are exactly opposite, so
    centring is a no-op and, for any sigma,
    g_t = (2/K) sum_p a_t^p sum_{s>=t} gamma^(s-t) <e_s, a_s^p>."""
    T, seq_len, d_out, K = 12, 6, 7, 8
    X, E = _inputs(T=T, d_out=d_out)
    out = oracle_mod.estimate_local(X, E, K=K, sigma=sigma, gamma=gamma, seed=21,
                                    antithetic=True, seq_len=seq_len)
    a = _noise(oracle_mod, 21, K // 2, T, d_out)
    P = np.einsum("tc,ntc->nt", E.astype(np.float64), a)
    g32 = float(np.float32(gamma))
    g_ref = np.zeros((T, d_out))
    for t in range(T):
        end = (t // seq_len + 1) * seq_len
        for p in range(K // 2):
            pi = sum(g32 ** (s - t) * P[p, s] for s in range(t, end))
            g_ref[t] += (2.0 / K) * pi * a[p, t]
    assert np.allclose(out["g"], g_ref, rtol=1e-10, atol=1e-12)
    # each pair's scores are opposite numbers
    assert np.allclose(out["rho"][:, 0::2], -out["rho"][:, 1::2], rtol=0, atol=1e-15)


@pytest.mark.parametrize("gamma", [0.0, 0.9])
def test_local_equals_loss_estimate_when_e_is_delta(oracle_mod, gamma):
    """With antithetic pairs the quadratic loss's curvature cancels inside
    each pair, so scoring against the exact output error e = delta gives the
    quadratic-loss estimator's g and G_W (the latter computed from literal
    perturbed losses)."""
    T, seq_len, d_in, d_out, K = 12, 4, 5, 7, 6
    inp = synth.random_inputs(T, d_in, d_out, "f32", 9)
    delta, _ = oracle_mod.true_gradient(inp["X"], inp["W"], inp["target"])
    kw = dict(K=K, sigma=0.05, gamma=gamma, seed=4, antithetic=True, seq_len=seq_len)
    loss = oracle_mod.estimate(inp["X"], inp["W"], inp["target"], **kw)
    # delta in fp32, the precision an error estimate is handed over in
    local = oracle_mod.estimate_local(inp["X"], delta.astype(np.float32), **kw)
    scale = np.abs(loss["g"]).max()
    assert np.allclose(local["g"], loss["g"], rtol=1e-5, atol=1e-6 * scale)
    assert np.allclose(local["G"], loss["G"], rtol=1e-5, atol=1e-6 * np.abs(loss["G"]).max())


@pytest.mark.parametrize("antithetic", [False, True])
def test_local_does_not_depend_on_sigma(oracle_mod, antithetic):
    """The score is linear in the jitter, so the 1/sigma of the estimator
    cancels it exactly: g and G_W are the same for every sigma."""
    X, E = _inputs()
    kw = dict(K=6, gamma=0.98, seed=13, antithetic=antithetic, seq_len=6)
    a = oracle_mod.estimate_local(X, E, sigma=1e-2, **kw)
    b = oracle_mod.estimate_local(X, E, sigma=0.75, **kw)
    assert np.allclose(a["g"], b["g"], rtol=1e-11, atol=1e-13)
    assert np.allclose(a["G"], b["G"], rtol=1e-11, atol=1e-13)


def test_local_is_linear_in_the_error_estimate(oracle_mod):
    """Same noise, so g(e1 + 2 e2) = g(e1) + 2 g(e2), also with credit decay
    and the centring of plain draws (both linear)."""
    X, E1 = _inputs(seed=5)
    _, E2 = _inputs(seed=6)
    kw = dict(K=5, sigma=0.1, gamma=0.98, seed=2, antithetic=False, seq_len=4)
    g1 = oracle_mod.estimate_local(X, E1, **kw)["g"]
    g2 = oracle_mod.estimate_local(X, E2, **kw)["g"]
    E3 = (E1.astype(np.float64) + 2.0 * E2.astype(np.float64)).astype(np.float32)
    g3 = oracle_mod.estimate_local(X, E3, **kw)["g"]
    # E3 is rounded to fp32, the rest is exact linear algebra
    assert np.allclose(g3, g1 + 2.0 * g2, rtol=1e-6, atol=1e-6 * np.abs(g3).max())


def test_local_gamma_zero_keeps_own_score(oracle_mod):
    """gamma = 0 (the query sites): each token keeps its own centred score."""
    X, E = _inputs(T=8)
    out = oracle_mod.estimate_local(X, E, K=4, sigma=0.2, gamma=0.0, seed=7,
                                    antithetic=False, seq_len=8)
    c = out["rho"] - out["rho"].mean(1, keepdims=True)
    assert np.array_equal(out["reward"], c)


@pytest.mark.parametrize("antithetic,K", [(True, 4), (False, 4)])
def test_local_expectation(oracle_mod, antithetic, K):
    """E[g_t] = e_t with antithetic pairs and (K-1)/K e_t with plain draws
    (the centring), with the keys' credit decay gamma = 0.98: later tokens'
    scores are independent of a_t and add variance only."""
    T, d_out = 4, 6
    X, E = _inputs(T=T, d_in=3, d_out=d_out, seed=8)
    S = 3000
    acc = np.zeros((T, d_out))
    for s in range(S):
        out = oracle_mod.estimate_local(X, E, K=K, sigma=0.2, gamma=0.98,
                                        seed=5000 + s, antithetic=antithetic,
                                        seq_len=T, threads=1)
        acc += out["g"]
    e = E.astype(np.float64)
    ratio = (acc / S * e).sum() / (e * e).sum()
    expect = 1.0 if antithetic else (K - 1) / K
    assert abs(ratio - expect) < 0.05, ratio
