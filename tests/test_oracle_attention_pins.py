"""Pins of the oracle's scores through a recomputed attention
(dust_oracle_estimate_attention) against what the mathematics fixes.

The site is one block's causal softmax attention ("Dust: every token is a
member of the population", section "What the released code actually does",
step 4, in the form that perturbs a query, key or value and evaluates the
block's attention again; a draw's score is c_s = -<g_s, Delta o_s> with g an
error estimate of the attention output).  The oracle recomputes the
jittered attention literally; these pins check it against independent numpy
algebra:

* values enter the output linearly, so Delta o_s = s_i sigma sum_t p_st a_t
  exactly (any sigma);
* for keys and queries the new probabilities are p'_st = p_st e^(x_st) / Z_s
  with x_st the jitter's change of the logit, an exact identity at any sigma,
  and to first order Delta o_s = sum_t p_st (v_t - o_s) x_st;
* antithetic pairs: the value scores are exactly opposite, the key and query
  scores opposite up to O(sigma^2);
* the first token of a sequence has nothing to re-weight: its key and query
  scores are exactly zero;
* sequences are independent (a sequence range reproduces the full run);
* with gamma = 1 and antithetic pairs, E[g_t] is the gradient of
  sum_s <e_s, o_s> with respect to the site at token t, checked over many
  seeds against the analytic Jacobian.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

SITES = ("query", "key", "value")


def inputs(T, H, dh, d_in, seed):
    rng = np.random.default_rng(seed)
    q, k, v, E = (rng.standard_normal((T, H * dh)).astype(np.float32) for _ in range(4))
    X = rng.standard_normal((T, d_in)).astype(np.float32)
    return X, q, k, v, E


def softmax_causal(q, k):
    """P [L,L] of one head: row s softmax over t <= s of <q_s,k_t>/sqrt(dh)."""
    L, dh = q.shape
    logits = (q @ k.T) / np.sqrt(dh)
    logits = np.where(np.tril(np.ones((L, L), dtype=bool)), logits, -np.inf)
    logits -= logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    return w / w.sum(axis=1, keepdims=True)


def noise(oracle_mod, seed, n, t0, L, D):
    _, g = oracle_mod.noise_fill(seed, n, 1, t0, L, D)
    return g.reshape(L, D)


def draw(i, antithetic):
    return (i // 2, -1.0 if (antithetic and i % 2) else 1.0) if antithetic else (i, 1.0)


def expected_scores(oracle_mod, q, k, v, E, H, L, site, K, sigma, seed, antithetic,
                    linear=False):
    """rho [T,K] from the exact re-weighting identity (or its first order)."""
    T, D = q.shape
    dh = D // H
    rho = np.zeros((T, K))
    for sq in range(T // L):
        sl = slice(sq * L, (sq + 1) * L)
        for i in range(K):
            n, s = draw(i, antithetic)
            A = noise(oracle_mod, seed, n, sq * L, L, D)
            for h in range(H):
                hs = slice(h * dh, (h + 1) * dh)
                qh, kh, vh, Eh = (x[sl, hs].astype(np.float64) for x in (q, k, v, E))
                Ah = A[:, hs]  # the noise of this sequence's tokens
                if site == "value":
                    dv = s * sigma * Ah
                    P = softmax_causal(qh, kh)
                    do = P @ dv
                else:
                    P = softmax_causal(qh, kh)
                    if site == "key":
                        x = s * sigma * (qh @ Ah.T) / np.sqrt(dh)
                    else:
                        x = s * sigma * (Ah @ kh.T) / np.sqrt(dh)
                    x = np.where(np.tril(np.ones((L, L), dtype=bool)), x, 0.0)
                    o = P @ vh
                    if linear:
                        do = (P * x) @ vh - (P * x).sum(axis=1, keepdims=True) * o
                    else:
                        Pn = P * np.exp(x)
                        Pn /= Pn.sum(axis=1, keepdims=True)
                        do = (Pn - P) @ vh
                rho[sl, i] -= (Eh * do).sum(axis=1)
    return rho


@pytest.mark.parametrize("site", SITES)
def test_scores_match_the_reweighting_identity(oracle_mod, site):
    T, L, H, dh, K = 12, 6, 2, 4, 6
    X, q, k, v, E = inputs(T, H, dh, 5, seed=1)
    for sigma in (1e-3, 0.3):
        r = oracle_mod.estimate_attention(X, q, k, v, E, heads=H, site=site, K=K, sigma=sigma,
                                          gamma=0.5, seed=11, antithetic=True, seq_len=L)
        ref = expected_scores(oracle_mod, q, k, v, E, H, L, site, K, np.float32(sigma), 11, True)
        scale = np.abs(ref).max()
        assert np.abs(r["rho"] - ref).max() <= 1e-10 * scale, (site, sigma)


@pytest.mark.parametrize("site", ("query", "key"))
def test_first_order_scores(oracle_mod, site):
    T, L, H, dh, K = 8, 8, 1, 8, 4
    X, q, k, v, E = inputs(T, H, dh, 3, seed=2)
    sigma = 1e-4
    r = oracle_mod.estimate_attention(X, q, k, v, E, heads=H, site=site, K=K, sigma=sigma,
                                      gamma=0.0, seed=5, antithetic=False, seq_len=L)
    lin = expected_scores(oracle_mod, q, k, v, E, H, L, site, K, np.float32(sigma), 5, False,
                          linear=True)
    assert np.abs(r["rho"] - lin).max() <= 1e-3 * np.abs(lin).max()


@pytest.mark.parametrize("site", SITES)
def test_antithetic_symmetry_and_first_token(oracle_mod, site):
    T, L, H, dh, K = 10, 5, 2, 4, 8
    X, q, k, v, E = inputs(T, H, dh, 4, seed=3)
    sigma = 1e-3
    r = oracle_mod.estimate_attention(X, q, k, v, E, heads=H, site=site, K=K, sigma=sigma,
                                      gamma=0.9, seed=7, antithetic=True, seq_len=L)
    rho = r["rho"]
    plus, minus = rho[:, 0::2], rho[:, 1::2]
    if site == "value":
        # the oracle forms o' - o, each output rounded relative to |o| <= max|v|
        # (o is a convex combination of the values), not to |o' - o|: the pair's
        # sum is that rounding, a few ulps of |v| per channel, weighted by |E|
        D = q.shape[1]
        bound = 8 * np.finfo(np.float64).eps * D * np.abs(E).max() * np.abs(v).max()
        assert np.abs(plus + minus).max() <= bound
    else:
        assert np.abs(plus + minus).max() <= 1e-2 * np.abs(plus).max()
        assert np.all(rho[::L] == 0.0)  # the first token of every sequence
        assert np.abs(rho[1::L]).max() > 0.0


@pytest.mark.parametrize("site", SITES)
def test_sequences_are_independent(oracle_mod, site):
    T, L, H, dh, K = 18, 6, 2, 4, 4
    X, q, k, v, E = inputs(T, H, dh, 5, seed=4)
    kw = dict(heads=H, site=site, K=K, sigma=0.05, gamma=0.8, seed=9, antithetic=False,
              seq_len=L)
    full = oracle_mod.estimate_attention(X, q, k, v, E, **kw)
    G = np.zeros_like(full["G"])
    for s0 in range(T // L):
        part = oracle_mod.estimate_attention(X, q, k, v, E, seq_range=(s0, s0 + 1), **kw)
        sl = slice(s0 * L, (s0 + 1) * L)
        for key in ("rho", "reward", "g"):
            assert np.array_equal(part[key], full[key][sl]), key
        G += part["G"]
    assert np.allclose(G, full["G"], rtol=1e-12, atol=1e-12)


def analytic_site_gradient(q, k, v, E, H, L, site):
    """d/d(site) of sum_s <e_s, o_s> for one block's causal attention."""
    T, D = q.shape
    dh = D // H
    grad = np.zeros((T, D))
    for sq in range(T // L):
        sl = slice(sq * L, (sq + 1) * L)
        for h in range(H):
            hs = slice(h * dh, (h + 1) * dh)
            qh, kh, vh, Eh = (x[sl, hs].astype(np.float64) for x in (q, k, v, E))
            P = softmax_causal(qh, kh)
            o = P @ vh
            if site == "value":
                gh = P.T @ Eh
            else:
                # B[s,t] = p_st <e_s, v_t - o_s> / sqrt(dh)
                B = P * (Eh @ vh.T - (Eh * o).sum(axis=1, keepdims=True)) / np.sqrt(dh)
                gh = B.T @ qh if site == "key" else B @ kh
            grad[sl, hs] = gh
    return grad


@pytest.mark.parametrize("site", SITES)
def test_expected_error_is_the_site_gradient(oracle_mod, site):
    T, L, H, dh, K, seeds = 8, 4, 1, 4, 32, 120
    X, q, k, v, E = inputs(T, H, dh, 2, seed=6)
    true = analytic_site_gradient(q, k, v, E, H, L, site)
    acc = np.zeros_like(true)
    for sd in range(seeds):
        r = oracle_mod.estimate_attention(None, q, k, v, E, heads=H, site=site, K=K,
                                          sigma=1e-3, gamma=1.0, seed=1000 + sd,
                                          antithetic=True, seq_len=L, threads=1)
        acc += r["g"]
    mean = acc / seeds
    err = np.linalg.norm(mean - true) / np.linalg.norm(true)
    # each of the seeds * K / 2 noise vectors adds independent spread: the
    # mean's relative error is about sqrt(D / (seeds * K / 2)) ~ 0.04 here
    assert err <= 0.15, err
    cos = float((mean * true).sum() / (np.linalg.norm(mean) * np.linalg.norm(true)))
    assert cos >= 0.98, cos
