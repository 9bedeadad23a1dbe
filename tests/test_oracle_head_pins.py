"""Pins of the oracle's cross-entropy head ("What the released code actually
does", step 5: the head's logits are perturbed in 256-column slabs of the
vocabulary, one slab per draw, and the cross-entropy alone is formed again).

Reading pinned here: the layer is the head z_t = W x_t with the per-token
loss CE(z_t, y_t) = logsumexp(z_t) - z_t[y_t]; each slab of columns is its
own site with K draws, draw i adding s_i sigma a_t^(n(i)) to that slab's
logits only; the loss reduction is clean minus perturbed cross-entropy,
centred over the slab's K draws (gamma = 0); g_t's slab columns come from
that slab's draws.  Each test compares the oracle with something other than
itself: finite differences against the analytic gradient softmax - one-hot,
the small-sigma limit of the estimator (an exact linear identity), and the
expectation law.
"""
import numpy as np
import pytest


def _head_inputs(T=6, d_in=5, V=32, seed=3):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((T, d_in)).astype(np.float32)
    W = (rng.standard_normal((V, d_in)) / np.sqrt(d_in)).astype(np.float32)
    y = rng.integers(0, V, size=T).astype(np.int32)
    return X, W, y


def _softmax_grad(X, W, y):
    """d CE / d z = softmax(z) - one_hot(y), z = W x, in fp64."""
    z = X.astype(np.float64) @ W.astype(np.float64).T
    z -= z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    p[np.arange(len(y)), y] -= 1.0
    return p


def _noise(oracle_mod, seed, K_n, T, V):
    _, g = oracle_mod.noise_fill(seed, 0, K_n, 0, T, V, words=False, gauss=True)
    return g  # [n][t][c]


def test_head_clean_loss_gradient_matches_finite_differences(oracle_mod):
    """Central differences of the oracle's clean cross-entropy in W equal
    sum_t (softmax(z_t) - onehot(y_t)) x_t^T."""
    X, W, y = _head_inputs(T=4, d_in=3, V=16)
    grad = _softmax_grad(X, W, y).T @ X.astype(np.float64)  # [V, d_in]
    kw = dict(K=2, sigma=0.05, seed=0, antithetic=True, slab=8)
    rng = np.random.default_rng(1)
    for _ in range(12):
        c, k = int(rng.integers(0, 16)), int(rng.integers(0, 3))
        Wp, Wm = W.copy(), W.copy()
        Wp[c, k] = np.float32(W[c, k] + np.float32(2.0 ** -10))
        Wm[c, k] = np.float32(W[c, k] - np.float32(2.0 ** -10))
        h2 = float(Wp[c, k]) - float(Wm[c, k])  # the perturbation actually applied
        Lp = oracle_mod.estimate_head(X, Wp, y, **kw)["loss"].sum()
        Lm = oracle_mod.estimate_head(X, Wm, y, **kw)["loss"].sum()
        assert abs((Lp - Lm) / h2 - grad[c, k]) <= 2e-5 * max(1.0, abs(grad[c, k]))


def test_head_clean_loss_is_cross_entropy(oracle_mod):
    X, W, y = _head_inputs()
    out = oracle_mod.estimate_head(X, W, y, K=2, sigma=0.05, seed=0, antithetic=True, slab=8)
    z = X.astype(np.float64) @ W.astype(np.float64).T
    m = z.max(axis=1)
    ce = m + np.log(np.exp(z - m[:, None]).sum(1)) - z[np.arange(len(y)), y]
    assert np.allclose(out["loss"], ce, rtol=1e-12)


@pytest.mark.parametrize("slab", [8, 32])
def test_head_small_sigma_limit(oracle_mod, slab):
    """As sigma -> 0 an antithetic pair's reduction difference is
    -2 sigma <grad, a> + O(sigma^3) (the even orders cancel), so
    g_t[slab] -> (2/K) sum_p a_p[slab] <grad_t[slab], a_p[slab]> with
    grad = softmax - one-hot: the identity of "What a zeroth-order gradient
    is" on each slab separately."""
    T, V, K = 5, 32, 8
    X, W, y = _head_inputs(T=T, V=V)
    sigma = 1e-4
    out = oracle_mod.estimate_head(X, W, y, K=K, sigma=sigma, seed=11, antithetic=True,
                                   slab=slab)
    grad = _softmax_grad(X, W, y)
    a = _noise(oracle_mod, 11, K // 2, T, V)
    ref = np.zeros((T, V))
    for j in range(V // slab):
        cs = slice(j * slab, (j + 1) * slab)
        P = np.einsum("tc,ntc->nt", grad[:, cs], a[:, :, cs])
        ref[:, cs] = (2.0 / K) * np.einsum("nt,ntc->tc", P, a[:, :, cs])
    assert np.allclose(out["g"], ref, rtol=1e-5, atol=1e-6 * np.abs(ref).max())
    # the weight gradient is the outer product of the head's error and input
    assert np.allclose(out["G"], out["g"].T @ X.astype(np.float64), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("antithetic", [False, True])
def test_head_g_from_centred_reductions(oracle_mod, antithetic):
    """g_t on slab j is -1/(K sigma) sum_i (rho_i - mean rho) s_i a_i over that
    slab's draws, with the noise generated independently here."""
    T, V, K, slab = 4, 16, 6, 8
    X, W, y = _head_inputs(T=T, V=V, seed=5)
    sigma = float(np.float32(0.2))
    out = oracle_mod.estimate_head(X, W, y, K=K, sigma=sigma, seed=3, antithetic=antithetic,
                                   slab=slab)
    K_n = K // 2 if antithetic else K
    a = _noise(oracle_mod, 3, K_n, T, V)
    ref = np.zeros((T, V))
    for j in range(V // slab):
        cs = slice(j * slab, (j + 1) * slab)
        rho = out["rho"][:, j, :]
        c = rho - rho.mean(1, keepdims=True)
        for i in range(K):
            n = i // 2 if antithetic else i
            s = -1.0 if (antithetic and i % 2) else 1.0
            ref[:, cs] += (c[:, i] * s)[:, None] * a[n, :, cs]
        ref[:, cs] *= -1.0 / (K * sigma)
    assert np.allclose(out["g"], ref, rtol=1e-12, atol=1e-14)


def test_head_expectation(oracle_mod):
    """E[g_t] = softmax - one-hot up to the O(sigma^2) curvature bias;
    averaged over many seeds and projected on the gradient."""
    T, V = 3, 16
    X, W, y = _head_inputs(T=T, V=V, seed=7)
    grad = _softmax_grad(X, W, y)
    S = 2000
    acc = np.zeros((T, V))
    for s in range(S):
        acc += oracle_mod.estimate_head(X, W, y, K=4, sigma=0.05, seed=7000 + s,
                                        antithetic=True, slab=8, threads=1)["g"]
    ratio = (acc / S * grad).sum() / (grad * grad).sum()
    assert abs(ratio - 1.0) < 0.05, ratio


def test_head_token_range_matches_full_run(oracle_mod):
    X, W, y = _head_inputs(T=6)
    kw = dict(K=4, sigma=0.05, seed=2, antithetic=False, slab=8)
    full = oracle_mod.estimate_head(X, W, y, **kw)
    part = oracle_mod.estimate_head(X, W, y, token_range=(2, 5), **kw)
    for k in ("loss", "rho", "g"):
        assert np.array_equal(part[k], full[k][2:5])
