"""Pins of the oracle's token embedding ("What the released code actually
does", step 7: an embedding's per-token error becomes its weight gradient by
a scatter-add, and every estimate is divided by the token count before it is
written to .grad).

Reading pinned here: the site is o_t = E[id_t] with the layer-local loss
(a gather in place of W x_t), the estimator's steps unchanged, and
G_E[v] = scale * sum_{t: id_t = v} g_t.  Each test compares the oracle with
something other than itself: the layer estimator (pinned in
test_oracle_pins.py) on one-hot inputs, a one-hot matrix product, finite
differences of the clean loss, exact identities of the scatter, and the
antithetic closed form of g.
"""
import numpy as np
import pytest

from token_activation_perturbation_amd import synth


def _inputs(T=12, V=9, d=7, seed=3):
    rng = np.random.default_rng(seed)
    table = rng.standard_normal((V, d)).astype(np.float32)
    target = rng.standard_normal((T, d)).astype(np.float32)
    # repeated ids, and some ids that never occur
    ids = rng.integers(0, V - 2, size=T).astype(np.int32)
    return table, ids, target


@pytest.mark.parametrize("gamma,antithetic", [(0.0, True), (0.9, False), (0.5, True)])
def test_embedding_equals_layer_estimator_on_one_hot_inputs(oracle_mod, gamma, antithetic):
    """An embedding is the linear layer y = W x with x_t = onehot(id_t) and
    W = E^T, so the layer oracle on those inputs gives the same loss, rho,
    credit and g, and G_W = G_E^T (scale 1)."""
    T, V, d, seq_len, K = 12, 9, 7, 4, 6
    table, ids, target = _inputs(T, V, d)
    X = np.zeros((T, V), dtype=np.float32)
    X[np.arange(T), ids] = 1.0
    W = np.ascontiguousarray(table.T)
    kw = dict(K=K, sigma=0.1, gamma=gamma, seed=5, antithetic=antithetic, seq_len=seq_len)
    emb = oracle_mod.estimate_embedding(table, ids, target, **kw)
    lay = oracle_mod.estimate(X, W, target, **kw)
    for k in ("loss", "rho", "reward", "g"):
        assert np.allclose(emb[k], lay[k], rtol=1e-13, atol=1e-15), k
    assert np.allclose(emb["G"], lay["G"].T, rtol=1e-13, atol=1e-15)


def test_reassembly_is_the_one_hot_product(oracle_mod):
    rng = np.random.default_rng(7)
    T, V, d = 40, 13, 5
    ids = rng.integers(0, V, size=T).astype(np.int32)
    g = rng.standard_normal((T, d))
    onehot = np.zeros((T, V))
    onehot[np.arange(T), ids] = 1.0
    G = oracle_mod.reassemble_embedding(ids, g, V, scale=0.25)
    assert np.allclose(G, 0.25 * (onehot.T @ g), rtol=1e-14, atol=1e-15)


def test_reassembly_identities(oracle_mod):
    """Rows of absent ids are exactly zero; an id that occurs once gets
    scale * g_t exactly; the rows sum to scale * sum_t g_t; and reordering
    the tokens changes nothing beyond rounding."""
    rng = np.random.default_rng(9)
    T, V, d = 64, 20, 6
    ids = rng.integers(0, 12, size=T).astype(np.int32)
    ids[5] = 15  # occurs once
    g = rng.standard_normal((T, d))
    scale = 1.0 / T
    G = oracle_mod.reassemble_embedding(ids, g, V, scale=scale)
    absent = sorted(set(range(V)) - set(ids.tolist()))
    assert absent and np.all(G[absent] == 0.0)
    assert np.array_equal(G[15], scale * g[5])
    assert np.allclose(G.sum(0), scale * g.sum(0), rtol=1e-13, atol=1e-15)
    perm = rng.permutation(T)
    G2 = oracle_mod.reassemble_embedding(ids[perm], g[perm], V, scale=scale)
    assert np.allclose(G, G2, rtol=1e-13, atol=1e-15)


def test_reassembly_rejects_out_of_range_ids(oracle_mod):
    g = np.zeros((3, 2))
    for bad in (-1, 4):
        with pytest.raises(ValueError):
            oracle_mod.reassemble_embedding(np.array([0, bad, 1], dtype=np.int32), g, 4)


def test_embedding_clean_loss_gradient_matches_finite_differences(oracle_mod):
    """Central differences of the oracle's clean loss sum_t L_t in a table
    entry E[v][c] equal sum_{t: id_t = v} delta_t[c]: the gradient of a
    gather is the scatter of the output error."""
    T, V, d = 10, 6, 4
    table, ids, target = _inputs(T, V, d, seed=11)
    kw = dict(K=2, sigma=0.1, gamma=0.0, seed=0, antithetic=True, seq_len=T)
    delta = table[ids].astype(np.float64) - target.astype(np.float64)
    grad = np.zeros((V, d))
    np.add.at(grad, ids, delta)
    h = np.float32(2.0 ** -8)
    for v in range(V):
        for c in range(d):
            tp, tm = table.copy(), table.copy()
            tp[v, c] += h
            tm[v, c] -= h
            h2 = float(tp[v, c]) - float(tm[v, c])
            Lp = oracle_mod.estimate_embedding(tp, ids, target, **kw)["loss"].sum()
            Lm = oracle_mod.estimate_embedding(tm, ids, target, **kw)["loss"].sum()
            # a quadratic: central differences are exact up to rounding
            assert abs((Lp - Lm) / h2 - grad[v, c]) <= 1e-9 * max(1.0, abs(grad[v, c]))


@pytest.mark.parametrize("sigma", [1e-3, 0.4])
def test_embedding_antithetic_closed_form(oracle_mod, sigma):
    """With antithetic pairs and gamma = 0 the quadratic loss's curvature
    cancels inside each pair, so for any sigma g_t = (2/K) sum_p a_p <delta_t, a_p>
    and G_E = scale * scatter(g): noise drawn independently here, delta from
    a numpy gather."""
    T, V, d, K = 16, 8, 5, 8
    table, ids, target = _inputs(T, V, d, seed=13)
    scale = 1.0 / T
    out = oracle_mod.estimate_embedding(table, ids, target, K=K, sigma=sigma, gamma=0.0,
                                        seed=17, antithetic=True, seq_len=8, scale=scale)
    _, a = oracle_mod.noise_fill(17, 0, K // 2, 0, T, d, words=False, gauss=True)
    delta = table[ids].astype(np.float64) - target.astype(np.float64)
    P = np.einsum("tc,ntc->nt", delta, a)
    g = (2.0 / K) * np.einsum("nt,ntc->tc", P, a)
    assert np.allclose(out["g"], g, rtol=1e-10, atol=1e-12)
    G = np.zeros((V, d))
    np.add.at(G, ids, g)
    assert np.allclose(out["G"], scale * G, rtol=1e-10, atol=1e-13)


def test_embedding_sequence_range_matches_full_run(oracle_mod):
    table, ids, target = _inputs(T=12)
    kw = dict(K=4, sigma=0.2, gamma=0.9, seed=2, antithetic=False, seq_len=4)
    full = oracle_mod.estimate_embedding(table, ids, target, **kw)
    part = oracle_mod.estimate_embedding(table, ids, target, seq_range=(1, 3), **kw)
    for k in ("loss", "rho", "reward", "g"):
        assert np.array_equal(part[k], full[k][4:12]), k
    G = np.zeros_like(full["G"])
    np.add.at(G, ids[4:12], full["g"][4:12])
    assert np.allclose(part["G"], G, rtol=1e-14, atol=1e-15)


def test_embedding_workload_ids_are_zipfian():
    """The synthetic ids follow a Zipf law over the vocabulary, as text
    tokens do: the most frequent id is far above the mean count."""
    w = synth.WORKLOADS["embed_bf16"]
    inp = synth.make_inputs(w)
    ids = inp["ids"]
    assert ids.min() >= 0 and ids.max() < w.V
    counts = np.bincount(ids, minlength=w.V)
    assert counts.max() > 50 * counts.mean()
    assert (counts == 0).sum() > 0  # some ids never occur in the batch
