"""TEST INFRASTRUCTURE ONLY: Python front end of the fp64 CPU oracle.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this module.  It loads ``oracle/libdust_oracle.so`` (plain C,
built with gcc by :func:`build`) and shares nothing with the HIP path.

Every function mirrors one in ``dust_oracle.c``; the method it follows is
stated there, step by step, with the passage of "Dust: every token is a member
of the population" each step comes from.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dust_oracle.c")
_LIB = os.path.join(_HERE, "libdust_oracle.so")
_lib = None


def build() -> str:
    """Compile the oracle with gcc (no fast-math; plain fp64)."""
    tmp = f"{_LIB}.{os.getpid()}.tmp"  # concurrent builds each write their own
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    u32p = ctypes.POINTER(ctypes.c_uint32)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64 = ctypes.c_int64
    lib.dust_oracle_philox4x32_10.argtypes = [u32p, u32p, u32p]
    lib.dust_oracle_philox4x32_10.restype = None
    lib.dust_oracle_noise_fill.argtypes = [ctypes.c_uint64, i64, i64, i64, i64, i64, u32p, f64p]
    lib.dust_oracle_noise_fill.restype = None
    lib.dust_oracle_estimate.argtypes = [
        f32p, f32p, f32p, i64, i64, i64, i64, ctypes.c_int32, ctypes.c_float,
        ctypes.c_float, ctypes.c_uint64, ctypes.c_int32, i64, i64, ctypes.c_int32,
        f64p, f64p, f64p, f64p, f64p]
    lib.dust_oracle_estimate.restype = ctypes.c_int
    lib.dust_oracle_estimate_local.argtypes = [
        f32p, f32p, i64, i64, i64, i64, ctypes.c_int32, ctypes.c_float, ctypes.c_float,
        ctypes.c_uint64, ctypes.c_int32, i64, i64, ctypes.c_int32, f64p, f64p, f64p, f64p]
    lib.dust_oracle_estimate_local.restype = ctypes.c_int
    i32p = ctypes.POINTER(ctypes.c_int32)
    lib.dust_oracle_estimate_head.argtypes = [
        f32p, f32p, i32p, i64, i64, i64, i64, ctypes.c_int32, ctypes.c_float, ctypes.c_uint64,
        ctypes.c_int32, i64, i64, ctypes.c_int32, f64p, f64p, f64p, f64p]
    lib.dust_oracle_estimate_head.restype = ctypes.c_int
    lib.dust_oracle_reassemble_embedding.argtypes = [i32p, f64p, i64, i64, i64,
                                                     ctypes.c_double, f64p]
    lib.dust_oracle_reassemble_embedding.restype = ctypes.c_int
    lib.dust_oracle_estimate_embedding.argtypes = [
        f32p, i32p, f32p, i64, i64, i64, i64, ctypes.c_int32, ctypes.c_float, ctypes.c_float,
        ctypes.c_uint64, ctypes.c_int32, ctypes.c_double, i64, i64, ctypes.c_int32, f64p, f64p,
        f64p, f64p, f64p]
    lib.dust_oracle_estimate_embedding.restype = ctypes.c_int
    lib.dust_oracle_estimate_attention.argtypes = [
        f32p, f32p, f32p, f32p, f32p, i64, i64, i64, i64, i64, ctypes.c_int32, ctypes.c_int32,
        ctypes.c_float, ctypes.c_float, ctypes.c_uint64, ctypes.c_int32, i64, i64, ctypes.c_int32,
        f64p, f64p, f64p, f64p]
    lib.dust_oracle_estimate_attention.restype = ctypes.c_int
    lib.dust_oracle_true_gradient.argtypes = [f32p, f32p, f32p, i64, i64, i64, f64p, f64p]
    lib.dust_oracle_true_gradient.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def philox4x32_10(ctr, key) -> np.ndarray:
    """Philox4x32-10 of one 4-word counter under one 2-word key."""
    lib = _load()
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    lib.dust_oracle_philox4x32_10(_ptr(c, ctypes.c_uint32), _ptr(k, ctypes.c_uint32),
                                  _ptr(out, ctypes.c_uint32))
    return out


def noise_fill(seed: int, n0: int, n_cnt: int, t0: int, t_cnt: int, d_out: int,
               words: bool = True, gauss: bool = True):
    """Hashed words [n][t][4*ceil(d_out/4)] (uint32) and Gaussians [n][t][d_out] (fp64)."""
    lib = _load()
    nq = (d_out + 3) // 4
    w = np.zeros((n_cnt, t_cnt, 4 * nq), dtype=np.uint32) if words else None
    g = np.zeros((n_cnt, t_cnt, d_out), dtype=np.float64) if gauss else None
    lib.dust_oracle_noise_fill(
        ctypes.c_uint64(seed), n0, n_cnt, t0, t_cnt, d_out,
        _ptr(w, ctypes.c_uint32) if w is not None else None,
        _ptr(g, ctypes.c_double) if g is not None else None)
    return w, g


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def estimate(X, W, target, *, K: int, sigma: float, gamma: float, seed: int,
             antithetic: bool, seq_len: int, seq_range=None, threads: int | None = None):
    """Run the fp64 oracle.

    X [T,d_in], W [d_out,d_in], target [T,d_out] hold the exact input values
    (bf16 inputs widened to fp32).  ``seq_range=(s0, s1)`` restricts the work
    to sequences s0..s1-1: every output then covers those tokens only and G
    is their contribution.  Returns a dict of fp64 arrays:
    G [d_out,d_in], loss [n], rho [n,K], reward [n,K], g [n,d_out].
    """
    lib = _load()
    X = np.ascontiguousarray(X, dtype=np.float32)
    W = np.ascontiguousarray(W, dtype=np.float32)
    target = np.ascontiguousarray(target, dtype=np.float32)
    T, d_in = X.shape
    d_out = W.shape[0]
    assert W.shape == (d_out, d_in) and target.shape == (T, d_out)
    assert T % seq_len == 0
    n_seq = T // seq_len
    s0, s1 = (0, n_seq) if seq_range is None else seq_range
    n_tok = (s1 - s0) * seq_len
    G = np.zeros((d_out, d_in), dtype=np.float64)
    loss = np.zeros(n_tok, dtype=np.float64)
    rho = np.zeros((n_tok, K), dtype=np.float64)
    reward = np.zeros((n_tok, K), dtype=np.float64)
    g = np.zeros((n_tok, d_out), dtype=np.float64)
    th = default_threads() if threads is None else threads
    rc = lib.dust_oracle_estimate(
        _ptr(X, ctypes.c_float), _ptr(W, ctypes.c_float), _ptr(target, ctypes.c_float),
        T, d_in, d_out, seq_len, K, ctypes.c_float(sigma), ctypes.c_float(gamma),
        ctypes.c_uint64(seed), int(bool(antithetic)), s0, s1, th,
        _ptr(G, ctypes.c_double), _ptr(loss, ctypes.c_double), _ptr(rho, ctypes.c_double),
        _ptr(reward, ctypes.c_double), _ptr(g, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return {"G": G, "loss": loss, "rho": rho, "reward": reward, "g": g,
            "threads": th}


def estimate_local(X, E, *, K: int, sigma: float, gamma: float, seed: int,
                   antithetic: bool, seq_len: int, seq_range=None, threads: int | None = None):
    """Run the fp64 oracle with local scoring: each draw's jitter of the
    layer's output is scored against the error estimate E [T,d_out] (fp32)
    instead of a loss.  X [T,d_in] as for :func:`estimate`.  Returns a dict
    of fp64 arrays: G [d_out,d_in], rho [n,K] (the scores), reward [n,K],
    g [n,d_out]."""
    lib = _load()
    X = np.ascontiguousarray(X, dtype=np.float32)
    E = np.ascontiguousarray(E, dtype=np.float32)
    T, d_in = X.shape
    d_out = E.shape[1]
    assert E.shape == (T, d_out) and T % seq_len == 0
    n_seq = T // seq_len
    s0, s1 = (0, n_seq) if seq_range is None else seq_range
    n_tok = (s1 - s0) * seq_len
    G = np.zeros((d_out, d_in), dtype=np.float64)
    rho = np.zeros((n_tok, K), dtype=np.float64)
    reward = np.zeros((n_tok, K), dtype=np.float64)
    g = np.zeros((n_tok, d_out), dtype=np.float64)
    th = default_threads() if threads is None else threads
    rc = lib.dust_oracle_estimate_local(
        _ptr(X, ctypes.c_float), _ptr(E, ctypes.c_float), T, d_in, d_out, seq_len, K,
        ctypes.c_float(sigma), ctypes.c_float(gamma), ctypes.c_uint64(seed),
        int(bool(antithetic)), s0, s1, th, _ptr(G, ctypes.c_double),
        _ptr(rho, ctypes.c_double), _ptr(reward, ctypes.c_double), _ptr(g, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return {"G": G, "rho": rho, "reward": reward, "g": g, "threads": th}


ATTENTION_SITES = {"query": 0, "key": 1, "value": 2}


def estimate_attention(X, q, k, v, E, *, heads: int, site: str, K: int, sigma: float,
                       gamma: float, seed: int, antithetic: bool, seq_len: int,
                       seq_range=None, threads: int | None = None):
    """Run the fp64 oracle with scores through a recomputed attention: the
    cached queries q, keys k and values v [T, heads*d_head] of one block's
    causal attention (head h on columns h*d_head .. (h+1)*d_head - 1), the
    site ("query", "key" or "value") jittered, and every draw's change of
    the attention output scored against the error estimate E [T,
    heads*d_head].  X [T,d_in] (or None) is the block's input for the site's
    weight gradient.  Returns a dict of fp64 arrays: G [heads*d_head,d_in]
    (absent without X), rho [n,K] (the scores), reward [n,K], g [n,
    heads*d_head]."""
    lib = _load()
    q, k, v, E = (np.ascontiguousarray(a, dtype=np.float32) for a in (q, k, v, E))
    T, D = q.shape
    assert k.shape == v.shape == E.shape == (T, D) and D % heads == 0 and T % seq_len == 0
    d_head = D // heads
    if X is not None:
        X = np.ascontiguousarray(X, dtype=np.float32)
        assert X.shape[0] == T
    d_in = X.shape[1] if X is not None else 0
    n_seq = T // seq_len
    s0, s1 = (0, n_seq) if seq_range is None else seq_range
    n_tok = (s1 - s0) * seq_len
    G = np.zeros((D, max(d_in, 1)), dtype=np.float64)
    rho = np.zeros((n_tok, K), dtype=np.float64)
    reward = np.zeros((n_tok, K), dtype=np.float64)
    g = np.zeros((n_tok, D), dtype=np.float64)
    th = default_threads() if threads is None else threads
    rc = lib.dust_oracle_estimate_attention(
        _ptr(X, ctypes.c_float) if X is not None else None, _ptr(q, ctypes.c_float),
        _ptr(k, ctypes.c_float), _ptr(v, ctypes.c_float), _ptr(E, ctypes.c_float), T, d_in,
        heads, d_head, seq_len, ATTENTION_SITES[site], K, ctypes.c_float(sigma),
        ctypes.c_float(gamma), ctypes.c_uint64(seed), int(bool(antithetic)), s0, s1, th,
        _ptr(G, ctypes.c_double) if X is not None else None, _ptr(rho, ctypes.c_double),
        _ptr(reward, ctypes.c_double), _ptr(g, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    out = {"rho": rho, "reward": reward, "g": g, "threads": th}
    if X is not None:
        out["G"] = G
    return out


def estimate_head(X, W, labels, *, K: int, sigma: float, seed: int, antithetic: bool,
                  slab: int = 256, token_range=None, threads: int | None = None):
    """Run the fp64 oracle of the cross-entropy head: logits z = W x, labels
    [T] (int), every slab of `slab` columns jittered by its own K draws.
    ``token_range=(t0, t1)`` restricts the work to those tokens.  Returns a
    dict of fp64 arrays: G [V,d_in] (those tokens' contribution), loss [n]
    (clean cross-entropy), rho [n, V/slab, K], g [n, V]."""
    lib = _load()
    X = np.ascontiguousarray(X, dtype=np.float32)
    W = np.ascontiguousarray(W, dtype=np.float32)
    labels = np.ascontiguousarray(labels, dtype=np.int32)
    T, d_in = X.shape
    V = W.shape[0]
    assert W.shape == (V, d_in) and labels.shape == (T,) and V % slab == 0
    t0, t1 = (0, T) if token_range is None else token_range
    n = t1 - t0
    G = np.zeros((V, d_in), dtype=np.float64)
    loss = np.zeros(n, dtype=np.float64)
    rho = np.zeros((n, V // slab, K), dtype=np.float64)
    g = np.zeros((n, V), dtype=np.float64)
    th = default_threads() if threads is None else threads
    rc = lib.dust_oracle_estimate_head(
        _ptr(X, ctypes.c_float), _ptr(W, ctypes.c_float), _ptr(labels, ctypes.c_int32), T, d_in,
        V, slab, K, ctypes.c_float(sigma), ctypes.c_uint64(seed), int(bool(antithetic)), t0, t1,
        th, _ptr(G, ctypes.c_double), _ptr(loss, ctypes.c_double), _ptr(rho, ctypes.c_double),
        _ptr(g, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return {"G": G, "loss": loss, "rho": rho, "g": g, "threads": th}


def reassemble_embedding(ids, g, V: int, scale: float = 1.0) -> np.ndarray:
    """G_E [V, d] = scale * sum over tokens t with ids[t] = v of g[t] (fp64,
    tokens added in order; rows of absent ids zero)."""
    lib = _load()
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    g = np.ascontiguousarray(g, dtype=np.float64)
    T, d = g.shape
    assert ids.shape == (T,)
    G = np.zeros((V, d), dtype=np.float64)
    rc = lib.dust_oracle_reassemble_embedding(_ptr(ids, ctypes.c_int32), _ptr(g, ctypes.c_double),
                                              T, V, d, float(scale), _ptr(G, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return G


def estimate_embedding(table, ids, target, *, K: int, sigma: float, gamma: float, seed: int,
                       antithetic: bool, seq_len: int, scale: float = 1.0, seq_range=None,
                       threads: int | None = None):
    """Run the fp64 oracle for a token embedding: table [V, d], ids [T],
    target [T, d]; ``seq_range=(s0, s1)`` restricts the work to those
    sequences.  Returns a dict of fp64 arrays: G [V, d] (scale x those
    tokens' scatter-added g), loss [n], rho [n, K], reward [n, K], g [n, d]."""
    lib = _load()
    table = np.ascontiguousarray(table, dtype=np.float32)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    target = np.ascontiguousarray(target, dtype=np.float32)
    V, d = table.shape
    T = ids.shape[0]
    assert target.shape == (T, d)
    s0, s1 = (0, 0) if seq_range is None else seq_range
    n = (T if seq_range is None else (s1 - s0) * seq_len)
    G = np.zeros((V, d), dtype=np.float64)
    loss = np.zeros(n, dtype=np.float64)
    rho = np.zeros((n, K), dtype=np.float64)
    reward = np.zeros((n, K), dtype=np.float64)
    g = np.zeros((n, d), dtype=np.float64)
    th = default_threads() if threads is None else threads
    rc = lib.dust_oracle_estimate_embedding(
        _ptr(table, ctypes.c_float), _ptr(ids, ctypes.c_int32), _ptr(target, ctypes.c_float), T,
        V, d, seq_len, K, ctypes.c_float(sigma), ctypes.c_float(gamma), ctypes.c_uint64(seed),
        int(bool(antithetic)), float(scale), s0, s1, th, _ptr(G, ctypes.c_double),
        _ptr(loss, ctypes.c_double), _ptr(rho, ctypes.c_double), _ptr(reward, ctypes.c_double),
        _ptr(g, ctypes.c_double))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    return {"G": G, "loss": loss, "rho": rho, "reward": reward, "g": g, "threads": th}


def true_gradient(X, W, target):
    """delta [T,d_out] and the backprop gradient sum_t delta_t x_t^T [d_out,d_in]."""
    lib = _load()
    X = np.ascontiguousarray(X, dtype=np.float32)
    W = np.ascontiguousarray(W, dtype=np.float32)
    target = np.ascontiguousarray(target, dtype=np.float32)
    T, d_in = X.shape
    d_out = W.shape[0]
    delta = np.zeros((T, d_out), dtype=np.float64)
    G = np.zeros((d_out, d_in), dtype=np.float64)
    lib.dust_oracle_true_gradient(_ptr(X, ctypes.c_float), _ptr(W, ctypes.c_float),
                                  _ptr(target, ctypes.c_float), T, d_in, d_out,
                                  _ptr(delta, ctypes.c_double), _ptr(G, ctypes.c_double))
    return delta, G
