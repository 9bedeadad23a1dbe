"""Seeded synthetic inputs for the Dust estimator of one linear layer.

This module holds no arithmetic of the estimator: it only draws X, W and
target (for local scoring X and an error estimate E; for a cross-entropy head
X, W and labels; for a token embedding its table, Zipfian ids and target;
for an attention site X, the cached q, k, v and E) with the shapes and
distributions of the workloads below,
and rounds them to the input dtype.
The pages train on FineWeb with a 37.7M parameter GPT whose layers are 512
wide ("Dust: every token is a member of the population", sections "What the
released code actually does" and "The results, checked against the tables");
neither the data nor the weights are available, so these draws stand in for
that layer's inputs, and the layer-local squared error (or the supplied error
estimate) stands in for the network.

Recipe: numpy ``default_rng(data_seed)`` (PCG64) standard normals in fp64,
scaled, cast to fp32 (round to nearest even) and, for bf16 workloads, rounded
once more from fp32 to bf16 (round to nearest even).  Both the HIP path and
the oracle consume exactly these values.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    seq_len: int
    d_in: int
    d_out: int
    K: int
    sigma: float
    gamma: float
    antithetic: bool
    dtype: str          # "f32" or "bf16"
    data_seed: int
    noise_seed: int
    target_kind: str    # "iid" (target ~ N(0,1)), "teacher" (bf16(X W'^T)),
                        # "local": scored against an error estimate
                        # E ~ N(0,1) (fp32) instead of a loss, or
                        # "head": a cross-entropy head, d_out = the vocabulary,
                        # labels uniform in [0, d_out); or "embedding": a token
                        # embedding table [d_in = vocabulary, d_out], Zipfian
                        # ids, target ~ N(0,1); or "attention": a block's
                        # cached queries, keys and values q, k, v ~ N(0,1)
                        # [T, d_out = heads * d_head] (bf16), the error
                        # estimate of its output E ~ N(0,1) (fp32) and the
                        # block's input X, one of q, k, v jittered (site)
    heads: int = 0      # attention: heads of width d_out / heads
    site: str = ""      # attention: "query", "key" or "value"

    @property
    def local(self) -> bool:
        return self.target_kind == "local"

    @property
    def head(self) -> bool:
        return self.target_kind == "head"

    @property
    def embedding(self) -> bool:
        return self.target_kind == "embedding"

    @property
    def attention(self) -> bool:
        return self.target_kind == "attention"

    @property
    def d_head(self) -> int:
        return self.d_out // self.heads if self.attention else 0

    @property
    def V(self) -> int:
        """Vocabulary size of a head (d_out) or an embedding (d_in)."""
        return self.d_out if self.head else (self.d_in if self.embedding else 0)

    @property
    def n_seq(self) -> int:
        return self.T // self.seq_len

    @property
    def n_slab(self) -> int:
        """256-column vocabulary slabs of a head (each its own site with K
        draws); 1 for the other layers."""
        return self.d_out // 256 if self.head else 1

    @property
    def rows(self) -> int:
        """Draw-token rows of one estimate: K*T, and K*T per slab for a
        head (K*T*V/256 slab-draw-token rows of 256 columns)."""
        return self.K * self.T * self.n_slab

    def describe(self) -> dict:
        d = {"workload": self.name, "T": self.T, "seq_len": self.seq_len,
             "d_in": self.d_in, "d_out": self.d_out, "K": self.K,
             "sigma": self.sigma, "gamma": self.gamma,
             "antithetic": self.antithetic, "dtype": self.dtype}
        if self.attention:
            d.update(heads=self.heads, d_head=self.d_head, site=self.site)
        return d


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_f32", 64, 64, 64, 64, 16, 1e-2, 0.0, False, "f32", 1001, 0, "iid"),
        Workload("bf16_layer", 4096, 512, 512, 512, 64, 1e-2, 0.0, True, "bf16", 1002, 0, "iid"),
        Workload("mlp_up_bf16", 16384, 512, 768, 3072, 256, 5e-3, 0.0, True, "bf16", 1003, 0, "teacher"),
        Workload("qkv_credit_bf16", 8192, 1024, 1024, 3072, 128, 1e-2, 0.9, False, "bf16", 1004, 0, "iid"),
        Workload("large_population_bf16", 2048, 1024, 1024, 1024, 4096, 1e-2, 0.5, True, "bf16", 1005, 0, "iid"),
        # The large population with plain draws (no antithetic pairs): the
        # single-generation walk for gamma > 0 then also carries each group's
        # noise sum and mean loss reduction for the centring.
        Workload("large_population_plain_bf16", 2048, 1024, 1024, 1024, 4096, 1e-2, 0.5, False,
                 "bf16", 1010, 0, "iid"),
        # Local scoring of attention internals ("What the released code
        # actually does", step 4) in the pages' 512-wide model and batches of
        # 8 sequences x 2048 tokens: keys / values (credit decay 0.98) and
        # queries (own token's score only).
        Workload("kv_local_bf16", 16384, 2048, 512, 512, 64, 0.2, 0.98, True, "bf16", 1006, 0, "local"),
        Workload("q_local_bf16", 16384, 2048, 512, 512, 64, 0.2, 0.0, True, "bf16", 1007, 0, "local"),
        # The untied head of the same model ("What the released code actually
        # does", step 5): a 4,096-token vocabulary jittered one 256-column
        # slab at a time, sigma = 0.05, 256 antithetic draws per slab
        # (4,096 slab draws per token), 8 sequences x 2048 tokens.
        Workload("head_ce_bf16", 16384, 2048, 512, 4096, 256, 0.05, 0.0, True, "bf16", 1008, 0, "head"),
        # The token embedding of the same model (step 7's scatter-add): a
        # 4,096 x 512 table, Zipfian token ids, the embedding's sigma 0.4,
        # own-token losses (gamma = 0), 8 sequences x 2048 tokens.
        Workload("embed_bf16", 16384, 2048, 4096, 512, 64, 0.4, 0.0, True, "bf16", 1009, 0, "embedding"),
        # Local scoring through the recomputed attention of one block of the
        # same model ("What the released code actually does", step 4): its
        # 512 channels as 4 heads of width 128 (the pages give no head
        # count), 8 sequences x 2048 tokens, the attention internals' sigma
        # 0.05 (SGD recipe), 64 antithetic draws; keys and values with credit
        # decay 0.98, queries with their own token's score only.
        Workload("attn_key_bf16", 16384, 2048, 512, 512, 64, 0.05, 0.98, True, "bf16", 1011, 0,
                 "attention", heads=4, site="key"),
        Workload("attn_value_bf16", 16384, 2048, 512, 512, 64, 0.05, 0.98, True, "bf16", 1012, 0,
                 "attention", heads=4, site="value"),
        Workload("attn_query_bf16", 16384, 2048, 512, 512, 64, 0.05, 0.0, True, "bf16", 1013, 0,
                 "attention", heads=4, site="query"),
    ]
}
WORKLOAD_ORDER = ["tiny_f32", "bf16_layer", "mlp_up_bf16", "qkv_credit_bf16",
                  "large_population_bf16", "large_population_plain_bf16", "kv_local_bf16",
                  "q_local_bf16", "head_ce_bf16", "embed_bf16", "attn_key_bf16",
                  "attn_value_bf16", "attn_query_bf16"]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns fp32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) << 16
    return rounded.astype(np.uint32).view(np.float32).reshape(x.shape)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """The upper 16 bits of fp32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not representable in bf16"
    return (b >> 16).astype(np.uint16)


def _round(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    return bf16_round(x32) if dtype == "bf16" else x32


def zipf_ids(rng: np.random.Generator, T: int, V: int) -> np.ndarray:
    """T token ids with Zipf-Mandelbrot frequencies p(rank r) ~ 1/(r + 2.7),
    the ranks assigned to ids by a random permutation."""
    p = 1.0 / (np.arange(1, V + 1, dtype=np.float64) + 2.7)
    p /= p.sum()
    ranked = rng.choice(V, size=T, p=p)
    return rng.permutation(V)[ranked].astype(np.int32)


def make_inputs(w: Workload, T: int | None = None, d_in: int | None = None,
                d_out: int | None = None, data_seed: int | None = None) -> dict:
    """X [T,d_in], W [d_out,d_in], target [T,d_out] as fp32 arrays holding the
    exact input values; for a local-scoring workload X and E [T,d_out] (fp32)
    instead, for a head X, W and int32 labels [T], and for an embedding the
    table [d_in, d_out], int32 ids [T] and target [T, d_out].  Sizes and seed
    default to the workload's."""
    T = w.T if T is None else T
    d_in = w.d_in if d_in is None else d_in
    d_out = w.d_out if d_out is None else d_out
    rng = np.random.default_rng(w.data_seed if data_seed is None else data_seed)
    if w.embedding:
        table = _round(rng.standard_normal((d_in, d_out)), w.dtype)
        ids = zipf_ids(rng, T, d_in)
        target = _round(rng.standard_normal((T, d_out)), w.dtype)
        return {"table": table, "ids": ids, "target": target}
    X = _round(rng.standard_normal((T, d_in)), w.dtype)
    if w.attention:
        q, k, v = (_round(rng.standard_normal((T, d_out)), w.dtype) for _ in range(3))
        return {"X": X, "q": q, "k": k, "v": v,
                "E": rng.standard_normal((T, d_out)).astype(np.float32)}
    if w.local:
        return {"X": X, "E": rng.standard_normal((T, d_out)).astype(np.float32)}
    W = _round(rng.standard_normal((d_out, d_in)) / np.sqrt(d_in), w.dtype)
    if w.head:
        return {"X": X, "W": W, "labels": rng.integers(0, d_out, size=T).astype(np.int32)}
    if w.target_kind == "teacher":
        # W' = W + E with E ~ N(0, 0.01) read as variance 0.01 (std 0.1).
        W_teacher = W.astype(np.float64) + 0.1 * rng.standard_normal((d_out, d_in))
        target = _round(X.astype(np.float64) @ W_teacher.T, w.dtype)
    else:
        target = _round(rng.standard_normal((T, d_out)), w.dtype)
    return {"X": X, "W": W, "target": target}


def attention_inputs(T: int, d_in: int, d_out: int, seed: int) -> dict:
    """Attention-site inputs of any shape with the recipe of the attention
    workloads: X [T,d_in], q, k, v [T,d_out] ~ N(0,1) rounded to bf16, E
    [T,d_out] ~ N(0,1) in fp32."""
    rng = np.random.default_rng(seed)
    X = _round(rng.standard_normal((T, d_in)), "bf16")
    q, k, v = (_round(rng.standard_normal((T, d_out)), "bf16") for _ in range(3))
    return {"X": X, "q": q, "k": k, "v": v,
            "E": rng.standard_normal((T, d_out)).astype(np.float32)}


def random_inputs(T: int, d_in: int, d_out: int, dtype: str, seed: int) -> dict:
    """Inputs of any shape with the iid recipe (X, target ~ N(0,1),
    W ~ N(0, 1/d_in)), for edge-case and ragged-shape tests."""
    rng = np.random.default_rng(seed)
    X = _round(rng.standard_normal((T, d_in)), dtype)
    W = _round(rng.standard_normal((d_out, d_in)) / np.sqrt(max(d_in, 1)), dtype)
    target = _round(rng.standard_normal((T, d_out)), dtype)
    return {"X": X, "W": W, "target": target}
