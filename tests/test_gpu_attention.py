"""Parity of dust_estimate_attention (scores through a recomputed causal
attention, "Dust: every token is a member of the population", section "What
the released code actually does", step 4) with the fp64 oracle, which
recomputes the jittered attention literally.

Every stage output (rho, the centred credit, g, G_W) is held to the bf16 bars
of parity_util.py, whole and token by token, over the three sites, antithetic
pairs and plain draws, both head widths, sequences that fill whole 64-token
blocks and ragged ones, one-token sequences, a large sigma (logit changes
past the series branch of e^x - 1), gamma 0, between and 1, and a call
without the block's input (g only).  At the attention workloads' full size
the scores of sampled draws of one sequence are compared with the oracle
run on that sequence alone (a draw's score does not depend on the others),
and g and G_W are checked against their definitions from the GPU's own
credit and the oracle's noise.
"""
import numpy as np
import pytest

from parity_util import assert_within, rel, report, rows_rel, stage_errors
from token_activation_perturbation_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import token_activation_perturbation_amd as dust
    dust._load()
    return torch.device("cuda:0")


@pytest.fixture(scope="module")
def threads(oracle_mod):
    return min(16, oracle_mod.default_threads())


def to_dev(dev, a, bf16=True):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return (t.to(torch.bfloat16) if bf16 else t).contiguous()


def run_case(dev, oracle_mod, threads, *, site, n_seq, L, heads, d_head, d_in, K, sigma, gamma,
             antithetic, seed, with_x=True):
    import torch
    import token_activation_perturbation_amd as dust
    T, D = n_seq * L, heads * d_head
    print(f"attention {site} n_seq={n_seq} L={L} H={heads} dh={d_head} d_in={d_in} K={K} "
          f"sigma={sigma} gamma={gamma} anti={antithetic} x={with_x}", flush=True)
    inp = synth.attention_inputs(T, d_in, D, seed=seed % 100003)
    X = to_dev(dev, inp["X"]) if with_x else None
    q, k, v = (to_dev(dev, inp[n]) for n in ("q", "k", "v"))
    E = to_dev(dev, inp["E"], bf16=False)
    kw = dict(K=K, sigma=sigma, gamma=gamma, seed=seed, antithetic=antithetic, seq_len=L)
    got = dust.dust_estimate_attention(X, q, k, v, E, heads=heads, site=site, want_rho=True,
                                       want_reward=True, want_g=True, **kw)
    torch.cuda.synchronize(dev)
    got = {n: t.cpu().numpy().astype(np.float64) for n, t in got.items()}
    ref = oracle_mod.estimate_attention(inp["X"] if with_x else None, inp["q"], inp["k"],
                                        inp["v"], inp["E"], heads=heads, site=site,
                                        threads=threads, **kw)
    errs = stage_errors(got, ref, keys=("rho", "reward", "g"))
    report("  rel err", errs)
    assert_within(errs, "bf16")
    if not with_x:
        assert "G_W" not in got
    return got, ref


SITES = ("query", "key", "value")


@pytest.mark.parametrize("site", SITES)
@pytest.mark.parametrize("antithetic", [True, False])
@pytest.mark.parametrize("d_head", [64, 128])
def test_sites_ragged(dev, oracle_mod, threads, site, antithetic, d_head):
    # 100-token sequences: two 64-token blocks, the second ragged
    run_case(dev, oracle_mod, threads, site=site, n_seq=2, L=100, heads=2, d_head=d_head,
             d_in=48, K=8 if antithetic else 6, sigma=0.05,
             gamma=0.0 if site == "query" else 0.9, antithetic=antithetic,
             seed=7100 + 10 * d_head + SITES.index(site) + (0 if antithetic else 3))


@pytest.mark.parametrize("site", SITES)
@pytest.mark.parametrize("L,n_seq", [(64, 3), (1, 40), (65, 2), (200, 1)])
def test_sequence_lengths(dev, oracle_mod, threads, site, L, n_seq):
    run_case(dev, oracle_mod, threads, site=site, n_seq=n_seq, L=L, heads=3, d_head=64, d_in=64,
             K=10, sigma=0.02, gamma=0.98 if site != "query" else 0.0, antithetic=True,
             seed=7200 + L + SITES.index(site))


@pytest.mark.parametrize("site", SITES)
def test_large_sigma_and_gamma_one(dev, oracle_mod, threads, site):
    # sigma = 0.5: logit changes of ~0.5 and more take e^x - 1 from the
    # exponential rather than the series
    run_case(dev, oracle_mod, threads, site=site, n_seq=2, L=130, heads=2, d_head=128, d_in=100,
             K=6, sigma=0.5, gamma=1.0, antithetic=False, seed=7300 + SITES.index(site))


@pytest.mark.parametrize("site", SITES)
def test_without_input_matrix(dev, oracle_mod, threads, site):
    run_case(dev, oracle_mod, threads, site=site, n_seq=2, L=96, heads=2, d_head=64, d_in=1,
             K=4, sigma=0.05, gamma=0.5, antithetic=True, seed=7400 + SITES.index(site),
             with_x=False)


@pytest.mark.parametrize("site", SITES)
def test_several_blocks_many_draws(dev, oracle_mod, threads, site):
    # six blocks per sequence and more noise groups than one workgroup round
    run_case(dev, oracle_mod, threads, site=site, n_seq=2, L=384, heads=2, d_head=128,
             d_in=128, K=34, sigma=0.05, gamma=0.98 if site != "query" else 0.0,
             antithetic=True, seed=7500 + SITES.index(site))


def test_repeat_calls_are_bitwise_equal(dev):
    import torch
    import token_activation_perturbation_amd as dust
    inp = synth.attention_inputs(2 * 100, 32, 128, seed=77)
    X, q, k, v = (to_dev(dev, inp[n]) for n in ("X", "q", "k", "v"))
    E = to_dev(dev, inp["E"], bf16=False)
    kw = dict(heads=2, site="key", K=8, sigma=0.05, gamma=0.9, seed=5, antithetic=True,
              seq_len=100, want_rho=True, want_g=True)
    a = dust.dust_estimate_attention(X, q, k, v, E, **kw)
    b = dust.dust_estimate_attention(X, q, k, v, E, **kw)
    torch.cuda.synchronize(dev)
    for n in ("G_W", "rho", "g"):
        assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("name", ["attn_key_bf16", "attn_value_bf16", "attn_query_bf16"])
def test_full_size_sampled(dev, oracle_mod, name):
    """The attention workloads at full size, as the bench runs them: the
    scores of draws 0 and 1 of one sequence against the oracle on that
    sequence with K = 2 (a draw's noise and score do not depend on K or on
    the other draws); g on sampled tokens against -1/(K sigma) sum_i r_i
    s_i a_i from the GPU's own credit and the oracle's noise; G_W on sampled
    rows against sum_t g_t x_t^T from the GPU's g."""
    import torch
    import token_activation_perturbation_amd as dust
    w = synth.WORKLOADS[name]
    inp = synth.make_inputs(w)
    X, q, k, v = (to_dev(dev, inp[n]) for n in ("X", "q", "k", "v"))
    E = to_dev(dev, inp["E"], bf16=False)
    kw = dict(K=w.K, sigma=w.sigma, gamma=w.gamma, seed=w.noise_seed, antithetic=w.antithetic,
              seq_len=w.seq_len)
    got = dust.dust_estimate_attention(X, q, k, v, E, heads=w.heads, site=w.site, want_rho=True,
                                       want_reward=True, want_g=True, **kw)
    torch.cuda.synchronize(dev)
    rho = got["rho"].cpu().numpy().astype(np.float64)
    reward = got["reward"].cpu().numpy().astype(np.float64)
    g = got["g"].cpu().numpy().astype(np.float64)
    G = got["G_W"].cpu().numpy().astype(np.float64)
    assert np.isfinite(G).all()
    seq = 5
    sl = slice(seq * w.seq_len, (seq + 1) * w.seq_len)
    ref = oracle_mod.estimate_attention(None, inp["q"], inp["k"], inp["v"], inp["E"],
                                        heads=w.heads, site=w.site, K=2, sigma=w.sigma,
                                        gamma=w.gamma, seed=w.noise_seed,
                                        antithetic=w.antithetic, seq_len=w.seq_len,
                                        seq_range=(seq, seq + 1), threads=1)
    e_rho = rel(rho[sl, :2], ref["rho"])
    e_rho_row, _ = rows_rel(rho[sl, :2], ref["rho"])
    # g from its definition on sampled tokens
    rng = np.random.default_rng(3)
    toks = rng.choice(w.T, size=6, replace=False)
    K_n = w.K // 2 if w.antithetic else w.K
    g_ref = np.zeros((len(toks), w.d_out))
    for j, t in enumerate(toks):
        _, a = oracle_mod.noise_fill(w.noise_seed, 0, K_n, int(t), 1, w.d_out)
        a = a.reshape(K_n, w.d_out)
        if w.antithetic:
            wgt = reward[t, 0::2] - reward[t, 1::2]
        else:
            wgt = reward[t]
        g_ref[j] = -(wgt @ a) / (w.K * w.sigma)
    e_g = rel(g[toks], g_ref)
    rows = rng.choice(w.d_out, size=8, replace=False)
    G_ref = g[:, rows].T @ inp["X"].astype(np.float64)
    e_G = rel(G[rows], G_ref)
    report(f"  {name}", {"rho": e_rho, "rho_row": e_rho_row, "g": e_g, "G_W": e_G})
    assert_within({"rho": e_rho, "rho_row": e_rho_row, "g": e_g, "G_W": e_G}, "bf16")


def draw_attention_case(i):
    rng = np.random.default_rng(9500 + i)
    anti = bool(rng.integers(0, 2))
    site = SITES[int(rng.integers(0, 3))]
    return dict(site=site, n_seq=int(rng.integers(1, 4)), L=int(rng.integers(1, 301)),
                heads=int(rng.integers(1, 5)), d_head=int(rng.choice([64, 128])),
                d_in=int(rng.choice([1, 16, 48, 100])),
                K=int(rng.integers(1, 13)) * 2 if anti else int(rng.integers(2, 25)),
                sigma=float(10 ** rng.uniform(-3, -0.5)),
                gamma=float(rng.choice([0.0, 1.0, rng.uniform(0.05, 0.99)])),
                antithetic=anti, seed=int(rng.integers(0, 2**62)),
                with_x=bool(rng.integers(0, 4) > 0))


RANDOM_CASES = [draw_attention_case(i) for i in range(16)]


@pytest.mark.parametrize("c", RANDOM_CASES, ids=[
    f"{c['site']}_S{c['n_seq']}_L{c['L']}_H{c['heads']}x{c['d_head']}_K{c['K']}"
    f"{'_pairs' if c['antithetic'] else '_plain'}_g{c['gamma']:.2f}{'' if c['with_x'] else '_nox'}"
    for c in RANDOM_CASES])
def test_random_shapes(dev, oracle_mod, threads, c):
    """Seeded random cases, every parameter at once: sequence count and
    length (ragged and one-token), heads and width, site, draw kind, K,
    sigma (1e-3 to 0.3, so some logit changes take the exponential form of
    e^x - 1), gamma and the block's input present or not."""
    run_case(dev, oracle_mod, threads, **c)
