"""Parity of the HIP path with the fp64 oracle on seeded random shapes.

The hand-picked shapes of test_gpu_parity.py cover the edges one at a time;
these cases draw every parameter at once from a fixed seed: sequence count
and length (so T, and the credit scan's restarts), d_in and d_out from 1 up
(ragged widths, widths below one quad, several quads per lane), K, sigma,
gamma (0, 1 and between), antithetic or plain draws, bf16 or fp32 inputs,
and the layer loss or local scoring against a supplied error estimate
("Dust: every token is a member of the population", section "Perturb the
activations, not the weights" for the estimator; "What the released code
actually does", step 4 for local scoring).  Every stage output is held to
the bars of parity_util.py, whole and token by token, and a second call
without per-draw outputs must give G_W within the bar of the first (it may
take another kernel variant or path).
"""
import numpy as np
import pytest

from parity_util import assert_within, rel, report, stage_errors
from token_activation_perturbation_amd import synth

pytestmark = pytest.mark.gpu

N_CASES = 40


def draw_case(i):
    rng = np.random.default_rng(9000 + i)
    n_seq = int(rng.integers(1, 5))
    seq_len = int(rng.integers(1, 49))
    d_in = int(rng.choice([1, 3, 8, 17, 64, 100, 200]))
    d_out = int(rng.choice([1, 2, 5, 64, 130, 256, 300, 511, 600]))
    anti = bool(rng.integers(0, 2))
    K = int(rng.integers(1, 49)) * 2 if anti else int(rng.integers(2, 97))
    gamma = float(rng.choice([0.0, 1.0, rng.uniform(0.05, 0.99)]))
    sigma = float(10 ** rng.uniform(-3, -1))
    dtype = "bf16" if rng.integers(0, 4) else "f32"
    local = bool(rng.integers(0, 4) == 0)
    return dict(T=n_seq * seq_len, seq_len=seq_len, d_in=d_in, d_out=d_out, K=K,
                antithetic=anti, gamma=gamma, sigma=sigma, dtype=dtype, local=local,
                seed=int(rng.integers(0, 2**63)))


CASES = [draw_case(i) for i in range(N_CASES)]


def case_id(c):
    return (f"T{c['T']}_L{c['seq_len']}_din{c['d_in']}_dout{c['d_out']}_K{c['K']}_"
            f"{'pairs' if c['antithetic'] else 'plain'}_g{c['gamma']:.2f}_{c['dtype']}"
            f"{'_local' if c['local'] else ''}")


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


@pytest.mark.parametrize("c", CASES, ids=[case_id(c) for c in CASES])
def test_random_shape_parity(dev, oracle_mod, threads, c):
    import torch
    import token_activation_perturbation_amd as dust
    print(f"random shape {case_id(c)}", flush=True)
    inp = synth.random_inputs(c["T"], c["d_in"], c["d_out"], c["dtype"], seed=c["seed"] % 100003)
    kw = dict(K=c["K"], sigma=c["sigma"], gamma=c["gamma"], seed=c["seed"],
              antithetic=c["antithetic"], seq_len=c["seq_len"])
    tdt = torch.float32 if c["dtype"] == "f32" else torch.bfloat16
    X = torch.from_numpy(inp["X"]).to(dev).to(tdt).contiguous()
    full_kw = dict(want_rho=True, want_reward=True, want_g=True)
    if c["local"]:
        E = np.random.default_rng(c["seed"] % 99991).standard_normal(
            (c["T"], c["d_out"])).astype(np.float32)
        Ed = torch.from_numpy(E).to(dev).contiguous()
        full = dust.dust_estimate_local(X, Ed, **full_kw, **kw)
        bare = dust.dust_estimate_local(X, Ed, **kw)["G_W"]
        ref = oracle_mod.estimate_local(inp["X"], E, threads=threads, **kw)
        keys = ("rho", "reward", "g")
    else:
        W = torch.from_numpy(inp["W"]).to(dev).to(tdt).contiguous()
        tg = torch.from_numpy(inp["target"]).to(dev).to(tdt).contiguous()
        full = dust.dust_estimate(X, W, tg, want_loss=True, **full_kw, **kw)
        bare = dust.dust_estimate(X, W, tg, **kw)["G_W"]
        ref = oracle_mod.estimate(inp["X"], inp["W"], inp["target"], threads=threads, **kw)
        keys = ("loss", "rho", "reward", "g")
    torch.cuda.synchronize(dev)
    got = {k: v.cpu().numpy().astype(np.float64) for k, v in full.items()}
    errs = stage_errors(got, ref, keys=keys)
    errs["bare_vs_full"] = rel(bare.cpu().numpy().astype(np.float64), got["G_W"])
    report("  rel err", errs)
    assert_within(errs, c["dtype"])
