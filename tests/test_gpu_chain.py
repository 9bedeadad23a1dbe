"""Single generation for gamma > 0 (the chain path).

With a workspace of dust_workspace_bytes_seq bytes and no per-draw output
asked for, dust_estimate and dust_estimate_local walk each sequence in
reverse token order, two chains per wave, and generate every noise value
once ("Dust: every token is a member of the population", section "Perturb
the activations, not the weights": the credit recursion).  For an
antithetic pair centring and curvature cancel and
g_t = (2/K) sum_p R_t^p a_t^p with R_t = P_t + gamma R_(t+1); for plain
draws r_t^(i) = R_t^(i) - M_t with R_t^(i) = rho_t^(i) + gamma R_(t+1)^(i)
and M_t the same recursion over the draws' mean loss reduction, so
g_t = -1/(K sigma) (sum_i R_t^(i) a_t^(i) - M_t sum_i a_t^(i)).  Checked: parity with the fp64
oracle at the estimate's bars (2e-3 for bf16 inputs, 1e-5 for the fp32
path) on G_W, g and the clean loss; agreement with the two-pass path of the
same call (given only dust_workspace_bytes), which adds the draws in another
order, so the two differ by rounding only and are not bitwise equal (which
also shows that the chain path ran); every register layout the path has
(1 to 4 channel quads per lane, whole and ragged widths); the path switch a
request for per-draw outputs makes; bitwise reproducibility.  The
large-population workload at full size, in the benchmarked configuration,
is checked against the oracle over every sequence in test_gpu_parity.py.
Errors are measured over whole tensors and token by token (parity_util.py).
"""
import numpy as np
import pytest

from parity_util import assert_within, rel, report, stage_errors
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


def dtype_code(dtype):
    import token_activation_perturbation_amd as dust
    return dust.DUST_F32 if dtype == "f32" else dust.DUST_BF16


def run(inp, dtype, dev, two_pass=False, local=False, **kw):
    """dust_estimate (or _local with E) with the chain path's workspace, or
    with exactly the two-pass workspace."""
    import torch
    import token_activation_perturbation_amd as dust
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    X = torch.from_numpy(inp["X"]).to(dev).to(tdt).contiguous()
    T, d_in = inp["X"].shape
    d_out = inp["E" if local else "W"].shape[1 if local else 0]
    ws = None
    if two_pass:
        nbytes = dust.dust_workspace_bytes(T, d_in, d_out, kw["K"], kw["antithetic"],
                                           dtype_code(dtype))
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if local:
        E = torch.from_numpy(inp["E"]).to(dev).contiguous()
        out = dust.dust_estimate_local(X, E, want_g=True, workspace=ws, **kw)
    else:
        W = torch.from_numpy(inp["W"]).to(dev).to(tdt).contiguous()
        tg = torch.from_numpy(inp["target"]).to(dev).to(tdt).contiguous()
        out = dust.dust_estimate(X, W, tg, want_loss=True, want_g=True, workspace=ws, **kw)
    torch.cuda.synchronize(dev)
    return {k: v.cpu().numpy().astype(np.float64) for k, v in out.items()}


CASES = [
    # T, seq_len, d_in, d_out, K, sigma, gamma, dtype (antithetic pairs)
    (16, 8, 32, 64, 4096, 1e-2, 0.5, "bf16"),    # 2 sequences x 2048 pairs
    (12, 6, 24, 70, 4096, 1e-2, 0.9, "bf16"),    # ragged width: quads past d_out
    (16, 4, 16, 32, 1024, 1e-2, 1.0, "f32"),     # 4 x 512 pairs, gamma = 1
    (8, 2, 20, 1024, 4096, 5e-3, 0.3, "bf16"),   # the widest layer the path takes
    (16, 8, 32, 64, 4100, 1e-2, 0.7, "bf16"),    # 2050 pairs: a partial last group
    (8, 4, 24, 300, 2048, 1e-2, 0.6, "bf16"),    # 2 quads per lane, ragged quads
    (8, 4, 24, 512, 2048, 1e-2, 0.8, "bf16"),    # 2 quads per lane, whole
    (8, 4, 24, 700, 2048, 1e-2, 0.5, "bf16"),    # 3 quads per lane
    (8, 4, 24, 1022, 2048, 1e-2, 0.9, "bf16"),   # 4 quads per lane, d_out % 4 != 0
]
PLAIN_CASES = [
    # T, seq_len, d_in, d_out, K, sigma, gamma, dtype (plain draws: K chains per sequence)
    (8, 4, 24, 300, 1024, 1e-2, 0.6, "bf16"),    # 2 sequences x 1024 draws, ragged quads
    (16, 8, 32, 64, 1030, 1e-2, 0.7, "bf16"),    # 1030 draws: a partial last group
    (8, 4, 16, 1022, 1024, 5e-3, 0.9, "f32"),    # 4 quads per lane, ragged, fp32
    (8, 2, 20, 512, 512, 1e-2, 1.0, "bf16"),     # 4 x 512 draws, gamma = 1: suffix sums
    (12, 6, 24, 700, 1024, 1e-2, 0.5, "bf16"),   # 3 quads per lane
]


ALL_CASES = [c + (True,) for c in CASES] + [c + (False,) for c in PLAIN_CASES]


@pytest.mark.parametrize("case", ALL_CASES,
                         ids=[f"T{c[0]}_L{c[1]}_dout{c[3]}_K{c[4]}_g{c[6]}_{c[7]}_"
                              f"{'pairs' if c[8] else 'plain'}" for c in ALL_CASES])
def test_chain_parity_with_oracle_and_two_pass(dev, oracle_mod, threads, case):
    import token_activation_perturbation_amd as dust
    T, seq_len, d_in, d_out, K, sigma, gamma, dtype, anti = case
    print(f"chain parity {case}", flush=True)
    code = dtype_code(dtype)
    assert dust.dust_workspace_bytes_seq(T, d_in, d_out, seq_len, K, gamma, anti, code) > \
        dust.dust_workspace_bytes(T, d_in, d_out, K, anti, code)
    inp = synth.random_inputs(T, d_in, d_out, dtype, seed=T * 13 + d_out + K)
    kw = dict(K=K, sigma=sigma, gamma=gamma, seed=K + 3, antithetic=anti, seq_len=seq_len)
    chain = run(inp, dtype, dev, **kw)
    two = run(inp, dtype, dev, two_pass=True, **kw)
    ref = oracle_mod.estimate(inp["X"], inp["W"], inp["target"], threads=threads, **kw)
    errs = stage_errors(chain, ref, keys=("loss", "g"))
    errs["vs_two_pass"] = rel(chain["G_W"], two["G_W"])
    report("  rel err", errs)
    assert_within(errs, dtype)
    assert_within(stage_errors(two, ref, keys=("loss", "g")), dtype)
    assert not np.array_equal(chain["g"], two["g"])


def test_asking_for_per_draw_outputs_keeps_G_within_the_bar(dev, oracle_mod, threads):
    """On a chain-eligible call, asking for rho or the credit switches to the
    two-pass path (every draw's centred credit is then formed): G_W changes
    by rounding only, and the per-draw outputs match the oracle token by
    token."""
    import torch
    import token_activation_perturbation_amd as dust
    T, seq_len, d_in, d_out, K = 8, 4, 40, 256, 2048
    inp = synth.random_inputs(T, d_in, d_out, "bf16", seed=77)
    kw = dict(K=K, sigma=1e-2, gamma=0.7, seed=5, antithetic=True, seq_len=seq_len)
    X, W, tg = (torch.from_numpy(inp[k]).to(dev).to(torch.bfloat16).contiguous()
                for k in ("X", "W", "target"))
    bare = dust.dust_estimate(X, W, tg, **kw)["G_W"].cpu().numpy().astype(np.float64)
    full = dust.dust_estimate(X, W, tg, want_rho=True, want_reward=True, want_g=True, **kw)
    torch.cuda.synchronize(dev)
    full = {k: v.cpu().numpy().astype(np.float64) for k, v in full.items()}
    ref = oracle_mod.estimate(inp["X"], inp["W"], inp["target"], threads=threads, **kw)
    errs = stage_errors(full, ref, keys=("rho", "reward", "g"))
    errs["bare_G_W"] = rel(bare, ref["G"])
    errs["full_vs_bare"] = rel(full["G_W"], bare)
    report("  path switch", errs)
    assert_within(errs, "bf16")
    assert not np.array_equal(full["G_W"], bare)  # the two paths really differ


@pytest.mark.parametrize("anti", [True, False], ids=["pairs", "plain"])
def test_chain_local_scoring(dev, oracle_mod, threads, anti):
    """dust_estimate_local: keys/values-style scoring with gamma = 0.98 (no
    curvature term: the score is linear in the jitter)."""
    T, seq_len, d_in, d_out, K = 16, 8, 32, 64, 4096 if anti else 2048
    rng = np.random.default_rng(41)
    inp = synth.random_inputs(T, d_in, d_out, "bf16", seed=41)
    inp["E"] = rng.standard_normal((T, d_out)).astype(np.float32)
    kw = dict(K=K, sigma=0.2, gamma=0.98, seed=9, antithetic=anti, seq_len=seq_len)
    chain = run(inp, "bf16", dev, local=True, **kw)
    two = run(inp, "bf16", dev, local=True, two_pass=True, **kw)
    ref = oracle_mod.estimate_local(inp["X"], inp["E"], threads=threads, **kw)
    errs = stage_errors(chain, ref, keys=("g",))
    errs["vs_two_pass"] = rel(chain["g"], two["g"])
    report("  local rel err", errs)
    assert_within(errs, "bf16")
    assert not np.array_equal(chain["g"], two["g"])


@pytest.mark.parametrize("anti", [True, False], ids=["pairs", "plain"])
def test_chain_bitwise_deterministic(dev, anti):
    inp = synth.random_inputs(16, 32, 64, "bf16", seed=5)
    kw = dict(K=4096 if anti else 2048, sigma=1e-2, gamma=0.5, seed=1, antithetic=anti,
              seq_len=8)
    a = run(inp, "bf16", dev, **kw)
    b = run(inp, "bf16", dev, **kw)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
