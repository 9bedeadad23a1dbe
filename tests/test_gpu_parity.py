"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Tolerances.  The estimate's own bar: G_W within relative Frobenius error
2e-3 for bf16 inputs with fp32 accumulation and 1e-5 for the fp32 path.  The
intermediate stages (per-token loss L_t, loss reductions rho, credit r,
error estimate g) are held to the same relative level, both over the whole
tensor and token by token (each row of G_W likewise; parity_util.py).
Noise words are compared bit for bit; Gaussians within GAUSS_ABS_TOL
(derivation in the comment there).
"""
import numpy as np
import pytest

from parity_util import TOL, assert_within, rel, report, stage_errors
from token_activation_perturbation_amd import synth

pytestmark = pytest.mark.gpu

# fp32 Box-Muller from the hardware transcendentals: v_log_f32, v_sqrt_f32,
# v_sin_f32 and v_cos_f32 are each accurate to a few ulp over the ranges used
# (u in [2^-23, 1]; the angle in revolutions in [1, 2), whose fraction is
# v); with |a| <= 5.65 a few ulp of the largest values is about 2e-6, so
# 1e-5 absolute leaves a 5x margin.
GAUSS_ABS_TOL = 1e-5


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


def to_dev(inp, dtype, dev):
    import torch
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    return [torch.from_numpy(inp[k]).to(dev).to(tdt).contiguous() for k in ("X", "W", "target")]


def gpu_estimate(inp, dtype, dev, **kw):
    import torch
    import token_activation_perturbation_amd as dust
    Xd, Wd, td = to_dev(inp, dtype, dev)
    out = dust.dust_estimate(Xd, Wd, td, want_loss=True, want_rho=True, want_reward=True,
                             want_g=True, **kw)
    torch.cuda.synchronize(dev)
    return {k: v.cpu().numpy().astype(np.float64) for k, v in out.items()}


# --------------------------------------------------------------------------
# Noise


NOISE_CASES = [
    # seed, n0, n_cnt, t0, t_cnt, d_out
    (0, 0, 4, 0, 64, 64),
    ((7 << 32) | 99, 3, 5, 1000, 17, 13),
    (2**64 - 1, 2**31 - 8, 4, 2**31 - 20, 10, 38),
    (12345, 100, 2, 4000, 3, 3072),
]


@pytest.mark.parametrize("case", NOISE_CASES)
def test_noise_words_bit_exact_and_gaussians(dev, oracle_mod, case):
    import torch
    import token_activation_perturbation_amd as dust
    seed, n0, n_cnt, t0, t_cnt, d_out = case
    print(f"noise case {case}", flush=True)
    w_gpu, g_gpu = dust.dust_noise_fill(seed, n0, n_cnt, t0, t_cnt, d_out, device=dev)
    torch.cuda.synchronize(dev)
    w_ref, g_ref = oracle_mod.noise_fill(seed, n0, n_cnt, t0, t_cnt, d_out)
    assert np.array_equal(w_gpu.cpu().numpy().view(np.uint32), w_ref)
    err = np.abs(g_gpu.cpu().numpy().astype(np.float64) - g_ref)
    print(f"  gauss max abs err {err.max():.3e}, rms {np.sqrt((err**2).mean()):.3e}", flush=True)
    assert err.max() <= GAUSS_ABS_TOL


def test_gaussian_error_over_many_values(dev, oracle_mod):
    """4M Gaussians: the worst case of the fp32 transform, including the
    extremes of u (tails) and v (angles near 0 and 1)."""
    import torch
    import token_activation_perturbation_amd as dust
    _, g_gpu = dust.dust_noise_fill(3, 0, 16, 0, 1024, 256, words=False, device=dev)
    torch.cuda.synchronize(dev)
    _, g_ref = oracle_mod.noise_fill(3, 0, 16, 0, 1024, 256, words=False)
    err = np.abs(g_gpu.cpu().numpy().astype(np.float64) - g_ref)
    relerr = err / np.maximum(np.abs(g_ref), 1e-3)
    print(f"gauss 4M: max abs {err.max():.3e} rms {np.sqrt((err**2).mean()):.3e} "
          f"max rel(|a|>1e-3) {relerr.max():.3e}", flush=True)
    assert err.max() <= GAUSS_ABS_TOL


# --------------------------------------------------------------------------
# Stage parity on small shapes (several tiles, ragged tails, every option)

SMALL = [
    # T, seq_len, d_in, d_out, K, sigma, gamma, antithetic, dtype
    (64, 64, 64, 64, 16, 1e-2, 0.0, False, "f32"),
    (192, 64, 96, 160, 32, 1e-2, 0.0, True, "bf16"),
    (130, 26, 45, 37, 10, 2e-2, 0.5, False, "bf16"),     # ragged everything
    (96, 32, 72, 300, 34, 5e-3, 0.9, True, "bf16"),      # K_n = 17: ragged batches
    (64, 16, 33, 19, 6, 1e-2, 1.0, False, "f32"),        # gamma = 1: suffix sums
    (40, 1, 24, 8, 2, 1e-1, 0.7, True, "bf16"),          # one-token sequences, K = 2
    (1, 1, 1, 1, 2, 1e-2, 0.0, False, "f32"),            # the smallest problem
    (256, 128, 128, 1024, 64, 1e-2, 0.5, True, "bf16"),  # d_out spans 4 quad rounds
    (140, 70, 40, 52, 8, 1e-2, 0.95, True, "bf16"),      # credit chunks 32 + 32 + 6
    (99, 33, 16, 24, 4, 1e-2, 1.0, False, "f32"),        # chunks 32 + 1, suffix sums
    (1000, 500, 64, 72, 8, 1e-2, 0.0, True, "bf16"),     # aligned: 2 token splits, ragged tail
    (64, 64, 8, 16, 4, 1e-2, 0.0, False, "bf16"),        # d_in = 8: one k-block, 7 chunks zeroed
    (300, 100, 392, 520, 8, 1e-2, 0.0, True, "bf16"),    # 8-wide edge tiles, 44-token tail
    (1000, 250, 1024, 200, 8, 1e-2, 0.5, False, "bf16"), # wide input, 104-token tail, two passes
]


@pytest.mark.parametrize("case", SMALL, ids=[f"T{c[0]}_dout{c[3]}_K{c[4]}_g{c[6]}_{c[8]}" for c in SMALL])
def test_stage_parity_small(dev, oracle_mod, threads, case):
    T, seq_len, d_in, d_out, K, sigma, gamma, anti, dtype = case
    print(f"stage parity case {case}", flush=True)
    inp = synth.random_inputs(T, d_in, d_out, dtype, seed=T * 7 + d_out)
    kw = dict(K=K, sigma=sigma, gamma=gamma, seed=T + 11, antithetic=anti, seq_len=seq_len)
    got = gpu_estimate(inp, dtype, dev, **kw)
    ref = oracle_mod.estimate(inp["X"], inp["W"], inp["target"], threads=threads, **kw)
    errs = stage_errors(got, ref)
    report("  rel err", errs)
    assert_within(errs, dtype)


# --------------------------------------------------------------------------
# The five workloads at full size


@pytest.mark.parametrize("name", ["tiny_f32", "bf16_layer"])
def test_workload_full_parity(dev, oracle_mod, threads, name):
    w = synth.WORKLOADS[name]
    print(f"full parity {name}", flush=True)
    inp = synth.make_inputs(w)
    kw = dict(K=w.K, sigma=w.sigma, gamma=w.gamma, seed=w.noise_seed, antithetic=w.antithetic,
              seq_len=w.seq_len)
    got = gpu_estimate(inp, w.dtype, dev, **kw)
    ref = oracle_mod.estimate(inp["X"], inp["W"], inp["target"], threads=threads, **kw)
    errs = stage_errors(got, ref)
    report(f"  {name}", errs)
    assert_within(errs, w.dtype)


@pytest.mark.parametrize("name", ["mlp_up_bf16", "qkv_credit_bf16", "large_population_bf16"])
def test_workload_full_size_oracle(dev, oracle_mod, threads, name):
    """Full size, the call bench.py times (its workspace, which lets the
    gamma > 0 antithetic workload take the single-generation chain path; G_W
    only), against the oracle over every sequence: G_W whole and row by
    row.  A second call with the clean loss and g asked for (the same path:
    neither changes the kernels) must give the same G_W bit for bit, and its
    g and L_t are checked token by token.  A third call asks for the
    per-draw outputs rho and r (the two-pass path where the bare call took
    the chain), which are checked token by token, and whose G_W must agree
    with the bare call's within the bar."""
    import torch
    import token_activation_perturbation_amd as dust
    w = synth.WORKLOADS[name]
    print(f"full-size oracle parity {name}", flush=True)
    inp = synth.make_inputs(w)
    kw = dict(K=w.K, sigma=w.sigma, gamma=w.gamma, seed=w.noise_seed, antithetic=w.antithetic,
              seq_len=w.seq_len)
    Xd, Wd, td = to_dev(inp, w.dtype, dev)
    code = dust.DUST_BF16 if w.dtype == "bf16" else dust.DUST_F32
    ws = torch.empty(dust.dust_workspace_bytes_seq(w.T, w.d_in, w.d_out, w.seq_len, w.K, w.gamma,
                                                   w.antithetic, code),
                     dtype=torch.uint8, device=dev)
    bare = dust.dust_estimate(Xd, Wd, td, workspace=ws, **kw)["G_W"].clone()
    lg = dust.dust_estimate(Xd, Wd, td, want_loss=True, want_g=True, workspace=ws, **kw)
    torch.cuda.synchronize(dev)
    assert torch.equal(bare, lg["G_W"])
    got = {"G_W": bare.cpu().numpy().astype(np.float64),
           "g": lg["g"].cpu().numpy().astype(np.float64),
           "loss": lg["loss"].cpu().numpy().astype(np.float64)}
    del lg
    ref = oracle_mod.estimate(inp["X"], inp["W"], inp["target"], threads=threads, **kw)
    errs = stage_errors(got, ref)
    errs["G_W_vs_gTX"] = rel(got["G_W"], got["g"].T @ inp["X"].astype(np.float64))
    report(f"  {name} (bench call)", errs)
    assert_within(errs, w.dtype)
    full = gpu_estimate(inp, w.dtype, dev, **kw)
    errs = stage_errors(full, ref, keys=("rho", "reward"), g_key="none")
    errs["G_W_vs_bare"] = rel(full["G_W"], got["G_W"])
    report(f"  {name} (per-draw outputs)", errs)
    assert_within(errs, w.dtype)


@pytest.mark.parametrize("T,d_out", [(256, 3072), (128, 4096)], ids=["qpl12", "qpl16"])
def test_bare_and_full_calls_agree_bitwise(dev, T, d_out):
    """The single-generation kernel skips ||a||^2 when an antithetic call asks
    for no per-draw output (the bare call bench.py times); its reduction slot
    then carries zeros, so P, g and G_W must equal those of the call that
    forms it bit for bit, at the widest register layouts (12 and 16 channel
    quads per lane)."""
    import torch
    import token_activation_perturbation_amd as dust
    inp = synth.random_inputs(T, 64, d_out, "bf16", seed=d_out)
    Xd, Wd, td = to_dev(inp, "bf16", dev)
    kw = dict(K=16, sigma=1e-2, gamma=0.0, seed=4, antithetic=True, seq_len=T)
    bare = dust.dust_estimate(Xd, Wd, td, want_g=True, **kw)
    full = dust.dust_estimate(Xd, Wd, td, want_loss=True, want_rho=True, want_reward=True,
                              want_g=True, **kw)
    torch.cuda.synchronize(dev)
    assert torch.equal(bare["G_W"], full["G_W"])
    assert torch.equal(bare["g"], full["g"])


# --------------------------------------------------------------------------
# Determinism and the statistical law on GPU outputs


def test_bitwise_deterministic(dev):
    w = synth.WORKLOADS["bf16_layer"]
    inp = synth.make_inputs(w, T=1024)
    kw = dict(K=w.K, sigma=w.sigma, gamma=0.5, seed=5, antithetic=w.antithetic,
              seq_len=w.seq_len)
    a = gpu_estimate(inp, w.dtype, dev, **kw)
    b = gpu_estimate(inp, w.dtype, dev, **kw)
    for k in a:
        assert np.array_equal(a[k], b[k]), k


def test_gpu_cosine_law(dev, oracle_mod):
    """Per-token cosine of g_t to delta_t about sqrt(K_e/(K_e+D+1)) ("What a
    zeroth-order gradient is"), on the bf16 layer workload (K_e = 32 pairs,
    D = 512): 0.242."""
    w = synth.WORKLOADS["bf16_layer"]
    inp = synth.make_inputs(w)
    got = gpu_estimate(inp, w.dtype, dev, K=w.K, sigma=w.sigma, gamma=w.gamma,
                       seed=w.noise_seed, antithetic=w.antithetic, seq_len=w.seq_len)
    delta, _ = oracle_mod.true_gradient(inp["X"], inp["W"], inp["target"])
    g = got["g"]
    cos = (g * delta).sum(1) / np.linalg.norm(g, axis=1) / np.linalg.norm(delta, axis=1)
    pred = np.sqrt(32 / (32 + 512 + 1))
    print(f"cosine mean {cos.mean():.4f} predicted {pred:.4f}", flush=True)
    assert abs(cos.mean() - pred) < 0.01


# --------------------------------------------------------------------------
# Paths, options and the boundary's behaviour on the device


def test_two_pass_fallback_at_gamma_zero(dev, oracle_mod, threads):
    """d_out above the single-generation kernel's register budget (4096
    channels) takes the two-pass path even for gamma = 0."""
    T, d_in, d_out = 32, 16, 4100
    inp = synth.random_inputs(T, d_in, d_out, "bf16", seed=77)
    kw = dict(K=4, sigma=1e-2, gamma=0.0, seed=3, antithetic=True, seq_len=16)
    got = gpu_estimate(inp, "bf16", dev, **kw)
    ref = oracle_mod.estimate(inp["X"], inp["W"], inp["target"], threads=threads, **kw)
    errs = {"g": rel(got["g"], ref["g"]), "G_W": rel(got["G_W"], ref["G"]),
            "reward": rel(got["reward"], ref["reward"])}
    report("  two-pass at gamma 0", errs)
    for k, v in errs.items():
        assert v <= TOL["bf16"], (k, v)


@pytest.mark.parametrize("gamma", [0.0, 0.5])
def test_optional_outputs_do_not_change_G(dev, gamma):
    import torch
    import token_activation_perturbation_amd as dust
    w = synth.WORKLOADS["bf16_layer"]
    inp = synth.make_inputs(w, T=1024)
    Xd, Wd, td = to_dev(inp, "bf16", dev)
    kw = dict(K=w.K, sigma=w.sigma, gamma=gamma, seed=9, antithetic=True, seq_len=w.seq_len)
    bare = dust.dust_estimate(Xd, Wd, td, **kw)["G_W"].clone()
    full = dust.dust_estimate(Xd, Wd, td, want_loss=True, want_rho=True, want_reward=True,
                              want_g=True, **kw)
    torch.cuda.synchronize(dev)
    assert torch.equal(bare, full["G_W"])


def test_runs_on_the_callers_stream(dev):
    import torch
    import token_activation_perturbation_amd as dust
    w = synth.WORKLOADS["bf16_layer"]
    inp = synth.make_inputs(w, T=512)
    Xd, Wd, td = to_dev(inp, "bf16", dev)
    kw = dict(K=w.K, sigma=w.sigma, gamma=0.3, seed=2, antithetic=True, seq_len=w.seq_len)
    ref = dust.dust_estimate(Xd, Wd, td, **kw)["G_W"]
    torch.cuda.synchronize(dev)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        out = dust.dust_estimate(Xd, Wd, td, **kw)["G_W"]
    side.synchronize()
    assert torch.equal(ref, out)


def test_misaligned_inputs_take_the_guarded_loads(dev, oracle_mod, threads):
    """X and W as views starting one element into their storage: no 16-byte
    alignment, so the GEMMs fall back to element-wise loads."""
    import torch
    import token_activation_perturbation_amd as dust
    T, d_in, d_out = 96, 64, 48
    inp = synth.random_inputs(T, d_in, d_out, "bf16", seed=5)
    kw = dict(K=8, sigma=1e-2, gamma=0.0, seed=4, antithetic=False, seq_len=32)

    def shifted(a):
        flat = torch.zeros(a.size + 1, dtype=torch.bfloat16, device=dev)
        flat[1:] = torch.from_numpy(a.ravel()).to(dev).to(torch.bfloat16)
        return flat[1:].view(a.shape)

    Xd, Wd = shifted(inp["X"]), shifted(inp["W"])
    td = torch.from_numpy(inp["target"]).to(dev).to(torch.bfloat16)
    assert Xd.data_ptr() % 16 != 0
    out = dust.dust_estimate(Xd, Wd, td, **kw)
    torch.cuda.synchronize(dev)
    ref = oracle_mod.estimate(inp["X"], inp["W"], inp["target"], threads=threads, **kw)
    assert rel(out["G_W"].cpu().numpy().astype(np.float64), ref["G"]) <= TOL["bf16"]


def test_misaligned_target_takes_the_guarded_epilogue(dev, oracle_mod, threads):
    """X and W aligned (the direct-to-LDS base GEMM runs) but target a view
    starting one element into its storage: the epilogue must fall back from
    its 16-byte target loads to element-wise ones."""
    import torch
    import token_activation_perturbation_amd as dust
    T, d_in, d_out = 128, 64, 64
    inp = synth.random_inputs(T, d_in, d_out, "bf16", seed=6)
    kw = dict(K=8, sigma=1e-2, gamma=0.0, seed=5, antithetic=True, seq_len=64)
    Xd, Wd = (torch.from_numpy(inp[k]).to(dev).to(torch.bfloat16).contiguous() for k in ("X", "W"))
    flat = torch.zeros(inp["target"].size + 1, dtype=torch.bfloat16, device=dev)
    flat[1:] = torch.from_numpy(inp["target"].ravel()).to(dev).to(torch.bfloat16)
    td = flat[1:].view(inp["target"].shape)
    assert td.data_ptr() % 16 != 0 and Xd.data_ptr() % 16 == 0
    out = dust.dust_estimate(Xd, Wd, td, want_loss=True, want_g=True, **kw)
    torch.cuda.synchronize(dev)
    ref = oracle_mod.estimate(inp["X"], inp["W"], inp["target"], threads=threads, **kw)
    assert rel(out["loss"].cpu().numpy().astype(np.float64), ref["loss"]) <= TOL["bf16"]
    assert rel(out["g"].cpu().numpy().astype(np.float64), ref["g"]) <= TOL["bf16"]
    assert rel(out["G_W"].cpu().numpy().astype(np.float64), ref["G"]) <= TOL["bf16"]


@pytest.mark.parametrize("gamma", [0.0, 0.5])
def test_direct_to_lds_and_register_staged_paths_agree_bitwise(dev, gamma):
    """The same aligned-size problem three ways: every operand 16-byte
    aligned (the direct-to-LDS GEMMs), X and W one element into their
    storage (the register-staged GEMMs), and target alone shifted (the
    element-wise epilogue).  The kernels share tiles, token split and
    contraction order, so every output is bitwise equal."""
    import torch
    import token_activation_perturbation_amd as dust
    T, d_in, d_out = 1000, 136, 200  # ragged 64-wide tiles, 8-element multiples
    print(f"aligned vs staged, gamma {gamma}", flush=True)
    inp = synth.random_inputs(T, d_in, d_out, "bf16", seed=8)
    kw = dict(K=8, sigma=1e-2, gamma=gamma, seed=6, antithetic=True, seq_len=250,
              want_loss=True, want_rho=True, want_reward=True, want_g=True)

    def place(a, shift):
        flat = torch.zeros(a.size + 8, dtype=torch.bfloat16, device=dev)
        flat[shift:shift + a.size] = torch.from_numpy(a.ravel()).to(dev).to(torch.bfloat16)
        return flat[shift:shift + a.size].view(a.shape)

    runs = {}
    for name, (sx, st) in {"aligned": (0, 0), "staged": (1, 0), "epilogue": (0, 1)}.items():
        Xd, Wd, td = place(inp["X"], sx), place(inp["W"], sx), place(inp["target"], st)
        assert (Xd.data_ptr() % 16 == 0) == (sx == 0) and (td.data_ptr() % 16 == 0) == (st == 0)
        out = dust.dust_estimate(Xd, Wd, td, **kw)
        torch.cuda.synchronize(dev)
        runs[name] = {k: v.cpu().numpy() for k, v in out.items()}
    for name in ("staged", "epilogue"):
        for k, v in runs["aligned"].items():
            assert np.array_equal(v, runs[name][k]), (name, k)


@pytest.mark.parametrize("gamma", [0.0, 0.5])
def test_big_tile_and_register_staged_paths_agree_bitwise(dev, gamma):
    """A shape with enough 128 x 128 tiles for both GEMMs to take their
    large-tile kernels (T 12010: a partial last row tile and a last token
    split of 746 tokens, 23 whole 32-token blocks and a 10-token tail; d_in
    1016 and d_out 1000: ragged 128-wide edge tiles and a partial last
    64-wide k-block).  There the base GEMM writes y = W x and the noise
    kernels (the single-generation kernel at gamma 0, the jitter-loss pass
    at gamma 0.5) subtract the target.  Against it: the same problem with X
    and W one element into their storage (the register-staged 64 x 64
    kernels), and with the target one element into its storage (the noise
    kernels' element-wise target loads).  Every output element is
    contracted over the same k-steps in the same order, the tokens are split
    alike and delta is the same fp32 subtraction, so every output is bitwise
    equal."""
    import torch
    import token_activation_perturbation_amd as dust
    T, d_in, d_out = 12010, 1016, 1000
    print(f"big tiles vs staged, gamma {gamma}", flush=True)
    inp = synth.random_inputs(T, d_in, d_out, "bf16", seed=12)
    kw = dict(K=4, sigma=1e-2, gamma=gamma, seed=3, antithetic=True, seq_len=1201,
              want_loss=True, want_g=True)

    def place(a, shift):
        flat = torch.zeros(a.size + 8, dtype=torch.bfloat16, device=dev)
        flat[shift:shift + a.size] = torch.from_numpy(a.ravel()).to(dev).to(torch.bfloat16)
        return flat[shift:shift + a.size].view(a.shape)

    runs = {}
    for name, (sx, st) in {"aligned": (0, 0), "staged": (1, 0), "target": (0, 1)}.items():
        Xd, Wd, td = place(inp["X"], sx), place(inp["W"], sx), place(inp["target"], st)
        out = dust.dust_estimate(Xd, Wd, td, **kw)
        torch.cuda.synchronize(dev)
        runs[name] = {k: v.cpu().numpy() for k, v in out.items()}
    for name in ("staged", "target"):
        for k, v in runs["aligned"].items():
            assert np.array_equal(v, runs[name][k]), (name, k)
    # and G_W is the outer product of the GPU's own g
    G = runs["aligned"]["g"].astype(np.float64).T @ inp["X"].astype(np.float64)
    assert rel(runs["aligned"]["G_W"].astype(np.float64), G) <= TOL["bf16"]


@pytest.fixture(scope="module")
def max_tokens_inputs():
    """The largest token count the library accepts, T = 2^24 - 1 = 4095 x 4097
    (4097 sequences of 4095 tokens), on a narrow layer so the inputs stay a
    few hundred MB."""
    T, d = (1 << 24) - 1, 8
    return synth.random_inputs(T, d, d, "bf16", seed=24), 4095


@pytest.mark.parametrize("gamma", [0.0, 0.9])
def test_maximum_token_count(dev, oracle_mod, threads, max_tokens_inputs, gamma):
    """T = 2^24 - 1 through every stage (the single-generation kernel at
    gamma = 0; the jitter-loss pass, the chunked scan over 4097 sequences and
    the reweight pass at gamma = 0.9): the oracle recomputes the first and the
    last sequence, and G_W is checked at full size against g^T X formed in
    fp64 from the GPU's own g."""
    import torch
    import token_activation_perturbation_amd as dust
    inp, seq_len = max_tokens_inputs
    T = inp["X"].shape[0]
    print(f"maximum token count T={T} gamma={gamma}", flush=True)
    Xd, Wd, td = (torch.from_numpy(inp[k]).to(dev).to(torch.bfloat16).contiguous()
                  for k in ("X", "W", "target"))
    kw = dict(K=2, sigma=1e-2, gamma=gamma, seed=77, antithetic=True, seq_len=seq_len)
    out = dust.dust_estimate(Xd, Wd, td, want_reward=True, want_g=True, **kw)
    torch.cuda.synchronize(dev)
    g = out["g"].cpu().numpy().astype(np.float64)
    reward = out["reward"].cpu().numpy().astype(np.float64)
    n_seq = T // seq_len
    for sq in (0, n_seq - 1):
        ref = oracle_mod.estimate(inp["X"], inp["W"], inp["target"], seq_range=(sq, sq + 1),
                                  threads=threads, **kw)
        sl = slice(sq * seq_len, (sq + 1) * seq_len)
        errs = stage_errors({"g": g, "reward": reward}, ref, keys=("g", "reward"), g_key="none",
                            token_slice=sl)
        report(f"  sequence {sq}:", errs)
        assert_within(errs, "bf16")
    G_ref = g.T @ inp["X"].astype(np.float64)
    e = rel(out["G_W"].cpu().numpy().astype(np.float64), G_ref)
    print(f"  G_W vs g^T X {e:.2e}", flush=True)
    assert e <= TOL["bf16"]


def test_small_workspace_is_an_error(dev):
    import torch
    import token_activation_perturbation_amd as dust
    X = torch.zeros(64, 16, dtype=torch.bfloat16, device=dev)
    W = torch.zeros(8, 16, dtype=torch.bfloat16, device=dev)
    t = torch.zeros(64, 8, dtype=torch.bfloat16, device=dev)
    ws = torch.empty(16, dtype=torch.uint8, device=dev)
    with pytest.raises(dust.DustError) as e:
        dust.dust_estimate(X, W, t, K=4, sigma=0.1, gamma=0.0, seed=0, antithetic=True,
                           seq_len=64, workspace=ws)
    assert e.value.status == 3


def test_noise_fill_rejects_bad_ranges(dev):
    import token_activation_perturbation_amd as dust
    with pytest.raises(dust.DustError):
        dust.dust_noise_fill(0, -1, 2, 0, 2, 8, device=dev)
    with pytest.raises(dust.DustError):
        dust.dust_noise_fill(0, 2**31 - 1, 2, 0, 2, 8, device=dev)
