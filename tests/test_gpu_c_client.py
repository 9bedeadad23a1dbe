"""The C ABI from a plain C program (tests/helpers/abi_client.c: no Python,
no torch, its own hipMalloc'd buffers, the default stream): G_W matches the
fp64 oracle within the bf16 tolerance and equals, bit for bit, what the
Python binding returns for the same inputs on torch's stream; the
documented error statuses come back for odd K with antithetic pairs and for
a workspace one byte short."""
import importlib.util
import os
import struct
import subprocess

import numpy as np
import pytest

from token_activation_perturbation_amd import synth

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def client_exe():
    spec = importlib.util.spec_from_file_location(
        "abi_client_build", os.path.join(HERE, "helpers", "abi_client_build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    if not os.path.exists(mod.EXE) or os.path.getmtime(mod.EXE) < os.path.getmtime(mod.SRC):
        mod.build()
    return mod.EXE


def bf16_bits(a):
    return (np.ascontiguousarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("gamma", [0.0, 0.9])
def test_c_client_matches_oracle_and_binding(oracle_mod, tmp_path, gamma):
    import torch
    import token_activation_perturbation_amd as dust
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    T, seq_len, d_in, d_out, K, sigma, seed = 300, 100, 72, 136, 8, 1e-2, 77
    print(f"C client, gamma {gamma}", flush=True)
    inp = synth.random_inputs(T, d_in, d_out, "bf16", seed=12)
    src = tmp_path / "in.bin"
    with open(src, "wb") as f:
        f.write(struct.pack("<7q2fQ", T, d_in, d_out, seq_len, dust.DUST_BF16, K, 1, sigma,
                            gamma, seed))
        for k in ("X", "W", "target"):
            f.write(bf16_bits(inp[k]).tobytes())
    dst = tmp_path / "out.bin"
    res = subprocess.run([client_exe(), str(src), str(dst)], capture_output=True, text=True,
                         timeout=120)
    print(res.stdout, res.stderr, flush=True)
    assert res.returncode == 0, res.stderr
    raw = dst.read_bytes()
    codes = struct.unpack("<3i", raw[:12])
    assert codes == (0, 1, 3)  # DUST_OK, DUST_ERR_INVALID_ARG, DUST_ERR_WORKSPACE
    G_c = np.frombuffer(raw[12:], dtype=np.float32).reshape(d_out, d_in)

    ref = oracle_mod.estimate(inp["X"], inp["W"], inp["target"], K=K, sigma=sigma, gamma=gamma,
                              seed=seed, antithetic=True, seq_len=seq_len)
    err = np.linalg.norm(G_c - ref["G"]) / np.linalg.norm(ref["G"])
    print(f"  rel err {err:.2e}", flush=True)
    assert err <= 2e-3

    dev = torch.device("cuda:0")
    X, W, tg = (torch.from_numpy(inp[k]).to(dev).to(torch.bfloat16).contiguous()
                for k in ("X", "W", "target"))
    G_py = dust.dust_estimate(X, W, tg, K=K, sigma=sigma, gamma=gamma, seed=seed,
                              antithetic=True, seq_len=seq_len)["G_W"]
    torch.cuda.synchronize(dev)
    assert np.array_equal(G_py.cpu().numpy(), G_c)
