"""The C-ABI library on a machine without a GPU: it loads, exports every
entry point include/dust.h declares, and its host-side validation and
workspace sizing behave as documented.  No compute call is made here."""
import ctypes
import math
import os
import re

import pytest

import token_activation_perturbation_amd as dust

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    path = dust.library_path()
    if not os.path.exists(path):
        from token_activation_perturbation_amd.build import build_library
        build_library()
    return ctypes.CDLL(path)


def declared_entry_points():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(dust_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported(lib):
    names = declared_entry_points()
    assert {"dust_estimate", "dust_validate", "dust_workspace_bytes", "dust_noise_fill",
            "dust_last_error", "dust_estimate_local", "dust_validate_local",
            "dust_estimate_head", "dust_validate_head", "dust_estimate_embedding",
            "dust_validate_embedding", "dust_reassemble_embedding", "dust_validate_reassemble",
            "dust_embedding_workspace_bytes", "dust_reassemble_workspace_bytes"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_library_is_built_for_gfx950():
    data = open(dust.library_path(), "rb").read()
    assert b"gfx950" in data


def _validate(**over):
    args = dict(X=1, W=2, target=3, T=64, d_in=16, d_out=8, seq_len=16, dtype=dust.DUST_BF16,
                K=4, sigma=0.01, gamma=0.5, antithetic=1, G=4, ws=5, ws_bytes=None)
    args.update(over)
    if args["ws_bytes"] is None:
        args["ws_bytes"] = dust.dust_workspace_bytes(args["T"], args["d_in"], args["d_out"],
                                                     args["K"], args["antithetic"],
                                                     dust.DUST_BF16) or 1
    return dust.dust_validate(args["X"], args["W"], args["target"], args["T"], args["d_in"],
                              args["d_out"], args["seq_len"], args["dtype"], args["K"],
                              args["sigma"], args["gamma"], args["antithetic"], args["G"],
                              args["ws"], args["ws_bytes"])


def test_valid_arguments_pass(lib):
    assert _validate() == 0
    assert dust.dust_last_error() == ""


@pytest.mark.parametrize("over,status", [
    (dict(X=None), 1), (dict(W=None), 1), (dict(target=None), 1), (dict(G=None), 1),
    (dict(T=0), 1), (dict(d_in=-1), 1), (dict(d_out=0), 1),
    (dict(seq_len=0), 1), (dict(seq_len=10), 1),
    (dict(K=1, antithetic=0), 1), (dict(K=3, antithetic=1), 1),
    (dict(sigma=0.0), 1), (dict(sigma=-1.0), 1), (dict(sigma=math.inf), 1),
    (dict(sigma=math.nan), 1), (dict(gamma=-0.1), 1), (dict(gamma=1.5), 1),
    (dict(gamma=math.nan), 1), (dict(T=2**31, seq_len=2**31), 1),
    (dict(dtype=7), 2), (dict(ws=None), 3), (dict(ws_bytes=16), 3),
])
def test_invalid_arguments_are_rejected(lib, over, status):
    assert _validate(**over) == status
    assert dust.dust_last_error() != ""


def test_edge_values_accepted(lib):
    assert _validate(gamma=0.0) == 0
    assert _validate(gamma=1.0) == 0
    assert _validate(K=2, antithetic=1) == 0
    assert _validate(K=3, antithetic=0) == 0
    assert _validate(seq_len=1) == 0
    assert _validate(T=64, seq_len=64) == 0


def test_workspace_bytes(lib):
    a = dust.dust_workspace_bytes(4096, 512, 512, 64, True, dust.DUST_BF16)
    b = dust.dust_workspace_bytes(4096, 512, 512, 64, False, dust.DUST_BF16)
    assert a > 0 and b > a  # plain draws need twice the per-noise buffers
    # at least delta and g (T x d_out fp32 each)
    assert a >= 2 * 4096 * 512 * 4
    assert dust.dust_workspace_bytes(0, 512, 512, 64, True, 1) == 0
    assert dust.dust_workspace_bytes(64, 8, 8, 3, True, 1) == 0
    assert dust.dust_workspace_bytes(64, 8, 8, 4, True, 9) == 0


def test_python_binding_rejects_bad_tensors():
    import torch
    X = torch.zeros(4, 4)
    with pytest.raises(ValueError):
        dust.dust_estimate(X, X, X, K=4, sigma=0.1, gamma=0.0, seed=0, antithetic=True,
                           seq_len=4)


def test_python_local_binding_rejects_bad_tensors():
    import torch
    E = torch.zeros(4, 4)
    with pytest.raises(ValueError):  # a host tensor, with or without X
        dust.dust_estimate_local(None, E, K=4, sigma=0.1, gamma=0.0, seed=0, antithetic=True,
                                 seq_len=4)


def test_python_binding_checks_devices_and_workspace():
    """Operands on different devices, or a workspace that is not a device
    tensor, are rejected before the library is called."""
    import torch
    X = torch.zeros(4, 4)
    with pytest.raises(ValueError):
        dust._check_tensors(None, X=X)
    with pytest.raises(ValueError):
        dust._workspace(torch.zeros(16, dtype=torch.uint8), 16, torch.device("cuda:0"))


def _validate_local(**over):
    args = dict(X=16, E=32, T=64, d_in=16, d_out=8, seq_len=16, dtype=dust.DUST_BF16,
                K=4, sigma=0.2, gamma=0.98, antithetic=1, G=48, ws=64, ws_bytes=None)
    args.update(over)
    if args["ws_bytes"] is None:
        args["ws_bytes"] = dust.dust_workspace_bytes(args["T"], args["d_in"], args["d_out"],
                                                     args["K"], args["antithetic"],
                                                     dust.DUST_BF16) or 1
    return dust.dust_validate_local(args["X"], args["E"], args["T"], args["d_in"],
                                    args["d_out"], args["seq_len"], args["dtype"], args["K"],
                                    args["sigma"], args["gamma"], args["antithetic"],
                                    args["G"], args["ws"], args["ws_bytes"])


def test_validate_local_accepts_good_arguments(lib):
    assert _validate_local() == 0
    # no input matrix (a value embedding): X and G_W omitted together
    assert _validate_local(X=None, G=None, d_in=1) == 0


@pytest.mark.parametrize("over,status", [
    (dict(X=None), 1), (dict(E=None), 1), (dict(G=None), 1), (dict(E=34), 1),
    (dict(T=0), 1), (dict(seq_len=5), 1), (dict(K=1), 1), (dict(K=5), 1),
    (dict(sigma=0.0), 1), (dict(gamma=1.5), 1), (dict(dtype=7), 2),
    (dict(T=1 << 24, seq_len=1), 2), (dict(ws=None), 3), (dict(ws_bytes=16), 3)])
def test_validate_local_rejects(lib, over, status):
    assert _validate_local(**over) == status
    assert dust.dust_last_error() != ""


def _validate_head(**over):
    args = dict(X=16, W=32, labels=48, T=64, d_in=16, V=512, dtype=dust.DUST_BF16,
                K=4, sigma=0.05, antithetic=1, G=64, ws=80, ws_bytes=None)
    args.update(over)
    if args["ws_bytes"] is None:
        args["ws_bytes"] = dust.dust_workspace_bytes(args["T"], args["d_in"], args["V"],
                                                     args["K"], args["antithetic"],
                                                     dust.DUST_BF16) or 1
    return dust.dust_validate_head(args["X"], args["W"], args["labels"], args["T"],
                                   args["d_in"], args["V"], args["dtype"], args["K"],
                                   args["sigma"], args["antithetic"], args["G"], args["ws"],
                                   args["ws_bytes"])


def test_validate_head_accepts_good_arguments(lib):
    assert _validate_head() == 0
    assert _validate_head(V=256, K=3, antithetic=0) == 0
    assert _validate_head(T=1, K=2) == 0


@pytest.mark.parametrize("over,status", [
    (dict(X=None), 1), (dict(W=None), 1), (dict(labels=None), 1), (dict(G=None), 1),
    (dict(labels=50), 1), (dict(V=0), 1), (dict(V=300), 1), (dict(V=128), 1),
    (dict(T=0), 1), (dict(K=1), 1), (dict(K=5), 1), (dict(sigma=0.0), 1),
    (dict(sigma=math.nan), 1), (dict(dtype=7), 2), (dict(T=1 << 24), 2), (dict(ws=None), 3),
    (dict(ws_bytes=16), 3)])
def test_validate_head_rejects(lib, over, status):
    assert _validate_head(**over) == status
    assert dust.dust_last_error() != ""


def test_head_binding_rejects_bad_tensors():
    import torch
    X = torch.zeros(4, 4)
    with pytest.raises(ValueError):
        dust.dust_estimate_head(X, X, torch.zeros(4, dtype=torch.int32), K=4, sigma=0.1, seed=0,
                                antithetic=True)


def _validate_embedding(**over):
    args = dict(table=16, ids=32, target=48, T=64, V=100, d=24, seq_len=16,
                dtype=dust.DUST_BF16, K=4, sigma=0.4, gamma=0.0, antithetic=1, scale=1 / 64,
                G=64, ws=80, ws_bytes=None)
    args.update(over)
    if args["ws_bytes"] is None:
        args["ws_bytes"] = dust.dust_embedding_workspace_bytes(
            args["T"], args["V"], args["d"], args["K"], args["antithetic"], dust.DUST_BF16) or 1
    return dust.dust_validate_embedding(args["table"], args["ids"], args["target"], args["T"],
                                        args["V"], args["d"], args["seq_len"], args["dtype"],
                                        args["K"], args["sigma"], args["gamma"],
                                        args["antithetic"], args["scale"], args["G"],
                                        args["ws"], args["ws_bytes"])


def test_validate_embedding_accepts_good_arguments(lib):
    assert _validate_embedding() == 0
    assert _validate_embedding(V=1, T=1, seq_len=1, K=2) == 0
    assert _validate_embedding(gamma=0.98, antithetic=0, K=3) == 0


@pytest.mark.parametrize("over,status", [
    (dict(table=None), 1), (dict(ids=None), 1), (dict(target=None), 1), (dict(G=None), 1),
    (dict(ids=34), 1), (dict(V=0), 1), (dict(V=2**31), 1), (dict(scale=math.inf), 1),
    (dict(scale=math.nan), 1), (dict(T=0), 1), (dict(seq_len=5), 1), (dict(K=1), 1),
    (dict(K=5), 1), (dict(sigma=0.0), 1), (dict(gamma=2.0), 1), (dict(d=0), 1),
    (dict(dtype=7), 2), (dict(T=1 << 24, seq_len=1), 2), (dict(ws=None), 3),
    (dict(ws_bytes=16), 3)])
def test_validate_embedding_rejects(lib, over, status):
    assert _validate_embedding(**over) == status
    assert dust.dust_last_error() != ""


def test_embedding_workspace_covers_the_estimator_and_the_reassembly(lib):
    T, V, d, K = 4096, 1000, 64, 16
    e = dust.dust_embedding_workspace_bytes(T, V, d, K, True, dust.DUST_BF16)
    r = dust.dust_reassemble_workspace_bytes(T, V, d)
    w = dust.dust_workspace_bytes(T, 1, d, K, True, dust.DUST_BF16)
    assert r > 0 and w > 0 and e >= w + r
    # histograms, run starts, the sorted order and two partial rows per tile
    assert r >= 4 * (V + 1) + 8 * T + 2 * 4 * d * (T // 32)
    assert dust.dust_reassemble_workspace_bytes(0, V, d) == 0
    assert dust.dust_reassemble_workspace_bytes(T, 0, d) == 0
    assert dust.dust_reassemble_workspace_bytes(1 << 24, V, d) == 0
    assert dust.dust_embedding_workspace_bytes(T, V, d, K, True, 9) == 0


def _validate_reassemble(**over):
    args = dict(ids=16, g=32, T=64, V=100, d=24, scale=1.0, G=48, ws=64, ws_bytes=None)
    args.update(over)
    if args["ws_bytes"] is None:
        args["ws_bytes"] = dust.dust_reassemble_workspace_bytes(args["T"], args["V"],
                                                                args["d"]) or 1
    return dust.dust_validate_reassemble(args["ids"], args["g"], args["T"], args["V"],
                                         args["d"], args["scale"], args["G"], args["ws"],
                                         args["ws_bytes"])


def test_validate_reassemble(lib):
    assert _validate_reassemble() == 0
    for over, status in [(dict(ids=None), 1), (dict(g=None), 1), (dict(G=None), 1),
                         (dict(g=34), 1), (dict(T=0), 1), (dict(V=-1), 1), (dict(d=0), 1),
                         (dict(scale=math.nan), 1), (dict(T=1 << 24), 2), (dict(ws=None), 3),
                         (dict(ws_bytes=8), 3)]:
        assert _validate_reassemble(**over) == status, over
        assert dust.dust_last_error() != ""


def test_embedding_binding_rejects_bad_tensors():
    import torch
    t = torch.zeros(4, 4)
    ids = torch.zeros(4, dtype=torch.int32)
    with pytest.raises(ValueError):
        dust.dust_estimate_embedding(t, ids, t, K=4, sigma=0.1, gamma=0.0, seed=0,
                                     antithetic=True, seq_len=4)
    with pytest.raises(ValueError):
        dust.dust_reassemble_embedding(ids, t, 4)


def test_header_is_plain_c_and_links(tmp_path):
    """include/dust.h compiles as C99 with every warning on, and a C program
    built against it links libdust.so and gets the same sizing and
    validation answers as the Python binding (no compute call)."""
    import shutil
    import subprocess
    if shutil.which("gcc") is None:
        pytest.skip("no gcc")
    src = tmp_path / "abi.c"
    src.write_text(r'''
#include <stdio.h>
#include "dust.h"
int main(void) {
  char a, b, c, ws; float G;
  size_t need = dust_workspace_bytes(4096, 512, 512, 64, 1, DUST_BF16);
  dust_status_t ok = dust_validate(&a, &b, &c, 4096, 512, 512, 512, DUST_BF16, 64, 0.01f,
                                   0.0f, 1, &G, &ws, need);
  dust_status_t bad = dust_validate(&a, &b, &c, 4096, 512, 512, 512, DUST_BF16, 63, 0.01f,
                                    0.0f, 1, &G, &ws, need);
  printf("%zu %d %d %d\n", need, (int)ok, (int)bad, dust_last_error()[0] != 0);
  return 0;
}
''')
    lib_dir = os.path.dirname(dust.library_path())
    exe = tmp_path / "abi"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                    "-L", lib_dir, "-ldust", f"-Wl,-rpath,{lib_dir}"], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    need = dust.dust_workspace_bytes(4096, 512, 512, 64, True, dust.DUST_BF16)
    assert out == [str(need), "0", "1", "1"]  # DUST_OK, DUST_ERR_INVALID_ARG, a message
