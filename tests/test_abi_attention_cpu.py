"""dust_estimate_attention's host side without a GPU: argument validation
(dust_validate_attention, the check the estimate runs first), workspace
sizing and the Python binding's tensor checks.  No compute call is made."""
import math

import pytest

import token_activation_perturbation_amd as dust

SITE = dust.ATTENTION_SITES


def _validate(**over):
    a = dict(X=16, Q=32, Kc=48, V=64, E=80, T=256, d_in=32, heads=2, d_head=64, seq_len=128,
             site=SITE["key"], dtype=dust.DUST_BF16, K=8, sigma=0.05, gamma=0.98, anti=1,
             G=96, ws=112, ws_bytes=None)
    a.update(over)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = dust.dust_attention_workspace_bytes(
            a["T"], a["d_in"], a["heads"], a["d_head"], a["seq_len"],
            {v: k for k, v in SITE.items()}.get(a["site"], "key"), a["K"], a["anti"]) or 1
    return dust.dust_validate_attention(a["X"], a["Q"], a["Kc"], a["V"], a["E"], a["T"],
                                        a["d_in"], a["heads"], a["d_head"], a["seq_len"],
                                        a["site"], a["dtype"], a["K"], a["sigma"], a["gamma"],
                                        a["anti"], a["G"], a["ws"], a["ws_bytes"])


@pytest.mark.parametrize("site", ["query", "key", "value"])
@pytest.mark.parametrize("d_head", [64, 128])
def test_valid_arguments_pass(site, d_head):
    assert _validate(site=SITE[site], d_head=d_head) == 0
    assert dust.dust_last_error() == ""
    # without the block's input: X and G_W both omitted
    assert _validate(site=SITE[site], d_head=d_head, X=None, G=None, d_in=1) == 0


@pytest.mark.parametrize("over,status", [
    (dict(Q=None), 1), (dict(Kc=None), 1), (dict(V=None), 1), (dict(E=None), 1),
    (dict(X=None), 1), (dict(G=None), 1),
    (dict(Q=40), 1), (dict(E=84), 1),                      # not 16-byte aligned
    (dict(site=3), 1), (dict(site=-1), 1),
    (dict(heads=0), 1), (dict(d_head=0), 1),
    (dict(T=0), 1), (dict(seq_len=100), 1), (dict(K=1, anti=0), 1), (dict(K=7), 1),
    (dict(sigma=0.0), 1), (dict(sigma=math.nan), 1), (dict(gamma=1.5), 1),
    (dict(dtype=dust.DUST_F32), 2), (dict(dtype=9), 2),
    (dict(d_head=96, ws_bytes=1 << 40), 2), (dict(d_head=32, ws_bytes=1 << 40), 2),
    (dict(seq_len=8192, T=8192, ws_bytes=1 << 40), 2),
    (dict(ws=None), 3), (dict(ws_bytes=4096), 3),
])
def test_invalid_arguments_are_rejected(over, status):
    assert _validate(**over) == status
    assert dust.dust_last_error() != ""


def test_workspace_bytes_cover_the_estimator_and_the_attention_buffers():
    T, d_in, H, dh, L, K = 4096, 256, 4, 128, 1024, 16
    D = H * dh
    base = dust.dust_workspace_bytes(T, d_in, D, K, True, dust.DUST_BF16)
    n_seq, Lp, nb = T // L, L, L // 64
    mat = 4 * n_seq * H * Lp * Lp
    part = lambda slots, sums: 4 * n_seq * H * slots * sums * K * Lp  # noqa: E731
    key = dust.dust_attention_workspace_bytes(T, d_in, H, dh, L, "key", K, True)
    value = dust.dust_attention_workspace_bytes(T, d_in, H, dh, L, "value", K, True)
    query = dust.dust_attention_workspace_bytes(T, d_in, H, dh, L, "query", K, True)
    # P and B and the partial sums, each region 256-byte aligned
    assert key >= base + 2 * mat + part(nb, 2)
    assert key - (base + 2 * mat + part(nb, 2)) < 4 * 256
    assert value >= base + mat + part(nb, 1)
    assert query >= base + 2 * mat + part(1, 2)
    assert value < key and query < key
    # a ragged sequence rounds up to whole 64-token blocks
    r = dust.dust_attention_workspace_bytes(3 * 100, d_in, H, dh, 100, "key", K, True)
    assert r >= 4 * 3 * H * 128 * 128 * 2
    # invalid sizes give 0
    assert dust.dust_attention_workspace_bytes(T, d_in, H, 96, L, "key", K, True) == 0
    assert dust.dust_attention_workspace_bytes(T, d_in, H, dh, 100, "key", K, True) == 0


def test_binding_rejects_bad_tensors():
    import torch
    x = torch.zeros(8, 4, dtype=torch.bfloat16)
    q = torch.zeros(8, 128, dtype=torch.bfloat16)
    e = torch.zeros(8, 128, dtype=torch.float32)
    with pytest.raises(ValueError, match="device"):
        dust.dust_estimate_attention(x, q, q, q, e, heads=2, site="key", K=4, sigma=0.1,
                                     gamma=0.0, seed=1, antithetic=True, seq_len=8)
