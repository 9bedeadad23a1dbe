"""The estimator's workspace layout (host only): delta and g (T x d_out
fp32), P, Q and the weights (T x K_n), rho, the local credit (T x K), the
per-token mean (T), the chunk carries (ceil(T / 2) x K) and the outer
product's split partials (splits x d_out x d_in fp32), each 256-byte
aligned.  The split count follows the tile the outer product takes: on
128 x 256 tiles where the 128 x 128 kernel would run and d_in >= 512 (512
workgroups), on 128 x 128 tiles otherwise when there are at least 768 of
them with >= 1024 tokens per split, else 64 x 64 tiles (about 2048
workgroups, >= 512 tokens per split)."""
import pytest

import token_activation_perturbation_amd as dust

BF16 = 1


def a256(x):
    return (x + 255) & ~255


def cdiv(a, b):
    return -(-a // b)


def expected_splits(T, d_in, d_out):
    aligned8 = d_in % 8 == 0 and d_out % 8 == 0
    tiles128 = cdiv(d_out, 128) * cdiv(d_in, 128)
    big = aligned8 and tiles128 * cdiv(T, 1024) >= 768
    wide = big and d_in >= 512
    if wide:
        tiles = cdiv(d_out, 128) * cdiv(d_in, 256)
        split = 512 // tiles
    elif big:
        tiles = tiles128
        split = 768 // tiles
    else:
        tiles = cdiv(d_out, 64) * cdiv(d_in, 64)
        split = cdiv(2048, tiles)
    split = min(split, cdiv(T, 1024 if big else 512), 64)
    split = max(split, 1)
    tokens = cdiv(cdiv(T, split), 64) * 64
    return cdiv(T, tokens)


def expected_bytes(T, d_in, d_out, K, anti):
    K_n = K // 2 if anti else K
    splits = expected_splits(T, d_in, d_out)
    parts = [4 * T * d_out, 4 * T * K_n, 4 * T * K_n, 4 * T * K, 4 * T, 4 * T * K_n,
             4 * T * d_out, 4 * splits * d_out * d_in if splits > 1 else 0, 4 * T * K,
             4 * cdiv(T, 2) * K]
    off = 0
    for p in parts:
        off = a256(off + p)
    return off


@pytest.mark.parametrize("T,d_in,d_out,K,anti,splits", [
    (16384, 768, 3072, 256, True, 7),    # the MLP up-projection: 128 x 256 tiles
    (8192, 1024, 3072, 128, False, 5),   # the QKV projection: 128 x 256 tiles
    (16384, 512, 4096, 64, True, 8),     # the head's logits: 128 x 256 tiles
    (12010, 1016, 1000, 4, True, 12),    # ragged 128 x 256 tiles
    (8192, 256, 8192, 16, True, 6),      # d_in < 512: 128 x 128 tiles
    (4096, 512, 512, 64, True, 8),       # the 512-wide layer: 64 x 64 tiles
    (64, 64, 64, 16, False, 1),          # one split, no partials
])
def test_workspace_holds_the_outer_products_split_partials(T, d_in, d_out, K, anti, splits):
    assert expected_splits(T, d_in, d_out) == splits
    assert dust.dust_workspace_bytes(T, d_in, d_out, K, anti, BF16) == \
        expected_bytes(T, d_in, d_out, K, anti)
