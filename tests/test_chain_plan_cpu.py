"""Workspace sizing of the single-generation path for gamma > 0 (host only):
dust_workspace_bytes_seq adds, per group of 16 chains (antithetic pairs or
plain draws), a partial sum of R a (T x d_out fp32), and for plain draws
also a partial sum of a (T x d_out) and of rho (T), plus the per-token credit
mean (T), exactly where the path applies (gamma > 0, seq_len >= 2 dividing T,
d_out <= 1024, (T / seq_len) * chains >= 2048 with K/2 chains for pairs and
K for plain draws, and seq_len <= 8192 for plain draws) and equals
dust_workspace_bytes elsewhere."""
import pytest

import token_activation_perturbation_amd as dust

BF16 = 1


def sizes(T, d_in, d_out, seq_len, K, gamma, anti=True):
    return (dust.dust_workspace_bytes(T, d_in, d_out, K, anti, BF16),
            dust.dust_workspace_bytes_seq(T, d_in, d_out, seq_len, K, gamma, anti, BF16))


def align256(x):
    return (x + 255) & ~255


@pytest.mark.parametrize("T,d_in,d_out,seq_len,K,gamma", [
    (2048, 1024, 1024, 1024, 4096, 0.5),   # the large-population workload
    (16, 32, 64, 8, 4096, 0.5),
    (12, 24, 70, 6, 4096, 0.9),
    (16, 32, 64, 8, 4100, 0.7),            # 2050 pairs: 129 groups
    (8, 20, 1024, 2, 4096, 1.0),
])
def test_adds_the_groups_partial_g(T, d_in, d_out, seq_len, K, gamma):
    base, seq = sizes(T, d_in, d_out, seq_len, K, gamma)
    groups = -(-(K // 2) // 16)
    assert base > 0
    assert seq == align256(align256(base) + 4 * groups * T * d_out)


@pytest.mark.parametrize("T,d_in,d_out,seq_len,K,gamma", [
    (2048, 1024, 1024, 1024, 4096, 0.5),   # the large population with plain draws
    (8, 24, 300, 4, 1024, 0.6),            # 2 sequences x 1024 draws
    (16, 32, 64, 8, 1030, 0.7),            # 1030 draws: 65 groups, the last partial
])
def test_plain_draws_add_both_partials_rho_and_the_mean(T, d_in, d_out, seq_len, K, gamma):
    base, seq = sizes(T, d_in, d_out, seq_len, K, gamma, anti=False)
    groups = -(-K // 16)
    rows = 4 * groups * T * d_out
    off = align256(base)
    off = align256(off + rows)          # sum of R a
    off = align256(off + rows)          # sum of a
    off = align256(off + 4 * groups * T)  # sum of rho
    off = align256(off + 4 * T)         # the credit mean
    assert base > 0 and seq == off


@pytest.mark.parametrize("T,d_in,d_out,seq_len,K,gamma,anti", [
    (2048, 1024, 1024, 1024, 4096, 0.0, True),    # gamma = 0: the fused kernel
    (2048, 1024, 1024, 1024, 4096, 0.0, False),
    (16384, 64, 64, 16384, 4096, 0.5, False),     # plain draws: sequence past the mean scan's LDS
    (8192, 1024, 3072, 1024, 128, 0.9, False),    # the QKV workload: too wide, too few chains
    (2048, 1024, 1024, 1, 4096, 0.5, True),       # one-token sequences: no credit chain
    (16384, 512, 512, 2048, 64, 0.98, True),      # 8 x 32 chains: too few to fill the chip
    (16, 32, 1028, 8, 4096, 0.5, True),           # d_out past the LDS budget
    (8192, 1024, 3072, 1024, 128, 0.9, True),     # the QKV layer's width
])
def test_equals_two_pass_size_elsewhere(T, d_in, d_out, seq_len, K, gamma, anti):
    base, seq = sizes(T, d_in, d_out, seq_len, K, gamma, anti)
    assert base > 0 and seq == base


def test_invalid_sizes_give_zero():
    assert dust.dust_workspace_bytes_seq(0, 8, 8, 1, 4, 0.5, True, BF16) == 0
    assert dust.dust_workspace_bytes_seq(8, 8, 8, 4, 3, 0.5, True, BF16) == 0  # odd K, pairs
    assert dust.dust_workspace_bytes_seq(8, 8, 8, 4, 4, 0.5, True, 7) == 0     # unknown dtype
