"""The ALU cost model the bench line's roofline fraction uses, against the
counts it states.  Issue classes (measured rate classes on gfx950):
single-pass 1 slot, integer products and integer-to-float conversion 2,
transcendentals 4.  Philox4x32-10 per quad and draw: the second round's two
xors, the third round's two products, three-input xor and xor, then seven
rounds of two products and two three-input xors (50 slots); Box-Muller per
pair 2 funnel shifts (the uniforms built in a float's bit fields), the
subtraction that forms u, 4 transcendentals and two multiplies by the
radius (21 slots, 42 per quad: the values come in units of sqrt(2 ln 2),
which the consumers apply per total, not per value); the consumers one
slot each."""
import pytest

from token_activation_perturbation_amd import roofline


def test_peak_is_the_fp32_vector_rate():
    # 157.3 TFLOP/s = 2 flops x 128 lanes x 256 CUs x 2.4 GHz
    assert roofline.PEAK_SLOTS_PER_S == pytest.approx(157.3e12 / 2, rel=1e-3)


def test_generation_slots_per_value():
    assert roofline.PHILOX_SLOTS_PER_QUAD == 2 + (4 + 2) + 7 * (4 + 2)
    assert roofline.BOX_MULLER_SLOTS_PER_QUAD == 2 * (2 + 1 + 16 + 2)
    assert roofline.GEN_SLOTS_PER_VALUE == 23.0


@pytest.mark.parametrize("anti,outputs,per_value", [
    (True, False, 25.0),   # P and g; the pair cancels the curvature: no Q
    (True, True, 26.0),    # rho or the credit asked for: Q too
    (False, False, 27.0),  # plain draws: Q in the weight, the noise sum for centring
    (False, True, 27.0),
])
def test_fused_kernel_slots(anti, outputs, per_value):
    T, d_out, K = 8, 12, 6
    K_n = K // 2 if anti else K
    got = roofline.fused_kernel_slots(T, d_out, K, anti, per_draw_outputs=outputs)
    assert got == pytest.approx(K_n * T * d_out * per_value)


def test_local_scoring_has_no_curvature_term():
    # P and g (antithetic) or P, g and the noise sum (plain): never Q
    assert roofline.fused_kernel_slots(2, 4, 4, True, per_draw_outputs=True, local=True) == \
        pytest.approx(2 * 2 * 4 * 25.0)
    assert roofline.fused_kernel_slots(2, 4, 4, False, local=True) == \
        pytest.approx(4 * 2 * 4 * 26.0)
    assert roofline.jitter_kernel_slots(2, 4, 4, True, local=True) == \
        pytest.approx(2 * 2 * 4 * 24.0)


def test_two_pass_and_head_slots():
    assert roofline.jitter_kernel_slots(2, 4, 4, True) == pytest.approx(2 * 2 * 4 * 25.0)
    assert roofline.head_slots_per_value(True) == 38.0
    assert roofline.head_slots_per_value(False) == 35.0
    assert roofline.head_kernel_slots(1, 256, 4, True) == pytest.approx(2 * 256 * 38.0)


def test_minimum_time_is_one_generation_at_peak():
    T, d_out, K = 4096, 512, 64
    assert roofline.estimate_min_seconds(T, d_out, K, True) == pytest.approx(
        32 * T * d_out * 25.0 / roofline.PEAK_SLOTS_PER_S)


def test_stage_roofline_picks_the_bound_of_each_kind():
    # a contraction: MFMA flops against the operand type's peak
    s = roofline.stage_roofline("base_gemm", 1.0, 2.5e12, 8.0e9, "bf16")
    assert s["bound"] == "mfma" and s["frac"] == pytest.approx(1.0)
    assert s["hbm_frac"] == pytest.approx(1.0)
    assert s["bound_ms"] == pytest.approx(1.0)
    s = roofline.stage_roofline("outer_gemm", 2.0, 157.3e9, 0.0, "f32")
    assert s["bound"] == "mfma" and s["frac"] == pytest.approx(0.5)
    # a noise stage: the slot model
    s = roofline.stage_roofline("fused_g0_kernel", 1.0, 0.0, 1e6, "bf16",
                                slots=roofline.PEAK_SLOTS_PER_S * 0.5e-3)
    assert s["bound"] == "alu" and s["frac"] == pytest.approx(0.5)
    assert s["bound_ms"] == pytest.approx(0.5)
    # anything else: HBM bytes against 8 TB/s
    s = roofline.stage_roofline("split_sum_kernel", 1.0, 0.0, 4.0e9, "bf16")
    assert s["bound"] == "hbm" and s["frac"] == pytest.approx(0.5)


@pytest.mark.parametrize("kernel,per_value", [
    ("fused_g0_kernel", 25.0), ("chain_g_kernel", 25.0), ("jitter_loss_kernel", 25.0),
    ("reweight_kernel", 24.0)])
def test_noise_stage_slots(kernel, per_value):
    T, d_out, K = 4, 8, 6
    assert roofline.noise_stage_slots(kernel, T, d_out, K, True) == \
        pytest.approx(K // 2 * T * d_out * per_value)


def test_attention_score_bound():
    from token_activation_perturbation_amd import roofline as r
    T, L, H, d, K = 16384, 2048, 4, 128, 64
    pairs = (T // L) * H * L * (L + 1) / 2
    assert r.attention_pairs(T, L, H) == pairs
    assert r.attention_score_flops(T, L, H, d, K, True) == 2 * pairs * d * (K // 2)
    gen = (K // 2) * T * H * d * (r.GEN_SLOTS_PER_VALUE + 1)
    assert r.attention_score_slots("key", T, L, H, d, K, True) == (K // 2) * pairs * 11 + gen
    assert r.attention_score_slots("query", T, L, H, d, K, False) == K * pairs * 9 + \
        K * T * H * d * (r.GEN_SLOTS_PER_VALUE + 1)
    assert r.attention_score_slots("value", T, L, H, d, K, True) == (K // 2) * pairs + gen
    # keys and queries spend more time on the ALU than on the MFMA contraction,
    # values the other way round
    for site, bound in (("key", "alu"), ("query", "alu"), ("value", "mfma")):
        b, work, peak, unit = r.attention_score_bound(site, T, L, H, d, K, True)
        assert b == bound
        assert unit == ("T lane-slot/s" if bound == "alu" else "TFLOP/s")
