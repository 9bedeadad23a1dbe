"""The ALU cost model the bench line's roofline fraction uses, against the
counts it states: Philox4x32-10 is 10 rounds of 2 quarter-rate 32x32->64
multiplies and 4 xors per quad, of which the first round's draw-independent
half (the quad index's product and the xor with the zero word and the key)
is shared by all draws (113 slots per quad); Box-Muller 8 quarter-rate
transcendentals and 18 simple ops per quad (50 slots); the consumers one
slot each."""
import pytest

from token_activation_perturbation_amd import roofline


def test_peak_is_the_fp32_vector_rate():
    # 157.3 TFLOP/s = 2 flops x 128 lanes x 256 CUs x 2.4 GHz
    assert roofline.PEAK_SLOTS_PER_S == pytest.approx(157.3e12 / 2, rel=1e-3)


def test_generation_slots_per_value():
    assert roofline.PHILOX_SLOTS_PER_QUAD == 9 * 12 + 5
    assert roofline.BOX_MULLER_SLOTS_PER_QUAD == 50
    assert roofline.GEN_SLOTS_PER_VALUE == 40.75


@pytest.mark.parametrize("anti,outputs,per_value", [
    (True, False, 42.75),   # P and g; the pair cancels the curvature: no Q
    (True, True, 43.75),    # rho or the credit asked for: Q too
    (False, False, 44.75),  # plain draws: Q in the weight, the noise sum for centring
    (False, True, 44.75),
])
def test_fused_kernel_slots(anti, outputs, per_value):
    T, d_out, K = 8, 12, 6
    K_n = K // 2 if anti else K
    got = roofline.fused_kernel_slots(T, d_out, K, anti, per_draw_outputs=outputs)
    assert got == pytest.approx(K_n * T * d_out * per_value)


def test_local_scoring_has_no_curvature_term():
    # P and g (antithetic) or P, g and the noise sum (plain): never Q
    assert roofline.fused_kernel_slots(2, 4, 4, True, per_draw_outputs=True, local=True) == \
        pytest.approx(2 * 2 * 4 * 42.75)
    assert roofline.fused_kernel_slots(2, 4, 4, False, local=True) == \
        pytest.approx(4 * 2 * 4 * 43.75)
    assert roofline.jitter_kernel_slots(2, 4, 4, True, local=True) == \
        pytest.approx(2 * 2 * 4 * 41.75)


def test_two_pass_and_head_slots():
    assert roofline.jitter_kernel_slots(2, 4, 4, True) == pytest.approx(2 * 2 * 4 * 42.75)
    assert roofline.head_slots_per_value(True) == 55.75
    assert roofline.head_slots_per_value(False) == 52.75
    assert roofline.head_kernel_slots(1, 256, 4, True) == pytest.approx(2 * 256 * 55.75)
