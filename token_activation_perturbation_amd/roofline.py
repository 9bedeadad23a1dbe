"""The ALU roofline of the estimator's noise kernels on MI355X (gfx950).

The noise kernels move almost no memory: each noise value is a pure function
of (seed, noise index, token, channel), generated in registers and consumed
at once.  Their bound is the vector ALU issue rate, counted in lane-slots:

* Peak.  MI355X: 256 compute units at 2.4 GHz; its fp32 vector peak of
  157.3 TFLOP/s is 2 flops x 128 lanes per clock per CU, so a full-rate
  32-bit VALU operation occupies one of 256 x 128 x 2.4e9 = 7.864e13
  lane-slots per second.  Quarter-rate operations (32x32->64 integer
  multiply, and the transcendentals log2, sqrt, sin, cos) occupy 4 slots.

* Work per distinct noise value (the minimum the method needs: each of the
  K_n * T * d_out values generated once, where K_n = K/2 with antithetic
  pairs, else K).  Per quad of four values:
    Philox4x32-10   9 rounds x (2 multiplies x 4 + 4 xor)
                    + first round 1 multiply x 4 + 1 xor         = 113 slots
    Box-Muller      8 transcendentals x 4 + 18 simple ops        =  50 slots
  The counter is (quad, token, noise index, 0), so the first round's product
  of the quad index and its xor with the zero word and the key are the same
  for every noise index of a (token, quad): only the product of the noise
  index and one xor depend on the draw.  That gives 40.75 slots per value,
  plus the consumers: 1 FMA for P = <delta, a>,
  1 FMA for Q = ||a||^2 (the quadratic loss's curvature term: needed by
  plain draws and by the per-draw outputs; with antithetic pairs it cancels
  inside each pair, so a call that asks only for g and G_W does without it,
  and local scoring, linear in the jitter, never needs it), 1 FMA for the
  reweighted sum g, and 1 add for the plain-draw noise sum used by the
  centring.

The cross-entropy head's slab kernel consumes each value as: 1 multiply
(sigma a), the jitter's expm1 (antithetic: both signs from the even and odd
Taylor parts, 9 + 2 slots; plain draws: 8 slots of Horner), the slab's
partial sums (one FMA per sign), 1 FMA for g and, for plain draws, 1 add for
the noise sum: 55.75 slots per value with antithetic pairs, 52.75 without.

Counted this way a two-pass pipeline (generate for the loss change, then
regenerate for g) is capped at about half of the roofline; a single
generation can reach all of it.
"""
from __future__ import annotations

CUS = 256
CLOCK_HZ = 2.4e9
LANES_PER_CU_CLOCK = 128
PEAK_SLOTS_PER_S = CUS * LANES_PER_CU_CLOCK * CLOCK_HZ  # 7.864e13

PHILOX_SLOTS_PER_QUAD = 9 * (2 * 4 + 4) + (4 + 1)  # 113
BOX_MULLER_SLOTS_PER_QUAD = 8 * 4 + 18             # 50
GEN_SLOTS_PER_VALUE = (PHILOX_SLOTS_PER_QUAD + BOX_MULLER_SLOTS_PER_QUAD) / 4.0  # 40.75


def distinct_noise_values(T: int, d_out: int, K: int, antithetic: bool) -> int:
    K_n = K // 2 if antithetic else K
    return K_n * T * d_out


def fused_kernel_slots(T: int, d_out: int, K: int, antithetic: bool,
                       per_draw_outputs: bool = False, local: bool = False) -> float:
    """Algorithmic lane-slots of the single-generation kernel (gamma = 0);
    `per_draw_outputs`: the call asks for rho or the credit; `local`: local
    scoring (no curvature term)."""
    need_q = not local and (per_draw_outputs or not antithetic)
    per_value = GEN_SLOTS_PER_VALUE + 2.0 + (1.0 if need_q else 0.0) + \
        (0.0 if antithetic else 1.0)
    return distinct_noise_values(T, d_out, K, antithetic) * per_value


def jitter_kernel_slots(T: int, d_out: int, K: int, antithetic: bool,
                        local: bool = False) -> float:
    """Algorithmic lane-slots of the jitter-loss kernel of the two-pass path
    (P and, for the quadratic loss, Q)."""
    per_value = GEN_SLOTS_PER_VALUE + (1.0 if local else 2.0)
    return distinct_noise_values(T, d_out, K, antithetic) * per_value


def estimate_min_seconds(T: int, d_out: int, K: int, antithetic: bool,
                         local: bool = False) -> float:
    """Lower bound on one estimate: one generation of every noise value."""
    return fused_kernel_slots(T, d_out, K, antithetic, local=local) / PEAK_SLOTS_PER_S


def head_slots_per_value(antithetic: bool) -> float:
    if antithetic:
        return GEN_SLOTS_PER_VALUE + 1.0 + 11.0 + 2.0 + 1.0
    return GEN_SLOTS_PER_VALUE + 1.0 + 8.0 + 1.0 + 1.0 + 1.0


def head_kernel_slots(T: int, V: int, K: int, antithetic: bool) -> float:
    """Algorithmic lane-slots of the cross-entropy head's slab kernel: every
    slab's K draws on every token, i.e. K_n * T * V noise values."""
    return distinct_noise_values(T, V, K, antithetic) * head_slots_per_value(antithetic)


def head_min_seconds(T: int, V: int, K: int, antithetic: bool) -> float:
    return head_kernel_slots(T, V, K, antithetic) / PEAK_SLOTS_PER_S
