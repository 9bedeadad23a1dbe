"""The ALU roofline of the estimator's noise kernels on MI355X (gfx950).

The noise kernels move almost no memory: each noise value is a pure function
of (seed, noise index, token, channel), generated in registers and consumed
at once.  Their bound is the vector ALU issue rate, counted in lane-slots:

* Peak.  MI355X: 256 compute units at 2.4 GHz; its fp32 vector peak of
  157.3 TFLOP/s is 2 flops x 128 lanes per clock per CU, so a single-pass
  32-bit VALU operation occupies one of 256 x 128 x 2.4e9 = 7.864e13
  lane-slots per second.

* Issue cost of each instruction, by the rate class measured on an MI355X
  with a one-off instruction-rate probe (each instruction alone, operands
  in vector registers, lanes per CU per clock at the clock measured during
  the run): single-pass operations (xor, shifts, fp32
  add / mul / fma, the three-input bitwise op) 1 slot (107-122 lanes per
  clock for the two-operand forms; the three-operand forms alone reach ~80,
  a register-read limit that a mixed stream does not hit, so they count 1);
  32x32->64 integer multiply-add, 32-bit high/low products and the
  integer-to-float conversion 2 slots (~61 lanes per clock); the
  transcendentals log2, sqrt, sin, cos 4 slots (~30.5).  Under-weighting a
  class only lowers the fraction, so the model stays a lower bound on time.

* Work per distinct noise value (the minimum the method needs: each of the
  K_n * T * d_out values generated once, where K_n = K/2 with antithetic
  pairs, else K).  The counter is (quad, token, noise index, 0): only the
  quad index differs per lane, and the first round's products are either
  wave-uniform (the noise index's, on the scalar unit) or the same for
  every noise index of a (token, quad) (the quad index's, computed once per
  lane), as is the second round's product of the first round's per-lane
  word.  Per quad of four values and draw:
    Philox4x32-10   second round: 2 xors                          =  2 slots
                    third round: 2 products x 2 + 1 three-input xor
                    + 1 xor (its other two words are wave-uniform) =  6
                    rounds 4-10: 7 x (2 products x 2 + 2 three-input
                    xors)                                          = 42
                                                                   = 50 slots
    Box-Muller      per pair: 2 funnel shifts (each word's top 23 bits
                    as the mantissa of a float in [1, 2)), 1 subtraction
                    for u, log2, sqrt, sin, cos x 4, 2 multiplies by
                    the radius = 21 (the values come in units of
                    sqrt(2 ln 2), which the consumers apply once per
                    reduced total or output, not per value);       = 42 slots
  That gives 23 slots per value, plus the consumers: 1 FMA for
  P = <delta, a>, 1 FMA for Q = ||a||^2 (the quadratic loss's curvature
  term: needed by plain draws and by the per-draw outputs; with antithetic
  pairs it cancels inside each pair, so a call that asks only for g and G_W
  does without it, and local scoring, linear in the jitter, never needs
  it), 1 FMA for the reweighted sum g, and 1 add for the plain-draw noise
  sum used by the centring.

The cross-entropy head's slab kernel consumes each value as: 1 multiply
(sigma a), the jitter's expm1 (antithetic: both signs from the even and odd
Taylor parts, 9 + 2 slots; plain draws: 8 slots of Horner), the slab's
partial sums (one FMA per sign), 1 FMA for g and, for plain draws, 1 add for
the noise sum: 38 slots per value with antithetic pairs, 35 without.

The generation alone (noise_quad in a loop, the probe's last row) runs at
~0.84 of this model's peak with the clock at 2.4 GHz: the
practical ceiling the noise kernels are measured against in the text.
Counted this way a two-pass pipeline (generate for the loss change, then
regenerate for g) is capped at about half of the roofline; a single
generation can reach all of it.
"""
from __future__ import annotations

CUS = 256
CLOCK_HZ = 2.4e9
LANES_PER_CU_CLOCK = 128
PEAK_SLOTS_PER_S = CUS * LANES_PER_CU_CLOCK * CLOCK_HZ  # 7.864e13

# issue cost classes, in lane-slots per lane: single-pass, half-rate
# (integer products, integer-to-float conversion), quarter-rate
# (transcendentals)
SINGLE, HALF, QUARTER = 1, 2, 4

PHILOX_SLOTS_PER_QUAD = (2 * SINGLE                         # second round
                         + 2 * HALF + 2 * SINGLE            # third round
                         + 7 * (2 * HALF + 2 * SINGLE))     # rounds 4-10: 50
BOX_MULLER_SLOTS_PER_QUAD = 2 * (2 * SINGLE               # funnel shifts: u, v fields
                                 + 1 * SINGLE               # u = 2 - (1 + m 2^-23)
                                 + 4 * QUARTER              # log2, sqrt, sin, cos
                                 + 2 * SINGLE)              # radius x 2: 42
GEN_SLOTS_PER_VALUE = (PHILOX_SLOTS_PER_QUAD + BOX_MULLER_SLOTS_PER_QUAD) / 4.0  # 23


def distinct_noise_values(T: int, d_out: int, K: int, antithetic: bool) -> int:
    K_n = K // 2 if antithetic else K
    return K_n * T * d_out


def fused_kernel_slots(T: int, d_out: int, K: int, antithetic: bool,
                       per_draw_outputs: bool = False, local: bool = False) -> float:
    """Algorithmic lane-slots of the single-generation kernels (gamma = 0;
    and the gamma > 0 chain kernel of antithetic pairs, which also adds P's
    and g's FMAs per value); `per_draw_outputs`: the call asks for rho or
    the credit; `local`: local scoring (no curvature term)."""
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


def reweight_kernel_slots(T: int, d_out: int, K: int, antithetic: bool) -> float:
    """The reweight pass of the two-pass path: the noise generated again and
    one FMA per value into g."""
    return distinct_noise_values(T, d_out, K, antithetic) * (GEN_SLOTS_PER_VALUE + 1.0)


# ---------------------------------------------------------------------------
# Every stage against its own roofline.  The other units' peaks on MI355X:
# dense MFMA (bf16 operands, fp32 accumulation) 2.5 PFLOP/s, fp32 MFMA
# 157.3 TFLOP/s, HBM3E 8 TB/s.

MFMA_PEAK_FLOPS = {"bf16": 2.5e15, "f32": 157.3e12}
HBM_PEAK_BYTES = 8.0e12

# ---------------------------------------------------------------------------
# Scores through a recomputed attention (the attention site's score kernel).
# Per (sequence, head, noise vector) the method computes, for every causal
# pair s >= t of the sequence, one d_head-long dot product of the jittered
# operand with the noise (the MFMA contraction, 2 d_head flops per pair,
# priced as one bf16 contraction although the kernel issues it twice, once
# per half of the noise's hi + lo split), then per pair: keys and queries
# e^x - 1 from its Taylor series to x^5 (enough below the |x| < 1/4 that
# holds for nearly every pair at the workloads' sigma: u = x^2, the odd
# part 3 slots, the even part 2), with antithetic pairs one FMA per row sum
# and part (p and B against the even and odd parts: 4) and the two signs'
# combination per tile (1 per pair) = 11, with plain draws e^x - 1 = even
# + odd (1) and one FMA per row sum (2) = 9; values one FMA.  The logit
# change's scale rides on the noise (one multiply per noise value).  Each
# noise value (K_n T d_out of them) is generated once.

def attention_pairs(T: int, seq_len: int, heads: int) -> float:
    """Causal (s, t) pairs of every (sequence, head)."""
    return (T // seq_len) * heads * seq_len * (seq_len + 1) / 2.0


def attention_score_flops(T: int, seq_len: int, heads: int, d_head: int, K: int,
                          antithetic: bool) -> float:
    K_n = K // 2 if antithetic else K
    return 2.0 * attention_pairs(T, seq_len, heads) * d_head * K_n


def attention_score_slots(site: str, T: int, seq_len: int, heads: int, d_head: int, K: int,
                          antithetic: bool) -> float:
    K_n = K // 2 if antithetic else K
    if site == "value":
        per_pair = 1.0
    else:
        per_pair = 11.0 if antithetic else 9.0
    gen = distinct_noise_values(T, heads * d_head, K, antithetic) * (GEN_SLOTS_PER_VALUE + 1.0)
    return K_n * attention_pairs(T, seq_len, heads) * per_pair + gen


def attention_score_bound(site: str, T: int, seq_len: int, heads: int, d_head: int, K: int,
                          antithetic: bool) -> tuple:
    """(bound, algorithmic work, peak per second, unit) of the score kernel:
    the unit whose work takes longer at its peak."""
    slots = attention_score_slots(site, T, seq_len, heads, d_head, K, antithetic)
    flops = attention_score_flops(T, seq_len, heads, d_head, K, antithetic)
    if slots / PEAK_SLOTS_PER_S >= flops / MFMA_PEAK_FLOPS["bf16"]:
        return "alu", slots, PEAK_SLOTS_PER_S, "T lane-slot/s"
    return "mfma", flops, MFMA_PEAK_FLOPS["bf16"], "TFLOP/s"


# stages whose bound is the vector ALU (each generates noise values)
NOISE_STAGES = ("fused_g0_kernel", "chain_g_kernel", "jitter_loss_kernel", "reweight_kernel",
                "head_ce_kernel")


def noise_stage_slots(kernel: str, T: int, d_out: int, K: int, antithetic: bool,
                      per_draw_outputs: bool = False, local: bool = False) -> float:
    """Algorithmic lane-slots of one launch of a noise stage (d_out is the
    vocabulary for the head)."""
    if kernel == "fused_g0_kernel":
        return fused_kernel_slots(T, d_out, K, antithetic, per_draw_outputs, local)
    if kernel == "chain_g_kernel":
        return fused_kernel_slots(T, d_out, K, antithetic, False, local)
    if kernel == "jitter_loss_kernel":
        return jitter_kernel_slots(T, d_out, K, antithetic, local)
    if kernel == "reweight_kernel":
        return reweight_kernel_slots(T, d_out, K, antithetic)
    if kernel == "head_ce_kernel":
        return head_kernel_slots(T, d_out, K, antithetic)
    raise KeyError(kernel)


def stage_roofline(kernel: str, ms: float, flops: float, nbytes: float, dtype: str,
                   slots: float | None = None) -> dict:
    """One stage's time against the bound of its kind: the ALU slot model for
    the noise stages (`slots`), the MFMA peak of the operand type for a
    contraction (`flops` > 0), HBM for the rest.  Every stage also carries its
    HBM rate (algorithmic bytes / time) and `bound_ms`, the time its slowest
    unit needs at peak (the larger of its ALU, MFMA and HBM times)."""
    t = ms * 1e-3
    hbm = nbytes / t if t > 0 else float("nan")
    alu_s = (slots or 0.0) / PEAK_SLOTS_PER_S
    mfma_s = flops / MFMA_PEAK_FLOPS[dtype] if flops > 0 else 0.0
    hbm_s = nbytes / HBM_PEAK_BYTES
    out = {"kernel": kernel, "ms": ms, "hbm_GBps": hbm / 1e9, "hbm_frac": hbm / HBM_PEAK_BYTES,
           "bound_ms": max(alu_s, mfma_s, hbm_s) * 1e3}
    if slots is not None:
        achieved = slots / t / 1e12
        out.update(bound="alu", achieved=achieved, peak=PEAK_SLOTS_PER_S / 1e12,
                   unit="T lane-slot/s", frac=achieved / (PEAK_SLOTS_PER_S / 1e12))
    elif flops > 0:
        achieved = flops / t / 1e12
        peak = MFMA_PEAK_FLOPS[dtype] / 1e12
        out.update(bound="mfma", achieved=achieved, peak=peak, unit="TFLOP/s",
                   frac=achieved / peak)
    else:
        out.update(bound="hbm", achieved=hbm / 1e9, peak=HBM_PEAK_BYTES / 1e9, unit="GB/s",
                   frac=hbm / HBM_PEAK_BYTES)
    return out
