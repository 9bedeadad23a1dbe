"""The ALU cost model against the instructions the compiler emits for the
noise.  A kernel that draws noise_quad for one (token, quad) per lane over a
loop of noise indices (the noise kernels' own shape: the quad index is the
only per-lane counter word) is compiled for gfx950 with the library's flags;
the loop body's instructions per quad must be the ones the model counts:
16 32x32->64 multiply-adds, 15 three-input xors and 3 xors for Philox
(50 slots at 2 per product and 1 per single-pass op), and for Box-Muller 4
funnel shifts (each uniform built in a float's bit fields, no
integer-to-float conversion), 2 subtractions (u = 2 - x), 8
transcendentals and 4 multiplies by the radius (the values come in units of
sqrt(2 ln 2): no multiply by -2 ln 2).  The same holds for noise_quad_x2, which the kernels use to
advance two quads' Philox rounds together (pairs of noise indices here): it
must not cost a single extra instruction per quad.  Needs hipcc
(cross-compiles, no GPU)."""
import os
import re
import shutil
import subprocess
from collections import Counter

import pytest

from token_activation_perturbation_amd import build, roofline

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
QUADS_PER_ITER = 4

KERNELS = {
    "single": r"""
#include <hip/hip_runtime.h>
#include "dust_noise.hpp"
__global__ void gen(float* out, unsigned t, int K, dust::NoiseKey key) {
  const unsigned q = threadIdx.x;
  float r = 0.f;
  for (int n = 0; n < K; n += 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 a = dust::noise_quad(q, t, (unsigned)(n + j), key);
      r += a.x + a.y + a.z + a.w;
    }
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = r;
}
""",
    "paired": r"""
#include <hip/hip_runtime.h>
#include "dust_noise.hpp"
__global__ void gen(float* out, unsigned t, int K, dust::NoiseKey key) {
  const unsigned q = threadIdx.x;
  float r = 0.f;
  for (int n = 0; n < K; n += 4) {
#pragma unroll
    for (int j = 0; j < 4; j += 2) {
      float4 a, b;
      dust::noise_quad_x2(q, (unsigned)(n + j), q, (unsigned)(n + j + 1), t, key, a, b);
      r += a.x + a.y + a.z + a.w;
      r += b.x + b.y + b.z + b.w;
    }
  }
  out[blockIdx.x * blockDim.x + threadIdx.x] = r;
}
""",
}


@pytest.fixture(scope="module", params=sorted(KERNELS))
def loop_ops(request, tmp_path_factory):
    if shutil.which(HIPCC) is None and not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("isa")
    src, asm = d / "gen.hip", d / "gen.s"
    src.write_text(KERNELS[request.param])
    flags = [f for f in build.COMMON_FLAGS]
    res = subprocess.run([HIPCC, *flags, "--cuda-device-only", "-S", "-o", str(asm), str(src)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    body, inside = [], False
    for line in asm.read_text().splitlines():
        if "Loop Header" in line:
            inside = True
            continue
        if inside:
            if re.match(r"\s+s_cbranch_scc", line):
                break
            m = re.match(r"\s+(v_\w+)", line)
            if m:
                body.append(m.group(1))
    assert body, "no loop body found"
    counts = Counter(body)
    return {k: v / QUADS_PER_ITER for k, v in counts.items()}


def count(ops, prefix):
    return sum(v for k, v in ops.items() if k.startswith(prefix))


def test_philox_stream_is_the_modelled_one(loop_ops):
    mads = count(loop_ops, "v_mad_u64_u32")
    bitop3 = count(loop_ops, "v_bitop3_b32")
    xors = count(loop_ops, "v_xor_b32")
    assert (mads, bitop3, xors) == (16, 15, 3)
    slots = roofline.HALF * mads + roofline.SINGLE * (bitop3 + xors)
    assert slots == roofline.PHILOX_SLOTS_PER_QUAD


def test_box_muller_stream_is_the_modelled_one(loop_ops):
    trans = sum(count(loop_ops, p) for p in ("v_log_f32", "v_sqrt_f32", "v_sin_f32", "v_cos_f32"))
    assert trans == 8
    assert count(loop_ops, "v_alignbit_b32") == 4
    assert count(loop_ops, "v_sub_f32") == 2
    # no integer-to-float conversion, no separate shift, and the log's
    # negation rides on the square root as a source modifier
    assert count(loop_ops, "v_cvt_f32") == 0
    assert count(loop_ops, "v_lshrrev_b32") == 0
    # 4 radius products per quad, of which the test loop's own sum fuses 3
    # into FMAs
    assert count(loop_ops, "v_mul_f32") + count(loop_ops, "v_fmac_f32") == 4
    # no other integer products or transcendentals in the generation
    assert count(loop_ops, "v_mul_hi_u32") == 0 and count(loop_ops, "v_mul_lo_u32") == 0
    assert count(loop_ops, "v_exp_f32") == 0 and count(loop_ops, "v_rcp_f32") == 0
