"""bench.py's command line on a machine without a GPU: more than one GPU is
refused with a message, and the workload names it accepts are the
synthetic workloads."""
import os
import subprocess
import sys

from token_activation_perturbation_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    res = run("--gpus", "2")
    assert res.returncode != 0
    assert "one GPU" in (res.stdout + res.stderr)


def test_unknown_workload_is_refused():
    res = run("--workload", "no_such_workload", "--cpu-budget", "0")
    assert res.returncode != 0
    assert "unknown workload" in res.stderr and "bf16_layer" in res.stderr


def test_default_workload_is_the_largest_reference_configuration():
    """The headline is the MLP up-projection: the reference configuration
    with the most noise values and MFMA work per call; the five reference
    configurations are all measured by default."""
    assert "mlp_up_bf16" in synth.WORKLOADS
    src = open(os.path.join(ROOT, "bench.py")).read()
    assert 'HEADLINE = "mlp_up_bf16"' in src
    ref = ["tiny_f32", "bf16_layer", "mlp_up_bf16", "qkv_credit_bf16", "large_population_bf16"]
    assert all(r in src for r in ref)
    big = max(ref, key=lambda n: (synth.WORKLOADS[n].K // (2 if synth.WORKLOADS[n].antithetic
                                                          else 1)) * synth.WORKLOADS[n].T
              * synth.WORKLOADS[n].d_out)
    assert big == "mlp_up_bf16"


def test_unknown_config_is_refused():
    res = run("--configs", "bf16_layer,nope", "--cpu-budget", "0")
    assert res.returncode != 0
    assert "unknown workload" in res.stderr


def test_kernel_hash_ignores_comments_only():
    """The committed HBM-traffic figures stay valid across comment edits of
    the kernel sources but not across code edits."""
    sys.path.insert(0, ROOT)
    import bench
    code = 'int a = 1; // note\n/* block\n comment */ const char* s = "//x"; int b;\n'
    assert bench._code_only(code) == bench._code_only(
        'int a = 1; // other note\n/* another */ const char* s = "//x";\n  int b;')
    assert bench._code_only(code) != bench._code_only(code.replace("int b;", "int c;"))
    assert bench._code_only(code) != bench._code_only(code.replace('"//x"', '"//y"'))


def test_kernel_hash_covers_the_attention_sources_only_for_attention_workloads(monkeypatch):
    import bench
    base = bench.kernel_source_hash("mlp_up_bf16")
    attn = bench.kernel_source_hash("attn_key_bf16")
    assert base != attn
    assert bench.kernel_source_hash("attn_value_bf16") == attn
    # another attention source changes the attention hash only
    monkeypatch.setattr(bench, "ATTENTION_SOURCES",
                        ["token_activation_perturbation_amd/csrc/dust_noise.hpp"])
    assert bench.kernel_source_hash("mlp_up_bf16") == base
    assert bench.kernel_source_hash("attn_key_bf16") != attn
