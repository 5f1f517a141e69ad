"""Host logic of bench.py (CPU only): the one-GPU contract, argument checks,
the pairing of stored counter readings with the kernel sources, the FLOP and
byte counts, and the CPU-baseline leg on the tiny workload."""

import math

import numpy as np
import pytest

import bench
from bf16_causal_prefill_fwd_amd.workloads import WORKLOADS, make_inputs


@pytest.mark.parametrize("argv", [["--gpus", "2"], ["--gpus", "8"], ["--steps", "0"], ["--warmup", "-1"]])
def test_bad_invocations_exit_2(argv, capsys):
    assert bench.main(argv) == 2
    assert capsys.readouterr().err


def test_world_size_above_one_exits_2(monkeypatch):
    monkeypatch.setenv("WORLD_SIZE", "2")
    assert bench.main([]) == 2


def test_causal_flops_and_bytes_match_the_counting_convention():
    # B*Hq*S^2*(d_qk+d_v): the causal half of the two products
    assert WORKLOADS["mha_fp8_32k"].causal_flops == 8796093022208.0
    assert WORKLOADS["tiny_mha_fp8"].causal_flops == 2 * 512 ** 2 * 256
    assert math.isclose(WORKLOADS["gqa_fp8_outlier_16k"].causal_flops, 2.199e12, rel_tol=1e-3)
    assert math.isclose(WORKLOADS["mla_fp8_16k"].causal_flops, 1.374e12, rel_tol=1e-3)
    # Q, K, V once (1 byte each in FP8), O in bf16, LSE in fp32
    w = WORKLOADS["mha_fp8_32k"]
    assert bench.algorithmic_bytes(w) == 3 * 32768 * 32 * 128 + 32768 * 32 * 128 * 2 + 32 * 32768 * 4


def test_source_hash_ignores_comments_and_spacing():
    a = "int f(int x) {\n  return x + 1;  // add one\n}\n/* block\n comment */"
    b = "int f(int x) { return x + 1; }"
    c = "int f(int x) { return x + 2; }"
    assert bench.code_only(a) == bench.code_only(b)
    assert bench.code_only(b) != bench.code_only(c)
    h = bench.kernel_source_hash()
    assert len(h) == 16 and h == bench.kernel_source_hash()


def test_traffic_reading_needs_the_current_sources():
    h = bench.kernel_source_hash()
    t = bench.traffic_from_profile("mha_fp8_32k", h)
    # when the summary matches the sources, its reading exceeds the algorithmic
    # bytes (K/V prefixes are re-read); a summary of other sources is ignored
    assert t is None or t > bench.algorithmic_bytes(WORKLOADS["mha_fp8_32k"])
    assert bench.traffic_from_profile("mha_fp8_32k", "0" * 16) is None
    assert bench.traffic_from_profile("no_such_workload", h) is None


@pytest.mark.parametrize("hadamard", [False, True])
def test_cpu_baseline_leg_on_the_tiny_workload(hadamard):
    w = WORKLOADS["tiny_mha_fp8"]
    q, k, v = make_inputs(w, seed=0)
    from oracle import prefill_reference
    ref = prefill_reference(q, k, v, "fp8", fold_q=True, hadamard=hadamard)
    # stand-ins for the GPU's outputs: the exact result, and one perturbed by 1 %
    r = bench.cpu_baseline(w, q, k, v, hadamard=hadamard, o_gpu=ref["o"][0], lse_gpu=ref["lse"][0])
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0 and r["cores"] >= 1
    assert "query heads 0-1" in r["sample"] and "2/2 of the workload" in r["sample"]
    e = r["gpu_error_on_sample"]
    assert e["o_rel_l2"] < 1e-12 and e["lse_max_abs"] < 1e-12
    r = bench.cpu_baseline(w, q, k, v, hadamard=hadamard, o_gpu=ref["o"][0] * 1.01, lse_gpu=ref["lse"][0] + 0.002)
    assert abs(r["gpu_error_on_sample"]["o_rel_l2"] - 0.01) < 1e-9
    assert abs(r["gpu_error_on_sample"]["lse_max_abs"] - 0.002) < 1e-9
    assert r["tiny_one_thread"]["threads"] == 1 and r["tiny_one_thread"]["gflops"] > 0
