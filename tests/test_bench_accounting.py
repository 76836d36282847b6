"""The benchmark's work accounting, checked on the CPU.

The throughput a benchmark line reports is only as good as its flop and byte
counts: 4 d flop per visible (query, key) pair (a multiply and an add for
each of the d terms of Q.K^T and of P.V), and one pass over Q, K, V, O and
the LSE.  These tests pin the visible-pair count against a brute-force count
over the oracle's own visibility rule, and against closed forms of the
standard masks; and the command-line contract's refusals, which need no GPU.
"""
import math

import numpy as np
import pytest

import bench
import oracle
from exact_attention_04_amd.workloads import WORKLOADS, Workload


def brute_pairs(n, causal, wl, wr):
    i = np.arange(n)[:, None]
    j = np.arange(n)[None, :]
    return int(oracle.visible(i, j, n, causal, wl, wr).sum())


@pytest.mark.parametrize("n", [1, 2, 7, 64, 65, 130, 257])
@pytest.mark.parametrize("causal,wl,wr", [(False, -1, -1), (True, -1, -1), (False, 3, 2), (True, 5, -1),
                                          (False, 0, 0), (False, -1, 0), (True, 100, 0), (False, 10, -1)])
def test_visible_pairs_match_brute_force(n, causal, wl, wr):
    w = Workload("t", 1, 1, n, 64, "f16", "bshd", causal, window_left=wl, window_right=wr)
    assert bench.visible_pairs_per_head(w) == brute_pairs(n, causal, wl, wr)


def test_closed_forms_of_the_named_workloads():
    # no mask: N^2; causal: N (N + 1) / 2; causal window of 4096 keys:
    # sum over rows of min(i + 1, 4096)
    assert bench.visible_pairs_per_head(WORKLOADS["sdpa_b2h8n2048d64_f16"]) == 2048 * 2048
    assert bench.visible_pairs_per_head(WORKLOADS["sdpa_b4h32n4096d128_bf16_causal"]) == 4096 * 4097 // 2
    n, w = 16384, 4096
    assert bench.visible_pairs_per_head(WORKLOADS["swa_b1h32n16384d128_bf16_w4095"]) == w * (w + 1) // 2 + (n - w) * w
    assert bench.visible_pairs_per_head(WORKLOADS["fp8_b1h16n65536d128_causal"]) == 65536 * 65537 // 2


def test_headline_flop_and_bytes():
    w = WORKLOADS["sdpa_b4h32n4096d128_bf16_causal"]
    assert bench.workload_flops(w) == 4 * 128 * (4096 * 4097 // 2) * 4 * 32 == 549890031616
    # Q, K, V read once and O written once in bf16, LSE in fp32
    elems = 4 * 32 * 4096 * 128
    assert bench.workload_bytes(w) == 4 * elems * 2 + 4 * 32 * 4096 * 4
    # shared K/V heads read fewer K/V bytes; fp8 inputs are one byte each
    g = WORKLOADS["gqa_b4h32kv8n4096d128_bf16_causal"]
    assert bench.workload_bytes(g) == (elems + 2 * elems // 4) * 2 + elems * 2 + 4 * 32 * 4096 * 4
    f = WORKLOADS["fp8_b1h16n65536d128_causal"]
    fe = 16 * 65536 * 128
    assert bench.workload_bytes(f) == 3 * fe + 2 * fe + 4 * 16 * 65536


def test_mixed_ceiling_is_the_harmonic_mean_of_the_two_rates():
    # half the flop at the fp8 rate, half at the bf16 rate
    t = 0.5 / bench.PEAK_TFLOPS["fp8"] + 0.5 / bench.PEAK_TFLOPS["bf16"]
    assert math.isclose(1.0 / t, 3355.47, rel_tol=1e-4)


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_e4m3_pv_needs_an_fp8_workload(capsys):
    assert bench.main(["--pv-dtype", "e4m3"]) == 2
    assert "fp8" in capsys.readouterr().err


def test_kernel_hash_ignores_comments_only():
    code = "int f(int x) {\n  return x + 1;  // add one\n}\n"
    recommented = "// a header comment\nint f(int x) {\n\n  return x + 1;  // a different note\n}\n"
    changed = "int f(int x) {\n  return x + 2;  // add one\n}\n"
    assert bench.kernel_code(code) == bench.kernel_code(recommented)
    assert bench.kernel_code(code) != bench.kernel_code(changed)


@pytest.mark.parametrize("name", ["sdpa_b4h32n4096d128_bf16_causal", "fp8_b1h16n65536d128_causal",
                                  "fp8_b1h16n65536d128_causal_pv8"])
def test_traffic_records_are_well_formed(name):
    # a committed HBM-traffic record: keyed by a 16-hex source hash, and at
    # least the one-pass algorithmic bytes (a kernel cannot read less)
    import json
    import os
    with open(os.path.join(bench.ROOT, "profiles", f"traffic_{name}.json")) as f:
        rec = json.load(f)
    assert len(rec["kernel_sha256_16"]) == 16 and int(rec["kernel_sha256_16"], 16) >= 0
    w = WORKLOADS[name.replace("_pv8", "")]
    assert rec["hbm_bytes_per_launch"] >= bench.workload_bytes(w)


def test_backward_traffic_record_is_well_formed():
    # the backward's record: keyed by the backward sources' hash, and at least
    # one pass over its algorithmic bytes (q, k, v, o, dout read; dq, dk, dv
    # written; lse read and delta written)
    import json
    import os
    name = "sdpa_b4h32n4096d128_bf16_causal"
    with open(os.path.join(bench.ROOT, "profiles", f"traffic_bwd_{name}.json")) as f:
        rec = json.load(f)
    assert len(rec["kernel_sha256_16"]) == 16 and int(rec["kernel_sha256_16"], 16) >= 0
    w = WORKLOADS[name]
    q_el = w.batch * w.heads * w.seqlen * w.headdim
    kv_el = w.batch * w.kv_heads * w.seqlen * w.headdim
    alg = 2 * (3 * q_el + 2 * kv_el) + 2 * (q_el + 2 * kv_el) + 8 * w.batch * w.heads * w.seqlen
    assert rec["hbm_bytes_per_launch"] >= alg
    assert rec["hbm_bytes_per_launch"] == rec["hbm_read_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]
