"""bench.py's contract pieces that need no GPU: the single-device refusal,
the algorithmic byte and op counts behind `value` and `roofline.achieved`
(pinned to the figures of the workload definitions), and the scaling of
HBM counters by a plain copy."""
from __future__ import annotations

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def run_bench(*args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT, env=e,
                          capture_output=True, text=True, timeout=120)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2 and "one GPU" in r.stderr
    r = run_bench(env={"WORLD_SIZE": "4"})
    assert r.returncode == 2


def step_bytes(key, m):
    wl = synth.BY_KEY[key]
    return wl.layers * sum(bench.forward_bytes(m, mt.n, mt.k) for mt in wl.matrices)


def test_step_bytes_match_the_workload_figures():
    # the decode workloads' algorithmic bytes per step (weights 2 bits, codes,
    # a', gamma, fp32 outputs), as stated with the workload definitions
    assert step_bytes("single2048", 1) == 1_058_824
    assert step_bytes("b2b_decode", 1) == 524_184_000
    assert round(step_bytes("l8b_decode", 1) / 1e9, 3) == 1.751
    assert round(step_bytes("l8b_decode", 4) / 1e9, 3) == 1.770
    assert round(step_bytes("l8b_decode", 8) / 1e9, 3) == 1.796
    assert round(step_bytes("l70b_layer", 1) / 1e6, 2) == 176.46
    wl = synth.BY_KEY["l8b_prefill"]
    ops = wl.layers * sum(2 * 512 * mt.n * mt.k for mt in wl.matrices)
    assert round(ops / 1e12, 3) == 7.147


def test_variant_byte_counts():
    n, k, m = 2560, 6912, 1
    base = bench.forward_bytes(m, n, k)
    assert bench.mode_forward_bytes("rowscale", m, n, k) == base - 4 + 2 * n       # fp16 row scales replace gamma
    assert bench.mode_forward_bytes("tensor128", 3, n, k) == bench.forward_bytes(3, n, k) - 12 + 4  # one g, not a' per token
    assert bench.mode_forward_bytes("binary", m, n, k) == base - (n * k) // 8      # one bit per weight
    assert bench.mode_forward_bytes("binary", m, n, k, fused=True) == (n * k) // 8 + 2 * m * k + 4 + 4 * m * n
    assert bench.swiglu_bytes(1, 6912, 2560) == 2 * (6912 * 2560 // 4) + 2560 + 4 + 8 + 4 * 6912


def write_counter_csv(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_counter_scaling(tmp_path):
    # a copy of 1 MiB whose FETCH_SIZE reads half the bytes gives the factor 2;
    # a kernel reading 300 KiB by the counter then moved 600 KiB
    cf, cw = tmp_path / "cf.csv", tmp_path / "cw.csv"
    write_counter_csv(cf, [{"Dispatch_Id": 1, "Kernel_Name": "copyBuffer", "Counter_Name": "FETCH_SIZE",
                            "Counter_Value": 512.0}])
    write_counter_csv(cw, [{"Dispatch_Id": 1, "Kernel_Name": "copyBuffer", "Counter_Name": "WRITE_SIZE",
                            "Counter_Value": 1024.0}])
    pf, pw = tmp_path / "pf.csv", tmp_path / "pw.csv"
    write_counter_csv(pf, [{"Dispatch_Id": d, "Kernel_Name": "void gemv_lds_kernel<16>(x)",
                            "Counter_Name": "FETCH_SIZE", "Counter_Value": 300.0} for d in (1, 2)])
    write_counter_csv(pw, [{"Dispatch_Id": d, "Kernel_Name": "void gemv_lds_kernel<16>(x)",
                            "Counter_Name": "WRITE_SIZE", "Counter_Value": 10.0} for d in (1, 2)])
    f_fetch = 1024.0 / bench._counter_avg_kib(str(cf), "copy")[0]
    f_write = 1024.0 / bench._counter_avg_kib(str(cw), "copy")[0]
    assert (f_fetch, f_write) == (2.0, 1.0)
    kf, nf = bench._counter_avg_kib(str(pf), "gemv_lds_kernel")
    kw, nw = bench._counter_avg_kib(str(pw), "gemv_lds_kernel")
    assert (kf, nf, kw, nw) == (300.0, 2, 10.0, 2)
    assert (kf * f_fetch + kw * f_write) * 1024 == 610 * 1024


def test_fused_default_follows_the_measured_limits():
    # the fused quant + forward entry is the step's default, per matrix, only
    # where it was measured faster than quant + forward: one token, or m * k
    # values within the limit
    assert bench.fused_default("plain", 1, 28672) and bench.fused_default("rmsnorm", 1, 28672)
    assert [bench.fused_default("plain", m, 4096) for m in (2, 4, 8, 9)] == [True, True, True, False]
    assert [bench.fused_default("plain", m, 14336) for m in (2, 4)] == [True, False]
    assert [bench.fused_default("plain", 4, k) for k in (2560, 6912, 14336)] == [True, True, False]
    assert [bench.fused_default("rmsnorm", m, 2560) for m in (2, 4, 8)] == [True, True, False]
    assert [bench.fused_default("rmsnorm", 2, k) for k in (4096, 6912, 14336)] == [True, True, False]
    assert not bench.fused_default("plain", 17, 64)  # past the decode entry points' token limit
    for variant in ("swiglu", "lut", "binary", "tensor128", "rowscale"):
        assert bench.fused_default(variant, 1, 4096) and not bench.fused_default(variant, 2, 64)
    # per matrix of the 8B stack: the k = 4096 matrices fused at 4 and 8 tokens, the down projection not
    wl = synth.BY_KEY["l8b_decode"]
    for m in (4, 8):
        assert bench.default_fused(wl, m, "plain") == tuple(mt.k == 4096 for mt in wl.matrices)
    assert bench.default_fused(wl, 16, "plain") == (False,) * len(wl.matrices)
    assert bench.default_fused(wl, 1, "lut") == (False,) * len(wl.matrices)
    assert bench.default_fused(wl, 1, "swiglu") == (True,) * len(wl.matrices)
    # the fused call's algorithmic bytes: bf16 activations instead of codes and a'
    n, k, m = 4096, 14336, 4
    assert bench.fused_bytes(m, n, k) - bench.forward_bytes(m, n, k) == 2 * m * k - (m * k + 4 * m)


def test_kernel_source_hash_ignores_comments_only():
    """The counters in profiles/ are tied to the kernels' code: a comment or
    whitespace edit keeps the hash, any code edit changes it, and comment
    markers inside string or character literals are code."""
    import bench
    base = 'int f(int a) { return a + 1; } // tail\n/* block\n comment */ const char* s = "//x";'
    assert bench._code_only(base) == bench._code_only(base.replace("// tail", "// other words"))
    assert bench._code_only(base) == bench._code_only(base.replace("a + 1", "a  +\n 1"))
    assert bench._code_only(base) != bench._code_only(base.replace("a + 1", "a + 2"))
    assert bench._code_only(base) != bench._code_only(base.replace('"//x"', '"//y"'))
    assert "//x" in bench._code_only(base) and "block" not in bench._code_only(base)
