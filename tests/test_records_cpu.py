"""Self-consistency of the committed bench records and counter files.

Every `profiles/bench_*.json` is one line that bench.py printed on the GPU.
These checks need no GPU: they re-derive what a record states from its own
fields (rate from bytes or ops and time, roofline fraction from achieved and
peak), check that it was checked against the oracle, and tie any HBM traffic
figure to a committed counter file taken from the current kernel sources.
"""
import glob
import json
import os

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
RECORDS = sorted(glob.glob(os.path.join(ROOT, "profiles", "bench_*.json")))
PEAKS = {"GB/s": 8000.0, "TOPS": 5000.0}  # MI355X HBM; dense int8 matrix cores (5.0 POP/s)


def _load(path):
    with open(path) as f:
        return json.load(f)


def test_records_exist_for_every_configuration():
    keys = {(_load(p)["config"]["key"], _load(p)["config"]["m"]) for p in RECORDS}
    for key in ("single2048", "b2b_decode", "l8b_decode", "l8b_prefill", "l70b_layer"):
        assert any(k == key for k, _ in keys), key
    assert ("l8b_decode", 4) in keys and ("l8b_decode", 8) in keys and ("l70b_layer", 64) in keys


@pytest.mark.parametrize("path", RECORDS, ids=[os.path.basename(p) for p in RECORDS])
def test_record_is_consistent(path):
    d = _load(path)
    assert d["n_gpus"] == 1 and d["higher_is_better"] is True
    assert d["steps"] > 0 and d["warmup"] >= 0
    assert d["data"].startswith("synthetic")
    assert d["parity_vs_oracle"]["ok"] is True
    cfg = d["config"]
    # the rate is the step's algorithmic work over the step time (ms_per_step
    # is printed to 4 decimals: allow for that rounding)
    ms = d["ms_per_step"]
    if d["unit"] == "GB/s":
        work = cfg["step_bytes"] / 1e9
    else:
        assert d["unit"] == "TOPS"
        work = cfg["step_ops"] / 1e12
    lo, hi = work / ((ms + 5e-5) * 1e-3), work / (max(ms - 5e-5, 1e-9) * 1e-3)
    assert lo * 0.999 <= d["value"] <= hi * 1.001, (d["value"], lo, hi)
    r = d["roofline"]
    assert r["peak"] == PEAKS[r["unit"]]
    assert r["bound"] == ("hbm" if r["unit"] == "GB/s" else "mfma")
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    # no kernel time longer than the step: the isolated replays' time per step
    # is either within the step's or the record says it was capped to it
    assert r["kernel_ms_per_step"] <= ms * 1.0005 or "exceeds the step's" in r["timing"], path
    assert r["achieved"] <= r["peak"]
    if r["unit"] == "TOPS":
        # the method's own work: one add or subtract per non-zero weight and token
        assert 0 < r["frac_nonzero_adds"] <= r["frac"] / 2 + 1e-4
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] >= 1 and c["value"] > 0 and c["sample"]


@pytest.mark.parametrize("path", RECORDS, ids=[os.path.basename(p) for p in RECORDS])
def test_traffic_comes_from_current_counters(path):
    d = _load(path)
    traffic = d["roofline"]["traffic"]
    if traffic is None:
        return
    cfg = d["config"]
    variant = cfg.get("variant", "plain")
    suffix = "" if variant == "plain" else "_" + variant
    counters = _load(os.path.join(ROOT, "profiles", "counters_%s_m%d%s.json" % (cfg["key"], cfg["m"], suffix)))
    # the counters may have been taken again on the same sources since the record
    assert abs(counters["hbm_bytes_per_launch"] - traffic) <= 0.01 * traffic
    sources = (bench.LUT_SOURCES if variant == "lut" else
               bench.DECODE_SOURCES if cfg["m"] <= 16 else bench.BATCHED_SOURCES)
    assert counters["kernel_source_hash"] == bench.kernel_source_hash(sources)


def test_default_record_carries_traffic_and_the_decode_extras():
    """The default run (no arguments): the 8B prefill, with the same stack's
    decode at 1, 4 and 8 tokens on the same weights, each checked against the
    oracle and each carrying HBM traffic from the current counters."""
    d = _load(os.path.join(ROOT, "profiles", "bench_l8b_prefill_m512.json"))
    assert d["config"]["key"] == "l8b_prefill" and d["roofline"]["traffic"] is not None
    extras = d["extra_configs"]
    assert sorted(extras) == ["l8b_decode_m1", "l8b_decode_m4", "l8b_decode_m8"]
    for key, e in extras.items():
        assert e["parity_vs_oracle"]["ok"] is True, key
        assert e["unit"] == "GB/s" and e["roofline"]["traffic"] is not None, key
        assert e["roofline"]["kernel_ms_per_step"] <= e["ms_per_step"] * 1.0005 or \
            "exceeds the step's" in e["roofline"]["timing"], key
