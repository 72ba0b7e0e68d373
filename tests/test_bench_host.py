"""Host-side logic of bench.py (no GPU): the one-GPU guard and the readers of the
committed counter summaries, which must report figures only for the sources
they were taken from."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def _write_counters(path, digest):
    rec = {"workload": "fwd-1x32x4096", "floor_bytes": 100, "call_bytes": 150, "bytes_over_floor": 1.5,
           "kernels": {"fa_fwd_kernel<128,false,8>": {"us": 1.0, "l2_hit": 0.9, "mfma_util_counted": 0.5,
                                                       "mfma_busy_est": 0.55, "clock_ghz_est": 1.8},
                       "other": {"us": 2.0, "l2_hit": 0.1, "mfma_util_counted": 0.0}}}
    path.write_text("# title\n\n| a | b |\n\n    " + json.dumps(rec) + f"\n\nsources_sha256_16: {digest}\n")


def test_counters_reported_only_for_matching_sources(tmp_path, monkeypatch):
    f = tmp_path / "counters.md"
    monkeypatch.setattr(bench, "ALL_COUNTERS_FILE", str(f))
    assert bench.measured_counters() is None  # missing file
    _write_counters(f, bench.all_sources_hash())
    got = bench.measured_counters()
    assert got == {"fwd-1x32x4096": {"bytes_over_floor": 1.5, "call_bytes": 150, "floor_bytes": 100, "l2_hit": 0.9,
                                     "mfma_util_counted": 0.5, "mfma_busy_est": 0.55, "clock_ghz_est": 1.8}}
    _write_counters(f, "0" * 16)
    assert bench.measured_counters() is None


def test_traffic_reported_only_for_matching_sources(tmp_path, monkeypatch):
    f = tmp_path / "c.txt"
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(f))
    assert bench.measured_traffic() == (None, None)
    f.write_text(f"# x\nhbm_bytes_per_launch: 12345\ncall_hbm_bytes: 20000\n"
                 f"kernel_source_sha256_16: {bench.kernel_source_hash()}\n")
    assert bench.measured_traffic() == (12345.0, 20000.0)
    f.write_text("hbm_bytes_per_launch: 12345\ncall_hbm_bytes: 20000\nkernel_source_sha256_16: deadbeefdeadbeef\n")
    assert bench.measured_traffic() == (None, None)


def test_committed_counter_summary_is_consistent():
    """Whatever sources it was taken from, the committed summary's records add up."""
    if not os.path.exists(bench.ALL_COUNTERS_FILE):
        pytest.skip("no committed counter summary")
    recs = [json.loads(line) for line in open(bench.ALL_COUNTERS_FILE) if line.strip().startswith("{")]
    assert {r["workload"] for r in recs} >= {"fwd-1x32x4096", "fwd-1x1x8192", "decode"}
    for r in recs:
        total = sum(k["read_bytes"] + k["write_bytes"] for k in r["kernels"].values())
        assert abs(total - r["call_bytes"]) <= len(r["kernels"])
        assert r["bytes_over_floor"] == pytest.approx(r["call_bytes"] / r["floor_bytes"], abs=1e-3)
        for k in r["kernels"].values():
            assert 0 <= k["l2_hit"] <= 1 and 0 <= k["mfma_util_counted"] <= 1


def test_oracle_seconds_by_config_scales_one_head():
    import dataclasses
    import seeded_inputs as si
    fwd = dataclasses.replace(si.TINY, name="tiny 3 heads", B=1, Hq=3, Hkv=3, N=256, sampled_rows=64)
    dec = si.DecodeCase("tiny decode", 2, 4, 2, 64, 64, 4, seed=1)
    r = bench.oracle_seconds_by_config(cases=(fwd,), decode_cases=(dec,))
    f = r["tiny 3 heads"]
    assert f["heads"] == 3 and f["rows_per_head"] == 64
    assert f["seconds"] == pytest.approx(3 * f["seconds_one_head"], abs=2e-3)
    assert f["seconds_all_rows_extrapolated"] == pytest.approx(f["seconds"] * 4, abs=0.1)
    d = r["tiny decode"]
    assert d["sequences"] == 2 and d["rows"] == 8
    assert d["seconds"] == pytest.approx(2 * d["seconds_one_sequence"], abs=2e-3)


def test_parity_by_config_reports_errors_against_the_oracle():
    """The bench's per-config parity report: stand-in results (the oracle's own values, then
    the same moved by a known amount) give the expected errors and pass flags."""
    import dataclasses
    import numpy as np
    import seeded_inputs as si
    from oracle import fa_oracle
    case = dataclasses.replace(si.TINY, name="tiny sampled", Hq=2, Hkv=2, N=200, sampled_rows=40)
    inputs = si.fwd_inputs(case)
    rows = np.stack([si.sample_rows(case.seed, h, case.N, case.sampled_rows) for h in range(case.Hq)])
    q, k, v = (si.bf16_bits_to_f32(x) for x in inputs)
    o_ref, lse_ref = fa_oracle.attention_ref(q, k, v, case.causal, case.scale, rows=rows)
    dec = si.DecodeCase("tiny decode", 2, 4, 2, 64, 64, 4, seed=1)
    dinp = si.decode_inputs(dec)
    od, ld = fa_oracle.decode_ref(*(si.bf16_bits_to_f32(x) for x in dinp), dec.scale)
    good = bench.parity_by_config({"a": (case, o_ref, lse_ref, rows, inputs), "d": (dec, od, ld, None, dinp)})
    assert good["a"]["pass"] and good["a"]["o_max_abs"] < 1e-12 and good["a"]["rows_checked"] == 80
    assert good["d"]["pass"] and good["d"]["rows_checked"] == 8
    bad = bench.parity_by_config({"a": (case, o_ref + 0.02, lse_ref * (1 + 2e-3) + 2e-3, rows, inputs)})
    assert not bad["a"]["pass"]
    assert bad["a"]["o_max_abs"] == pytest.approx(0.02, rel=1e-6)
    assert bad["a"]["lse_max_rel"] >= 2e-3
