"""CPU: bench.py's host logic (workload names, FLOP model, multi-GPU refusal)."""
import argparse
import os

import numpy as np
import pytest

import bench


def test_named_workloads_follow_the_shape_pattern():
    for name, cfg in bench.WORKLOADS.items():
        assert bench.WORKLOAD_RE.match(name), name
        assert bench.workload_config(name) == cfg


def test_shape_named_workload():
    assert bench.workload_config("causal_b2_h16_n8192_d128_fwdbwd") == dict(
        B=2, H=16, N=8192, d=128, causal=True, sparse=False, bwd=True)
    assert bench.workload_config("blocksparse_b1_h4_n1000_d64_fwd") == dict(
        B=1, H=4, N=1000, d=64, causal=False, sparse=True, bwd=False)


@pytest.mark.parametrize("name", ["dense_b1_h2_n256_d96_fwd", "causal_b0_h2_n256_d64_fwd", "sparse_b1_h2_n256_d64_fwd",
                                  "dense_b1_h2_n256_d64_bwd", "dense_b1_h2_n256_d64"])
def test_bad_workload_names_are_rejected(name):
    with pytest.raises(argparse.ArgumentTypeError):
        bench.workload_config(name)


def test_flop_model():
    cfg = dict(B=2, H=3, N=256, d=64, causal=False, sparse=False, bwd=False)
    assert bench.fwd_flops(cfg) == 4.0 * 2 * 3 * 256 * 256 * 64
    assert bench.fwd_flops(dict(cfg, causal=True)) == 2.0 * 2 * 3 * 256 * 256 * 64
    # a full block mask counts every 128 x 128 block; under causal the
    # diagonal blocks count half
    m = np.ones((3, 2, 2), dtype=np.uint8)
    assert bench.fwd_flops(dict(cfg, sparse=True), m) == bench.fwd_flops(cfg)
    assert bench.fwd_flops(dict(cfg, sparse=True, causal=True), m) == bench.fwd_flops(dict(cfg, causal=True))


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def _fake_run(path, values):
    """A rocprofv3-like results database: values {kernel_name: {counter: value}}."""
    import sqlite3
    os.makedirs(path, exist_ok=True)
    con = sqlite3.connect(os.path.join(path, "run_results.db"))
    con.execute("create table counters_collection (dispatch_id int, kernel_name text, counter_name text, value real)")
    for d, (kn, cs) in enumerate(values.items()):
        for c, v in cs.items():
            con.execute("insert into counters_collection values (?, ?, ?, ?)", (d, "void fa::" + kn + "(fa::X)", c, v))
    con.commit()
    con.close()


def test_summarize_counters(tmp_path, monkeypatch):
    """Counter summary arithmetic: HBM bytes scaled by the copy calibration,
    MFMA busy over the SIMDs' clock, keyed by kernel role and source hash."""
    import json
    monkeypatch.setattr(bench, "COUNTERS_JSON", str(tmp_path / "counters.json"))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    monkeypatch.setattr(bench, "source_sha", lambda name: "feedbeef")
    fwd = "fa_fwd_kernel<128, 64, 4, true, false, false, false>"
    _fake_run(tmp_path / "r" / "cal_fetch", {"copy": {"FETCH_SIZE": 524288.0}})
    _fake_run(tmp_path / "r" / "cal_write", {"copy": {"WRITE_SIZE": 1048576.0}})
    _fake_run(tmp_path / "r" / "fetch", {fwd: {"FETCH_SIZE": 1000.0}})
    _fake_run(tmp_path / "r" / "write", {fwd: {"WRITE_SIZE": 500.0}})
    sq = {c: 1.0 for c in bench.SQ_COUNTERS.split()}
    sq.update(GRBM_GUI_ACTIVE=8.0 * 1000, SQ_VALU_MFMA_BUSY_CYCLES=0.5 * 1024 * 1000, SQ_INSTS_MFMA=10.0,
              SQ_INSTS_VALU=60.0, SQ_WAVE_CYCLES=0.25 * 1024 * 1000 * 1.5)
    _fake_run(tmp_path / "r" / "sq", {fwd: sq})
    assert bench.summarize_counters(str(tmp_path / "r"), "causal_b4_h16_n4096_d128_fwdbwd") == 0
    rec = json.load(open(tmp_path / "counters.json"))["causal_b4_h16_n4096_d128_fwdbwd"]["fwd"]
    assert rec["fetch_bytes"] == 1000 * 1024 * 2 and rec["write_bytes"] == 500 * 1024
    assert rec["mfma_busy"] == 0.5 and rec["waves_per_simd"] == 1.5 and rec["valu_per_mfma"] == 6.0
    assert rec["source_sha"] == "feedbeef"
    assert bench.load_counters("causal_b4_h16_n4096_d128_fwdbwd", "fwd")["mfma_busy"] == 0.5
    monkeypatch.setattr(bench, "source_sha", lambda name: "changed")
    assert bench.load_counters("causal_b4_h16_n4096_d128_fwdbwd", "fwd") is None
