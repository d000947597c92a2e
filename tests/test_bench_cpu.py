"""CPU: bench.py's host logic (workload names, FLOP model, multi-GPU refusal)."""
import argparse

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
