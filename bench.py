#!/usr/bin/env python3
"""Throughput of the exact-attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
the forward kernel (O, lse) and the three backward kernels (D = rowsum(dO*O),
dK/dV, dQ), all through the C ABI of libfa.so, inputs resident in HBM.

Default workload: causal attention, B=4, H=16, N=4096, d=128, bf16 inputs
drawn i.i.d. N(0,1) from seed 0, forward + backward -- the causal d=128
N>=4k case the headline figure (attention TFLOP/s, fwd and fwd+bwd, % of
the bf16 MFMA peak) is stated for. Other workloads: --workload, a named one
or any shape written KIND_bB_hH_nN_dD_PASS (e.g. causal_b2_h16_n8192_d128_fwdbwd).

FLOP model: forward 4*B*H*N^2*d, halved for causal; backward 2.5x forward.
Block-sparse counts kept 128x128 blocks only (a diagonal block counts 1/2
under causal).

Prints one JSON line. Besides the contract fields it carries
  roofline: the dominant kernel's algorithmic TFLOP/s (HIP events around
            each launch inside the timed steps) against the bf16 dense MFMA
            peak, and its HBM traffic from rocprofv3 counters when the
            committed counter summary matches the current kernel source;
  cpu_baseline: the fp64 CPU oracle timed on this host on a bounded sample
            (whole heads of the same workload), in the same unit.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention TFLOPs/s fwd and fwd+bwd (bf16, d=64/128, causal) and % MFMA peak"
# MI355X: 256 CUs x 2.4 GHz x 4096 bf16 flop/clk/CU (dense) = the published 2.5 PFLOP/s.
CUS, SCLK_GHZ, BF16_FLOP_PER_CLK_CU = 256, 2.4, 4096
PEAK_TFLOPS = CUS * SCLK_GHZ * BF16_FLOP_PER_CLK_CU / 1e3

WORKLOADS = {
    "causal_b4_h16_n4096_d128_fwdbwd": dict(B=4, H=16, N=4096, d=128, causal=True, sparse=False, bwd=True),
    "causal_b1_h16_n16384_d128_fwdbwd": dict(B=1, H=16, N=16384, d=128, causal=True, sparse=False, bwd=True),
    "causal_b8_h16_n2048_d64_fwd": dict(B=8, H=16, N=2048, d=64, causal=True, sparse=False, bwd=False),
    "dense_b8_h16_n2048_d64_fwd": dict(B=8, H=16, N=2048, d=64, causal=False, sparse=False, bwd=False),
    "blocksparse_b2_h16_n8192_d64_fwdbwd": dict(B=2, H=16, N=8192, d=64, causal=False, sparse=True, bwd=True),
    # dense counterpart of the block-sparse workload (comparison for its skipped work and traffic)
    "dense_b2_h16_n8192_d64_fwdbwd": dict(B=2, H=16, N=8192, d=64, causal=False, sparse=False, bwd=True),
    "dense_b1_h2_n256_d64_fwd": dict(B=1, H=2, N=256, d=64, causal=False, sparse=False, bwd=False),
}
DEFAULT = "causal_b4_h16_n4096_d128_fwdbwd"
WORKLOAD_RE = re.compile(r"^(dense|causal|blocksparse)_b(\d+)_h(\d+)_n(\d+)_d(64|128)_(fwd|fwdbwd)$")


def workload_config(name: str) -> dict:
    """Shape and flags of a workload: a named one above, or any name of the
    same form, KIND_bB_hH_nN_dD_PASS with KIND dense, causal or blocksparse
    and PASS fwd or fwdbwd (synthetic inputs of that shape)."""
    if name in WORKLOADS:
        return dict(WORKLOADS[name])
    m = WORKLOAD_RE.match(name)
    if not m:
        raise argparse.ArgumentTypeError(
            f"unknown workload {name!r}: one of {', '.join(sorted(WORKLOADS))}, or "
            "KIND_bB_hH_nN_dD_PASS (KIND dense|causal|blocksparse, D 64|128, PASS fwd|fwdbwd)")
    kind, B, H, N, d, pss = m.groups()
    if min(int(B), int(H), int(N)) < 1:
        raise argparse.ArgumentTypeError(f"workload {name!r}: B, H and N must be at least 1")
    return dict(B=int(B), H=int(H), N=int(N), d=int(d), causal=kind == "causal", sparse=kind == "blocksparse",
                bwd=pss == "fwdbwd")


def _workload_arg(name: str) -> str:
    workload_config(name)
    return name

KERNEL_SOURCES = {
    "fwd": "fa_fwd.hip", "bwd_pre": "fa_bwd.hip", "bwd_dkdv": "fa_bwd.hip", "bwd_dq": "fa_bwd.hip",
}


def fwd_flops(cfg, mask=None) -> float:
    import numpy as np

    B, H, N, d = cfg["B"], cfg["H"], cfg["N"], cfg["d"]
    if mask is not None:
        nb = mask.shape[1]
        kept = float(mask.astype(bool).sum())
        if cfg["causal"]:
            diag = float(mask[:, np.arange(nb), np.arange(nb)].astype(bool).sum())
            tri = float(np.tril(mask.astype(bool), -1).sum())
            kept = tri + 0.5 * diag
        return 4.0 * 128 * 128 * d * B * kept
    f = 4.0 * B * H * N * N * d
    return f / 2 if cfg["causal"] else f


def source_sha(name: str) -> str:
    path = os.path.join(ROOT, "exact_io_aware_69_amd", "csrc", name)
    h = hashlib.sha256()
    for p in sorted({path, os.path.join(ROOT, "exact_io_aware_69_amd", "csrc", "fa_device.h"),
                     os.path.join(ROOT, "exact_io_aware_69_amd", "csrc", "fa_params.h")}):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary,
    or None if there is none for this workload or the kernel source changed."""
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    rec = data.get(workload, {}).get(kernel)
    if not rec or rec.get("source_sha") != source_sha(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("bytes_per_launch")


def cpu_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(cfg, inp, budget_s: float = 12.0, max_s: float = 30.0):
    """Time the fp64 oracle on whole heads of the workload until ~budget_s."""
    import numpy as np

    import oracle

    B, H, N, d, causal = cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["causal"]
    scale = 1.0 / math.sqrt(d)
    mask = inp.get("mask")
    done, flops, performed, t_total = 0, 0.0, 0.0, 0.0
    heads = [(b, h) for b in range(B) for h in range(H)]
    for (b, h) in heads:
        Q, K, V = (oracle.widen_bf16(inp[n][b, h]) for n in ("q", "k", "v"))
        mh = None if mask is None else mask[h]
        sub = dict(cfg, B=1, H=1)
        f_fwd = fwd_flops(sub, None if mask is None else mask[h:h + 1])
        t0 = time.perf_counter()
        if cfg["bwd"]:
            dO = oracle.widen_bf16(inp["do"][b, h])
            oracle.head_backward(Q, K, V, dO, causal, scale, mh)
            f = 3.5 * f_fwd
            # products the oracle computes over all N x N entries: Q K^T and P V
            # in its forward, then Q K^T, P^T dO, dO V^T, dS K and dS^T Q
            fp = 14.0 * N * N * d
        else:
            for r0 in range(0, N, 1024):
                oracle.head_forward(Q, K, V, causal, scale, mh, rows=np.arange(r0, min(N, r0 + 1024)))
            f = f_fwd
            fp = 4.0 * N * N * d
        dt = time.perf_counter() - t0
        t_total += dt
        flops += f
        performed += fp
        done += 1
        if t_total >= budget_s or t_total + dt > max_s:
            break
    what = "forward+backward" if cfg["bwd"] else "forward"
    return {
        "value": flops / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": cpu_threads(),
        "kind": "oracle",
        "sample": f"fp64 numpy oracle, {what} of {done} whole head(s) (b, h) of this workload at full N={N}, "
                  f"{t_total:.1f} s; algorithmic FLOPs of the sample / wall time",
        # the same run on the FLOPs the oracle performs (it materialises every
        # score and skips nothing)
        "value_performed_flops": performed / t_total / 1e12,
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT, type=_workload_arg,
                    help="one of " + ", ".join(sorted(WORKLOADS)) + "; or any KIND_bB_hH_nN_dD_PASS "
                         "(KIND dense|causal|blocksparse, D 64|128, PASS fwd|fwdbwd)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--standard", action="store_true",
                    help="time the standard attention baseline (materialised S; fa_std_fwd) instead of the "
                         "IO-aware forward; forward only")
    ap.add_argument("--fa1", action="store_true",
                    help="time the FlashAttention-1-style forward (fa_fwd_fa1; ablation) instead of the "
                         "IO-aware forward; forward only, dense or causal")
    ap.add_argument("--dropout", type=float, default=0.0, metavar="P",
                    help="attention dropout probability (fa_fwd_dropout / fa_bwd_dropout; the backward is timed "
                         "as one call)")
    ap.add_argument("--fa1-seq-groups", type=int, default=1, metavar="G",
                    help="with --fa1: query-tile groups per head (1 = the published one workgroup per head)")
    ap.add_argument("--fwd-tiles", default=None, metavar="BM,BN",
                    help="run the forward through fa_fwd_tiles with this tile configuration (tile-size study)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM counters) and exit")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from exact_io_aware_69_amd import _lib
    from synth import make_inputs

    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": a.numel(), "copy_bytes_written": b.numel(), "launches": 3}))
        return 0

    _lib.lib()  # raises if libfa.so is missing: there is no other path
    cfg = workload_config(args.workload)
    if args.standard or args.fa1:
        cfg["bwd"] = False
    if args.fa1 and cfg["sparse"]:
        print("--fa1 runs dense or causal attention only", file=sys.stderr)
        return 2
    B, H, N, d, causal = cfg["B"], cfg["H"], cfg["N"], cfg["d"], cfg["causal"]
    scale = 1.0 / math.sqrt(d)
    inp = make_inputs(args.seed, B, H, N, d, with_do=cfg["bwd"], sparse=cfg["sparse"])

    def dev(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda:0")

    q, k, v = dev(inp["q"]), dev(inp["k"]), dev(inp["v"])
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda:0")
    mask = torch.from_numpy(inp["mask"]).to("cuda:0") if cfg["sparse"] else None
    mptr = mask.data_ptr() if mask is not None else None
    if cfg["bwd"]:
        do = dev(inp["do"])
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        st, ws_bytes = _lib.fa_bwd_workspace_size(B, H, N, d)
        _lib.check(st, "fa_bwd_workspace_size")
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda:0")
    stream = torch.cuda.current_stream()
    sptr = stream.cuda_stream
    tiles = tuple(int(x) for x in args.fwd_tiles.split(",")) if args.fwd_tiles else None
    fa1_ws = None
    if args.fa1:
        st, fa1_bytes = _lib.fa_fa1_workspace_size(B, H, N, d)
        _lib.check(st, "fa_fa1_workspace_size")
        fa1_ws = torch.empty(fa1_bytes, dtype=torch.uint8, device="cuda:0")
    std_ws = None
    if args.standard:
        st, std_bytes = _lib.fa_std_workspace_size(B, H, N, d)
        _lib.check(st, "fa_std_workspace_size")
        std_ws = torch.empty(std_bytes, dtype=torch.uint8, device="cuda:0")
    drop = args.dropout > 0
    if drop and (args.standard or args.fa1 or tiles is not None):
        print("--dropout runs the IO-aware kernels with the default tiles only", file=sys.stderr)
        return 2
    if drop:
        names = ["fwd"] + (["bwd"] if cfg["bwd"] else [])
    else:
        names = ["fwd"] + (["bwd_pre", "bwd_dkdv", "bwd_dq"] if cfg["bwd"] else [])

    def step(events=None):
        if events is not None:
            events[0].record(stream)
        if drop:
            st = _lib.fa_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                     B, H, N, d, causal, scale, mptr, args.dropout, args.seed, 0, sptr)
        elif fa1_ws is not None:
            st = _lib.fa_fwd_fa1(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                 B, H, N, d, causal, scale, args.fa1_seq_groups, fa1_ws.data_ptr(), fa1_ws.numel(),
                                 sptr)
        elif std_ws is not None:
            st = _lib.fa_std_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                 B, H, N, d, causal, scale, mptr, std_ws.data_ptr(), std_ws.numel(), sptr)
        elif tiles is not None:
            st = _lib.fa_fwd_tiles(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                   B, H, N, d, causal, scale, mptr, tiles[0], tiles[1], sptr)
        elif mptr is None:
            st = _lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                             B, H, N, d, causal, scale, sptr)
        else:
            st = _lib.fa_fwd_blocksparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                         B, H, N, d, causal, scale, mptr, sptr)
        _lib.check(st, "fa_fwd")
        if events is not None:
            events[1].record(stream)
        if cfg["bwd"] and drop:
            st = _lib.fa_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                     do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, causal,
                                     scale, mptr, args.dropout, args.seed, 0, ws.data_ptr(), ws_bytes, sptr)
            _lib.check(st, "fa_bwd_dropout")
            if events is not None:
                events[2].record(stream)
        elif cfg["bwd"]:
            for stage in range(3):
                st = _lib.fa_bwd_stage(stage, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                       B, H, N, d, causal, scale, mptr, ws.data_ptr(), ws_bytes, sptr)
                _lib.check(st, "fa_bwd_stage")
                if events is not None:
                    events[2 + stage].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    kern_ms = {n: sum(e[j].elapsed_time(e[j + 1]) for e in ev) / args.steps for j, n in enumerate(names)}

    f_fwd = fwd_flops(cfg, inp.get("mask"))
    f_step = f_fwd * (3.5 if cfg["bwd"] else 1.0)
    value = f_step / (ms_per_step * 1e-3) / 1e12
    # Algorithmic FLOPs attributed to each kernel: the forward's two GEMMs;
    # the dK/dV kernel's four of the backward's five GEMMs (S, dP, dV, dK);
    # the dQ kernel's dQ GEMM (its S and dP recomputation is not counted).
    kern_flops = {"fwd": f_fwd, "bwd_pre": 0.0, "bwd_dkdv": 2.0 * f_fwd, "bwd_dq": 0.5 * f_fwd, "bwd": 2.5 * f_fwd}
    dom = max(names, key=lambda n: kern_ms[n])
    achieved = kern_flops[dom] / (kern_ms[dom] * 1e-3) / 1e12
    roofline = {
        "kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": round(PEAK_TFLOPS, 1),
        "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4),
        # counters were taken for the default kernels only
        "traffic": None if (args.standard or args.fa1 or tiles or drop) else load_traffic(args.workload, dom),
        "avg_ms": round(kern_ms[dom], 4),
        "flops_per_launch": kern_flops[dom],
    }
    fwd_tf = f_fwd / (kern_ms["fwd"] * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": B, "H": H, "N": N, "d": d, "causal": causal,
                   "block_sparse": cfg["sparse"], "pass": "fwd+bwd" if cfg["bwd"] else "fwd",
                   "seed": args.seed, "parallelism": "single GPU",
                   "fwd_tiles": list(tiles) if tiles else [128, 64],
                   **({"fa1_seq_groups": args.fa1_seq_groups} if args.fa1 else {}),
                   **({"dropout_p": args.dropout} if drop else {}),
                   "impl": ("standard (materialised S)" if args.standard else
                            "flashattention-1-style (ablation)" if args.fa1 else "io-aware")},
        "frac_peak": round(value / PEAK_TFLOPS, 4),
        "fwd_tflops": round(fwd_tf, 2),
        "fwd_frac_peak": round(fwd_tf / PEAK_TFLOPS, 4),
        "kernel_ms": {n: round(x, 4) for n, x in kern_ms.items()},
        "flops_per_step": f_step,
        "peak_tflops": round(PEAK_TFLOPS, 1),
        "cus": torch.cuda.get_device_properties(0).multi_processor_count,
        "roofline": roofline,
    }
    if std_ws is not None:
        out["workspace_bytes"] = std_ws.numel()
    if fa1_ws is not None:
        out["workspace_bytes"] = fa1_ws.numel()
    if cfg["sparse"]:
        out["dense_equivalent_flops_per_step"] = fwd_flops(dict(cfg), None) * (3.5 if cfg["bwd"] else 1.0)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(cfg, inp)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
