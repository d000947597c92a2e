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
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published

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
    "fwd": "fa_fwd.hip", "bwd_sched": "fa_bwd.hip", "bwd_dq": "fa_bwd.hip", "bwd_dkdv": "fa_bwd.hip",
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


COUNTERS_JSON = os.path.join(ROOT, "profiles", "counters.json")
# Counter passes (one rocprofv3 --pmc run each; see --summarize-counters).
SQ_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS "
               "SQ_WAVES GRBM_GUI_ACTIVE")
SIMDS = 4 * CUS  # SIMDs of the chip
XCDS = 8


def load_counters(workload: str, kernel: str):
    """Counter record of `kernel` (HBM bytes per launch, MFMA busy, ...) from
    the committed summary, or None if there is none for this workload or the
    kernel's source changed since the counters were taken."""
    try:
        with open(COUNTERS_JSON) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    rec = data.get(workload, {}).get(kernel)
    if not rec or rec.get("source_sha") != source_sha(KERNEL_SOURCES[kernel]):
        return None
    return rec


def _kernel_role(name: str):
    if "fa_fwd_kernel" in name:
        return "fwd"
    if "fa_bwd_sched_kernel" in name:
        return "bwd_sched"
    if "fa_bwd_dkdv_kernel" in name:
        return "bwd_dkdv"
    if "fa_bwd_dq_kernel" in name:
        return "bwd_dq"
    return None


def _counter_means(run_dir: str, counters):
    """Mean value per dispatch of each counter, per kernel name, from the
    rocprofv3 database(s) under run_dir."""
    import collections
    import glob
    import sqlite3
    dbs = glob.glob(os.path.join(run_dir, "**", "*_results.db"), recursive=True)
    if len(dbs) != 1:
        raise SystemExit(f"{run_dir}: expected one rocprofv3 *_results.db, found {len(dbs)}")
    con = sqlite3.connect(dbs[0])
    out = collections.defaultdict(dict)
    for cname in counters:
        rows = con.execute("select dispatch_id, kernel_name, sum(value) from counters_collection where counter_name=? "
                           "group by dispatch_id, kernel_name", (cname,)).fetchall()
        acc = collections.defaultdict(list)
        for _, kn, v in rows:
            acc[re.sub(r"\(.*", "", kn).replace("void fa::", "")].append(v)
        for kn, vals in acc.items():
            out[kn][cname] = sum(vals) / len(vals)
    return out


def summarize_counters(run_root: str, workload: str) -> int:
    """Turn the counter runs of one workload into profiles/counters.json and
    profiles/counters_<workload>.txt. run_root holds one rocprofv3 output
    directory per pass, each made from the repository root with
    TMPDIR=/tmp:
      cal_fetch, cal_write: rocprofv3 --pmc FETCH_SIZE (WRITE_SIZE) -d RUN_ROOT/cal_fetch (cal_write)
                            -o run -- python3 bench.py --copy-calibration
      fetch, write:         rocprofv3 --pmc FETCH_SIZE (WRITE_SIZE) -d RUN_ROOT/fetch (write) -o run
                            -- python3 bench.py --workload W --steps 3 --warmup 1 --no-cpu-baseline
      sq:                   rocprofv3 --pmc <SQ_COUNTERS> -d RUN_ROOT/sq -o run -- python3 bench.py
                            --workload W --steps 3 --warmup 1 --no-cpu-baseline
    FETCH_SIZE and WRITE_SIZE are in KiB and are scaled by what they read for
    a plain 1 GiB device copy (bytes = KiB * 1024 * (2^30 / 1024) / copy's
    reading). MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (SIMDs * GRBM_GUI_ACTIVE
    / XCDs) (GRBM_GUI_ACTIVE sums the XCDs' clocks); resident waves per SIMD =
    4 * SQ_WAVE_CYCLES / (SIMDs * GRBM_GUI_ACTIVE / XCDs)."""
    cal = {}
    for c, sub in (("FETCH_SIZE", "cal_fetch"), ("WRITE_SIZE", "cal_write")):
        vals = _counter_means(os.path.join(run_root, sub), [c])
        cal[c] = max(v[c] for v in vals.values())  # the 1 GiB copy kernel
    ff, wf = (1 << 30) / 1024 / cal["FETCH_SIZE"], (1 << 30) / 1024 / cal["WRITE_SIZE"]
    fe = _counter_means(os.path.join(run_root, "fetch"), ["FETCH_SIZE"])
    wr = _counter_means(os.path.join(run_root, "write"), ["WRITE_SIZE"])
    sq = _counter_means(os.path.join(run_root, "sq"), SQ_COUNTERS.split())
    recs = {}
    for kn in sorted(set(fe) | set(sq)):
        role = _kernel_role(kn)
        if role is None:
            continue
        rec = {"kernel": kn, "source_sha": source_sha(KERNEL_SOURCES[role])}
        if kn in fe and kn in wr:
            fb, wb = fe[kn]["FETCH_SIZE"] * 1024 * ff, wr[kn]["WRITE_SIZE"] * 1024 * wf
            rec.update(fetch_kib_raw=fe[kn]["FETCH_SIZE"], write_kib_raw=wr[kn]["WRITE_SIZE"],
                       fetch_factor=round(ff, 4), write_factor=round(wf, 4), fetch_bytes=int(fb),
                       write_bytes=int(wb), bytes_per_launch=int(fb + wb))
        if kn in sq:
            v = sq[kn]
            g = v["GRBM_GUI_ACTIVE"] / XCDS
            mf = v["SQ_INSTS_MFMA"]
            rec.update(mfma_busy=round(v["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS * g), 4),
                       waves_per_simd=round(4 * v["SQ_WAVE_CYCLES"] / (SIMDS * g), 3),
                       valu_per_mfma=round(v["SQ_INSTS_VALU"] / mf, 3) if mf else None,
                       lds_per_mfma=round(v["SQ_INSTS_LDS"] / mf, 3) if mf else None,
                       gpu_cycles=round(g), raw_sq={k: v[k] for k in sorted(v)})
        recs[role] = rec
    try:
        with open(COUNTERS_JSON) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {}
    data[workload] = recs
    with open(COUNTERS_JSON, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    cmd = ("rocprofv3 --pmc {c} -d RUN_ROOT/{d} -o run -- python3 bench.py --workload " + workload +
           " --steps 3 --warmup 1 --no-cpu-baseline")
    lines = [f"# Counters per launch (mean of the warm-up and timed dispatches), workload {workload}",
             "# commands (one pass each, from the repository root, TMPDIR=/tmp):",
             "#   " + cmd.format(c="FETCH_SIZE", d="fetch"), "#   " + cmd.format(c="WRITE_SIZE", d="write"),
             "#   " + cmd.format(c=SQ_COUNTERS, d="sq"),
             "#   rocprofv3 --pmc FETCH_SIZE (WRITE_SIZE) -d RUN_ROOT/cal_fetch (cal_write) -o run -- "
             "python3 bench.py --copy-calibration",
             f"#   python3 bench.py --summarize-counters RUN_ROOT --workload {workload}",
             f"# copy calibration: FETCH_SIZE {cal['FETCH_SIZE']:.1f} KiB and WRITE_SIZE {cal['WRITE_SIZE']:.1f} KiB "
             f"for a 1 GiB copy -> factors {ff:.4f}, {wf:.4f}",
             "# MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs * GRBM_GUI_ACTIVE / 8)",
             f"{'kernel':10s} {'fetch_MiB':>10s} {'write_MiB':>10s} {'MFMA_busy':>10s} {'waves/SIMD':>11s} "
             f"{'VALU/MFMA':>10s} {'LDS/MFMA':>9s}"]
    for role in ("fwd", "bwd_sched", "bwd_dq", "bwd_dkdv"):
        r = recs.get(role)
        if not r:
            continue
        def fm(k, scale=1.0, fmt="{:10.1f}"):
            return fmt.format(r[k] / scale) if r.get(k) is not None else f"{'-':>10s}"
        lines.append(f"{role:10s} {fm('fetch_bytes', 2**20)} {fm('write_bytes', 2**20)} "
                     f"{fm('mfma_busy', 1, '{:10.3f}')} {fm('waves_per_simd', 1, '{:11.2f}')} "
                     f"{fm('valu_per_mfma', 1, '{:10.2f}')} {fm('lds_per_mfma', 1, '{:9.2f}')}")
    with open(os.path.join(ROOT, "profiles", f"counters_{workload}.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))
    return 0


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
    ap.add_argument("--atomic-rate", action="store_true",
                    help="only measure the fp32 atomic-add rate in the dQ accumulation layout and the time a "
                         "dQ-by-atomics backward of --workload would spend on its adds, then exit")
    ap.add_argument("--summarize-counters", metavar="RUN_ROOT", default=None,
                    help="turn the rocprofv3 counter runs under RUN_ROOT (for --workload) into "
                         "profiles/counters.json and profiles/counters_<workload>.txt, then exit (no GPU)")
    args = ap.parse_args(argv)

    if args.summarize_counters:
        return summarize_counters(args.summarize_counters, args.workload)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from exact_io_aware_69_amd import _lib
    from synth import make_inputs

    if args.atomic_rate:
        # fp32 atomic adds in the dQ accumulation layout (fa_atomic_add_probe),
        # against the adds a dQ-by-atomics backward of --workload would need:
        # one per (query row, head-dimension element) per visited dK/dV key tile.
        _lib.lib()
        cfg = workload_config(args.workload)
        dst = torch.zeros(4096 * 64 * 128, dtype=torch.float32, device="cuda:0")
        sptr = torch.cuda.current_stream().cuda_stream
        wgs, reps = 256 * 8, 64
        _lib.check(_lib.fa_atomic_add_probe(dst.data_ptr(), dst.numel(), wgs, 2, sptr), "fa_atomic_add_probe")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        _lib.check(_lib.fa_atomic_add_probe(dst.data_ptr(), dst.numel(), wgs, reps, sptr), "fa_atomic_add_probe")
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        rate = wgs * 256 * 16 * reps / (ms * 1e-3)
        st, _, bn = _lib.fa_tile_config(1, cfg["d"], cfg["causal"])
        _lib.check(st, "fa_tile_config")
        B, H, N, d = cfg["B"], cfg["H"], cfg["N"], cfg["d"]
        nk = -(-N // bn)
        if cfg["sparse"]:
            # each kept 128 x 128 mask block: 128 query rows per key tile of the block
            mask = make_inputs(args.seed, B, H, N, d, with_do=False, sparse=True)["mask"]
            adds = B * int(mask.astype(bool).sum()) * 128 * d * (128 // bn)
        else:
            rows = sum(N - t * bn for t in range(nk)) if cfg["causal"] else nk * N  # query rows per key tile
            adds = B * H * rows * d
        print(json.dumps({"atomic_add_rate_per_s": rate, "probe_ms": round(ms, 4), "workload": args.workload,
                          "dq_atomic_adds": adds, "dq_atomic_ms_at_this_rate": round(adds / rate * 1e3, 4),
                          "key_tile": bn}))
        return 0

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
        # Backward stages: 0 = block-sparse schedule (enqueues nothing without
        # a mask, so it is neither called nor timed then), 1 = dQ and the
        # per-row terms, 2 = dK/dV.
        bwd_stages = ([0] if mptr is not None else []) + [1, 2]
        names = ["fwd"] + ([("bwd_sched", "bwd_dq", "bwd_dkdv")[s] for s in bwd_stages] if cfg["bwd"] else [])

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
            for i, stage in enumerate(bwd_stages):
                st = _lib.fa_bwd_stage(stage, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                       B, H, N, d, causal, scale, mptr, ws.data_ptr(), ws_bytes, sptr)
                _lib.check(st, "fa_bwd_stage")
                if events is not None:
                    events[2 + i].record(stream)

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
    kern_flops = {"fwd": f_fwd, "bwd_sched": 0.0, "bwd_dkdv": 2.0 * f_fwd, "bwd_dq": 0.5 * f_fwd, "bwd": 2.5 * f_fwd}
    dom = max(names, key=lambda n: kern_ms[n])
    achieved = kern_flops[dom] / (kern_ms[dom] * 1e-3) / 1e12
    # Counter figures (HBM bytes, MFMA busy) come from the committed rocprofv3
    # summary of the same workload, valid while the kernel source is the one
    # they were taken on; the GB/s divide those bytes by this run's live
    # launch time. Counters exist for the default kernels only.
    default_kernels = not (args.standard or args.fa1 or tiles or drop)
    counters = {}
    for n in names:
        rec = load_counters(args.workload, n) if default_kernels and n in KERNEL_SOURCES else None
        if rec is None:
            continue
        c = {"mfma_busy": rec.get("mfma_busy"), "waves_per_simd": rec.get("waves_per_simd")}
        if rec.get("bytes_per_launch") is not None:
            gbps = rec["bytes_per_launch"] / (kern_ms[n] * 1e-3) / 1e9
            c.update(hbm_bytes=rec["bytes_per_launch"], hbm_gbps=round(gbps, 1),
                     hbm_frac=round(gbps / HBM_PEAK_GBPS, 4))
        counters[n] = c
    dc = counters.get(dom, {})
    roofline = {
        "kernel": dom, "bound": "mfma", "achieved": round(achieved, 2), "peak": round(PEAK_TFLOPS, 1),
        "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4),
        "traffic": dc.get("hbm_bytes"),
        "hbm_gbps": dc.get("hbm_gbps"), "hbm_frac": dc.get("hbm_frac"), "mfma_busy": dc.get("mfma_busy"),
        "counters_source": ("stored: profiles/counters.json (rocprofv3 --pmc on this kernel source); "
                            "hbm_gbps = those bytes / this run's launch time") if dc else None,
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
                   "fwd_tiles": list(tiles) if tiles else list(_lib.fa_tile_config(0, d, causal)[1:]),
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
        "counters": counters or None,
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
