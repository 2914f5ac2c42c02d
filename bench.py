#!/usr/bin/env python3
"""Benchmark of the draft-sampling / verification hot path on one MI355X.

One step = one speculative block over the workload's batch: by default the fused call
vt_spec_block (at batch 1: the LM head launch with the draft and target softmax partials, one
chunk pass that draws, accepts and sums the residual, one final draw; larger batches: LM head
with the draft partials, target partials, one combine launch, two verify launches); with
--calls the four separate calls
  vt_lmhead_trimmed -> vt_softmax_temp (draft, with draws) -> vt_softmax_temp (target) -> vt_spec_verify
on synthetic inputs already resident in HBM.  Default workload: the large drafter, B=256,
gamma=8, hidden 4096, 65536-row VocabTrim head of a 128256-id vocabulary, bf16 target logits,
T=0.8 (config 5 of the workload recipe, the largest that fits one GPU); afterwards the batch-1
VocabTrim block (B=1, gamma=5, hidden 3072, 32768 kept rows, config 3) is measured as a side
record, so that its whole-block HBM fraction is reported too.

Prints ONE JSON line on stdout (progress goes to stderr):
  value        verified draft positions / s = B * gamma / (seconds per step)
  roofline     the LM-head kernel (the dominant kernel), from its average duration measured live
               with HIP events on the launch stream: algorithmic flops per launch against the bf16
               MFMA peak (2.5 PFLOP/s) when the head is a dense contraction (256+ hidden rows),
               else algorithmic bytes per launch against 8 TB/s
  config       also the LM head's and the whole block's HBM GB/s and fraction of 8 TB/s, and in
               config.side the same for the side config
  cpu_baseline the float64 CPU oracle timed on a bounded sample of the same workload

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config C] [--greedy] [--no-cpu-baseline] [--calls] [--graph]
       python bench.py --copy-calibration   (a plain copy of known size, for PMC byte scaling)
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20
# the LM head's MFMA kernels (past the GEMV's 8 rows): with H % 32 == 0 all rows in one block up
# to ROWS_MAX_M rows (when W^Trim has fewer than 256 blocks of 256 rows: up to ROWS_MAX_M_NARROW
# rows in one block and up to 2 ROWS_MAX_M in two), then
# 256 x 256 or (fused call, when they give fewer rows per CU) 384 x 256 tiles; otherwise 128 x 128
# tiles below BIG_MIN_M rows and register-staged 256 x 256 tiles from there
ROWS_MAX_M, ROWS_MAX_M_NARROW = 192, 256
BIG_MIN_M = 129
CUS = 256


def gemv_head(M: int, H: int) -> bool:
    """Whether the LM head is the GEMV: at most 8 rows whose 512-column slices fit its registers."""
    nit = -(-H // 512)
    return M <= 8 and nit <= 8 and M * nit <= 48


def head_kernel(M: int, H: int, calls: bool, Vt: int) -> str:
    """Name of the LM-head kernel vt_spec_block (calls=False) or vt_lmhead_trimmed runs."""
    if gemv_head(M, H):
        return "lmhead_gemv"
    if H % 32 == 0:
        nbn = -(-Vt // 256)
        # one block of all rows, or on narrow heads up to two blocks of at most ROWS_MAX_M rows
        if M <= (ROWS_MAX_M_NARROW if nbn < CUS else ROWS_MAX_M) or (nbn < CUS and M <= 2 * ROWS_MAX_M):
            return "lmhead_mfma_rows"
        # 384- or 256-row tiles, whichever gives fewer rows per CU (one tile per CU at a time)
        tall = not calls and -(-(-(-M // 384) * nbn) // CUS) * 384 <= -(-(-(-M // 256) * nbn) // CUS) * 256
        return "lmhead_mfma_tall" if tall else "lmhead_mfma_dma8"
    return "lmhead_mfma_big" if M >= BIG_MIN_M else "lmhead_mfma"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--side-config", type=int, default=3, choices=[0, 2, 3, 4, 5],
                    help="a second config measured after the main one, reported in config.side (0: none); "
                         "by default the batch-1 VocabTrim block, whose whole-block HBM fraction is tracked")
    ap.add_argument("--side-steps", type=int, default=200)
    ap.add_argument("--batch", type=int, default=1,
                    help="sequences per step for the toy (--config 1); the other configs fix their batch")
    ap.add_argument("--sequences", type=int, default=None,
                    help="sequences per step for --config 2-5 in place of the config's own batch (the same "
                         "recipe at another batch size, e.g. the medium batches of a serving loop); the "
                         "configs' own batches are the reference workloads")
    ap.add_argument("--workload", default="block", choices=["block", "keepset", "generate"],
                    help="block: one speculative block per step (the default); keepset: token counter -> "
                         "Top-K -> trimmed head over a Zipf calibration stream; generate: the chained "
                         "generation loop on the order-1 toy")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--valu-record", metavar="CSV",
                    help="SQ_INSTS_VALU counter csv of --workload generate: write the generation kernel's record")
    ap.add_argument("--traffic-record", nargs=4, metavar="CSV",
                    help="bench FETCH_SIZE, bench WRITE_SIZE, copy FETCH_SIZE, copy WRITE_SIZE counter csv "
                         "files from rocprofv3 --pmc: write the LM-head traffic record for --config")
    ap.add_argument("--calls", action="store_true",
                    help="run the step as the four separate calls instead of the fused vt_spec_block")
    ap.add_argument("--overlap", action="store_true",
                    help="run the target softmax on a second stream, concurrently with the LM head")
    ap.add_argument("--follow", type=float, default=0.0, metavar="SIGMA",
                    help="a drafter that follows the target (target = the head's own two columns + N(0, SIGMA)): "
                         "drafts get accepted; the default is the recipe's unrelated random head")
    ap.add_argument("--keep-order", default="id", choices=["id", "rank"],
                    help="storage order of the kept ids: ascending id (the default) or rank order, best first")
    ap.add_argument("--greedy", action="store_true",
                    help="temperature 0 for target and draft: argmax drafts and greedy verification")
    ap.add_argument("--graph", action="store_true",
                    help="replay captured HIP graphs instead of launching eagerly: with --calls the LM head | "
                         "the rest; for the toy (--config 1) the whole step")
    ap.add_argument("--head", default="tiled", choices=["tiled", "gather"],
                    help="what the fused call's large-batch head reads: the K-tiled W^Trim built once per keep "
                         "set by vt_trim_head_tiled (the default), or rows of the full head gathered through "
                         "keep_ids")
    return ap.parse_args()


class DeviceEvent:
    """A HIP timing event created with hipEventDisableSystemFence: recording it takes the
    timestamp once the work before it on the stream has completed (stream order is unchanged) but
    performs no memory fence.  Default events fence at system scope (an L2 write-back and
    invalidate that stalls the next kernel); measured on the fused batch-1 block with two events
    around the LM head: +5.3 us per step with default events, +4.9 with device-scope release
    (the head's fresh logits are written back), +1.5 with no fence.  Timing device work needs no
    host visibility of memory.  Same interface as the torch events this script uses:
    .cuda_event (the raw handle the binding passes on), record(stream), elapsed_time(end) in ms."""

    _hip = None
    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        import ctypes
        if DeviceEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            DeviceEvent._hip = hip
        h = ctypes.c_void_p()
        st = DeviceEvent._hip.hipEventCreateWithFlags(ctypes.byref(h), DeviceEvent.FLAGS)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")
        self.cuda_event = h.value

    def record(self, stream=None):
        import torch
        s = stream if stream is not None else torch.cuda.current_stream()
        st = DeviceEvent._hip.hipEventRecord(self.cuda_event, s.cuda_stream)
        if st != 0:
            raise RuntimeError(f"hipEventRecord failed ({st})")

    def elapsed_time(self, end) -> float:
        import ctypes
        ms = ctypes.c_float()
        st = DeviceEvent._hip.hipEventElapsedTime(ctypes.byref(ms), self.cuda_event, end.cuda_event)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value


def lmhead_bytes(cfg) -> int:
    """Algorithmic HBM bytes of one LM-head launch: kept weight rows + hidden + logits (+ keep_ids)."""
    M = cfg.B * cfg.R
    b = cfg.Vt * cfg.H * 2 + M * cfg.H * 2 + M * cfg.Vt * 4
    if cfg.trimmed:
        b += cfg.Vt * 4
    return b


def small_batch_block(cfg, greedy: bool = False) -> bool:
    """Batch-1-sized blocks (at most 8 draft rows, both sides sampled): the GEMV head launch also
    runs the target rows' first softmax pass in extra workgroups."""
    return gemv_head(cfg.B * cfg.R, cfg.H) and cfg.R <= 8 and not greedy


def lmhead_launch_bytes(cfg, greedy: bool = False, calls: bool = False) -> int:
    """Algorithmic bytes of the timed head launch: the LM head's, plus the target logits when the
    fused call's GEMV launch also takes the target partials."""
    b = lmhead_bytes(cfg)
    if small_batch_block(cfg, greedy) and not calls:
        b += cfg.B * (cfg.gamma + 1) * cfg.V * (4 if cfg.target_dtype == "f32" else 2)
    return b


def lmhead_flops(cfg) -> float:
    return 2.0 * cfg.B * cfg.R * cfg.H * cfg.Vt


def block_bytes(cfg, greedy: bool = False) -> int:
    """Algorithmic bytes of the whole block (each kernel's distinct inputs and outputs once)."""
    M, B, g, V, Vt = cfg.B * cfg.R, cfg.B, cfg.gamma, cfg.V, cfg.Vt
    s_t = 4 if cfg.target_dtype == "f32" else 2
    lm = lmhead_bytes(cfg)
    if greedy:  # argmax of the draft rows, argmax of every target row, outputs
        return lm + M * Vt * 4 + M * 12 + B * (g + 1) * V * s_t + B * ((g + 2) * 4 + g * 4)
    draft_sm = M * Vt * 4 + M * (8 + 4 + 4)  # read logits; write lse, ids; read u
    target_sm = B * (g + 1) * V * s_t + B * (g + 1) * 8
    verify = B * (V * s_t + Vt * 4 + (V * 4 if cfg.trimmed else 0) + (g + 2) * 4 + g * 4 + 4)
    return lm + draft_sm + target_sm + verify


LMHEAD_SOURCES = ("lmhead_impl.hpp", "softmax_impl.hpp", "vt_common.hpp", "block.hip")


def kernel_source_hash() -> str:
    """Hash of every source the timed LM-head kernel is compiled from (a traffic record taken on
    other code does not describe this one)."""
    h = hashlib.sha256()
    for name in LMHEAD_SOURCES:
        with open(os.path.join(ROOT, "draft_sampling_verification_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def measured_traffic(workload_key: str):
    """HBM bytes per LM-head launch from a committed PMC measurement, if taken on this source."""
    path = os.path.join(ROOT, "profiles", f"lmhead_traffic_{workload_key}.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("lmhead_source_sha256") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def _pmc_rows(csv_path, counter):
    import csv
    with open(csv_path, newline="") as f:
        return [(r["Kernel_Name"], float(r["Counter_Value"])) for r in csv.DictReader(f)
                if r["Counter_Name"] == counter]


def write_traffic_record(config: int, fetch_csv, write_csv, copy_fetch_csv, copy_write_csv) -> str:
    """Turn two `rocprofv3 --pmc` passes over this bench (FETCH_SIZE, then WRITE_SIZE) and the same
    two over --copy-calibration into profiles/lmhead_traffic_config<C>.json: HBM bytes per launch of
    the LM-head kernel the timed loop runs (the most frequent lmhead_* kernel), each counter scaled
    by what it reads for a copy of known size."""
    from collections import Counter

    from workloads import CONFIGS

    def lm_avg(path, counter):
        rows = [(k, v) for k, v in _pmc_rows(path, counter) if "lmhead_" in k]
        name = Counter(k for k, _ in rows).most_common(1)[0][0]
        vals = [v for k, v in rows if k == name]
        return name, sum(vals) / len(vals), len(vals)

    def copy_avg(path, counter):
        vals = [v for k, v in _pmc_rows(path, counter) if "AUnaryFunctor" in k]
        return sum(vals) / len(vals)

    cfg = CONFIGS[config]
    kname, fetch_kib, nf = lm_avg(fetch_csv, "FETCH_SIZE")
    kname_w, write_kib, nw = lm_avg(write_csv, "WRITE_SIZE")
    assert kname == kname_w, (kname, kname_w)
    n = 1 << 30
    cf, cw = copy_avg(copy_fetch_csv, "FETCH_SIZE"), copy_avg(copy_write_csv, "WRITE_SIZE")
    fs, wsc = n / (cf * 1024), n / (cw * 1024)
    M = cfg.B * cfg.R
    alg_w = M * cfg.Vt * 4
    rec = {
        "kernel": kname.replace("void vt::(anonymous namespace)::", "").strip('"')[:160],
        "workload": cfg.name,
        "lmhead_source_sha256": kernel_source_hash(),
        "fetch_size_kib_per_launch_raw": fetch_kib, "write_size_kib_per_launch_raw": write_kib,
        "launches_sampled": [nf, nw],
        "copy_calibration": {"bytes_read_per_launch": n, "bytes_written_per_launch": n,
                             "fetch_size_kib_raw": cf, "write_size_kib_raw": cw,
                             "fetch_scale": fs, "write_scale": wsc},
        "hbm_fetch_bytes_per_launch": round(fetch_kib * 1024 * fs),
        "hbm_write_bytes_per_launch": round(write_kib * 1024 * wsc),
        "algorithmic_read_bytes": lmhead_launch_bytes(cfg) - alg_w, "algorithmic_write_bytes": alg_w,
        "commands": [
            f"rocprofv3 --pmc FETCH_SIZE -f csv -d <out> -o bench -- python3 bench.py --config {config} "
            "--side-config 0 --no-cpu-baseline --steps 10 --warmup 3",
            f"rocprofv3 --pmc WRITE_SIZE -f csv -d <out> -o bench -- python3 bench.py --config {config} "
            "--side-config 0 --no-cpu-baseline --steps 10 --warmup 3",
            "rocprofv3 --pmc FETCH_SIZE -f csv -d <out> -o copy -- python3 bench.py --copy-calibration",
            "rocprofv3 --pmc WRITE_SIZE -f csv -d <out> -o copy -- python3 bench.py --copy-calibration",
            f"python3 bench.py --config {config} --traffic-record <4 csv files>"],
    }
    rec["hbm_bytes_per_launch"] = rec["hbm_fetch_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]
    rec["traffic_over_algorithmic"] = round(rec["hbm_bytes_per_launch"] / lmhead_launch_bytes(cfg), 4)
    out = os.path.join(ROOT, "profiles", f"lmhead_traffic_config{config}.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return out


def copy_calibration():
    """A plain elementwise copy of 1 GiB (reads 1 GiB, writes 1 GiB per launch), 5 launches."""
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    log(f"copy calibration: 5 launches, each reads {n} and writes {n} bytes")
    print(json.dumps({"copy_bytes": n, "launches": 5}))


def cpu_baseline(cfg, wl_one, budget_s: float):
    """Time the oracle as it stands on whole blocks of the same workload until ~budget_s."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import ref

    threadpool_limits(limits=len(os.sched_getaffinity(0)))
    used = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    blocks, t0 = 0, time.perf_counter()
    while True:
        ref.block(wl_one.hidden, wl_one.weight, wl_one.keep_ids, None, wl_one.target, cfg.target_dtype,
                  wl_one.T, wl_one.u_draft, wl_one.u_acc, wl_one.u_fin, cfg.gamma, cfg.R)
        blocks += 1
        el = time.perf_counter() - t0
        if el >= budget_s or blocks >= 50:
            break
    per_block = el / blocks
    return {"value": wl_one.B * cfg.gamma / per_block, "unit": "verified draft positions/s",
            "cores": int(used), "kind": "oracle",
            "sample": f"{blocks} whole block(s) of {wl_one.B} sequence(s) of this workload, float64 numpy, "
                      f"{el:.1f} s total, {per_block:.2f} s per block"}


# ---------------------------------------------------------------- config 1: the order-1 toy

def bench_toy(args):
    """One step = one speculative block of the order-1 toy (V = 18, gamma = 4) for --batch
    sequences, through the separate calls: gamma draft rows looked up from the draft table by the
    previous token (the toy's "model", a torch gather) and drawn with vt_softmax_temp, the gamma+1
    target rows looked up the same way, vt_softmax_temp for their log-normalisers, vt_spec_verify.
    At batch 1 this is launch latency; the verify kernel is timed with HIP events for the
    roofline line."""
    import torch

    import draft_sampling_verification_amd as vt
    from workloads import CONFIGS, make_workload

    cfg = CONFIGS[1]
    B, g, V = args.batch, cfg.gamma, cfg.V
    wl = make_workload(cfg, B=B)

    def f(x):
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    Q, P = f(wl.toy.draft_logits), f(wl.toy.target_logits)
    ud_cols = [f(wl.u_draft[:, k]) for k in range(g)]
    ua, uf = f(wl.u_acc), f(wl.u_fin)
    lse_k = [torch.empty(B, dtype=torch.float64, device="cuda") for _ in range(g)]
    ids_k = [torch.empty(B, dtype=torch.int32, device="cuda") for _ in range(g)]
    tlse = torch.empty(B * (g + 1), dtype=torch.float64, device="cuda")
    tok = torch.empty(B, g + 1, dtype=torch.int32, device="cuda")
    nacc = torch.empty(B, dtype=torch.int32, device="cuda")
    ctx0 = torch.zeros(B, dtype=torch.long, device="cuda")
    ws_d = vt.softmax_workspace(B, V)
    ws_t = vt.softmax_workspace(B * (g + 1), V)
    ws_v = vt.verify_workspace(B, g, V)
    main_s = torch.cuda.current_stream()
    ev_a = [DeviceEvent() for _ in range(args.steps)]
    ev_b = [DeviceEvent() for _ in range(args.steps)]

    def step(i=None):
        ctx = ctx0
        rows, tcols = [], [P[ctx]]
        for k in range(g):
            r = Q[ctx]
            vt.vt_softmax_temp(r, wl.T, lse_k[k], None, ud_cols[k], ids_k[k], workspace=ws_d)
            rows.append(r)
            ctx = ids_k[k].long() + 1
            tcols.append(P[ctx])
        target = torch.stack(tcols, 1)
        vt.vt_softmax_temp(target.view(-1, V), wl.T, tlse, workspace=ws_t)
        draft, dl, di = torch.stack(rows, 1), torch.stack(lse_k, 1), torch.stack(ids_k, 1)
        if i is not None:
            ev_a[i].record(main_s)
        vt.vt_spec_verify(target, tlse, wl.T, draft, dl, wl.T, di, None, None, ua, uf, tok, nacc, workspace=ws_v)
        if i is not None:
            ev_b[i].record(main_s)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    if args.graph:
        # the verify kernel timed on eager steps; the step itself as replays of one captured graph
        # (the toy's inner loop is launch-bound: ~20 small launches per step)
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(main_s)
        with torch.cuda.stream(side):
            step()
        main_s.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        step()
        torch.cuda.synchronize()
        want = (tok.clone(), nacc.clone())
        for _ in range(3):
            tok.fill_(-3)
            nacc.fill_(-3)
            graph.replay()
            torch.cuda.synchronize()
            if not (torch.equal(tok, want[0]) and torch.equal(nacc, want[1])):
                raise SystemExit("toy graph replay differs from the eager step")
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
    else:
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(i)
        torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = 1e3 * wall / args.steps
    v_ms = sum(a.elapsed_time(b) for a, b in zip(ev_a, ev_b)) / args.steps
    # verify kernel: target rows + draft rows + lse + ids + uniforms in, tokens + n out
    vb = B * ((g + 1) * V * 4 + g * V * 4 + (g + 1) * 8 + g * 8 + g * 4 + (g + 1) * 4 + (g + 2) * 4)
    log(f"step {ms:.4f} ms ({1e3 * ms:.1f} us), verify call {v_ms * 1e3:.1f} us; "
        f"mean accepted {float(nacc.double().mean()):.3f}")
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import ref
        one = make_workload(cfg, B=min(B, 1000))
        n, t1 = 0, time.perf_counter()
        while time.perf_counter() - t1 < min(args.cpu_seconds, 5.0):
            ref.toy_block(one.toy.target_logits, one.toy.draft_logits, one.T, g, one.u_draft, one.u_acc, one.u_fin)
            n += 1
        el = time.perf_counter() - t1
        cpu = {"value": one.B * g * n / el, "unit": "verified draft positions/s", "cores": 1, "kind": "oracle",
               "sample": f"{n} toy block(s) of {one.B} sequence(s), float64 numpy, {el:.1f} s"}
    out = {
        "metric": "verified draft positions/sec (order-1 toy, launch-latency bound at batch 1), 1 GPU",
        "value": round(B * g / (ms / 1e3), 1),
        "unit": "verified draft positions/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"{cfg.name}; batch {B}", "batch": B, "gamma": g, "vocab": V,
                   "launch": "gamma draft draws + target softmax + verify, separate calls (toy rows gathered by torch)"
                             + ("; the step replayed as one captured HIP graph" if args.graph else ""),
                   "us_per_step": round(1e3 * ms, 2),
                   "mean_accepted": round(float(nacc.double().mean()), 4)},
        "roofline": {"bound": "hbm", "achieved": round(vb / (v_ms / 1e3) / 1e9, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(vb / (v_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 5), "traffic": None,
                     "kernel": "verify_single (vt_spec_verify)", "algorithmic_bytes_per_launch": vb,
                     "avg_launch_ms": round(v_ms, 5)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------- keep-set construction

KS_TOKENS, KS_V, KS_K, KS_H = 1 << 26, 128256, 32768, 3072


def bench_keepset(args):
    """One step = vt_token_histogram over a 64M-token Zipf(1.1) stream (V = 128256) ->
    vt_keep_select Top-K 32768 -> vt_trim_head of the 3072-wide bf16 head.  Each launch is
    bracketed by HIP events on the stream it runs on."""
    import torch

    import draft_sampling_verification_amd as vt
    from workloads import token_stream
    from workloads.gen import lm_head_weights

    t0 = time.perf_counter()
    toks_h = token_stream(KS_V, KS_TOKENS, seed=1)
    W_h = lm_head_weights(KS_V, KS_H)
    log(f"keep-set inputs generated in {time.perf_counter() - t0:.1f} s")
    toks = torch.from_numpy(toks_h).cuda()
    W = torch.from_numpy(W_h.view(np.int16)).cuda().view(torch.bfloat16)
    counts = torch.empty(KS_V, dtype=torch.int32, device="cuda")
    keep = torch.empty(KS_V, dtype=torch.int32, device="cuda")
    f2t = torch.empty(KS_V, dtype=torch.int32, device="cuda")
    nk = torch.empty(1, dtype=torch.int32, device="cuda")
    trimmed = torch.empty(KS_K, KS_H, dtype=torch.bfloat16, device="cuda")
    ws = vt.histogram_workspace(KS_TOKENS, KS_V)
    keep_k = keep[:KS_K]
    main = torch.cuda.current_stream()
    ev = [[DeviceEvent() for _ in range(4)] for _ in range(args.steps)]

    def step(e=None):
        if e: e[0].record(main)
        vt.vt_token_histogram(toks, KS_V, counts, workspace=ws)
        if e: e[1].record(main)
        vt.vt_keep_select(counts, vt.VT_SELECT_TOP_K, keep, f2t, nk, k=KS_K)
        if e: e[2].record(main)
        vt.vt_trim_head(W, keep_k, trimmed)
        if e: e[3].record(main)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = 1e3 * wall / args.steps
    hist_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps
    sel_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps
    trim_ms = sum(e[2].elapsed_time(e[3]) for e in ev) / args.steps
    hist_bytes = KS_TOKENS * 4 + KS_V * 4
    trim_bytes = 2 * KS_K * KS_H * 2 + KS_K * 4
    kern = {"vt_token_histogram": (hist_ms, hist_bytes), "vt_trim_head": (trim_ms, trim_bytes)}
    dom = max(kern, key=lambda k: kern[k][0])
    d_ms, d_bytes = kern[dom]
    ach = d_bytes / (d_ms / 1e3) / 1e9
    log(f"step {ms:.4f} ms: histogram {hist_ms:.4f} ms ({hist_bytes / hist_ms / 1e6:.0f} GB/s), select "
        f"{sel_ms:.4f} ms, trim {trim_ms:.4f} ms ({trim_bytes / trim_ms / 1e6:.0f} GB/s)")
    cpu = None
    if not args.no_cpu_baseline:
        from threadpoolctl import threadpool_info, threadpool_limits

        from oracle import keepset
        threadpool_limits(limits=len(os.sched_getaffinity(0)))
        used = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
        sample = toks_h[: 1 << 24]
        runs, t0 = 0, time.perf_counter()
        while True:
            c = keepset.count_tokens(sample, KS_V)
            kp, _ = keepset.top_k(c, KS_K)
            keepset.trim_head(W_h, kp)
            runs += 1
            el = time.perf_counter() - t0
            if el >= args.cpu_seconds or runs >= 50:
                break
        cpu = {"value": round(runs * len(sample) / el, 1), "unit": "calibration tokens/s", "cores": int(used),
               "kind": "oracle",
               "sample": f"{runs} pass(es) of count + Top-K + head slice over the first {len(sample)} tokens "
                         f"of the same stream, {el:.1f} s"}
    out = {
        "metric": "calibration tokens/s through token counting, Top-K selection and head trimming, 1 GPU",
        "value": round(KS_TOKENS / (ms / 1e3), 1), "unit": "calibration tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "u32", "data": "synthetic",
        "config": {"workload": f"keep-set construction: {KS_TOKENS} Zipf(1.1) tokens, V={KS_V}, Top-K {KS_K}, "
                               f"head {KS_V}x{KS_H} bf16",
                   "kernel_ms": {"histogram": round(hist_ms, 5), "select": round(sel_ms, 5),
                                 "trim_head": round(trim_ms, 5)}},
        "roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None, "kernel": dom,
                     "algorithmic_bytes_per_launch": d_bytes, "avg_launch_ms": round(d_ms, 5)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------- generation loop

GEN_B, GEN_L, GEN_GAMMA, GEN_W = 16384, 256, 4, 0.5
VALU_PEAK_LANE_OPS = 256 * 2.4e9 * 64 / 1e12  # T lane-ops/s: one wave64 VALU instruction per CU per clock


def bench_generate(args):
    """One step = vt_spec_generate_markov: 16384 sequences x 256 tokens of the order-1 toy
    (V = 18, gamma = 4, draft = 0.5 target + 0.5 unigram)."""
    import torch

    import draft_sampling_verification_amd as vt
    from workloads import CONFIGS, counter_uniforms, toy_tables

    t = toy_tables(CONFIGS[1], GEN_W)
    g, B, L = GEN_GAMMA, GEN_B, GEN_L
    u_h = counter_uniforms(1, 70, B, L * (2 * g + 1)).reshape(B, L, 2 * g + 1)
    tt = torch.from_numpy(t.target_logits).cuda()
    dt = torch.from_numpy(t.draft_logits).cuda()
    u = torch.from_numpy(u_h).cuda()
    tok = torch.empty(B, L, dtype=torch.int32, device="cuda")
    st = torch.empty(B, 4, dtype=torch.int32, device="cuda")
    main = torch.cuda.current_stream()
    ev = [(DeviceEvent(), DeviceEvent()) for _ in range(args.steps)]
    for _ in range(args.warmup):
        vt.vt_spec_generate_markov(tt, dt, 1.0, 1.0, g, u, tok, st)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        ev[i][0].record(main)
        vt.vt_spec_generate_markov(tt, dt, 1.0, 1.0, g, u, tok, st)
        ev[i][1].record(main)
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / args.steps
    k_ms = sum(a.elapsed_time(b) for a, b in ev) / args.steps
    s = st.cpu().numpy().astype(np.int64)
    a_hat = s[:, 2].sum() / s[:, 1].sum()
    tau = s[:, 3].sum() / s[:, 0].sum()
    log(f"step {ms:.4f} ms, kernel {k_ms:.4f} ms; measured acceptance {a_hat:.5f}, tokens/block {tau:.4f}")
    rec = valu_record()
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import ref
        n_seq, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < args.cpu_seconds and n_seq < B:
            ref.toy_generate(t.target_logits, t.draft_logits, 1.0, 1.0, g, L, u_h[n_seq:n_seq + 8])
            n_seq += 8
        el = time.perf_counter() - t0
        cpu = {"value": round(n_seq * L / el, 1), "unit": "generated tokens/s", "cores": 1, "kind": "oracle",
               "sample": f"the first {n_seq} sequences of the same workload ({n_seq * L} tokens), {el:.1f} s"}
    roof = {"bound": "alu", "achieved": None, "peak": VALU_PEAK_LANE_OPS, "unit": "T lane-ops/s", "frac": None,
            "traffic": None, "kernel": "markov_generate", "avg_launch_ms": round(k_ms, 5)}
    if rec is not None:
        lane_ops = rec["valu_insts_per_launch"] * 64
        roof["achieved"] = round(lane_ops / (k_ms / 1e3) / 1e12, 3)
        roof["frac"] = round(roof["achieved"] / VALU_PEAK_LANE_OPS, 4)
        roof["valu_insts_per_launch"] = rec["valu_insts_per_launch"]
    out = {
        "metric": "generated tokens/s, chained speculative blocks on the order-1 toy, 1 GPU",
        "value": round(B * L / (ms / 1e3), 1), "unit": "generated tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": f"toy generation loop: B={B} sequences x {L} tokens, V=18, gamma={g}, w={GEN_W}",
                   "measured_acceptance": round(float(a_hat), 5), "tokens_per_block": round(float(tau), 5)},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def generate_source_hash() -> str:
    h = hashlib.sha256()
    for name in ("generate.hip", "verify_impl.hpp", "vt_common.hpp"):
        with open(os.path.join(ROOT, "draft_sampling_verification_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def write_valu_record(csv_path) -> str:
    """profiles/generate_valu_toy.json from a `rocprofv3 --pmc SQ_INSTS_VALU` pass over
    `bench.py --workload generate`: VALU instructions (per wavefront, summed over the device)
    per launch of the generation kernel."""
    vals = [v for k, v in _pmc_rows(csv_path, "SQ_INSTS_VALU") if "markov_generate" in k]
    rec = {"kernel": "markov_generate", "workload": f"toy generation loop B={GEN_B} L={GEN_L} gamma={GEN_GAMMA}",
           "source_sha256": generate_source_hash(), "launches_sampled": len(vals),
           "valu_insts_per_launch": sum(vals) / len(vals),
           "commands": ["rocprofv3 --pmc SQ_INSTS_VALU -f csv -d <out> -o gen -- python3 bench.py --workload generate "
                        "--no-cpu-baseline --steps 10 --warmup 2",
                        "python3 bench.py --valu-record <counter csv>"]}
    out = os.path.join(ROOT, "profiles", "generate_valu_toy.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return out


def valu_record():
    """VALU instructions per launch of the generation kernel from a committed PMC record."""
    path = os.path.join(ROOT, "profiles", "generate_valu_toy.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    return rec if rec.get("source_sha256") == generate_source_hash() else None


def bench_block(args, config: int, steps: int, warmup: int, sequences: int | None = None):
    """Time `steps` speculative blocks of a config after `warmup` untimed ones.  Returns the fields
    of the result line: step time, the LM-head launch time from HIP events on its own stream, the
    algorithmic bytes and flops, and the side statistics."""
    import torch

    import draft_sampling_verification_amd as vt
    from workloads import CONFIGS, make_workload

    cfg = CONFIGS[config]
    if sequences:
        cfg = dataclasses.replace(cfg.scaled(B=sequences), name=re.sub(r"B=\d+", f"B={sequences}", cfg.name))
    B, g, R = cfg.B, cfg.gamma, cfg.R
    log(f"workload: {cfg.name}")
    t0 = time.perf_counter()
    wl = make_workload(cfg, follow=args.follow, keep_order=args.keep_order)
    log(f"inputs generated in {time.perf_counter() - t0:.1f} s")

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    def f(x):
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()

    # enough copies of the inputs that the 256 MB MALL cannot serve a step from cache
    bb = block_bytes(cfg, args.greedy)
    n_sets = max(2, math.ceil(3 * MALL_BYTES / bb))
    base = dict(weight=bf16(wl.weight), hidden=bf16(wl.hidden),
                target=f(wl.target) if cfg.target_dtype == "f32" else bf16(wl.target),
                u_draft=f(wl.u_draft.reshape(-1)), u_acc=f(wl.u_acc), u_fin=f(wl.u_fin))
    sets = [base] + [{k: v.clone() for k, v in base.items()} for _ in range(n_sets - 1)]
    keep = f(wl.keep_ids) if wl.keep_ids is not None else None
    f2t = f(wl.full_to_trim) if wl.full_to_trim is not None else None
    M = B * R
    logits = torch.empty(M, cfg.Vt, dtype=torch.float32, device="cuda")
    dlse = torch.empty(M, dtype=torch.float64, device="cuda")
    dids = torch.empty(M, dtype=torch.int32, device="cuda")
    tlse = torch.empty(B * (g + 1), dtype=torch.float64, device="cuda")
    tokens = torch.empty(B, g + 1, dtype=torch.int32, device="cuda")
    nacc = torch.empty(B, dtype=torch.int32, device="cuda")
    ws_sm_d = vt.softmax_workspace(M, cfg.Vt)
    ws_sm_t = vt.softmax_workspace(B * (g + 1), cfg.V)
    ws_vf = vt.verify_workspace(B, g, cfg.V)
    log(f"{n_sets} input sets on device ({bb / 1e6:.1f} MB algorithmic per step)")

    main = torch.cuda.current_stream()

    side = torch.cuda.Stream() if args.overlap else None  # default priority
    ev_tgt, ev_free = torch.cuda.Event(), torch.cuda.Event()
    ev_free.record(main)

    T = 0.0 if args.greedy else float(wl.T)

    def target_lse(s):
        if not args.greedy:  # greedy verification reads no log-normalisers
            vt.vt_softmax_temp(s["target"].view(B * (g + 1), cfg.V), T, tlse, workspace=ws_sm_t)

    def lmhead(s):
        if side is not None:
            # the target's log-normalisers do not depend on the draft: overlap them with the head
            side.wait_event(ev_free)  # the previous step's verify is done with tlse
            with torch.cuda.stream(side):
                target_lse(s)
                ev_tgt.record(side)
        vt.vt_lmhead_trimmed(s["hidden"], s["weight"], keep, logits)

    def rest(s):
        vt.vt_softmax_temp(logits, T, dlse, None, None if args.greedy else s["u_draft"], dids, workspace=ws_sm_d)
        if side is None:
            target_lse(s)
        else:
            main.wait_event(ev_tgt)
        vt.vt_spec_verify(s["target"], tlse, T, logits.view(B, R, cfg.Vt), dlse, T, dids.view(B, R), keep,
                          f2t, s["u_acc"], s["u_fin"], tokens, nacc, workspace=ws_vf)
        if side is not None:
            ev_free.record(main)

    ws_blk = vt.block_workspace(B, g, R, cfg.H, cfg.Vt, cfg.V)
    # W^Trim is built once per keep set, before decoding (VocabTrim §3): the K-tiled copy is made
    # here, outside the timed region, one per input set; the fused call reads it only where its
    # large-batch head runs
    tiled = tiled_head_used(cfg, args)
    if tiled:
        for s in sets:
            s["weight_tiled"] = vt.vt_trim_head_tiled(s["weight"], keep, k=cfg.Vt)
        torch.cuda.synchronize()
        log("K-tiled W^Trim built for each input set")

    def fused(s, events=None):
        vt.vt_spec_block(s["hidden"], s["weight"], keep, f2t, s["target"], T, T, s["u_draft"], s["u_acc"],
                         s["u_fin"], logits, dlse, dids, tlse, tokens, nacc, workspace=ws_blk, lmhead_events=events,
                         weight_tiled=s.get("weight_tiled"))

    outs = (logits, dlse, dids, tlse, tokens, nacc)
    if not args.calls and (args.graph or args.overlap):
        raise SystemExit("--graph and --overlap apply to --calls")
    if args.graph and args.overlap:
        raise SystemExit("--graph and --overlap are exclusive")
    if not args.graph:
        runners = [((lambda s=s: lmhead(s)), (lambda s=s: rest(s))) for s in sets]
    else:
        # one graph for the LM head and one for the rest of the step, per input set: replaying
        # them leaves the GPU no host-side gaps; the events between the two replays still time
        # the LM head on the stream it runs on
        # (warm-up on a stream of its own; `side` stays None: no overlap inside the graphs)
        warm = torch.cuda.Stream()
        warm.wait_stream(main)
        with torch.cuda.stream(warm):
            for s in sets:
                lmhead(s)
                rest(s)
        main.wait_stream(warm)
        torch.cuda.synchronize()
        runners = []
        for s in sets:
            ga, gb = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
            with torch.cuda.graph(ga):
                lmhead(s)
            with torch.cuda.graph(gb):
                rest(s)
            runners.append((ga.replay, gb.replay))
        torch.cuda.synchronize()
        # the replays must give the eager step's bits
        lmhead(sets[0]); rest(sets[0]); torch.cuda.synchronize()
        want = [t.clone() for t in outs]
        for t in outs:
            t.fill_(-3)
        runners[0][0](); runners[0][1](); torch.cuda.synchronize()
        if not all(torch.equal(a, b) for a, b in zip(want, outs)):
            raise RuntimeError("graph replay differs from the eager step")

    ev_a = [DeviceEvent() for _ in range(steps)]
    ev_b = [DeviceEvent() for _ in range(steps)]
    if not args.calls:
        # the fused call must agree with the four separate calls on the LM head and the target
        # log-normalisers bit for bit (draws may differ only at rounding-level CDF boundaries)
        runners[0][0](); runners[0][1](); torch.cuda.synchronize()
        want = [t.clone() for t in outs]
        fused(sets[0]); torch.cuda.synchronize()
        same = torch.equal(want[0], logits) and (args.greedy or torch.equal(want[3], tlse))
        if args.greedy:  # argmax decisions on the same logits: every output agrees
            same = same and all(torch.equal(a, b) for a, b in zip(want[1:3] + want[4:], (dlse, dids, tokens, nacc)))
        if not same:
            raise RuntimeError("vt_spec_block differs from the separate calls")
    for i in range(warmup):
        if args.calls:
            a, b = runners[i % n_sets]
            a()
            b()
        else:
            fused(sets[i % n_sets])
    torch.cuda.synchronize()
    # timed region: K steps between two synchronisations; inside it, every LM-head launch is
    # bracketed by events on the stream it is launched on
    if args.calls:
        t0 = time.perf_counter()
        for i in range(steps):
            a, b = runners[i % n_sets]
            ev_a[i].record(main)
            a()
            ev_b[i].record(main)
            b()
        torch.cuda.synchronize()
    else:
        for e in ev_a + ev_b:  # materialise the events the library records into
            e.record(main)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fused(sets[i % n_sets], (ev_a[i], ev_b[i]))
        torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = 1e3 * wall / steps
    lm_ms = sum(x.elapsed_time(y) for x, y in zip(ev_a, ev_b)) / steps
    lmb = lmhead_launch_bytes(cfg, args.greedy, args.calls)
    mean_acc = float(nacc.double().mean())
    res = dict(cfg=cfg, wl=wl, n_sets=n_sets, tiled=tiled, ms_per_step=ms_per_step, lm_ms=lm_ms, lm_bytes=lmb,
               lm_gbs=lmb / (lm_ms / 1e3) / 1e9, block_bytes=bb, block_gbs=bb / (ms_per_step / 1e3) / 1e9,
               value=B * g / (ms_per_step / 1e3), mean_accepted=mean_acc,
               mfma=B * R > 8 and not small_batch_block(cfg, args.greedy) and B * R >= 256)
    if B * R > 8:
        res["lm_tflops"] = lmhead_flops(cfg) / (lm_ms / 1e3) / 1e12
    log(f"step {ms_per_step:.4f} ms, LM head {lm_ms:.4f} ms = {res['lm_gbs']:.0f} GB/s"
        + (f" = {res['lm_tflops']:.1f} TFLOP/s" if "lm_tflops" in res else "")
        + f"; block {res['block_gbs']:.0f} GB/s algorithmic")
    del sets, base, logits
    torch.cuda.empty_cache()
    return res


def tiled_head_used(cfg, args) -> bool:
    """Whether the fused call's head reads the K-tiled W^Trim: an MFMA head (past the GEMV's sizes)
    with whole 32-column K steps, unless --head gather."""
    return not args.calls and args.head == "tiled" and not gemv_head(cfg.B * cfg.R, cfg.H) and cfg.H % 32 == 0


def side_record(res) -> dict:
    """The whole-block HBM figures of a config, for the line's side fields."""
    cfg = res["cfg"]
    return {"workload": cfg.name, "ms_per_step": round(res["ms_per_step"], 5),
            "value": round(res["value"], 1), "unit": "verified draft positions/s",
            "block_algorithmic_bytes": res["block_bytes"], "block_gbs": round(res["block_gbs"], 1),
            "block_hbm_frac": round(res["block_gbs"] / HBM_PEAK_GBS, 4),
            "lmhead_ms": round(res["lm_ms"], 5), "lmhead_gbs": round(res["lm_gbs"], 1),
            "lmhead_hbm_frac": round(res["lm_gbs"] / HBM_PEAK_GBS, 4)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.traffic_record:
        print(write_traffic_record(args.config, *args.traffic_record))
        return
    if args.valu_record:
        print(write_valu_record(args.valu_record))
        return
    if args.sequences is not None and (args.config == 1 or args.workload != "block" or args.sequences < 1):
        raise SystemExit("--sequences takes a positive count and applies to --config 2-5")
    if args.workload == "keepset":
        bench_keepset(args)
        return
    if args.workload == "generate":
        bench_generate(args)
        return
    if args.config == 1:
        bench_toy(args)
        return

    from workloads import make_workload

    res = bench_block(args, args.config, args.steps, args.warmup, args.sequences)
    cfg = res["cfg"]
    B, g = cfg.B, cfg.gamma
    # PMC records are per config at the config's own batch
    traffic = None if args.sequences else measured_traffic(f"config{args.config}")
    M = B * cfg.R
    kernel = (head_kernel(M, cfg.H, args.calls, cfg.Vt)
              + (" + target softmax partials" if small_batch_block(cfg, args.greedy) and not args.calls else ""))
    if res["mfma"]:
        # a real dense contraction: the head is priced against the bf16 MFMA peak
        tf = res["lm_tflops"]
        roof = {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": traffic, "kernel": kernel,
                "algorithmic_flops_per_launch": lmhead_flops(cfg), "algorithmic_bytes_per_launch": res["lm_bytes"],
                "avg_launch_ms": round(res["lm_ms"], 5),
                "hbm_gbs": round(res["lm_gbs"], 1), "hbm_frac": round(res["lm_gbs"] / HBM_PEAK_GBS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(res["lm_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(res["lm_gbs"] / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": kernel,
                "algorithmic_bytes_per_launch": res["lm_bytes"], "avg_launch_ms": round(res["lm_ms"], 5)}
        if "lm_tflops" in res:
            roof["mfma_tflops"] = round(res["lm_tflops"], 1)
            roof["mfma_frac"] = round(res["lm_tflops"] / BF16_MFMA_PEAK_TFLOPS, 4)

    side = {}
    if args.side_config and args.side_config != args.config and not args.greedy and not args.calls:
        side[f"config{args.side_config}"] = side_record(
            bench_block(args, args.side_config, args.side_steps, max(5, args.warmup // 2)))

    cpu = None
    if not args.no_cpu_baseline:
        wl_one = make_workload(cfg, B=1, follow=args.follow, keep_order=args.keep_order)
        log("timing the CPU oracle ...")
        cpu = cpu_baseline(cfg, wl_one, args.cpu_seconds)

    ms_per_step = res["ms_per_step"]
    out = {
        "metric": "verified draft positions/sec + LM-head HBM GB/s (% of 8 TB/s), 1 GPU",
        "value": round(res["value"], 1),
        "unit": "verified draft positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if res["mfma"] else "f32",
        "data": "synthetic",
        "config": {"workload": cfg.name, "batch": B, "gamma": g, "hidden": cfg.H, "vocab": cfg.V,
                   "kept_rows": cfg.Vt, "keep_order": args.keep_order, "target_logits": cfg.target_dtype,
                   "temperature": 0.0 if args.greedy else cfg.T,
                   "weights": "bf16", "accumulate": "f32", "input_sets_rotated": res["n_sets"],
                   "head_rows": ("K-tiled W^Trim, built once per keep set outside the timed region" if res["tiled"]
                                 else "gathered from the full head through keep_ids" if cfg.trimmed
                                 else "the full head"),
                   "verification": "greedy (temperature 0)" if args.greedy else "sampling",
                   "launch": ("vt_spec_block: one fused call per step" if not args.calls else
                              "four calls, hip graphs (LM head | rest) replayed" if args.graph else
                              "four calls, target softmax on a second stream" if args.overlap else
                              "four calls, eager, one stream"),
                   "block_algorithmic_bytes": res["block_bytes"],
                   "block_gbs": round(res["block_gbs"], 1),
                   "block_hbm_frac": round(res["block_gbs"] / HBM_PEAK_GBS, 4),
                   "lmhead_gbs": round(res["lm_gbs"], 1),
                   "lmhead_hbm_frac": round(res["lm_gbs"] / HBM_PEAK_GBS, 4),
                   "drafter": f"follows the target, noise sd {args.follow}" if args.follow > 0 else
                              "unrelated random head (the recipe)",
                   "mean_accepted": round(res["mean_accepted"], 4),
                   "tokens_per_block": round(res["mean_accepted"] + 1.0, 4),
                   "side": side or None},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
