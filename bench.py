#!/usr/bin/env python3
"""Benchmark of the HySparse2 inner-level attention hot path on one MI355X.

Workload (default): the 128k-token long prefill -- 1 sequence, L = T = 131072,
16 query heads over one shared K/V head (MQA), head dim 256, bf16, causal,
inputs N(0,1)/16 with 64 planted needle keys.  One step is the whole path on
that batch:
  scored full attention (queries processed in chunks; each chunk writes its
  float32 score rows) -> token top-k with the forced 128-token window (1024
  picks per query) -> 2 sparse layers reusing the indices (own queries each).

Printed: one JSON line with the whole-step prefill rate (tokens/s), the
roofline of the dominant kernel (the MFMA-bound full-attention kernel), the
stage breakdown, and the float64 CPU oracle timed on a bounded sample of the
same workload (rows of the same sequence, incl. the needle targets), whose
outputs are also compared with the GPU's for those rows.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--chunk C]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, TFLOP/s
D = 256


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--chunk", type=int, default=32768, help="queries per full-attention call")
    ap.add_argument("--workload", default="prefill_128k")
    ap.add_argument("--cpu-rows", type=int, default=74, help="oracle sample size (rows)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline")
    ap.add_argument("--no-others", action="store_true",
                    help="skip the decode (16 x 32k, 1M FP8) and bridge (64k) workload lines")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="run one warm-up step and one step of the full-attention launches, then a 1 GiB "
                         "copy-calibration kernel (the target of the traffic counter runs)")
    ap.add_argument("--collect-traffic", action="store_true",
                    help="run rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE over --pmc-probe and record the "
                         "per-launch HBM traffic of the full-attention kernel under profiles/")
    ap.add_argument("--out-dir", default="profile_runs",
                    help="directory (relative to the repository root) for the raw counter output of "
                         "--collect-traffic and a copy of the record")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_128k_traffic.txt")
KERNEL_SOURCES = ["attn_prefill_bf16.hip", "hs2_device.hpp", "hs2_internal.hpp"]
CALIB_BYTES = 1 << 30          # the calibration kernel reads and writes exactly this many bytes


def kernel_source_hash() -> str:
    """sha256 over the sources the full-attention kernel is compiled from."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "token_level_sparse_full_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic_record() -> dict:
    """The counter record written by --collect-traffic, or {} when there is none or the
    kernel sources changed since it was taken."""
    try:
        rec = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if "=" in line and not line.startswith("#"):
                    key, val = line.split("=", 1)
                    rec[key.strip()] = val.strip()
        return rec if rec.get("kernel_source_sha256_16") == kernel_source_hash() else {}
    except OSError:
        return {}


def read_traffic():
    """Per-launch HBM bytes of the full-attention kernel recorded by --collect-traffic,
    or None when there is no record or the kernel sources changed since it was taken."""
    try:
        return float(read_traffic_record()["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_mfma_busy():
    """MFMA busy fraction (counters, against 2.4 GHz) of the same record, or None."""
    try:
        return float(read_traffic_record()["mfma_busy_frac_at_2p4ghz"])
    except (KeyError, ValueError):
        return None


def collect_traffic(args):
    """Two counter passes (FETCH_SIZE, then WRITE_SIZE) over `bench.py --pmc-probe`, each
    scaled by what the same counter reads for a copy kernel that moves exactly CALIB_BYTES."""
    import csv
    import glob
    import subprocess

    out_root = os.path.join(ROOT, args.out_dir, "traffic")
    res = {}
    for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
        d = os.path.join(out_root, ctr.lower())
        cmd = ["rocprofv3", "--pmc", ctr, "--output-format", "csv", "-d", d, "-o", "p", "--",
               sys.executable, os.path.join(ROOT, "bench.py"), "--pmc-probe", "--workload", args.workload,
               "--chunk", str(args.chunk)]
        print("[traffic] " + " ".join(cmd), flush=True)
        env = dict(os.environ, TMPDIR="/tmp")
        r = subprocess.run(cmd, cwd="/tmp", env=env, timeout=300)
        if r.returncode != 0:
            raise SystemExit(f"rocprofv3 {ctr} pass failed with status {r.returncode}")
        rows = []
        for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            rows += list(csv.DictReader(open(fn)))
        per = {}
        for row in rows:
            if row["Counter_Name"] != ctr:
                continue
            key = (int(row["Dispatch_Id"]), row["Kernel_Name"])
            per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
        disp = sorted(per.items())
        attn = [v for (i, n), v in disp if "prefill_bf16_kernel" in n]
        calib = [v for (i, n), v in disp if "elementwise" in n]
        n_launch = len(range(0, inputs_L(args), min(args.chunk, inputs_L(args))))
        # one full-attention call = the lse dispatch + the P/V dispatch; the
        # measured step is the last n_launch calls (the warm-up step comes first)
        attn = attn[-2 * n_launch:]
        res[ctr] = {"attn_kib_per_launch": sum(attn) / n_launch, "calib_kib": calib[-1], "launches": n_launch}
    # one more pass: MFMA busy cycles of the same launches (utilisation of the matrix cores)
    d = os.path.join(out_root, "sq")
    sq_ctrs = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "GRBM_GUI_ACTIVE"]
    cmd = ["rocprofv3", "--pmc", *sq_ctrs, "--output-format", "csv", "-d", d, "-o", "p", "--",
           sys.executable, os.path.join(ROOT, "bench.py"), "--pmc-probe", "--workload", args.workload,
           "--chunk", str(args.chunk)]
    print("[traffic] " + " ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd="/tmp", env=dict(os.environ, TMPDIR="/tmp"), timeout=300)
    if r.returncode != 0:
        raise SystemExit(f"rocprofv3 SQ pass failed with status {r.returncode}")
    rows = []
    for fn in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        rows += list(csv.DictReader(open(fn)))
    sq, dur = {}, {}
    for row in rows:
        if "prefill_bf16_kernel" not in row["Kernel_Name"]:
            continue
        i = int(row["Dispatch_Id"])
        sq.setdefault(i, {}).setdefault(row["Counter_Name"], 0.0)
        sq[i][row["Counter_Name"]] += float(row["Counter_Value"])
        dur[i] = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-9
    n_launch = res["FETCH_SIZE"]["launches"]
    last = sorted(sq)[-2 * n_launch:]            # both dispatches of each call
    sq_avg = {c: sum(sq[i].get(c, 0.0) for i in last) / n_launch for c in sq_ctrs}
    dur_avg = sum(dur[i] for i in last) / n_launch
    # busy cycles of all 1024 SIMDs over the launch at the 2.4 GHz peak clock (a lower bound
    # on the utilisation when the clock runs below peak)
    mfma_util = sq_avg["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * dur_avg * 2.4e9)
    f_fetch = CALIB_BYTES / (res["FETCH_SIZE"]["calib_kib"] * 1024.0)
    f_write = CALIB_BYTES / (res["WRITE_SIZE"]["calib_kib"] * 1024.0)
    fetch_b = res["FETCH_SIZE"]["attn_kib_per_launch"] * 1024.0 * f_fetch
    write_b = res["WRITE_SIZE"]["attn_kib_per_launch"] * 1024.0 * f_write
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        f.write("# HBM traffic of one scored full-attention call (its two dispatches: prefill_bf16_kernel<H,1>,\n")
        f.write("# the lse pass, and prefill_bf16_kernel<H,2>, the P/V pass), one call of the\n")
        f.write(f"# {args.workload} step ({res['FETCH_SIZE']['launches']} launches of {args.chunk} queries,"
                " averaged), from rocprofv3 counter passes.\n")
        f.write("# command: python bench.py --collect-traffic   (runs, one pass per counter set:)\n")
        f.write(f"#   rocprofv3 --pmc <FETCH_SIZE | WRITE_SIZE | {' '.join(sq_ctrs)}> --output-format csv -d <dir> -o p"
                f" -- python bench.py --pmc-probe --workload {args.workload} --chunk {args.chunk}\n")
        f.write("# calibration: a float32 copy kernel (torch.mul by 1.0) that reads and writes exactly 1 GiB;\n")
        f.write("# each counter is scaled by (1 GiB / what it reads for that kernel).\n")
        f.write(f"fetch_kib_per_launch_raw = {res['FETCH_SIZE']['attn_kib_per_launch']:.1f}\n")
        f.write(f"write_kib_per_launch_raw = {res['WRITE_SIZE']['attn_kib_per_launch']:.1f}\n")
        f.write(f"calib_fetch_kib = {res['FETCH_SIZE']['calib_kib']:.1f}\n")
        f.write(f"calib_write_kib = {res['WRITE_SIZE']['calib_kib']:.1f}\n")
        f.write(f"scale_fetch = {f_fetch:.4f}\n")
        f.write(f"scale_write = {f_write:.4f}\n")
        f.write(f"fetch_bytes_per_launch = {fetch_b:.4e}\n")
        f.write(f"write_bytes_per_launch = {write_b:.4e}\n")
        f.write(f"traffic_bytes_per_launch = {fetch_b + write_b:.4e}\n")
        f.write("# MFMA utilisation of the same launches (third pass, SQ counters, per launch):\n")
        for c in sq_ctrs:
            f.write(f"{c.lower()} = {sq_avg[c]:.4e}\n")
        f.write(f"launch_seconds_under_counters = {dur_avg:.4f}\n")
        f.write(f"mfma_busy_frac_at_2p4ghz = {mfma_util:.4f}\n")
        f.write(f"kernel_source_sha256_16 = {kernel_source_hash()}\n")
    text = open(TRAFFIC_FILE).read()
    os.makedirs(os.path.join(ROOT, args.out_dir), exist_ok=True)
    with open(os.path.join(ROOT, args.out_dir, os.path.basename(TRAFFIC_FILE)), "w") as f:
        f.write(text)
    print(text, flush=True)


def inputs_L(args) -> int:
    from token_level_sparse_full_amd import inputs
    return inputs.WORKLOADS[args.workload].L


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "bench.py measures a single GPU; multi-GPU runs are not supported: use --gpus 1"}))
        sys.exit(2)
    if args.collect_traffic:      # orchestration only: this process never touches the GPU
        collect_traffic(args)
        return

    import numpy as np
    import torch

    from token_level_sparse_full_amd import hs2, inputs

    wl = inputs.WORKLOADS[args.workload]
    assert wl.kind == "prefill" and wl.kv == "bf16"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    L, H, n_sparse = wl.L, wl.H, wl.n_sparse
    scale = 1.0 / math.sqrt(D)
    window, topk = 128, 1024
    max_sel = window + topk

    # ---------------------------------------------------------------- inputs (resident in HBM)
    inp = inputs.attention_inputs(B=1, n_q=L, T=L, H=H, d=D, kv=wl.kv, n_sparse=n_sparse, seed=wl.seed, device=dev)
    needles = inputs.plant_needles(inp["q"][0], inp["k"][0], wl.needles, wl.seed) if wl.needles else []
    q, k, v, qs = inp["q"], inp["k"], inp["v"], inp["q_sparse"]
    C = min(args.chunk, L)
    chunks = [(c0, min(L, c0 + C)) for c0 in range(0, L, C)]
    ld = (L + 3) // 4 * 4
    scores = torch.empty((1, C, ld), dtype=torch.float32, device=dev)
    idx = torch.empty((1, L, max_sel), dtype=torch.int32, device=dev)
    cnt = torch.empty((1, L), dtype=torch.int32, device=dev)
    o_full = torch.empty_like(q)
    lse_full = torch.empty((1, L, H), dtype=torch.float32, device=dev)
    o_sp = [torch.empty_like(q) for _ in range(n_sparse)]
    lse_sp = [torch.empty((1, L, H), dtype=torch.float32, device=dev) for _ in range(n_sparse)]
    torch.cuda.synchronize()

    n_ev = len(chunks) * 2 + n_sparse + 1
    keep_rows = {}

    def step(events=None, sample_rows=None):
        ev = iter(events) if events else None
        mark = (lambda: next(ev).record()) if ev else (lambda: None)
        mark()
        for c0, c1 in chunks:
            hs2.hs2_full_attn_scored(q[:, c0:c1], k, v, q_pos0=c0, sm_scale=scale, o=o_full[:, c0:c1],
                                     lse=lse_full[:, c0:c1], scores=scores[:, : c1 - c0], ld_scores=ld)
            mark()
            if sample_rows:
                for p in sample_rows:
                    if c0 <= p < c1:
                        keep_rows[p] = scores[0, p - c0, : p + 1].clone()
            hs2.hs2_select_topk_window(scores[:, : c1 - c0], q_pos0=c0, T=L, n_q=c1 - c0, window=window, topk=topk,
                                       idx=idx[:, c0:c1], count=cnt[:, c0:c1])
            mark()
        for s in range(n_sparse):
            hs2.hs2_sparse_attn_reuse(qs[s], k, v, idx, cnt, sm_scale=scale, o=o_sp[s], lse=lse_sp[s])
            mark()

    if args.pmc_probe:
        step()                                   # warm-up step
        torch.cuda.synchronize()
        for c0, c1 in chunks:                    # the measured full-attention launches
            hs2.hs2_full_attn_scored(q[:, c0:c1], k, v, q_pos0=c0, sm_scale=scale, o=o_full[:, c0:c1],
                                     lse=lse_full[:, c0:c1], scores=scores[:, : c1 - c0], ld_scores=ld)
        torch.cuda.synchronize()
        a = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.mul(a, 1.0, out=b)                 # copy calibration: reads and writes 1 GiB
        torch.cuda.synchronize()
        print("pmc probe done", flush=True)
        return

    # ---------------------------------------------------------------- warmup + timed steps
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total, ms_fa, ms_sel, ms_sp = [], [], [], []
    for e in evs:
        ms_total.append(e[0].elapsed_time(e[-1]))
        j = 0
        fa = sel = 0.0
        for _ in chunks:
            fa += e[j].elapsed_time(e[j + 1])
            sel += e[j + 1].elapsed_time(e[j + 2])
            j += 2
        ms_fa.append(fa)
        ms_sel.append(sel)
        ms_sp.append([e[j + i].elapsed_time(e[j + i + 1]) for i in range(n_sparse)])
    ms_step = float(np.mean(ms_total))
    fa_ms = float(np.mean(ms_fa))
    sel_ms = float(np.mean(ms_sel))
    sp_ms = float(np.mean([np.mean(x) for x in ms_sp]))

    # ---------------------------------------------------------------- algorithmic work
    npos = np.arange(L, dtype=np.float64) + 1.0                     # keys seen by each query
    fa_flop = 4.0 * H * D * npos.sum()                               # QK^T + PV, causal
    fa_tflops = fa_flop / (fa_ms * 1e-3) / 1e12
    counts = np.minimum(npos, max_sel)
    sp_bytes = counts.sum() * 2 * D * 2 + L * (2 * H * D * 2 + max_sel * 4 + 4 + H * 4)
    sp_gbs = sp_bytes / (sp_ms * 1e-3) / 1e9
    cand = np.maximum(npos - window, 0)
    sel_bytes = np.where(cand > topk, cand, 0).sum() * 4 + L * max_sel * 4
    sel_gbs = sel_bytes / (sel_ms * 1e-3) / 1e9

    result = {
        "metric": "sparse-reuse attn queries/s at 128k ctx + prefill tokens/s; % HBM/MFMA peak",
        "value": L / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)/16 Q/K/V, 64 planted needle keys)",
        "config": {"workload": "prefill_128k", "seq_len": L, "query_heads": H, "kv_heads": 1, "head_dim": D,
                   "window": window, "topk": topk, "sparse_layers": n_sparse, "query_chunk": C,
                   "global_batch": 1, "parallelism": "single GPU"},
        "roofline": {"kernel": "hs2_full_attn_scored, prefill path (lse dispatch + P/V dispatch)", "bound": "mfma",
                     "achieved": fa_tflops, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": fa_tflops / BF16_PEAK_TFLOPS, "traffic": read_traffic(),
                     "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "algorithmic_flop_per_step": fa_flop, "launches_per_step": len(chunks),
                     # the lse dispatch repeats QK^T: executed MFMA work is 1.5x the algorithmic
                     "executed_frac": 1.5 * fa_tflops / BF16_PEAK_TFLOPS,
                     "mfma_busy_frac_counters": read_mfma_busy()},
        "stages": {
            "full_attn_ms": fa_ms, "select_ms": sel_ms, "sparse_ms_per_layer": sp_ms,
            "sparse_reuse_queries_per_s": L / (sp_ms * 1e-3),
            "sparse_reuse_gbs_algorithmic": sp_gbs, "sparse_reuse_hbm_frac": sp_gbs / HBM_PEAK_GBS,
            "select_gbs_algorithmic": sel_gbs,
            "wall_s_timed": wall,
        },
    }

    if not args.no_others:
        result["ablation_block_selection"] = ablation_blocks(hs2, q, k, v, qs, chunks, scale, ld, window, topk)
        result["other_workloads"] = other_workloads(dev)

    # ---------------------------------------------------------------- oracle sample (host cores)
    if not args.no_cpu:
        result["cpu_baseline"], result["sample_parity"] = cpu_baseline(
            args, inp, needles, step, keep_rows, idx, cnt, o_full, o_sp, L, H, scale, window, topk)
    print(json.dumps(result), flush=True)


def ablation_blocks(hs2, q, k, v, qs, chunks, scale, ld, window, topk, block=64):
    """The block-level selection (aligned 64-token blocks, same 1024-token budget) on the
    same scores as the token-level one, and the sparse layer on its indices: HIP-event
    times of both selectors per chunk (second of two runs each) and the median of 3 sparse
    layers on each index set.  The full-attention launches that produce the scores are
    not timed."""
    import numpy as np
    import torch

    dev = q.device
    L, H = q.shape[1], q.shape[2]
    C = chunks[0][1] - chunks[0][0]
    ms = window + topk
    scores = torch.empty((1, C, ld), dtype=torch.float32, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((1, L, H), dtype=torch.float32, device=dev)
    idx_t = torch.empty((1, L, ms), dtype=torch.int32, device=dev)
    cnt_t = torch.empty((1, L), dtype=torch.int32, device=dev)
    idx_b, cnt_b = torch.empty_like(idx_t), torch.empty_like(cnt_t)
    ws_b = hs2.workspace(max(hs2.select_blocks_workspace_bytes(1, c1 - c0, L, c0, window, block)
                             for c0, c1 in chunks), dev)

    def ev_time(fn, reps):
        t = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            t.append(a.elapsed_time(b))
        return t

    t_tok = t_blk = 0.0
    for c0, c1 in chunks:
        hs2.hs2_full_attn_scored(q[:, c0:c1], k, v, q_pos0=c0, sm_scale=scale, o=o[:, c0:c1], lse=lse[:, c0:c1],
                                 scores=scores[:, : c1 - c0], ld_scores=ld)
        t_tok += ev_time(lambda: hs2.hs2_select_topk_window(scores[:, : c1 - c0], q_pos0=c0, T=L, n_q=c1 - c0,
                                                            window=window, topk=topk, idx=idx_t[:, c0:c1],
                                                            count=cnt_t[:, c0:c1]), 2)[-1]
        t_blk += ev_time(lambda: hs2.hs2_select_blocks_window(scores[:, : c1 - c0], q_pos0=c0, T=L, n_q=c1 - c0,
                                                              window=window, topk=topk, block=block,
                                                              idx=idx_b[:, c0:c1], count=cnt_b[:, c0:c1], ws=ws_b),
                         2)[-1]
    o2 = torch.empty_like(q)
    l2 = torch.empty_like(lse)
    sp_tok = float(np.median(ev_time(lambda: hs2.hs2_sparse_attn_reuse(qs[0], k, v, idx_t, cnt_t, sm_scale=scale,
                                                                       o=o2, lse=l2), 3)))
    sp_blk = float(np.median(ev_time(lambda: hs2.hs2_sparse_attn_reuse(qs[0], k, v, idx_b, cnt_b, sm_scale=scale,
                                                                       o=o2, lse=l2), 3)))
    rows = np.arange(L, dtype=np.float64) + 1.0
    cand = np.maximum(rows - window, 0)
    read_bytes = np.where(cand > topk, cand, 0).sum() * 4
    n_sel_tok = float(cnt_t.sum().item())
    n_sel_blk = float(cnt_b.sum().item())
    del scores, o, lse, idx_t, cnt_t, idx_b, cnt_b, ws_b, o2, l2
    torch.cuda.empty_cache()
    return {"block": block, "select_token_ms": t_tok, "select_block_ms": t_blk,
            "select_block_gbs_of_scores": read_bytes / (t_blk * 1e-3) / 1e9,
            "sparse_layer_token_ms": sp_tok, "sparse_layer_block_ms": sp_blk,
            "selected_keys_token": n_sel_tok, "selected_keys_block": n_sel_blk,
            "note": "same scores, same 1024-token budget; block sums in float32 (pairwise tree)"}


def _timed(run, stages: int, reps: int = 10, warm: int = 3, flush=None):
    """Median over reps of the HIP-event times between stage marks (run(mark) calls mark()
    after each stage).  flush() runs between reps, outside the timed region."""
    import numpy as np
    import torch

    for _ in range(warm):
        run(lambda: None)
    torch.cuda.synchronize()
    per = []
    for _ in range(reps):
        if flush is not None:
            flush()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(stages + 1)]
        it = iter(ev)
        next(it).record()
        run(lambda: next(it).record())
        torch.cuda.synchronize()
        per.append([ev[i].elapsed_time(ev[i + 1]) for i in range(stages)])
    return np.median(np.array(per), axis=0)


def other_workloads(dev):
    """The decode and bridge workloads at their own sizes: HIP-event times of each stage
    (median of 10 after 3 warm-ups; a 512 MiB buffer write between reps pushes K/V out of
    L2 and MALL) against the HBM (decode stages) or bf16 MFMA (bridge) roofline."""
    import torch

    from token_level_sparse_full_amd import hs2, inputs

    out = {}
    junk = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flush = lambda: junk.fill_(1)  # noqa: E731
    win, topk, ms = 128, 1024, 128 + 1024
    scale = 1.0 / 16

    def decode_step(q, qs, k, v, T, p, ks=None, vs=None):
        B, _, H, _ = q.shape
        kvd = hs2._dtype_code(k)
        ws = hs2.workspace(hs2.full_attn_workspace_bytes(B, 1, H, T, kvd), dev)
        o = torch.empty_like(q)
        lse = torch.empty((B, 1, H), dtype=torch.float32, device=dev)
        ld = (p + 1 + 3) // 4 * 4
        sc = torch.empty((B, 1, ld), dtype=torch.float32, device=dev)
        idx = torch.empty((B, 1, ms), dtype=torch.int32, device=dev)
        cnt = torch.empty((B, 1), dtype=torch.int32, device=dev)
        o2 = [torch.empty_like(x) for x in qs]
        l2 = [torch.empty((B, 1, H), dtype=torch.float32, device=dev) for _ in qs]
        ws_sp = hs2.workspace(hs2.sparse_workspace_bytes(B, 1, H, ms), dev)

        def run(mark):
            hs2.hs2_full_attn_scored(q, k, v, q_pos0=p, sm_scale=scale, k_scale=ks, v_scale=vs, o=o, lse=lse,
                                     scores=sc, ld_scores=ld, ws=ws)
            mark()
            hs2.hs2_select_topk_window(sc, q_pos0=p, T=T, idx=idx, count=cnt)
            mark()
            for i, x in enumerate(qs):
                hs2.hs2_sparse_attn_reuse(x, k, v, idx, cnt, sm_scale=scale, k_scale=ks, v_scale=vs, o=o2[i],
                                          lse=l2[i], ws=ws_sp)
            mark()
        return _timed(run, 3, flush=flush)

    def prefill_over_bridge(wl, kl, vl, ksl=None, vsl=None):
        """Every prompt position runs the cross-decoder on the bridged cache: per full layer,
        scored full attention over all L positions (query chunks of 32768), the selection,
        and the layer's sparse layers on its indices.  Returns (full attention, select,
        sparse) ms summed over the layers (median of 3 after 1 warm-up; inputs resident)."""
        L, H, C = wl.L, wl.H, 32768
        chunks = [(c0, min(L, c0 + C)) for c0 in range(0, L, C)]
        kvd = hs2._dtype_code(kl)
        qf = [inputs.cast(inputs.normal((1, L, H, 256), inputs.STD_QKV, wl.seed, inputs.S_QFULL_LAYER + m, dev),
                          "bf16") for m in range(wl.n_full)]
        qsp = [[inputs.cast(inputs.normal((1, L, H, 256), inputs.STD_QKV, wl.seed, inputs.S_QSPARSE + 8 * m + i, dev),
                            "bf16") for i in range(wl.n_sparse)] for m in range(wl.n_full)]
        sc = torch.empty((1, C, L), dtype=torch.float32, device=dev)
        idx = torch.empty((1, L, ms), dtype=torch.int32, device=dev)
        cnt = torch.empty((1, L), dtype=torch.int32, device=dev)
        o = torch.empty((1, L, H, 256), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((1, L, H), dtype=torch.float32, device=dev)
        o2, l2 = torch.empty_like(o), torch.empty_like(lse)
        ws_fa = hs2.workspace(hs2.full_attn_workspace_bytes(1, C, H, L, kvd), dev)
        ws_sp = hs2.workspace(hs2.sparse_workspace_bytes(1, L, H, ms), dev)

        def run(mark):
            for m in range(wl.n_full):
                ks_m = None if ksl is None else ksl[m:m + 1]
                vs_m = None if vsl is None else vsl[m:m + 1]
                for c0, c1 in chunks:
                    hs2.hs2_full_attn_scored(qf[m][:, c0:c1], kl[m:m + 1], vl[m:m + 1], q_pos0=c0, sm_scale=scale,
                                             k_scale=ks_m, v_scale=vs_m, o=o[:, c0:c1], lse=lse[:, c0:c1],
                                             scores=sc[:, : c1 - c0], ld_scores=L, ws=ws_fa)
                    mark()
                    hs2.hs2_select_topk_window(sc[:, : c1 - c0], q_pos0=c0, T=L, n_q=c1 - c0, window=win, topk=topk,
                                               idx=idx[:, c0:c1], count=cnt[:, c0:c1])
                    mark()
                for x in qsp[m]:
                    hs2.hs2_sparse_attn_reuse(x, kl[m:m + 1], vl[m:m + 1], idx, cnt, sm_scale=scale, k_scale=ks_m,
                                              v_scale=vs_m, o=o2, lse=l2, ws=ws_sp)
                mark()
        per_layer = 2 * len(chunks) + 1
        t = _timed(run, wl.n_full * per_layer, reps=3, warm=1)
        t = t.reshape(wl.n_full, per_layer)
        t_fa = float(t[:, 0:-1:2].sum())
        t_sel = float(t[:, 1:-1:2].sum())
        t_sp = float(t[:, -1].sum())
        del qf, qsp, sc, idx, cnt, o, lse, o2, l2, ws_fa, ws_sp
        torch.cuda.empty_cache()
        return t_fa, t_sel, t_sp

    def reading_b_entry(wl, t_br, t_fa, t_sel, t_sp, note):
        fa_flop = wl.n_full * 4.0 * wl.H * D * (wl.L * (wl.L + 1) / 2.0)
        total = t_br + t_fa + t_sel + t_sp
        return {"ms_per_prompt": total, "prefill_tokens_per_s": wl.L / (total * 1e-3), "bridge_ms": float(t_br),
                "full_attn_ms_all_layers": t_fa, "full_attn_tflops": fa_flop / (t_fa * 1e-3) / 1e12,
                "full_attn_mfma_frac": fa_flop / (t_fa * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
                "select_ms_all_layers": t_sel, "sparse_ms_all_layers": t_sp, "note": note}

    # batched decode: 16 sequences x 32k keys, 3 sparse layers
    wl = inputs.WORKLOADS["decode_b16_32k"]
    inp = inputs.attention_inputs(B=wl.B, n_q=1, T=wl.T, H=wl.H, d=D, kv="bf16", n_sparse=wl.n_sparse, seed=wl.seed,
                                  device=dev)
    t_fa, t_sel, t_sp = decode_step(inp["q"], inp["q_sparse"], inp["k"], inp["v"], wl.T, wl.T - 1)
    kv_bytes = 2.0 * wl.B * wl.T * 512
    sp_bytes = wl.B * (ms * 2 * 512 + 2 * wl.H * D * 2 + ms * 4)
    out[wl.name] = {
        "ms_per_step": float(t_fa + t_sel + t_sp), "queries_per_s": wl.B / ((t_fa + t_sel + t_sp) * 1e-3),
        "full_attn_ms": float(t_fa), "full_attn_hbm_frac": kv_bytes / (t_fa * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "select_ms": float(t_sel), "sparse_ms_all_layers": float(t_sp),
        "sparse_hbm_frac": wl.n_sparse * sp_bytes / (t_sp * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "note": "cold: a 512 MiB write between reps; K/V 512 MiB per step"}
    del inp
    torch.cuda.empty_cache()

    # one 1M-token sequence, FP8 e4m3 K/V with per-row scales, 4 decode steps, 4 sparse layers each
    wl = inputs.WORKLOADS["decode_1m_fp8"]
    k, v, ks, vs = inputs.kv_cache((1, wl.T, 256), "e4m3", wl.seed, dev)
    steps = []
    for st in range(wl.steps):
        p = wl.T - wl.steps + st
        q = inputs.cast(inputs.normal((1, 1, wl.H, 256), inputs.STD_QKV, wl.seed, inputs.S_Q + 10 * st, dev), "bf16")
        qs = [inputs.cast(inputs.normal((1, 1, wl.H, 256), inputs.STD_QKV, wl.seed, inputs.S_QSPARSE + 10 * st + i,
                                        dev), "bf16") for i in range(wl.n_sparse)]
        steps.append(decode_step(q, qs, k, v, wl.T, p, ks, vs))
    t_fa = sum(x[0] for x in steps) / len(steps)
    t_sel = sum(x[1] for x in steps) / len(steps)
    t_sp = sum(x[2] for x in steps) / len(steps)
    kv_bytes = 2.0 * wl.T * (256 + 4)
    out[wl.name] = {
        "ms_per_step": float(t_fa + t_sel + t_sp), "queries_per_s": 1.0 / ((t_fa + t_sel + t_sp) * 1e-3),
        "full_attn_ms": float(t_fa), "full_attn_hbm_frac": kv_bytes / (t_fa * 1e-3) / (HBM_PEAK_GBS * 1e9),
        "select_ms": float(t_sel), "sparse_ms_all_layers": float(t_sp),
        "note": "mean of the 4 steps (p = T-4 .. T-1); cold between reps"}
    del k, v, ks, vs
    torch.cuda.empty_cache()

    # KV bridging: 4 projections of a 64k-token hidden state, then 4 bridged decode steps
    wl = inputs.WORKLOADS["bridge_64k"]
    br = inputs.bridge_inputs(L=wl.L, D=wl.D, n_layers=wl.n_full, d=256, seed=wl.seed, device=dev)
    k_all = torch.empty((wl.n_full, wl.L, 256), dtype=torch.bfloat16, device=dev)
    v_all = torch.empty_like(k_all)

    def run_bridge(mark):
        hs2.hs2_bridge_kv_proj(br["x"], br["w_k"], br["w_v"], k_out=k_all, v_out=v_all)
        mark()
    (t_br,) = _timed(run_bridge, 1)
    br_flop = 2.0 * wl.L * wl.D * (2 * wl.n_full * 256)
    t_layers = []
    for m in range(wl.n_full):
        q = inputs.cast(inputs.normal((1, 1, wl.H, 256), inputs.STD_QKV, wl.seed, inputs.S_QFULL_LAYER + m, dev),
                        "bf16")
        qs = [inputs.cast(inputs.normal((1, 1, wl.H, 256), inputs.STD_QKV, wl.seed, inputs.S_QSPARSE + 8 * m + i, dev),
                          "bf16") for i in range(wl.n_sparse)]
        t_layers.append(decode_step(q, qs, k_all[m:m + 1], v_all[m:m + 1], wl.L, wl.L - 1))
    t_cross = float(sum(sum(x) for x in t_layers))
    out[wl.name] = {
        "bridge_ms": float(t_br), "bridge_tflops": br_flop / (t_br * 1e-3) / 1e12,
        "bridge_mfma_frac": br_flop / (t_br * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
        "cross_decoder_step_ms": t_cross, "prefill_tokens_per_s": wl.L / ((t_br + t_cross) * 1e-3),
        "note": "bridge warm (inputs resident); the 4 bridged decode steps cold"}
    out[wl.name + "_every_position"] = reading_b_entry(
        wl, t_br, *prefill_over_bridge(wl, k_all, v_all),
        "the cross-decoder at every prompt position: 4 full layers x (scored full attention over 65536 "
        "positions, select, 8 sparse layers) on the bf16 bridged cache")
    del k_all, v_all
    torch.cuda.empty_cache()

    # the same bridge writing the FP8 e4m3 cache (codes + per-row scales), then the
    # 4 bridged decode steps reading that cache
    k8 = torch.empty((wl.n_full, wl.L, 256), dtype=torch.uint8, device=dev)
    v8 = torch.empty_like(k8)
    ks8 = torch.empty((wl.n_full, wl.L), dtype=torch.float32, device=dev)
    vs8 = torch.empty_like(ks8)

    def run_bridge8(mark):
        hs2.hs2_bridge_kv_proj_fp8(br["x"], br["w_k"], br["w_v"], k_out=k8, v_out=v8, k_scale=ks8, v_scale=vs8)
        mark()
    (t_br8,) = _timed(run_bridge8, 1)
    t_layers = []
    for m in range(wl.n_full):
        q = inputs.cast(inputs.normal((1, 1, wl.H, 256), inputs.STD_QKV, wl.seed, inputs.S_QFULL_LAYER + m, dev),
                        "bf16")
        qs = [inputs.cast(inputs.normal((1, 1, wl.H, 256), inputs.STD_QKV, wl.seed, inputs.S_QSPARSE + 8 * m + i, dev),
                          "bf16") for i in range(wl.n_sparse)]
        t_layers.append(decode_step(q, qs, k8[m:m + 1], v8[m:m + 1], wl.L, wl.L - 1, ks8[m:m + 1], vs8[m:m + 1]))
    t_cross8 = float(sum(sum(x) for x in t_layers))
    out[wl.name + "_fp8"] = {
        "bridge_ms": float(t_br8), "bridge_tflops": br_flop / (t_br8 * 1e-3) / 1e12,
        "bridge_mfma_frac": br_flop / (t_br8 * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
        "cross_decoder_step_ms": t_cross8, "prefill_tokens_per_s": wl.L / ((t_br8 + t_cross8) * 1e-3),
        "note": "bridge into the e4m3 cache (per-row scales) and the bridged decode steps on it"}
    out[wl.name + "_fp8_every_position"] = reading_b_entry(
        wl, t_br8, *prefill_over_bridge(wl, k8, v8, ks8, vs8),
        "the cross-decoder at every prompt position on the e4m3 bridged cache (many-query e4m3 kernel)")
    del junk
    return out


def cpu_baseline(args, inp, needles, step, keep_rows, idx, cnt, o_full, o_sp, L, H, scale, window, topk):
    """Time the float64 oracle on sampled query rows of the same sequence and
    compare the GPU results of those rows with it."""
    import numpy as np
    import torch

    import oracle
    from token_level_sparse_full_amd import inputs

    edge = [0, 1, 127, 128, 129, 1151, 1152, 1153, L // 2, L - 1]
    rows = sorted(set(edge + [i for _, i in needles]))[: max(args.cpu_rows, len(edge))]
    # one more pass that also keeps the score rows of the sampled queries
    step(sample_rows=rows)
    torch.cuda.synchronize()
    k64 = oracle.decode_rows(inputs.raw_numpy(inp["k"][0]), "bf16")
    v64 = oracle.decode_rows(inputs.raw_numpy(inp["v"][0]), "bf16")
    q_np = inputs.raw_numpy(inp["q"][0])
    qs_np = [inputs.raw_numpy(t[0]) for t in inp["q_sparse"]]
    idx_np, cnt_np = idx[0].cpu().numpy(), cnt[0].cpu().numpy()
    o_np = o_full[0].float().cpu().numpy()
    osp_np = [t[0].float().cpu().numpy() for t in o_sp]
    worst = {"full_o": 0.0, "scores_rel": 0.0, "sparse_o": 0.0, "sel_swaps": 0, "needles_found": 0}
    t0 = time.perf_counter()
    for p in rows:
        qrow = oracle.decode_rows(q_np[p:p + 1], "bf16")
        o_ref, _, s_ref = oracle.full_attn_scored(qrow, k64, v64, p, scale)
        sel, n, tau = oracle.select_topk_window(s_ref[0], p, window, topk)
        o2_refs = [oracle.sparse_attn_reuse(oracle.decode_rows(qs_np[s][p], "bf16"), k64, v64, sel, scale)[0]
                   for s in range(len(qs_np))]
        # comparisons (not part of the timed oracle work: cheap)
        worst["full_o"] = max(worst["full_o"], float(np.abs(o_np[p] - o_ref[0]).max()))
        g = keep_rows[p].cpu().numpy().astype(np.float64)
        worst["scores_rel"] = max(worst["scores_rel"], float((np.abs(g - s_ref[0]) / s_ref[0]).max()))
        got = idx_np[p, : cnt_np[p]]
        diff = np.setxor1d(got, sel)
        if tau is not None and diff.size:
            assert (np.abs(s_ref[0][diff] - tau) <= 1e-5 * tau).all(), f"selection outside tolerance at row {p}"
        worst["sel_swaps"] += int(diff.size)
        # the sparse layers are compared on the GPU's own index set (stage-wise inputs)
        for s in range(len(qs_np)):
            o2_on_gpu_set, _ = oracle.sparse_attn_reuse(oracle.decode_rows(qs_np[s][p], "bf16"), k64, v64, got, scale)
            worst["sparse_o"] = max(worst["sparse_o"], float(np.abs(osp_np[s][p] - o2_on_gpu_set).max()))
        del o2_refs
    t_cpu = time.perf_counter() - t0
    for j, i in needles:
        worst["needles_found"] += int(np.isin(j, idx_np[i, : cnt_np[i]]))
    worst["needles"] = len(needles)
    worst["rows"] = len(rows)
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = 1
    cores = min(len(os.sched_getaffinity(0)), blas_threads)
    base = {"value": len(rows) / t_cpu, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{len(rows)} query rows of the same 128k sequence (64 needle targets + edge positions), "
                      f"each through full attention + select + {len(qs_np)} sparse layers in float64",
            "seconds": t_cpu}
    return base, worst


if __name__ == "__main__":
    main()
