"""Benchmark of the WorldKV KV-memory hot path on one GPU.

One step is one pass of the whole path for one denoising chunk at one layer:
  1. World Compression of the chunk leaving the recent window (1 unit),
  2. pose top-k retrieval over the stored chunks,
  3. window assembly sink | retrieved | recent | current,
  4. chunk attention of the current queries over the window, once per
     denoising step of the chunk.
Steps 1-2 of chunk i+1 run on a second stream beside steps 3-4 of chunk i
(the timed throughput); the same steps on one stream are reported too.
Inputs are seeded synthetic tensors resident in HBM before the timed region;
several input sets rotate so the bandwidth-bound calls are not served from the
last-level cache. After the timed region the CPU oracle runs on a bounded
sample of the same workload (reported as ``cpu_baseline``).

The default workload is the 14B-class single layer (40 heads x d128, 3x1560-token
chunks, 4 denoising steps), the largest that fits one GPU; the 1.3B-class, tiny
and int4-store configurations and the compression sweep are selected with
--config. The breakdown also times batched compression of 300 units of the
1.3B-class chunk shape (bf16 and int4 stores, r = 0.25 and 0.5).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 14b]
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import gc
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("chunk-attention TFLOP/s + compress/gather GB/s; "
          "per-chunk denoise-step latency")
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E

# Workloads: heads x head dim, tokens per frame, frames per chunk, keep ratio,
# stored chunks, retrieved k, recent chunks, denoising steps, int4 bank, and
# the streams the timed step uses: 2 runs step i+1's compression and
# retrieval beside step i's attention; 1 runs every call in order. The
# 14B-class step is 98 % attention, whose 0.9 ms blocks fill the chip in
# under three rounds: work beside it delays blocks into a later round, which
# cost 0.4-0.7 ms per step on three boxes, against 0.06 ms of work hidden.
CONFIGS = {
    "tiny": dict(H=2, D=64, T=64, F=3, r=0.5, M=8, k=2, n_recent=1, S=1, int4=False, streams=2,
                 name="tiny: 2 heads x d64, 3x64-token chunks, 8 stored chunks, "
                      "window sink + 2 retrieved (r=0.5) + 1 recent + current"),
    "1.3b": dict(H=12, D=128, T=880, F=3, r=0.5, M=20, k=3, n_recent=2, S=1, int4=False, streams=2,
                 name="1.3B-class single layer: 12 heads x d128, 3x880-token chunks, "
                      "20 stored chunks, window sink + 3 retrieved (r=0.5) + 2 recent "
                      "+ current"),
    "14b": dict(H=40, D=128, T=1560, F=3, r=0.25, M=120, k=6, n_recent=2, S=4, int4=False, streams=1,
                name="14B-class single layer: 40 heads x d128, 3x1560-token chunks, "
                     "120 stored chunks, window sink + 6 retrieved (r=0.25) + 2 recent "
                     "+ current, 4 denoising steps"),
    "int4": dict(H=12, D=128, T=880, F=3, r=0.5, M=1000, k=4, n_recent=2, S=1, int4=True, streams=2,
                 name="long-rollout int4 store: 12 heads x d128, 3x880-token chunks, "
                      "1000 stored int4 chunks (r=0.5, g32 bf16 scales), extrapolated "
                      "query pose, window sink + 4 retrieved + 2 recent + current"),
}
CFG_SEED = {"tiny": 1, "1.3b": 2, "14b": 4, "int4": 5, "sweep": 3}
# Compression sweep: 60 evicted chunks x 30 layers of the 1.3B-class shape,
# every keep ratio and redundancy fraction below.
SWEEP = dict(H=12, D=128, T=880, F=3, units=1800, batch=300, ratios=(0.0, 0.25, 0.5, 1.0),
             p_red=(0.5, 0.7, 0.9),
             name="compression sweep: 60 chunks x 30 layers = 1800 units of 3x880 tokens x "
                  "12 heads x d128, r in {0, 0.25, 0.5, 1}, redundancy in {50, 70, 90}%")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="14b", choices=sorted(CONFIGS) + ["sweep"])
    ap.add_argument("--r", type=float, default=None, help="override the keep ratio")
    ap.add_argument("--score-mode", default="position", choices=["position", "anchor_mean"],
                    help="compression score: cosine to the anchor key at the same position "
                         "(default) or the mean cosine to every anchor key")
    ap.add_argument("--tier", action="store_true",
                    help="keep the bank in pinned host memory and stage retrieved chunks into "
                         "HBM slots from the extrapolated pose (host tier)")
    ap.add_argument("--tier-copy", default="engine", choices=["engine", "kernel"],
                    help="host tier staging copies: copy engine (default) or a copy kernel")
    ap.add_argument("--store", default="bf16", choices=["bf16", "int4"],
                    help="format of the compressed rows in the sweep")
    ap.add_argument("--sets", type=int, default=4, help="rotating input sets")
    ap.add_argument("--streams", type=int, default=None, choices=[1, 2],
                    help="streams of the timed step (default: the workload's)")
    ap.add_argument("--cpu-rows", type=int, default=512,
                    help="query rows per oracle attention call in the CPU baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate oracle work in the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-batches", action="store_true",
                    help="skip the batched 300-unit compression cells of the breakdown")
    ap.add_argument("--sweep-cells", default=None,
                    help="restrict the sweep to cells 'p_red:r,...' (e.g. 0.7:0.25,0.7:0.5)")
    ap.add_argument("--sample-units", type=int, default=30,
                    help="units per sweep cell checked against the oracle (CPU baseline leg)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, run one plain 1 GiB device copy (counter calibration)")
    return ap.parse_args()


def measured_traffic(cfg):
    """HBM bytes per attention call (read + write, forward + split merge) from
    the committed counter summary of this workload, or None when there is
    none or the attention source (kernels and launch planner) changed since
    it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{cfg}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    if h.hexdigest() != rec["sha256"]:
        return None
    return int(rec["attention_call_bytes"])


def compress_bytes(c, Lc, n_keep, int4=False):
    """Bytes one compression unit must move: the keys it scores (all F*T
    rows when a selection is needed, else the Lc kept ones), the kept values,
    and the Lc compressed K and V rows written (bf16, or int4 codes + bf16
    scale per 32 elements)."""
    R = c["H"] * c["D"] * 2
    N = (c["F"] - 1) * c["T"]
    s_read = c["F"] * c["T"] if 0 < n_keep < N else Lc
    out_row = (c["H"] * c["D"] // 2 + c["H"] * c["D"] // 32 * 2) if int4 else R
    return R * (s_read + Lc) + 2 * Lc * out_row


def algorithmic_bytes(c, Lc, n_keep, Nk):
    """Bytes the method must move (per call): compress and assemble."""
    R = c["H"] * c["D"] * 2
    comp = compress_bytes(c, Lc, n_keep)
    ret_rows = c["k"] * Lc
    other_rows = Nk - ret_rows
    if c["int4"]:
        hd = c["H"] * c["D"]
        per_bank_row = 2 * (hd * 0.5 + (hd // 32) * 2) + 2 * R
        asm = 4 * R * other_rows + per_bank_row * ret_rows
    else:
        asm = 4 * R * Nk
    return comp, asm


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only; --gpus {a.gpus} is not "
              "supported (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import ar_video_world_amd.wkv as w
    import wkv_synth as S

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if a.config == "sweep":
        sweep(a, torch, w, S, dev)
        return
    if a.tier:
        tier_bench(a, torch, w, S, dev)
        return
    c = dict(CONFIGS[a.config])
    if a.r is not None:
        c["r"] = a.r
    seed = CFG_SEED[a.config]
    H, D, T, F, r = c["H"], c["D"], c["T"], c["F"], c["r"]
    FT = F * T
    n_keep = w.wkv_keep_count(F, T, r)
    Lc = T + n_keep
    M, k, nrec, nsteps = c["M"], c["k"], c["n_recent"], c["S"]
    Nq = FT
    Nk = FT + k * Lc + nrec * FT + FT
    stream = torch.cuda.Stream()

    with torch.cuda.stream(stream):
        # ---- stored bank (compressed chunks) and its poses
        if c["int4"]:
            kp, vp, ks, vs = S.int4_bank(seed, M, Lc, H, D, device=dev)
            bank = {"k": kp, "v": vp, "k_scale": ks, "v_scale": vs}
        else:
            bk = torch.empty((M, Lc, H, D), dtype=torch.bfloat16, device=dev)
            bv = torch.empty_like(bk)
            for m in range(M):
                bk[m], bv[m] = S.segment_kv(seed, 100 + m, Lc, H, D, device=dev)
            bank = {"k": bk, "v": bv}
        walk = S.pose_walk(seed, M + 3)
        poses = walk[1:M + 1].contiguous().to(dev)
        if c["int4"]:
            qhist = [walk[M + 1].tolist(), walk[M + 2].tolist()]  # extrapolated
        else:
            qhist = [walk[M + 2].tolist()]

        # ---- rotating per-step input sets
        sets = []
        for i in range(a.sets):
            ek, ev = S.chunk_kv(seed, 1000 + i, 0, F, T, H, D, device=dev)
            segs = [S.segment_kv(seed, 2000 + 10 * i + j, FT, H, D, device=dev)
                    for j in range(nrec + 2)]
            qs = [S.queries(seed, s, Nq, H, D, device=dev, layer=i) for s in range(nsteps)]
            sets.append(dict(
                ek=ek, ev=ev, sink=segs[0], recent=segs[1:1 + nrec], cur=segs[-1], q=qs,
                ko=torch.empty((Lc, H, D), dtype=torch.bfloat16, device=dev),
                vo=torch.empty((Lc, H, D), dtype=torch.bfloat16, device=dev),
                kidx=torch.empty((Lc,), dtype=torch.int32, device=dev),
                wk=torch.empty((Nk, H, D), dtype=torch.bfloat16, device=dev),
                wv=torch.empty((Nk, H, D), dtype=torch.bfloat16, device=dev),
                out=torch.empty((Nq, H, D), dtype=torch.bfloat16, device=dev)))
        cws = torch.empty(max(w.wkv_compress_workspace_bytes(1, F, T, H, D, "anchor_mean"), 16),
                          dtype=torch.uint8, device=dev)
        aws = torch.empty(max(w.wkv_attention_workspace_bytes(Nq, Nk, H, D), 16),
                          dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()

        def step(i, ev=None):
            s = sets[i % len(sets)]
            if ev is not None:
                ev[0].record()
            w.wkv_compress_chunk(s["ek"], s["ev"], F, T, r, k_out=s["ko"], v_out=s["vo"],
                                 kept_idx=s["kidx"], ws=cws, score_mode=a.score_mode)
            if ev is not None:
                ev[1].record()
            idx, _, _ = w.wkv_pose_topk(poses, qhist, k, want_dist=False)
            if ev is not None:
                ev[2].record()
            w.wkv_assemble_window(s["sink"], bank, idx, s["recent"], s["cur"], H, D,
                                  win_k=s["wk"], win_v=s["wv"])
            if ev is not None:
                ev[3].record()
            for j in range(nsteps):
                if ev is not None:
                    ev[4 + 2 * j].record()
                w.wkv_chunk_attention(s["q"][j], s["wk"], s["wv"], out=s["out"], ws=aws)
                if ev is not None:
                    ev[5 + 2 * j].record()

        # ---- the pipelined step. The compression of a chunk and the pose
        # retrieval that follows it (the retrieval may pick the chunk just
        # stored) run on a side stream; the window assembly and attention of
        # that step run on the main stream after an event from the side
        # stream. The side stream takes step i+1's compression and retrieval
        # right after step i's attention is enqueued, so they run beside it.
        # Each compressed chunk goes to a buffer of its own (as an appended
        # bank slot would), so the side stream may run one step ahead. Two
        # retrieval slots alternate: step i+1 rewrites the slot step i-1's
        # assembly read, so it waits for that assembly.
        side = torch.cuda.Stream()
        ridx = [torch.empty((k,), dtype=torch.int32, device=dev) for _ in range(2)]
        ready = [torch.cuda.Event() for _ in range(2)]
        assembled = [torch.cuda.Event() for _ in range(2)]

        def front(i):
            s = sets[i % len(sets)]
            with torch.cuda.stream(side):
                if i >= 2:
                    side.wait_event(assembled[i % 2])
                w.wkv_compress_chunk(s["ek"], s["ev"], F, T, r, k_out=s["ko"], v_out=s["vo"],
                                     kept_idx=s["kidx"], ws=cws, score_mode=a.score_mode)
                w.wkv_pose_topk(poses, qhist, k, want_dist=False, out_idx=ridx[i % 2])
                ready[i % 2].record(side)

        def back(i):
            s = sets[i % len(sets)]
            stream.wait_event(ready[i % 2])
            w.wkv_assemble_window(s["sink"], bank, ridx[i % 2], s["recent"], s["cur"], H, D,
                                  win_k=s["wk"], win_v=s["wv"])
            assembled[i % 2].record(stream)
            for j in range(nsteps):
                w.wkv_chunk_attention(s["q"][j], s["wk"], s["wv"], out=s["out"], ws=aws)

        def run_pipelined(n):
            front(0)
            for i in range(n):
                back(i)
                if i + 1 < n:
                    front(i + 1)

        # The cyclic GC pass runs before the warmup, not between it and the
        # timed region: an idle gap there lets the GPU clock fall back.
        gc.collect()
        gc.disable()
        for i in range(a.warmup):
            step(i)
        run_pipelined(max(2, a.warmup))
        torch.cuda.synchronize()

        # ---- timed regions: wall clock over exactly K steps (no cyclic-GC
        # pass inside either), first on one stream, one call after another,
        # then pipelined on two (the first step's compression and retrieval
        # inside it). The workload's schedule gives the value; the other is
        # reported beside it.
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for i in range(a.steps):
            step(i)
        torch.cuda.synchronize()
        t3 = time.perf_counter()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run_pipelined(a.steps)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        gc.enable()
        wall_pipe = t1 - t0
        wall_serial = t3 - t2
        nstreams = a.streams or c["streams"]
        wall = wall_serial if nstreams == 1 else wall_pipe

        # ---- per-call durations, from HIP events on the launch stream
        nev = 4 + 2 * nsteps
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)]
               for _ in range(a.steps)]
        for i in range(a.steps):
            step(i, evs[i])
        torch.cuda.synchronize()
        t_comp = [e[0].elapsed_time(e[1]) for e in evs]
        t_pose = [e[1].elapsed_time(e[2]) for e in evs]
        t_asm = [e[2].elapsed_time(e[3]) for e in evs]
        t_att = [e[4 + 2 * j].elapsed_time(e[5 + 2 * j]) for e in evs for j in range(nsteps)]

        # ---- compression alone under each score mode and output format
        # (event-timed, same rotating sets)
        q4 = [(torch.empty((Lc, H, D // 2), dtype=torch.uint8, device=dev),
               torch.empty((Lc, H, D // 2), dtype=torch.uint8, device=dev),
               torch.empty((Lc, H, D // 32), dtype=torch.bfloat16, device=dev),
               torch.empty((Lc, H, D // 32), dtype=torch.bfloat16, device=dev))
              for _ in sets]
        comp_modes = {}
        for mode, fmt in (("position", "bf16"), ("anchor_mean", "bf16"), ("position", "int4"),
                          ("anchor_mean", "int4")):
            cev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(20)]
            for i in range(25):
                s = sets[i % len(sets)]
                if i >= 5:
                    cev[i - 5][0].record()
                if fmt == "bf16":
                    w.wkv_compress_chunk(s["ek"], s["ev"], F, T, r, k_out=s["ko"], v_out=s["vo"],
                                         kept_idx=s["kidx"], ws=cws, score_mode=mode)
                else:
                    kp, vp, ks, vs = q4[i % len(sets)]
                    w.wkv_compress_chunk_int4(s["ek"], s["ev"], F, T, r, k_packed=kp, v_packed=vp,
                                              k_scale=ks, v_scale=vs, kept_idx=s["kidx"],
                                              ws=cws, score_mode=mode)
                if i >= 5:
                    cev[i - 5][1].record()
            torch.cuda.synchronize()
            comp_modes[f"{mode}/{fmt}"] = statistics.fmean(e[0].elapsed_time(e[1]) for e in cev)
        del q4

        # ---- query-based retrieval, timed on its own: the mean key of the
        # chunk just compressed (store time), the mean query of the current
        # chunk, and the top-k over the bank's mean keys
        qr = None
        if not c["int4"]:
            km_bank = w.wkv_mean_rows(bank["k"])                      # [M, H, D] float64
            mws = torch.empty(max(w.wkv_mean_rows_workspace_bytes(1, max(Lc, Nq), H, D), 16),
                              dtype=torch.uint8, device=dev)
            kmo = torch.empty((1, H, D), dtype=torch.float64, device=dev)
            qmo = torch.empty((1, H, D), dtype=torch.float64, device=dev)
            qidx = torch.empty((k,), dtype=torch.int32, device=dev)
            qsc = torch.empty((M,), dtype=torch.float64, device=dev)
            qev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(20)]
            for i in range(25):
                s = sets[i % len(sets)]
                e = qev[i - 5] if i >= 5 else None
                if e:
                    e[0].record()
                w.wkv_mean_rows(s["ko"][None], out=kmo, ws=mws)
                if e:
                    e[1].record()
                w.wkv_mean_rows(s["q"][0][None], out=qmo, ws=mws)
                if e:
                    e[2].record()
                w.wkv_query_topk(km_bank, qmo[0], k, out_idx=qidx, scores=qsc)
                if e:
                    e[3].record()
            torch.cuda.synchronize()
            t_mk = statistics.fmean(e[0].elapsed_time(e[1]) for e in qev)
            t_mq = statistics.fmean(e[1].elapsed_time(e[2]) for e in qev)
            t_tk = statistics.fmean(e[2].elapsed_time(e[3]) for e in qev)
            # The mean key as a by-product of compression: the same call with
            # and without its key_mean output, alternating
            kws = torch.empty(max(w.wkv_compress_workspace_bytes(1, F, T, H, D, a.score_mode,
                                                                 True), 16),
                              dtype=torch.uint8, device=dev)
            kev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(20)]
            for i in range(25):
                s = sets[i % len(sets)]
                e = kev[i - 5] if i >= 5 else None
                if e:
                    e[0].record()
                w.wkv_compress_chunk(s["ek"], s["ev"], F, T, r, k_out=s["ko"], v_out=s["vo"],
                                     kept_idx=s["kidx"], ws=kws, score_mode=a.score_mode)
                if e:
                    e[1].record()
                w.wkv_compress_chunk(s["ek"], s["ev"], F, T, r, k_out=s["ko"], v_out=s["vo"],
                                     kept_idx=s["kidx"], ws=kws, score_mode=a.score_mode,
                                     key_mean=kmo[0])
                if e:
                    e[2].record()
            torch.cuda.synchronize()
            t_c0 = statistics.fmean(e[0].elapsed_time(e[1]) for e in kev)
            t_c1 = statistics.fmean(e[1].elapsed_time(e[2]) for e in kev)
            R = H * D * 2
            qr = {"mean_key_us": round(t_mk * 1e3, 2),
                  "mean_key_GBps": round(Lc * R / (t_mk * 1e-3) / 1e9, 1),
                  "compress_us": round(t_c0 * 1e3, 2),
                  "compress_with_mean_key_us": round(t_c1 * 1e3, 2),
                  "mean_query_us": round(t_mq * 1e3, 2),
                  "mean_query_GBps": round(Nq * R / (t_mq * 1e-3) / 1e9, 1),
                  "query_topk_us": round(t_tk * 1e3, 2)}
            del km_bank, mws, kws

        # ---- the window read in place (bf16 banks): the same serial steps
        # with wkv_chunk_attention_window in place of assembly + attention,
        # on the same sets; and that attention call alone, event-timed
        inplace = None
        if not c["int4"]:
            nk_pad = sum(64 * ((n + 63) // 64) for n in [FT] + [Lc] * k + [FT] * nrec + [FT])
            wws = torch.empty(max(w.wkv_attention_window_workspace_bytes(Nq, nk_pad, H, D), 256),
                              dtype=torch.uint8, device=dev)

            def step_in_place(i, ev=None):
                s = sets[i % len(sets)]
                w.wkv_compress_chunk(s["ek"], s["ev"], F, T, r, k_out=s["ko"], v_out=s["vo"],
                                     kept_idx=s["kidx"], ws=cws, score_mode=a.score_mode)
                idx, _, _ = w.wkv_pose_topk(poses, qhist, k, want_dist=False)
                for j in range(nsteps):
                    if ev is not None:
                        ev[2 * j].record()
                    w.wkv_chunk_attention_window(s["q"][j], s["sink"], bank, idx, s["recent"],
                                                 s["cur"], out=s["out"], ws=wws)
                    if ev is not None:
                        ev[2 * j + 1].record()

            for i in range(a.warmup):
                step_in_place(i)
            torch.cuda.synchronize()
            t4 = time.perf_counter()
            for i in range(a.steps):
                step_in_place(i)
            torch.cuda.synchronize()
            t5 = time.perf_counter()
            iev = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * nsteps)]
                   for _ in range(a.steps)]
            for i in range(a.steps):
                step_in_place(i, iev[i])
            torch.cuda.synchronize()
            t_win = statistics.fmean(e[2 * j].elapsed_time(e[2 * j + 1]) for e in iev
                                     for j in range(nsteps))
            # the two-stream pipeline of the timed step, with the in-place
            # attention in place of assembly + attention: the retrieval slot
            # step i+1 rewrites is free once step i-1's attention has read it
            def back_in_place(i):
                s = sets[i % len(sets)]
                stream.wait_event(ready[i % 2])
                for j in range(nsteps):
                    w.wkv_chunk_attention_window(s["q"][j], s["sink"], bank, ridx[i % 2],
                                                 s["recent"], s["cur"], out=s["out"], ws=wws)
                assembled[i % 2].record(stream)

            def run_pipelined_in_place(n):
                front(0)
                for i in range(n):
                    back_in_place(i)
                    if i + 1 < n:
                        front(i + 1)

            run_pipelined_in_place(max(2, a.warmup))
            torch.cuda.synchronize()
            t6 = time.perf_counter()
            run_pipelined_in_place(a.steps)
            torch.cuda.synchronize()
            t7 = time.perf_counter()
            inplace = {"ms_per_step": round((t7 - t6) / a.steps * 1e3, 4),
                       "serial_ms_per_step": round((t5 - t4) / a.steps * 1e3, 4),
                       "attention_window_us": round(t_win * 1e3, 2),
                       "attention_window_TFLOPs": round(4.0 * Nq * Nk * D * H / (t_win * 1e-3)
                                                        / 1e12, 1),
                       "padded_keys": nk_pad}
            del wws

        # ---- pose top-k with full rotations (the walk's yaw as z-axis
        # quaternions), timed on its own
        P8 = torch.zeros((M, 8), dtype=torch.float32, device=dev)
        P8[:, :3] = poses[:, :3]
        P8[:, 3] = torch.cos(poses[:, 3].double() / 2).float()
        P8[:, 6] = torch.sin(poses[:, 3].double() / 2).float()
        qq = qhist[-1]
        q8 = [qq[0], qq[1], qq[2], math.cos(qq[3] / 2), 0.0, 0.0, math.sin(qq[3] / 2)]
        sidx = torch.empty((k,), dtype=torch.int32, device=dev)
        pev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(20)]
        for i in range(25):
            if i >= 5:
                pev[i - 5][0].record()
            w.wkv_pose_topk_so3(P8, q8, k, want_dist=False, out_idx=sidx)
            if i >= 5:
                pev[i - 5][1].record()
        torch.cuda.synchronize()
        t_so3 = statistics.fmean(e[0].elapsed_time(e[1]) for e in pev)

        copy_gbps = _copy_probe(torch, dev) if a.copy_probe else None

    # batched compression of 300 units beside the step (timed cells)
    batches = None if a.no_batches else compress_batches(a, torch, w, S, dev)

    ms_per_step = wall / a.steps * 1e3
    comp_b, asm_b = algorithmic_bytes(c, Lc, n_keep, Nk)
    flops = 4.0 * Nq * Nk * D * H
    mean = statistics.fmean
    att_ms = mean(t_att)
    att_tflops = flops / (att_ms * 1e-3) / 1e12
    comp_ms, asm_ms, pose_ms = mean(t_comp), mean(t_asm), mean(t_pose)
    splits = w.wkv_attention_workspace_bytes(Nq, Nk, H, D) > 0

    rec = {
        "metric": METRIC,
        "value": round(a.steps / wall, 3),
        "unit": "chunk-steps/s (one step = compress + pose top-k + assemble + "
                f"{nsteps} attention pass{'es' if nsteps > 1 else ''})",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded rho-mixture keys, N(0,1) values and queries, "
                "random-walk poses)",
        "config": {"workload": c["name"], "heads": H, "head_dim": D, "tokens_per_frame": T,
                   "frames_per_chunk": F, "keep_ratio": r, "score_mode": a.score_mode,
                   "compressed_rows": Lc,
                   "stored_chunks": M, "retrieved": k, "window_keys": Nk, "queries": Nq,
                   "denoise_steps": nsteps, "int4_bank": c["int4"], "parallelism": "none",
                   "input_sets": a.sets,
                   "streams": ("1 (every call in order)" if nstreams == 1 else
                               "2 (compression and retrieval of step i+1 beside step i's "
                               "attention)")},
        "breakdown": {
            "serial_ms_per_step": round(wall_serial / a.steps * 1e3, 4),
            "pipelined_ms_per_step": round(wall_pipe / a.steps * 1e3, 4),
            "compress_us": round(comp_ms * 1e3, 2),
            "compress_GBps": round(comp_b / (comp_ms * 1e-3) / 1e9, 1),
            "compress_bytes": comp_b,
            "compress_modes": {m: {"us": round(v * 1e3, 2),
                                   "bytes": compress_bytes(c, Lc, n_keep, m.endswith("int4")),
                                   "GBps": round(compress_bytes(c, Lc, n_keep, m.endswith("int4"))
                                                 / (v * 1e-3) / 1e9, 1)}
                               for m, v in comp_modes.items()},
            "pose_topk_us": round(pose_ms * 1e3, 2),
            "pose_topk_so3_us": round(t_so3 * 1e3, 2),
            "query_retrieval": qr,
            "assemble_us": round(asm_ms * 1e3, 2),
            "assemble_GBps": round(asm_b / (asm_ms * 1e-3) / 1e9, 1),
            "assemble_bytes": int(asm_b),
            "attention_us": round(att_ms * 1e3, 2),
            "attention_TFLOPs": round(att_tflops, 1),
            "attention_flop": flops,
            "attention_split_keys": splits,
            "event_step_ms": round(comp_ms + pose_ms + asm_ms + att_ms * nsteps, 4),
            "percentiles_us": {name: {"p10": round(np.percentile(v, 10) * 1e3, 2),
                                      "p50": round(np.percentile(v, 50) * 1e3, 2),
                                      "p90": round(np.percentile(v, 90) * 1e3, 2)}
                               for name, v in (("compress", t_comp), ("pose_topk", t_pose),
                                               ("assemble", t_asm), ("attention", t_att))},
            "copy_probe_GBps": None if copy_gbps is None else round(copy_gbps, 1),
            "window_in_place": inplace,
            "compress_batches": batches,
        },
        "roofline": {
            "kernel": "wkv_chunk_attention" + (" (fwd + split merge)" if splits else ""),
            "bound": "mfma",
            "achieved": round(att_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(att_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(a.config) if a.r is None else None,
        },
        "cpu_baseline": None,
    }

    if not a.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(a, c, sets[0], bank, poses, qhist, Nq, Nk, Lc)
    print(json.dumps(rec), flush=True)


def _copy_probe(torch, dev):
    """One plain 1 GiB device-to-device copy (the HBM counters' calibration:
    it reads and writes exactly 2^30 bytes). Returns its GB/s."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    ce0, ce1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ce0.record()
    dst.copy_(src)
    ce1.record()
    torch.cuda.synchronize()
    gbps = 2 * (1 << 30) / (ce0.elapsed_time(ce1) * 1e-3) / 1e9
    del src, dst
    return gbps


def _compress_outputs(torch, B, Lc, H, D, store, dev):
    """Output buffers of one batched compression call."""
    ki = torch.empty((B, Lc), dtype=torch.int32, device=dev)
    if store == "int4":
        ko = torch.empty((B, Lc, H, D // 2), dtype=torch.uint8, device=dev)
        ks = torch.empty((B, Lc, H, D // 32), dtype=torch.bfloat16, device=dev)
        return dict(kp=ko, vp=torch.empty_like(ko), ks=ks, vs=torch.empty_like(ks), ki=ki)
    ko = torch.empty((B, Lc, H, D), dtype=torch.bfloat16, device=dev)
    return dict(ko=ko, vo=torch.empty_like(ko), ki=ki)


def _compress_call(w, kin, vin, F, T, r, out, ws, score_mode):
    if "kp" in out:
        w.wkv_compress_chunk_int4(kin, vin, F, T, r, k_packed=out["kp"], v_packed=out["vp"],
                                  k_scale=out["ks"], v_scale=out["vs"], kept_idx=out["ki"],
                                  ws=ws, score_mode=score_mode, key_mean=out.get("km"))
    else:
        w.wkv_compress_chunk(kin, vin, F, T, r, k_out=out["ko"], v_out=out["vo"],
                             kept_idx=out["ki"], ws=ws, score_mode=score_mode,
                             key_mean=out.get("km"))


def _time_compress(torch, w, kin, vin, F, T, r, out, ws, score_mode, calls, warm, reps):
    """Mean ms of `calls` back-to-back batched compression calls, event-timed
    on the current stream (median of `reps` repetitions after `warm`)."""
    for _ in range(warm):
        for _ in range(calls):
            _compress_call(w, kin, vin, F, T, r, out, ws, score_mode)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(calls):
            _compress_call(w, kin, vin, F, T, r, out, ws, score_mode)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    return statistics.median(ts)


def compress_batches(a, torch, w, S, dev):
    """Batched World Compression beside the step: one call over 300 resident
    units of the 1.3B-class chunk shape (3x880 tokens x 12 heads x d128, 70%
    redundancy; 4.9 GB of keys and values, far past the last-level cache),
    bf16 and int4 stores at r = 0.25 and 0.5, position score, each also with
    the mean key of every unit written beside it; GB/s of algorithmic bytes
    (the mean key's 12 KiB per unit aside) from HIP events on the launch
    stream."""
    c = SWEEP
    H, D, T, F, B = c["H"], c["D"], c["T"], c["F"], c["batch"]
    cells = {}
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        kin = torch.empty((B, F * T, H, D), dtype=torch.bfloat16, device=dev)
        vin = torch.empty_like(kin)
        for u in range(B):
            kin[u], vin[u] = S.chunk_kv(3, u, 1, F, T, H, D, p_red=0.7, device=dev)
        ws = torch.empty(max(w.wkv_compress_workspace_bytes(B, F, T, H, D, "position", True),
                             16), dtype=torch.uint8, device=dev)
        for store in ("bf16", "int4"):
            for r in (0.25, 0.5):
                n_keep = w.wkv_keep_count(F, T, r)
                Lc = T + n_keep
                out = _compress_outputs(torch, B, Lc, H, D, store, dev)
                for km in (False, True):
                    out["km"] = (torch.empty((B, H, D), dtype=torch.float64, device=dev)
                                 if km else None)
                    ms = _time_compress(torch, w, kin, vin, F, T, r, out, ws, "position", 1, 2,
                                        7)
                    nbytes = compress_bytes(c, Lc, n_keep, store == "int4") * B
                    gbps = nbytes / (ms * 1e-3) / 1e9
                    cells[f"{store} r={r}" + (" +mean key" if km else "")] = {
                        "ms": round(ms, 4), "GB": round(nbytes / 1e9, 3), "GBps": round(gbps, 1),
                        "frac": round(gbps / PEAK_HBM_GBPS, 4)}
                del out
        del kin, vin, ws
    torch.cuda.synchronize()
    return {"workload": f"{B} units of 3x880 tokens x 12 heads x d128 per call, 70% "
                        "redundancy, position score", "cells": cells}


def sweep(a, torch, w, S, dev):
    """wkv_compress_chunk over all 1800 units for every (redundancy, r) cell.
    300 distinct units are resident per redundancy fraction; one step
    compresses all 1800 units as 6 batched calls over them (each call streams
    4.9 GB of keys and values, far past the last-level cache). After the
    timing, the oracle compresses a few sampled units of every cell (the
    first, the last and evenly spread ones) on the host: its time is the CPU
    baseline and its outputs give each cell's exactness (kept sets outside the
    1e-6 band around the selection threshold, band sizes, and bitwise outputs)."""
    import numpy as np
    c = SWEEP
    H, D, T, F = c["H"], c["D"], c["T"], c["F"]
    B, nb = c["batch"], c["units"] // c["batch"]
    only = None
    if a.sweep_cells:
        only = {(float(x.split(":")[0]), float(x.split(":")[1])) for x in a.sweep_cells.split(",")}
    ns = max(0, min(a.sample_units, B))
    sample = sorted({0, B - 1} | {int(round(i * (B - 1) / max(ns - 1, 1))) for i in range(ns)}) \
        if ns > 0 and not a.no_cpu_baseline else []
    stream = torch.cuda.Stream()
    cells, samples = [], []

    def bits(t):
        if t.dtype == torch.bfloat16:
            t = t.view(torch.int16)
        return t.cpu().numpy().view(np.uint16) if t.dtype == torch.int16 else t.cpu().numpy()

    with torch.cuda.stream(stream):
        kin = torch.empty((B, F * T, H, D), dtype=torch.bfloat16, device=dev)
        vin = torch.empty_like(kin)
        ws = torch.empty(max(w.wkv_compress_workspace_bytes(B, F, T, H, D, a.score_mode), 16),
                         dtype=torch.uint8, device=dev)
        for pi, p_red in enumerate(c["p_red"]):
            if only is not None and not any(p == p_red for p, _ in only):
                continue
            for u in range(B):
                kin[u], vin[u] = S.chunk_kv(3, u, pi, F, T, H, D, p_red=p_red, device=dev)
            src = {u: (bits(kin[u]), bits(vin[u])) for u in sample}
            for r in c["ratios"]:
                if only is not None and (p_red, r) not in only:
                    continue
                n_keep = w.wkv_keep_count(F, T, r)
                Lc = T + n_keep
                out = _compress_outputs(torch, B, Lc, H, D, a.store, dev)
                ms = _time_compress(torch, w, kin, vin, F, T, r, out, ws, a.score_mode, nb,
                                    max(1, a.warmup // 5), max(1, a.steps // 10))
                unit_bytes = compress_bytes(c, Lc, n_keep, a.store == "int4")
                gbps = unit_bytes * c["units"] / (ms * 1e-3) / 1e9
                cells.append({"p_red": p_red, "r": r, "ms": round(ms, 3),
                              "GB": round(unit_bytes * c["units"] / 1e9, 2),
                              "GBps": round(gbps, 1), "frac": round(gbps / PEAK_HBM_GBPS, 4)})
                for u in sample:
                    samples.append(dict(cell=len(cells) - 1, unit=u, r=r, src=src[u],
                                        out={n: bits(t[u]) for n, t in out.items()}))
                del out
        del kin, vin, ws
        if a.copy_probe:
            _copy_probe(torch, dev)
    main_cell = next((x for x in cells if x["p_red"] == 0.7 and x["r"] == 0.5), cells[0])
    rec = {
        "metric": METRIC,
        "value": main_cell["GBps"],
        "unit": "GB/s (wkv_compress_chunk over 1800 units, algorithmic bytes, r=0.5, 70% redundancy)",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": main_cell["ms"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 in, f64 scores",
        "data": "synthetic (seeded rho-mixture keys, N(0,1) values)",
        "config": {"workload": c["name"], "heads": H, "head_dim": D, "tokens_per_frame": T,
                   "frames_per_chunk": F, "units": c["units"], "batch": B,
                   "score_mode": a.score_mode, "store": a.store, "parallelism": "none"},
        "sweep": cells,
        "roofline": {"kernel": "wkv_compress_chunk (score + select + gather)", "bound": "hbm",
                     "achieved": main_cell["GBps"], "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": main_cell["frac"], "traffic": None},
        "cpu_baseline": None,
    }
    if samples:
        rec["cpu_baseline"] = sweep_cpu_baseline(a, c, cells, samples)
    print(json.dumps(rec), flush=True)


def sweep_cpu_baseline(a, c, cells, samples):
    """The oracle, as it stands, on the sampled units of every sweep cell:
    its per-unit time (scaled to the 1800-unit step) and each cell's
    exactness against the GPU outputs of those units."""
    import numpy as np
    import threadpoolctl

    from oracle import wkv_oracle as O

    F, T = c["F"], c["T"]
    t_all = 0.0
    for smp in samples:
        kb, vb = smp["src"]
        r = smp["r"]
        t0 = time.perf_counter()
        if a.store == "int4":
            ok, ov, oks, ovs, oi, osc = O.compress_chunk_int4(kb, vb, F, T, r,
                                                              score_mode=a.score_mode)
            ref = {"kp": ok, "vp": ov, "ks": oks, "vs": ovs}
        else:
            ok, ov, oi, osc = O.compress_chunk(kb, vb, F, T, r, score_mode=a.score_mode)
            ref = {"ko": ok, "vo": ov}
        t_all += time.perf_counter() - t0
        g = smp["out"]
        n_keep = O.keep_count(F, T, r)
        N = (F - 1) * T
        band = set()
        if 0 < n_keep < N:
            key = np.where(np.isnan(osc), np.inf, osc)
            srt = np.sort(key)
            thr = 0.5 * (srt[n_keep - 1] + srt[n_keep])
            band = set(np.nonzero(np.abs(key - thr) <= 1e-6)[0].tolist())
        okept = set((oi[T:] - T).tolist())
        gkept = set((g["ki"][T:] - T).tolist())
        outside_ok = (okept - band) == (gkept - band)
        ndiff = len((okept ^ gkept) & band)
        bitwise = ndiff == 0 and np.array_equal(g["ki"], oi) and all(
            np.array_equal(g[n], ref[n]) for n in ref)
        cell = cells[smp["cell"]]
        st = cell.setdefault("exactness", {"units_checked": 0, "band_tokens": 0,
                                           "band_differing": 0, "kept_exact_outside_band": True,
                                           "outputs_bitwise": True})
        st["units_checked"] += 1
        st["band_tokens"] += len(band)
        st["band_differing"] += ndiff
        st["kept_exact_outside_band"] &= bool(outside_ok)
        st["outputs_bitwise"] &= bool(bitwise)
    per_unit = t_all / len(samples)
    blas = [p for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p["num_threads"] for p in blas] or [1])
    return {
        "value": round(1.0 / (per_unit * c["units"]), 6),
        "unit": "sweep cells/s (1800 units per cell)",
        "cores": threads,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"numpy fp64 oracle compression of {len(samples)} sampled units "
                   f"({len(samples) // max(len(cells), 1)} per cell, first and last included), "
                   f"{per_unit:.3f} s per unit, scaled to the 1800 units of one cell"),
        "seconds": round(t_all, 3),
    }


def tier_bench(a, torch, w, S, dev):
    """The hot path with the bank in pinned host memory (WorldPager: int4
    store in pinned DRAM, next retrieval set staged from the extrapolated
    pose, stale reuse on a miss). Per chunk step t on the compute stream:
    compress, wait for the staging of step t, pose top-k on the true pose,
    resolve against the staged slots, assemble from the staging bank,
    attention. The host plans step t + 1's set from the extrapolated pose
    (the pose is known before compute) and queues the copies of the chunks
    not yet staged on a copy stream, after step t's assembly, so they overlap
    step t's attention. The query
    walks back along the bank's own trajectory (a revisit). The same steps
    with the bank resident in HBM and direct retrieval are timed beside it."""
    import numpy as np
    c = dict(CONFIGS[a.config])
    if a.r is not None:
        c["r"] = a.r
    seed = CFG_SEED[a.config]
    H, D, T, F, r = c["H"], c["D"], c["T"], c["F"], c["r"]
    FT = F * T
    Lc = T + w.wkv_keep_count(F, T, r)
    M, k, nrec, nsteps = c["M"], c["k"], c["n_recent"], c["S"]
    Nq, Nk = FT, FT + k * Lc + nrec * FT + FT
    # staging holds the next set beside the current retrieved and predicted sets
    n_slots = 3 * k + 2
    copy_mode = w.WKV_TIER_COPY_ENGINE if a.tier_copy == "engine" else w.WKV_TIER_COPY_KERNEL
    # compute and copy streams (both at the default priority)
    cs, xs = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(cs):
        if c["int4"]:
            kp, vp, ksc, vsc = S.int4_bank(seed, M, Lc, H, D, device=dev)
            bank = {"k": kp, "v": vp, "k_scale": ksc, "v_scale": vsc}
        else:
            bk = torch.empty((M, Lc, H, D), dtype=torch.bfloat16, device=dev)
            bv = torch.empty_like(bk)
            for m in range(M):
                bk[m], bv[m] = S.segment_kv(seed, 100 + m, Lc, H, D, device=dev)
            bank = {"k": bk, "v": bv}
        torch.cuda.synchronize()
        host = {n: torch.empty(t.shape, dtype=t.dtype, pin_memory=True).copy_(t)
                for n, t in bank.items()}
        staging = {n: torch.empty((n_slots,) + tuple(t.shape[1:]), dtype=t.dtype, device=dev)
                   for n, t in bank.items()}
        chunk_bytes = sum(t[0].numel() * t.element_size() for t in host.values())
        walk = S.pose_walk(seed, M + 3)
        poses = walk[1:M + 1].contiguous().to(dev)
        nstep_all = a.warmup + a.steps + 2
        # a smooth revisit: a 5-point moving average of the bank's own path,
        # walked backwards (and forwards again at the ends)
        path = walk[1:M + 1].double()
        sm = torch.stack([path[max(0, i - 2):i + 3].mean(0) for i in range(M)]).float()
        order = list(range(M - 1, -1, -1)) + list(range(1, M - 1))
        traj = [sm[order[t % len(order)]].tolist() for t in range(nstep_all + 1)]
        ck, cv = S.chunk_kv(seed, 1000, 0, F, T, H, D, device=dev)
        segs = [S.segment_kv(seed, 2000 + j, FT, H, D, device=dev) for j in range(nrec + 2)]
        qs = [S.queries(seed, s_, Nq, H, D, device=dev) for s_ in range(nsteps)]
        ko = torch.empty((Lc, H, D), dtype=torch.bfloat16, device=dev)
        vo = torch.empty_like(ko)
        kidx = torch.empty((Lc,), dtype=torch.int32, device=dev)
        wk = torch.empty((Nk, H, D), dtype=torch.bfloat16, device=dev)
        wv = torch.empty_like(wk)
        out = torch.empty((Nq, H, D), dtype=torch.bfloat16, device=dev)
        cws = torch.empty(max(w.wkv_compress_workspace_bytes(1, F, T, H, D), 16),
                          dtype=torch.uint8, device=dev)
        aws = torch.empty(max(w.wkv_attention_workspace_bytes(Nq, Nk, H, D), 16),
                          dtype=torch.uint8, device=dev)
        # device slot tables, one per step parity: the copy stream writes the
        # next step's table while the current step may still read its own
        dsc = [torch.empty((n_slots,), dtype=torch.int32, device=dev) for _ in range(2)]
        dps = [torch.empty((64,), dtype=torch.int32, device=dev) for _ in range(2)]
        slots = torch.empty((k,), dtype=torch.int32, device=dev)
        # misses of every step, written in place by the resolve (no per-step
        # allocation: torch's allocator would synchronise on stream events)
        miss = torch.zeros((nstep_all + 1, 4), dtype=torch.int32, device=dev)   # 16-byte rows
        tier = w.Tier(n_slots)
        torch.cuda.synchronize()

    stats = {"copies": 0, "misses": [], "stall": [], "att": []}

    poses_host = walk[1:M + 1].contiguous().numpy()
    import ctypes as C
    host_b, stg_bank_b = w._bank_struct(host), w._bank_struct(staging)
    hist_arr = (w.wkv_pose * 2)()
    ids_arr = (C.c_int32 * max(k, 1))()
    n_cp = C.c_int32(0)
    k_eff = min(k, M)

    pred = {}    # step -> predicted ids (host)

    def host_topk(hist):
        for i_, p_ in enumerate(hist):
            hist_arr[i_].x, hist_arr[i_].y, hist_arr[i_].z, hist_arr[i_].yaw = p_
        st_ = w._pose_host(poses_host.ctypes.data, M, hist_arr, len(hist), k,
                           C.cast(ids_arr, C.c_void_p), None)
        if st_ != 0:
            raise RuntimeError(w.wkv_last_error())
        return [int(ids_arr[i_]) for i_ in range(k_eff)]

    def stage(t_next, hist, keep, timed):
        """Plan the staging set of step t_next on the host from its
        extrapolated pose (the pose is known before compute) and enqueue its
        copies on the copy stream. The chunks still read by enqueued steps
        are kept, and the table goes to the buffer of t_next's parity, so the
        copy stream waits for nothing; returns the event marking it done."""
        ids = host_topk(hist)
        pred[t_next] = ids
        keep_arr = (C.c_int32 * max(len(keep), 1))(*keep)
        st_ = w._tier_prefetch(C.byref(tier.t), C.cast((C.c_int32 * k_eff)(*ids), C.c_void_p),
                               k_eff, C.cast(keep_arr, C.c_void_p), len(keep),
                               C.byref(host_b), C.byref(stg_bank_b), H, D, copy_mode,
                               C.c_void_p(dsc[t_next % 2].data_ptr()),
                               C.c_void_p(dps[t_next % 2].data_ptr()), C.byref(n_cp),
                               C.c_void_p(xs.cuda_stream))
        if st_ != 0:
            raise RuntimeError(w.wkv_last_error())
        if timed:
            stats["copies"] += n_cp.value
        ready = torch.cuda.Event()
        ready.record(xs)
        return ready

    # Prepared C calls: the step's arguments are marshalled once, so the host
    # cost per step is the library's, not the Python wrappers' (the staging
    # path must enqueue each step behind a host decision, so it cannot run
    # many steps ahead of the GPU as the resident path does).
    P = C.c_void_p
    cs_h, xs_h = P(cs.cuda_stream), P(xs.cuda_stream)
    idx = torch.empty((k,), dtype=torch.int32, device=dev)
    qpose = (w.wkv_pose * 1)()
    sk_, cur_ = w._seg(segs[0]), w._seg(segs[-1])
    rec_ = (w.wkv_segment * max(nrec, 1))(*[w._seg(p_) for p_ in segs[1:1 + nrec]])
    stg_b, bank_b = w._bank_struct(staging), w._bank_struct(bank)
    comp_args = (P(ck.data_ptr()), P(cv.data_ptr()), 1, F, T, H, D, float(r), 0,
                 P(ko.data_ptr()), P(vo.data_ptr()), P(kidx.data_ptr()), None, None,
                 P(cws.data_ptr()), cws.numel(), cs_h)
    attn_args = [(P(qs[j].data_ptr()), P(wk.data_ptr()), P(wv.data_ptr()), Nq, Nk, H, D, 0.0,
                  P(out.data_ptr()), None, P(aws.data_ptr()), aws.numel(), cs_h)
                 for j in range(nsteps)]

    def call(f, *args):
        st_ = f(*args)
        if st_ != 0:
            raise RuntimeError(w.wkv_last_error())

    def set_pose(p_):
        qpose[0].x, qpose[0].y, qpose[0].z, qpose[0].yaw = p_

    asm_prev = [None]

    def step_tier(t, ready, timed):
        """Enqueue step t, then plan and enqueue the staging of step t + 1."""
        tev = [torch.cuda.Event(enable_timing=True) for _ in range(4)] if timed else None
        call(w._compress, *comp_args)
        if timed:
            tev[0].record(cs)
        cs.wait_event(ready)
        if timed:
            tev[1].record(cs)
        set_pose(traj[t])
        call(w._pose_topk, P(poses.data_ptr()), M, qpose, 1, k, P(idx.data_ptr()), None, None,
             cs_h)
        call(w._tier_resolve, P(idx.data_ptr()), k_eff, P(dsc[t % 2].data_ptr()), n_slots,
             P(dps[t % 2].data_ptr()), P(slots.data_ptr()), P(miss[t].data_ptr()), cs_h)
        call(w._assemble, C.byref(sk_), C.byref(stg_b), P(slots.data_ptr()), k_eff, rec_,
             nrec, C.byref(cur_), H, D, P(wk.data_ptr()), P(wv.data_ptr()), Nk, cs_h)
        if timed:
            stats["misses"].append(t)
        asm = torch.cuda.Event()
        asm.record(cs)
        for j in range(nsteps):
            if timed and j == 0:
                tev[2].record(cs)
            call(w._attn, *attn_args[j])
        if timed:
            tev[3].record(cs)
            stats["stall"].append(tev)
        # Step t - 1 has finished reading the staging bank and its table
        # buffer once its assembly is done: the host stays one step ahead.
        if asm_prev[0] is not None:
            asm_prev[0].synchronize()
        asm_prev[0] = asm
        # chunks step t may still read: its retrieved set and its prediction
        keep = sorted(set(host_topk([traj[t]])) | set(pred.get(t, [])))
        # the pose of step t + 1 extrapolated from those of steps t - 1 and t
        hist = [traj[t - 1], traj[t]] if t > 0 else [traj[t]]
        return stage(t + 1, hist, keep, timed)

    def step_hbm(t):
        call(w._compress, *comp_args)
        set_pose(traj[t])
        call(w._pose_topk, P(poses.data_ptr()), M, qpose, 1, k, P(idx.data_ptr()), None, None,
             cs_h)
        call(w._assemble, C.byref(sk_), C.byref(bank_b), P(idx.data_ptr()), min(k, M), rec_,
             nrec, C.byref(cur_), H, D, P(wk.data_ptr()), P(wv.data_ptr()), Nk, cs_h)
        for j in range(nsteps):
            call(w._attn, *attn_args[j])

    # the loop makes a few Python objects per step; a cyclic-GC pass over the
    # large bank setup (tens of ms) would land inside the timed region. It
    # runs before the warmup: an idle gap after it lets the GPU clock fall.
    gc.collect()
    gc.disable()
    # step 0's set is staged from its own pose before the loop
    ready = stage(0, [traj[0]], [], False)
    for t in range(a.warmup):
        ready = step_tier(t, ready, False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    host_s = 0.0
    for t in range(a.warmup, a.warmup + a.steps):
        h0 = time.perf_counter()
        ready = step_tier(t, ready, True)
        host_s += time.perf_counter() - h0
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    for t in range(a.warmup):
        step_hbm(t)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for t in range(a.warmup, a.warmup + a.steps):
        step_hbm(t)
    torch.cuda.synchronize()
    wall_hbm = time.perf_counter() - t1
    gc.enable()

    stall_us = [e[0].elapsed_time(e[1]) * 1e3 for e in stats["stall"]]
    # step period on the compute stream, from one step's compression to the
    # next: its median is robust to a rare host hiccup in the wall clock
    period_ms = [a_[0].elapsed_time(b_[0]) for a_, b_ in zip(stats["stall"], stats["stall"][1:])]
    att_ms = statistics.fmean(e[2].elapsed_time(e[3]) for e in stats["stall"]) / nsteps
    misses = int(miss[stats["misses"], 0].sum().item())
    flops = 4.0 * Nq * Nk * D * H
    att_tflops = flops / (att_ms * 1e-3) / 1e12
    rec = {
        "metric": METRIC,
        "value": round(a.steps / wall, 3),
        "unit": "chunk-steps/s (one step = compress + pose top-k + tier resolve + assemble from "
                f"HBM staging + {nsteps} attention pass{'es' if nsteps > 1 else ''}; staging "
                "copies overlap the attention)",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(wall / a.steps * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded bank and queries; the query pose walks back along the bank's "
                "own trajectory)",
        "config": {"workload": c["name"] + f"; bank in pinned host memory, staged through "
                                           f"{n_slots} HBM slots by {a.tier_copy} copies",
                   "heads": H, "head_dim": D, "tier_copy": a.tier_copy,
                   "stored_chunks": M, "retrieved": k, "staging_slots": n_slots,
                   "int4_bank": c["int4"], "window_keys": Nk, "queries": Nq,
                   "parallelism": "none"},
        "breakdown": {
            "step_period_ms_p50": round(float(np.percentile(period_ms, 50)), 4),
            "step_period_ms_p90": round(float(np.percentile(period_ms, 90)), 4),
            "step_period_ms_max": round(max(period_ms), 4),
            "step_period_argmax": int(np.argmax(period_ms)),
            "hbm_resident_ms_per_step": round(wall_hbm / a.steps * 1e3, 4),
            "host_enqueue_ms_per_step": round(host_s / a.steps * 1e3, 4),
            "chunks_copied_per_step": round(stats["copies"] / a.steps, 3),
            "copy_MB_per_step": round(stats["copies"] * chunk_bytes / a.steps / 1e6, 3),
            "miss_rate": round(misses / (a.steps * min(k, M)), 4),
            "stall_us_mean": round(statistics.fmean(stall_us), 2),
            "stall_us_max": round(max(stall_us), 2),
            "attention_us": round(att_ms * 1e3, 2),
        },
        "roofline": {"kernel": "wkv_chunk_attention", "bound": "mfma",
                     "achieved": round(att_tflops, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(att_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": None},
        "cpu_baseline": None,
    }
    print(json.dumps(rec), flush=True)


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(a, c, s, bank, poses, qhist, Nq, Nk, Lc):
    """The oracle, as it stands, on a bounded sample of one step's work."""
    import numpy as np
    import threadpoolctl

    from oracle import wkv_oracle as O

    def bits(t):
        import torch
        return t.view(torch.int16).cpu().numpy().view(np.uint16)

    F, T, r, k, nsteps = c["F"], c["T"], c["r"], c["k"], c["S"]
    ek, ev = bits(s["ek"]), bits(s["ev"])
    P = poses.cpu().numpy()
    t0 = time.perf_counter()
    O.compress_chunk(ek, ev, F, T, r, score_mode=a.score_mode)
    t1 = time.perf_counter()
    if len(qhist) == 2:
        q = O.pose_extrapolate(np.asarray(qhist[0], np.float32), np.asarray(qhist[1], np.float32))
    else:
        q = np.asarray(qhist[0], np.float32)
    idx, _ = O.pose_topk(P, q, k)
    t2 = time.perf_counter()
    # only the retrieved chunks leave the device; the oracle indexes them 0..k-1
    sel = [int(i) for i in idx]
    ridx = np.arange(len(sel))
    if c["int4"]:
        kp, vp = bank["k"][sel].cpu().numpy(), bank["v"][sel].cpu().numpy()
        kss, vss = bits(bank["k_scale"][sel]), bits(bank["v_scale"][sel])
        t_deq = time.perf_counter()
        hb = O.dequant_bank_chunks(kp, vp, kss, vss, ridx)
        t_deq = time.perf_counter() - t_deq
    else:
        hb = (bits(bank["k"][sel]), bits(bank["v"][sel]))
        t_deq = 0.0
    sink = (bits(s["sink"][0]), bits(s["sink"][1]))
    rec = [(bits(x), bits(y)) for x, y in s["recent"]]
    cur = (bits(s["cur"][0]), bits(s["cur"][1]))
    t3 = time.perf_counter()
    wk, wv = O.assemble_window(sink, hb, ridx, rec, cur)
    t4 = time.perf_counter()
    # attention: chunks of query rows (cycling over the chunk's rows) until
    # about cpu_seconds of oracle work have run in total
    qb_all = bits(s["q"][0])
    chunk = min(Nq, a.cpu_rows)
    rows_done, q0 = 0, 0
    t5 = time.perf_counter()
    while True:
        idx_rows = (q0 + np.arange(chunk)) % Nq
        O.chunk_attention(qb_all[idx_rows], wk, wv)
        rows_done += chunk
        q0 = (q0 + chunk) % Nq
        el = time.perf_counter() - t5
        if el + (t4 - t0) >= a.cpu_seconds or rows_done >= 16 * Nq * nsteps:
            break
    t6 = time.perf_counter()
    t_att_full = (t6 - t5) / rows_done * Nq
    t_step = (t1 - t0) + (t2 - t1) + t_deq + (t4 - t3) + nsteps * t_att_full
    blas = [p for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
    threads = max([p["num_threads"] for p in blas] or [1])
    return {
        "value": round(1.0 / t_step, 6),
        "unit": "chunk-steps/s",
        "cores": threads,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"numpy fp64 oracle: compress of 1 unit, pose top-k over {len(P)} poses "
                   f"and window assembly ({Nk} rows) in full; attention for {rows_done} query "
                   f"rows ({rows_done / Nq:.2f} passes over the chunk's {Nq} rows) x {c['H']} "
                   f"heads over the full window, per-row time scaled to {Nq} rows x "
                   f"{nsteps} denoising step(s); BLAS threads = cores, elementwise work "
                   "single-threaded"),
        "seconds": {"compress": round(t1 - t0, 3), "pose_topk": round(t2 - t1, 4),
                    "assemble": round(t4 - t3 + t_deq, 3), "attention_sample": round(t6 - t5, 3),
                    "step_estimate": round(t_step, 3)},
    }


if __name__ == "__main__":
    main()
