#!/usr/bin/env python3
"""QSA layer-path throughput on one MI355X.

A step is one pass of the whole per-layer path -- append + pool the rows'
index keys, score every visible pooled block, select the top 512 blocks,
gathered attention with the split-K LSE merge -- over all 12 QSA layers of
one synthetic batch, captured once as a HIP graph and replayed.  Inputs are
resident in HBM before the timed region.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload verify_262k]

The metric is query-rows/s per layer (rows x layers x steps / time).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
CSRC = os.path.join(ROOT, "long_context_sparse_qsa_amd", "csrc")
# sources of the scoring kernel (the dominant kernel): PMC figures taken on
# another build of them are not reported
SCORE_SOURCES = ("score.hip", "select_common.h", "qsa_device.h", "append_common.h")
PMC_FILE = os.path.join(ROOT, "profiles", "score_fewrow_kernel.verify_262k.pmc.txt")
COPY_BYTES = 256 << 20  # plain copy of known size used to scale the PMC byte counters
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
PREFILL_MIN_ROWS = 64  # rows at which scoring takes the many-row matrix-core kernel


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="verify_262k",
                    choices=["verify_262k", "decode_262k", "decode_32k", "prefill", "batched"])
    ap.add_argument("--layers", type=int, default=12)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-m1", action="store_true", help="skip the M=1 companion measurement")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8 K/V companion measurement")
    ap.add_argument("--no-flat", action="store_true", help="skip the memory-flat selection measurement (many rows)")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a graph")
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="run a plain 256 MiB device copy first (scales FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


def score_source_hash() -> str:
    h = hashlib.sha256()
    for f in SCORE_SOURCES:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def append_alg_bytes(new_pos, elt: int) -> int:
    """Algorithmic bytes of appending index keys at positions ``new_pos``
    (``elt`` bytes per element): new keys read and written to the cache, the
    earlier keys of every completed block read from the cache, the pooled
    key (float32) written."""
    pos = set(int(p) for p in new_pos)
    b = len(pos) * 128 * elt * 2
    for p in pos:
        if p % 4 == 3:
            b += 128 * 4 + sum(128 * elt for q in range(p - 3, p) if q not in pos)
    return b


def stored_traffic() -> int | None:
    """HBM bytes per launch of the scoring kernel from the committed PMC
    summary, if it was taken on the current kernel sources."""
    try:
        kv = {}
        for line in open(PMC_FILE):
            if ":" in line and not line.startswith("#"):
                a, b = line.split(":", 1)
                kv[a.strip()] = b.strip()
        if kv.get("source_hash") != score_source_hash():
            return None
        return int(float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


# ----------------------------------------------------------------- set-up

class SeqLayer:
    """One layer of one sequence, resident on the device."""

    def __init__(self, Q, wl, layer, dev):
        import torch
        import datagen

        n = wl.n_ctx
        self.cap = -(-(n + 4) // 256) * 256
        bf = torch.bfloat16
        self.idx_cache = torch.zeros((1, self.cap, 128), dtype=bf, device=dev)
        self.pooled = torch.zeros((1, self.cap // 4, 128), dtype=torch.float32, device=dev)
        self.k = torch.zeros((wl.hkv, self.cap, wl.head_dim), dtype=bf, device=dev)
        self.v = torch.zeros_like(self.k)
        m = wl.m
        self.idx_q = torch.empty((m, 4, 128), dtype=bf, device=dev)
        self.q = torch.empty((m, wl.hq, wl.head_dim), dtype=bf, device=dev)
        idx32 = torch.empty((n, 128), dtype=torch.float32, device=dev)
        datagen.fill_layer_device(wl, layer, idx32, self.idx_q, self.q, self.k, self.v)
        idx = idx32.to(bf)
        del idx32
        Q.qsa_append_pool(idx, torch.arange(n, dtype=torch.int64, device=dev), self.idx_cache, self.pooled)
        self.rows = torch.tensor(wl.rows, dtype=torch.int64, device=dev)
        self.new_idx = idx[self.rows].contiguous()   # the rows' own keys, re-appended each step
        self.new_pos = self.rows.clone()
        self.kv = Q.KvSegments.single(self.k, self.v, n)
        self.row_seq = None


class BatchedLayer:
    """One layer of a batched decode: one row per sequence, each sequence's
    K/V in 1..5 separately allocated segments (seeded lengths and cut points),
    resident on the device."""

    def __init__(self, Q, specs, layer, dev):
        import torch
        import datagen
        from datagen.synth import BATCHED

        bf = torch.bfloat16
        n_seq = len(specs)
        self.cap = max(-(-(sp.n_ctx + 4) // 256) * 256 for sp in specs)
        self.idx_cache = torch.zeros((n_seq, self.cap, 128), dtype=bf, device=dev)
        self.pooled = torch.zeros((n_seq, self.cap // 4, 128), dtype=torch.float32, device=dev)
        self.idx_q = torch.empty((n_seq, 4, 128), dtype=bf, device=dev)
        self.q = torch.empty((n_seq, 24, 256), dtype=bf, device=dev)
        segs, new_idx = [], []
        for s, sp in enumerate(specs):
            wl_s = datagen.Workload(f"batched_seq{s}", 3, sp.n_ctx, (sp.row,), "bf16", 256,
                                    plant=BATCHED["plant"], seed=s)
            idx32 = torch.empty((sp.n_ctx, 128), dtype=torch.float32, device=dev)
            k = torch.empty((2, sp.n_ctx, 256), dtype=bf, device=dev)
            v = torch.empty_like(k)
            datagen.fill_layer_device(wl_s, layer, idx32, self.idx_q[s:s + 1], self.q[s:s + 1], k, v)
            idx = idx32.to(bf)
            del idx32
            Q.qsa_append_pool(idx, torch.arange(sp.n_ctx, dtype=torch.int64, device=dev),
                              self.idx_cache[s:s + 1], self.pooled[s:s + 1])
            new_idx.append(idx[sp.row:sp.row + 1])
            seq_segs = []
            for st, ln, cp in zip(sp.seg_start, sp.seg_len, sp.seg_cap):
                kt = torch.zeros((2, cp, 256), dtype=bf, device=dev)
                vt = torch.zeros_like(kt)
                kt[:, :ln] = k[:, st:st + ln]
                vt[:, :ln] = v[:, st:st + ln]
                seq_segs.append((st, ln, kt, vt))
            segs.append(seq_segs)
            del k, v
        self.kv = Q.KvSegments(segs)
        self.rows = torch.tensor([sp.row for sp in specs], dtype=torch.int64, device=dev)
        self.row_seq = torch.arange(n_seq, dtype=torch.int32, device=dev)
        self.seq = self.row_seq
        self.new_idx = torch.cat(new_idx).contiguous()  # each row's own key, re-appended each step
        self.new_pos = self.rows.clone()


def build_batched(Q, layers, dev):
    import datagen

    specs = datagen.batched_specs()
    wl = datagen.Workload("batched", 3, max(sp.n_ctx for sp in specs), tuple(sp.row for sp in specs), "bf16", 256)
    L = [BatchedLayer(Q, specs, i, dev) for i in range(layers)]
    return wl, L, shared_buffers(Q, wl, dev), (max(wl.rows) + 1) // 4, [sp.n_ctx // 4 for sp in specs]


def build_single(Q, wl, layers, dev):
    L = [SeqLayer(Q, wl, i, dev) for i in range(layers)]
    return L, shared_buffers(Q, wl, dev), (max(wl.rows) + 1) // 4


def shared_buffers(Q, wl, dev):
    import torch

    nb_max = (max(wl.rows) + 1) // 4
    m = wl.m
    k = wl.k_blocks
    shared = dict(
        scores=torch.empty((m, -(-nb_max // 4) * 4), dtype=torch.float32, device=dev),
        sel=torch.empty((m, k), dtype=torch.int32, device=dev),
        n_sel=torch.empty((m,), dtype=torch.int32, device=dev),
        out=torch.empty((m, wl.hq, wl.head_dim), dtype=torch.bfloat16, device=dev),
        lse=torch.empty((m, wl.hq), dtype=torch.float32, device=dev),
        ws=torch.empty(max(1, Q.qsa_attn_workspace_bytes(m, wl.hq, wl.head_dim, k)), dtype=torch.uint8, device=dev),
        ws_sel=None,
    )
    wsb = Q.qsa_select_workspace_bytes(m, nb_max, k)
    if wsb:
        shared["ws_sel"] = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    return shared


def step_fn(Q, L, sh, nb_max, wl, only=None, flat=False):
    """Enqueue one step (all layers).  ``only`` restricts to one kernel family;
    ``flat`` scores and selects through the memory-flat entry point."""
    def run():
        for ly in L:
            # one sequence: the append rides in the scoring launch
            fused = only in (None, "append_score") and not flat and ly.row_seq is None
            if fused:
                Q.qsa_append_score(ly.new_idx, ly.new_pos, ly.idx_cache, ly.pooled, ly.idx_q, ly.rows, sh["scores"],
                                   nb_max, sel_workspace=sh["ws_sel"])
            elif only in (None, "append"):
                Q.qsa_append_pool(ly.new_idx, ly.new_pos, ly.idx_cache, ly.pooled, seq=getattr(ly, "seq", None))
            if flat and only in (None, "flat"):
                Q.qsa_score_select(ly.idx_q, ly.rows, ly.pooled, nb_max, wl.k_blocks, sh["sel"], sh["n_sel"],
                                   sh["ws_flat"])
            elif flat or fused:
                pass
            elif only in (None, "score"):
                Q.qsa_score_blocks(ly.idx_q, ly.rows, ly.pooled, sh["scores"], nb_max, row_seq=ly.row_seq,
                                   sel_workspace=sh["ws_sel"])
            if not flat and only in (None, "select"):
                Q.qsa_select_topk(sh["scores"], ly.rows, nb_max, wl.k_blocks, sh["sel"], sh["n_sel"], sh["ws_sel"],
                                  prepared=True)
            if only in (None, "attn"):
                Q.qsa_gathered_attn(ly.q, ly.rows, ly.kv, sh["sel"], sh["n_sel"], sh["out"], sh["lse"], wl.hkv,
                                    row_seq=ly.row_seq, workspace=sh["ws"])
    return run


def per_launch_us(Q, L, sh, nb_max, wl, kind, reps=4):
    """Average device time of one launch of ``kind``, from HIP events on the
    launch stream around ``reps`` x layers launches queued back to back.  A
    spin kernel runs first so that the whole sequence is queued before the
    device reaches it (no host gaps inside the interval).  The prepared
    selection consumes what the scoring pass left in the workspace, so
    "select" is timed as score+select pairs minus the scoring time."""
    import torch

    def timed(kinds):
        torch.cuda.synchronize()
        try:
            torch.cuda._sleep(int(2e8))
        except Exception:  # pragma: no cover - spin kernel unavailable: host gaps may inflate the figure
            pass
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            for ly in L:
                for k_ in kinds:
                    step_fn(Q, [ly], sh, nb_max, wl, only=k_)()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * len(L))

    if kind == "select":
        return timed(("score", "select")) - timed(("score",))
    return timed((kind,))


# ----------------------------------------------------------- CPU baseline

def cpu_baseline(wl_name: str, budget_s: float = 12.0) -> dict:
    """The oracle, as it stands, on the host: same per-layer work for the
    same rows (pool the blocks the new tokens complete, score, select, attend)."""
    import numpy as np

    import datagen
    import oracle as O

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = 1
    d = datagen.gen_layer(wl_name)
    wl = d["workload"]
    pooled = O.pool_index_keys(d["idx"])
    scale = 1.0 / math.sqrt(wl.head_dim)
    rows = [int(r) for r in d["rows"]]
    t0 = time.perf_counter()
    done = 0
    while True:
        for i, p in enumerate(rows):
            lo = (p // 4) * 4
            if p % 4 == 3:
                pooled[p // 4] = O.pool_index_keys(d["idx"][lo:lo + 4])[0]
            s = O.score_blocks(d["idx_q"][i], pooled, p + 1)
            sel = O.select_blocks(s, wl.k_blocks)
            tok = O.attended_tokens(sel, p + 1)
            O.attend(d["q"][i], d["k"], d["v"], tok, scale)
            done += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    return {"value": done / el, "unit": "query-rows/s per layer", "cores": int(cores), "kind": "oracle",
            "sample": f"{done} rows of one {wl_name} layer (n_ctx {wl.n_ctx}) in {el:.1f} s, numpy fp64"}


# ------------------------------------------------------------------ main

def flat_leg(Q, L, sh, nb_max, wl, args, kt):
    """Many rows scored and selected without the score matrix
    (qsa_score_select): the whole step through a graph, the launch beside the
    materialized score + select, and the memory each needs."""
    import torch

    sh = dict(sh)
    wsb = Q.qsa_score_select_workspace_bytes(wl.m, nb_max, wl.k_blocks)
    sh["ws_flat"] = torch.empty(wsb, dtype=torch.uint8, device=L[0].pooled.device)
    run = step_fn(Q, L, sh, nb_max, wl, flat=True)
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)

    def one(only):
        torch.cuda.synchronize()
        try:
            torch.cuda._sleep(int(2e8))
        except Exception:  # pragma: no cover
            pass
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        step_fn(Q, L, sh, nb_max, wl, only=only, flat=True)()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / len(L)

    flat_us = one("flat")
    ld = -(-nb_max // 4) * 4
    return {"workload": wl.name + " memory-flat select", "value": wl.m * len(L) * args.steps / (ms / 1e3),
            "unit": "query-rows/s per layer", "ms_per_step": ms / args.steps,
            "layer_us": ms * 1e3 / args.steps / len(L),
            "score_select_us": round(flat_us, 1), "score_plus_select_us": round(kt["score"] + kt["select"], 1),
            "workspace_bytes": wsb, "score_matrix_bytes": wl.m * ld * 4 + Q.qsa_select_workspace_bytes(wl.m, nb_max, wl.k_blocks)}


def fp8_leg(Q, L, sh, nb_max, wl, args, attn_bf16_us):
    """The same layers with K/V in the fp8 state (E4M3 codes + f16 scale per
    head and token), quantized on the device from the bf16 K/V: the whole
    step through a graph, the attention launch beside the bf16 one, and the
    quantize launch that writes one step's new K (or V) rows."""
    import torch

    for ly in L:
        ly.k8 = torch.empty((wl.hkv, ly.cap, wl.head_dim), dtype=torch.uint8, device=ly.k.device)
        ly.v8 = torch.empty_like(ly.k8)
        ly.ks = torch.empty((wl.hkv, ly.cap), dtype=torch.float16, device=ly.k.device)
        ly.vs = torch.empty_like(ly.ks)
        Q.qsa_quantize_kv_fp8(ly.k, ly.k8, ly.ks)
        Q.qsa_quantize_kv_fp8(ly.v, ly.v8, ly.vs)
        ly.kv_bf16, ly.kv = ly.kv, Q.KvSegments.single(ly.k8, ly.v8, wl.n_ctx, ly.ks, ly.vs)
        ly.new_k = ly.k[:, ly.rows[0]:ly.rows[0] + min(wl.m, 4)].contiguous()  # new K rows [hkv, T, D]
    torch.cuda.synchronize()
    run = step_fn(Q, L, sh, nb_max, wl)
    run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    attn_us = per_launch_us(Q, L, sh, nb_max, wl, "attn")
    # one step's K write: M rows x hkv heads quantized into the cache
    t0 = int(wl.rows[0])
    torch.cuda.synchronize()
    try:  # queue every launch before the device reaches them (no host gaps in the interval)
        torch.cuda._sleep(int(2e8))
    except Exception:  # pragma: no cover
        pass
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(4):
        for ly in L:
            Q.qsa_quantize_kv_fp8(ly.new_k, ly.k8, ly.ks, t0=t0)
    b.record()
    torch.cuda.synchronize()
    quant_us = a.elapsed_time(b) * 1e3 / (4 * len(L))
    tok = sum(min((p + 1) // 4, wl.k_blocks) * 4 + (p + 1) % 4 for p in wl.rows)
    gather_fp8 = tok * wl.hkv * 2 * (wl.head_dim + 2)
    gather_bf16 = tok * wl.hkv * 2 * wl.head_dim * 2
    for ly in L:  # back to the bf16 state for whatever runs next
        ly.kv = ly.kv_bf16
        del ly.k8, ly.v8, ly.ks, ly.vs, ly.new_k
    torch.cuda.synchronize()
    return {"workload": wl.name + " fp8 K/V", "value": wl.m * len(L) * args.steps / (ms / 1e3),
            "unit": "query-rows/s per layer", "ms_per_step": ms / args.steps,
            "layer_us": ms * 1e3 / args.steps / len(L),
            "attn_us": round(attn_us, 2), "attn_us_bf16": round(attn_bf16_us, 2),
            "gather_bytes": gather_fp8, "gather_bytes_bf16": gather_bf16,
            "quantize_us_per_kv_write": round(quant_us, 2)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import datagen
    import long_context_sparse_qsa_amd as Q

    dev = "cuda:0"
    torch.cuda.set_device(0)
    Q.qsa_device_check()
    layers = args.layers
    t_setup = time.time()
    if args.workload == "batched":
        wl, L, sh, nb_max, seq_nb = build_batched(Q, layers, dev)
    else:
        wl = datagen.WORKLOADS[args.workload]
        L, sh, nb_max = build_single(Q, wl, layers, dev)
        seq_nb = None  # one sequence: its pooled keys are read once for all rows
    torch.cuda.synchronize()
    print(f"[bench] set-up {wl.name}: {layers} layers, n_ctx {wl.n_ctx}, M {wl.m} in "
          f"{time.time() - t_setup:.1f} s", file=sys.stderr, flush=True)

    if args.pmc_calibration:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    run = step_fn(Q, L, sh, nb_max, wl)
    run()
    torch.cuda.synchronize()
    if args.eager:
        replay = run
    else:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            run()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            run()
        replay = g.replay
    for _ in range(args.warmup):
        replay()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(args.steps):
        replay()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    ms_step = ms / args.steps
    rows_per_s = wl.m * layers * args.steps / (ms / 1e3)

    # per-kernel device time (dominant kernel: scoring, HBM-bound)
    kt = {kind: per_launch_us(Q, L, sh, nb_max, wl, kind) for kind in ("score", "select", "attn", "append")}
    if L[0].row_seq is None:
        kt["append_score"] = per_launch_us(Q, L, sh, nb_max, wl, "append_score")
    pooled_bytes = nb_max * 512 if seq_nb is None else sum(seq_nb) * 512
    score_bytes = pooled_bytes + wl.m * 4 * 128 * 2 + (wl.m * nb_max if seq_nb is None else sum(seq_nb)) * 4
    # the step scores through the launch that also appends (one sequence,
    # few rows): its bytes include the append's
    folded = L[0].row_seq is None and wl.m < PREFILL_MIN_ROWS
    score_us = kt["append_score"] if folded else kt["score"]
    if folded:
        score_bytes += append_alg_bytes(L[0].new_pos.cpu().tolist(), 2)
    achieved = score_bytes / (score_us * 1e-6) / 1e9
    if wl.m >= PREFILL_MIN_ROWS:
        # many-row scoring runs on the bf16 matrix cores with three-plane
        # pooled keys: report issued bf16 flops against the bf16 peak, and the
        # float32-equivalent (algorithmic) rate beside it
        alg_flops = sum(min((p + 1) // 4, nb_max) for p in wl.rows) * 4 * 128 * 2
        roofline = {"bound": "mfma", "kernel": "score_prefill_pipe_kernel",
                    "achieved": 3 * alg_flops / (score_us * 1e-6) / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": 3 * alg_flops / (score_us * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                    "traffic": None, "algorithmic_tflops": alg_flops / (score_us * 1e-6) / 1e12,
                    "flops_per_launch_bf16": 3 * alg_flops, "launch_us": score_us}
    else:
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                    "kernel": ("score_fewrow_kernel (append folded in)" if folded else
                               "score_fewrow_kernel" if seq_nb is None else
                               "score_fewrow_kernel (one row per sequence)"),
                    "traffic": stored_traffic() if wl.name == "verify_262k" else None,
                    "bytes_per_launch": score_bytes, "launch_us": score_us}
    # whole-path algorithmic bytes per layer step: pooled once + gathered K/V + q/out/index queries
    tok = sum(min((p + 1) // 4, wl.k_blocks) * 4 + (p + 1) % 4 for p in wl.rows)
    path_bytes = pooled_bytes + tok * wl.hkv * 2 * wl.head_dim * 2 + wl.m * (2 * wl.hq * wl.head_dim * 2 + 4 * 128 * 2)
    layer_us = ms_step * 1e3 / layers
    res = {
        "metric": "QSA query-rows/s per layer at 262K ctx (M=1,4) + achieved HBM GB/s / MFMA %",
        "value": rows_per_s,
        "unit": "query-rows/s per layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "n_ctx": wl.n_ctx, "rows": wl.m, "row_pos": [wl.rows[0], wl.rows[-1]],
                   "layers": layers, "budget_tokens": wl.k_blocks * 4, "hq": wl.hq, "hkv": wl.hkv,
                   "head_dim": wl.head_dim, "graph": not args.eager},
        "roofline": roofline,
        "path": {"layer_us": layer_us, "bytes_per_layer_step": path_bytes,
                 "achieved_GBs": path_bytes / (layer_us * 1e-6) / 1e9,
                 "frac": path_bytes / (layer_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                 "kernel_us": {k_: round(v, 2) for k_, v in kt.items()}},
    }
    if not args.no_flat and wl.m >= PREFILL_MIN_ROWS:
        res["flat"] = flat_leg(Q, L, sh, nb_max, wl, args, kt)
    if not args.no_fp8 and wl.name in ("verify_262k", "decode_262k", "decode_32k", "prefill"):
        res["fp8"] = fp8_leg(Q, L, sh, nb_max, wl, args, kt["attn"])
    if not args.no_m1 and wl.name == "verify_262k":
        wl1 = datagen.WORKLOADS["decode_262k"]
        for ly in L:
            ly.rows = ly.rows[-1:].contiguous()
            ly.new_idx = ly.new_idx[-1:].contiguous()
            ly.new_pos = ly.new_pos[-1:].contiguous()
            ly.idx_q = ly.idx_q[-1:].contiguous()
            ly.q = ly.q[-1:].contiguous()
        sh1 = dict(sh)
        sh1["out"] = sh["out"][-1:].contiguous()
        sh1["lse"] = sh["lse"][-1:].contiguous()
        run1 = step_fn(Q, L, sh1, nb_max, wl1)
        run1()
        torch.cuda.synchronize()
        g1 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g1):
            run1()
        for _ in range(args.warmup):
            g1.replay()
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            g1.replay()
        end.record()
        torch.cuda.synchronize()
        ms1 = start.elapsed_time(end)
        res["m1"] = {"workload": "decode_262k", "value": layers * args.steps / (ms1 / 1e3),
                     "ms_per_step": ms1 / args.steps, "layer_us": ms1 * 1e3 / args.steps / layers}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
