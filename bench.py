#!/usr/bin/env python3
"""QSA layer-path throughput on one MI355X.

A step is one pass of the whole per-layer path -- append + pool the rows'
index keys, score every visible pooled block, select the top 512 blocks,
gathered attention with the split-K LSE merge -- over all 12 QSA layers of
one synthetic batch, captured once as a HIP graph and replayed.  Inputs are
resident in HBM before the timed region.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload verify_262k] [--legs all]

The metric is query-rows/s per layer (rows x layers x steps / time) of the
main workload (default: the 4-row verify at 261,122 context).  Every other
workload of the benchmark set is timed as a leg of the same run and reported
beside it: M = 1 at 262K, fp8 and Q8_0 K/V, decode M = 1 at 32K, batched
segmented decode, and the 2,048-row prefill chunk (with its matrix-core
utilisation).

Each timed sweep rotates over R replicas of the 12 layers' state, R chosen so
that one sweep touches at least 1 GiB, so that the 256 MB last-level cache
cannot hold what a step reads from one step to the next.
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
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
ROTATE_BYTES = 1 << 30  # bytes one sweep over the layer states touches at least
CSRC = os.path.join(ROOT, "long_context_sparse_qsa_amd", "csrc")
# sources of the scoring kernel (the dominant kernel): PMC figures taken on
# another build of them are not reported
SCORE_SOURCES = ("score.hip", "select_common.h", "qsa_device.h", "append_common.h")
PMC_FILE = os.path.join(ROOT, "profiles", "score_fewrow_kernel.verify_262k.pmc.txt")
COPY_BYTES = 256 << 20  # plain copy of known size used to scale the PMC byte counters
PREFILL_MIN_ROWS = 64  # rows at which scoring takes the many-row matrix-core kernel
LEGS = ("m1", "fp8", "q8", "decode_32k", "batched", "prefill")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="verify_262k",
                    choices=["verify_262k", "decode_262k", "decode_32k", "prefill", "batched"])
    ap.add_argument("--layers", type=int, default=12)
    ap.add_argument("--legs", default="all",
                    help="comma list of " + ",".join(LEGS) + ", or all / none (legs of the verify_262k run)")
    ap.add_argument("--replicas", type=int, default=0, help="layer-state replicas per sweep (0: the 1 GiB rule)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-flat", action="store_true", help="skip the memory-flat selection measurement (prefill)")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8 K/V measurements")
    ap.add_argument("--no-m1", action="store_true", help="skip the M=1 leg")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graphs")
    ap.add_argument("--pmc-calibration", action="store_true",
                    help="run a plain 256 MiB device copy first (scales FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--probes", action="store_true",
                    help="time the memory-pattern probes (libqsa_probe.so) and exit")
    ap.add_argument("--cpu-table", action="store_true",
                    help="time the CPU oracle on every workload (1 thread and all threads) and exit")
    a = ap.parse_args()
    if a.legs == "all":
        a.legs = set(LEGS)
    elif a.legs == "none":
        a.legs = set()
    else:
        a.legs = set(x for x in a.legs.split(",") if x)
        bad = a.legs - set(LEGS)
        if bad:
            ap.error(f"unknown legs {sorted(bad)}")
    if a.no_m1:
        a.legs.discard("m1")
    if a.no_fp8:
        a.legs.discard("fp8")
    return a


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


def kept_tokens(rows, k_blocks: int) -> int:
    """Tokens the rows attend: min(k, nb) blocks of 4 plus each row's tail."""
    return sum(min((p + 1) // 4, k_blocks) * 4 + (p + 1) % 4 for p in rows)


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


def replicas(per_layer_bytes: int, layers: int, forced: int = 0) -> int:
    """Replicas of the layers' state so that one sweep touches >= 1 GiB."""
    if forced > 0:
        return forced
    return max(1, -(-ROTATE_BYTES // max(1, per_layer_bytes * layers)))


def step_fn(Q, L, sh, nb_max, wl, only=None, flat=False):
    """Enqueue one step (the layers ``L``).  ``only`` restricts to one kernel
    family; ``flat`` scores and selects through the memory-flat entry point."""
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


def spin():
    """Queue a long device-side spin first, so that everything enqueued after
    it is queued before the device reaches it (no host gaps in an interval)."""
    import torch

    try:
        torch.cuda._sleep(int(2e8))
    except Exception:  # pragma: no cover - spin kernel unavailable: host gaps may inflate a figure
        pass


def timed_sweeps(Q, groups, sh, nb_max, wl, steps, warmup, eager=False, flat=False) -> float:
    """Milliseconds per step: step i runs replica i % R of the layers (one
    HIP graph per replica), ``steps`` steps between two HIP events on the
    launch stream after ``warmup`` untimed ones."""
    import torch

    runs = [step_fn(Q, grp, sh, nb_max, wl, flat=flat) for grp in groups]
    for r in runs:
        r()
    torch.cuda.synchronize()
    if eager:
        replays = runs
    else:
        replays = []
        for r in runs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                r()
            replays.append(g)
        replays = [g.replay for g in replays]
    for i in range(warmup):
        replays[i % len(replays)]()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        replays[i % len(replays)]()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


def per_launch_us(Q, L, sh, nb_max, wl, kind, reps=4, flat=False):
    """Average device time of one launch of ``kind``, from HIP events on the
    launch stream around ``reps`` x layers launches queued back to back over
    every layer state.  The prepared selection consumes what the scoring pass
    left in the workspace, so "select" is timed as score+select pairs minus
    the scoring time."""
    import torch

    def timed(kinds):
        torch.cuda.synchronize()
        spin()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            for ly in L:
                for k_ in kinds:
                    step_fn(Q, [ly], sh, nb_max, wl, only=k_, flat=flat)()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * len(L))

    if kind == "select":
        return timed(("score", "select")) - timed(("score",))
    return timed((kind,))


def path_bytes(wl, rows, pooled_blocks: int) -> int:
    """Algorithmic bytes of one layer step: pooled keys read once (per
    sequence), gathered K/V, queries, outputs and index queries."""
    tok = kept_tokens(rows, wl.k_blocks)
    return (pooled_blocks * 512 + tok * wl.hkv * 2 * wl.head_dim * 2
            + len(rows) * (2 * wl.hq * wl.head_dim * 2 + 4 * 128 * 2))


def leg_record(name, m, layers, R, ms, pbytes, kt) -> dict:
    layer_us = ms * 1e3 / layers
    return {"workload": name, "value": m * layers / (ms / 1e3), "unit": "query-rows/s per layer",
            "ms_per_step": ms, "layer_us": layer_us, "layers": layers, "replicas": R,
            "path": {"bytes_per_layer_step": pbytes, "achieved_GBs": pbytes / (layer_us * 1e-6) / 1e9,
                     "frac": pbytes / (layer_us * 1e-6) / 1e9 / HBM_PEAK_GBS},
            "kernel_us": {k_: round(v, 2) for k_, v in kt.items()}}


def groups_of(L, layers):
    return [L[i:i + layers] for i in range(0, len(L), layers)]


def free():
    import gc

    import torch

    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


# ----------------------------------------------------------- CPU baseline

def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        return 1


def cpu_baseline(wl_name: str = "verify_262k", budget_s: float = 10.0, table: bool = False) -> dict:
    """The CPU oracle, as it stands, on the host (the only part of this script
    that runs it).  By default: rows/s per layer on rows of one ``wl_name``
    layer, once with BLAS limited to one thread and once with every thread
    BLAS starts with.  With ``table``: every workload of the benchmark set,
    both thread counts, and where the time goes (pool / score / select /
    attend)."""
    import datagen
    import oracle as O

    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None

    def limited(n):
        if threadpool_limits is None or n is None:
            import contextlib
            return contextlib.nullcontext()
        return threadpool_limits(limits=n)

    def oracle_rows(d, budget, bd, rows_idx=None):
        """Rows of one layer (pool the block a row's own token completes,
        score, select, attend), repeated until ``budget`` seconds have
        passed; returns (rows done, seconds)."""
        wl = d["workload"]
        pooled = O.pool_index_keys(d["idx"])
        scale = 1.0 / math.sqrt(wl.head_dim)
        rows = list(range(len(d["rows"]))) if rows_idx is None else list(rows_idx)
        for key in ("pool", "score", "select", "attend"):
            bd.setdefault(key, 0.0)
        t0 = time.perf_counter()
        done = 0
        while True:
            for i in rows:
                p = int(d["rows"][i])
                ta = time.perf_counter()
                if p % 4 == 3:
                    lo = (p // 4) * 4
                    pooled[p // 4] = O.pool_index_keys(d["idx"][lo:lo + 4])[0]
                tb = time.perf_counter()
                s = O.score_blocks(d["idx_q"][i], pooled, p + 1)
                tc = time.perf_counter()
                sel = O.select_blocks(s, wl.k_blocks)
                td = time.perf_counter()
                O.attend(d["q"][i], d["k"], d["v"], O.attended_tokens(sel, p + 1), scale)
                te = time.perf_counter()
                bd["pool"] += tb - ta
                bd["score"] += tc - tb
                bd["select"] += td - tc
                bd["attend"] += te - td
                done += 1
                if time.perf_counter() - t0 >= budget:
                    return done, time.perf_counter() - t0

    if not table:
        d = datagen.gen_layer(wl_name)
        wl = d["workload"]
        with limited(1):
            n1, t1 = oracle_rows(d, budget_s, {})
        cores = blas_threads()
        n, t = oracle_rows(d, budget_s, {})
        sample = f"rows of one {wl_name} layer (n_ctx {wl.n_ctx}), numpy fp64"
        return {"value": n / t, "unit": "query-rows/s per layer", "cores": int(cores), "kind": "oracle",
                "sample": f"{n} {sample} in {t:.1f} s", "cpu_model": cpu_model(), "host_cpus": os.cpu_count(),
                "single_thread": {"value": n1 / t1, "cores": 1,
                                  "sample": f"{n1} {sample} in {t1:.1f} s, BLAS limited to one thread"}}

    out = {"cpu_model": cpu_model(), "host_cpus": os.cpu_count(), "all_threads": blas_threads(), "rows": {}}
    cases = [("tiny", None), ("decode_32k", None), ("decode_262k", None), ("verify_262k", None),
             ("prefill", list(range(0, 2048, 8)))]
    for name, rows_idx in cases:
        d = datagen.gen_layer(name)
        rec = {}
        for label, lim in (("1", 1), ("all", None)):
            bd = {}
            with limited(lim):
                n, t = oracle_rows(d, budget_s, bd, rows_idx)
            rec[label] = {"rows_per_s": n / t, "rows": n, "seconds": t, "share": {k_: v / t for k_, v in bd.items()}}
        out["rows"][name] = rec
        print(json.dumps({name: rec}), file=sys.stderr, flush=True)
        del d
    # batched decode: one row per sequence, each against its own context
    specs = datagen.batched_specs()
    data = datagen.gen_batched_layer(specs)
    rec = {}
    for label, lim in (("1", 1), ("all", None)):
        done, tt, bd = 0, 0.0, {}
        with limited(lim):
            t0 = time.perf_counter()
            while time.perf_counter() - t0 < budget_s:
                for h in data:
                    dd = dict(h)
                    dd["workload"] = datagen.WORKLOADS["decode_32k"]
                    n, t = oracle_rows(dd, 0.0, bd)
                    done += n
                    tt += t
        rec[label] = {"rows_per_s": done / tt, "rows": done, "seconds": tt,
                      "share": {k_: v / tt for k_, v in bd.items()}}
    out["rows"]["batched"] = rec
    return out


# ------------------------------------------------------------------ legs

def quant_leg(Q, L, groups, sh, nb_max, wl, args, attn_bf16_us, fmt="fp8", flat=False):
    """The same layers with K/V in a quantized state -- fp8 (E4M3 codes + f16
    scale per head and token) or q8 (Q8_0: int8 codes + f16 scale per 32
    values) -- quantized on the device from the bf16 K/V: the whole step
    through graphs, the attention launch beside the bf16 one, and the
    quantize launch that writes one step's new K (or V) rows.  ``flat``: the
    step selects through the memory-flat entry point (sh["ws_flat"])."""
    import torch

    q8 = fmt == "q8"
    quantize = Q.qsa_quantize_kv_q8_0 if q8 else Q.qsa_quantize_kv_fp8
    for ly in L:
        ly.k8 = torch.empty((wl.hkv, ly.cap, wl.head_dim), dtype=torch.int8 if q8 else torch.uint8,
                            device=ly.k.device)
        ly.v8 = torch.empty_like(ly.k8)
        ly.ks = torch.empty((wl.hkv, ly.cap, wl.head_dim // 32) if q8 else (wl.hkv, ly.cap), dtype=torch.float16,
                            device=ly.k.device)
        ly.vs = torch.empty_like(ly.ks)
        quantize(ly.k, ly.k8, ly.ks)
        quantize(ly.v, ly.v8, ly.vs)
        ly.kv_bf16, ly.kv = ly.kv, Q.KvSegments.single(ly.k8, ly.v8, wl.n_ctx, ly.ks, ly.vs)
        ly.new_k = ly.k[:, ly.rows[0]:ly.rows[0] + min(wl.m, 4)].contiguous()  # new K rows [hkv, T, D]
    torch.cuda.synchronize()
    ms = timed_sweeps(Q, groups, sh, nb_max, wl, args.steps, args.warmup, args.eager, flat=flat)
    attn_us = per_launch_us(Q, L, sh, nb_max, wl, "attn")
    # one step's K write: M rows x hkv heads quantized into the cache
    t0 = int(wl.rows[0])
    torch.cuda.synchronize()
    spin()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(4):
        for ly in L:
            quantize(ly.new_k, ly.k8, ly.ks, t0=t0)
    b.record()
    torch.cuda.synchronize()
    quant_us = a.elapsed_time(b) * 1e3 / (4 * len(L))
    tok = kept_tokens(wl.rows, wl.k_blocks)
    gather_q = tok * wl.hkv * 2 * (wl.head_dim + (wl.head_dim // 16 if q8 else 2))
    gather_bf16 = tok * wl.hkv * 2 * wl.head_dim * 2
    for ly in L:  # back to the bf16 state for whatever runs next
        ly.kv = ly.kv_bf16
        del ly.k8, ly.v8, ly.ks, ly.vs, ly.new_k
    free()
    layers = len(groups[0])
    return {"workload": wl.name + (" Q8_0 K/V" if q8 else " fp8 K/V"), "value": wl.m * layers / (ms / 1e3),
            "unit": "query-rows/s per layer", "ms_per_step": ms, "layer_us": ms * 1e3 / layers,
            "attn_us": round(attn_us, 2), "attn_us_bf16": round(attn_bf16_us, 2),
            "gather_bytes": gather_q, "gather_bytes_bf16": gather_bf16,
            "quantize_us_per_kv_write": round(quant_us, 2)}


def single_leg(Q, name, args, dev, kinds=("append_score", "select", "attn")):
    """A one-sequence workload over rotating replicas of its layer states."""
    import datagen

    wl = datagen.WORKLOADS[name]
    nb_max = (max(wl.rows) + 1) // 4
    pb = path_bytes(wl, wl.rows, nb_max)
    R = replicas(pb, args.layers, args.replicas)
    L = [SeqLayer(Q, wl, i, dev) for i in range(args.layers * R)]
    sh = shared_buffers(Q, wl, dev)
    groups = groups_of(L, args.layers)
    ms = timed_sweeps(Q, groups, sh, nb_max, wl, args.steps, args.warmup, args.eager)
    kt = {k_: per_launch_us(Q, L, sh, nb_max, wl, k_) for k_ in kinds}
    rec = leg_record(name, wl.m, args.layers, R, ms, pb, kt)
    del L, sh, groups
    free()
    return rec


def batched_leg(Q, args, dev):
    import datagen

    specs = datagen.batched_specs()
    wl = datagen.Workload("batched", 3, max(sp.n_ctx for sp in specs), tuple(sp.row for sp in specs), "bf16", 256)
    nb_max = (max(wl.rows) + 1) // 4
    pb = path_bytes(wl, wl.rows, sum(sp.n_ctx // 4 for sp in specs))
    R = replicas(pb, args.layers, args.replicas)
    L = [BatchedLayer(Q, specs, i, dev) for i in range(args.layers * R)]
    sh = shared_buffers(Q, wl, dev)
    groups = groups_of(L, args.layers)
    ms = timed_sweeps(Q, groups, sh, nb_max, wl, args.steps, args.warmup, args.eager)
    kt = {k_: per_launch_us(Q, L, sh, nb_max, wl, k_) for k_ in ("append", "score", "select", "attn")}
    rec = leg_record("batched", wl.m, args.layers, R, ms, pb, kt)
    rec["sequences"] = len(specs)
    rec["contexts"] = [sp.n_ctx for sp in specs]
    rec["segments"] = [len(sp.seg_len) for sp in specs]
    del L, sh, groups
    free()
    return rec


def prefill_leg(Q, args, dev):
    """The 2,048-row prefill chunk at 200,000..202,047: rows/s per layer and
    the matrix-core utilisation of its scoring pass, its attention and the
    whole path, on algorithmic flops (and, for the scoring pass, on the bf16
    flops its three-plane pooled keys issue).  The step selects through the
    memory-flat entry point (qsa_score_select: no score matrix, and the faster
    of the two); the materialized path (qsa_score_blocks + qsa_select_topk) is
    timed beside it, and its score-only kernel gives the scoring pass's
    matrix-core figures."""
    import torch

    import datagen

    wl = datagen.WORKLOADS["prefill"]
    nb_max = (max(wl.rows) + 1) // 4
    steps = max(3, args.steps // 20)
    warm = max(1, min(args.warmup, 3))
    L = [SeqLayer(Q, wl, i, dev) for i in range(args.layers)]
    sh = shared_buffers(Q, wl, dev)
    groups = [L]
    ms = timed_sweeps(Q, groups, sh, nb_max, wl, steps, warm, args.eager)
    kt = {k_: per_launch_us(Q, L, sh, nb_max, wl, k_, reps=1) for k_ in ("append", "score", "select", "attn")}
    pairs = sum(min((p + 1) // 4, nb_max) for p in wl.rows)
    score_flops = pairs * 4 * 128 * 2                        # float32-equivalent products of the scores
    tok = kept_tokens(wl.rows, wl.k_blocks)
    attn_flops = tok * wl.hq * wl.head_dim * 2 * 2            # QK and PV over the kept tokens
    tf = lambda f, us: f / (us * 1e-6) / 1e12  # noqa: E731
    pbytes = path_bytes(wl, wl.rows, nb_max)
    ld = -(-nb_max // 4) * 4
    matrix_bytes = wl.m * ld * 4 + Q.qsa_select_workspace_bytes(wl.m, nb_max, wl.k_blocks)
    rec = leg_record("prefill", wl.m, args.layers, 1, ms, pbytes, kt)
    rec["selection"] = "materialized (qsa_score_blocks + qsa_select_topk)"
    flat = None
    if not args.no_flat:
        sh2 = dict(sh)
        wsb = Q.qsa_score_select_workspace_bytes(wl.m, nb_max, wl.k_blocks)
        sh2["ws_flat"] = torch.empty(wsb, dtype=torch.uint8, device=dev)
        msf = timed_sweeps(Q, groups, sh2, nb_max, wl, steps, warm, args.eager, flat=True)
        flat_us = per_launch_us(Q, L, sh2, nb_max, wl, "flat", reps=1, flat=True)
        flat = {"ms_per_step": msf, "score_select_us": flat_us, "workspace_bytes": wsb}
        if msf < ms:  # the step's figure is the faster path's
            sh = sh2
            mat = {"workload": "prefill, materialized scores", "value": rec["value"], "ms_per_step": ms,
                   "layer_us": rec["layer_us"], "kernel_us": rec["kernel_us"],
                   "score_plus_select_us": round(kt["score"] + kt["select"], 1),
                   "score_matrix_bytes": matrix_bytes}
            rec = leg_record("prefill", wl.m, args.layers, 1, msf, pbytes,
                             {"append": kt["append"], "score_select": flat_us, "attn": kt["attn"]})
            rec["selection"] = "memory-flat (qsa_score_select)"
            rec["materialized"] = mat
    layer_us = rec["layer_us"]
    # the gathered K/V above is counted per row (8.6 GB); rows share blocks, so
    # the unique K/V is far less (at most the layer's 202,048 tokens)
    rec["path"]["unique_kv_bytes"] = wl.n_ctx * wl.hkv * 2 * wl.head_dim * 2
    rec["path"]["note"] = ("gathered K/V counted per row: the rows' selections are nearly independent, so each "
                           "row's gather is its own traffic (bench.py --probes: random 2 KiB gathers over the "
                           "same 413.8 MB run at ~7.7 TB/s)")
    rec["mfma"] = {
        "peak_tflops": MFMA_BF16_PEAK_TFLOPS,
        "scoring": {"kernel": "score_prefill_pipe_kernel (score-only mode)", "launch_us": kt["score"],
                    "alg_flops": score_flops, "alg_tflops": tf(score_flops, kt["score"]),
                    "alg_frac": tf(score_flops, kt["score"]) / MFMA_BF16_PEAK_TFLOPS,
                    "issued_bf16_flops": 3 * score_flops,
                    "issued_frac": tf(3 * score_flops, kt["score"]) / MFMA_BF16_PEAK_TFLOPS},
        "attention": {"kernel": "attn_mfma_kernel", "launch_us": kt["attn"], "alg_flops": attn_flops,
                      "alg_tflops": tf(attn_flops, kt["attn"]),
                      "alg_frac": tf(attn_flops, kt["attn"]) / MFMA_BF16_PEAK_TFLOPS,
                      "gathered_bytes": tok * wl.hkv * 2 * wl.head_dim * 2,
                      "gathered_TBs": tok * wl.hkv * 2 * wl.head_dim * 2 / (kt["attn"] * 1e-6) / 1e12},
        "path": {"alg_flops": score_flops + attn_flops, "alg_tflops": tf(score_flops + attn_flops, layer_us),
                 "alg_frac": tf(score_flops + attn_flops, layer_us) / MFMA_BF16_PEAK_TFLOPS},
    }
    if flat is not None:
        fus = flat["score_select_us"]
        rec["flat"] = {"workload": "prefill memory-flat select", "value": wl.m * args.layers / (flat["ms_per_step"] / 1e3),
                       "ms_per_step": flat["ms_per_step"], "layer_us": flat["ms_per_step"] * 1e3 / args.layers,
                       "score_select_us": round(fus, 1),
                       "score_plus_select_us": round(kt["score"] + kt["select"], 1),
                       "scoring_alg_frac": tf(score_flops, fus) / MFMA_BF16_PEAK_TFLOPS,
                       "workspace_bytes": flat["workspace_bytes"], "score_matrix_bytes": matrix_bytes}
    for fmt in ("fp8", "q8"):
        if fmt in args.legs:
            rec[fmt] = quant_leg(Q, L, groups, sh, nb_max, wl,
                                 argparse.Namespace(**{**vars(args), "steps": steps, "warmup": warm}), kt["attn"], fmt,
                                 flat="ws_flat" in sh)
    del L, sh, groups
    free()
    return rec


# ------------------------------------------------------------------ main

def probes(dev) -> dict:
    """What the memory system delivers for the path's access patterns, with
    no arithmetic (libqsa_probe.so): a one-launch contiguous read of one
    layer's pooled keys at 262K (the scoring pass's bytes and workgroup
    shape), random 2 KiB gathers (4-token K or V rows at head_dim 256) over
    working sets from L2-sized to the prefill chunk's K/V and beyond, and the
    cost of one more launch in a graph of dependent launches."""
    import ctypes

    import numpy as np
    import torch

    lib = ctypes.CDLL(os.path.join(ROOT, "long_context_sparse_qsa_amd", "libqsa_probe.so"))
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.qsa_probe_read.argtypes = [vp, i64, i32, vp, vp]
    lib.qsa_probe_gather.argtypes = [vp, i64, vp, i64, vp, vp]
    lib.qsa_probe_empty.argtypes = [i32, vp]
    lib.qsa_probe_last_error.restype = ctypes.c_char_p
    stream = vp(torch.cuda.current_stream().cuda_stream)

    def ok(r):
        if r != 0:
            raise RuntimeError(lib.qsa_probe_last_error().decode())

    sink = torch.zeros(1, dtype=torch.float32, device=dev)

    def timed(fn, reps):
        fn(0)
        torch.cuda.synchronize()
        spin()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(reps):
            fn(i)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / reps

    out = {"peak_GBs": HBM_PEAK_GBS}
    # one launch reading the pooled keys of one 262K layer (65,280 blocks x 512 B)
    pooled = 65280 * 512
    nbuf = -(-ROTATE_BYTES // pooled)
    big = torch.empty(nbuf * pooled // 4, dtype=torch.float32, device=dev).fill_(1.0)
    rd = {}
    for wgb in (16384, 32768, 65536):
        us = timed(lambda i: ok(lib.qsa_probe_read(vp(big.data_ptr() + (i % nbuf) * pooled), pooled, wgb,
                                                   vp(sink.data_ptr()), stream)), 4 * nbuf)
        rd[f"{wgb // 1024}KiB_per_wg"] = {"workgroups": pooled // wgb, "us": round(us, 2),
                                          "GBs": round(pooled / us / 1e3, 1),
                                          "frac": round(pooled / us / 1e3 / HBM_PEAK_GBS, 3)}
    out["read_33MB_one_launch"] = rd
    del big
    # random 2 KiB gathers: the prefill chunk's count (2,048 rows x 2 KV heads
    # x 512 blocks x K and V) over several working sets
    n = 2048 * 2 * 512 * 2
    buf = torch.empty((1 << 30) // 4, dtype=torch.float32, device=dev).fill_(1.0)
    rng = np.random.default_rng(0)
    ga = {}
    for name, ws in (("4MiB", 4 << 20), ("64MiB", 64 << 20), ("prefill_kv_413.8MB", 413794304),
                     ("1GiB", 1 << 30)):
        ids = torch.from_numpy(rng.integers(0, ws // 2048, size=n, dtype=np.int64).astype(np.int32)).to(dev)
        us = timed(lambda i: ok(lib.qsa_probe_gather(vp(buf.data_ptr()), ws, vp(ids.data_ptr()), n,
                                                     vp(sink.data_ptr()), stream)), 5)
        ga[name] = {"working_set_bytes": ws, "us": round(us, 1), "GBs": round(n * 2048 / us / 1e3, 1),
                    "frac": round(n * 2048 / us / 1e3 / HBM_PEAK_GBS, 3)}
        del ids
    out["gather_2KiB_8.6GB"] = ga
    del buf
    # one more launch in a graph: 48 dependent empty launches (12 layers x 4)
    em = {}
    for wgs in (1, 256):
        g = torch.cuda.CUDAGraph()
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for _ in range(48):
                ok(lib.qsa_probe_empty(wgs, vp(torch.cuda.current_stream().cuda_stream)))
        us = timed(lambda i: g.replay(), 50)
        em[f"{wgs}_workgroups"] = {"us_per_launch": round(us / 48, 2)}
    out["empty_launch_in_graph"] = em
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    if args.cpu_table:
        print(json.dumps(cpu_baseline(budget_s=8.0, table=True)), flush=True)
        return
    import torch

    import datagen
    import long_context_sparse_qsa_amd as Q

    dev = "cuda:0"
    torch.cuda.set_device(0)
    Q.qsa_device_check()
    if args.probes:
        print(json.dumps({"probes": probes(dev)}), flush=True)
        return
    if args.pmc_calibration:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload in ("decode_32k", "prefill", "batched"):
        # one workload on its own (profiling runs)
        t0 = time.time()
        rec = (prefill_leg(Q, args, dev) if args.workload == "prefill" else
               batched_leg(Q, args, dev) if args.workload == "batched" else single_leg(Q, "decode_32k", args, dev))
        print(f"[bench] {args.workload} in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
        print(json.dumps(rec), flush=True)
        return

    # ---- main leg: the verify (or M = 1) workload at 261,122 context
    wl = datagen.WORKLOADS[args.workload]
    layers = args.layers
    nb_max = (max(wl.rows) + 1) // 4
    pbytes = path_bytes(wl, wl.rows, nb_max)
    R = replicas(pbytes, layers, args.replicas)
    t_setup = time.time()
    L = [SeqLayer(Q, wl, i, dev) for i in range(layers * R)]
    sh = shared_buffers(Q, wl, dev)
    groups = groups_of(L, layers)
    torch.cuda.synchronize()
    print(f"[bench] set-up {wl.name}: {layers} layers x {R} replicas, n_ctx {wl.n_ctx}, M {wl.m} in "
          f"{time.time() - t_setup:.1f} s", file=sys.stderr, flush=True)
    ms_step = timed_sweeps(Q, groups, sh, nb_max, wl, args.steps, args.warmup, args.eager)
    rows_per_s = wl.m * layers / (ms_step / 1e3)

    # per-kernel device time (dominant kernel: scoring, HBM-bound)
    kt = {kind: per_launch_us(Q, L, sh, nb_max, wl, kind) for kind in ("score", "select", "attn", "append")}
    kt["append_score"] = per_launch_us(Q, L, sh, nb_max, wl, "append_score")
    score_bytes = nb_max * 512 + wl.m * 4 * 128 * 2 + wl.m * nb_max * 4
    # the step scores through the launch that also appends: its bytes include the append's
    score_us = kt["append_score"]
    score_bytes += append_alg_bytes(L[0].new_pos.cpu().tolist(), 2)
    achieved = score_bytes / (score_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "kernel": "score_fewrow_kernel (append folded in)",
                "traffic": stored_traffic() if wl.name == "verify_262k" else None,
                "bytes_per_launch": score_bytes, "launch_us": score_us}
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
                   "layers": layers, "replicas": R, "budget_tokens": wl.k_blocks * 4, "hq": wl.hq, "hkv": wl.hkv,
                   "head_dim": wl.head_dim, "graph": not args.eager},
        "roofline": roofline,
        "path": {"layer_us": layer_us, "bytes_per_layer_step": pbytes,
                 "achieved_GBs": pbytes / (layer_us * 1e-6) / 1e9,
                 "frac": pbytes / (layer_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                 "kernel_us": {k_: round(v, 2) for k_, v in kt.items()}},
    }
    for fmt in ("fp8", "q8"):
        if fmt in args.legs and wl.name == "verify_262k":
            res[fmt] = quant_leg(Q, L, groups, sh, nb_max, wl, args, kt["attn"], fmt)
    if "m1" in args.legs and wl.name == "verify_262k":
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
        ms1 = timed_sweeps(Q, groups, sh1, nb_max, wl1, args.steps, args.warmup, args.eager)
        kt1 = {k_: per_launch_us(Q, L, sh1, nb_max, wl1, k_) for k_ in ("append_score", "select", "attn")}
        res["m1"] = leg_record("decode_262k", 1, layers, R, ms1, path_bytes(wl1, wl1.rows, nb_max), kt1)
        del sh1
    del L, sh, groups
    free()
    if wl.name == "verify_262k":
        for leg in ("decode_32k", "batched", "prefill"):
            if leg in args.legs:
                t0 = time.time()
                res[leg] = (prefill_leg(Q, args, dev) if leg == "prefill" else
                            batched_leg(Q, args, dev) if leg == "batched" else single_leg(Q, leg, args, dev))
                print(f"[bench] leg {leg} in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline()
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
