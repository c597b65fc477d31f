"""Helpers shared by the GPU parity tests: device set-up through the binding,
the selection acceptance rule and the oracle comparisons (test code only)."""
from __future__ import annotations

import concurrent.futures as cf
import math
import os

import numpy as np
import torch

import datagen
import oracle as O

DEV = "cuda"


def to_dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Host float32 array (bf16-exact when dtype == 'bf16') -> device tensor."""
    if dtype == "bf16":
        bits = datagen.bf16_bits(x).view(np.int16)
        return torch.from_numpy(bits).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def to_host_f32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def round_up(a: int, b: int) -> int:
    return -(-a // b) * b


class Layer:
    """One sequence's QSA layer state on the device, filled from host data."""

    def __init__(self, d: dict, capacity: int | None = None, prefix_split: int | None = None,
                 kv: str = "same"):
        import long_context_sparse_qsa_amd as Q

        wl = d["workload"]
        self.d = d
        self.wl = wl
        self.dtype = wl.dtype
        n = d["idx"].shape[0]
        self.n_ctx = n
        self.cap = capacity or round_up(n + 4, 256)
        tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        self.idx_cache = torch.zeros((1, self.cap, 128), dtype=tdt, device=DEV)
        self.pooled = torch.zeros((1, self.cap // 4, 128), dtype=torch.float32, device=DEV)
        idx_dev = to_dev(d["idx"], wl.dtype)
        # append the history first, then the last tokens (the rows' own) in a
        # second call, so pooling reads both cached and in-call keys
        cut = prefix_split if prefix_split is not None else max(0, n - len(d["rows"]))
        for lo, hi in ((0, cut), (cut, n)):
            if hi > lo:
                pos = torch.arange(lo, hi, dtype=torch.int64, device=DEV)
                Q.qsa_append_pool(idx_dev[lo:hi].contiguous(), pos, self.idx_cache, self.pooled)
        self.k = torch.zeros((wl.hkv, self.cap, wl.head_dim), dtype=tdt, device=DEV)
        self.v = torch.zeros_like(self.k)
        self.k[:, :n] = to_dev(d["k"], wl.dtype)
        self.v[:, :n] = to_dev(d["v"], wl.dtype)
        self.kv = Q.KvSegments.single(self.k, self.v, n)
        self.kv_mode = kv
        if kv == "q8":  # Q8_0 int8 codes + one f16 scale per 32 values, quantized on the device
            self.k8 = torch.zeros((wl.hkv, self.cap, wl.head_dim), dtype=torch.int8, device=DEV)
            self.v8 = torch.zeros_like(self.k8)
            self.ks = torch.zeros((wl.hkv, self.cap, wl.head_dim // 32), dtype=torch.float16, device=DEV)
            self.vs = torch.zeros_like(self.ks)
            Q.qsa_quantize_kv_q8_0(to_dev(d["k"], "bf16"), self.k8, self.ks)
            Q.qsa_quantize_kv_q8_0(to_dev(d["v"], "bf16"), self.v8, self.vs)
            self.kv = Q.KvSegments.single(self.k8, self.v8, n, self.ks, self.vs)
        if kv == "fp8":  # E4M3 codes + f16 scales, quantized on the device
            self.k8 = torch.zeros((wl.hkv, self.cap, wl.head_dim), dtype=torch.uint8, device=DEV)
            self.v8 = torch.zeros_like(self.k8)
            self.ks = torch.zeros((wl.hkv, self.cap), dtype=torch.float16, device=DEV)
            self.vs = torch.zeros_like(self.ks)
            Q.qsa_quantize_kv_fp8(to_dev(d["k"], "bf16"), self.k8, self.ks)
            Q.qsa_quantize_kv_fp8(to_dev(d["v"], "bf16"), self.v8, self.vs)
            self.kv = Q.KvSegments.single(self.k8, self.v8, n, self.ks, self.vs)
        self.q = to_dev(d["q"], wl.dtype)
        self.idx_q = to_dev(d["idx_q"], wl.dtype)
        self.rows = torch.from_numpy(d["rows"]).to(DEV)
        self.m = len(d["rows"])
        self.nb_max = (int(d["rows"].max()) + 1) // 4
        self.ld = max(4, round_up(self.nb_max, 4))

    def run(self, k_blocks: int | None = None):
        import long_context_sparse_qsa_amd as Q

        wl = self.wl
        k = k_blocks or wl.k_blocks
        m = self.m
        scores = torch.full((m, self.ld), -7.0, dtype=torch.float32, device=DEV)
        Q.qsa_score_blocks(self.idx_q, self.rows, self.pooled, scores, self.nb_max)
        sel = torch.empty((m, k), dtype=torch.int32, device=DEV)
        n_sel = torch.empty((m,), dtype=torch.int32, device=DEV)
        wsb = Q.qsa_select_workspace_bytes(m, self.nb_max, k)
        # the workspace needs no initialisation: start from garbage
        ws_sel = torch.randint(0, 255, (max(wsb, 1),), dtype=torch.uint8, device=DEV)
        Q.qsa_select_topk(scores, self.rows, self.nb_max, k, sel, n_sel, ws_sel)
        # the prepared path (sample stored while scoring) must give the same
        # scores and selection, call after call
        for _ in range(2):
            scores_f = torch.full_like(scores, -7.0)
            sel_f = torch.full_like(sel, -5)
            n_sel_f = torch.full_like(n_sel, -5)
            Q.qsa_score_blocks(self.idx_q, self.rows, self.pooled, scores_f, self.nb_max, sel_workspace=ws_sel)
            Q.qsa_select_topk(scores_f, self.rows, self.nb_max, k, sel_f, n_sel_f, ws_sel, prepared=True)
            torch.cuda.synchronize()
            assert torch.equal(scores_f, scores), "prepared-path scores differ"
            assert torch.equal(sel_f, sel) and torch.equal(n_sel_f, n_sel), "prepared-path selection differs"
        # word 0 of each row's workspace record: how the prepared selection went
        rec_words = Q.qsa_select_workspace_bytes(1, self.nb_max, k) // 4
        paths = ws_sel[: m * rec_words * 4].view(torch.int32).view(m, rec_words)[:, 0].cpu().numpy() \
            if rec_words > 0 else np.ones(m, dtype=np.int32)
        out = torch.empty_like(self.q)
        lse = torch.empty((m, wl.hq), dtype=torch.float32, device=DEV)
        wsa = Q.qsa_attn_workspace_bytes(m, wl.hq, wl.head_dim, k)
        ws = torch.empty(max(wsa, 1), dtype=torch.uint8, device=DEV)
        Q.qsa_gathered_attn(self.q, self.rows, self.kv, sel, n_sel, out, lse, wl.hkv,
                            scale=1.0 / math.sqrt(wl.head_dim), workspace=ws)
        torch.cuda.synchronize()
        return {"scores": scores, "sel": sel, "n_sel": n_sel, "out": out, "lse": lse, "paths": paths}


def band_mask(scores64: np.ndarray, k: int) -> tuple[np.ndarray, float]:
    """Blocks whose fp64 score lies within max(1e-5 |c|, 1e-6) of the k-th cutoff c."""
    nb = len(scores64)
    order = np.lexsort((np.arange(nb), -scores64))
    c = float(scores64[order[min(k, nb) - 1]])
    return np.abs(scores64 - c) <= max(1e-5 * abs(c), 1e-6), c


def check_selection(sel_gpu: np.ndarray, n_sel_gpu: int, scores64: np.ndarray, k: int) -> dict:
    """Acceptance: same count, ascending unique ids, and equal to the oracle's
    selection outside the near-cutoff band."""
    nb = len(scores64)
    want = O.select_blocks(scores64, k)
    assert n_sel_gpu == len(want) == min(k, nb), (n_sel_gpu, len(want))
    s = sel_gpu[:n_sel_gpu]
    assert np.all(sel_gpu[n_sel_gpu:] == -1)
    assert np.all(np.diff(s) > 0) and (len(s) == 0 or (s[0] >= 0 and s[-1] < nb))
    if nb <= k:
        assert np.array_equal(s, np.arange(nb))
        return {"band": 0}
    band, _ = band_mask(scores64, k)
    g, o = set(s.tolist()), set(want.tolist())
    bad = (g ^ o) - set(np.nonzero(band)[0].tolist())
    assert not bad, f"selection differs outside the cutoff band at blocks {sorted(bad)[:10]}"
    return {"band": int(band.sum()), "diff_in_band": len(g ^ o)}


def check_attention_fp8(out_gpu: np.ndarray, lse_gpu: np.ndarray, layer, row_i: int, sel: np.ndarray):
    """fp8 or Q8_0 K/V: the device cache holds the oracle's codes and scales
    for every attended token (bit for bit), and attention matches fp64
    attention over the oracle's dequantized rows within the bf16 tolerances."""
    d = layer.d
    wl = d["workload"]
    p = int(d["rows"][row_i])
    tok = O.attended_tokens(sel, p + 1)
    ti = torch.from_numpy(tok).to(DEV)
    quant, dequant = ((O.quantize_kv_q8_0, O.dequantize_kv_q8_0) if layer.kv_mode == "q8" else
                      (O.quantize_kv_fp8, O.dequantize_kv_fp8))
    deq = []
    for src, codes, sc in ((d["k"], layer.k8, layer.ks), (d["v"], layer.v8, layer.vs)):
        c_ref, s_ref = quant(src[:, tok])
        assert np.array_equal(codes[:, ti].cpu().numpy(), c_ref), f"{layer.kv_mode} codes differ from the oracle"
        assert np.array_equal(sc[:, ti].cpu().numpy().view(np.uint16), s_ref.view(np.uint16)), \
            f"{layer.kv_mode} scales differ"
        deq.append(dequant(c_ref, s_ref))
    ref, ref_lse = O.attend(d["q"][row_i], deq[0], deq[1], np.arange(len(tok)), 1.0 / math.sqrt(wl.head_dim))
    err = float(np.max(np.abs(out_gpu - ref)))
    lerr = float(np.max(np.abs(lse_gpu - ref_lse)))
    # as for bf16 K/V (probabilities rounded to bf16), plus one more bf16
    # rounding of each weight times its V scale; the lse comes from the
    # float32 probabilities, before any rounding
    assert err <= 2e-2, f"attention max-abs {err} > 2e-2"
    assert lerr <= 1e-3, f"lse max-abs {lerr} > 1e-3"
    return err, lerr


def check_attention(out_gpu: np.ndarray, lse_gpu: np.ndarray, d: dict, row_i: int,
                    sel: np.ndarray, dtype: str):
    """Recompute attention in fp64 over the GPU's own selection (plus tail)."""
    wl = d["workload"]
    p = int(d["rows"][row_i])
    tok = O.attended_tokens(sel, p + 1)
    ref, ref_lse = O.attend(d["q"][row_i], d["k"], d["v"], tok, 1.0 / math.sqrt(wl.head_dim))
    tol = 2e-2 if dtype == "bf16" else 1e-4
    # the output is normalised by the sum of the bf16-rounded probabilities
    # P.V consumes; the lse comes from the float32 probabilities
    ltol = 1e-3 if dtype == "bf16" else 1e-5
    err = float(np.max(np.abs(out_gpu - ref)))
    lerr = float(np.max(np.abs(lse_gpu - ref_lse)))
    assert err <= tol, f"attention max-abs {err} > {tol}"
    assert lerr <= ltol, f"lse max-abs {lerr} > {ltol}"
    return err, lerr


def host_map(fn, items):
    """fn over items, in host threads when there are many (numpy's matrix
    products and sorts release the interpreter lock); BLAS kept to one thread
    per worker meanwhile."""
    items = list(items)
    if len(items) <= 4:
        return [fn(x) for x in items]
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    workers = max(1, min(16, os.cpu_count() or 1))
    if threadpool_limits is None:
        with cf.ThreadPoolExecutor(workers) as ex:
            return list(ex.map(fn, items))
    with threadpool_limits(1), cf.ThreadPoolExecutor(workers) as ex:
        return list(ex.map(fn, items))


def check_layer(d, res, layer, k=None, rows=None, attn_rows=None):
    """Pooling bit-exact, scores within the fp64 band, selection exact on the
    GPU's scores and equal to the oracle's outside the band, attention within
    tolerance over the GPU's selection (fp8 K/V: over the oracle's
    dequantized rows).  Returns per-row statistics."""
    wl = d["workload"]
    k = k or wl.k_blocks
    n = d["idx"].shape[0]
    # index keys copied bit for bit; pooled keys bit-exact
    cache = layer.idx_cache[0, :n].float().cpu().numpy()
    assert np.array_equal(cache, d["idx"])
    pooled_gpu = layer.pooled[0, : n // 4].cpu().numpy()
    pooled_ref = O.pool_index_keys(d["idx"])
    assert np.array_equal(pooled_gpu.view(np.uint32), pooled_ref.view(np.uint32))
    pooled64 = pooled_ref.astype(np.float64)  # exact; converted once for every row
    sc = res["scores"].cpu().numpy()
    sel = res["sel"].cpu().numpy()
    n_sel = res["n_sel"].cpu().numpy()
    out = to_host_f32(res["out"])
    lse = res["lse"].cpu().numpy()
    rows = range(len(d["rows"])) if rows is None else rows
    attn_rows = set(rows if attn_rows is None else attn_rows)

    def one(i):
        p = int(d["rows"][i])
        s64 = O.score_blocks(d["idx_q"][i], pooled64, p + 1)
        nb = len(s64)
        g32 = sc[i, :nb].astype(np.float64)
        # entries past the row's block count are left untouched (the fill value)
        assert np.all(sc[i, nb:] == -7.0), f"row {i}: scores written past the row's block count"
        # scores: float32 accumulation against fp64
        assert np.all(np.abs(g32 - s64) <= 1e-5 * np.abs(s64) + 1e-6), (i, float(np.max(np.abs(g32 - s64))))
        # the select kernel is exact on its own input
        assert np.array_equal(sel[i, : n_sel[i]], O.select_blocks(g32, k)), f"row {i}: select != exact top-k of GPU scores"
        st = check_selection(sel[i], int(n_sel[i]), s64, k)
        if i in attn_rows and layer.kv_mode in ("fp8", "q8"):
            err, lerr = check_attention_fp8(out[i], lse[i], layer, i, sel[i, : n_sel[i]])
            st.update(err=err, lse_err=lerr)
        elif i in attn_rows:
            err, lerr = check_attention(out[i], lse[i], d, i, sel[i, : n_sel[i]], wl.dtype)
            st.update(err=err, lse_err=lerr)
        return st

    return host_map(one, rows)


def assert_candidate_path(res, layer, k=None):
    """Every row longer than the budget was selected from the conservative
    candidates (the exact whole-row fallback is correct but slow)."""
    k = k or layer.wl.k_blocks
    nb = (layer.rows.cpu().numpy() + 1) // 4
    want = np.where(nb <= k, 1, 2)
    assert np.array_equal(res["paths"], want), (res["paths"][:16], want[:16])
