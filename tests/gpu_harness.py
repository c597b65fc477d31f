"""Helpers shared by the GPU parity tests: device set-up through the binding,
the selection acceptance rule and the oracle comparisons (test code only)."""
from __future__ import annotations

import math

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

    def __init__(self, d: dict, capacity: int | None = None, prefix_split: int | None = None):
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


def check_attention(out_gpu: np.ndarray, lse_gpu: np.ndarray, d: dict, row_i: int,
                    sel: np.ndarray, dtype: str):
    """Recompute attention in fp64 over the GPU's own selection (plus tail)."""
    wl = d["workload"]
    p = int(d["rows"][row_i])
    tok = O.attended_tokens(sel, p + 1)
    ref, ref_lse = O.attend(d["q"][row_i], d["k"], d["v"], tok, 1.0 / math.sqrt(wl.head_dim))
    tol = 2e-2 if dtype == "bf16" else 1e-4
    # bf16 K/V: the kernel rounds each probability to bf16 (relative error at
    # most 2^-9) and normalises by the sum of the rounded values, so lse may
    # differ by up to log(1 + 2^-9) ~ 1.95e-3 when a few tokens dominate
    ltol = 2.5e-3 if dtype == "bf16" else 1e-5
    err = float(np.max(np.abs(out_gpu - ref)))
    lerr = float(np.max(np.abs(lse_gpu - ref_lse)))
    assert err <= tol, f"attention max-abs {err} > {tol}"
    assert lerr <= ltol, f"lse max-abs {lerr} > {ltol}"
    return err, lerr
