"""Seeded synthetic workloads for one QSA layer.

Shapes follow the Flash-Next layout on the hipfire "QSA sparse attention"
page (section 02: 128-wide index keys, 4 index-query heads, 4-token pooled
blocks, 2,048-token budget) and the MTPLX PR #482 page (section 2: 24 query
heads over 2 KV heads at head_dim 256).  Values are N(0, 1); a subset of
complete 4-token blocks gets a "planted relevance" shift of its index keys
along the normalised sum of the workload's index queries.

Nothing in this module pools, scores, selects or attends.  Draws are made
with numpy's PCG64 seeded by ``SeedSequence(seed, spawn_key=(workload,
layer, tensor, chunk))`` so that every tensor chunk is reproducible on its
own and can be drawn in parallel threads.  bf16 inputs are float32 draws
rounded to nearest-even; they are returned as float32 arrays holding exactly
representable bf16 values (``bf16_bits`` gives the raw 16-bit patterns).
"""
from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from dataclasses import dataclass, field

import numpy as np

INDEX_DIM = 128
INDEX_HEADS = 4
BLOCK_TOKENS = 4

# tensor ids used in seed spawn keys
_T_IDX, _T_IDXQ, _T_Q, _T_K, _T_V, _T_PLANT, _T_ZIPF, _T_SEQLEN, _T_SEGS = range(9)
_CHUNK = 1 << 16  # rows per independently seeded chunk


@dataclass(frozen=True)
class Workload:
    """One query batch against one sequence's layer state.

    ``rows`` are absolute positions of the query rows; a row at position p
    sees tokens 0..p (inclusive causal visibility).
    """

    name: str
    wid: int
    n_ctx: int
    rows: tuple
    dtype: str  # "f32" or "bf16"
    head_dim: int
    hq: int = 24
    hkv: int = 2
    k_blocks: int = 512
    layers: int = 12
    plant: tuple = ("frac", 0.05, 0.5)
    seed: int = 0
    base: str | None = None  # draw the data of another workload, keep these rows

    @property
    def m(self) -> int:
        return len(self.rows)


@dataclass
class SeqSpec:
    """One sequence of a batched decode: context length and K/V segments."""

    n_ctx: int
    row: int
    seg_start: list = field(default_factory=list)
    seg_len: list = field(default_factory=list)
    seg_cap: list = field(default_factory=list)


def _rows(first: int, count: int) -> tuple:
    return tuple(range(first, first + count))


WORKLOADS = {
    # 1 layer, fp32, context 1,023 (tail of 3), one row at the last position,
    # head_dim 128, budget 256 tokens, 8 planted blocks at +0.8, seed 0.
    "tiny": Workload("tiny", 0, 1023, (1022,), "f32", 128, k_blocks=64, layers=1,
                     plant=("count", 8, 0.8)),
    # decode M=1 at 32,768, 5 % of blocks planted at +0.5.
    "decode_32k": Workload("decode_32k", 1, 32768, (32767,), "bf16", 256,
                           plant=("frac", 0.05, 0.5)),
    # verify M=4 at 261,122 with Zipf(1.1) planted relevance.
    "verify_262k": Workload("verify_262k", 2, 261122, _rows(261118, 4), "bf16", 256,
                            plant=("zipf", 1.1, 1.0)),
    # M=1 at 262K: the verify workload's data, last row only.
    "decode_262k": Workload("decode_262k", 2, 261122, (261121,), "bf16", 256,
                            plant=("zipf", 1.1, 1.0), base="verify_262k"),
    # 2,048-row prefill chunk at positions 200,000..202,047, 3 % planted.
    "prefill": Workload("prefill", 4, 202048, _rows(200000, 2048), "bf16", 256,
                        plant=("frac", 0.03, 0.5)),
}

BATCHED = {
    "n_seq": 16, "ctx_lo": 4096, "ctx_hi": 131072, "seg_lo": 1, "seg_hi": 5,
    "wid": 3, "dtype": "bf16", "head_dim": 256, "hq": 24, "hkv": 2,
    "k_blocks": 512, "layers": 12, "plant": ("frac", 0.05, 0.5), "seed": 0,
}


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); float32 out."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Raw bf16 bit patterns (uint16) of float32 values that are bf16-exact."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def _normal(shape, seed, *key) -> np.ndarray:
    """N(0,1) float32 of ``shape``; the leading axis is drawn in seeded chunks."""
    shape = tuple(shape)
    out = np.empty(shape, dtype=np.float32)
    lead = shape[0]
    nchunks = max(1, -(-lead // _CHUNK))

    def work(c):
        lo, hi = c * _CHUNK, min(lead, (c + 1) * _CHUNK)
        out[lo:hi] = _rng(seed, *key, c).standard_normal((hi - lo,) + shape[1:], dtype=np.float32)

    if nchunks == 1:
        work(0)
    else:
        workers = min(nchunks, max(1, min(16, os.cpu_count() or 1)))
        with _cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def planting_direction(idx_q: np.ndarray) -> np.ndarray:
    """Unit vector along the sum of all index-query heads of all rows (float64)."""
    s = np.asarray(idx_q, dtype=np.float64).reshape(-1, INDEX_DIM).sum(axis=0)
    return s / np.linalg.norm(s)


def _plant_amplitudes(nb: int, plant: tuple, seed: int, wid: int, layer: int, extra=()):
    """(block ids, amplitudes) of the planted shift among ``nb`` complete blocks."""
    kind = plant[0]
    if nb == 0:
        return np.zeros(0, np.int64), np.zeros(0, np.float64)
    if kind in ("count", "frac"):
        cnt = int(plant[1]) if kind == "count" else int(round(plant[1] * nb))
        cnt = min(cnt, nb)
        blocks = _rng(seed, wid, layer, _T_PLANT, *extra).choice(nb, size=cnt, replace=False)
        return np.sort(blocks).astype(np.int64), np.full(cnt, float(plant[2]))
    if kind == "zipf":
        s, amp = float(plant[1]), float(plant[2])
        perm = _rng(seed, wid, layer, _T_ZIPF, *extra).permutation(nb)
        ranks = np.arange(1, nb + 1, dtype=np.float64)
        return perm.astype(np.int64), amp * ranks ** (-s)
    raise ValueError(f"unknown planting {plant!r}")


def _index_keys(n_ctx, idx_q, plant, seed, wid, layer, dtype, extra=()):
    idx = _normal((n_ctx, INDEX_DIM), seed, wid, layer, _T_IDX, *extra)
    blocks, amps = _plant_amplitudes(n_ctx // BLOCK_TOKENS, plant, seed, wid, layer, extra)
    if len(blocks):
        u = planting_direction(idx_q)
        v = idx[: (n_ctx // 4) * 4].reshape(-1, BLOCK_TOKENS, INDEX_DIM)
        shift = (amps[:, None] * u[None, :]).astype(np.float32)
        v[blocks] += shift[:, None, :]
    if dtype == "bf16":
        idx = round_bf16(idx)
    return idx, blocks, amps


def gen_layer(wl: Workload | str, layer: int = 0) -> dict:
    """Draw one layer's inputs for ``wl`` on the host.

    Returns float32 arrays (bf16-exact values when ``wl.dtype == "bf16"``):
    ``idx`` [n_ctx,128] index keys, ``idx_q`` [M,4,128] index queries,
    ``q`` [M,hq,D], ``k``/``v`` [hkv,n_ctx,D], plus ``rows`` int64 [M].
    """
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    if wl.base is not None:
        base = WORKLOADS[wl.base]
        d = gen_layer(base, layer)
        keep = [base.rows.index(r) for r in wl.rows]
        for key in ("idx_q", "q"):
            d[key] = np.ascontiguousarray(d[key][keep])
        d["rows"] = np.asarray(wl.rows, dtype=np.int64)
        d["workload"] = wl
        return d
    rnd = round_bf16 if wl.dtype == "bf16" else (lambda a: a)
    m = wl.m
    idx_q = rnd(_normal((m, INDEX_HEADS, INDEX_DIM), wl.seed, wl.wid, layer, _T_IDXQ))
    q = rnd(_normal((m, wl.hq, wl.head_dim), wl.seed, wl.wid, layer, _T_Q))
    idx, blocks, amps = _index_keys(wl.n_ctx, idx_q, wl.plant, wl.seed, wl.wid, layer, wl.dtype)
    k = np.empty((wl.hkv, wl.n_ctx, wl.head_dim), np.float32)
    v = np.empty_like(k)
    for g in range(wl.hkv):
        k[g] = rnd(_normal((wl.n_ctx, wl.head_dim), wl.seed, wl.wid, layer, _T_K, g))
        v[g] = rnd(_normal((wl.n_ctx, wl.head_dim), wl.seed, wl.wid, layer, _T_V, g))
    return {"idx": idx, "idx_q": idx_q, "q": q, "k": k, "v": v,
            "rows": np.asarray(wl.rows, dtype=np.int64), "planted": blocks,
            "plant_amp": amps, "workload": wl}


def batched_specs(cfg: dict | None = None, n_seq: int | None = None,
                  ctx_lo: int | None = None, ctx_hi: int | None = None) -> list:
    """Per-sequence context lengths and K/V segment tables (seeded).

    Context n ~ U{ctx_lo..ctx_hi}; the row sits at p = n-1.  Each sequence
    holds its K/V in 1..5 segments with seeded cut points; every segment is
    allocated on its own with capacity = its length, except the growing last
    segment, whose capacity is rounded up to a multiple of 256 tokens.
    """
    c = dict(BATCHED if cfg is None else cfg)
    if n_seq is not None:
        c["n_seq"] = n_seq
    if ctx_lo is not None:
        c["ctx_lo"] = ctx_lo
    if ctx_hi is not None:
        c["ctx_hi"] = ctx_hi
    r = _rng(c["seed"], c["wid"], 0, _T_SEQLEN)
    lens = r.integers(c["ctx_lo"], c["ctx_hi"] + 1, size=c["n_seq"])
    specs = []
    for i, n in enumerate(lens):
        n = int(n)
        rs = _rng(c["seed"], c["wid"], 0, _T_SEGS, i)
        nseg = int(rs.integers(c["seg_lo"], c["seg_hi"] + 1))
        cuts = np.sort(rs.choice(np.arange(1, n), size=nseg - 1, replace=False)) if nseg > 1 else []
        bounds = [0] + [int(x) for x in cuts] + [n]
        st = bounds[:-1]
        ln = [bounds[j + 1] - bounds[j] for j in range(nseg)]
        cap = list(ln)
        cap[-1] = -(-ln[-1] // 256) * 256
        specs.append(SeqSpec(n_ctx=n, row=n - 1, seg_start=st, seg_len=ln, seg_cap=cap))
    return specs


def gen_batched_layer(specs: list, layer: int = 0, cfg: dict | None = None) -> list:
    """Host inputs for each sequence of a batched decode (one row each)."""
    c = dict(BATCHED if cfg is None else cfg)
    rnd = round_bf16 if c["dtype"] == "bf16" else (lambda a: a)
    D, hq, hkv, seed, wid = c["head_dim"], c["hq"], c["hkv"], c["seed"], c["wid"]
    out = []
    for i, sp in enumerate(specs):
        idx_q = rnd(_normal((1, INDEX_HEADS, INDEX_DIM), seed, wid, layer, _T_IDXQ, i))
        q = rnd(_normal((1, hq, D), seed, wid, layer, _T_Q, i))
        idx, blocks, amps = _index_keys(sp.n_ctx, idx_q, c["plant"], seed, wid, layer,
                                        c["dtype"], extra=(i,))
        k = np.empty((hkv, sp.n_ctx, D), np.float32)
        v = np.empty_like(k)
        for g in range(hkv):
            k[g] = rnd(_normal((sp.n_ctx, D), seed, wid, layer, _T_K, i, g))
            v[g] = rnd(_normal((sp.n_ctx, D), seed, wid, layer, _T_V, i, g))
        out.append({"idx": idx, "idx_q": idx_q, "q": q, "k": k, "v": v,
                    "rows": np.asarray([sp.row], np.int64), "spec": sp})
    return out


def fill_layer_device(wl: Workload, layer: int, idx, idx_q, q, k, v, seed_offset: int = 0):
    """Fill preallocated device tensors with one layer of ``wl``-shaped data.

    Used where drawing on the host would take minutes (12 full-size layers).
    The values follow the same recipe as :func:`gen_layer` (N(0,1), planted
    shift along the normalised index-query sum, bf16 rounding by the tensor
    dtype) but come from torch's device generator, so they differ from the
    host draws.  ``idx``: [n_ctx,128]; ``idx_q``: [M,4,128]; ``q``: [M,hq,D];
    ``k``/``v``: [hkv, cap, D] (only the first n_ctx rows are filled).
    """
    import torch

    dev = idx.device
    g = torch.Generator(device=dev)
    g.manual_seed(int(wl.seed) * 1_000_003 + wl.wid * 10_007 + layer * 101 + seed_offset)
    iq = torch.randn(idx_q.shape, generator=g, device=dev, dtype=torch.float32)
    idx_q.copy_(iq)
    q.copy_(torch.randn(q.shape, generator=g, device=dev, dtype=torch.float32))
    n = wl.n_ctx
    x = torch.randn((n, INDEX_DIM), generator=g, device=dev, dtype=torch.float32)
    u = idx_q.float().reshape(-1, INDEX_DIM).double().sum(0)
    u = (u / u.norm()).float()
    nb = n // BLOCK_TOKENS
    kind = wl.plant[0]
    xb = x[: nb * BLOCK_TOKENS].view(nb, BLOCK_TOKENS, INDEX_DIM)
    if kind in ("count", "frac"):
        cnt = int(wl.plant[1]) if kind == "count" else int(round(wl.plant[1] * nb))
        sel = torch.randperm(nb, generator=g, device=dev)[:cnt]
        xb[sel] += float(wl.plant[2]) * u
    elif kind == "zipf":
        perm = torch.randperm(nb, generator=g, device=dev)
        ranks = torch.arange(1, nb + 1, device=dev, dtype=torch.float64)
        amp = (float(wl.plant[2]) * ranks.pow(-float(wl.plant[1]))).float()
        xb[perm] += amp[:, None, None] * u[None, None, :]
    idx.copy_(x)
    for t in (k, v):
        for h in range(t.shape[0]):
            t[h, :n].copy_(torch.randn((n, t.shape[2]), generator=g, device=dev, dtype=torch.float32))
    return u
