"""GPU parity of the memory-flat score -> top-k (``qsa_score_select``):
many rows of one sequence selected without a score matrix.

Bar: the selection equals, row for row and bit for bit, the materialized
path's (``qsa_score_blocks`` + ``qsa_select_topk``, the same matrix-core
scores), which is itself checked against the oracle; every long row takes
the candidate path except rows built to fail it (all-tie rows), which take
the exact whole-row path and still select exactly.
"""
import sys

import numpy as np
import pytest
import torch

import datagen
import oracle as O

pytestmark = pytest.mark.gpu

from gpu_harness import DEV, Layer, check_layer, check_selection  # noqa: E402


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def Q():
    import long_context_sparse_qsa_amd as Q
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    Q.qsa_device_check()
    return Q


def _flat(Q, layer, k):
    m = layer.m
    sel = torch.full((m, k), -5, dtype=torch.int32, device=DEV)
    n_sel = torch.full((m,), -5, dtype=torch.int32, device=DEV)
    wsb = Q.qsa_score_select_workspace_bytes(m, layer.nb_max, k)
    # no initialisation needed: start from garbage
    ws = torch.randint(0, 255, (wsb,), dtype=torch.uint8, device=DEV)
    Q.qsa_score_select(layer.idx_q, layer.rows, layer.pooled, layer.nb_max, k, sel, n_sel, ws)
    torch.cuda.synchronize()
    r64 = -(-m // 64) * 64
    paths = ws.view(torch.int32)[2 * r64: 2 * r64 + m].cpu().numpy()
    return sel, n_sel, paths, ws


def _want_paths(layer, k):
    nb = (layer.rows.cpu().numpy() + 1) // 4
    return np.where(nb <= k, 1, 2)


def test_flat_prefill_full_size_equals_materialized(Q):
    """2,048 rows at 200,000..202,047 (the prefill chunk at full size): the
    flat selection equals the materialized one on every row, and every row's
    selection is checked against the oracle (scores within the fp64 band,
    the exact top-k of the GPU's scores, equal to the oracle's outside the
    band)."""
    say("flat select, prefill 2048 rows at 200000 (full size, every row)")
    d = datagen.gen_layer("prefill")
    layer = Layer(d, prefix_split=200000)
    res = layer.run()
    k = layer.wl.k_blocks
    sel, n_sel, paths, _ = _flat(Q, layer, k)
    assert np.array_equal(paths, _want_paths(layer, k)), np.unique(paths, return_counts=True)
    assert torch.equal(n_sel, res["n_sel"])
    assert torch.equal(sel, res["sel"]), int((sel != res["sel"]).any(dim=1).sum())
    flat_res = dict(res, sel=sel, n_sel=n_sel)
    st = check_layer(d, flat_res, layer, attn_rows=[])
    assert len(st) == 2048
    say(f"{len(st)} rows; band sizes up to {max(x['band'] for x in st)}")


def test_flat_many_rows_ragged_and_short(Q):
    """Rows with no complete block, with nb <= k, ending inside a tile, and a
    partial 128-row tile, next to long rows."""
    say("flat select, 137 scattered rows of a 32K context")
    base = datagen.gen_layer("decode_32k")
    d = dict(base)
    rng = np.random.default_rng(17)
    fixed = [0, 1, 2, 3, 4, 7, 63, 64, 255, 2047, 2048, 2050, 2051, 4099]
    rest = rng.choice(np.arange(5, 32768), 123, replace=False)
    rows = np.sort(np.unique(np.concatenate([fixed, rest]))).astype(np.int64)
    m = len(rows)
    d["rows"] = rows
    d["idx_q"] = datagen.round_bf16(rng.standard_normal((m, 4, 128)).astype(np.float32))
    d["q"] = datagen.round_bf16(rng.standard_normal((m, 24, 256)).astype(np.float32))
    layer = Layer(d, prefix_split=32768)
    res = layer.run()
    k = layer.wl.k_blocks
    sel, n_sel, paths, _ = _flat(Q, layer, k)
    assert np.array_equal(paths, _want_paths(layer, k)), paths
    assert torch.equal(n_sel, res["n_sel"]) and torch.equal(sel, res["sel"])
    say(len(check_layer(d, res, layer, attn_rows=[])), "rows checked")


def test_flat_all_tie_rows_take_the_exact_path(Q):
    """Zero index queries score every block 0: all keys tie, every block is a
    candidate (more than the 4,096 slots), and the exact whole-row path keeps
    the k lowest ids.  Mixed with ordinary rows in one call."""
    say("flat select, all-tie rows (exact fallback)")
    base = datagen.gen_layer("decode_32k")
    d = dict(base)
    rows = np.array([9000, 20000, 32767, 32000, 25000], dtype=np.int64)
    rng = np.random.default_rng(23)
    q = datagen.round_bf16(rng.standard_normal((5, 4, 128)).astype(np.float32))
    q[1] = 0.0
    q[3] = 0.0
    d["rows"] = rows
    d["idx_q"] = q
    d["q"] = datagen.round_bf16(rng.standard_normal((5, 24, 256)).astype(np.float32))
    layer = Layer(d, prefix_split=32768)
    res = layer.run()
    k = layer.wl.k_blocks
    sel, n_sel, paths, _ = _flat(Q, layer, k)
    assert paths.tolist() == [2, 4, 2, 4, 2], paths
    assert torch.equal(n_sel, res["n_sel"]) and torch.equal(sel, res["sel"])
    s = sel.cpu().numpy()
    assert np.array_equal(s[1], np.arange(k)) and np.array_equal(s[3], np.arange(k))
    pooled = O.pool_index_keys(d["idx"])
    for i in (0, 2, 4):
        s64 = O.score_blocks(d["idx_q"][i], pooled, int(rows[i]) + 1)
        check_selection(s[i], int(n_sel[i]), s64, k)


def test_flat_small_budget_and_ties_at_the_cut(Q):
    """k = 64 with duplicated pooled keys, so equal scores straddle the cut and
    the lowest ids must win among them."""
    say("flat select, k = 64 with duplicated blocks")
    base = datagen.gen_layer("decode_32k")
    d = dict(base)
    idx = d["idx"].copy()
    # blocks 100..199 repeat block 50's four keys: 101 equal top scores per
    # row, more than k, so the cut falls inside the equal group
    for b in range(100, 200):
        idx[4 * b:4 * b + 4] = idx[200:204]
    d["idx"] = idx
    rng = np.random.default_rng(29)
    rows = np.array([8191, 16383, 32767], dtype=np.int64)
    # queries along block 50's pooled key so the duplicates rank near the top
    pk = O.pool_index_keys(idx[200:204])[0]
    q = datagen.round_bf16((rng.standard_normal((3, 4, 128)) * 0.3 + pk[None, None, :]).astype(np.float32))
    d["rows"] = rows
    d["idx_q"] = q
    d["q"] = datagen.round_bf16(rng.standard_normal((3, 24, 256)).astype(np.float32))
    layer = Layer(d, prefix_split=32768)
    k = 64
    res = layer.run(k_blocks=k)
    sel, n_sel, paths, _ = _flat(Q, layer, k)
    assert torch.equal(n_sel, res["n_sel"]) and torch.equal(sel, res["sel"])
    assert np.all(paths == 2), paths
    s_ = sel.cpu().numpy()
    assert all(np.array_equal(s_[i], np.concatenate([[50], np.arange(100, 163)])) for i in range(3)), s_[:, :8]
    say(check_layer(d, res, layer, k=k, attn_rows=[]))


def test_flat_every_block_a_candidate(Q):
    """2,048 short rows at positions 2,100..4,147 (525..1,037 blocks): rows
    whose sample is too small to set a threshold make every visible block a
    candidate, so a row's candidate count must equal its block count.  Every
    scoring workgroup's run (one or two 64-block tiles here: 17 tiles over 16
    runs per 128-row tile) starts with an empty record for the group before
    its first, which must add no candidate."""
    say("flat select, 2048 short rows where every block is a candidate")
    base = datagen.gen_layer("decode_32k")
    d = dict(base)
    rng = np.random.default_rng(31)
    m = 2048
    rows = np.arange(2100, 2100 + m, dtype=np.int64)
    d["rows"] = rows
    d["idx_q"] = datagen.round_bf16(rng.standard_normal((m, 4, 128)).astype(np.float32))
    d["q"] = datagen.round_bf16(rng.standard_normal((m, 24, 256)).astype(np.float32))
    layer = Layer(d, prefix_split=32768)
    k = layer.wl.k_blocks
    n_tiles = -(-layer.nb_max // 64)
    runs = -(-256 // -(-m // 128))  # the scorer's runs per 128-row tile
    assert n_tiles > runs, (n_tiles, runs)  # some runs hold two tiles
    res = layer.run()
    sel, n_sel, paths, ws = _flat(Q, layer, k)
    assert np.array_equal(paths, _want_paths(layer, k)), np.unique(paths, return_counts=True)
    r64 = -(-m // 64) * 64
    words = ws.view(torch.int32).cpu().numpy().view(np.uint32)
    thr, cnt = words[:m], words[r64:r64 + m]
    nb = (rows + 1) // 4
    every = (thr == 0) & (nb > k)
    assert every.sum() > 100, int(every.sum())
    assert np.array_equal(cnt[every], nb[every]), (cnt[every][:8], nb[every][:8])
    assert torch.equal(n_sel, res["n_sel"]) and torch.equal(sel, res["sel"])
    say(f"{int(every.sum())} rows with every block a candidate")


def test_flat_candidates_past_the_first_slot_load(Q):
    """Rows of 1,600..1,727 blocks whose scores all fall in one histogram
    digit: every index key is 1 + j/128 (j = 0..7, drawn per token) on
    dimension 0 and zero elsewhere, and each row's query is 1 on dimension 0
    of one head, so its scores take 27 distinct values within 6 % and every
    block is a candidate -- more than the 1,536 slots the finalize loads with
    the count, so it loads the rest in a second round trip.  The cut's ties
    (about 120) fit the on-chip tie list, so these rows take the candidate
    path.  One row in eight has zero queries instead: every block ties at
    score 0, more than the tie list holds, and the exact whole-row path keeps
    the k lowest ids.  Every selection equals the materialized path's."""
    say("flat select, rows with 1,600..1,727 candidates")
    base = datagen.gen_layer("decode_32k")
    d = dict(base)
    rng = np.random.default_rng(37)
    n_ctx = d["idx"].shape[0]
    idx = np.zeros((n_ctx, 128), dtype=np.float32)
    idx[:, 0] = 1.0 + rng.integers(0, 8, size=n_ctx) / 128.0  # exact in bf16
    d["idx"] = idx
    m = 256
    rows = np.arange(6400, 6400 + 2 * m, 2, dtype=np.int64)
    q = np.zeros((m, 4, 128), dtype=np.float32)
    tie = np.arange(m) % 8 == 7
    for i in np.flatnonzero(~tie):
        q[i, i % 4, 0] = 1.0
    d["rows"] = rows
    d["idx_q"] = q
    d["q"] = datagen.round_bf16(rng.standard_normal((m, 24, 256)).astype(np.float32))
    layer = Layer(d, prefix_split=32768)
    k = layer.wl.k_blocks
    res = layer.run()
    sel, n_sel, paths, ws = _flat(Q, layer, k)
    assert np.array_equal(paths, np.where(tie, 5, 2)), np.unique(paths, return_counts=True)
    r64 = -(-m // 64) * 64
    cnt = ws.view(torch.int32).cpu().numpy().view(np.uint32)[r64:r64 + m]
    nb = (rows + 1) // 4
    assert np.array_equal(cnt, nb) and (cnt > 1536).all(), cnt[:8]
    assert torch.equal(n_sel, res["n_sel"]) and torch.equal(sel, res["sel"])
    s = sel.cpu().numpy()
    assert (s[tie] == np.arange(k)).all()
    pooled = O.pool_index_keys(d["idx"])
    for i in list(np.flatnonzero(~tie)[:4]) + [int(np.flatnonzero(tie)[0])]:
        s64 = O.score_blocks(d["idx_q"][i], pooled, int(rows[i]) + 1)
        check_selection(s[i], int(n_sel[i]), s64, k)
