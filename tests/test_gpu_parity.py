"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bar: index keys and pooled keys bit-exact; selection bit-exact against the
oracle's own selection rule applied to the GPU's float32 scores, and equal
to the oracle's fp64 selection outside the near-cutoff band; attention
within max-abs 2e-2 (bf16 K/V) / 1e-4 (fp32), recomputed in fp64 over the
GPU's selection plus the tail.
"""
import math
import sys

import numpy as np
import pytest
import torch

import datagen
import oracle as O

pytestmark = pytest.mark.gpu

from gpu_harness import DEV, Layer, check_attention, check_selection, to_dev, to_host_f32  # noqa: E402
from gpu_harness import assert_candidate_path as _assert_candidate_path  # noqa: E402
from gpu_harness import check_layer as _check_layer  # noqa: E402


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def Q():
    import long_context_sparse_qsa_amd as Q
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    Q.qsa_device_check()
    return Q


def test_tiny_fp32(Q):
    say("tiny fp32 N=1023")
    d = datagen.gen_layer("tiny")
    layer = Layer(d)
    res = layer.run()
    st = _check_layer(d, res, layer)
    say(st)
    # the planted blocks are found
    assert len(set(d["planted"].tolist()) & set(res["sel"][0].cpu().tolist())) >= 6


def test_tiny_budget_covers_context_is_dense(Q):
    say("tiny with budget >= context")
    d = datagen.gen_layer("tiny")
    layer = Layer(d)
    res = layer.run(k_blocks=256)
    assert int(res["n_sel"][0]) == 255
    st = _check_layer(d, res, layer, k=256)
    say(st)


def test_decode_32k(Q):
    say("decode M=1 at 32768 bf16")
    d = datagen.gen_layer("decode_32k")
    layer = Layer(d)
    res = layer.run()
    say(_check_layer(d, res, layer))
    _assert_candidate_path(res, layer)


@pytest.mark.parametrize("name,k", [("verify_262k", 1024), ("verify_262k", 1), ("decode_32k", 1024),
                                    ("decode_32k", 1)])
def test_budget_extremes(Q, name, k):
    """The largest budget the library serves (QSA_MAX_K_BLOCKS = 1,024 blocks,
    4,096 tokens: the attention plans walk twice the slices, the selections
    keep twice the candidates) and the smallest (one block plus the tail),
    at full size through the chunked selection (262K) and the one-workgroup
    selection (32K)."""
    say("budget extremes", name, "k =", k)
    d = datagen.gen_layer(name)
    layer = Layer(d)
    res = layer.run(k_blocks=k)
    st = _check_layer(d, res, layer, k=k)
    nb = (layer.rows.cpu().numpy() + 1) // 4
    assert np.array_equal(res["n_sel"].cpu().numpy(), np.minimum(nb, k))
    _assert_candidate_path(res, layer, k=k)
    say(f"{len(st)} rows; band sizes up to {max(x['band'] for x in st)}")


def test_decode_32k_layers_differ(Q):
    say("decode 32k, layer 5")
    d = datagen.gen_layer("decode_32k", layer=5)
    layer = Layer(d)
    say(_check_layer(d, layer.run(), layer))


def test_verify_262k_full_size(Q):
    say("verify M=4 at 261122 bf16 (full size)")
    d = datagen.gen_layer("verify_262k")
    layer = Layer(d)
    res = layer.run()
    say(_check_layer(d, res, layer))
    _assert_candidate_path(res, layer)


def test_decode_262k_full_size(Q):
    say("decode M=1 at 261122 bf16 (full size)")
    d = datagen.gen_layer("decode_262k")
    layer = Layer(d)
    res = layer.run()
    say(_check_layer(d, res, layer))
    _assert_candidate_path(res, layer)


def test_clustered_relevance_full_size(Q):
    """Relevance concentrated in 1,000 consecutive blocks: one 4,096-block
    chunk then holds most of the candidates, more than its share of the
    selection's first (speculative) gather, so the second gather path runs."""
    say("verify M=4 at 261122, relevance clustered in blocks 40000..40999")
    d = dict(datagen.gen_layer("verify_262k"))
    idx = d["idx"].copy()
    u = datagen.planting_direction(d["idx_q"]).astype(np.float32)
    lo, hi = 40000 * 4, 41000 * 4
    idx[lo:hi] = datagen.round_bf16(idx[lo:hi] + np.float32(6.0) * u[None, :])
    d["idx"] = idx
    layer = Layer(d)
    res = layer.run()
    st = _check_layer(d, res, layer)
    sel = res["sel"].cpu().numpy()
    # chunk 9 = blocks 36,864..40,959; with 16 chunks each chunk's speculative
    # share is 256 candidates, and every kept block was a candidate
    in_chunk = ((sel >= 9 * 4096) & (sel < 10 * 4096)).sum(axis=1)
    assert np.all(in_chunk > 256), in_chunk
    _assert_candidate_path(res, layer)
    say(st, in_chunk)


def prefill_attention_rows(m: int = 2048, tile: int = 64) -> list:
    """8 rows of every 64-row tile (first, last and six inside): 256 rows at
    the 2,048-row chunk, spread over every tile of the many-row scorer and
    every workgroup position of the attention launch."""
    offs = (0, 7, 15, 21, 31, 42, 55, 63)
    return [t + o for t in range(0, m, tile) for o in offs if t + o < m]


def test_prefill_full_size_all_rows(Q):
    """The 2,048-row prefill chunk at 200,000..202,047: scores and selection
    of every row against the oracle, attention of 256 rows (8 per 64-row
    tile) over the GPU's selection.  The attention plan walks 17 tiles of 128
    tokens per (row, KV head) in one split."""
    say("prefill 2048 rows at 200000 bf16 (full size, every row)")
    plan = Q.qsa_attn_plan(2048, 2, 512)
    assert plan["tiles_per_split"] == 17 and plan["splits"] == 1, plan
    d = datagen.gen_layer("prefill")
    layer = Layer(d, prefix_split=200000)
    res = layer.run()
    st = _check_layer(d, res, layer, attn_rows=prefill_attention_rows())
    _assert_candidate_path(res, layer)
    errs = [x["err"] for x in st if "err" in x]
    lerrs = [x["lse_err"] for x in st if "lse_err" in x]
    assert len(errs) == 256
    say(f"{len(st)} rows; attention max-abs {max(errs):.3g}, lse {max(lerrs):.3g}; "
        f"band sizes up to {max(x['band'] for x in st)}")


def test_many_rows_ragged(Q):
    """131 bf16 rows of one sequence at scattered positions -- rows with fewer
    blocks than one 64-block tile, rows ending inside a tile, a partial
    second 128-row tile: the many-row matrix-core scoring path."""
    say("many rows (131) at scattered positions of a 32,768-token context")
    base = datagen.gen_layer("decode_32k")
    d = dict(base)
    rng = np.random.default_rng(7)
    fixed = [0, 1, 2, 3, 4, 63, 64, 255, 256, 257, 2050]
    rest = rng.choice(np.arange(5, 32768), 120, replace=False)
    rows = np.sort(np.unique(np.concatenate([fixed, rest]))).astype(np.int64)
    m = len(rows)
    d["rows"] = rows
    d["idx_q"] = datagen.round_bf16(rng.standard_normal((m, 4, 128)).astype(np.float32))
    d["q"] = datagen.round_bf16(rng.standard_normal((m, 24, 256)).astype(np.float32))
    layer = Layer(d, prefix_split=32768)
    res = layer.run()
    st = _check_layer(d, res, layer, attn_rows=[0, 4, 5, 10, m - 1])
    _assert_candidate_path(res, layer)
    say(len(st), "rows checked")


@pytest.mark.parametrize("rows", [(0,), (1,), (2,), (3,), (4,), (5, 6, 7), (30, 100, 255),
                                  (1019, 1020, 1021, 1022)])
def test_short_and_ragged_rows(Q, rows):
    """Rows with nb <= k (every block kept), empty block sets (tail only) and
    ragged tails inside one call."""
    say("ragged rows", rows)
    base = datagen.gen_layer("tiny")
    d = dict(base)
    d["rows"] = np.asarray(rows, dtype=np.int64)
    rng = np.random.default_rng(sum(rows))
    d["idx_q"] = rng.standard_normal((len(rows), 4, 128)).astype(np.float32)
    d["q"] = rng.standard_normal((len(rows), 24, 128)).astype(np.float32)
    layer = Layer(d, prefix_split=1023)
    res = layer.run(k_blocks=16)
    say(_check_layer(d, res, layer, k=16))


def test_thirteen_rows_two_row_groups(Q):
    """13 bf16 rows of one sequence at scattered positions of a 32K context:
    the few-row scorer's 8-row groups (a full one and a ragged one of 5, two
    column sets each), the selection and the attention plan for M = 13."""
    say("13 rows, decode_32k context")
    d = dict(datagen.gen_layer("decode_32k"))
    n = d["idx"].shape[0]
    rows = np.asarray([n - 1, n - 2, n - 3, n - 4, n - 5, n - 9, n - 17, n - 100, n - 777, n - 2048, n - 4097,
                       n - 9001, 5000], dtype=np.int64)
    d["rows"] = rows
    rng = np.random.default_rng(13)
    d["idx_q"] = datagen.round_bf16(rng.standard_normal((len(rows), 4, 128)).astype(np.float32))
    d["q"] = datagen.round_bf16(rng.standard_normal((len(rows), 24, 256)).astype(np.float32))
    layer = Layer(d, prefix_split=n - 4)
    res = layer.run()
    say(_check_layer(d, res, layer))
    _assert_candidate_path(res, layer)


def _context_prefix(name, n):
    """The first n tokens of a workload's layer (index keys, K, V)."""
    d = dict(datagen.gen_layer(name))
    d["idx"] = np.ascontiguousarray(d["idx"][:n])
    d["k"] = np.ascontiguousarray(d["k"][:, :n])
    d["v"] = np.ascontiguousarray(d["v"][:, :n])
    return d


@pytest.mark.parametrize("n_ctx", [32768, 40000, 65536])
def test_many_rows_selection_paths(Q, n_ctx):
    """288 bf16 rows of one sequence.  Rows 0..95 sit in the first 2,048
    tokens (at most k blocks: all kept), rows 96..191 have zero index queries
    (every score 0: every block is a candidate and ties at the cut; the lowest
    ids are kept), rows 192..287 are ordinary.  Every row's selection is the
    exact top-k of the GPU scores and its path word says how it went.  The
    context picks the selection's form: 8,192 blocks one workgroup per row,
    10,000 blocks the one-launch collect + finalize (3 chunks x 288 rows),
    16,384 blocks the separate threshold, collect and finalize launches
    (4 chunks x 288 rows is more than the one-launch form takes)."""
    say("288 rows, selection paths, context", n_ctx)
    d = dict(datagen.gen_layer("decode_32k")) if n_ctx == 32768 else _context_prefix("verify_262k", n_ctx)
    n = d["idx"].shape[0]
    assert n == n_ctx
    rng = np.random.default_rng(288)
    rows = np.concatenate([rng.integers(0, 2048, 96), rng.integers(8192, n, 96), rng.integers(8192, n, 96)])
    d["rows"] = rows.astype(np.int64)
    idx_q = datagen.round_bf16(rng.standard_normal((288, 4, 128)).astype(np.float32))
    idx_q[96:192] = 0.0
    d["idx_q"] = idx_q
    d["q"] = datagen.round_bf16(rng.standard_normal((288, 24, 256)).astype(np.float32))
    layer = Layer(d, prefix_split=n - 4)
    # the form this context is meant to exercise (4,096-block chunks)
    chunks = -(-layer.nb_max // 4096)
    assert {32768: layer.nb_max <= 8192, 40000: chunks == 3, 65536: chunks == 4}[n_ctx], layer.nb_max
    res = layer.run()
    st = _check_layer(d, res, layer, rows=list(range(0, 288, 7)), attn_rows=[0, 100, 200, 287])
    say(st[:3])
    k = d["workload"].k_blocks
    nb = (rows + 1) // 4
    want = np.where(nb <= k, 1, 2)
    # all-equal rows: more candidates than the 4,096 the finalize pass holds
    # -> exact by count (4); else the candidates' levels end on one cut bin of
    # equal keys, ranked by block id (2)
    zb = nb[96:192]
    want[96:192] = np.where(zb <= k, 1, np.where(zb > 4096, 4, 2))
    assert {2, 4} <= set(want[96:192].tolist())
    assert np.array_equal(res["paths"], want), (res["paths"][:8], res["paths"][96:104])
    sel = res["sel"].cpu().numpy()
    for i in range(96, 192):
        assert np.array_equal(sel[i], np.arange(k)), i


@pytest.mark.parametrize("accepted", [0, 1, 2, 3])
def test_verify_rollback_reappend(Q, accepted):
    """Speculative verify with rollback (MTPLX PR #482, section 3,
    optimization 1: in-place verify write, rollback by trimming).  A verify
    writes 4 index keys in place, pooling the block they complete; only
    ``accepted`` of them are kept and the length goes back; the next verify
    writes 4 keys from there.  Nothing is restored: positions are explicit,
    rows past the length are never read, and a block's pooled key is rebuilt
    from its four cached keys whenever its last token is written, so the block
    the rejected keys completed is pooled again when it completes again.  With
    accepted = 0..3 the first verify starts at every block offset.  Cache and
    pooled keys must equal a from-scratch build of the accepted history byte
    for byte, and the layer on the rolled-back state must pass the oracle."""
    say(f"verify rollback, {accepted} of 4 accepted, 32K context")
    base = datagen.gen_layer("decode_32k")
    n = base["idx"].shape[0] - 1          # accepted history after the second verify
    n0 = n - 4 - accepted                 # length before the first verify
    d = dict(base)
    d["idx"] = np.ascontiguousarray(base["idx"][:n])
    d["k"] = np.ascontiguousarray(base["k"][:, :n])
    d["v"] = np.ascontiguousarray(base["v"][:, :n])
    d["rows"] = np.asarray([n - 1], dtype=np.int64)
    layer = Layer(d)                      # the accepted history, appended from scratch
    rng = np.random.default_rng(100 + accepted)
    rejected = datagen.round_bf16(rng.standard_normal((4 - accepted, 128)).astype(np.float32))
    cache = torch.zeros_like(layer.idx_cache)
    pooled = torch.zeros_like(layer.pooled)

    def append(keys, lo):
        pos = torch.arange(lo, lo + len(keys), dtype=torch.int64, device=DEV)
        Q.qsa_append_pool(to_dev(np.ascontiguousarray(keys), "bf16"), pos, cache, pooled)

    append(d["idx"][:n0], 0)
    append(np.concatenate([d["idx"][n0:n0 + accepted], rejected]), n0)   # first verify
    torch.cuda.synchronize()
    last = n0 + (3 - n0) % 4              # the one position of the verify that ends a block
    cb = last // 4                        # the block the first verify completed ...
    assert last >= n0 + accepted          # ... holds a rejected key
    stale = pooled[0, cb].clone()
    append(d["idx"][n0 + accepted:n], n0 + accepted)                      # second verify
    torch.cuda.synchronize()
    nb = n // 4
    assert not torch.equal(stale.view(torch.int32), pooled[0, cb].view(torch.int32)), "block not re-pooled"
    assert torch.equal(cache[:, :n], layer.idx_cache[:, :n])
    assert torch.equal(pooled[:, :nb].view(torch.int32), layer.pooled[:, :nb].view(torch.int32))
    layer.idx_cache, layer.pooled = cache, pooled
    res = layer.run()
    say(_check_layer(d, res, layer))
    _assert_candidate_path(res, layer)


def test_row_without_visible_token_gives_zeros(Q):
    say("row at position -1")
    d = dict(datagen.gen_layer("tiny"))
    d["rows"] = np.asarray([-1, 1022], dtype=np.int64)
    d["q"] = np.concatenate([d["q"], d["q"]])
    d["idx_q"] = np.concatenate([d["idx_q"], d["idx_q"]])
    layer = Layer(d, prefix_split=1023)
    res = layer.run()
    assert int(res["n_sel"][0]) == 0
    out = res["out"].cpu().numpy()
    lse = res["lse"].cpu().numpy()
    assert np.all(out[0] == 0) and np.all(np.isneginf(lse[0]))
    assert np.all(np.isfinite(out[1]))


def test_zero_queries_tie_rule(Q):
    """All index queries zero: every score is 0 and the lowest k blocks win."""
    say("zero index queries")
    d = dict(datagen.gen_layer("decode_32k"))
    d["idx_q"] = np.zeros_like(d["idx_q"])
    layer = Layer(d)
    res = layer.run()
    assert np.all(res["scores"][0, : 8192].cpu().numpy() == 0)
    assert res["sel"][0].cpu().tolist() == list(range(512))


def test_deterministic_bitwise(Q):
    say("determinism")
    d = datagen.gen_layer("decode_32k")
    layer = Layer(d)
    a = layer.run()
    b = layer.run()
    for key in ("scores", "sel", "n_sel", "lse"):
        assert torch.equal(a[key], b[key]), key
    assert torch.equal(a["out"].view(torch.int16), b["out"].view(torch.int16))


def _segmented_case(Q, n_ctx_list, nseg_list, seed, k=512, head_dim=256, quant=None):
    """Sequences with K/V in several segments (some empty, some cutting a
    4-token block), one row per sequence, scored and attended in one call.
    With quant ("fp8" or "q8") every segment holds codes and f16 scales
    quantized on the device from the bf16 rows (checked bit for bit against
    the oracle), and attention is compared with the oracle's dequantized
    K/V."""
    import dataclasses

    rng = np.random.default_rng(seed)
    wl = dataclasses.replace(datagen.WORKLOADS["decode_32k"], head_dim=head_dim)
    D = head_dim
    n_seq = len(n_ctx_list)
    cap_max = max(-(-(n + 4) // 256) * 256 for n in n_ctx_list)
    idx_cache = torch.zeros((n_seq, cap_max, 128), dtype=torch.bfloat16, device=DEV)
    pooled = torch.zeros((n_seq, cap_max // 4, 128), dtype=torch.float32, device=DEV)
    seqs, segs_dev, host = [], [], []
    for s, (n, nseg) in enumerate(zip(n_ctx_list, nseg_list)):
        idx = datagen.round_bf16(rng.standard_normal((n, 128)).astype(np.float32))
        iq = datagen.round_bf16(rng.standard_normal((1, 4, 128)).astype(np.float32))
        q = datagen.round_bf16(rng.standard_normal((1, 24, D)).astype(np.float32))
        k_ = datagen.round_bf16(rng.standard_normal((2, n, D)).astype(np.float32))
        v_ = datagen.round_bf16(rng.standard_normal((2, n, D)).astype(np.float32))
        cuts = sorted(rng.choice(np.arange(0, n + 1), size=nseg - 1, replace=True).tolist()) if nseg > 1 else []
        bounds = [0] + cuts + [n]
        segs = []
        for lo, hi in zip(bounds[:-1], bounds[1:]):
            cap = max(hi - lo, 1) + int(rng.integers(0, 9))
            kt = torch.zeros((2, cap, D), dtype=torch.bfloat16, device=DEV)
            vt = torch.zeros_like(kt)
            if hi > lo:
                kt[:, : hi - lo] = to_dev(np.ascontiguousarray(k_[:, lo:hi]), "bf16")
                vt[:, : hi - lo] = to_dev(np.ascontiguousarray(v_[:, lo:hi]), "bf16")
            if quant:
                q8 = quant == "q8"
                k8 = torch.full((2, cap, D), 0x55, dtype=torch.int8 if q8 else torch.uint8, device=DEV)
                v8 = torch.full_like(k8, 0x55)
                ks = torch.zeros((2, cap, D // 32) if q8 else (2, cap), dtype=torch.float16, device=DEV)
                vs = torch.zeros_like(ks)
                qfn = Q.qsa_quantize_kv_q8_0 if q8 else Q.qsa_quantize_kv_fp8
                ofn = O.quantize_kv_q8_0 if q8 else O.quantize_kv_fp8
                if hi > lo:
                    qfn(kt[:, : hi - lo].contiguous(), k8, ks)
                    qfn(vt[:, : hi - lo].contiguous(), v8, vs)
                    for src, c8, sc8 in ((k_, k8, ks), (v_, v8, vs)):
                        c_ref, s_ref = ofn(src[:, lo:hi])
                        assert np.array_equal(c8[:, : hi - lo].cpu().numpy(), c_ref), "fp8 codes differ"
                        assert np.array_equal(sc8[:, : hi - lo].cpu().numpy().view(np.uint16), s_ref.view(np.uint16))
                segs.append((lo, hi - lo, k8, v8, ks, vs))
            else:
                segs.append((lo, hi - lo, kt, vt))
        segs_dev.append(segs)
        Q.qsa_append_pool(to_dev(idx, "bf16"), torch.arange(n, dtype=torch.int64, device=DEV),
                          idx_cache[s : s + 1], pooled[s : s + 1])
        host.append(dict(idx=idx, idx_q=iq, q=q, k=k_, v=v_, n=n))
    kv = Q.KvSegments(segs_dev)
    m = n_seq
    rows = torch.tensor([h["n"] - 1 for h in host], dtype=torch.int64, device=DEV)
    row_seq = torch.arange(m, dtype=torch.int32, device=DEV)
    idx_q = to_dev(np.concatenate([h["idx_q"] for h in host]), "bf16")
    q = to_dev(np.concatenate([h["q"] for h in host]), "bf16")
    nb_max = max(h["n"] for h in host) // 4
    plan = Q.qsa_attn_plan(m, 2, k)
    scores = torch.zeros((m, -(-(nb_max + 4) // 4) * 4), dtype=torch.float32, device=DEV)
    Q.qsa_score_blocks(idx_q, rows, pooled, scores, nb_max, row_seq=row_seq)
    sel = torch.empty((m, k), dtype=torch.int32, device=DEV)
    n_sel = torch.empty((m,), dtype=torch.int32, device=DEV)
    ws_sel = torch.zeros(Q.qsa_select_workspace_bytes(m, nb_max, k), dtype=torch.uint8, device=DEV)
    Q.qsa_select_topk(scores, rows, nb_max, k, sel, n_sel, ws_sel)
    out = torch.empty_like(q)
    lse = torch.empty((m, 24), dtype=torch.float32, device=DEV)
    ws = torch.empty(Q.qsa_attn_workspace_bytes(m, 24, D, k), dtype=torch.uint8, device=DEV)
    Q.qsa_gathered_attn(q, rows, kv, sel, n_sel, out, lse, 2, row_seq=row_seq, workspace=ws)
    torch.cuda.synchronize()
    out = to_host_f32(out)
    lse = lse.cpu().numpy()
    sc = scores.cpu().numpy()
    sel = sel.cpu().numpy()
    n_sel = n_sel.cpu().numpy()
    errs = []
    for i, h in enumerate(host):
        pr = O.pool_index_keys(h["idx"])
        assert np.array_equal(pooled[i, : h["n"] // 4].cpu().numpy().view(np.uint32), pr.view(np.uint32))
        s64 = O.score_blocks(h["idx_q"][0], pr, h["n"])
        g32 = sc[i, : len(s64)].astype(np.float64)
        assert np.array_equal(sel[i, : n_sel[i]], O.select_blocks(g32, k))
        check_selection(sel[i], int(n_sel[i]), s64, k)
        if quant:
            tok = O.attended_tokens(sel[i, : n_sel[i]], h["n"])
            qo, dq = ((O.quantize_kv_q8_0, O.dequantize_kv_q8_0) if quant == "q8" else
                      (O.quantize_kv_fp8, O.dequantize_kv_fp8))
            deq = [dq(*qo(src[:, tok])) for src in (h["k"], h["v"])]
            ref, ref_lse = O.attend(h["q"][0], deq[0], deq[1], np.arange(len(tok)), 1.0 / math.sqrt(D))
            err, lerr = float(np.max(np.abs(out[i] - ref))), float(np.max(np.abs(lse[i] - ref_lse)))
            assert err <= 2e-2 and lerr <= 1e-3, (i, err, lerr)
        else:
            dd = {"workload": wl, "rows": np.asarray([h["n"] - 1]), "q": h["q"], "k": h["k"], "v": h["v"]}
            err, lerr = check_attention(out[i], lse[i], dd, 0, sel[i, : n_sel[i]], "bf16")
        errs.append((err, lerr))
    return plan, errs


@pytest.mark.parametrize("seed,nseg", [(1, [1, 2, 3]), (2, [13, 5, 1]), (3, [4, 12, 7, 9]), (4, [16])])
def test_segments_small(Q, seed, nseg):
    say("segments", seed, nseg)
    rng = np.random.default_rng(seed)
    ctx = [int(x) for x in rng.integers(1500, 9000, size=len(nseg))]
    _segmented_case(Q, ctx, nseg, seed)


@pytest.mark.parametrize("seed,nseg", [(5, [1, 3, 2]), (6, [12, 1, 5, 16]),
                                       (15, [1, 2, 3, 1, 2, 1, 4, 1, 2, 1, 1, 3, 2, 1, 5, 1])])
def test_segments_head_dim_128(Q, seed, nseg):
    """The batched segmented decode at head_dim 128 (MTPLX PR #610, "Tests":
    segments at head_dims 128 and 256)."""
    say("segments, head_dim 128", seed, nseg)
    rng = np.random.default_rng(seed)
    ctx = [int(x) for x in rng.integers(1500, 9000, size=len(nseg))]
    _segmented_case(Q, ctx, nseg, seed, head_dim=128)


@pytest.mark.parametrize("head_dim", [256, 128])
def test_segments_many_rows_walk(Q, head_dim):
    """131 sequences, one row each, 1..3 K/V segments: the attention plan is 8
    waves walking several 128-token tiles per split (the multi-tile walk of
    the prefill plan, here over segments and rows of different sequences)."""
    say("segments, 131 sequences, head_dim", head_dim)
    rng = np.random.default_rng(131 + head_dim)
    ctx = [int(x) for x in rng.integers(1500, 9000, size=131)]
    nseg = [int(x) for x in rng.integers(1, 4, size=131)]
    plan, errs = _segmented_case(Q, ctx, nseg, 131 + head_dim, head_dim=head_dim)
    assert plan["waves"] == 8 and plan["tiles_per_split"] > 1 and plan["splits"] > 1, plan
    say(plan, max(e for e, _ in errs), max(l for _, l in errs))


@pytest.mark.parametrize("quant,seed,nseg,head_dim", [("fp8", 7, [1, 4, 2], 256), ("fp8", 8, [16, 3, 5, 1, 9], 256),
                                                      ("fp8", 9, [2, 13, 1], 128), ("q8", 10, [1, 5, 2], 256),
                                                      ("q8", 11, [12, 3, 1, 7], 256), ("q8", 12, [3, 1, 16], 128),
                                                      ("fp8", 13, [2, 1, 3, 1, 2, 4, 1, 1, 2, 3, 1, 5, 1, 2, 1, 3], 256),
                                                      ("q8", 14, [1, 2, 1, 3, 5, 1, 2, 1, 1, 4, 2, 1, 3, 1, 2, 1], 256)])
def test_segments_quantized(Q, quant, seed, nseg, head_dim):
    """fp8 (E4M3 + f16 row scales) or Q8_0 (int8 + f16 scale per 32 values)
    K/V across several segments, some empty or cutting a block, rows of
    different sequences in one call (row_seq).  With 16 sequences the
    attention plan is the 4-wave walk of several tiles per split."""
    say("segments,", quant, "K/V", seed, nseg, head_dim)
    rng = np.random.default_rng(seed)
    ctx = [int(x) for x in rng.integers(1500, 9000, size=len(nseg))]
    plan, errs = _segmented_case(Q, ctx, nseg, seed, head_dim=head_dim, quant=quant)
    assert plan["splits"] > 1, plan  # split partials merged by the combine
    if len(nseg) == 16:
        assert plan["waves"] == 4 and plan["tiles_per_split"] > 1, plan
    say(plan, max(e for e, _ in errs), max(l for _, l in errs))


def test_batched_segmented_full_size(Q):
    """16 sequences, contexts 4,096..131,072, 1..5 segments each (seeded).
    The attention plan is the 4-wave walk: 5 tiles of 64 tokens per split."""
    say("batched segmented decode, 16 sequences (full size)")
    plan = Q.qsa_attn_plan(16, 2, 512)
    assert plan["waves"] == 4 and plan["tiles_per_split"] == 5 and plan["splits"] == 7, plan
    specs = datagen.batched_specs()
    data = datagen.gen_batched_layer(specs)
    n_seq = len(specs)
    cap_max = max(-(-(sp.n_ctx + 4) // 256) * 256 for sp in specs)
    idx_cache = torch.zeros((n_seq, cap_max, 128), dtype=torch.bfloat16, device=DEV)
    pooled = torch.zeros((n_seq, cap_max // 4, 128), dtype=torch.float32, device=DEV)
    segs_dev = []
    for s, (sp, h) in enumerate(zip(specs, data)):
        Q.qsa_append_pool(to_dev(h["idx"], "bf16"), torch.arange(sp.n_ctx, dtype=torch.int64, device=DEV),
                          idx_cache[s : s + 1], pooled[s : s + 1])
        segs = []
        for st, ln, cap in zip(sp.seg_start, sp.seg_len, sp.seg_cap):
            kt = torch.zeros((2, cap, 256), dtype=torch.bfloat16, device=DEV)
            vt = torch.zeros_like(kt)
            kt[:, :ln] = to_dev(np.ascontiguousarray(h["k"][:, st : st + ln]), "bf16")
            vt[:, :ln] = to_dev(np.ascontiguousarray(h["v"][:, st : st + ln]), "bf16")
            segs.append((st, ln, kt, vt))
        segs_dev.append(segs)
    kv = Q.KvSegments(segs_dev)
    rows = torch.tensor([sp.row for sp in specs], dtype=torch.int64, device=DEV)
    row_seq = torch.arange(n_seq, dtype=torch.int32, device=DEV)
    idx_q = to_dev(np.concatenate([h["idx_q"] for h in data]), "bf16")
    q = to_dev(np.concatenate([h["q"] for h in data]), "bf16")
    nb_max = max(sp.n_ctx for sp in specs) // 4
    k = 512
    scores = torch.zeros((n_seq, -(-nb_max // 4) * 4), dtype=torch.float32, device=DEV)
    Q.qsa_score_blocks(idx_q, rows, pooled, scores, nb_max, row_seq=row_seq)
    sel = torch.empty((n_seq, k), dtype=torch.int32, device=DEV)
    n_sel = torch.empty((n_seq,), dtype=torch.int32, device=DEV)
    ws_sel = torch.zeros(Q.qsa_select_workspace_bytes(n_seq, nb_max, k), dtype=torch.uint8, device=DEV)
    Q.qsa_select_topk(scores, rows, nb_max, k, sel, n_sel, ws_sel)
    out = torch.empty_like(q)
    lse = torch.empty((n_seq, 24), dtype=torch.float32, device=DEV)
    ws = torch.empty(Q.qsa_attn_workspace_bytes(n_seq, 24, 256, k), dtype=torch.uint8, device=DEV)
    Q.qsa_gathered_attn(q, rows, kv, sel, n_sel, out, lse, 2, row_seq=row_seq, workspace=ws)
    torch.cuda.synchronize()
    out, lse = to_host_f32(out), lse.cpu().numpy()
    sc, sel, n_sel = scores.cpu().numpy(), sel.cpu().numpy(), n_sel.cpu().numpy()
    wl = datagen.WORKLOADS["decode_32k"]
    for i, (sp, h) in enumerate(zip(specs, data)):
        pr = O.pool_index_keys(h["idx"])
        assert np.array_equal(pooled[i, : sp.n_ctx // 4].cpu().numpy().view(np.uint32), pr.view(np.uint32))
        s64 = O.score_blocks(h["idx_q"][0], pr, sp.n_ctx)
        assert np.array_equal(sel[i, : n_sel[i]], O.select_blocks(sc[i, : len(s64)].astype(np.float64), k))
        check_selection(sel[i], int(n_sel[i]), s64, k)
        dd = {"workload": wl, "rows": np.asarray([sp.row]), "q": h["q"], "k": h["k"], "v": h["v"]}
        check_attention(out[i], lse[i], dd, 0, sel[i, : n_sel[i]], "bf16")
