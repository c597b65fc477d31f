"""Pins of the CPU oracle against things other than itself (CPU only).

Each test names what it pins: a library routine for a special case (torch
SDPA for dense attention), brute force on tiny inputs, closed forms and
hand-derived golden values (tests/golden/).  A plausible slip in the oracle
(a dropped ReLU, a wrong scale, a swapped KV-head mapping, a missing tail,
the wrong tie rule, a different pooling order) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import datagen
import oracle as O

F64 = torch.float64


def _bits_to_f32(h):
    return np.array([int(h, 16)], dtype=np.uint32).view(np.float32)[0]


# ---------------------------------------------------------------- pooling (P7)

def test_pool_golden_order(golden_dir):
    """Pooling order fixed by hand-derived float32 bit patterns."""
    g = json.load(open(os.path.join(golden_dir, "pool_order.json")))
    for case in g["cases"]:
        keys = np.zeros((4, 128), np.float32)
        keys[:, 5] = [_bits_to_f32(h) for h in case["keys"]]
        pooled = O.pool_index_keys(keys)
        assert pooled.shape == (1, 128)
        got = pooled[0, 5].view(np.uint32)
        assert got == int(case["pooled"], 16), (case["name"], hex(got))
        assert np.all(pooled[0, :5] == 0) and np.all(pooled[0, 6:] == 0)


def test_pool_closed_forms():
    rng = np.random.default_rng(1)
    # four equal keys pool to that key exactly
    x = rng.standard_normal((1, 128)).astype(np.float32)
    assert np.array_equal(O.pool_index_keys(np.repeat(x, 4, axis=0))[0], x[0])
    # small integers (exact in float32): pooled * 4 equals the exact sum
    ints = rng.integers(-1000, 1000, size=(64, 128)).astype(np.float32)
    p = O.pool_index_keys(ints).astype(np.float64)
    exact = ints.astype(np.float64).reshape(16, 4, 128).sum(axis=1)
    assert np.array_equal(p * 4, exact)
    # only complete blocks are pooled; a trailing partial block is ignored
    assert O.pool_index_keys(np.ones((11, 128), np.float32)).shape == (2, 128)
    assert O.pool_index_keys(np.ones((3, 128), np.float32)).shape == (0, 128)


def test_pool_within_rounding_of_mean():
    """Random keys: float32 result within 2 ulp-scale of the exact mean."""
    x = np.random.default_rng(2).standard_normal((4096, 128)).astype(np.float32)
    p = O.pool_index_keys(x).astype(np.float64)
    mean = x.astype(np.float64).reshape(-1, 4, 128).mean(axis=1)
    mag = np.abs(x.astype(np.float64)).reshape(-1, 4, 128).max(axis=1)
    assert np.all(np.abs(p - mean) <= 3 * 2.0 ** -24 * mag + 1e-45)


# ---------------------------------------------------------------- scoring (P8)

def _small_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "score_select_small.json")))
    pooled = np.zeros((g["n_blocks"], 128), np.float32)
    for b, j, val in g["pooled_nonzero"]:
        pooled[b, j] = val
    q = np.zeros((4, 128), np.float32)
    for h, j, val in g["idx_q_nonzero"]:
        q[h, j] = val
    return g, pooled, q


def test_score_golden(golden_dir):
    g, pooled, q = _small_golden(golden_dir)
    s = O.score_blocks(q, pooled, n_visible=g["row_pos"] + 1)
    np.testing.assert_allclose(s, g["scores"], rtol=1e-15, atol=0)


def test_score_closed_forms():
    rng = np.random.default_rng(3)
    pooled = rng.standard_normal((300, 128)).astype(np.float32)
    # zero index queries: every score is 0
    assert np.all(O.score_blocks(np.zeros((4, 128)), pooled, 1200) == 0)
    # one-hot head 0 on dim j: s = relu(pooled[b, j]) / sqrt(128)
    for j in (0, 77, 127):
        q = np.zeros((4, 128))
        q[0, j] = 1.0
        s = O.score_blocks(q, pooled, 1200)
        np.testing.assert_allclose(s, np.maximum(pooled[:, j].astype(np.float64), 0) / math.sqrt(128),
                                   rtol=1e-15, atol=0)
    # the same one-hot on all four heads gives 4x (heads are summed unweighted)
    q = np.zeros((4, 128))
    q[:, 9] = 1.0
    s = O.score_blocks(q, pooled, 1200)
    np.testing.assert_allclose(s, 4 * np.maximum(pooled[:, 9].astype(np.float64), 0) / math.sqrt(128),
                               rtol=1e-15)
    # scores are never negative, and only complete visible blocks are scored
    q = rng.standard_normal((4, 128))
    assert np.all(O.score_blocks(q, pooled, 1200) >= 0)
    assert O.score_blocks(q, pooled, 7).shape == (1,)
    assert O.score_blocks(q, pooled, 3).shape == (0,)


# ------------------------------------------------------------- selection (P2)

def _brute_topk(s, k):
    nb = len(s)
    if nb <= k:
        return list(range(nb))
    return sorted(sorted(range(nb), key=lambda b: (-s[b], b))[:k])


def test_select_golden(golden_dir):
    g, _, _ = _small_golden(golden_dir)
    s = np.asarray(g["scores"])
    for k, want in g["select"].items():
        assert O.select_blocks(s, int(k)).tolist() == want
    sel = O.select_blocks(s, 3)
    assert O.attended_tokens(sel, g["row_pos"] + 1).tolist() == g["tokens_k3"]


@settings(max_examples=300, deadline=None)
@given(st.lists(st.sampled_from([0.0, 0.0, 0.25, 0.5, 0.5, 1.0, 3.0]), min_size=0, max_size=24),
       st.integers(min_value=1, max_value=8))
def test_select_brute_force_with_ties(vals, k):
    s = np.asarray(vals, dtype=np.float64)
    assert O.select_blocks(s, k).tolist() == _brute_topk(list(s), k)


def test_select_all_zero_row():
    assert O.select_blocks(np.zeros(100), 7).tolist() == list(range(7))


# ---------------------------------------------------- key-axis chunking (P5)

@settings(max_examples=200, deadline=None)
@given(st.lists(st.sampled_from([0.0, 0.1, 0.2, 0.2, 0.7, 1.5]), min_size=1, max_size=40),
       st.integers(1, 9), st.lists(st.integers(1, 40), min_size=1, max_size=8))
def test_topk_of_union_of_chunk_topk(vals, k, cuts):
    """topk(all) == topk(union of per-chunk topk) under the same tie rule
    (the identity the SGLang prefill-memory note, section 2.3, relies on)."""
    s = np.asarray(vals)
    nb = len(s)
    bounds = sorted(set([0, nb] + [c for c in cuts if c < nb]))
    cand = []
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        cand.extend((lo + O.select_blocks(s[lo:hi], k)).tolist())
    cand = np.asarray(cand)
    order = np.lexsort((cand, -s[cand]))
    merged = np.sort(cand[order[:k]]) if len(cand) > k else np.sort(cand)
    assert merged.tolist() == O.select_blocks(s, k).tolist()


# ------------------------------------------------------------------ tail (P3)

@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 1021, 1022, 1023, 1024, 4099])
def test_tail_always_attended(n):
    rng = np.random.default_rng(n)
    idx = rng.standard_normal((n, 128)).astype(np.float32)
    q = rng.standard_normal((4, 128)).astype(np.float32)
    u = datagen.planting_direction(q)
    nb = n // 4
    idx[4 * nb:] = (-100.0 * u).astype(np.float32)   # tail keys point away from the query
    pooled = O.pool_index_keys(idx)
    s = O.score_blocks(q, pooled, n)
    for k in (1, 2, 64):
        tok = O.attended_tokens(O.select_blocks(s, k), n)
        assert set(range(4 * nb, n)) <= set(tok.tolist())
        assert len(tok) == 4 * min(k, nb) + n % 4
        assert len(set(tok.tolist())) == len(tok)
        assert tok.max(initial=-1) <= n - 1                  # causality (P11)


# -------------------------------------------------- attention vs SDPA (P1, P6)

def _sdpa_dense(q_rows, k, v, rows, scale, gqa_native):
    """Dense causal GQA attention of the given rows through torch SDPA (CPU, fp64)."""
    m, hq, d = q_rows.shape
    hkv, n, _ = k.shape
    qt = torch.from_numpy(np.asarray(q_rows, np.float64)).permute(1, 0, 2)[None]     # [1,hq,M,D]
    kt = torch.from_numpy(np.asarray(k[:, :n], np.float64))[None]                    # [1,hkv,N,D]
    vt = torch.from_numpy(np.asarray(v[:, :n], np.float64))[None]
    mask = torch.arange(n)[None, :] <= torch.as_tensor(rows)[:, None]               # [M,N]
    if gqa_native:
        o = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=mask, scale=scale, enable_gqa=True)
    else:
        g = hq // hkv
        kt = kt.repeat_interleave(g, dim=1).contiguous()
        vt = vt.repeat_interleave(g, dim=1).contiguous()
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    logits = torch.einsum("bhmd,bhnd->bhmn", qt, kt if not gqa_native else kt.repeat_interleave(hq // hkv, 1)) * scale
    logits = logits.masked_fill(~mask, float("-inf"))
    lse = torch.logsumexp(logits, dim=-1)
    return o[0].permute(1, 0, 2).numpy(), lse[0].permute(1, 0).numpy()


@pytest.mark.parametrize("gqa_native", [False, True])
def test_budget_covers_context_equals_dense_attention(gqa_native):
    """P1: with a budget >= the context every block is kept, so QSA equals
    dense causal attention (the tiny fp32 workload with a 1,024-token budget)."""
    d = datagen.gen_layer("tiny")
    wl = d["workload"]
    scale = 1.0 / math.sqrt(wl.head_dim)
    p = int(d["rows"][0])
    r = O.qsa_row(d["idx"], d["idx_q"][0], d["q"][0], d["k"], d["v"], p, 1024 // 4, scale)
    assert len(r["sel"]) == (p + 1) // 4 and len(r["tokens"]) == p + 1
    ref, ref_lse = _sdpa_dense(d["q"], d["k"], d["v"], d["rows"], scale, gqa_native)
    np.testing.assert_allclose(r["out"], ref[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["lse"], ref_lse[0], rtol=0, atol=1e-12)


def test_dense_several_rows_causal():
    """P1 at several rows with distinct tails (rows see 1..4 partial tokens)."""
    rng = np.random.default_rng(7)
    hq, hkv, dd, n = 6, 2, 32, 37
    k = rng.standard_normal((hkv, n, dd))
    v = rng.standard_normal((hkv, n, dd))
    rows = np.array([30, 33, 34, 35, 36])
    q = rng.standard_normal((len(rows), hq, dd))
    idx = rng.standard_normal((n, 128)).astype(np.float32)
    iq = rng.standard_normal((len(rows), 4, 128))
    ref, ref_lse = _sdpa_dense(q, k, v, rows, 0.3, False)
    for i, p in enumerate(rows):
        r = O.qsa_row(idx, iq[i], q[i], k, v, int(p), 100, 0.3)
        np.testing.assert_allclose(r["out"], ref[i], atol=1e-12, rtol=0)
        np.testing.assert_allclose(r["lse"], ref_lse[i], atol=1e-12, rtol=0)


def test_sparse_equals_dense_over_kept_rows():
    """With a small budget, QSA equals SDPA restricted (by mask) to the kept rows."""
    d = datagen.gen_layer("tiny")
    wl = d["workload"]
    scale = 1.0 / math.sqrt(wl.head_dim)
    p = int(d["rows"][0])
    r = O.qsa_row(d["idx"], d["idx_q"][0], d["q"][0], d["k"], d["v"], p, wl.k_blocks, scale)
    assert len(r["tokens"]) == 4 * wl.k_blocks + 3
    mask = torch.zeros(1, p + 1, dtype=torch.bool)
    mask[0, torch.from_numpy(r["tokens"])] = True
    qt = torch.from_numpy(d["q"].astype(np.float64)).permute(1, 0, 2)[None]
    kt = torch.from_numpy(d["k"].astype(np.float64))[None].repeat_interleave(12, 1)
    vt = torch.from_numpy(d["v"].astype(np.float64))[None].repeat_interleave(12, 1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    np.testing.assert_allclose(r["out"], o[0, :, 0].numpy(), atol=1e-12, rtol=0)
    # the planted blocks dominate the kept set
    assert len(set(d["planted"].tolist()) & set(r["sel"].tolist())) >= 6


def test_attend_closed_forms():
    rng = np.random.default_rng(5)
    k = rng.standard_normal((2, 10, 8))
    v = rng.standard_normal((2, 10, 8))
    q = rng.standard_normal((4, 8))
    # one token: output is that token's V row, lse its logit
    out, lse = O.attend(q, k, v, np.array([6]), 0.5)
    for h in range(4):
        np.testing.assert_allclose(out[h], v[h // 2, 6], rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse[h], 0.5 * q[h] @ k[h // 2, 6], rtol=1e-15)
    # empty token set: zeros and -inf, never NaN
    out, lse = O.attend(q, k, v, np.array([], np.int64), 0.5)
    assert np.all(out == 0) and np.all(np.isneginf(lse))


# ------------------------------------------------------------ LSE merge (P4)

@pytest.mark.parametrize("seed", range(12))
def test_merge_of_partitions_equals_single_buffer(seed):
    rng = np.random.default_rng(100 + seed)
    hq, hkv, dd, n = 12, 2, 16, 300
    k = rng.standard_normal((hkv, n, dd))
    v = rng.standard_normal((hkv, n, dd))
    q = rng.standard_normal((hq, dd))
    tokens = np.sort(rng.choice(n, size=rng.integers(1, 200), replace=False))
    nparts = int(rng.integers(1, 14))
    lab = rng.integers(0, nparts, size=len(tokens))
    parts = [np.nonzero(lab == i)[0] for i in range(nparts)] + [np.zeros(0, np.int64)]
    out, lse = O.attend_partitioned(q, k, v, tokens, 0.2, parts)
    ref, ref_lse = O.attend(q, k, v, tokens, 0.2)
    np.testing.assert_allclose(out, ref, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, ref_lse, atol=1e-12, rtol=0)


def test_merge_all_empty_gives_zeros():
    out, lse = O.merge_partials(np.full((5, 3), -np.inf), np.full((5, 3, 4), np.nan))
    assert np.all(out == 0) and np.all(np.isneginf(lse)) and not np.any(np.isnan(out))


# ------------------------------------------- layout byte counts (P9, P10)

def test_state_byte_counts_match_pages():
    """f32 state: K + V at 2 KV heads x 256 + index key + pooled share = 4,736 B
    per token per layer; 12 layers x 262,144 tokens = 14,208 MiB (hipfire
    page, 'State formats' and section 04).  bf16 K buffer [2, 261,128, 256]
    is ~0.27 GB and 12 layers of K+V ~6.42 GB (MTPLX PR #482, section 2)."""
    per_tok = 2 * 256 * 4 * 2 + O.INDEX_DIM * 4 + O.INDEX_DIM * 4 // O.BLOCK_TOKENS
    assert per_tok == 4736
    assert per_tok * 262144 * 12 == 14208 * 2 ** 20
    kbuf = 2 * 261128 * 256 * 2
    assert abs(kbuf / 1e9 - 0.27) < 0.005
    assert abs(2 * 12 * kbuf / 1e9 - 6.42) < 0.01
    # 15,360 pooled blocks hold 61,440 tokens; 512 blocks = 2,048 tokens
    assert 15360 * O.BLOCK_TOKENS == 61440 and 512 * O.BLOCK_TOKENS == 2048


# ------------------------------------------------- determinism (P12), datagen

def test_oracle_and_datagen_deterministic():
    a = datagen.gen_layer("tiny")
    b = datagen.gen_layer("tiny")
    for key in ("idx", "idx_q", "q", "k", "v"):
        assert np.array_equal(a[key], b[key])
    ra = O.qsa_row(a["idx"], a["idx_q"][0], a["q"][0], a["k"], a["v"], 1022, 64, 0.1)
    rb = O.qsa_row(b["idx"], b["idx_q"][0], b["q"][0], b["k"], b["v"], 1022, 64, 0.1)
    for key in ("pooled", "scores", "sel", "out", "lse"):
        assert np.array_equal(ra[key], rb[key])


def test_datagen_bf16_exact_and_shapes():
    d = datagen.gen_layer("decode_32k")
    for key in ("idx", "idx_q", "q", "k", "v"):
        assert np.array_equal(datagen.round_bf16(d[key]), d[key])
    assert d["k"].shape == (2, 32768, 256) and d["idx_q"].shape == (1, 4, 128)
    assert len(d["planted"]) == 410
    specs = datagen.batched_specs()
    assert len(specs) == 16
    for sp in specs:
        assert 4096 <= sp.n_ctx <= 131072 and 1 <= len(sp.seg_len) <= 5
        assert sum(sp.seg_len) == sp.n_ctx and sp.seg_start[0] == 0


# ------------------------------------------------------- fp8 K/V (NEXT: fp8 state)

def test_e4m3_decode_all_codes_match_torch():
    """All 256 E4M3 codes decode as torch's float8_e4m3fn does (NaN at 0x7f/0xff)."""
    c = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(c).view(torch.float8_e4m3fn).to(F64).numpy()
    got = O.e4m3_decode(c)
    assert np.array_equal(got, want, equal_nan=True)
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_e4m3_encode_matches_torch_including_ties():
    """Nearest value, ties to the even code: against torch's float8_e4m3fn cast on
    random values over every binade, the grid values and the exact midpoints."""
    grid = O.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (grid[:-1] + grid[1:]) / 2
    rng = np.random.default_rng(11)
    mags = rng.choice([2.0 ** -11, 2.0 ** -7, 0.01, 0.3, 1.0, 7.0, 60.0, 300.0], 20000)
    rnd = rng.standard_normal(20000) * mags
    y = np.concatenate([grid, -grid, mids, -mids, rnd, [0.0, -0.0, 2.0 ** -10, -2.0 ** -10]])
    y = np.clip(y, -448.0, 448.0).astype(np.float32)
    want = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(y), want)
    # midpoints do split between the two neighbours (ties are exercised)
    codes = O.e4m3_encode(mids.astype(np.float32))
    assert np.all(codes % 2 == 0) and len(set(codes.tolist())) > 60


def test_e4m3_encode_saturates():
    """Finite magnitudes above 448 saturate to +-448 (codes 0x7e / 0xfe)."""
    y = np.array([448.0, 449.0, 464.0, 479.9, 480.0, 1e4, 3e38], dtype=np.float32)
    assert np.all(O.e4m3_encode(y) == 0x7E)
    assert np.all(O.e4m3_encode(-y) == 0xFE)


def test_quantize_kv_fp8_matches_torch_recipe():
    """Per-row scale = f16(amax / 448) and codes = E4M3(x / scale), both through
    torch (float32 quotients, torch's f16 and float8_e4m3fn casts)."""
    rng = np.random.default_rng(5)
    x = datagen.round_bf16(rng.standard_normal((64, 256)).astype(np.float32))
    x[3] *= 1e-3
    x[4] *= 1e-6            # scale in the f16 subnormal range
    x[5] = 0.0              # zero row
    x[6, 7] = 56.0          # an amax whose scale is exact (0.125)
    x[6] = np.clip(x[6], -56.0, 56.0)
    codes, scale = O.quantize_kv_fp8(x)
    xt = torch.from_numpy(x)
    amax = xt.abs().amax(dim=-1)
    s = (amax / torch.tensor(448.0)).to(torch.float16)
    sf = s.to(torch.float32)[:, None]
    y = torch.where(sf > 0, xt / torch.where(sf > 0, sf, torch.ones_like(sf)), torch.zeros_like(xt))
    want_codes = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(scale.view(np.uint16), s.numpy().view(np.uint16))
    assert np.array_equal(codes, want_codes)
    assert codes[6, 7] == 0x7E and scale[6] == np.float16(0.125)
    assert scale[5] == 0 and np.all(codes[5] == 0)


def test_quantize_kv_fp8_closed_forms():
    """Sign symmetry, the largest magnitude maps to about 448, the round trip is
    within half an E4M3 step, and a scale that overflows f16 clamps to 65504."""
    rng = np.random.default_rng(9)
    x = datagen.round_bf16(rng.standard_normal((32, 128)).astype(np.float32) * 3.0)
    c, s = O.quantize_kv_fp8(x)
    cn, sn = O.quantize_kv_fp8(-x)
    assert np.array_equal(s, sn)
    assert np.array_equal(cn, c ^ 0x80)
    r = O.dequantize_kv_fp8(c, s)
    sd = s.astype(np.float64)[:, None]
    # E4M3: 3 mantissa bits (relative half-step 2^-4), subnormal step 2^-9
    assert np.all(np.abs(r - x) <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * sd) * (1 + 1e-6))
    top = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(O.e4m3_decode(c[np.arange(32), top])) >= 416.0)
    big = np.full((1, 16), 3.0e7, np.float32)
    cb, sb = O.quantize_kv_fp8(big)
    assert sb[0] == np.float16(65504.0) and np.all(cb == 0x7E)


# ------------------------------------------------------- Q8_0 K/V (the q8 state)

def _q8_brute(x: np.ndarray):
    """Nearest integer code by exhaustive search over [-127, 127] (ties to the
    even integer), against float32 quotients by the f16 scale -- no rint."""
    x = np.asarray(x, dtype=np.float32).reshape(-1, 32)
    codes = np.zeros(x.shape, dtype=np.int64)
    scales = np.zeros(x.shape[0], dtype=np.float16)
    cand = np.arange(-127, 128, dtype=np.float64)
    for b in range(x.shape[0]):
        amax = float(np.max(np.abs(x[b])))
        q = np.float32(amax) / np.float32(127.0)
        s16 = np.float16(q) if np.isfinite(np.float16(q)) else np.float16(65504.0)
        scales[b] = s16
        if float(s16) == 0.0:
            continue
        for j in range(32):
            y = float(np.float32(x[b, j]) / np.float32(s16))
            dist = np.abs(cand - y)
            best = cand[dist == dist.min()]
            codes[b, j] = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
    return codes, scales


def test_q8_0_matches_brute_force():
    """Codes are the nearest integers (ties to even, clamped to 127) of the
    float32 quotients by the stored f16 scale, one scale per 32 values."""
    rng = np.random.default_rng(21)
    x = datagen.round_bf16(rng.standard_normal((24, 256)).astype(np.float32) * 2.0)
    x[1] *= 1e-4      # scale in the f16 subnormal range
    x[2, :32] = 0.0   # a zero block
    x[3] *= 1e-9      # scales that round to zero
    c, s = O.quantize_kv_q8_0(x)
    assert c.dtype == np.int8 and c.shape == x.shape and s.shape == (24, 8)
    bc, bs = _q8_brute(x)
    assert np.array_equal(s.reshape(-1).view(np.uint16), bs.view(np.uint16))
    assert np.array_equal(c.reshape(-1, 32).astype(np.int64), bc)
    assert np.all(s[2, 0] == 0) and np.all(c[2, :32] == 0) and np.all(c[3] == 0)


def test_q8_0_ties_go_to_even():
    """A block scaled exactly by 2^-4 (largest value 127 / 16): values at
    n + 1/2 steps round to the even neighbour, integer steps are exact."""
    n = np.arange(-31, 32, dtype=np.float32)
    blk = np.zeros((2, 32), np.float32)
    blk[0] = np.resize(n[:32], 32) / 16.0
    blk[0, 0] = 127.0 / 16.0
    blk[1, :16] = (np.arange(16, dtype=np.float32) + 0.5) / 16.0
    blk[1, 16] = 127.0 / 16.0
    c, s = O.quantize_kv_q8_0(blk.reshape(1, 64))
    assert s[0, 0] == np.float16(0.0625) and s[0, 1] == np.float16(0.0625)
    assert np.array_equal(c[0, :32].astype(np.float32), blk[0] * 16.0)
    half = c[0, 32:48].astype(np.int64)
    want = np.array([int(2 * round((k + 0.5) / 2)) for k in range(16)])  # even neighbour of k + 1/2
    assert np.array_equal(half, want)


def test_q8_0_round_trip_and_bytes():
    """Round trip within half a step of each block; sign symmetry; an f16
    overflow clamps to 65504; 34 bytes per 32 values, so the page's 1,408
    bytes per token and layer at 2 KV heads x 256 dims = K + V (1,088) + a
    bf16 index key (256) + 64 bytes of pooled share."""
    rng = np.random.default_rng(22)
    x = datagen.round_bf16(rng.standard_normal((16, 128)).astype(np.float32) * 5.0)
    c, s = O.quantize_kv_q8_0(x)
    cn, sn = O.quantize_kv_q8_0(-x)
    assert np.array_equal(s, sn) and np.array_equal(cn, -c)
    r = O.dequantize_kv_q8_0(c, s)
    step = np.repeat(s.astype(np.float64), 32, axis=1)
    assert np.all(np.abs(r - x) <= 0.5 * step * (1 + 1e-3) + 1e-12)
    assert np.all(np.abs(c).max(axis=1) >= 126)
    big = np.full((1, 32), 3.0e7, np.float32)
    cb, sb = O.quantize_kv_q8_0(big)
    assert sb[0, 0] == np.float16(65504.0) and np.all(cb == 127)
    per_block = 32 * 1 + 2
    assert per_block == 34
    assert 2 * 2 * 256 // 32 * per_block + 128 * 2 + 64 == 1408
