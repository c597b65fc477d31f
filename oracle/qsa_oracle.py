"""Plain CPU oracle of the QSA per-layer path (TEST INFRASTRUCTURE ONLY).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The HIP library never calls it and shares no code with
it; the two meet only through the seeded inputs of ``datagen``.

Everything here is written from the method statement on the hipfire page
"QSA sparse attention and the VMM KV backend", section 02 ("How QSA chooses
what to read"): every token gets one 128-wide index key; each run of 4
consecutive keys is averaged into one pooled block key; four index-query
heads score each pooled block as the sum of their ReLU'd dot products times
1/sqrt(128); the best blocks inside a 2,048-token budget (512 blocks) are
kept together with the incomplete block at the end; attention then runs over
the kept rows only.  The log-sum-exp merge of partial results follows the
MTPLX PR #610 page, section "How it works" (segments merged by their
log-sum-exp) and its "What changes" list (rows with no visible key give
zeros, partials merged in float32 and rounded once).

Arithmetic is float64 except pooling, which is float32 by contract (the
reading is that pooled keys are stored in float32 and must be bit-exact, so
one fixed order of adds is prescribed: ((x0 + x1) + x2) + x3, then x 0.25,
IEEE round-to-nearest-even, no fused multiply-add).

Pins (tests/test_oracle_pins.py) tie every function below to something other
than itself: dense causal attention through torch SDPA, brute-force sorting,
closed forms and hand-derived golden values.  No function here is
"parity unpinned".  The fp8 K/V functions at the end follow the same page,
section 03 ("State formats"), and are pinned to torch's own float8_e4m3fn
conversions; the Q8_0 functions after them (same section) are pinned to a
brute-force nearest-integer search, closed forms and the page's byte count.
"""
from __future__ import annotations

import numpy as np

INDEX_DIM = 128      # width of the index key / each index-query head
INDEX_HEADS = 4      # index-query heads per query row
BLOCK_TOKENS = 4     # tokens folded into one pooled block key
SCORE_SCALE = 1.0 / np.sqrt(128.0)


def n_blocks(n_visible: int) -> int:
    """Complete 4-token blocks among ``n_visible`` tokens (section 02)."""
    return int(n_visible) // BLOCK_TOKENS


def pool_index_keys(idx_keys: np.ndarray) -> np.ndarray:
    """Average each run of 4 index keys into one pooled key (section 02).

    ``idx_keys`` [N, 128] holds float32 (or bf16-exact float32) values; the
    result is float32 [N // 4, 128].  The adds run left to right in float32,
    then the sum is multiplied by 0.25 (exact: a power of two).
    """
    x = np.asarray(idx_keys, dtype=np.float32)
    nb = n_blocks(x.shape[0])
    x = x[: nb * BLOCK_TOKENS].reshape(nb, BLOCK_TOKENS, x.shape[1])
    acc = x[:, 0] + x[:, 1]
    acc = acc + x[:, 2]
    acc = acc + x[:, 3]
    return acc * np.float32(0.25)


def score_blocks(idx_q_row: np.ndarray, pooled: np.ndarray, n_visible: int) -> np.ndarray:
    """Block scores of one query row over its causally visible blocks (section 02).

    s[b] = (sum over the 4 index heads of max(0, q_h . pooled[b])) / sqrt(128),
    for every complete block b < n_visible // 4.  float64 result.
    """
    nb = n_blocks(n_visible)
    p = np.asarray(pooled[:nb], dtype=np.float64)
    q = np.asarray(idx_q_row, dtype=np.float64).reshape(INDEX_HEADS, INDEX_DIM)
    dots = p @ q.T                              # [nb, 4]
    return np.maximum(dots, 0.0).sum(axis=1) * SCORE_SCALE


def select_blocks(scores: np.ndarray, k_blocks: int) -> np.ndarray:
    """Kept blocks of one row: the k best by score, ascending block order.

    Section 02 keeps "the top-scoring blocks within a 2,048-token budget";
    when every visible block fits the budget all are kept.  Equal scores go
    to the lower block index (the reading adopted for ties).
    """
    s = np.asarray(scores, dtype=np.float64)
    nb = s.shape[0]
    if nb <= k_blocks:
        return np.arange(nb, dtype=np.int64)
    order = np.lexsort((np.arange(nb), -s))     # by -score, then by index
    return np.sort(order[:k_blocks]).astype(np.int64)


def attended_tokens(sel: np.ndarray, n_visible: int) -> np.ndarray:
    """Token positions a row attends: its kept blocks plus the incomplete tail.

    Section 02: the incomplete block at the end is always kept in addition to
    the budget, so a row reads at most 2,048 + 3 tokens.
    """
    nb = n_blocks(n_visible)
    sel = np.asarray(sel, dtype=np.int64)
    body = (BLOCK_TOKENS * sel[:, None] + np.arange(BLOCK_TOKENS)[None, :]).reshape(-1)
    tail = np.arange(BLOCK_TOKENS * nb, int(n_visible), dtype=np.int64)
    return np.concatenate([body, tail])


def attend(q_row: np.ndarray, k: np.ndarray, v: np.ndarray, tokens: np.ndarray,
           scale: float) -> tuple[np.ndarray, np.ndarray]:
    """Softmax attention of one query row over the given tokens, float64.

    ``q_row`` [hq, D]; ``k``/``v`` [hkv, N, D]; query head h reads KV head
    h // (hq / hkv) (24 query heads over 2 KV heads, 12 per group, from the
    MTPLX PR #482 page, "Terms used"; the contiguous grouping is the reading
    adopted).  Returns (out [hq, D], lse [hq]); an empty token set gives
    out = 0 and lse = -inf.
    """
    q_row = np.asarray(q_row, dtype=np.float64)
    hq, d = q_row.shape
    hkv = k.shape[0]
    group = hq // hkv
    out = np.zeros((hq, d), dtype=np.float64)
    lse = np.full(hq, -np.inf, dtype=np.float64)
    tokens = np.asarray(tokens, dtype=np.int64)
    if tokens.size == 0:
        return out, lse
    for g in range(hkv):
        kg = np.asarray(k[g, tokens], dtype=np.float64)     # [T, D]
        vg = np.asarray(v[g, tokens], dtype=np.float64)
        for h in range(g * group, (g + 1) * group):
            logits = scale * (kg @ q_row[h])
            mx = logits.max()
            e = np.exp(logits - mx)
            tot = e.sum()
            lse[h] = mx + np.log(tot)
            out[h] = (e / tot) @ vg
    return out, lse


def merge_partials(lses: np.ndarray, outs: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Merge attention partials over disjoint token sets by log-sum-exp.

    ``lses`` [P, hq], ``outs`` [P, hq, D] (each partial normalised over its
    own tokens).  lse = log(sum_i exp(lse_i)); out = sum_i exp(lse_i - lse)
    out_i.  Empty partials carry lse_i = -inf and weigh nothing; if every
    partial is empty the row has no visible key and gives zeros (MTPLX PR
    #610, "What changes": such rows merge to zeros, not NaN).
    """
    lses = np.asarray(lses, dtype=np.float64)
    outs = np.asarray(outs, dtype=np.float64)
    mx = lses.max(axis=0)                                   # [hq]
    finite = np.isfinite(mx)
    safe_mx = np.where(finite, mx, 0.0)
    w = np.where(np.isfinite(lses), np.exp(lses - safe_mx[None, :]), 0.0)
    tot = w.sum(axis=0)
    lse = np.where(finite, safe_mx + np.log(np.where(finite, tot, 1.0)), -np.inf)
    wn = np.where(finite[None, :], w / np.where(finite, tot, 1.0)[None, :], 0.0)
    live = np.isfinite(lses)[:, :, None]         # an empty partial contributes nothing
    out = np.where(live, wn[:, :, None] * np.where(live, outs, 0.0), 0.0).sum(axis=0)
    return out, lse


def qsa_row(idx_keys: np.ndarray, idx_q_row: np.ndarray, q_row: np.ndarray,
            k: np.ndarray, v: np.ndarray, pos: int, k_blocks: int,
            scale: float, pooled: np.ndarray | None = None) -> dict:
    """The whole per-row path: pool, score, select (+tail), attend.

    ``pos`` is the row's absolute position; it sees tokens 0..pos.
    """
    n = int(pos) + 1
    if pooled is None:
        pooled = pool_index_keys(idx_keys[: (n // BLOCK_TOKENS) * BLOCK_TOKENS])
    s = score_blocks(idx_q_row, pooled, n)
    sel = select_blocks(s, k_blocks)
    tok = attended_tokens(sel, n)
    out, lse = attend(q_row, k, v, tok, scale)
    return {"pooled": pooled, "scores": s, "sel": sel, "tokens": tok, "out": out, "lse": lse}


def attend_partitioned(q_row, k, v, tokens, scale, parts) -> tuple[np.ndarray, np.ndarray]:
    """Attention computed per part of a partition of ``tokens`` and merged.

    ``parts`` is a list of index arrays into ``tokens`` (disjoint, covering,
    possibly empty).  Used by the pins to show the merge reproduces
    single-buffer attention.
    """
    hq, d = np.asarray(q_row).shape
    lses = np.full((len(parts), hq), -np.inf)
    outs = np.zeros((len(parts), hq, d))
    for i, p in enumerate(parts):
        outs[i], lses[i] = attend(q_row, k, v, np.asarray(tokens)[np.asarray(p, dtype=np.int64)], scale)
    return merge_partials(lses, outs)


# ----------------------------------------------------------- fp8 K/V state
# hipfire page, section 03, "State formats": the fp8 state stores K and V as
# E4M3 with one f16 scale per head and token, index keys staying bf16.  The
# page names the format only.  Readings: E4M3 is the OCP "FN" variant (bias
# 7, no infinities, largest finite value 448, S.1111.111 is NaN); a row's
# scale is its largest magnitude divided by 448 in float32, rounded to f16;
# each code is the E4M3 value nearest to the float32 quotient x / scale, ties
# to the even code, magnitudes above 448 saturating to 448; a row whose scale
# rounds to zero stores zero codes.

E4M3_MAX = 448.0
F16_MAX = 65504.0


def e4m3_decode(codes) -> np.ndarray:
    """float64 value of each E4M3 code (uint8), from the format's fields:
    sign, 4 exponent bits (bias 7), 3 mantissa bits; exponent 0 holds the
    subnormals m * 2^-9; exponent 15 with mantissa 7 is NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


_E4M3_GRID = e4m3_decode(np.arange(127, dtype=np.uint8))  # codes 0..126, ascending magnitudes


def e4m3_encode(y) -> np.ndarray:
    """Code (uint8) of the E4M3 value nearest to each finite ``y``: ties go to
    the even code, magnitudes above 448 saturate to 448 (code 0x7e), and the
    sign bit is the input's (-0 and negative values that round to zero give
    0x80)."""
    y = np.asarray(y, dtype=np.float64)
    a = np.minimum(np.abs(y), E4M3_MAX)
    lo = np.searchsorted(_E4M3_GRID, a, side="right") - 1   # largest grid value <= a
    hi = np.minimum(lo + 1, len(_E4M3_GRID) - 1)
    d_lo = a - _E4M3_GRID[lo]
    d_hi = _E4M3_GRID[hi] - a
    up = (hi != lo) & ((d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0)))
    code = np.where(up, hi, lo).astype(np.int64)
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def quantize_kv_fp8(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """E4M3 codes and f16 scales of the rows of ``x`` [..., D] (float32, or
    bf16-exact float32): one scale per row, i.e. per head and token."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    with np.errstate(over="ignore"):  # an f16 overflow is clamped just below
        scale = (amax / np.float32(E4M3_MAX)).astype(np.float16)
    scale = np.where(np.isinf(scale), np.float16(F16_MAX), scale)
    sf = scale.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(sf > 0, x / np.where(sf > 0, sf, np.float32(1.0)), np.float32(0.0))
    return e4m3_encode(y), scale


def dequantize_kv_fp8(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """float64 K or V rows from E4M3 codes [..., D] and f16 scales [...]."""
    return e4m3_decode(codes) * np.asarray(scale, dtype=np.float64)[..., None]



# ----------------------------------------------------------- Q8_0 K/V state
# hipfire page, section 03, "State formats": the opt-in q8 state keeps K and
# V as Q8_0 with bf16 index keys, 1,408 bytes per token and layer -- at 2 KV
# heads x 256 dims that is 34 bytes per 32 values of K and V (1,088 bytes)
# plus the index key and its pooled share.  Q8_0 is a block of 32 signed
# 8-bit integers with one f16 scale.  The page names the format only.
# Readings: a block's scale is its largest magnitude divided by 127 in
# float32, rounded to f16 (nearest even; an f16 overflow clamps to 65504);
# each code is the integer nearest to the float32 quotient x / scale (the
# stored f16 scale), ties to the even integer, clamped to [-127, 127]; a
# block whose scale rounds to zero stores zero codes.

Q8_BLOCK = 32
Q8_MAX = 127.0


def quantize_kv_q8_0(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Q8_0 codes (int8, same shape as ``x`` [..., D]) and f16 scales
    [..., D / 32] of float32 (or bf16-exact float32) rows."""
    x = np.asarray(x, dtype=np.float32)
    d = x.shape[-1]
    xb = x.reshape(x.shape[:-1] + (d // Q8_BLOCK, Q8_BLOCK))
    amax = np.max(np.abs(xb), axis=-1)
    with np.errstate(over="ignore"):  # an f16 overflow is clamped just below
        scale = (amax / np.float32(Q8_MAX)).astype(np.float16)
    scale = np.where(np.isinf(scale), np.float16(F16_MAX), scale)
    sf = scale.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(sf > 0, xb / np.where(sf > 0, sf, np.float32(1.0)), np.float32(0.0))
    codes = np.clip(np.rint(y), -Q8_MAX, Q8_MAX).astype(np.int8)  # rint: nearest, ties to even
    return codes.reshape(x.shape), scale


def dequantize_kv_q8_0(codes: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """float64 K or V rows from Q8_0 codes [..., D] and f16 scales [..., D / 32]."""
    c = np.asarray(codes, dtype=np.int8).astype(np.float64)
    d = c.shape[-1]
    cb = c.reshape(c.shape[:-1] + (d // Q8_BLOCK, Q8_BLOCK))
    return (cb * np.asarray(scale, dtype=np.float64)[..., None]).reshape(c.shape)
