"""The C ABI on the CPU: the library loads, exports every symbol qsa.h
declares, and refuses bad arguments with its status codes before anything
is enqueued (no GPU work is started by these calls)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")

Q = pytest.importorskip("long_context_sparse_qsa_amd", reason="libqsa.so not built")


def declared_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(qsa_[a-z_0-9]+)\s*\(", txt, flags=re.M)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("qsa_append_pool", "qsa_score_blocks", "qsa_select_topk", "qsa_gathered_attn"):
        assert n in names
    assert set(names) == set(Q.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(Q.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_empty_error():
    assert "gfx950" in Q.version()


L = Q.lib()
ERR_ARG, ERR_UNS, ERR_WS = Q.QSA_ERR_ARG, Q.QSA_ERR_UNSUPPORTED, Q.QSA_ERR_WORKSPACE
FAKE = 0x1000  # never dereferenced: every call below fails validation first


def _err():
    return L.qsa_last_error().decode()


@pytest.mark.parametrize("args,code,word", [
    ((FAKE, 7, 1, FAKE, None, FAKE, FAKE, 1, 16, None), ERR_ARG, "dtype"),
    ((FAKE, 1, -1, FAKE, None, FAKE, FAKE, 1, 16, None), ERR_ARG, "n_new"),
    ((FAKE, 1, 1, FAKE, None, FAKE, FAKE, 0, 16, None), ERR_ARG, "n_seq"),
    ((FAKE, 1, 1, FAKE, None, FAKE, FAKE, 1, 18, None), ERR_ARG, "capacity"),
    ((FAKE, 1, 1, None, None, FAKE, FAKE, 1, 16, None), ERR_ARG, "null"),
    ((None, 1, 0, None, None, None, None, 1, 16, None), Q.QSA_OK, ""),
])
def test_append_pool_validation(args, code, word):
    assert L.qsa_append_pool(*args) == code
    assert word in _err()


@pytest.mark.parametrize("args,code,word", [
    ((FAKE, 3, 1, FAKE, None, FAKE, 1, 64, 16, FAKE, 16, None, 0, None), ERR_ARG, "dtype"),
    ((FAKE, 1, -2, FAKE, None, FAKE, 1, 64, 16, FAKE, 16, None, 0, None), ERR_ARG, "M ="),
    ((FAKE, 1, 1, FAKE, None, FAKE, 1, 64, 17, FAKE, 17, None, 0, None), ERR_ARG, "nb_max"),
    ((FAKE, 1, 1, FAKE, None, FAKE, 1, 64, 16, FAKE, 8, None, 0, None), ERR_ARG, "ld"),
    ((FAKE, 1, 1, FAKE, None, FAKE, 1, 64, 16, FAKE, 18, None, 0, None), ERR_ARG, "aligned"),
    ((FAKE, 1, 1, FAKE, None, FAKE, 1, 64, 16, FAKE + 4, 16, None, 0, None), ERR_ARG, "aligned"),
    ((FAKE, 1, 1, FAKE, None, None, 1, 64, 16, FAKE, 16, None, 0, None), ERR_ARG, "null"),
    # the index queries are read 16 bytes at a time
    ((FAKE + 8, 1, 1, FAKE, None, FAKE, 1, 64, 16, FAKE, 16, None, 0, None), ERR_ARG, "idx_q must be 16-byte"),
    ((FAKE, 1, 1, FAKE, None, FAKE, 1, 64, 16, FAKE, 16, FAKE, 100, None), ERR_WS, "workspace"),
    # 64 bf16 rows take the many-row kernel, whose buffer views of 16 score
    # rows must stay under 2 GiB
    ((FAKE, 1, 64, FAKE, None, FAKE, 1, 64, 16, FAKE, 1 << 25, None, 0, None), ERR_UNS, "many-row"),
    ((None, 1, 0, None, None, None, 1, 64, 16, None, 16, None, 0, None), Q.QSA_OK, ""),
])
def test_score_validation(args, code, word):
    assert L.qsa_score_blocks(*args) == code
    assert word in _err()


@pytest.mark.parametrize("args,code,word", [
    ((FAKE, 16, 1, FAKE, 16, 0, FAKE, FAKE, None, 0, 0, None), ERR_ARG, "k_blocks"),
    ((FAKE, 16, 1, FAKE, 16, 2000, FAKE, FAKE, None, 0, 0, None), ERR_ARG, "k_blocks"),
    ((FAKE, 8, 1, FAKE, 16, 4, FAKE, FAKE, None, 0, 0, None), ERR_ARG, "ld"),
    ((FAKE, 18, 1, FAKE, 16, 4, FAKE, FAKE, None, 0, 0, None), ERR_ARG, "aligned"),
    ((FAKE + 4, 16, 1, FAKE, 16, 4, FAKE, FAKE, None, 0, 0, None), ERR_ARG, "aligned"),
    ((FAKE, 16, 1, FAKE, 16, 4, FAKE, FAKE, None, 0, 0, None), ERR_WS, "workspace"),
    ((FAKE, 16, 1, FAKE, 16, 4, FAKE, FAKE, FAKE, 100, 0, None), ERR_WS, "workspace"),
    ((FAKE, 16, 1, FAKE, 16, 4, None, FAKE, FAKE, 1 << 30, 0, None), ERR_ARG, "null"),
    ((FAKE, 16, 1, FAKE, 16, 4, FAKE, FAKE, FAKE, 1 << 30, 2, None), ERR_ARG, "prepared"),
    ((None, 16, 0, None, 16, 4, None, None, None, 0, 0, None), Q.QSA_OK, ""),
])
def test_select_validation(args, code, word):
    assert L.qsa_select_topk(*args) == code
    assert word in _err()


def _kv(n_seq=1, n_seg=1, max_seg=1, null=False, fmt=0, scales=False):
    sc = FAKE if scales else None
    return Q.QsaKvSegments(n_seq, n_seg, max_seg, fmt, None if null else FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                           sc, sc)


def _attn(dtype=1, M=1, hq=24, hkv=2, d=256, scale=0.0625, kv=None, k=512, ws=FAKE, wsb=1 << 30,
          out=FAKE, q=FAKE):
    kv = kv or _kv()
    return L.qsa_gathered_attn(q, dtype, M, hq, hkv, d, scale, FAKE, None, ctypes.byref(kv), FAKE,
                               FAKE, k, out, FAKE, ws, wsb, None)


@pytest.mark.parametrize("kw,code,word", [
    (dict(dtype=5), ERR_ARG, "dtype"),
    (dict(M=-1), ERR_ARG, "M ="),
    (dict(hq=25), ERR_ARG, "multiple"),
    (dict(hq=16, hkv=2), ERR_UNS, "12"),
    (dict(d=64), ERR_UNS, "head_dim"),
    (dict(dtype=0, d=256), ERR_UNS, "float32"),
    (dict(scale=float("nan")), ERR_ARG, "scale"),
    (dict(scale=float("inf")), ERR_ARG, "scale"),
    (dict(k=0), ERR_ARG, "k_blocks"),
    (dict(kv=_kv(n_seq=0)), ERR_ARG, "n_seq"),
    (dict(kv=_kv(max_seg=17)), ERR_UNS, "max_seg"),
    (dict(kv=_kv(null=True)), ERR_ARG, "null"),
    (dict(ws=None, wsb=0), ERR_WS, "workspace"),
    (dict(wsb=100), ERR_WS, "workspace"),
    (dict(out=None), ERR_ARG, "null"),
    (dict(out=FAKE + 8), ERR_ARG, "aligned"),
    (dict(q=FAKE + 8), ERR_ARG, "q must be 16-byte"),
    (dict(ws=FAKE + 4), ERR_ARG, "aligned"),
    (dict(M=0, ws=None, wsb=0), Q.QSA_OK, ""),
])
def test_attn_validation(kw, code, word):
    assert _attn(**kw) == code
    assert word in _err()


@pytest.mark.parametrize("kw,code,word", [
    (dict(kv=_kv(fmt=7)), ERR_ARG, "kv_format"),
    (dict(kv=_kv(fmt=Q.QSA_KV_FP8_E4M3)), ERR_ARG, "scale"),
    (dict(kv=_kv(fmt=Q.QSA_KV_FP8_E4M3, scales=True), dtype=0, d=128), Q.QSA_ERR_UNSUPPORTED, "bf16"),
    (dict(kv=_kv(fmt=Q.QSA_KV_FP8_E4M3, scales=True), wsb=0), Q.QSA_ERR_WORKSPACE, "workspace"),
    (dict(kv=_kv(fmt=Q.QSA_KV_Q8_0)), ERR_ARG, "Q8_0 K/V needs"),
    (dict(kv=_kv(fmt=Q.QSA_KV_Q8_0, scales=True), dtype=0, d=128), Q.QSA_ERR_UNSUPPORTED, "bf16"),
    (dict(kv=_kv(fmt=Q.QSA_KV_Q8_0, scales=True), wsb=0), Q.QSA_ERR_WORKSPACE, "workspace"),
])
def test_attn_quantized_validation(kw, code, word):
    assert _attn(**kw) == code
    assert word in _err()


def _quant(src=FAKE, nh=2, nt=4, d=256, shs=4, dst=FAKE, dsc=FAKE, dhs=16):
    return L.qsa_quantize_kv_fp8(src, nh, nt, d, shs, dst, dsc, dhs, None)


@pytest.mark.parametrize("kw,code,word", [
    (dict(nh=-1), ERR_ARG, "n_head"),
    (dict(nt=-3), ERR_ARG, "n_tok"),
    (dict(d=64), Q.QSA_ERR_UNSUPPORTED, "head_dim"),
    (dict(shs=3), ERR_ARG, "stride"),
    (dict(dhs=2), ERR_ARG, "stride"),
    (dict(src=None), ERR_ARG, "null"),
    (dict(dst=FAKE + 8), ERR_ARG, "aligned"),
    (dict(dsc=FAKE + 1), ERR_ARG, "aligned"),
    (dict(nt=0, src=None, dst=None, dsc=None), Q.QSA_OK, ""),
])
def test_quantize_kv_fp8_validation(kw, code, word):
    assert _quant(**kw) == code
    assert word in _err()


def _quant_q8(src=FAKE, nh=2, nt=4, d=256, shs=4, dst=FAKE, dsc=FAKE, dhs=16):
    return L.qsa_quantize_kv_q8_0(src, nh, nt, d, shs, dst, dsc, dhs, None)


@pytest.mark.parametrize("kw,code,word", [
    (dict(nh=-1), ERR_ARG, "n_head"),
    (dict(nt=-3), ERR_ARG, "n_tok"),
    (dict(d=64), Q.QSA_ERR_UNSUPPORTED, "head_dim"),
    (dict(d=192), Q.QSA_ERR_UNSUPPORTED, "head_dim"),
    (dict(shs=3), ERR_ARG, "stride"),
    (dict(dhs=2), ERR_ARG, "stride"),
    (dict(dst=None), ERR_ARG, "null"),
    (dict(dsc=None), ERR_ARG, "null"),
    (dict(src=FAKE + 2), ERR_ARG, "aligned"),
    (dict(dst=FAKE + 8), ERR_ARG, "aligned"),
    (dict(dsc=FAKE + 1), ERR_ARG, "aligned"),
    (dict(nh=0, src=None, dst=None, dsc=None), Q.QSA_OK, ""),
])
def test_quantize_kv_q8_0_validation(kw, code, word):
    assert _quant_q8(**kw) == code
    assert "qsa_quantize_kv_q8_0" in _err() or code == Q.QSA_OK
    assert word in _err()


def test_attn_null_kv():
    r = L.qsa_gathered_attn(FAKE, 1, 1, 24, 2, 256, 0.1, FAKE, None, None, FAKE, FAKE, 512, FAKE,
                            FAKE, FAKE, 1 << 30, None)
    assert r == ERR_ARG and "kv" in _err()


def test_workspace_sizes():
    # one row, 2 KV heads, budget 512 blocks = 2,051 tokens at most: 43
    # splits of 48 tokens in the bf16 plan (3 waves), 33 of 64 in the float32
    # one; a partial per head holds 256 floats of output and two lse values
    # (that of the normaliser it was divided by, and that of the float32
    # probabilities)
    assert Q.qsa_attn_workspace_bytes(1, 24, 256, 512) == 1 * 24 * 43 * 258 * 4
    # up to four rows: the bf16 plan needs at most 4 x 26 partials per head
    # (four rows in 5-wave workgroups); the float32 plan keeps 33 splits of
    # 64 tokens at four rows, which is the largest need
    assert Q.qsa_attn_workspace_bytes(4, 24, 256, 512) == 4 * 24 * 33 * 258 * 4
    # sizing is monotone in max_M (a call with fewer rows always fits)
    prev = 0
    for m in (1, 2, 3, 4, 8, 16, 64, 256, 2048):
        cur = Q.qsa_attn_workspace_bytes(m, 24, 256, 512)
        assert cur >= prev
        prev = cur
    assert Q.qsa_attn_workspace_bytes(0, 24, 256, 512) == 0


def test_attn_plan_query():
    """The plan query answers on the host and refuses bad arguments."""
    p1 = Q.qsa_attn_plan(1, 2, 512)
    assert p1 == {"waves": 3, "tile_tokens": 48, "tiles_per_split": 1, "splits": 43}
    assert Q.qsa_attn_plan(4, 2, 512) == {"waves": 5, "tile_tokens": 80, "tiles_per_split": 1, "splits": 26}
    pf = Q.qsa_attn_plan(2048, 2, 512)
    assert pf["waves"] == 8 and pf["tiles_per_split"] * pf["tile_tokens"] * pf["splits"] >= 2051
    out = (ctypes.c_int32 * 4)()
    assert L.qsa_attn_plan(0, 2, 512, 1, out) == ERR_ARG and "M" in _err()
    assert L.qsa_attn_plan(1, 2, 0, 1, out) == ERR_ARG and "k_blocks" in _err()
    assert L.qsa_attn_plan(1, 2, 512, 9, out) == ERR_ARG and "dtype" in _err()
    assert L.qsa_attn_plan(1, 2, 512, 1, None) == ERR_ARG and "NULL" in _err()
    # select: one fixed-size record per row (histogram, candidate list)
    per_row = Q.qsa_select_workspace_bytes(1, 65280, 512)
    assert per_row > 0 and Q.qsa_select_workspace_bytes(4, 65280, 512) == 4 * per_row


def _ssel(M=2, nb=100, k=16, ws=FAKE, wsb=1 << 30, idx=FAKE):
    return L.qsa_score_select(idx, M, FAKE, FAKE, nb, k, FAKE, FAKE, ws, wsb, None)


@pytest.mark.parametrize("kw,code,word", [
    (dict(M=-1), ERR_ARG, "M ="),
    (dict(nb=-1), ERR_ARG, "nb_max"),
    (dict(nb=(1 << 30) + 1), ERR_ARG, "nb_max"),
    (dict(k=0), ERR_ARG, "k_blocks"),
    (dict(k=5000), ERR_ARG, "k_blocks"),
    (dict(wsb=100), ERR_WS, "workspace"),
    (dict(ws=None), ERR_WS, "workspace"),
    (dict(ws=FAKE + 4), ERR_ARG, "aligned"),
    (dict(idx=None), ERR_ARG, "null"),
    (dict(idx=FAKE + 8), ERR_ARG, "idx_q must be 16-byte"),
    (dict(M=0, ws=None, wsb=0), Q.QSA_OK, ""),
])
def test_score_select_validation(kw, code, word):
    assert _ssel(**kw) == code
    assert word in _err()


def test_score_select_workspace_bytes():
    # per row: threshold, count, path (rounded to 64 rows), the sample (one
    # word per 16 blocks, rounded to 64 words), 4,096 (key, id) slots
    m, nb = 2048, 50512
    n_grp = -(-nb // 16)
    words = 3 * 2048 + (-(-(m * n_grp) // 64) * 64) + 2 * m * 4096
    assert Q.qsa_score_select_workspace_bytes(m, nb, 512) == 4 * words
    assert Q.qsa_score_select_workspace_bytes(0, nb, 512) == 0
    # far below the M x nb score matrix it replaces
    assert Q.qsa_score_select_workspace_bytes(m, nb, 512) < m * nb * 4 / 4


def _apsc(dtype=1, n_new=4, M=1, cap=64, nb=16, ld=16, scores=FAKE, ws=None, wsb=0, new=FAKE, idx_q=FAKE):
    return L.qsa_append_score(new, n_new, FAKE, FAKE, FAKE, cap, idx_q, dtype, M, FAKE, nb, scores, ld, ws, wsb, None)


@pytest.mark.parametrize("kw,code,word", [
    (dict(dtype=4), ERR_ARG, "dtype"),
    (dict(n_new=-1), ERR_ARG, "n_new"),
    (dict(M=-1), ERR_ARG, "M ="),
    (dict(cap=62), ERR_ARG, "capacity"),
    (dict(nb=17), ERR_ARG, "nb_max"),
    (dict(ld=8), ERR_ARG, "ld"),
    (dict(ld=18), ERR_ARG, "aligned"),
    (dict(ws=FAKE, wsb=100), ERR_WS, "workspace"),
    (dict(M=64, ld=1 << 25), ERR_UNS, "many-row"),
    (dict(new=None), ERR_ARG, "null"),
    (dict(idx_q=None), ERR_ARG, "null"),
    (dict(idx_q=FAKE + 2), ERR_ARG, "idx_q must be 16-byte"),
    (dict(n_new=0, M=0, new=None, idx_q=None), Q.QSA_OK, ""),
])
def test_append_score_validation(kw, code, word):
    assert _apsc(**kw) == code
    assert word in _err()

