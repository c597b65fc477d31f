"""GPU parity of the fp8 K/V state (E4M3 codes + f16 scale per head and
token; hipfire page, section 03, "State formats") through the C ABI.

Bar: codes and scales written by ``qsa_quantize_kv_fp8`` equal the oracle's
bit for bit; the attention kernel decodes every E4M3 code to its exact value;
a full-size verify layer over fp8 K/V matches fp64 attention over the
oracle's dequantized rows within the bf16 tolerances.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import datagen
import oracle as O

pytestmark = pytest.mark.gpu

from gpu_harness import DEV, Layer, assert_candidate_path, check_layer, to_dev, to_host_f32  # noqa: E402


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def Q():
    import long_context_sparse_qsa_amd as Q
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    Q.qsa_device_check()
    return Q


def _edge_rows(d: int, rng) -> np.ndarray:
    """bf16 rows that reach every branch of the encoder: random, a zero row,
    scales in the f16 subnormal range, an exact scale (amax 56 -> 1/8) whose
    quotients hit every E4M3 midpoint (ties), negative zeros, values that
    round up to 448, and a scale that overflows f16."""
    grid = O.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = (grid[:-1] + grid[1:]) / 2
    rows = [rng.standard_normal(d) * 2.0 for _ in range(20)]
    rows.append(np.zeros(d))
    rows.append(rng.standard_normal(d) * 1e-3)   # scale in the f16 subnormal range
    rows.append(rng.standard_normal(d) * 3e-9)   # scale rounds to zero
    tie = np.resize(np.concatenate([mids, -mids]), d) * 0.125
    tie[0] = 56.0
    rows.append(tie)
    nz = rng.standard_normal(d)
    nz[::3] = -0.0
    rows.append(nz)
    up = np.full(d, 1.0)
    up[0] = 447.5 / 448.0 * 64.0  # quotient just below 448 after the scale rounds
    rows.append(up * rng.choice([-1.0, 1.0], d))
    rows.append(rng.standard_normal(d) * 1e8)
    x = np.stack(rows).astype(np.float32)
    return datagen.round_bf16(x)


@pytest.mark.parametrize("head_dim", [256, 128])
def test_quantize_kv_fp8_bit_exact(Q, head_dim):
    say("fp8 quantize, head_dim", head_dim)
    rng = np.random.default_rng(head_dim)
    rows = _edge_rows(head_dim, rng)                      # [R, D]
    n_tok = rows.shape[0]
    src = np.stack([rows, rows[::-1] * np.float32(0.5)])  # [2 heads, T, D]
    src = datagen.round_bf16(src)
    cap, t0 = n_tok + 13, 5
    dst = torch.full((2, cap, head_dim), 0xAA, dtype=torch.uint8, device=DEV)
    dsc = torch.full((2, cap), 7.0, dtype=torch.float16, device=DEV)
    Q.qsa_quantize_kv_fp8(to_dev(src, "bf16"), dst, dsc, t0=t0)
    torch.cuda.synchronize()
    c_ref, s_ref = O.quantize_kv_fp8(src)
    got_c = dst.cpu().numpy()
    got_s = dsc.cpu().numpy()
    assert np.array_equal(got_c[:, t0:t0 + n_tok], c_ref), np.argwhere(got_c[:, t0:t0 + n_tok] != c_ref)[:8]
    assert np.array_equal(got_s[:, t0:t0 + n_tok].view(np.uint16), s_ref.view(np.uint16))
    # rows outside [t0, t0 + T) are untouched
    assert np.all(got_c[:, :t0] == 0xAA) and np.all(got_c[:, t0 + n_tok:] == 0xAA)
    assert np.all(got_s[:, :t0] == 7.0) and np.all(got_s[:, t0 + n_tok:] == 7.0)
    # the edge rows did reach their branches
    assert s_ref[0, 20] == 0 and np.all(c_ref[0, 20] == 0)             # zero row
    assert 0 < s_ref[0, 21] < np.float16(6.1e-5)                       # subnormal scale
    assert s_ref[0, 22] == 0 and np.all(c_ref[0, 22] == 0)             # scale rounds to zero
    assert s_ref[0, 23] == np.float16(0.125)                           # exact scale: ties
    assert s_ref[0, 26] == np.float16(65504.0)                         # clamped scale


def test_fp8_attention_decodes_every_code(Q):
    """One visible token per row (p = 0): each row attends to token 0 alone,
    so out = V(0) exactly and lse = scale * q . K(0).  Token 0's K and V rows
    hold all 254 finite E4M3 codes (NaN codes replaced by 0) with scale 1;
    every (row, head) query is one-hot on a different dimension, so the 264
    logits read every K code once, through the kernel's dim permutation."""
    say("fp8 decode of every E4M3 code through the attention kernel")
    d, hq, hkv, m = 256, 24, 2, 22
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0xFF]] = 0
    k8 = torch.zeros((hkv, 16, d), dtype=torch.uint8, device=DEV)
    k8[:, 0] = torch.from_numpy(codes).to(DEV)
    v8 = k8.clone()
    ks = torch.full((hkv, 16), 1.0, dtype=torch.float16, device=DEV)
    vs = ks.clone()
    q = np.zeros((m, hq, d), np.float32)
    dims = np.zeros((m, hq), np.int64)
    for r in range(m):
        for h in range(hq):
            dims[r, h] = (r * 12 + h % 12) % 256
            q[r, h, dims[r, h]] = 1.0
    qd = to_dev(q, "bf16")
    rows = torch.zeros(m, dtype=torch.int64, device=DEV)
    k_blocks = 16
    sel = torch.full((m, k_blocks), -1, dtype=torch.int32, device=DEV)
    n_sel = torch.zeros(m, dtype=torch.int32, device=DEV)
    out = torch.empty_like(qd)
    lse = torch.empty((m, hq), dtype=torch.float32, device=DEV)
    wsa = Q.qsa_attn_workspace_bytes(m, hq, d, k_blocks)
    ws = torch.empty(max(wsa, 1), dtype=torch.uint8, device=DEV)
    kv = Q.KvSegments.single(k8, v8, 1, ks, vs)
    Q.qsa_gathered_attn(qd, rows, kv, sel, n_sel, out, lse, hkv, scale=1.0 / 16.0, workspace=ws)
    torch.cuda.synchronize()
    val = O.e4m3_decode(codes)
    o = to_host_f32(out)
    assert np.array_equal(o, np.broadcast_to(val, o.shape)), "V codes decoded wrongly"
    want = val[dims] / 16.0
    got = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - want) <= 1e-6 * np.abs(want) + 1e-12), np.max(np.abs(got - want))


def test_fp8_verify_262k_full_size(Q):
    """The verify layer (4 rows at 261,122 context) with K/V quantized on the
    device: scores and selection as for bf16, attention against the oracle's
    dequantized K/V over the GPU's selection."""
    say("fp8 K/V verify M=4 at 261122 (full size)")
    d = datagen.gen_layer("verify_262k")
    layer = Layer(d, kv="fp8")
    res = layer.run()
    say(check_layer(d, res, layer))
    assert_candidate_path(res, layer)


def test_fp8_decode_32k_head_dim_128_tail_rows(Q):
    """head_dim 128 fp8 path with ragged tails and a row whose budget covers
    the context (every block kept)."""
    say("fp8 K/V head_dim 128, ragged rows")
    base = datagen.gen_layer("decode_32k")
    d = dict(base)
    rng = np.random.default_rng(3)
    rows = np.array([1500, 20001, 20002, 32766], dtype=np.int64)
    d["rows"] = rows
    d["idx_q"] = datagen.round_bf16(rng.standard_normal((4, 4, 128)).astype(np.float32))
    d["q"] = datagen.round_bf16(rng.standard_normal((4, 24, 128)).astype(np.float32))
    d["k"] = np.ascontiguousarray(base["k"][:, :, :128])
    d["v"] = np.ascontiguousarray(base["v"][:, :, :128])
    d["workload"] = dataclasses.replace(base["workload"], head_dim=128)
    layer = Layer(d, prefix_split=32768, kv="fp8")
    res = layer.run()
    say(check_layer(d, res, layer))


def test_fp8_prefill_full_size_multi_tile(Q):
    """The 2,048-row prefill chunk over fp8 K/V: the attention plan walks 17
    tiles of 128 tokens per (row, KV head) in one workgroup, so the next
    slice's codes and scales are loaded while the current one is used.  256
    rows (8 per 64-row tile) are checked against fp64 attention over the
    oracle's dequantized K/V."""
    say("fp8 K/V prefill 2048 rows at 200000 (full size, multi-tile plan)")
    plan = Q.qsa_attn_plan(2048, 2, 512)
    assert plan["tiles_per_split"] == 17 and plan["waves"] == 8, plan
    d = datagen.gen_layer("prefill")
    layer = Layer(d, prefix_split=200000, kv="fp8")
    res = layer.run()
    offs = (0, 7, 15, 21, 31, 42, 55, 63)
    rows = [t + o for t in range(0, 2048, 64) for o in offs]
    st = check_layer(d, res, layer, rows=rows)
    assert_candidate_path(res, layer)
    say(f"{len(st)} rows; max-abs {max(x['err'] for x in st):.3g}, lse {max(x['lse_err'] for x in st):.3g}")


def test_fp8_many_rows_split_and_multi_tile(Q):
    """131 scattered rows of a 32K context over fp8 K/V: 6 tiles per workgroup
    and 3 split partials per (row, KV head) merged by the combine."""
    say("fp8 K/V, 131 scattered rows of a 32K context")
    plan = Q.qsa_attn_plan(131, 2, 512)
    assert plan["tiles_per_split"] > 1 and plan["splits"] > 1, plan
    base = datagen.gen_layer("decode_32k")
    d = dict(base)
    rng = np.random.default_rng(131)
    fixed = [0, 3, 4, 2047, 2050, 2051, 4097, 32767]
    rest = rng.choice(np.arange(5, 32767), 123, replace=False)
    rows = np.sort(np.unique(np.concatenate([fixed, rest]))).astype(np.int64)[:131]
    d["rows"] = rows
    d["idx_q"] = datagen.round_bf16(rng.standard_normal((len(rows), 4, 128)).astype(np.float32))
    d["q"] = datagen.round_bf16(rng.standard_normal((len(rows), 24, 256)).astype(np.float32))
    layer = Layer(d, prefix_split=32768, kv="fp8")
    res = layer.run()
    st = check_layer(d, res, layer)
    say(plan, f"max-abs {max(x['err'] for x in st):.3g}, lse {max(x['lse_err'] for x in st):.3g}")


@pytest.mark.parametrize("rows", [[32767], [20001, 32766]])
def test_fp8_one_and_two_rows_three_wave_plan(Q, rows):
    """One or two rows at a 512-block budget take the 3-wave plan (48-token
    tiles, 43 one-tile splits) with fp8 K/V."""
    plan = Q.qsa_attn_plan(len(rows), 2, 512)
    assert plan["waves"] == 3 and plan["tiles_per_split"] == 1 and plan["splits"] == 43, plan
    say("fp8 K/V, rows", rows, plan)
    base = datagen.gen_layer("decode_32k")
    d = dict(base)
    rng = np.random.default_rng(5 + len(rows))
    m = len(rows)
    d["rows"] = np.array(rows, dtype=np.int64)
    d["idx_q"] = datagen.round_bf16(rng.standard_normal((m, 4, 128)).astype(np.float32))
    d["q"] = datagen.round_bf16(rng.standard_normal((m, 24, 256)).astype(np.float32))
    layer = Layer(d, prefix_split=32768, kv="fp8")
    res = layer.run()
    say(check_layer(d, res, layer))
