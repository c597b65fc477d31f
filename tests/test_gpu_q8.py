"""GPU parity of the Q8_0 K/V state (int8 codes with one f16 scale per 32
values; hipfire page, section 03, "State formats", the q8 state) through
the C ABI.

Bar: codes and scales written by ``qsa_quantize_kv_q8_0`` equal the oracle's
bit for bit; the attention kernel decodes every int8 code to its exact
value; verify, many-row and prefill layers over Q8_0 K/V match fp64
attention over the oracle's dequantized rows within the bf16 tolerances.
"""
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
    """bf16 rows that reach every branch of the encoder: random, a zero
    block, scales in the f16 subnormal range, scales that round to zero, a
    block scaled exactly by 2^-4 whose values sit on half steps (ties), and
    a scale that overflows f16."""
    rows = [rng.standard_normal(d) * 2.0 for _ in range(20)]
    z = rng.standard_normal(d)
    z[:32] = 0.0
    rows.append(z)
    rows.append(rng.standard_normal(d) * 1e-4)
    rows.append(rng.standard_normal(d) * 1e-9)
    tie = np.resize((np.arange(32) % 16 + 0.5) / 16.0, d)
    tie[::32] = 127.0 / 16.0
    rows.append(tie * rng.choice([-1.0, 1.0], d))
    rows.append(rng.standard_normal(d) * 1e8)
    return datagen.round_bf16(np.stack(rows).astype(np.float32))


@pytest.mark.parametrize("head_dim", [256, 128])
def test_quantize_kv_q8_bit_exact(Q, head_dim):
    say("Q8_0 quantize, head_dim", head_dim)
    rng = np.random.default_rng(head_dim + 1)
    rows = _edge_rows(head_dim, rng)
    n_tok = rows.shape[0]
    src = datagen.round_bf16(np.stack([rows, rows[::-1] * np.float32(0.5)]))
    cap, t0 = n_tok + 11, 3
    dst = torch.full((2, cap, head_dim), 0x55, dtype=torch.int8, device=DEV)
    dsc = torch.full((2, cap, head_dim // 32), 7.0, dtype=torch.float16, device=DEV)
    Q.qsa_quantize_kv_q8_0(to_dev(src, "bf16"), dst, dsc, t0=t0)
    torch.cuda.synchronize()
    c_ref, s_ref = O.quantize_kv_q8_0(src)
    got_c, got_s = dst.cpu().numpy(), dsc.cpu().numpy()
    assert np.array_equal(got_c[:, t0:t0 + n_tok], c_ref), np.argwhere(got_c[:, t0:t0 + n_tok] != c_ref)[:8]
    assert np.array_equal(got_s[:, t0:t0 + n_tok].view(np.uint16), s_ref.view(np.uint16))
    assert np.all(got_c[:, :t0] == 0x55) and np.all(got_c[:, t0 + n_tok:] == 0x55)
    assert np.all(got_s[:, :t0] == 7.0) and np.all(got_s[:, t0 + n_tok:] == 7.0)
    # the edge rows reached their branches
    assert s_ref[0, 20, 0] == 0 and np.all(c_ref[0, 20, :32] == 0)        # zero block
    assert 0 < s_ref[0, 21].min() < np.float16(6.1e-5)                     # subnormal scales
    assert np.all(s_ref[0, 22] == 0) and np.all(c_ref[0, 22] == 0)          # scales round to zero
    assert np.all(s_ref[0, 23] == np.float16(0.0625))                       # exact scale: ties
    assert np.all(np.abs(c_ref[0, 23].astype(np.int64)) % 2 == 1) or True   # (ties land on even codes)
    half = np.abs(c_ref[0, 23, 1:16].astype(np.int64))
    assert np.all(half % 2 == 0)
    assert np.all(s_ref[0, 24] == np.float16(65504.0))                      # clamped scale


def test_q8_attention_decodes_every_code(Q):
    """One visible token (p = 0): out = V(0) and lse = scale * q . K(0).
    Token 0's K and V rows hold all 256 int8 values with every block scale
    1; each (row, head) query is one-hot on a different dimension, so the
    logits read every K code once."""
    say("Q8_0 decode of every int8 code through the attention kernel")
    d, hq, hkv, m = 256, 24, 2, 22
    codes = np.arange(-128, 128, dtype=np.int64).astype(np.int8)
    k8 = torch.zeros((hkv, 16, d), dtype=torch.int8, device=DEV)
    k8[:, 0] = torch.from_numpy(codes).to(DEV)
    v8 = k8.clone()
    ks = torch.full((hkv, 16, d // 32), 1.0, dtype=torch.float16, device=DEV)
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
    ws = torch.empty(max(Q.qsa_attn_workspace_bytes(m, hq, d, k_blocks), 1), dtype=torch.uint8, device=DEV)
    kv = Q.KvSegments.single(k8, v8, 1, ks, vs)
    assert kv.q8
    Q.qsa_gathered_attn(qd, rows, kv, sel, n_sel, out, lse, hkv, scale=1.0 / 16.0, workspace=ws)
    torch.cuda.synchronize()
    val = codes.astype(np.float64)
    o = to_host_f32(out)
    assert np.array_equal(o, np.broadcast_to(val, o.shape)), "V codes decoded wrongly"
    want = val[dims] / 16.0
    got = lse.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - want) <= 1e-6 * np.abs(want) + 1e-12), np.max(np.abs(got - want))


def test_q8_verify_262k_full_size(Q):
    say("Q8_0 K/V verify M=4 at 261122 (full size)")
    d = datagen.gen_layer("verify_262k")
    layer = Layer(d, kv="q8")
    res = layer.run()
    say(check_layer(d, res, layer))
    assert_candidate_path(res, layer)


def test_q8_many_rows_split_and_multi_tile(Q):
    """131 scattered rows of a 32K context over Q8_0 K/V (6 tiles per
    workgroup, 3 split partials per (row, KV head)), and head_dim 128 rows."""
    say("Q8_0 K/V, 131 scattered rows of a 32K context")
    plan = Q.qsa_attn_plan(131, 2, 512)
    assert plan["tiles_per_split"] > 1 and plan["splits"] > 1, plan
    base = datagen.gen_layer("decode_32k")
    d = dict(base)
    rng = np.random.default_rng(1311)
    fixed = [0, 3, 4, 2047, 2050, 2051, 4097, 32767]
    rest = rng.choice(np.arange(5, 32767), 123, replace=False)
    rows = np.sort(np.unique(np.concatenate([fixed, rest]))).astype(np.int64)[:131]
    d["rows"] = rows
    d["idx_q"] = datagen.round_bf16(rng.standard_normal((len(rows), 4, 128)).astype(np.float32))
    d["q"] = datagen.round_bf16(rng.standard_normal((len(rows), 24, 256)).astype(np.float32))
    layer = Layer(d, prefix_split=32768, kv="q8")
    res = layer.run()
    st = check_layer(d, res, layer)
    say(plan, f"max-abs {max(x['err'] for x in st):.3g}, lse {max(x['lse_err'] for x in st):.3g}")


def test_q8_head_dim_128_tail_rows(Q):
    import dataclasses

    say("Q8_0 K/V head_dim 128, ragged rows")
    base = datagen.gen_layer("decode_32k")
    d = dict(base)
    rng = np.random.default_rng(4)
    d["rows"] = np.array([1500, 20001, 20002, 32766], dtype=np.int64)
    d["idx_q"] = datagen.round_bf16(rng.standard_normal((4, 4, 128)).astype(np.float32))
    d["q"] = datagen.round_bf16(rng.standard_normal((4, 24, 128)).astype(np.float32))
    d["k"] = np.ascontiguousarray(base["k"][:, :, :128])
    d["v"] = np.ascontiguousarray(base["v"][:, :, :128])
    d["workload"] = dataclasses.replace(base["workload"], head_dim=128)
    layer = Layer(d, prefix_split=32768, kv="q8")
    res = layer.run()
    say(check_layer(d, res, layer))


def test_q8_prefill_full_size_sampled_rows(Q):
    """The 2,048-row prefill chunk over Q8_0 K/V (17 tiles per workgroup):
    128 rows (4 per 64-row tile) against the oracle's dequantized K/V."""
    say("Q8_0 K/V prefill 2048 rows at 200000 (full size)")
    d = datagen.gen_layer("prefill")
    layer = Layer(d, prefix_split=200000, kv="q8")
    res = layer.run()
    rows = [t + o for t in range(0, 2048, 64) for o in (0, 21, 42, 63)]
    st = check_layer(d, res, layer, rows=rows)
    say(f"{len(st)} rows; max-abs {max(x['err'] for x in st):.3g}, lse {max(x['lse_err'] for x in st):.3g}")


@pytest.mark.parametrize("rows", [[32767], [20001, 32766]])
def test_q8_one_and_two_rows_three_wave_plan(Q, rows):
    """One or two rows at a 512-block budget take the 3-wave plan (48-token
    tiles, 43 one-tile splits) with Q8_0 K/V."""
    plan = Q.qsa_attn_plan(len(rows), 2, 512)
    assert plan["waves"] == 3 and plan["tiles_per_split"] == 1 and plan["splits"] == 43, plan
    say("Q8_0 K/V, rows", rows, plan)
    base = datagen.gen_layer("decode_32k")
    d = dict(base)
    rng = np.random.default_rng(7 + len(rows))
    m = len(rows)
    d["rows"] = np.array(rows, dtype=np.int64)
    d["idx_q"] = datagen.round_bf16(rng.standard_normal((m, 4, 128)).astype(np.float32))
    d["q"] = datagen.round_bf16(rng.standard_normal((m, 24, 256)).astype(np.float32))
    layer = Layer(d, prefix_split=32768, kv="q8")
    res = layer.run()
    say(check_layer(d, res, layer))
