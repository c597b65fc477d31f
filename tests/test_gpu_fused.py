"""GPU parity of qsa_append_score: the index-key append folded into the
scoring launch must leave exactly the bytes that qsa_append_pool followed by
qsa_score_blocks leave (cache, pooled keys, scores, the prepared selection),
and the pooled keys must equal the oracle's."""
import sys

import numpy as np
import pytest
import torch

import datagen
import oracle as O

pytestmark = pytest.mark.gpu

from gpu_harness import DEV, round_up, to_dev  # noqa: E402


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def Q():
    import long_context_sparse_qsa_amd as Q
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    Q.qsa_device_check()
    return Q


def _state(Q, idx, n_hist, cap, dtype):
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    cache = torch.zeros((cap, 128), dtype=tdt, device=DEV)
    pooled = torch.zeros((cap // 4, 128), dtype=torch.float32, device=DEV)
    if n_hist:
        Q.qsa_append_pool(to_dev(idx[:n_hist], dtype), torch.arange(n_hist, dtype=torch.int64, device=DEV),
                          cache, pooled)
    return cache, pooled


@pytest.mark.parametrize("wl_name,n_new,rows_back,extra_rows", [
    ("decode_32k", 1, [0], 0),          # completes the last block (nb_max - 1)
    ("decode_32k", 3, [1], 0),          # ends inside a block
    ("decode_32k", 8, [0, 1, 2, 3], 0),  # completes two blocks, M = 4
    ("decode_32k", 2, [0, 2, 5, 9, 11], 0),  # M = 5 (8-row groups)
    ("tiny", 5, [0, 1], 0),             # float32
    ("decode_32k", 4, [0], 79),         # 80 bf16 rows: the two-launch path
    ("verify_262k", 4, [0, 1, 2, 3], 0),  # full size
])
def test_append_score_equals_two_calls(Q, wl_name, n_new, rows_back, extra_rows):
    say("append+score", wl_name, "n_new", n_new, "rows", len(rows_back) + extra_rows)
    d = datagen.gen_layer(wl_name)
    wl = d["workload"]
    idx = d["idx"]
    n = idx.shape[0] - (1 if wl_name == "decode_32k" and n_new == 3 else 0)
    idx = idx[:n]
    cap = round_up(n + 4, 256)
    rng = np.random.default_rng(n_new)
    rows = sorted(set([n - 1 - b for b in rows_back] + rng.choice(n - n_new, extra_rows, replace=False).tolist()))
    rows_t = torch.tensor(rows, dtype=torch.int64, device=DEV)
    m = len(rows)
    idx_q = to_dev(datagen.round_bf16(rng.standard_normal((m, 4, 128)).astype(np.float32)), wl.dtype)
    nb_max = (max(rows) + 1) // 4
    ld = max(4, round_up(nb_max, 4))
    new = to_dev(np.ascontiguousarray(idx[n - n_new:]), wl.dtype)
    pos = torch.arange(n - n_new, n, dtype=torch.int64, device=DEV)
    k = wl.k_blocks
    wsb = Q.qsa_select_workspace_bytes(m, nb_max, k)
    outs = []
    for fused in (False, True):
        cache, pooled = _state(Q, idx, n - n_new, cap, wl.dtype)
        scores = torch.full((m, ld), -3.0, dtype=torch.float32, device=DEV)
        ws = torch.zeros(max(wsb, 1), dtype=torch.uint8, device=DEV)
        if fused:
            Q.qsa_append_score(new, pos, cache, pooled, idx_q, rows_t, scores, nb_max, sel_workspace=ws)
        else:
            Q.qsa_append_pool(new, pos, cache, pooled)
            Q.qsa_score_blocks(idx_q, rows_t, pooled, scores, nb_max, sel_workspace=ws)
        sel = torch.empty((m, k), dtype=torch.int32, device=DEV)
        n_sel = torch.empty((m,), dtype=torch.int32, device=DEV)
        Q.qsa_select_topk(scores, rows_t, nb_max, k, sel, n_sel, ws, prepared=True)
        torch.cuda.synchronize()
        outs.append((cache, pooled, scores, sel, n_sel))
    (c0, p0, s0, sel0, n0), (c1, p1, s1, sel1, n1) = outs
    assert torch.equal(c0.view(torch.int16) if c0.dtype == torch.bfloat16 else c0.view(torch.int32),
                       c1.view(torch.int16) if c1.dtype == torch.bfloat16 else c1.view(torch.int32))
    assert torch.equal(p0.view(torch.int32), p1.view(torch.int32))
    assert torch.equal(s0.view(torch.int32), s1.view(torch.int32))
    assert torch.equal(sel0, sel1) and torch.equal(n0, n1)
    ref = O.pool_index_keys(idx)
    assert np.array_equal(p1[: n // 4].cpu().numpy().view(np.uint32), ref.view(np.uint32))
