"""The few-row scorer's two store forms give the same bytes.

Scores (and the selection sample of a prepared selection) normally leave
through buffer views of each 4-row column set; a score matrix whose rows are
2^27 floats or longer does not fit such a view and takes the branching
stores instead.  Both forms must write exactly the same scores, touch no
entry past a row's visible blocks, and prepare the same selection.  The
scores of the ordinary form are also checked against the oracle's fp64
scores within the acceptance band, on seeded synthetic inputs."""
import sys

import numpy as np
import pytest
import torch

import oracle as O

pytestmark = pytest.mark.gpu

from gpu_harness import DEV, round_up  # noqa: E402

WIDE_LD = (1 << 27) + 4  # floats per score row: past what a 4-row buffer view can address


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def Q():
    import long_context_sparse_qsa_amd as Q
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    Q.qsa_device_check()
    return Q


def _inputs(nb_max, m, seed):
    rng = np.random.default_rng(seed)
    pooled = rng.standard_normal((nb_max, 128)).astype(np.float32)
    idx_q = rng.standard_normal((m, 4, 128)).astype(np.float32)
    idx_q = torch.from_numpy(idx_q).to(torch.bfloat16)  # the rows' queries, rounded to bf16
    # rows ending at the last visible block and at ragged earlier positions
    pos = np.array([4 * nb_max - 1 - 4 * 97 * i - (i % 4) for i in range(m)], dtype=np.int64)
    return pooled, idx_q, pos


@pytest.mark.parametrize("nb_max", [3000, 20000])  # two-wave and four-wave workgroups
@pytest.mark.parametrize("m", [1, 3, 6])            # one and two column sets
def test_wide_rows_take_the_branching_stores_with_equal_bytes(Q, nb_max, m):
    say(f"store forms nb_max={nb_max} m={m}")
    pooled, idx_q, pos = _inputs(nb_max, m, seed=1000 + nb_max + m)
    pooled_d = torch.from_numpy(pooled).to(DEV)
    q_d = idx_q.to(DEV).contiguous()
    pos_d = torch.from_numpy(pos).to(DEV)
    nb = np.minimum((pos + 1) // 4, nb_max)
    k = 512
    wsb = Q.qsa_select_workspace_bytes(m, nb_max, k)
    res = {}
    for name, ld in (("views", round_up(nb_max, 4)), ("wide", WIDE_LD)):
        scores = torch.full((m, ld), float("nan"), dtype=torch.float32, device=DEV)
        ws = torch.zeros(wsb // 4, dtype=torch.int32, device=DEV)
        Q.qsa_score_blocks(q_d, pos_d, pooled_d, scores, nb_max, sel_workspace=ws)
        sel = torch.empty((m, k), dtype=torch.int32, device=DEV)
        n_sel = torch.empty(m, dtype=torch.int32, device=DEV)
        Q.qsa_select_topk(scores, pos_d, nb_max, k, sel, n_sel, workspace=ws, prepared=True)
        torch.cuda.synchronize()
        res[name] = (scores[:, :nb_max + 64].cpu().numpy() if ld > nb_max + 64 else scores.cpu().numpy(),
                     sel.cpu().numpy(), n_sel.cpu().numpy())
        del scores, ws
    torch.cuda.empty_cache()
    sv, sw = res["views"][0], res["wide"][0]
    for r in range(m):
        n = int(nb[r])
        assert np.array_equal(sv[r, :n].view(np.uint32), sw[r, :n].view(np.uint32)), f"row {r}: scores differ"
        # nothing past the row's visible blocks is written (NaN sentinels stay)
        assert np.isnan(sw[r, n:nb_max + 64]).all(), f"row {r}: wide form wrote past block {n}"
        assert np.isnan(sv[r, n:]).all(), f"row {r}: view form wrote past block {n}"
    assert np.array_equal(res["views"][1], res["wide"][1]) and np.array_equal(res["views"][2], res["wide"][2])
    # the scores against the oracle's fp64 ones (two rows are enough for the pin)
    q32 = idx_q.to(torch.float32).numpy().astype(np.float64)
    for r in range(min(m, 2)):
        n = int(nb[r])
        s64 = O.score_blocks(q32[r], pooled.astype(np.float64), int(pos[r]) + 1)[:n]
        tol = 1e-5 * np.abs(s64) + 1e-6
        assert np.all(np.abs(sv[r, :n].astype(np.float64) - s64) <= tol), f"row {r}: scores off the oracle"
