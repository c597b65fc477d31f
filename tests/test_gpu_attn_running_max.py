"""GPU parity of the gathered attention's online softmax when the running
maximum moves (MTPLX PR #610, "What changes": float32 partials merged by
log-sum-exp, rounded once).

The kernel lets a head's running maximum lag the true one by up to 2^8 (in
base-2 logit units) and rescales its accumulators only when a logit exceeds
it by more.  Each wave of a workgroup owns one 16-token slice of every tile
its workgroup walks, so the maximum can only lag or move between slices of
one wave when the plan gives a workgroup several tiles.  The cases run
twice: with one row (one tile per workgroup: every wave sees one slice, so
its maximum is set once) and with 131 identical rows, where the plan walks 6
tiles of 128 tokens per workgroup (asserted).  The logits are steered along
the token order so that the maximum creeps up in small steps (kept,
probabilities above 1), jumps by more than the slack (the accumulators are
rescaled: a host replay of the rule over the plan's slices counts the
rescales) or only falls, and every row is compared with float64 attention
within the bf16 tolerances.
"""
import math
import sys

import numpy as np
import pytest
import torch

import datagen
import oracle as O

pytestmark = pytest.mark.gpu

from gpu_harness import DEV, to_dev, to_host_f32  # noqa: E402

HQ, HKV, D = 24, 2, 256
K_BLOCKS = 512
N_CTX = 4 * K_BLOCKS + 3  # every block kept, plus a 3-token tail


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def Q():
    import long_context_sparse_qsa_amd as Q
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    Q.qsa_device_check()
    return Q


def _case(alpha: np.ndarray, seed: int):
    """q, K, V (bf16-exact float32) whose base-2 logits follow ``alpha`` per
    token for every query head (up to small per-head and per-token noise)."""
    rng = np.random.default_rng(seed)
    scale = 1.0 / math.sqrt(D)
    u = rng.standard_normal((HKV, D)).astype(np.float32)
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    q = np.repeat(u, HQ // HKV, axis=0) * np.float32(4.0)
    q += np.float32(0.02) * rng.standard_normal(q.shape).astype(np.float32)
    q = datagen.round_bf16(q[None])
    # q_h . k_t * scale * log2(e) ~ alpha_t
    c = alpha / (4.0 * scale * math.log2(math.e))
    k = c[None, :, None] * u[:, None, :]
    k = k + np.float32(0.01) * rng.standard_normal(k.shape)
    k = datagen.round_bf16(k.astype(np.float32))
    v = datagen.round_bf16(rng.standard_normal((HKV, len(alpha), D)).astype(np.float32))
    return q, k, v, scale


def _run(Q, q, k, v, scale, m):
    n = k.shape[1]
    cap = -(-(n + 4) // 256) * 256
    kd = torch.zeros((HKV, cap, D), dtype=torch.bfloat16, device=DEV)
    vd = torch.zeros_like(kd)
    kd[:, :n] = to_dev(k, "bf16")
    vd[:, :n] = to_dev(v, "bf16")
    kv = Q.KvSegments.single(kd, vd, n)
    rows = torch.full((m,), n - 1, dtype=torch.int64, device=DEV)
    sel = torch.arange(K_BLOCKS, dtype=torch.int32, device=DEV)[None].repeat(m, 1).contiguous()
    n_sel = torch.full((m,), K_BLOCKS, dtype=torch.int32, device=DEV)
    qd = to_dev(np.repeat(q, m, axis=0), "bf16")
    out = torch.empty_like(qd)
    lse = torch.empty((m, HQ), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(1, Q.qsa_attn_workspace_bytes(m, HQ, D, K_BLOCKS)), dtype=torch.uint8, device=DEV)
    Q.qsa_gathered_attn(qd, rows, kv, sel, n_sel, out, lse, HKV, scale=scale, workspace=ws)
    torch.cuda.synchronize()
    return to_host_f32(out), lse.cpu().numpy()


def rescales(alpha: np.ndarray, plan: dict, slack: float = 8.0) -> int:
    """Host replay of the lagging-maximum rule over the plan's slices: wave w
    of split s reads tokens s*T*W + t*T + 16 w .. + 15 for tile t < tiles per
    split (T tokens per tile); its maximum moves when a slice's maximum
    exceeds it by more than the slack.  Counts the moves from a finite
    maximum, i.e. the accumulator rescales."""
    tt, tps, sp = plan["tile_tokens"], plan["tiles_per_split"], plan["splits"]
    count = 0
    for s in range(sp):
        for w in range(plan["waves"]):
            m = -np.inf
            for t in range(tps):
                j0 = s * tps * tt + t * tt + 16 * w
                if j0 >= len(alpha):
                    break
                rmax = float(np.max(alpha[j0:j0 + 16]))
                if rmax > m + slack:
                    count += np.isfinite(m)
                    m = rmax
    return count


ROWS = [1, 131]  # one tile per workgroup; 6 tiles per workgroup (3 splits)


def _check(Q, alpha, seed, what, m):
    plan = Q.qsa_attn_plan(m, HKV, K_BLOCKS)
    if m > 1:
        assert plan["tiles_per_split"] > 1, plan
    q, k, v, scale = _case(alpha, seed)
    out, lse = _run(Q, q, k, v, scale, m)
    tok = O.attended_tokens(np.arange(K_BLOCKS), N_CTX)
    ref, ref_lse = O.attend(q[0], k, v, tok, scale)
    err = float(np.max(np.abs(out - ref[None])))
    lerr = float(np.max(np.abs(lse - ref_lse[None])))
    n_resc = rescales(alpha, plan)
    say(what, f"M={m} plan {plan}: {n_resc} rescales; max-abs {err:.3g}, lse {lerr:.3g}")
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    assert err <= 2e-2, f"{what}: attention max-abs {err}"
    assert lerr <= 1e-3, f"{what}: lse max-abs {lerr}"
    return plan, n_resc


@pytest.mark.parametrize("m", ROWS)
def test_running_max_creeps_and_jumps(Q, m):
    """Base-2 logits rising 0 -> 24 along the tokens (about 0.19 per 16-token
    slice: the lagging maximum is kept and probabilities exceed 1), with two
    jumps of +12 (past the slack: the accumulators are rescaled when a wave
    walks several tiles)."""
    t = np.arange(N_CTX, dtype=np.float64)
    alpha = 24.0 * t / N_CTX + 12.0 * (t >= 700) + 12.0 * (t >= 1500)
    plan, n_resc = _check(Q, alpha, 3, "creep + jumps", m)
    if plan["tiles_per_split"] > 1:
        assert n_resc > 0


@pytest.mark.parametrize("m", ROWS)
def test_running_max_small_steps_only(Q, m):
    """Logits on a slow ramp, alternating every 128 tokens between two levels
    6.9 apart (below the slack): a wave's maximum, set on its first slice,
    moves only where the ramp adds up past 2^8, and its probabilities reach
    about 2^7 in between."""
    t = np.arange(N_CTX, dtype=np.float64)
    alpha = 7.0 * np.floor(t / 128.0) / 16.0 + np.where(t % 256 < 128, 0.0, 6.9)
    _check(Q, alpha, 5, "small steps", m)


@pytest.mark.parametrize("m", ROWS)
def test_running_max_falling(Q, m):
    """Logits falling along the tokens: the first slice of each wave holds its
    maximum; later probabilities underflow towards zero."""
    t = np.arange(N_CTX, dtype=np.float64)
    alpha = 40.0 - 60.0 * t / N_CTX
    _check(Q, alpha, 7, "falling", m)
