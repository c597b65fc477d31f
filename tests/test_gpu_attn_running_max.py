"""GPU parity of the gathered attention's online softmax when the running
maximum moves (MTPLX PR #610, "What changes": float32 partials merged by
log-sum-exp, rounded once).

The kernel lets a head's running maximum lag the true one by up to 2^8 (in
base-2 logit units) and rescales its accumulators only when a logit exceeds
it by more: these cases steer the logits along the token order so that the
maximum creeps up in small steps (kept, probabilities above 1), jumps by more
than the slack (rescaled), or only falls (never moves after the first
slice), and compare with float64 attention within the bf16 tolerances.
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


def _run(Q, q, k, v, scale):
    n = k.shape[1]
    cap = -(-(n + 4) // 256) * 256
    kd = torch.zeros((HKV, cap, D), dtype=torch.bfloat16, device=DEV)
    vd = torch.zeros_like(kd)
    kd[:, :n] = to_dev(k, "bf16")
    vd[:, :n] = to_dev(v, "bf16")
    kv = Q.KvSegments.single(kd, vd, n)
    rows = torch.tensor([n - 1], dtype=torch.int64, device=DEV)
    sel = torch.arange(K_BLOCKS, dtype=torch.int32, device=DEV)[None].contiguous()
    n_sel = torch.tensor([K_BLOCKS], dtype=torch.int32, device=DEV)
    qd = to_dev(q, "bf16")
    out = torch.empty_like(qd)
    lse = torch.empty((1, HQ), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(1, Q.qsa_attn_workspace_bytes(1, HQ, D, K_BLOCKS)), dtype=torch.uint8, device=DEV)
    Q.qsa_gathered_attn(qd, rows, kv, sel, n_sel, out, lse, HKV, scale=scale, workspace=ws)
    torch.cuda.synchronize()
    return to_host_f32(out)[0], lse.cpu().numpy()[0]


def _check(Q, alpha, seed, what):
    q, k, v, scale = _case(alpha, seed)
    out, lse = _run(Q, q, k, v, scale)
    tok = O.attended_tokens(np.arange(K_BLOCKS), N_CTX)
    ref, ref_lse = O.attend(q[0], k, v, tok, scale)
    err = float(np.max(np.abs(out - ref)))
    lerr = float(np.max(np.abs(lse - ref_lse)))
    say(what, f"max-abs {err:.3g}, lse {lerr:.3g}")
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    assert err <= 2e-2, f"{what}: attention max-abs {err}"
    assert lerr <= 2.5e-3, f"{what}: lse max-abs {lerr}"


def test_running_max_creeps_and_jumps(Q):
    """Base-2 logits rising 0 -> 24 along the tokens (about 0.19 per 16-token
    slice: the lagging maximum is kept and probabilities exceed 1), with two
    jumps of +12 (past the slack: the accumulators are rescaled)."""
    t = np.arange(N_CTX, dtype=np.float64)
    alpha = 24.0 * t / N_CTX + 12.0 * (t >= 700) + 12.0 * (t >= 1500)
    _check(Q, alpha, 3, "creep + jumps")


def test_running_max_small_steps_only(Q):
    """Logits on a slow ramp, alternating every 128 tokens between two levels
    6.9 apart (below the slack): a wave's maximum, set on its first slice,
    moves only where the ramp adds up past 2^8, and its probabilities reach
    about 2^7 in between."""
    t = np.arange(N_CTX, dtype=np.float64)
    alpha = 7.0 * np.floor(t / 128.0) / 16.0 + np.where(t % 256 < 128, 0.0, 6.9)
    _check(Q, alpha, 5, "small steps")


def test_running_max_falling(Q):
    """Logits falling along the tokens: the first slice of each wave holds its
    maximum; later probabilities underflow towards zero."""
    t = np.arange(N_CTX, dtype=np.float64)
    alpha = 40.0 - 60.0 * t / N_CTX
    _check(Q, alpha, 7, "falling")
