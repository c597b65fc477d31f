"""GPU check of qsa_gathered_attn_noalloc, the allocation-free variant of
qsa_gathered_attn (split partials in the library's static device scratch):
through the C ABI, two calls in a row -- the 261,122-token verify layer with
4 rows, then the same layer with its last row only (a smaller call, whose
split plan differs, over scratch that still holds the first call's
partials) -- each bit-identical to qsa_gathered_attn with a caller
workspace, and within the attention bar of the oracle."""
import math
import sys

import numpy as np
import pytest
import torch

import datagen

pytestmark = pytest.mark.gpu

from gpu_harness import DEV, Layer, check_attention, to_host_f32  # noqa: E402


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def Q():
    import long_context_sparse_qsa_amd as Q
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    Q.qsa_device_check()
    return Q


def _both(Q, layer, rows, q, sel, n_sel):
    """(out, lse) of the workspace entry point and of the allocation-free one."""
    wl = layer.wl
    m = q.shape[0]
    scale = 1.0 / math.sqrt(wl.head_dim)
    out_ws = torch.full_like(q, 7.0)
    lse_ws = torch.full((m, wl.hq), 7.0, dtype=torch.float32, device=DEV)
    ws = torch.empty(max(1, Q.qsa_attn_workspace_bytes(m, wl.hq, wl.head_dim, sel.shape[1])), dtype=torch.uint8,
                     device=DEV)
    Q.qsa_gathered_attn(q, rows, layer.kv, sel, n_sel, out_ws, lse_ws, wl.hkv, scale=scale, workspace=ws)
    out_na = torch.full_like(q, -3.0)
    lse_na = torch.full((m, wl.hq), -3.0, dtype=torch.float32, device=DEV)
    Q.qsa_gathered_attn_noalloc(q, rows, layer.kv, sel, n_sel, out_na, lse_na, wl.hkv, scale=scale)
    torch.cuda.synchronize()
    return out_ws, lse_ws, out_na, lse_na


def test_noalloc_attention_two_calls(Q):
    say("allocation-free attention: verify M=4 at 261122, then M=1")
    d = datagen.gen_layer("verify_262k")
    layer = Layer(d)
    res = layer.run()  # scores and selection through the ordinary entry points
    sel, n_sel = res["sel"], res["n_sel"]
    calls = [("M=4", layer.rows, layer.q, sel, n_sel, list(range(4))),
             ("M=1", layer.rows[3:].contiguous(), layer.q[3:].contiguous(), sel[3:].contiguous(),
              n_sel[3:].contiguous(), [3])]
    for what, rows, q, s_, ns, host_rows in calls:
        plan = Q.qsa_attn_plan(q.shape[0], layer.wl.hkv, s_.shape[1])
        assert plan["splits"] > 1, plan  # the partials go through the static scratch
        out_ws, lse_ws, out_na, lse_na = _both(Q, layer, rows, q, s_, ns)
        assert torch.equal(out_na.view(torch.int16), out_ws.view(torch.int16)), what
        assert torch.equal(lse_na, lse_ws), what
        o, l_ = to_host_f32(out_na), lse_na.cpu().numpy()
        sh = s_.cpu().numpy()
        nh = ns.cpu().numpy()
        for j, i in enumerate(host_rows):
            err, lerr = check_attention(o[j], l_[j], d, i, sh[j, : nh[j]], "bf16")
        say(what, plan, "bit-identical to the workspace entry point; last row max-abs", f"{err:.3g}")


def test_noalloc_rejects_bad_arguments(Q):
    """Validation is the ordinary entry point's (nothing launched)."""
    d = datagen.gen_layer("tiny")
    layer = Layer(d)
    q = layer.q
    sel = torch.zeros((1, 64), dtype=torch.int32, device=DEV)
    n_sel = torch.zeros((1,), dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty((1, 24), dtype=torch.float32, device=DEV)
    with pytest.raises(Q.QsaError, match="qsa_gathered_attn_noalloc: scale"):
        Q.qsa_gathered_attn_noalloc(q, layer.rows, layer.kv, sel, n_sel, out, lse, 2, scale=float("nan"))
