"""A whole layer step captured in a HIP graph gives, on every replay, exactly
the bytes the same step gives when enqueued eagerly.

The library promises that every entry point enqueues only kernels on the
caller's stream (no allocation, no memset, no host synchronisation), so a
step can be captured and replayed; and that the selection workspace needs no
initialisation between calls (the scoring launch clears each row's arrival
counter and the last arriving collect workgroup clears it again).  Replays
are interleaved with eager steps and with eager writes over every output, and
each replay is compared with the eager result bit for bit.  The step is the
one the benchmark captures: the append folded into the scoring launch (the
rows' own last tokens appended again, which rewrites the same bytes), the
prepared selection, the gathered attention with its split merge; for the
prefill chunk also the memory-flat step (the append launch, then the
memory-flat score + select, whose workspace needs no initialisation either:
its threshold launch clears each row's candidate counter).
"""
import math
import sys

import numpy as np
import pytest
import torch

import datagen

pytestmark = pytest.mark.gpu

from gpu_harness import DEV, Layer, to_dev  # noqa: E402


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def Q():
    import long_context_sparse_qsa_amd as Q
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    Q.qsa_device_check()
    return Q


class Step:
    """Buffers and enqueue function of one layer step; ``flat``: the append
    launch, then the memory-flat score + select entry point."""

    def __init__(self, Q, d, layer, flat=False):
        wl = d["workload"]
        self.Q, self.layer, self.wl, self.flat = Q, layer, wl, flat
        n = d["idx"].shape[0]
        self.new = to_dev(d["idx"][n - 4:], wl.dtype).contiguous()
        self.pos = torch.arange(n - 4, n, dtype=torch.int64, device=DEV)
        m, k = layer.m, wl.k_blocks
        self.k = k
        self.scores = torch.empty((m, layer.ld), dtype=torch.float32, device=DEV)
        self.sel = torch.empty((m, k), dtype=torch.int32, device=DEV)
        self.n_sel = torch.empty((m,), dtype=torch.int32, device=DEV)
        self.out = torch.empty_like(layer.q)
        self.lse = torch.empty((m, wl.hq), dtype=torch.float32, device=DEV)
        wsb = Q.qsa_select_workspace_bytes(m, layer.nb_max, k)
        # the selection workspace starts as garbage and is never cleared again
        self.ws_sel = torch.randint(0, 255, (max(wsb, 1),), dtype=torch.uint8, device=DEV)
        wsf = Q.qsa_score_select_workspace_bytes(m, layer.nb_max, k) if flat else 1
        self.ws_flat = torch.randint(0, 255, (max(wsf, 1),), dtype=torch.uint8, device=DEV)
        wsa = Q.qsa_attn_workspace_bytes(m, wl.hq, wl.head_dim, k)
        self.ws_attn = torch.empty(max(wsa, 1), dtype=torch.uint8, device=DEV)

    def clobber(self):
        """Eager writes over every output (not over the workspaces)."""
        self.scores.fill_(-1.0)
        self.sel.fill_(-9)
        self.n_sel.fill_(-9)
        self.out.fill_(3.0)
        self.lse.fill_(7.0)

    def enqueue(self):
        Q, ly = self.Q, self.layer
        if self.flat:
            Q.qsa_append_pool(self.new, self.pos, ly.idx_cache, ly.pooled)
            Q.qsa_score_select(ly.idx_q, ly.rows, ly.pooled, ly.nb_max, self.k, self.sel, self.n_sel, self.ws_flat)
        else:
            Q.qsa_append_score(self.new, self.pos, ly.idx_cache, ly.pooled, ly.idx_q, ly.rows, self.scores,
                               ly.nb_max, sel_workspace=self.ws_sel)
            Q.qsa_select_topk(self.scores, ly.rows, ly.nb_max, self.k, self.sel, self.n_sel, self.ws_sel,
                              prepared=True)
        Q.qsa_gathered_attn(ly.q, ly.rows, ly.kv, self.sel, self.n_sel, self.out, self.lse, self.wl.hkv,
                            scale=1.0 / math.sqrt(self.wl.head_dim), workspace=self.ws_attn)

    def snapshot(self):
        torch.cuda.synchronize()
        return [t.clone() for t in (self.scores, self.sel, self.n_sel, self.out, self.lse, self.layer.idx_cache,
                                    self.layer.pooled)]


def same(a, b):
    # bitwise, NaN-safe: compare the raw bytes
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


@pytest.mark.parametrize("name,flat", [("verify_262k", False), ("decode_32k", False), ("prefill", False),
                                       ("prefill", True)])
def test_graph_replays_equal_eager(Q, name, flat):
    say("graph replay vs eager,", name, "memory-flat selection" if flat else "")
    d = datagen.gen_layer(name)
    n = d["idx"].shape[0]
    layer = Layer(d, prefix_split=n - 4)
    st = Step(Q, d, layer, flat=flat)
    st.clobber()
    st.enqueue()
    ref = st.snapshot()
    assert int(st.n_sel.min()) >= 0
    # capture on a side stream after a warm-up there (torch's capture protocol)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.clobber()
        st.enqueue()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.enqueue()
    names = ("scores", "sel", "n_sel", "out", "lse", "idx_cache", "pooled")
    for r in range(4):
        st.clobber()
        g.replay()
        got = st.snapshot()
        for nm, a, b in zip(names, got, ref):
            assert same(a, b), f"replay {r}: {nm} differs from the eager step"
        # eager work between replays: a whole eager step, checked as well
        st.clobber()
        st.enqueue()
        got = st.snapshot()
        for nm, a, b in zip(names, got, ref):
            assert same(a, b), f"eager step after replay {r}: {nm} differs"
    say(f"4 replays and 4 eager steps identical ({layer.m} rows)")
