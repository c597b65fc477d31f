"""Host-side logic of bench.py (no GPU): the algorithmic byte counts its
roofline and path figures divide by, its replica rule, the stored-traffic
gate, and its refusal of more than one GPU.

The byte counts are pinned to the workload's own arithmetic (the verify step at
261,122 tokens: four rows at 261,118..261,121, k = 512 blocks of 4 tokens,
24 query heads over 2 KV heads of width 256, bf16), worked out by hand below,
so that a dropped term or a wrong factor in bench.py fails here.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import datagen  # noqa: E402

VERIFY = datagen.WORKLOADS["verify_262k"]


def test_kept_tokens_verify_rows():
    # each row keeps min(nb, 512) = 512 blocks of 4 tokens plus its tail:
    # positions 261,118..261,121 end after 261,119..261,122 tokens, tails 3, 0, 1, 2
    assert bench.kept_tokens(VERIFY.rows, VERIFY.k_blocks) == 4 * 512 * 4 + (3 + 0 + 1 + 2)
    # rows that keep every block: all their tokens
    assert bench.kept_tokens([0, 5, 2046], 512) == 1 + 6 + 2047


def test_append_bytes():
    # four bf16 keys read and written (4 x 128 x 2 B x 2); position 261,119 ends
    # a block whose first two keys (261,116 and 261,117) come from the cache
    # (2 x 256 B) and whose float32 pooled key is written (512 B)
    assert bench.append_alg_bytes(list(VERIFY.rows), 2) == 4 * 512 + 2 * 256 + 512
    # a whole block appended at once reads nothing back from the cache
    assert bench.append_alg_bytes([0, 1, 2, 3], 2) == 4 * 512 + 512
    # a key that completes no block: read and written only
    assert bench.append_alg_bytes([5], 4) == 128 * 4 * 2


def test_path_bytes_verify():
    nb_max = (max(VERIFY.rows) + 1) // 4
    assert nb_max == 65280
    pooled = 65280 * 512                       # float32 pooled keys, read once
    kv = 8198 * 2 * 2 * 256 * 2                # kept tokens x KV heads x (K, V) x 256 x bf16
    per_row = 2 * 24 * 256 * 2 + 4 * 128 * 2   # queries and outputs, index queries
    assert bench.path_bytes(VERIFY, VERIFY.rows, nb_max) == pooled + kv + 4 * per_row == 50_315_264


def test_replica_rule():
    # one sweep over the replicated layer states touches at least 1 GiB
    assert bench.replicas(50_000_000, 12) == 2
    assert bench.replicas((1 << 30) // 12 + 1, 12) == 1
    assert bench.replicas(1, 1) == 1 << 30
    assert bench.replicas(10, 12, forced=3) == 3


def test_stored_traffic_gated_by_source_hash(tmp_path, monkeypatch):
    f = tmp_path / "pmc.txt"
    f.write_text(f"source_hash: {bench.score_source_hash()}\nfetch_bytes_per_launch: 100\n"
                 "write_bytes_per_launch: 20.0\n")
    monkeypatch.setattr(bench, "PMC_FILE", str(f))
    assert bench.stored_traffic() == 120
    f.write_text("source_hash: 0000\nfetch_bytes_per_launch: 100\nwrite_bytes_per_launch: 20\n")
    assert bench.stored_traffic() is None  # counters taken on other sources are not reported


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_is_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
