"""The product path is the HIP library alone.

The package (Python binding and HIP sources) never names the CPU oracle, which
is test infrastructure, and the binding refuses to import when the built
library is missing instead of falling back to any CPU computation.
"""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "long_context_sparse_qsa_amd")


def _sources():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                yield os.path.join(dirpath, f)


def test_package_never_names_the_oracle():
    pat = re.compile(r"\boracle\b|qsa_oracle|import\s+datagen|\bdatagen\b")
    hits = []
    for p in _sources():
        for i, line in enumerate(open(p, encoding="utf-8"), 1):
            if pat.search(line):
                hits.append(f"{os.path.relpath(p, ROOT)}:{i}: {line.strip()}")
    assert not hits, "\n".join(hits)


def test_bench_reaches_the_oracle_only_in_its_cpu_baseline():
    src = open(os.path.join(ROOT, "bench.py"), encoding="utf-8").read()
    # every line naming the oracle sits inside the cpu_baseline function
    body = re.search(r"\ndef cpu_baseline\b.*?(?=\ndef |\Z)", src, re.S)
    assert body, "bench.py has no cpu_baseline function"
    outside = src.replace(body.group(0), "")
    assert not re.search(r"^\s*(import|from)\s+oracle\b|\boracle\.", outside, re.M)


def test_import_fails_loudly_without_the_library(tmp_path):
    # a copy of the binding with no libqsa.so beside it must not import
    dst = tmp_path / "long_context_sparse_qsa_amd"
    dst.mkdir()
    for f in os.listdir(PKG):
        if f.endswith(".py"):
            (dst / f).write_bytes(open(os.path.join(PKG, f), "rb").read())
    r = subprocess.run([sys.executable, "-c", "import long_context_sparse_qsa_amd"], cwd=str(tmp_path),
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "libqsa.so" in r.stderr, r.stderr[-2000:]
