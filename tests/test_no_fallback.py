"""The product path has no CPU fallback and never reaches the oracle (CPU checks).

* a missing library raises instead of degrading to another implementation;
* CPU tensors are rejected by every entry point before anything runs;
* no module of the package, nor bench.py's timed paths, imports the oracle: only the
  tests, ``__graft_entry__.smoke()`` and bench.py's CPU-baseline functions may.
"""

from __future__ import annotations

import ast
import glob
import os

import pytest
import torch

from exact_attention_89_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_missing_library_raises(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        api.load_library(str(tmp_path / "libattn89.so"))


@pytest.mark.parametrize("fn", ["attn_fwd", "attn_fwd_f32", "attn_materialized", "attn_partial",
                                "attn_fwd_splitkv"])
def test_cpu_tensors_rejected(fn):
    dtype = torch.float32 if fn == "attn_fwd_f32" else torch.bfloat16
    q = torch.zeros(1, 1, 8, 64, dtype=dtype)
    with pytest.raises(ValueError, match="GPU tensor"):
        getattr(api, fn)(q, q, q)


def test_fp8_and_varlen_reject_cpu_tensors():
    q8 = torch.zeros(1, 1, 8, 64, dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU tensor"):
        api.attn_fwd_fp8(q8, q8, q8, 1.0, 1.0, 1.0)
    qb = torch.zeros(8, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        api.attn_fwd_varlen(qb, qb, qb, [0, 8], [0, 8])


def _imports(path):
    tree = ast.parse(open(path).read())
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names |= {a.name.split(".")[0] for a in node.names}
        elif isinstance(node, ast.ImportFrom) and node.module:
            names.add(node.module.split(".")[0])
    return names


def test_package_never_imports_the_oracle():
    files = glob.glob(os.path.join(ROOT, "exact_attention_89_amd", "**", "*.py"), recursive=True)
    assert files
    for f in files:
        assert "oracle" not in _imports(f), f"{f} imports the oracle"


def test_bench_imports_the_oracle_only_in_cpu_baselines():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    # the oracle leg: the timed CPU baselines and the reference rows of the parity check
    allowed = {"cpu_baseline_attention", "_cpu_oracle_chunk", "oracle_reference_rows",
               "softmax_cpu_baseline", "bench_decode", "bench_fp8"}
    for fn in [n for n in tree.body if isinstance(n, ast.FunctionDef)]:
        imports_oracle = any(isinstance(n, ast.Import) and any(a.name == "oracle" for a in n.names)
                             for n in ast.walk(fn))
        if imports_oracle:
            assert fn.name in allowed, f"bench.py: {fn.name} imports the oracle"
    top = [n for n in tree.body if isinstance(n, (ast.Import, ast.ImportFrom))]
    assert all("oracle" not in _imports_node(n) for n in top)


def _imports_node(node):
    if isinstance(node, ast.Import):
        return {a.name.split(".")[0] for a in node.names}
    return {node.module.split(".")[0]} if node.module else set()
