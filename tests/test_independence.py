"""The oracle and the product path share no code and never import each other."""

import ast
import os

from tests.conftest import ROOT


def _imports(path):
    names = set()
    for dirpath, _, files in os.walk(path):
        for f in files:
            if f.endswith(".py"):
                tree = ast.parse(open(os.path.join(dirpath, f)).read())
                for node in ast.walk(tree):
                    if isinstance(node, ast.Import):
                        names |= {a.name.split(".")[0] for a in node.names}
                    elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
                        names.add(node.module.split(".")[0])
    return names


def test_oracle_imports_no_product_code():
    bad = _imports(os.path.join(ROOT, "oracle")) & {"paged_kv_cache_136_amd", "workloads", "bench"}
    assert not bad, bad


def test_product_never_imports_oracle():
    pkg = os.path.join(ROOT, "paged_kv_cache_136_amd")
    if os.path.isdir(pkg):
        assert "oracle" not in _imports(pkg)
        for dirpath, _, files in os.walk(pkg):
            for f in files:
                if f.endswith((".cpp", ".hip", ".h", ".hpp")):
                    assert "oracle" not in open(os.path.join(dirpath, f)).read().lower()


def test_workloads_holds_no_method_code():
    src = open(os.path.join(ROOT, "workloads.py")).read()
    for word in ("import oracle", "from oracle", "paged_kv_cache_136_amd", "softmax"):
        assert word not in src, word
