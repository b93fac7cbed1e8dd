"""Host logic of bench.py that needs no GPU: the kernel-source fingerprint
that decides whether a committed counter summary still describes the code
(it must ignore comments and blank lines, and nothing else), and that every
committed counter summary still matches the source it was taken on."""

import importlib.util
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _sha_of(bench, tmp_path, text):
    p = tmp_path / "k.hip"
    p.write_text(text)
    return bench.source_sha(str(p))


def test_fingerprint_ignores_comments_only(bench, tmp_path):
    base = "int f(int a) {\n  return a + 1;  // one more\n}\n"
    same = [
        "// header\nint f(int a) {\n  return a + 1;\n}\n",
        "/* block\n   comment */\nint f(int a) {\n\n  return a + 1;  // another note\n}\n",
        base.replace("\n}", "\n\n\n}"),
    ]
    different = [
        base.replace("a + 1", "a + 2"),
        base.replace("return", "return -"),
        "int f(int a) {\n  return a+1;\n}\n",          # whitespace inside a line is code
    ]
    ref = _sha_of(bench, tmp_path, base)
    for t in same:
        assert _sha_of(bench, tmp_path, t) == ref, t
    for t in different:
        assert _sha_of(bench, tmp_path, t) != ref, t


def test_committed_counter_summaries_match_the_sources(bench):
    """Every profiles/*_pmc.json names its source file and a fingerprint
    that the current code has, so the bench lines report its traffic."""
    names = [f[:-len("_pmc.json")] for f in os.listdir(os.path.join(ROOT, "profiles"))
             if f.endswith("_pmc.json")]
    assert names
    for n in names:
        with open(os.path.join(ROOT, "profiles", n + "_pmc.json")) as f:
            pmc = json.load(f)
        assert bench.load_traffic(n) == pmc["traffic_bytes_per_launch"], n
