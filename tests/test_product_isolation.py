"""The product path never touches the oracle, and the oracle never touches
the product (CPU only)."""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "combine_moe_route_topk_amd")


def _sources(folder, exts):
    for dirpath, _, files in os.walk(folder):
        for f in files:
            if f.endswith(exts):
                yield os.path.join(dirpath, f)


def test_package_sources_do_not_mention_the_oracle():
    for path in _sources(PKG, (".py", ".hip", ".cpp", ".hpp", ".h")):
        text = open(path).read()
        assert not re.search(r"\boracle\b", text), path


def test_oracle_does_not_import_the_package_or_workloads():
    for path in _sources(os.path.join(ROOT, "oracle"), (".py",)):
        text = open(path).read()
        assert "combine_moe_route_topk_amd" not in text, path
        assert not re.search(r"^\s*(from|import)\s+workloads", text, re.M), path


def test_importing_the_package_loads_no_oracle_module():
    code = ("import sys, combine_moe_route_topk_amd; "
            "print(any(m == 'oracle' or m.startswith('oracle.') for m in sys.modules))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         timeout=120)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "False"


def test_generators_hold_no_method_arithmetic():
    text = open(os.path.join(ROOT, "workloads", "gen.py")).read()
    for call in ("argsort(", "bincount(", "cumsum(", "topk(", "softmax(", "searchsorted("):
        assert call not in text, call
