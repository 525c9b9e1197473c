"""CPU checks that the product path and the oracle stay apart: nothing in the
package (Python binding, harness, workloads, HIP and host sources) imports,
includes or names the oracle, the oracle does not use the package's
arithmetic, and the binding fails loudly when the HIP library is missing
instead of falling back to anything."""

import ast
import os
import re

import pytest

from decode_attention_gemma_amd import g4attn as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "decode_attention_gemma_amd")


def _package_files():
    for d, _, files in os.walk(PKG):
        if "_build" in d or "__pycache__" in d:
            continue
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                yield os.path.join(d, f)


def test_package_never_names_the_oracle():
    for path in _package_files():
        text = open(path).read()
        assert not re.search(r"\boracle\b|attn64", text), path


def test_oracle_imports_nothing_from_the_package():
    path = os.path.join(ROOT, "oracle", "attn64.py")
    tree = ast.parse(open(path).read())
    mods = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            mods.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom):
            mods.add((node.module or "").split(".")[0])
    assert mods <= {"__future__", "numpy"}, mods


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(G, "LIB_PATH", str(tmp_path / "libg4attn.so"))
    monkeypatch.setattr(G, "_lib", None)
    with pytest.raises(ImportError):
        G.load()
    with pytest.raises(ImportError):
        G.g4attn_stack_create([], 1, 64, 16)
