"""The product path has no fallback: the binding fails loudly without the HIP
library, and no module of the package imports the oracle (CPU only)."""
import ast
import os

import pytest

from sparse_mla_decode_smla_amd import binding as B

PKG = os.path.dirname(os.path.abspath(B.__file__))


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        B.load(os.path.join(PKG, "no_such_library.so"))


def test_package_never_imports_the_oracle():
    for name in sorted(os.listdir(PKG)):
        if not name.endswith(".py"):
            continue
        tree = ast.parse(open(os.path.join(PKG, name), encoding="utf-8").read(), filename=name)
        for node in ast.walk(tree):
            if isinstance(node, ast.Import):
                mods = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                mods = [node.module or ""]
            else:
                continue
            assert not any(m == "oracle" or m.startswith("oracle.") for m in mods), f"{name} imports the oracle"
