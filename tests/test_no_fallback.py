"""The product path has no fallback: without the HIP library every call
raises, and no module of the package imports the oracle (CPU checks)."""
import ast
import os

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "mla_latent_cache_amd")


def test_missing_library_raises(monkeypatch):
    from mla_latent_cache_amd import _lib, ops
    monkeypatch.setattr(_lib, "LIB_PATH", os.path.join(PKG, "no_such_library.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load()
    with pytest.raises(RuntimeError, match="not built"):
        _lib.call("mla_absorb_q", None, None, 0, None, 0, 1, 1, 4, 8, None)


def test_host_tensors_are_refused():
    """No CPU path: a host tensor is an error, not a slower route."""
    from mla_latent_cache_amd import ops
    with pytest.raises(ValueError, match="GPU"):
        ops.absorb_q(torch.zeros((1, 2, 4)), torch.zeros((2, 4, 8)))


def test_package_never_imports_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if not f.endswith(".py"):
                continue
            path = os.path.join(dirpath, f)
            tree = ast.parse(open(path).read(), path)
            for node in ast.walk(tree):
                names = []
                if isinstance(node, ast.Import):
                    names = [a.name for a in node.names]
                elif isinstance(node, ast.ImportFrom):
                    names = [node.module or ""]
                for n in names:
                    assert not n.split(".")[0] == "oracle", f"{path} imports {n}"
