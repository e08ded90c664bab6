"""The product path never reaches the oracle: no file of the package or the
C sources imports, links or names it, and the binding refuses to run without
the compiled library (no CPU fallback)."""

import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "io_aware_exact_24_amd")


def product_files():
    for dirpath, _, names in os.walk(PKG):
        for n in names:
            if n.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                yield os.path.join(dirpath, n)


def test_package_does_not_import_oracle():
    pat = re.compile(r"^\s*(from\s+oracle|import\s+oracle)|oracle[./]", re.M)
    for path in product_files():
        text = open(path).read()
        assert not pat.search(text), path


def test_oracle_does_not_import_package():
    for n in os.listdir(os.path.join(ROOT, "oracle")):
        if n.endswith(".py"):
            text = open(os.path.join(ROOT, "oracle", n)).read()
            assert "io_aware_exact_24_amd" not in text, n


def test_binding_raises_without_library(tmp_path, monkeypatch):
    from io_aware_exact_24_amd import binding

    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "PKG", str(tmp_path))
    try:
        binding.load_library()
    except OSError as e:
        assert "missing" in str(e)
    else:
        raise AssertionError("load_library must fail when libfa.so is absent")
