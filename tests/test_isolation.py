"""The product path and the CPU oracle stay apart, and the library has no
fallback.

* Nothing in the package (Python binding, HIP sources, C headers) names the
  oracle.
* bench.py imports the oracle only inside its CPU-baseline leg.
* With the shared library missing, the first call into the binding raises
  instead of computing anything another way.
* bench.py measures one GPU: asked for several, it exits with a message
  before touching a device.
"""
import ast
import os
import subprocess
import sys

import pytest

import gemv_nvfp4_int8_amd as qp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "gemv_nvfp4_int8_amd")


def _product_sources():
    for base in (PKG, os.path.join(ROOT, "include")):
        for dirpath, _, files in os.walk(base):
            if "__pycache__" in dirpath:
                continue
            for f in files:
                if f.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                    yield os.path.join(dirpath, f)


def test_product_sources_never_name_the_oracle():
    srcs = list(_product_sources())
    assert any(s.endswith(".hip") for s in srcs) and any(s.endswith(".py") for s in srcs)
    for path in srcs:
        text = open(path, encoding="utf-8").read().lower()
        assert "oracle" not in text, f"{os.path.relpath(path, ROOT)} names the oracle"


def _oracle_imports(tree):
    """(import node, enclosing function names) for every import of oracle."""
    found = []

    def walk(node, stack):
        for child in ast.iter_child_nodes(node):
            inner = stack + [child.name] if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)) else stack
            if isinstance(child, ast.Import) and any(a.name.split(".")[0] == "oracle" for a in child.names):
                found.append((child, stack))
            elif isinstance(child, ast.ImportFrom) and (child.module or "").split(".")[0] == "oracle":
                found.append((child, stack))
            walk(child, inner)

    walk(tree, [])
    return found


def test_bench_imports_the_oracle_only_in_its_cpu_baseline():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py"), encoding="utf-8").read())
    imports = _oracle_imports(tree)
    assert imports, "bench.py should time the oracle in its CPU-baseline leg"
    for node, stack in imports:
        assert "cpu_baseline" in stack, f"bench.py line {node.lineno} imports the oracle outside cpu_baseline"


def test_missing_library_raises_on_first_call(monkeypatch):
    monkeypatch.setattr(qp, "_lib", None)
    monkeypatch.setattr(qp, "LIB_PATH", os.path.join(ROOT, "no-such-dir", "libqproj.so"))
    with pytest.raises(ImportError, match="no fallback"):
        qp.abi_version()


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
