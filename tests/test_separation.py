"""The oracle and the HIP path stay apart (CPU checks of the sources).

The oracle is test infrastructure: the package (the binding and its HIP
sources) never imports, includes or loads it, the oracle never reaches into
the package's kernels or headers, and outside the tests only the smoke check
and the CPU-baseline legs of bench.py call it.  Without its built library the
binding raises instead of computing anything on the host."""
import ast
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "long_context_blockwise_attn_amd")
ORACLE = os.path.join(ROOT, "oracle")
SOURCE_EXT = (".py", ".hip", ".hpp", ".cpp", ".h", ".c")


def sources(top):
    for dirpath, dirnames, files in os.walk(top):
        dirnames[:] = [d for d in dirnames if not d.startswith(("_build", "__pycache__"))]
        for f in files:
            if f.endswith(SOURCE_EXT):
                yield os.path.join(dirpath, f)


def test_package_never_reaches_the_oracle():
    bad = re.compile(r"^\s*(import\s+oracle|from\s+oracle\b|from\s+\.\.\s*import\s+oracle)|#\s*include\s*[<\"].*oracle"
                     r"|liboracle|oracle\.c\b", re.M)
    found = [p for p in sources(PKG) if bad.search(open(p, encoding="utf-8").read())]
    assert not found, "package sources that reach the oracle: %s" % found


def test_oracle_shares_nothing_with_the_hip_path():
    bad = re.compile(r"long_context_blockwise_attn_amd|libbwattn|#\s*include\s*[<\"](?!(math|stdint|stdlib|string|omp)\.h)"
                     r"|csrc|bwattn\.h")
    found = [p for p in sources(ORACLE) if bad.search(open(p, encoding="utf-8").read())]
    assert not found, "oracle sources that reach the HIP path: %s" % found


def oracle_imports(path):
    """(enclosing function names, enclosing if-tests) of each import of the oracle in `path`."""
    tree = ast.parse(open(path, encoding="utf-8").read())
    out = []

    def walk(node, funcs, tests):
        for child in ast.iter_child_nodes(node):
            f, t = funcs, tests
            if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)):
                f = funcs + [child.name]
            if isinstance(child, ast.If):
                t = tests + [ast.unparse(child.test)]
            names = []
            if isinstance(child, ast.Import):
                names = [a.name for a in child.names]
            elif isinstance(child, ast.ImportFrom):
                names = [child.module or ""]
            if any(n == "oracle" or n.startswith("oracle.") for n in names):
                out.append((f, t))
            walk(child, f, t)

    walk(tree, [], [])
    return out


def test_only_smoke_and_the_cpu_baseline_use_the_oracle():
    for f in os.listdir(ROOT):
        if f.endswith(".py") and f not in ("bench.py", "__graft_entry__.py"):
            assert not oracle_imports(os.path.join(ROOT, f)), f
    uses = oracle_imports(os.path.join(ROOT, "bench.py"))
    assert uses, "bench.py's CPU baseline times the oracle"
    for funcs, tests in uses:
        assert funcs, "bench.py imports the oracle at module level"
        assert "cpu_baseline" in funcs or any("no_cpu_baseline" in t for t in tests), (funcs, tests)
    for funcs, _ in oracle_imports(os.path.join(ROOT, "__graft_entry__.py")):
        assert funcs and funcs[0] in ("build", "smoke"), funcs


def test_binding_raises_without_its_library(tmp_path, monkeypatch):
    import long_context_blockwise_attn_amd as bw

    monkeypatch.setattr(bw, "library_path", str(tmp_path / "missing.so"))
    monkeypatch.setattr(bw, "_lib", None)
    with pytest.raises(bw.AttnError):
        bw.load()
