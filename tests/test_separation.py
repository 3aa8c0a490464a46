"""The oracle and the GPU path share no code (checked on the sources).

* Nothing in the package (Python binding, HIP sources, headers) imports,
  includes or names the oracle module; the seeded input generators
  (inputs.py) are the one module both sides use, and they import nothing
  from the package or the oracle.
* The oracle imports nothing from the package.
* bench.py imports the oracle only inside its CPU-baseline functions.
"""
import ast
import glob
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "structured_attention_video_monarch_amd")


def _imports(path):
    """(module name, enclosing function or None) of every import in a file."""
    tree = ast.parse(open(path).read(), path)
    out = []

    def visit(node, func):
        for child in ast.iter_child_nodes(node):
            f = child.name if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)) else func
            if isinstance(child, ast.Import):
                out.extend((a.name, func) for a in child.names)
            elif isinstance(child, ast.ImportFrom):
                out.append(("." * child.level + (child.module or ""), func))
            visit(child, f)

    visit(tree, None)
    return out


def test_package_never_touches_the_oracle():
    py = glob.glob(os.path.join(PKG, "**", "*.py"), recursive=True)
    assert py
    for path in py:
        for mod, _ in _imports(path):
            assert not mod.split(".")[0] == "oracle", (path, mod)
    native = glob.glob(os.path.join(PKG, "csrc", "*")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    assert native
    for path in native:
        txt = open(path, errors="replace").read()
        assert not re.search(r'#\s*include\s*[<"][^>"]*oracle', txt), path
        assert "monarch_oracle" not in txt and "monarch_grad" not in txt, path


def test_inputs_module_imports_neither_side():
    for mod, _ in _imports(os.path.join(PKG, "inputs.py")):
        top = mod.split(".")[0]
        assert top not in ("oracle", "structured_attention_video_monarch_amd") and not mod.startswith("."), mod


def test_oracle_imports_nothing_from_the_package():
    for path in glob.glob(os.path.join(ROOT, "oracle", "*.py")):
        for mod, _ in _imports(path):
            assert not mod.startswith("structured_attention_video_monarch_amd"), (path, mod)
            assert mod.split(".")[0] in ("", "__future__", "math", "numpy") or mod.startswith("."), (path, mod)


def test_bench_uses_the_oracle_only_for_the_cpu_baseline():
    uses = [(m, f) for m, f in _imports(os.path.join(ROOT, "bench.py")) if m.split(".")[0] == "oracle"]
    assert uses
    assert all(f is not None and f.startswith("cpu_baseline") for _, f in uses), uses


def test_entry_point_uses_the_oracle_only_in_smoke():
    uses = [(m, f) for m, f in _imports(os.path.join(ROOT, "__graft_entry__.py")) if m.split(".")[0] == "oracle"]
    assert uses
    assert all(f == "smoke" for _, f in uses), uses
