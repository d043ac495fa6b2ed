"""The product path and the oracle stay apart (CPU only).

The HIP library and its binding never import, link, load or name the
oracle; the oracle never touches the library; bench.py imports the oracle
only inside its CPU-baseline functions and __graft_entry__ only in build()
(compiling the checker) and smoke() (checking against it).
"""
import ast
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "combine_ep_route_amd")


def _files(top, exts):
    for d, _, fs in os.walk(top):
        if "__pycache__" in d:
            continue
        for f in fs:
            if f.endswith(exts):
                yield os.path.join(d, f)


def test_package_never_names_the_oracle():
    for path in _files(PKG, (".py", ".hip", ".h", ".cpp", ".c")):
        text = open(path).read()
        assert not re.search(r"\boracle\b|ep_oracle|orc_", text), path


def test_oracle_never_touches_the_library():
    for path in _files(os.path.join(ROOT, "oracle"), (".py", ".c", ".h")):
        text = open(path).read()
        assert "combine_ep_route_amd" not in text and "libep.so" not in text, path


def _functions_importing_oracle(path):
    tree = ast.parse(open(path).read())
    found = []

    def visit(node, func):
        for child in ast.iter_child_nodes(node):
            f = child.name if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)) else func
            if isinstance(child, ast.Import) and any(a.name.split(".")[0] == "oracle" for a in child.names):
                found.append(func)
            if isinstance(child, ast.ImportFrom) and (child.module or "").split(".")[0] == "oracle":
                found.append(func)
            visit(child, f)

    visit(tree, None)
    return found


def test_bench_imports_the_oracle_only_for_the_cpu_baseline():
    funcs = _functions_importing_oracle(os.path.join(ROOT, "bench.py"))
    assert funcs and set(funcs) <= {"cpu_baseline", "ll_cpu_baseline"}, funcs


def test_graft_entry_imports_the_oracle_only_in_build_and_smoke():
    funcs = _functions_importing_oracle(os.path.join(ROOT, "__graft_entry__.py"))
    assert funcs and set(funcs) <= {"build", "smoke"}, funcs


def test_input_generator_imports_neither_side():
    """ep_inputs.py, shared by both sides, draws inputs only."""
    tree = ast.parse(open(os.path.join(ROOT, "ep_inputs.py")).read())
    mods = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            mods |= {a.name.split(".")[0] for a in node.names}
        elif isinstance(node, ast.ImportFrom):
            mods.add((node.module or "").split(".")[0])
    assert not mods & {"oracle", "combine_ep_route_amd"}, mods
