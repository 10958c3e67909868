"""bench.py runs only where there is a GPU; these CPU checks cover what can be
checked without one: every name its functions read is bound somewhere, every
workload it offers has step defaults and a builder, and --gpus other than 1
exits with a message before touching a device."""
from __future__ import annotations

import ast
import builtins
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _module_names(tree: ast.Module) -> set:
    names = set(dir(builtins))
    for node in ast.walk(tree):
        if isinstance(node, (ast.Import, ast.ImportFrom)):
            for a in node.names:
                names.add((a.asname or a.name).split(".")[0])
    for node in tree.body:
        if isinstance(node, (ast.FunctionDef, ast.ClassDef)):
            names.add(node.name)
        elif isinstance(node, (ast.Assign, ast.AnnAssign)):
            for t in (node.targets if isinstance(node, ast.Assign) else [node.target]):
                names.update(n.id for n in ast.walk(t) if isinstance(n, ast.Name))
    return names


def _unbound_reads(fn: ast.FunctionDef, module_names: set) -> list:
    """Names read in fn (nested functions included) that nothing binds."""
    bound = set()
    for n in ast.walk(fn):
        if isinstance(n, ast.Name) and isinstance(n.ctx, (ast.Store, ast.Del)):
            bound.add(n.id)
        elif isinstance(n, ast.FunctionDef):
            bound.add(n.name)
        elif isinstance(n, ast.arg):
            bound.add(n.arg)
        elif isinstance(n, ast.ExceptHandler) and n.name:
            bound.add(n.name)
    return sorted({(n.id, n.lineno) for n in ast.walk(fn)
                   if isinstance(n, ast.Name) and isinstance(n.ctx, ast.Load)
                   and n.id not in bound and n.id not in module_names})


def test_bench_functions_read_only_bound_names():
    tree = ast.parse(open(BENCH).read())
    names = _module_names(tree)
    bad = []
    for node in tree.body:
        if isinstance(node, ast.FunctionDef):
            bad += [(node.name, n, line) for n, line in _unbound_reads(node, names)]
    assert not bad, f"unbound names in bench.py: {bad}"


def test_every_workload_has_defaults_and_a_builder():
    src = open(BENCH).read()
    tree = ast.parse(src)
    consts = {}
    for node in tree.body:
        if isinstance(node, ast.Assign) and isinstance(node.targets[0], ast.Name):
            try:
                consts[node.targets[0].id] = ast.literal_eval(node.value)
            except ValueError:
                pass
    workloads, defaults = consts["WORKLOADS"], consts["DEFAULT_STEPS"]
    assert set(workloads) == set(defaults)
    build = next(n for n in tree.body if isinstance(n, ast.FunctionDef) and n.name == "build_workload")
    text = ast.get_source_segment(src, build)
    for wl in workloads:
        assert f'"{wl}"' in text or wl == "scissor_decode", wl  # scissor_decode is the fall-through


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=300,
                       cwd=ROOT, env={**os.environ, "HIP_VISIBLE_DEVICES": ""})
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""
