"""Structural guards (CPU only): the oracle is test infrastructure, so the
library package and the seeded-input module never import it, and bench.py
runs it only in its CPU-baseline functions; bench.py measures one GPU and
refuses a larger count before touching any device."""
import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _imports_oracle(node):
    if isinstance(node, ast.Import):
        return any(a.name == "oracle" or a.name.startswith("oracle.") for a in node.names)
    if isinstance(node, ast.ImportFrom):
        return (node.module or "").split(".")[0] == "oracle"
    return False


def _py_files(*dirs):
    for d in dirs:
        for base, _, files in os.walk(os.path.join(ROOT, d)):
            for f in files:
                if f.endswith(".py"):
                    yield os.path.join(base, f)


def test_product_and_inputs_never_import_the_oracle():
    for path in _py_files("mla_latent_kv_32_amd", "synth"):
        tree = ast.parse(open(path).read(), path)
        bad = [n.lineno for n in ast.walk(tree) if _imports_oracle(n)]
        assert not bad, f"{os.path.relpath(path, ROOT)} imports the oracle at lines {bad}"


def test_bench_runs_the_oracle_only_in_its_cpu_leg():
    path = os.path.join(ROOT, "bench.py")
    tree = ast.parse(open(path).read(), path)
    allowed = set()
    for fn in ast.walk(tree):
        if isinstance(fn, ast.FunctionDef) and fn.name.startswith("cpu_baseline"):
            allowed |= {id(n) for n in ast.walk(fn)}
    bad = [n.lineno for n in ast.walk(tree) if _imports_oracle(n) and id(n) not in allowed]
    assert not bad, f"bench.py imports the oracle outside the cpu_baseline functions (lines {bad})"
    assert any(_imports_oracle(n) for n in ast.walk(tree)), "the CPU leg should time the oracle"


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
