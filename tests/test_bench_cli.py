"""bench.py checks that need no GPU: it refuses more than one GPU with a
message, and none of its functions reads a name that is never bound (a
misspelled or stale variable in a rarely used mode would otherwise surface
only as a NameError on the GPU)."""
import ast
import builtins
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _module_names(tree):
    names = set(dir(builtins))
    for n in tree.body:
        if isinstance(n, (ast.FunctionDef, ast.ClassDef)):
            names.add(n.name)
        elif isinstance(n, (ast.Import, ast.ImportFrom)):
            names.update((a.asname or a.name).split(".")[0] for a in n.names)
        elif isinstance(n, (ast.Assign, ast.AnnAssign)):
            targets = n.targets if isinstance(n, ast.Assign) else [n.target]
            for t in targets:
                names.update(x.id for x in ast.walk(t) if isinstance(x, ast.Name))
    return names


def _bound_in(fn):
    """Every name a top-level function binds anywhere inside it (its own and
    its nested functions' arguments, assignments, imports, loop targets)."""
    bound = set()
    for x in ast.walk(fn):
        if isinstance(x, ast.Name) and isinstance(x.ctx, (ast.Store, ast.Del)):
            bound.add(x.id)
        elif isinstance(x, ast.arg):
            bound.add(x.arg)
        elif isinstance(x, ast.FunctionDef):
            bound.add(x.name)
        elif isinstance(x, (ast.Import, ast.ImportFrom)):
            bound.update((a.asname or a.name).split(".")[0] for a in x.names)
        elif isinstance(x, ast.ExceptHandler) and x.name:
            bound.add(x.name)
    return bound


def test_no_function_reads_an_unbound_name():
    tree = ast.parse(open(BENCH).read())
    module = _module_names(tree)
    missing = []
    for fn in tree.body:
        if not isinstance(fn, ast.FunctionDef):
            continue
        bound = _bound_in(fn) | module
        for x in ast.walk(fn):
            if isinstance(x, ast.Name) and isinstance(x.ctx, ast.Load) and x.id not in bound:
                missing.append((fn.name, x.lineno, x.id))
    assert not missing, missing
