"""bench.py runs only on a GPU; this CPU check catches a call to a function
that no longer exists (every name called at module level or in a function
must be defined in the file, imported, local, or a builtin)."""

import ast
import builtins
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_calls_only_defined_names():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    known = set(dir(builtins))
    for n in ast.walk(tree):
        if isinstance(n, (ast.FunctionDef, ast.ClassDef)):
            known.add(n.name)
        elif isinstance(n, (ast.Import, ast.ImportFrom)):
            known.update((a.asname or a.name).split(".")[0] for a in n.names)
        elif isinstance(n, ast.Name) and isinstance(n.ctx, ast.Store):
            known.add(n.id)
        elif isinstance(n, ast.arg):
            known.add(n.arg)
    called = {n.func.id for n in ast.walk(tree) if isinstance(n, ast.Call) and isinstance(n.func, ast.Name)}
    assert not called - known, sorted(called - known)
