"""bench.py and __graft_entry__.py run only on a GPU machine; a name that no
scope binds (a module used in a function that never imports it) would only
show there, at the end of a long run.  This walks their functions and checks
every name they read is bound in the function, an enclosing function, the
module, or builtins."""
import ast
import builtins
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bound(node) -> set:
    """Names a function body binds (assignments, imports, nested defs, arguments,
    comprehension and except targets, with/for targets)."""
    out = set()
    for n in ast.walk(node):
        if isinstance(n, ast.Name) and isinstance(n.ctx, (ast.Store, ast.Del)):
            out.add(n.id)
        elif isinstance(n, (ast.Import, ast.ImportFrom)):
            out.update((a.asname or a.name).split(".")[0] for a in n.names)
        elif isinstance(n, (ast.FunctionDef, ast.AsyncFunctionDef, ast.ClassDef)):
            out.add(n.name)
        elif isinstance(n, ast.arg):
            out.add(n.arg)
        elif isinstance(n, ast.ExceptHandler) and n.name:
            out.add(n.name)
    return out


@pytest.mark.parametrize("path", ["bench.py", "__graft_entry__.py"])
def test_every_name_is_bound(path):
    tree = ast.parse(open(os.path.join(ROOT, path)).read())
    module = set()
    for n in tree.body:
        if isinstance(n, (ast.FunctionDef, ast.ClassDef)):
            module.add(n.name)
        elif isinstance(n, (ast.Import, ast.ImportFrom)):
            module.update((a.asname or a.name).split(".")[0] for a in n.names)
        elif isinstance(n, (ast.Assign, ast.AnnAssign)):
            targets = n.targets if isinstance(n, ast.Assign) else [n.target]
            for t in targets:
                module.update(x.id for x in ast.walk(t) if isinstance(x, ast.Name))
        elif isinstance(n, (ast.If, ast.Try)):
            module |= _bound(n)
    missing = []
    for f in [n for n in tree.body if isinstance(n, ast.FunctionDef)]:
        scope = _bound(f)
        for n in ast.walk(f):
            if isinstance(n, ast.Name) and isinstance(n.ctx, ast.Load):
                if n.id not in scope and n.id not in module and not hasattr(builtins, n.id):
                    missing.append(f"{f.name}: {n.id} (line {n.lineno})")
    assert not missing, missing
