"""Static checks of the top-level scripts that need a GPU to run (bench.py,
__graft_entry__.py): every name a function reads must be defined somewhere -
a local, a parameter, a module-level definition or import, or a builtin. A
name lost in an edit would otherwise surface only on the GPU."""
import builtins
import os
import symtable

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MODULE_DUNDERS = {"__file__", "__name__", "__doc__", "__spec__", "__package__"}
SCRIPTS = ["bench.py", "__graft_entry__.py"] + [
    os.path.join("structure_aware_grouped_amd", f) for f in ("binding.py", "build.py", "__init__.py")]


def _undefined(path):
    src = open(os.path.join(ROOT, path)).read()
    top = symtable.symtable(src, path, "exec")
    module_names = {s.get_name() for s in top.get_symbols() if s.is_assigned() or s.is_imported()}
    missing = []

    def walk(t):
        for s in t.get_symbols():
            if not s.is_referenced():
                continue
            if s.is_local() or s.is_parameter() or s.is_free() or s.is_imported() or s.is_assigned():
                continue
            n = s.get_name()
            if n in module_names or hasattr(builtins, n) or n in MODULE_DUNDERS:
                continue
            missing.append(f"{t.get_name()}:{n}")
        for c in t.get_children():
            walk(c)

    walk(top)
    return missing


@pytest.mark.parametrize("path", SCRIPTS)
def test_every_name_read_is_defined(path):
    assert _undefined(path) == []


def test_the_check_catches_a_missing_name(tmp_path):
    """A planted mistake: a function that calls an undefined class."""
    p = tmp_path / "s.py"
    p.write_text("import os\n\ndef f():\n    return Missing(os.sep)\n")
    rel = os.path.relpath(p, ROOT)
    assert _undefined(rel) == ["f:Missing"]


def test_bench_and_product_do_not_import_the_test_tree():
    """bench.py, the package and the input generators take nothing from tests/."""
    import re
    paths = ["bench.py", "__graft_entry__.py"]
    for d in ("structure_aware_grouped_amd", "workloads"):
        paths += [os.path.join(d, f) for f in os.listdir(os.path.join(ROOT, d)) if f.endswith(".py")]
    for p in paths:
        src = open(os.path.join(ROOT, p)).read()
        assert not re.search(r"^\s*(from|import)\s+tests\b", src, re.M), p
