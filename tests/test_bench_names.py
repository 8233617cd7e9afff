"""bench.py and __graft_entry__.py only run whole on a GPU; this CPU test reads
their symbol tables and fails on any name a function uses that is bound
neither in it, in an enclosing function, at module level nor in builtins (the
kind of slip that otherwise surfaces as a NameError on the GPU)."""
import builtins
import os
import symtable

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def unbound_globals(path):
    src = open(path).read()
    top = symtable.symtable(src, path, "exec")
    module_names = {s.get_name() for s in top.get_symbols() if s.is_assigned() or s.is_imported()}
    known = module_names | set(dir(builtins)) | {"__file__", "__name__"}
    bad = []

    def walk(table):
        for child in table.get_children():
            for s in child.get_symbols():
                if s.is_global() and s.is_referenced() and s.get_name() not in known:
                    bad.append("%s: %s" % (child.get_name(), s.get_name()))
            walk(child)

    walk(top)
    return bad


@pytest.mark.parametrize("name", ["bench.py", "__graft_entry__.py"])
def test_no_unbound_names(name):
    assert unbound_globals(os.path.join(ROOT, name)) == []


def test_the_check_sees_an_unbound_name(tmp_path):
    p = tmp_path / "m.py"
    p.write_text("import os\nX = 1\ndef f(a):\n    b = a + X\n    return os.sep, b, Nk\n")
    assert unbound_globals(str(p)) == ["f: Nk"]
