"""Every name a function of the committed Python files reads is defined: a
free name inside a function must be a module-level binding or a builtin.
(The functions of bench.py that time the GPU only run on a GPU; this finds a
misspelt or stale name in them on the CPU.)"""
import builtins
import os
import symtable

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FILES = sorted(
    os.path.relpath(os.path.join(d, f), ROOT)
    for top in ("", "learned_kv_cache_head_amd", "oracle", "tests",
                "tests/golden")
    for d in [os.path.join(ROOT, top)]
    for f in (os.listdir(d) if os.path.isdir(d) else [])
    if f.endswith(".py"))


def _undefined(path):
    src = open(path).read()
    top = symtable.symtable(src, path, "exec")
    known = {s.get_name() for s in top.get_symbols()
             if s.is_assigned() or s.is_imported()}
    known |= set(dir(builtins)) | {"__file__", "__name__", "__doc__"}
    bad = []

    def walk(t):
        for c in t.get_children():
            if c.get_type() == "function":
                for s in c.get_symbols():
                    if (s.is_global() and s.is_referenced()
                            and s.get_name() not in known):
                        bad.append(f"{c.get_name()}: {s.get_name()}")
            walk(c)

    walk(top)
    return bad


@pytest.mark.parametrize("rel", FILES)
def test_no_undefined_names(rel):
    path = os.path.join(ROOT, rel)
    if not os.path.exists(path):
        pytest.skip(f"{rel} absent")
    assert _undefined(path) == []


def test_checker_finds_a_stale_name(tmp_path):
    p = tmp_path / "m.py"
    p.write_text("x = 1\ndef f():\n    y = 2\n    return x + y + z\n")
    assert _undefined(str(p)) == ["f: z"]
