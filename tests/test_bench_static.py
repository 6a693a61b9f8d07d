"""bench.py on the CPU: every global name its functions use is defined (a
renamed or deleted helper fails here rather than on the GPU), the cache flush
of the cold legs runs, and a request for more than one GPU exits with a
message before anything touches a device."""
import builtins
import os
import subprocess
import sys
import symtable

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def _globals_used(table):
    for sym in table.get_symbols():
        if sym.is_global() and sym.is_referenced():
            yield table.get_name(), sym.get_name()
    for child in table.get_children():
        yield from _globals_used(child)


def test_bench_global_names_resolve():
    src = open(BENCH).read()
    top = symtable.symtable(src, BENCH, "exec")
    defined = {s.get_name() for s in top.get_symbols() if s.is_assigned() or s.is_imported()}
    defined |= {"__file__", "__name__", "__doc__"}
    missing = sorted({(fn, name) for fn, name in _globals_used(top)
                      if name not in defined and not hasattr(builtins, name)})
    assert not missing, f"undefined globals in bench.py: {missing}"


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_bench_flush_runs():
    """The cache-flushing read the cold legs issue, on a small CPU buffer."""
    import importlib.util
    import torch
    spec = importlib.util.spec_from_file_location("bench_mod", BENCH)
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    bench._flusher(torch, device="cpu", nbytes=1 << 16)()
