"""bench.py's command line without a GPU: a request for more than one GPU is
refused with a message, before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2 and "one GPU" in res.stderr


def test_kernel_source_hash_ignores_comments_only():
    """The hash that keys the stored HBM-counter records follows the code: a comment
    or a line break does not change it, a change inside the code or a string does."""
    sys.path.insert(0, ROOT)
    import bench
    base = 'int f(int a) { return a + 1; } const char* s = "x // y";\n'
    assert bench.code_text(base) == bench.code_text("// head\n" + base.replace(" { ", " {\n  /* c */ "))
    assert bench.code_text(base) != bench.code_text(base.replace("+ 1", "+ 2"))
    assert bench.code_text(base) != bench.code_text(base.replace("x // y", "x y"))
    assert bench.code_text("char c = '\"'; int b; // '") == "char c = '\"'; int b;"
    for rel in bench.KERNEL_SOURCES:
        assert os.path.isfile(os.path.join(ROOT, rel)), rel
    assert len(bench.kernel_source_hash()) == 16
