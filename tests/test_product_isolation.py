"""The product path stands on the HIP library alone: importing and using the package loads no
part of the oracle, and without the built library every call raises (no CPU fallback)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(code: str) -> subprocess.CompletedProcess:
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=240)


def test_package_never_imports_the_oracle():
    r = _run("import sys, zero_sharded_mixed_amd as Z, zero_sharded_mixed_amd.step, zero_sharded_mixed_amd.build\n"
             "bad = [m for m in sys.modules if m == 'oracle' or m.startswith('oracle.')]\n"
             "print('LOADED', bad)\n"
             "assert not bad, bad\n"
             "import ctypes\n"
             "names = [l for l in open('/proc/self/maps').read().splitlines() if 'zero_oracle' in l]\n"
             "assert not names, names\n")
    assert r.returncode == 0, r.stdout + r.stderr


def test_missing_library_raises_instead_of_falling_back():
    r = _run("import zero_sharded_mixed_amd._binding as B\n"
             "B.LIB_PATH = '/nonexistent/libzero_shard.so'\n"
             "B._lib = None\n"
             "try:\n"
             "    B.lib()\n"
             "except RuntimeError as e:\n"
             "    print('RAISED', e)\n"
             "else:\n"
             "    raise SystemExit('no error')\n")
    assert r.returncode == 0 and "RAISED" in r.stdout and "no fallback" in r.stdout, r.stdout + r.stderr


def test_product_sources_do_not_name_the_oracle():
    pkg = os.path.join(ROOT, "zero_sharded_mixed_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "zero_oracle" not in text, f
