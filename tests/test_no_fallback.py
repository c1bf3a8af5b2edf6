"""The product path has no CPU fallback: without liblbsr.so a call raises
LibraryNotBuilt, and the package's code never reaches the oracle (which is
test infrastructure only)."""

import os
import pathlib
import re
import subprocess
import sys

ROOT = pathlib.Path(__file__).resolve().parents[1]


def test_missing_library_fails_loudly():
    code = (
        "import load_balanced_split_rope_amd as lb\n"
        "try:\n"
        "    lb.device_workers(0)\n"
        "except lb.LibraryNotBuilt as e:\n"
        "    print('raised:', e)\n"
        "else:\n"
        "    raise SystemExit('no error without the library')\n")
    env = dict(os.environ, LBSR_LIB=str(ROOT / "no_such_dir" / "liblbsr.so"))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "raised:" in r.stdout


def test_package_never_imports_the_oracle():
    pkg = ROOT / "load_balanced_split_rope_amd"
    for f in pkg.rglob("*.py"):
        text = f.read_text()
        assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
        assert "oracle." not in text.replace("the oracle.", ""), f
