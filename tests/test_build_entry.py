"""build() must work on a fresh checkout, where libqsaidx.so does not exist yet:
loading the build script may not import the package (whose import loads the
library and fails loudly when it is absent)."""
from __future__ import annotations

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_build_script_loads_without_package():
    code = (
        "import sys, __graft_entry__ as g\n"
        "mod = g._load_build_module()\n"
        "assert callable(mod.build)\n"
        "assert 'paged_mqa_logits_block_amd' not in sys.modules, sorted(sys.modules)\n"
        "print('ok')\n"
    )
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "ok"
