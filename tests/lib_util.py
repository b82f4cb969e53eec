"""Helpers for tests that need the built library (builds it when missing)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def ensure_built():
    from bit_moe_expert_fp9_amd import duckmoe
    if not os.path.exists(duckmoe.LIB_PATH):
        subprocess.run([sys.executable, "-m", "bit_moe_expert_fp9_amd.build"], cwd=ROOT,
                       check=True)
    return duckmoe.lib()
