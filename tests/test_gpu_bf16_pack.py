"""The library's fp32 -> bf16 packing rounds to nearest even, as the oracle's
storage mirror does: every stored bf16 value of the path (a, b, y, dA, dB, A',
out, dx) goes through it.  Runs the program tests/bf16_pack_check.hip, which
build() compiles next to the library."""
import os
import subprocess

import pytest

from dropless_moe_dispatch_amd import build as Bld


@pytest.mark.gpu
def test_bf16_packing_is_round_to_nearest_even():
    assert os.path.exists(Bld.PACK_CHECK), "build first: python -c 'import __graft_entry__ as g; g.build()'"
    p = subprocess.run([Bld.PACK_CHECK], capture_output=True, text=True, timeout=120)
    print(p.stdout, flush=True)
    assert p.returncode == 0 and "mismatches: normal 0 nan 0 denormal 0" in p.stdout, (p.returncode, p.stdout,
                                                                                   p.stderr[-2000:])
