"""Positive control of the count kernel's cross-block hand-off (per-block
totals stored write-through, an arrival ticket, the last block reading them
back): block 0 is held back from the host (MOE_COUNT_DELAY, in a child
process since the library reads it once) so that it arrives last, and the
dispatch and forward metadata must stay bit-exact against the oracle.  The
kernel exits normally; the hold-back is a bounded sleep."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_count_handoff_with_block_zero_arriving_last():
    env = dict(os.environ, MOE_COUNT_DELAY="100")
    print("[gpu-case] count hand-off, block 0 held back", flush=True)
    p = subprocess.run([sys.executable, "-u", os.path.join(HERE, "count_handoff_case.py")],
                       env=env, capture_output=True, text=True, timeout=240)
    print(p.stdout[-2000:], p.stderr[-2000:], flush=True)
    assert p.returncode == 0 and p.stdout.strip().endswith("ok")
