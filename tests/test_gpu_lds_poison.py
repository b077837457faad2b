"""Race test: the search and W4A16 parity cases of tests/lds_poison_cases.py against the LDS-poison
debug build (weight_only_int4_act_amd/libawq_ldspoison.so, built next to libawq.so with
AWQ_LDS_POISON).  There every pipelined LDS buffer holds NaN between its last reader and its next
writer, so a missing wait or barrier would surface as NaN or a parity failure rather than as stale
data that happens to pass.  The binding loads one library per process, so the cases run in a child
process with AWQ_LIBRARY set.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "weight_only_int4_act_amd", "libawq_ldspoison.so")

pytestmark = pytest.mark.gpu


def test_parity_under_lds_poison():
    assert os.path.exists(LIB), f"{LIB} is missing: build with `python -m weight_only_int4_act_amd.build`"
    env = dict(os.environ)
    env["AWQ_LIBRARY"] = LIB
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "tests", "lds_poison_cases.py")],
                       capture_output=True, text=True, env=env, timeout=240)
    print(r.stdout[-6000:])
    assert r.returncode == 0, f"{r.stdout[-4000:]}\n{r.stderr[-4000:]}"
    assert "[poison] all cases ok" in r.stdout
