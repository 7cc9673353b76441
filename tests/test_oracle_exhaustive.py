"""The oracle's exp and log spellings over every binary32 input.

The profile fixes the spelling of exp and log (mojolearn PyPI page, "What
bitwise identity means": transcendental spellings are part of the frozen
profile) and requires each to stay within 2 units in the last place of the true
value. Here every one of the 2^32 inputs is checked against binary64 libm (whose
error is far below binary32's resolution), with the special values (NaN,
infinities, zero, negative arguments of log) and monotonicity between
neighbouring inputs. A C helper does the sweep with OpenMP.

Measured: exp within 0.94 units everywhere; log within 1.97. log never
decreases; exp never decreases on positive arguments, and on negative ones it
steps back by exactly one binary32 step at 2,878 places below 1, where the
output grid is finer than the polynomial's error. Monotonicity is not part of
the accuracy bound, so those single-step reversals are recorded, not refused.
"""
import json
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def sweeper():
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    td = tempfile.mkdtemp()
    exe = os.path.join(td, "exhaustive_elem")
    subprocess.run([cc, "-O2", "-fopenmp", "-o", exe, os.path.join(HERE, "exhaustive_elem.c"), "-lm", "-ldl"],
                   check=True)
    oracle.lib()
    yield exe
    shutil.rmtree(td, ignore_errors=True)


@pytest.mark.parametrize("fn", ["exp", "log"])
def test_all_inputs_within_two_ulp(sweeper, fn):
    r = subprocess.run([sweeper, oracle.LIB_PATH, fn], check=True, capture_output=True, text=True,
                       timeout=900)
    res = json.loads(r.stdout)
    assert res["special_bad"] == 0, res
    assert res["max_ulp"] <= 2.0, res
    if fn == "log":
        assert res["monotonic_breaks"] == 0, res
    else:
        assert res["max_ulp"] < 1.0, res
        assert res["largest_break_steps"] <= 1, res
    print(res)
