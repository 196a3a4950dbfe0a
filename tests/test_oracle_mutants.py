"""Pin sensitivity: every planted mistake in the oracle fails some pin.

`oracle/hba_oracle.c` compiled with -DORC_MUTANT=n makes one plausible slip
(a dropped term, a wrong sign, index or operand; the list is in the file).
For each n this builds that variant with gcc, points the oracle loader at it
(HBA_ORACLE_LIB) and runs the CPU pin suites in a subprocess: they must
fail.  The same build with ORC_MUTANT=0 must pass, which shows that the
harness itself works.  CPU only.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "hba_oracle.c")
PINS = [os.path.join(ROOT, "tests", "test_oracle_pins.py"), os.path.join(ROOT, "tests", "test_oracle_transfer.py")]

MUTANTS = {
    1: "negative half of phi takes softmax(u)",
    2: "negative half of phi normalised by the positive sum",
    3: "W read transposed in the projection",
    4: "commit drops the Z update",
    5: "commit folds k in place of v",
    6: "step drops 1/sqrt(d)",
    7: "gate missing from the shared denominator",
    8: "linear denominator phi(q).Z dropped",
    9: "a query does not see its own key",
    10: "key/value head h % Hkv instead of h / G",
    11: "comparator drops the block's own keys",
    12: "comparator drops 1/sqrt(d)",
    13: "transfer: sign of dL/dden",
    14: "transfer: Z term of dphi(q) dropped",
    15: "transfer: sigmoid factor w(1-w) of dL/dalpha reduced to w",
    16: "transfer: Gz term of dphi(k) dropped",
    17: "transfer: sign of the softmax(-u) half in the feature-map Jacobian",
    18: "transfer: block committed before its own queries read the state",
}


def _build(n, out_dir):
    lib = os.path.join(out_dir, f"liboracle_m{n}.so")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", f"-DORC_MUTANT={n}",
                    "-o", lib, SRC, "-lm"], check=True, capture_output=True)
    return lib


def _run_pins(lib):
    env = dict(os.environ, HBA_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    return r.returncode, r.stdout[-2000:]


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    out_dir = str(tmp_path_factory.mktemp("mutants"))
    ids = [0, *MUTANTS]
    libs = {n: _build(n, out_dir) for n in ids}
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        res = dict(zip(ids, ex.map(lambda n: _run_pins(libs[n]), ids)))
    return res


def test_unmutated_build_passes(outcomes):
    rc, tail = outcomes[0]
    assert rc == 0, tail


@pytest.mark.parametrize("n", sorted(MUTANTS))
def test_planted_mistake_is_caught(outcomes, n):
    rc, tail = outcomes[n]
    assert rc != 0, f"mutant {n} ({MUTANTS[n]}) passed every pin:\n{tail}"
