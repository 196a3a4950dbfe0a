"""Pin sensitivity: every planted mistake in the oracle fails some pin.

Each mistake below is a plausible slip (a dropped term, a wrong sign, index or
operand), written as textual substitutions applied to a temporary copy of
`oracle/hba_oracle.c`.  Every substitution must match the committed source
exactly once, so a mistake cannot silently stop applying when the oracle
changes.  For each one the test builds the mutated copy with gcc, points the
oracle loader at it (HBA_ORACLE_LIB) and runs the CPU pin suites in a
subprocess: they must fail.  The unmodified source, built the same way, must
pass, which shows that the harness itself works.  CPU only; the committed
oracle holds no switch for any of this.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "hba_oracle.c")
PINS = [os.path.join(ROOT, "tests", "test_oracle_pins.py"), os.path.join(ROOT, "tests", "test_oracle_transfer.py")]

_I12, _I16 = " " * 12, " " * 16
# n -> (description, [(text in the oracle, replacement), ...])
MUTANTS = {
    1: ("negative half of phi takes softmax(u)",
        [("phi[F + f] = exp(-u[f] + mn) / sn;", "phi[F + f] = exp(u[f] - mx) / sp;")]),
    2: ("negative half of phi normalised by the positive sum",
        [("phi[F + f] = exp(-u[f] + mn) / sn;", "phi[F + f] = exp(-u[f] + mn) / sp;")]),
    3: ("W read transposed in the projection",
        [("acc += x[i] * W[(int64_t)i * F + f];", "acc += x[i] * W[(int64_t)f * d + i];")]),
    4: ("commit drops the Z update",
        [(f"Z[f] += p[f];\n{_I16}for (int n = 0; n < d; ++n)", "for (int n = 0; n < d; ++n)")]),
    5: ("commit folds k in place of v",
        [("S[(int64_t)f * d + n] += p[f] * vt[n];", "S[(int64_t)f * d + n] += p[f] * kt[n];")]),
    6: ("step drops 1/sqrt(d)",
        [(f"kb[(int64_t)j * d + n];\n{_I16}sc *= scale;", "kb[(int64_t)j * d + n];")]),
    7: ("gate missing from the shared denominator",
        [("double den = w * sm_den + lin_den;", "double den = sm_den + lin_den;")]),
    8: ("linear denominator phi(q).Z dropped",
        [("double den = w * sm_den + lin_den;", "double den = w * sm_den;")]),
    9: ("a query does not see its own key",
        [("for (int j = 0; j < L; ++j) {", "for (int j = 0; j < L; ++j) {\n" + _I16 + "if (j == i) continue;")]),
    10: ("key/value head h % Hkv instead of h / G",
         [("return (int64_t)b * Hkv + h / (H / Hkv);", "return (int64_t)b * Hkv + h % Hkv;")]),
    11: ("comparator drops the block's own keys",
         [("for (int j = 0; j < P + L; ++j) {", "for (int j = 0; j < P; ++j) {")]),
    12: ("comparator drops 1/sqrt(d)",
         [(f"sc += qi[n] * kj[n];\n{_I16}sc *= scale;", "sc += qi[n] * kj[n];")]),
    13: ("transfer: sign of dL/dden",
         [("dden[i] = -go / den;", "dden[i] = go / den;")]),
    14: ("transfer: Z term of dphi(q) dropped",
         [("double acc = Z[f] * dden[i];", "double acc = 0.0;")]),
    15: ("transfer: sigmoid factor w(1-w) of dL/dalpha reduced to w",
         [("pw[bh] *= w * (1.0 - w);", "pw[bh] *= w;")]),
    16: ("transfer: Gz term of dphi(k) dropped",
         [("double acc = Gz[f];", "double acc = 0.0;")]),
    17: ("transfer: sign of the softmax(-u) half in the feature-map Jacobian",
         [("du[f] = phi[f] * (dphi[f] - sp) - phi[F + f]", "du[f] = phi[f] * (dphi[f] - sp) + phi[F + f]")]),
    18: ("transfer: block committed before its own queries read the state",
         [(f"const int64_t i0 = (int64_t)n * L;\n{_I12}for (int64_t i = i0; i < i0 + L; ++i) {{",
           f"const int64_t i0 = (int64_t)n * L;\n{_I12}for (int64_t t = i0; t < i0 + L; ++t) {{\n"
           f"{_I16}phi_row(d, F, kb + t * d, Wh, u, p);\n"
           f"{_I16}for (int f = 0; f < P2; ++f) {{\n"
           f"{_I16}    Z[f] += p[f];\n"
           f"{_I16}    for (int c = 0; c < d; ++c) S[(int64_t)f * d + c] += p[f] * vb[t * d + c];\n"
           f"{_I16}}}\n{_I12}}}\n"
           f"{_I12}for (int64_t i = i0; i < i0 + L; ++i) {{"),
          (f"/* commit block n */\n{_I12}for (int64_t t = i0; t < i0 + L; ++t) {{",
           f"/* commit block n */\n{_I12}for (int64_t t = i0; 0 && t < i0 + L; ++t) {{")]),
    19: ("commit folds every token, ignoring n_valid",
         [("int nv = n_valid ? n_valid[b] : T;", "int nv = T;")]),
    20: ("commit writes request b's state, ignoring the slot map",
         [("int64_t s = slot ? slot[b] : b;\n        double *S = S_pool",
           "int64_t s = b;\n        double *S = S_pool")]),
    21: ("step reads request b's state, ignoring the slot map",
         [("int64_t s = slot ? slot[b] : b;\n        const double *S = S_pool",
           "int64_t s = b;\n        const double *S = S_pool")]),
    22: ("comparator reads the whole cache, ignoring prefix_len",
         [("int P = prefix_len ? prefix_len[b] : max_prefix;", "int P = max_prefix;")]),
}


def mutate(src: str, subs) -> str:
    for old, new in subs:
        count = src.count(old)
        if count != 1:
            raise AssertionError(f"substitution {old!r} matches {count} times, expected exactly once")
        src = src.replace(old, new)
    return src


def _build(n, out_dir):
    with open(SRC) as fh:
        src = fh.read()
    if n:
        src = mutate(src, MUTANTS[n][1])
    csrc = os.path.join(out_dir, f"oracle_m{n}.c")
    with open(csrc, "w") as fh:
        fh.write(src)
    lib = os.path.join(out_dir, f"liboracle_m{n}.so")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-o", lib, csrc, "-lm"],
                   check=True, capture_output=True)
    return lib


def _run_pins(lib):
    env = dict(os.environ, HBA_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True)
    return r.returncode, r.stdout[-2000:]


def test_oracle_source_holds_no_switch():
    with open(SRC) as fh:
        src = fh.read()
    assert "MUTANT" not in src and "ORC_M(" not in src


@pytest.mark.parametrize("n", sorted(MUTANTS))
def test_each_substitution_applies_once(n):
    with open(SRC) as fh:
        src = fh.read()
    assert mutate(src, MUTANTS[n][1]) != src


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
    assert rc != 0, f"mutant {n} ({MUTANTS[n][0]}) passed every pin:\n{tail}"
