"""The oracle's pins catch planted mistakes.

For every mutant in tests/oracle_mutants.py (one plausible mistake each: a dropped term, a wrong
sign, index or axis, a wrong rounding, a wrong slice order), the oracle's pin suite is run in a
fresh interpreter with that mutant applied, and at least one pin must fail.  An unmutated run must
pass, so a failure is the mutant's doing.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

from tests.oracle_mutants import MUTANTS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = ["tests/test_oracle_moe.py", "tests/test_oracle_codecs.py", "tests/test_oracle_prefetch.py",
        "tests/test_golden.py"]


def _run(mutant: str) -> int:
    env = dict(os.environ, ORACLE_MUTANT=mutant, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "tests.oracle_mutants",
                        "-p", "no:cacheprovider", "-m", "not gpu", *PINS],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode


def test_every_planted_mistake_fails_a_pin():
    names = [""] + sorted(MUTANTS)
    with cf.ThreadPoolExecutor(4) as ex:
        codes = dict(zip(names, ex.map(_run, names)))
    assert codes[""] == 0, "the unmutated pin suite must pass"
    survivors = [n for n in names[1:] if codes[n] != 1]
    assert not survivors, f"mutants no pin caught (or that broke the run): {survivors} -> {[codes[n] for n in survivors]}"
