"""The oracle's pins catch planted mistakes: for each of the mistakes in tests/oracle_mutants.py (a
wrong sign, scale, gate order, missing 1+, swapped RoPE halves, patch feature order, shift formula,
SwiGLU operand order, variance ddof, reversed V, sin/cos order, CFG formula, exclusive SLG window,
swapped final shift/scale), a child pytest run of tests/test_oracle_pins.py with that one mistake
planted in the oracle must fail; with none planted it must pass. CPU only."""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

from tests.oracle_mutants import MUTANTS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(name):
    env = dict(os.environ, MOSS_ORACLE_MUTANT=name)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-p",
                        "tests.oracle_mutants", "-m", "not gpu", "tests/test_oracle_pins.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-1500:]


def test_pins_catch_every_planted_mistake():
    names = ["none"] + sorted(MUTANTS)
    with cf.ThreadPoolExecutor(4) as ex:
        results = {n: (rc, out) for n, rc, out in ex.map(_run, names)}
    rc, out = results.pop("none")
    assert rc == 0, out                           # the unmodified oracle passes its pins
    missed = [n for n, (rc, _) in results.items() if rc != 1]
    assert not missed, {n: results[n][1] for n in missed}
