"""The oracle's pins catch plausible mistakes: each mutant in oracle_mutants.py plants one in the
CPU oracle, in a subprocess, and at least one of its listed pin tests must then fail (CPU only)."""
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

from oracle_mutants import MUTANTS

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _run(name):
    _, _, pins = MUTANTS[name]
    env = dict(os.environ, ORACLE_MUTANT=name, COLUMNS="200")
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "--tb=short", "-p", "no:cacheprovider", "-m", "not gpu",
           *[os.path.join("tests", p) for p in pins]]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return name, r.returncode, r.stdout[-6000:]


@pytest.fixture(scope="module")
def results():
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        return {name: (rc, out) for name, rc, out in ex.map(_run, sorted(MUTANTS))}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(results, name):
    rc, out = results[name]
    # exit code 1: tests ran and at least one failed (2 or more would be a broken mutant or run),
    # and it failed on a comparison, not on an exception the mutant itself raised
    assert rc == 1, f"mutant {name} not caught (pytest exit {rc}):\n{out}"
    errors = set(re.findall(r"^E\s+(\w+(?:Error|Exception))", out, flags=re.M))
    asserted = "AssertionError" in errors or re.search(r"^E\s+assert ", out, flags=re.M)
    assert asserted and errors <= {"AssertionError"}, out


def test_pins_pass_without_a_mutant():
    pins = sorted({p for _, _, ps in MUTANTS.values() for p in ps})
    env = {k: v for k, v in os.environ.items() if k != "ORACLE_MUTANT"}
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        *[os.path.join("tests", p) for p in pins]],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:]
