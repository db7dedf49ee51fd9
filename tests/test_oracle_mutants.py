"""The oracle's pins catch plausible mistakes in it.

For every planted mistake in ``oracle_mutants`` (a dropped factor, a wrong
sign, root, exponent or index, a flipped tie rule) the CPU pin tests of the
oracle run in a child process with that mistake installed, and at least one
of them must fail.  A mistake that every pin lets through would show a
function whose parity rests on nothing.
"""
import os
import subprocess
import sys

import pytest

import oracle_mutants

HERE = os.path.dirname(os.path.abspath(__file__))
PINS = [os.path.join(HERE, "test_oracle_entmax.py"),
        os.path.join(HERE, "test_oracle_pages.py")]


@pytest.mark.parametrize("name", sorted(oracle_mutants.MUTANTS))
def test_pins_catch_planted_mistake(name):
    env = dict(os.environ, EKV_ORACLE_MUTANT=name)
    res = subprocess.run(
        [sys.executable, "-m", "pytest", *PINS, "-x", "-q", "-m", "not gpu",
         "-p", "no:cacheprovider"],
        env=env, capture_output=True, text=True, timeout=600)
    tail = "\n".join(res.stdout.splitlines()[-5:])
    assert res.returncode == 1, "mutant %s survived the pins:\n%s" % (name, tail)
