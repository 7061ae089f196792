"""Each planted oracle mistake (tests/oracle_mutants.py) is caught by the
oracle's pins: a child pytest run of the pin files with the mistake planted
must fail.  The mistakes are planted in the CPU oracle only."""
import os
import subprocess
import sys

import pytest

from oracle_mutants import MUTANTS

HERE = os.path.dirname(os.path.abspath(__file__))
PIN_FILES = [os.path.join(HERE, "test_oracle.py"), os.path.join(HERE, "test_oracle_properties.py")]


def run_pins(mutant=None):
    env = dict(os.environ)
    env.pop("MOE_ORACLE_MUTANT", None)
    if mutant:
        env["MOE_ORACLE_MUTANT"] = mutant
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *PIN_FILES],
                          capture_output=True, text=True, env=env, timeout=300, cwd=os.path.dirname(HERE))


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
def test_planted_mistake_is_caught(mutant):
    r = run_pins(mutant)
    assert r.returncode == 1, f"{mutant}: pins did not fail\n{r.stdout[-2000:]}"
    assert " failed" in r.stdout
