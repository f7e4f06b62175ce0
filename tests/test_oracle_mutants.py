"""The oracle pins catch planted mistakes.

For every mutant in tests/oracle_mutants.py (a plausible slip written into a
copy of the oracle: eps outside the root, the mean replaced by the sum, the
gain dropped or turned into 1+g, a sign flip or a sigmoid in silu, gate and
up swapped, the residual dropped or taken from n, a transposed weight, the
wrong Q8 block axis, unsigned quants, flushed fp16 subnormals, a wrong bf16
decode; in the stored-format wrappers, gate and up weights swapped, the down
weights taken from another operand, fp32 decoded through fp16 or truncated
to bf16, the norm's gain decoded in the wrong format or dropped), the pin suite run against the mutated oracle must fail.  The
mutants run on the CPU, each in its own interpreter.
"""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
import oracle_mutants  # noqa: E402


def _run(name):
    return subprocess.run([sys.executable, os.path.join(HERE, "oracle_mutants.py"), name],
                          capture_output=True, text=True, timeout=300)


@pytest.mark.parametrize("name", sorted(oracle_mutants.MUTANTS))
def test_pins_reject_mutant(name):
    res = _run(name)
    # pytest exit status 1: tests ran and at least one failed
    assert res.returncode == 1, f"mutant {name} survived the pins:\n{res.stdout[-2000:]}"


def test_unmutated_oracle_passes_through_the_same_harness():
    res = _run("none")
    assert res.returncode == 0, res.stdout[-2000:]


def test_every_mutant_applies_to_the_current_source():
    for name in oracle_mutants.MUTANTS:
        src = oracle_mutants.mutated_source(name)
        assert src != open(oracle_mutants.SRC).read()
