"""The oracle still reproduces its stored regression values bit for bit.

``tests/golden/oracle_regression.txt`` is written by
``tests/golden/make_oracle_regression.py`` from the oracle alone; it locks the
oracle's arithmetic against silent change (correctness is pinned elsewhere).
"""
import os

import tests.golden.make_oracle_regression as gen


def _read():
    cases, cur = {}, None
    with open(gen.OUT) as f:
        for line in f:
            if line.startswith("#"):
                continue
            if line.startswith("case "):
                cur = line[5:].strip()
                cases[cur] = {}
            else:
                i, h = line.split()
                cases[cur][int(i)] = float.fromhex(h)
    return cases


def test_oracle_matches_regression_lock():
    stored = _read()
    assert len(stored) == len(gen.CASES) + len(gen.ADALN_CASES) + len(gen.GN_CASES)
    for name, vals in gen.cases():
        for i, v in stored[name].items():
            assert vals[i] == v, (name, i)
