"""The oracle still reproduces the fixtures it wrote (CPU only)."""
import json
import os

import numpy as np
import pytest

import oracle
from workloads import make

from tests.golden.make_golden import CASES  # noqa: E402

HERE = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("name", sorted(CASES))
def test_oracle_reproduces_golden(name):
    with open(os.path.join(HERE, f"{name}.json")) as f:
        gold = json.load(f)
    res = oracle.select(make(CASES[name]))
    for r, g in zip(res, gold["sequences"]):
        np.testing.assert_array_equal(r.cand_idx, g["cand_idx"])
        np.testing.assert_array_equal(r.path, g["path"])
        np.testing.assert_array_equal(r.slots, g["slots"])
        np.testing.assert_allclose(r.scores, g["scores"], rtol=1e-12, atol=1e-12)
