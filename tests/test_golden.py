"""Hand-worked cases of the EFLA update (tests/golden/hand_cases.json) against
the fp64 oracle.  The expected values were derived by hand from the pages'
closed form and update rule (Method steps 2-3); see the file's derivations."""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))
TOL = GOLDEN["tolerance"]


def test_ln2_constant():
    assert GOLDEN["ln2"] == math.log(2.0)


@pytest.mark.parametrize("case", GOLDEN["coefficient_cases"], ids=lambda c: c["why"][:30])
def test_coefficient_cases(case):
    got = oracle.alpha(case["beta"], case["lambda"])
    assert abs(got - case["alpha"]) <= TOL * max(abs(case["alpha"]), 1e-300)


@pytest.mark.parametrize("case", GOLDEN["sequence_cases"], ids=lambda c: c["name"])
def test_sequence_cases(case):
    s0 = np.array(case["s0"], np.float64)
    k = np.array(case["k"], np.float64)
    v = np.array(case["v"], np.float64)
    q = np.array(case["q"], np.float64)
    beta = np.array(case["beta"], np.float64)
    L, dk = k.shape
    dv = v.shape[1]
    o, sf = oracle.forward(q.reshape(1, L, 1, dk), k.reshape(1, L, 1, dk), v.reshape(1, L, 1, dv),
                           beta.reshape(1, L, 1), s0.reshape(1, 1, dk, dv))
    np.testing.assert_allclose(o[0, :, 0], np.array(case["o"]), rtol=0, atol=TOL * 32)
    np.testing.assert_allclose(sf[0, 0], np.array(case["s_final"]), rtol=0, atol=TOL * 32)
