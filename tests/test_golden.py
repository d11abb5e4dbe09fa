"""Hand-worked examples (tests/golden/*.json) against the oracle."""
import json
import math
import os
from fractions import Fraction

import numpy as np

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _num(x):
    return float(Fraction(x)) if isinstance(x, str) else x


def _arr(x):
    return np.array([[_num(y) for y in row] for row in x]) if isinstance(x[0], list) else \
        np.array([_num(y) for y in x])


def test_diag_worked_example(oracle_lib):
    g = json.load(open(os.path.join(GOLD, "diag_worked_example.json")))
    i = g["inputs"]
    d = np.array([math.log(2.0), 2.0 * math.log(2.0)])
    res = oracle.diag_head(np.array(i["q"]), np.array(i["k"]), np.array(i["v"]),
                           np.array(i["beta"]), d, i["A"], i["I_prior"], lib=oracle_lib)
    for n in ("o", "I_T", "mu_T"):
        np.testing.assert_allclose(res[n], _arr(g["expected"][n]), rtol=1e-14, atol=1e-15)


def test_iso_worked_example(oracle_lib):
    g = json.load(open(os.path.join(GOLD, "iso_worked_example.json")))
    i = g["inputs"]
    ones = np.ones((2, 1))
    res = oracle.iso_head(np.array(i["a"]), np.array(i["p"]), np.array(i["Lambda"]), i["lambda0"],
                          q=ones, k=ones, v=np.array(i["v"])[:, None], lib=oracle_lib)
    np.testing.assert_allclose(res["lambda"], _arr(g["expected"]["lambda"]), rtol=1e-15)
    np.testing.assert_allclose(res["o"][:, 0], _arr(g["expected"]["o"]), rtol=1e-14)
