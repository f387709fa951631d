"""Hand-worked route-layer instance (tests/golden/hand_worked_route.json) against the oracle."""
import json
import math
import os

import numpy as np

from oracle import route as O

HERE = os.path.dirname(os.path.abspath(__file__))


def test_hand_worked_route_layer():
    g = json.load(open(os.path.join(HERE, "golden", "hand_worked_route.json")))
    exp = g["expected"]
    N, d, SL, CT = 4, 2, 64, 63
    L = N * SL
    w = np.array([[0.0, 0.0], [math.sqrt(2) * math.log(3), 0.0], [math.sqrt(2) * math.log(2), 0.0], [-1.0, 0.0]])
    k = np.zeros((1, 1, L, d))
    v = np.zeros((1, 1, L, d))
    v[..., 1] = 1.0
    for c in range(N):
        k[0, 0, c * SL: c * SL + CT] = w[c]
        k[0, 0, c * SL + CT] = (5.0, 5.0)
    v[0, 0, SL: SL + CT] = np.stack([np.arange(CT), np.zeros(CT)], axis=1)
    q = np.zeros((1, 1, L, d))
    q[0, 0, SL - 1::SL] = (0.3, -0.2)
    q[0, 0, 10] = (1.0, 0.0)
    x = np.ones((1, L, 1))
    A = np.zeros((1, 1))
    Bm = np.ones((1, d))
    r = O.route_layer(q, k, v, x, A, Bm, K=1, R=0, beta=0.0, scale=1 / math.sqrt(2), queries=np.array([10]))
    np.testing.assert_allclose(r["s"][0, 0, 1], exp["s_1"], atol=1e-12)
    np.testing.assert_allclose(r["H"][0, 0], exp["H"], atol=1e-12)
    assert list(r["idx"][0, 0, 0]) == exp["idx"]
    np.testing.assert_allclose(r["zsel"][0, 0, 0], exp["zsel"], atol=1e-12)
    np.testing.assert_allclose(r["o"][0, 0, 0], exp["o"], atol=1e-12)
    np.testing.assert_allclose(r["lse"][0, 0, 0], exp["lse"], atol=1e-12)
