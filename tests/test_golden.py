"""Golden fixtures: values the WAITS README states, and exact closed forms."""
import math
import os
from fractions import Fraction

import numpy as np

from oracle import waits_oracle as orc
from synth import ACTIONS

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_actions_match_the_readme():
    rows = {r[0]: r[1:] for r in _lines("actions.txt") if r[0] != "alias"}
    parsed = tuple((float(x.split(":")[0]), int(x.split(":")[1])) for x in rows["actions"])
    assert parsed == ACTIONS


def test_snap_aliases_are_window_limits():
    # TOVA / SnapKV / H2O are the snap scorer with a window; the window-W snap
    # score is the a -> inf limit with b = W of the forgetting curve
    n = 40
    q = np.random.default_rng(1).standard_normal((n, 2, 8))
    k = np.random.default_rng(2).standard_normal((n, 1, 8))
    cu = np.array([0, n])
    for _, name, window in (r for r in _lines("actions.txt") if r[0] == "alias"):
        window = int(window)
        s = orc.waits_scores(q, k, cu, 2, 1, [math.inf], [window], 0.35)[0]
        w = orc.sigmoid_weights(n, math.inf, window)
        assert w.sum() == min(n, window), name
        if name == "TOVA":
            assert np.count_nonzero(s) == n      # the last row attends to all keys
        if name == "H2O":
            s0 = orc.waits_scores(q, k, cu, 2, 1, [0.0], [1], 0.35)[0]
            np.testing.assert_allclose(s, 2 * s0, rtol=1e-12)


def _fixture(name):
    return [(int(k), Fraction(v)) for k, v in _lines(name)]


def test_uniform_h2o_fixture():
    n, g = 12, 4
    s = orc.waits_scores(np.zeros((n, g, 4)), np.random.default_rng(0).random((n, 1, 4)),
                         np.array([0, n]), g, 1, [0.0], [7], 1.0)[0]
    for k, v in _fixture("uniform_h2o_n12_g4.txt"):
        assert abs(s[k] - float(v)) <= 1e-14 * float(v)


def test_uniform_snap_fixture():
    n = 12
    s = orc.waits_scores(np.zeros((n, 1, 4)), np.random.default_rng(0).random((n, 1, 4)),
                         np.array([0, n]), 1, 1, [math.inf], [5], 1.0)[0]
    for k, v in _fixture("uniform_snap_n12_w5.txt"):
        assert abs(s[k] - float(v)) <= 1e-15
