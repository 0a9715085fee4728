"""The stored oracle fixture: reproduced bitwise, and equal to the exact closed forms."""
import json
import os
from fractions import Fraction

import numpy as np

from tests import exact
from tests.golden import make_golden

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_dyadic.json")


def _load():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def _fr(x):
    if isinstance(x, list):
        return [_fr(e) for e in x]
    return Fraction(x)


def test_oracle_reproduces_fixture_bitwise():
    for case in _load():
        res = make_golden.run_case(case)
        got_out = [[float(x).hex() for x in row] for row in res["out"][:, 0]]
        got_state = [[float(x).hex() for x in row] for row in res["states"][0, 0]]
        assert got_out == case["out_hex"], case["op"]
        assert got_state == case["final_state_hex"], case["op"]


def test_fixture_matches_exact_closed_form():
    for case in _load():
        op, dk = case["op"], case["dk"]
        S0, qs, ks, vs = _fr(case["S0"]), _fr(case["q"]), _fr(case["k"]), _fr(case["v"])
        if op == "rwkv6":
            states, outs = exact.rwkv6_closed_form(S0, qs, ks, vs, _fr(case["decay"]), _fr(case["bonus"]))
        else:
            decs = _fr(case["decay"])
            if op == "gdn":
                decs = [[a] * dk for a in decs]
            states, outs = exact.delta_closed_form(S0, qs, ks, vs, _fr(case["beta"]), decs)
        out = np.array([[float.fromhex(x) for x in row] for row in case["out_hex"]])
        fin = np.array([[float.fromhex(x) for x in row] for row in case["final_state_hex"]])
        want_out = np.array([[float(x) for x in row] for row in outs])
        want_fin = np.array([[float(x) for x in row] for row in states[-1]])
        assert np.linalg.norm(out - want_out) <= 1e-12 * np.linalg.norm(want_out)
        assert np.linalg.norm(fin - want_fin) <= 1e-12 * np.linalg.norm(want_fin)
