"""Frozen oracle outputs (tests/golden/oracle_small.json, written by
tests/golden/make_golden.py from oracle/ only) and one QDQ tile worked by
hand from the QDQ reading in oracle/qdq.py."""
import json
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_frozen_golden():
    import importlib.util
    spec = importlib.util.spec_from_file_location('make_golden',
                                                  os.path.join(HERE, 'golden', 'make_golden.py'))
    mg = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mg)
    want = json.load(open(os.path.join(HERE, 'golden', 'oracle_small.json')))
    got = mg.compute()
    for tag in ('e4m3', 'int8'):
        for key, w in want[tag].items():
            np.testing.assert_allclose(got[tag][key], w, rtol=1e-11, atol=1e-13, err_msg=key)


def test_hand_worked_qdq_tile():
    """x = [3, -1.5, 0.1, 0]: amax 3, d = fl32(3/448), y = x * fl32(1/d)
    = [448, -224, 14.93.., 0] -> E4M3 codes [448, -224, 15, 0]
    (14.93 lies in the binade [8, 16) whose step is 1)."""
    want = json.load(open(os.path.join(HERE, 'golden', 'oracle_small.json')))['qdq_tile']
    assert want['codes'] == [[448.0, -224.0, 15.0, 0.0]]
    d = np.float32(3.0) / np.float32(448.0)
    assert np.float32(want['d']) == d
    np.testing.assert_array_equal(np.float32(want['out']),
                                  (np.float32([448.0, -224.0, 15.0, 0.0]) * d)[None])
