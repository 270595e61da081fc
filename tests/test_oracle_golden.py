"""The oracle against its frozen results on the tiny workload (tests/golden/oracle_tiny.json).

The file was written by tests/golden/make_golden.py from the oracle itself; it
pins nothing to the pages, but any later change of the oracle's arithmetic makes
this test fail, and the change then has to name the passage that justifies it.
"""

import json
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_reproduces_its_frozen_tiny_results():
    import sys
    sys.path.insert(0, os.path.join(HERE, "golden"))
    import make_golden
    with open(os.path.join(HERE, "golden", "oracle_tiny.json")) as fh:
        ref = json.load(fh)
    got = make_golden.compute()
    assert got["problem"] == ref["problem"] and got["seed"] == ref["seed"]
    assert got["sha256_float32"] == ref["sha256_float32"]
    assert got["sha256_int32"] == ref["sha256_int32"]
    assert got["y_first_row"] == ref["y_first_row"]
    np.testing.assert_allclose(got["d_topk_weights"], ref["d_topk_weights"], rtol=1e-12, atol=1e-12)
    for name, (n, mx, sm) in ref["dev_summary"].items():
        gn, gmx, gsm = got["dev_summary"][name]
        assert abs(gn - n) <= max(1, n // 1000), name
        np.testing.assert_allclose([gmx, gsm], [mx, sm], rtol=1e-6, err_msg=name)
