"""The test-input helpers (CPU): the threaded oracle helper is the oracle."""
import numpy as np

import oracle
from cases import gapped_rows, oracle_rows, weights
from decode_moe_layer_amd import synth


def test_oracle_rows_equals_one_call():
    """Rows split over threads give the same results, bit for bit, as one
    call on all rows (the method treats rows independently)."""
    cfg = synth.CONFIGS["c0"].with_rows(7)
    w = weights("c0")
    x, r, _ = gapped_rows(cfg, w)
    a = oracle.moe_tail(x, r, w, cfg)
    b = oracle_rows(x, r, w, cfg)
    assert sorted(a) == sorted(b)
    for k in a:
        np.testing.assert_array_equal(np.asarray(a[k]), np.asarray(b[k]), err_msg=k)
