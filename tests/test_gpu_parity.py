"""Parity of the HIP path with the CPU oracle on every workload, through the C ABI."""
import sys

import numpy as np
import pytest

import oracle
from cases import gapped_rows, weights
from decode_moe_layer_amd import synth
from gpu_harness import check_against_oracle, device_weights, handle_for, run

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("name", ["c0", "c1", "c2", "c3", "c4"])
def test_parity_workloads(name):
    cfg = synth.CONFIGS[name]
    _say("parity", name, cfg)
    w = weights(name)
    x, r, _ = gapped_rows(cfg, w)
    o = oracle.moe_tail(x, r, w, cfg)
    h = handle_for(cfg)
    g = run(h, cfg, device_weights(name), x, r)
    assert h.get_error() == 0
    check_against_oracle(g, o, cfg)
    if name == "c2":
        distinct = len(set(g["ids"].ravel().tolist()))
        assert 54 <= distinct <= 58, distinct


@pytest.mark.parametrize("rows,max_rows", [(2, 2), (3, 8), (4, 16), (5, 5), (16, 16)])
def test_parity_row_counts_on_the_shard(rows, max_rows):
    cfg = synth.CONFIGS["c1"].with_rows(rows)
    _say("rows", rows, "max_rows", max_rows)
    w = weights("c1")
    x, r, _ = gapped_rows(cfg, w)
    o = oracle.moe_tail(x, r, w, cfg)
    h = handle_for(cfg, max_rows=max_rows)
    g = run(h, cfg, device_weights("c1"), x, r)
    check_against_oracle(g, o, cfg)


def test_no_residual_means_h_is_x():
    cfg = synth.CONFIGS["c0"].with_rows(3)
    w = weights("c0")
    x, r, _ = gapped_rows(cfg, w)
    x2 = x.copy()
    o = oracle.moe_tail(x2, None, w, cfg)
    # re-check the gap for the residual-free rows; keep only if well posed
    from cases import key_gaps

    if np.any(key_gaps(o["keys"], cfg.topk) < 1e-4):
        pytest.skip("residual-free rows not well posed")
    h = handle_for(cfg)
    g = run(h, cfg, device_weights("c0"), x2, None)
    np.testing.assert_array_equal(g["res_out"], x2)
    check_against_oracle(g, o, cfg)


@pytest.mark.parametrize("name,rows", [("c0", 1), ("c1", 8), ("c4", 16)])
def test_parity_with_a_shared_gate(name, rows):
    """The shared expert's output scaled by sigmoid(wg . xn) per row ("[AMD]
    integrate kimi k3 monokernel", K2 commit text, Kernel Replacement), on the
    three kernel paths: routed sums by every reader (c0), xn in LDS (c1 at 8
    rows), xn read from global scratch (c4 at 16 rows)."""
    from gpu_harness import dev

    cfg = synth.CONFIGS[name].with_rows(rows)
    _say("gate", name, rows)
    w = dict(weights(name))
    w["shared_gate"] = synth.make_shared_gate(cfg)
    x, r, _ = gapped_rows(cfg, w)
    o = oracle.moe_tail(x, r, w, cfg)
    dw = dict(device_weights(name))
    dw["shared_gate"] = dev(w["shared_gate"])
    h = handle_for(cfg)
    g = run(h, cfg, dw, x, r)
    assert h.get_error() == 0
    check_against_oracle(g, o, cfg)
    plain = oracle.moe_tail(x, r, weights(name), cfg)
    assert not np.allclose(plain["y_shared"], o["y_shared"])  # the gate changed the shared part
