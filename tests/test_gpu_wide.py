"""Wide launches: 17 to 32 rows in one launch, experts de-duplicated across
all rows, through the C ABI against the oracle.

An expert picked by more than 16 rows runs as one slot per 16 of its users;
repeated rows force that case.  Rows are independent in the method, so the
oracle's results for a repeated row are its results for the row once.
"""
import dataclasses
import sys

import numpy as np
import pytest

import oracle
from cases import gapped_rows, oracle_rows, weights
from decode_moe_layer_amd import synth
from gpu_harness import check_against_oracle, device_weights, handle_for, run

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _tile(o, idx, n):
    """The oracle's per-row results (n distinct rows) for rows idx of them."""
    return {k: (v[idx] if isinstance(v, np.ndarray) and v.ndim >= 1 and v.shape[0] == n else v) for k, v in o.items()}


@pytest.mark.parametrize("name,rows,n_a", [("c1", 32, 20), ("c1", 32, 16), ("c1", 17, 17), ("c3", 24, 24)])
def test_wide_repeated_rows(name, rows, n_a):
    """Rows 0..n_a-1 repeat row A and the rest repeat row B: A's experts have
    n_a users (two slots above 16), an expert both rows pick has all of them.
    Parity with the oracle, every copy of a row bit-identical, and equal bit
    for bit to a narrow call on [A, B]."""
    cfg2 = synth.CONFIGS[name].with_rows(2)
    _say("wide repeated", name, rows, n_a)
    w = weights(name)
    x2, r2, _ = gapped_rows(cfg2, w)
    o2 = oracle.moe_tail(x2, r2, w, cfg2)
    idx = np.array([0] * n_a + [1] * (rows - n_a))
    cfg = cfg2.with_rows(rows)
    x, r = x2[idx], r2[idx]
    h = handle_for(cfg, max_rows=32)
    g = run(h, cfg, device_weights(name), x, r)
    assert h.get_error() == 0
    check_against_oracle(g, _tile(o2, idx, 2), cfg)
    shared = set(o2["ids"][0].tolist()) & set(o2["ids"][1].tolist())
    _say("experts picked by both rows:", len(shared))
    hn = handle_for(cfg2, max_rows=2)
    gn = run(hn, cfg2, device_weights(name), x2, r2)
    assert hn.get_error() == 0
    for k in ("ids", "w", "out", "res_out", "y_routed", "y_shared", "logits"):
        for row in range(rows):
            np.testing.assert_array_equal(g[k][row], gn[k][idx[row]], err_msg="%s row %d" % (k, row))


@pytest.mark.parametrize("name,rows", [("c0", 24), ("c3", 20)])
def test_wide_all_options(name, rows):
    """The optional steps in a wide launch (MXFP8 experts, folded norm,
    group-limited routing, routed scale, shared gate) against the oracle, and
    the first 16 rows equal a narrow call on them."""
    n_group, topk_group = (2, 1) if name == "c0" else (8, 4)
    cfg = dataclasses.replace(synth.CONFIGS[name].with_rows(rows), weight_format=1, fold_norm=1, n_group=n_group,
                              topk_group=topk_group, routed_scale=2.5)
    _say("wide all options", name, rows)
    w = dict(synth.make_weights(cfg))
    w["shared_gate"] = synth.make_shared_gate(cfg)
    from test_gpu_parity import _grouped_rows
    from gpu_harness import dev

    x, r = _grouped_rows(cfg, w)
    o = oracle.moe_tail(x, r, w, cfg)
    dw = {k: dev(v) for k, v in w.items()}
    h = handle_for(cfg, max_rows=32)
    g = run(h, cfg, dw, x, r)
    assert h.get_error() == 0
    check_against_oracle(g, o, cfg)
    c16 = cfg.with_rows(16)
    g16 = run(handle_for(c16), c16, dw, x[:16], r[:16])
    for k in ("ids", "w", "out", "res_out", "y_routed", "y_shared", "logits"):
        np.testing.assert_array_equal(g[k][:16], g16[k], err_msg=k)
    del dw, h


# (config, max_rows): c1's shard at 32 rows with top-16 is 512 picks, the most
# a wide launch takes; at that top-k even 16 rows do not fit a narrow launch's
# LDS, so the handle runs every call wide, its routed activations staged in
# groups.  A small shard at 32 rows with top-17 is 544 picks: narrow launches.
PICK_LIMIT = {
    "wide_512": (dataclasses.replace(synth.CONFIGS["c1"].with_rows(32), topk=16), 32),
    "narrow_544": (synth.Config("narrow_544", 12, 32, 512, 64, 17, 64, 64), 32),
}


@pytest.mark.parametrize("case", sorted(PICK_LIMIT))
def test_wide_pick_limit(case):
    """Parity with the oracle at the wide launch's pick limit and just past
    it, and the first 16 rows equal a 16-row call, bit for bit."""
    cfg, max_rows = PICK_LIMIT[case]
    _say("pick limit", case, cfg.rows, "rows, top", cfg.topk)
    w = weights("c1") if case == "wide_512" else synth.make_weights(cfg)
    x, r, _ = gapped_rows(cfg, w)
    o = oracle_rows(x, r, w, cfg)
    from gpu_harness import dev

    dw = device_weights("c1") if case == "wide_512" else {k: dev(v) for k, v in w.items()}
    h = handle_for(cfg, max_rows=max_rows)
    g = run(h, cfg, dw, x, r)
    assert h.get_error() == 0
    check_against_oracle(g, o, cfg)
    c16 = cfg.with_rows(16)
    g16 = run(handle_for(c16), c16, dw, x[:16], r[:16])
    for k in ("ids", "w", "out", "res_out", "y_routed", "y_shared", "logits"):
        np.testing.assert_array_equal(g[k][:16], g16[k], err_msg=k)


def test_wide_deadline_drill_then_recovery_on_the_same_handle():
    """A wide launch (c0's shard, 24 rows) whose workgroup 3 is held at its
    first cross-workgroup wait on the first call only: the deadline fires,
    the error reads ETIMEOUT, and the same handle's next call is at parity."""
    from decode_moe_layer_amd import binding

    cfg = synth.CONFIGS["c0"].with_rows(24)
    w = weights("c0")
    x, r, _ = gapped_rows(cfg, w)
    o = oracle_rows(x, r, w, cfg)
    dw = device_weights("c0")
    h = handle_for(cfg, max_rows=32, deadline_us=20000, debug_flags=binding.DEBUG_STALL_ONCE, debug_block=3)
    run(h, cfg, dw, x, r)
    assert h.get_error() == binding.ETIMEOUT
    g = run(h, cfg, dw, x, r)
    assert h.get_error() == binding.OK
    check_against_oracle(g, o, cfg)
