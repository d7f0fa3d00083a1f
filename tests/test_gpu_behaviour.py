"""Determinism, batch invariance, ties, graph replay and the deadline, on the GPU."""
import numpy as np
import pytest

import oracle
from cases import gapped_rows, weights
from decode_moe_layer_amd import binding, synth
from gpu_harness import check_against_oracle, dev, device_weights, handle_for, run

pytestmark = pytest.mark.gpu


def test_run_to_run_bitwise():
    cfg = synth.CONFIGS["c2"]
    w = weights("c2")
    x, r, _ = gapped_rows(cfg, w)
    h = handle_for(cfg)
    dw = device_weights("c2")
    a = run(h, cfg, dw, x, r)
    for _ in range(3):
        b = run(h, cfg, dw, x, r)
        for k in a:
            np.testing.assert_array_equal(a[k], b[k])


@pytest.mark.parametrize("max_rows", [8, 16])
def test_batch_invariance(max_rows):
    """A row's outputs do not depend on the other rows or on the row count.
    max_rows 8 stages activations in LDS, 16 reads them from global scratch."""
    cfg = synth.CONFIGS["c1"].with_rows(8)
    w = weights("c1")
    x, r, _ = gapped_rows(cfg, w)
    h = handle_for(cfg, max_rows=max_rows)
    dw = device_weights("c1")
    full = run(h, cfg, dw, x, r)
    for rows in (1, 3, 5):
        part = run(h, cfg, dw, x[:rows], r[:rows], rows=rows)
        for k in ("out", "res_out", "ids", "w", "y_routed", "y_shared", "logits"):
            np.testing.assert_array_equal(part[k], full[k][:rows])
    # reversed order of rows
    rev = run(h, cfg, dw, x[::-1].copy(), r[::-1].copy())
    for k in ("out", "ids", "w"):
        np.testing.assert_array_equal(rev[k][::-1], full[k])


def test_exact_ties_go_to_the_lower_expert():
    """Experts with identical router rows give bit-equal fp32 logits; the lower id must win."""
    cfg = synth.Config("ties", 21, 4, 512, 16, 3, 64, 64)
    w = synth.make_weights(cfg)
    rw = w["router_w"].copy()
    for lo, hi in ((1, 9), (2, 5), (3, 12), (0, 15)):
        rw[hi] = rw[lo]
    w["router_w"] = rw
    x, r = synth.make_rows(cfg)
    o = oracle.moe_tail(x, r, w, cfg)
    h = handle_for(cfg)
    dwe = {k: dev(v) for k, v in w.items()}
    g = run(h, cfg, dwe, x, r)
    np.testing.assert_array_equal(g["ids"], o["ids"])
    for row in range(cfg.rows):
        for lo, hi in ((1, 9), (2, 5), (3, 12), (0, 15)):
            assert g["logits"][row][lo] == g["logits"][row][hi]
            if hi in g["ids"][row]:
                assert lo in g["ids"][row]


@pytest.mark.parametrize("max_rows", [8, 16])
def test_graph_replay_of_mixed_row_counts(max_rows):
    t = pytest.importorskip("torch")
    cfg = synth.CONFIGS["c1"].with_rows(8)
    w = weights("c1")
    x, r, _ = gapped_rows(cfg, w)
    h = handle_for(cfg, max_rows=max_rows)
    dw = device_weights("c1")
    widths = [8, 1, 3, 8, 2, 5]
    xd, rd = dev(x), dev(r)
    outs = [t.empty((n, cfg.hidden), dtype=t.int16, device="cuda") for n in widths]
    eager = []
    for n, o in zip(widths, outs):
        eager.append(run(h, cfg, dw, x[:n], r[:n], rows=n, debug=False)["out"])
    s = t.cuda.Stream()
    g = t.cuda.CUDAGraph()
    with t.cuda.stream(s):
        with t.cuda.graph(g, stream=s):
            for n, o in zip(widths, outs):
                h.run(n, xd, rd, dw["gamma"], dw["router_w"], None, dw["w13_q"], dw["w13_s"], dw["w2_q"], dw["w2_s"],
                      dw["ws13"], dw["ws2"], o, stream=s.cuda_stream)
    for rep in range(20):
        for o in outs:
            o.fill_(0)
        g.replay()
        t.cuda.synchronize()
        for n, o, e in zip(widths, outs, eager):
            np.testing.assert_array_equal(o.cpu().numpy().view(np.uint16), e)
    assert h.get_error() == binding.OK


def test_graph_replay_above_16_rows():
    """Calls of more than 16 rows (one wide launch each) captured in one graph
    with a 5-row call between them: every replay equals the eager results."""
    t = pytest.importorskip("torch")
    cfg = synth.CONFIGS["c1"].with_rows(24)
    w = weights("c1")
    x, r, _ = gapped_rows(cfg, w)
    h = handle_for(cfg, max_rows=32)
    dw = device_weights("c1")
    widths = [24, 5, 17]
    xd, rd = dev(x), dev(r)
    outs = [t.empty((n, cfg.hidden), dtype=t.int16, device="cuda") for n in widths]
    eager = [run(h, cfg, dw, x[:n], r[:n], rows=n, debug=False)["out"] for n in widths]
    s = t.cuda.Stream()
    g = t.cuda.CUDAGraph()
    with t.cuda.stream(s):
        with t.cuda.graph(g, stream=s):
            for n, o in zip(widths, outs):
                h.run(n, xd, rd, dw["gamma"], dw["router_w"], None, dw["w13_q"], dw["w13_s"], dw["w2_q"], dw["w2_s"],
                      dw["ws13"], dw["ws2"], o, stream=s.cuda_stream)
    for rep in range(10):
        for o in outs:
            o.fill_(0)
        g.replay()
        t.cuda.synchronize()
        for n, o, e in zip(widths, outs, eager):
            np.testing.assert_array_equal(o.cpu().numpy().view(np.uint16), e)
    assert h.get_error() == binding.OK


def test_deadline_fault_drill_then_recovery():
    """One workgroup never passes its first wait: the deadline fires, the whole
    launch exits, the error reads ETIMEOUT, and the next call is correct."""
    cfg = synth.CONFIGS["c0"]
    w = weights("c0")
    x, r, _ = gapped_rows(cfg, w)
    o = oracle.moe_tail(x, r, w, cfg)
    dw = device_weights("c0")
    bad = handle_for(cfg, deadline_us=20000, debug_flags=binding.DEBUG_STALL, debug_block=3)
    run(bad, cfg, dw, x, r)
    assert bad.get_error() == binding.ETIMEOUT
    assert bad.get_error() == binding.OK  # read-and-clear
    good = handle_for(cfg, deadline_us=20000)
    g = run(good, cfg, dw, x, r)
    assert good.get_error() == binding.OK
    check_against_oracle(g, o, cfg)


def test_calls_after_a_timeout_fail_fast_until_the_error_is_read():
    """After a deadline fires, later calls on the handle give up at their first
    unmet wait instead of waiting out a deadline each; reading the error
    reports the failed wait and resets the handle's control block."""
    import time

    cfg = synth.CONFIGS["c0"]
    w = weights("c0")
    x, r, _ = gapped_rows(cfg, w)
    dw = device_weights("c0")
    bad = handle_for(cfg, deadline_us=50000, debug_flags=binding.DEBUG_STALL, debug_block=3)
    run(bad, cfg, dw, x, r)  # times out after 50 ms
    t0 = time.perf_counter()
    for _ in range(5):
        run(bad, cfg, dw, x, r)  # the error word is still set: these exit at once
    assert (time.perf_counter() - t0) < 0.2, "calls after a timeout waited out their deadlines"
    assert bad.get_error() == binding.ETIMEOUT
    msg = binding.strerror(bad.h)
    assert "deadline" in msg and "epochs" in msg, msg


@pytest.mark.parametrize("name,rows", [("c0", 1), ("c1", 8)])
def test_same_handle_is_correct_after_a_timeout(name, rows):
    """The first call times out (one workgroup held from the host); reading the
    error resets the handle, whose epochs then start over.  The next calls on
    the same handle must be correct: no word left by the failed call may pass
    for one of theirs.  c0 sums the router partials in every workgroup, c1 at 8
    rows reads the logits of the blocks' last chunks."""
    cfg = synth.CONFIGS[name].with_rows(rows)
    w = weights(name)
    x, r, _ = gapped_rows(cfg, w)
    o = oracle.moe_tail(x, r, w, cfg)
    dw = device_weights(name)
    h = handle_for(cfg, deadline_us=20000, debug_flags=binding.DEBUG_STALL_ONCE, debug_block=3)
    run(h, cfg, dw, x, r)
    assert h.get_error() == binding.ETIMEOUT
    for _ in range(2):
        g = run(h, cfg, dw, x, r)
        assert h.get_error() == binding.OK
        check_against_oracle(g, o, cfg)
