"""moe_tail_run_noalloc (the entry point with no handle and no allocation)
against moe_tail_run on a handle: the same kernels on the same inputs must give
the same bits, call after call, when the second call is smaller, when the
configuration changes between calls, and inside a captured graph."""
import sys

import numpy as np
import pytest

from cases import gapped_rows, weights
from decode_moe_layer_amd import binding, synth
from gpu_harness import dev, device_weights, handle_for, run

pytestmark = pytest.mark.gpu

KEYS = ("out", "res_out", "ids", "w", "logits", "y_routed", "y_shared")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _config(cfg, max_rows):
    return binding.make_config(max_rows, cfg.hidden, cfg.experts, cfg.topk, cfg.inter, cfg.shared_inter,
                               cfg.scoring, cfg.eps, n_group=cfg.n_group, topk_group=cfg.topk_group,
                               routed_scale=cfg.routed_scale, weight_format=cfg.weight_format,
                               fold_norm=cfg.fold_norm)


def run_noalloc(cfg, max_rows, dw, x, r):
    t = __import__("torch")
    R, H, E, K = x.shape[0], cfg.hidden, cfg.experts, cfg.topk
    o = {
        "out": t.empty((R, H), dtype=t.int16, device="cuda"),
        "res_out": t.empty((R, H), dtype=t.int16, device="cuda"),
        "ids": t.full((R, K), -1, dtype=t.int32, device="cuda"),
        "w": t.empty((R, K), dtype=t.float32, device="cuda"),
        "logits": t.empty((R, E), dtype=t.float32, device="cuda"),
        "y_routed": t.empty((R, H), dtype=t.float32, device="cuda"),
        "y_shared": t.empty((R, H), dtype=t.float32, device="cuda"),
    }
    binding.run_noalloc(_config(cfg, max_rows), R, dev(x), dev(r) if r is not None else None, dw["gamma"],
                        dw["router_w"], dw.get("router_bias"), dw["w13_q"], dw["w13_s"], dw["w2_q"], dw["w2_s"],
                        dw.get("ws13"), dw.get("ws2"), o["out"], o["res_out"], o["ids"], o["w"], o["logits"],
                        o["y_routed"], o["y_shared"], shared_gate=dw.get("shared_gate"))
    t.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in o.items()}
    res["out"] = res["out"].view(np.uint16)
    res["res_out"] = res["res_out"].view(np.uint16)
    return res


def _same(a, b, what):
    for k in KEYS:
        np.testing.assert_array_equal(a[k], b[k], err_msg="%s: %s" % (what, k))


def test_noalloc_matches_the_handle_twice_then_smaller():
    cfg = synth.CONFIGS["c2"]
    _say("noalloc c2 8 rows, then 3 rows")
    w = weights("c2")
    x, r, _ = gapped_rows(cfg, w)
    dw = device_weights("c2")
    h = handle_for(cfg)
    ref8 = run(h, cfg, dw, x, r)
    ref3 = run(h, cfg, dw, x[:3], r[:3], rows=3)
    assert h.get_error() == binding.OK
    _same(run_noalloc(cfg, 8, dw, x, r), ref8, "first call, 8 rows")
    _same(run_noalloc(cfg, 8, dw, x[:3], r[:3]), ref3, "second call, 3 rows")
    _same(run_noalloc(cfg, 8, dw, x, r), ref8, "third call, 8 rows again")
    h.close()


def test_noalloc_across_configurations():
    """The scratch layout changes with the configuration; successive calls on
    one device must not see each other's words."""
    seq = [("c0", 1), ("c4", 16), ("c3", 4), ("c0", 1), ("c1", 2)]
    refs = {}
    for name, rows in seq:
        cfg = synth.CONFIGS[name].with_rows(rows)
        w = weights(name)
        x, r, _ = gapped_rows(cfg, w)
        dw = device_weights(name)
        if name not in refs:
            h = handle_for(cfg)
            refs[name] = run(h, cfg, dw, x, r)
            assert h.get_error() == binding.OK
            h.close()
        _say("noalloc", name, rows)
        _same(run_noalloc(cfg, rows, dw, x, r), refs[name], name)


@pytest.mark.parametrize("name,rows", [("c0", 24), ("c1", 32)])
def test_noalloc_above_16_rows(name, rows):
    """More than 16 rows without a handle: c0's wide-launch scratch fits the
    static array, c1's at 32 rows does not, so that call runs as narrow
    launches.  Both give the handle's (wide launch) bits."""
    cfg = synth.CONFIGS[name].with_rows(rows)
    _say("noalloc above 16 rows", name, rows)
    w = weights(name)
    x, r, _ = gapped_rows(cfg, w)
    dw = device_weights(name)
    h = handle_for(cfg, max_rows=32)
    ref = run(h, cfg, dw, x, r)
    assert h.get_error() == binding.OK
    h.close()
    _same(run_noalloc(cfg, 32, dw, x, r), ref, "%s %d rows" % (name, rows))


def test_noalloc_in_a_captured_graph():
    t = pytest.importorskip("torch")
    cfg = synth.CONFIGS["c1"].with_rows(8)
    w = weights("c1")
    x, r, _ = gapped_rows(cfg, w)
    dw = device_weights("c1")
    h = handle_for(cfg)
    widths = [8, 2, 5]
    eager = [run(h, cfg, dw, x[:n], r[:n], rows=n, debug=False)["out"] for n in widths]
    h.close()
    xd, rd = dev(x), dev(r)
    outs = [t.empty((n, cfg.hidden), dtype=t.int16, device="cuda") for n in widths]
    c = _config(cfg, 8)
    s = t.cuda.Stream()
    g = t.cuda.CUDAGraph()
    with t.cuda.stream(s):
        with t.cuda.graph(g, stream=s):
            for n, o in zip(widths, outs):
                binding.run_noalloc(c, n, xd[:n], rd[:n], dw["gamma"], dw["router_w"], None, dw["w13_q"], dw["w13_s"],
                                    dw["w2_q"], dw["w2_s"], dw["ws13"], dw["ws2"], o, stream=s.cuda_stream)
    for rep in range(6):
        for o in outs:
            o.fill_(0)
        with t.cuda.stream(s):
            g.replay()
        s.synchronize()
        for n, o, e in zip(widths, outs, eager):
            np.testing.assert_array_equal(o.cpu().numpy().view(np.uint16), e, err_msg="replay %d rows %d" % (rep, n))
        # eager work of the program's own between replays
        run_noalloc(cfg, 8, dw, x[:1], r[:1])


def test_noalloc_refuses_what_does_not_fit_or_needs_a_handle():
    cfg = synth.CONFIGS["c0"]
    w = weights("c0")
    x, r, _ = gapped_rows(cfg, w)
    dw = device_weights("c0")
    # 288 shared blocks x 8 K-chunks of router/shared partials: about 5 MB of scratch
    big = binding.make_config(8, 6144, 512, 10, 256, 2048)
    with pytest.raises(binding.MoeTailError) as ei:
        binding.run_noalloc(big, 1, dev(x), dev(r), dw["gamma"], dw["router_w"], None, dw["w13_q"], dw["w13_s"],
                            dw["w2_q"], dw["w2_s"], dw["ws13"], dw["ws2"], dw["gamma"])
    assert ei.value.status == binding.EINVAL and "scratch" in str(ei.value)
    once = _config(cfg, 1)
    once.debug_flags = binding.DEBUG_STALL_ONCE
    with pytest.raises(binding.MoeTailError) as ei:
        binding.run_noalloc(once, 1, dev(x), dev(r), dw["gamma"], dw["router_w"], None, dw["w13_q"], dw["w13_s"],
                            dw["w2_q"], dw["w2_s"], dw["ws13"], dw["ws2"], dw["gamma"])
    assert ei.value.status == binding.EINVAL
