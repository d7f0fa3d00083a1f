"""Device-side helpers for the GPU tests: upload seeded inputs, call the C ABI, fetch results."""
import functools

import numpy as np

from decode_moe_layer_amd import binding, synth


def torch():
    import torch as _t

    return _t


def dev(a, device="cuda"):
    t = torch()
    if a is None:
        return None
    if a.dtype == np.uint16:
        return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)
    return t.from_numpy(np.ascontiguousarray(a)).to(device)


@functools.lru_cache(maxsize=2)
def device_weights(name: str):
    from cases import weights

    w = weights(name)
    return {k: dev(v) for k, v in w.items()}


def handle_for(cfg, max_rows=None, **kw):
    c = binding.make_config(max_rows or cfg.rows, cfg.hidden, cfg.experts, cfg.topk, cfg.inter, cfg.shared_inter,
                            cfg.scoring, cfg.eps, n_group=cfg.n_group, topk_group=cfg.topk_group,
                            routed_scale=cfg.routed_scale, weight_format=cfg.weight_format,
                            fold_norm=cfg.fold_norm, **kw)
    return binding.MoeTail(c)


def run(handle, cfg, dw, x, r, rows=None, stream=None, debug=True, front=None):
    """One call; returns a dict of numpy outputs.  front = (attn, w_o) device
    tensors runs the out_proj front instead of passing x (x may then be None)."""
    t = torch()
    R = (x.shape[0] if front is None else front[0].shape[0]) if rows is None else rows
    H, E, K = cfg.hidden, cfg.experts, cfg.topk
    xd, rd = (dev(x) if x is not None else None), dev(r) if r is not None else None
    o = {
        "out": t.empty((R, H), dtype=t.int16, device="cuda"),
        "res_out": t.empty((R, H), dtype=t.int16, device="cuda"),
        "ids": t.full((R, K), -1, dtype=t.int32, device="cuda"),
        "w": t.empty((R, K), dtype=t.float32, device="cuda"),
    }
    if debug:
        o["logits"] = t.empty((R, E), dtype=t.float32, device="cuda")
        o["y_routed"] = t.empty((R, H), dtype=t.float32, device="cuda")
        o["y_shared"] = t.empty((R, H), dtype=t.float32, device="cuda")
    handle.run(R, xd, rd, dw["gamma"], dw["router_w"], dw.get("router_bias"), dw["w13_q"], dw["w13_s"], dw["w2_q"],
               dw["w2_s"], dw.get("ws13"), dw.get("ws2"), o["out"], o["res_out"], o["ids"], o["w"],
               o.get("logits"), o.get("y_routed"), o.get("y_shared"), stream=stream,
               shared_gate=dw.get("shared_gate"), attn=None if front is None else front[0],
               w_o=None if front is None else front[1])
    t.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in o.items()}
    res["out"] = res["out"].view(np.uint16)
    res["res_out"] = res["res_out"].view(np.uint16)
    return res


def rel_l2(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def row_cos(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return np.sum(a * b, axis=1) / np.maximum(np.linalg.norm(a, axis=1) * np.linalg.norm(b, axis=1), 1e-300)


def bf(a):
    return synth.bf16_bits_to_f32(a).astype(np.float64)


def check_against_oracle(g, o, cfg, tol=1e-2):
    """The parity bar: ids bit-exact as sets (order where keys are apart), weights 1e-5,
    res_out bitwise, y_routed / y_shared / out rel-L2 <= 1e-2, per-row cosine >= 0.999."""
    R, K = g["ids"].shape
    for r in range(R):
        assert set(g["ids"][r].tolist()) == set(o["ids"][r].tolist()), (r, g["ids"][r], o["ids"][r])
        ky = o["keys"][r]
        for k in range(K - 1):
            a, b = ky[o["ids"][r][k]], ky[o["ids"][r][k + 1]]
            if (a - b) >= 1e-4 * max(abs(a), abs(b)):
                assert g["ids"][r][k] == o["ids"][r][k], (r, k, g["ids"][r], o["ids"][r])
        # weights, matched by expert id
        wo = dict(zip(o["ids"][r].tolist(), o["w"][r].tolist()))
        for e, wv in zip(g["ids"][r].tolist(), g["w"][r].tolist()):
            assert abs(wv - wo[e]) <= 1e-5 * abs(wo[e]) + 1e-7, (r, e, wv, wo[e])
    np.testing.assert_array_equal(g["res_out"], o["h"])
    if "logits" in g:
        err = np.abs(g["logits"] - o["logits"]).max()
        assert err <= 1e-4 * np.abs(o["logits"]).max() + 1e-6, err
        assert rel_l2(g["y_routed"], o["y_routed"]) <= tol
        if cfg.shared_inter:
            assert rel_l2(g["y_shared"], o["y_shared"]) <= tol
    assert rel_l2(bf(g["out"]), bf(o["out"])) <= tol
    assert np.all(row_cos(bf(g["out"]), bf(o["out"])) >= 0.999)
