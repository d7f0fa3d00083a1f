"""Parity of the HIP path with the CPU oracle on every workload, through the C ABI."""
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


def _grouped_rows(cfg, w, max_attempts=64):
    """Rows whose group ranking and kept top-k are both well posed: the
    topk_group-th and next group scores, and the K-th and next keys among the
    kept experts, differ by at least 1e-4 relative (oracle keys, double)."""
    from cases import GAP_REL, key_gaps

    gs = cfg.experts // cfg.n_group
    xs, rs = [], []
    for row in range(cfg.rows):
        for a in range(max_attempts):
            x, res = synth.make_row(cfg, row, a, 0.0)
            _, ky = oracle.router_keys(x[None], res[None], w, cfg)
            k = ky[0]
            sc = -np.sort(-k.reshape(cfg.n_group, gs), axis=1)[:, :2].sum(axis=1)
            s = np.sort(sc)[::-1]
            t = cfg.topk_group
            gap_g = np.inf if t >= cfg.n_group else (s[t - 1] - s[t]) / max(abs(s[t - 1]), abs(s[t]), 1e-300)
            kept = np.argsort(-sc, kind="stable")[:t]
            kk = np.concatenate([k[g * gs:(g + 1) * gs] for g in kept])
            if gap_g >= GAP_REL and key_gaps(kk[None], cfg.topk)[0] >= GAP_REL:
                break
        else:
            raise RuntimeError("no well-posed grouped row")
        xs.append(x)
        rs.append(res)
    return np.stack(xs), np.stack(rs)


@pytest.mark.parametrize("name,rows,n_group,topk_group,scale", [
    ("c0", 2, 2, 1, 1.0), ("c1", 8, 8, 3, 1.0), ("c3", 4, 8, 4, 2.5), ("c4", 16, 8, 4, 1.0)])
def test_parity_grouped_routing_and_routed_scale(name, rows, n_group, topk_group, scale):
    """Group-limited top-k and a routed scaling factor on the GPU against the
    oracle: one lane per group (c0), 8 lanes per group with softmax keys (c1
    at 8 rows), sigmoid keys with a selection bias and a scale of 2.5 (c3),
    and 6 lanes per group, not a power of two (c4's 384 experts in 8 groups
    at 16 rows)."""
    import dataclasses

    cfg = dataclasses.replace(synth.CONFIGS[name].with_rows(rows), n_group=n_group, topk_group=topk_group,
                              routed_scale=scale)
    _say("grouped", name, rows, n_group, topk_group, scale)
    w = weights(name)
    x, r = _grouped_rows(cfg, w)
    o = oracle.moe_tail(x, r, w, cfg)
    h = handle_for(cfg)
    g = run(h, cfg, device_weights(name), x, r)
    assert h.get_error() == 0
    check_against_oracle(g, o, cfg)
    gs = cfg.experts // n_group
    for row in range(rows):
        assert len({int(e) // gs for e in g["ids"][row]}) <= topk_group


@pytest.mark.parametrize("experts,n_group,topk_group,topk", [
    (192, 8, 3, 6), (320, 8, 2, 8), (384, 4, 2, 8), (64, 4, 2, 4), (96, 4, 1, 3)])
def test_parity_grouped_routing_any_group_width(experts, n_group, topk_group, topk):
    """Group-limited routing where a group spans a number of 8-expert lanes
    that is not a power of two (3, 5, 12 lanes) or is small (2, 3 lanes):
    every group's two largest keys must be found inside the group only."""
    import dataclasses

    from gpu_harness import dev

    cfg = dataclasses.replace(synth.Config("grp%d" % experts, 30 + experts % 97, 4, 1024, experts, topk, 64, 64),
                              n_group=n_group, topk_group=topk_group)
    _say("grouped width", experts, n_group, topk_group, topk)
    w = synth.make_weights(cfg)
    x, r = _grouped_rows(cfg, w)
    o = oracle.moe_tail(x, r, w, cfg)
    h = handle_for(cfg)
    g = run(h, cfg, {k: dev(v) for k, v in w.items()}, x, r)
    assert h.get_error() == 0
    check_against_oracle(g, o, cfg)
    gs = experts // n_group
    for row in range(cfg.rows):
        assert len({int(e) // gs for e in g["ids"][row]}) <= topk_group


@pytest.mark.parametrize("name,rows", [("c0", 1), ("c1", 8), ("c4", 16)])
def test_parity_mxfp8_experts(name, rows):
    """MXFP8 routed experts (E4M3 codes, one E8M0 scale per 32 elements; OCP
    Microscaling Formats v1.0) against the oracle on the three kernel paths:
    routed sums by every reader (c0), xn in LDS (c1 at 8 rows), xn read from
    global scratch (c4 at 16 rows)."""
    import dataclasses

    from gpu_harness import dev

    cfg = dataclasses.replace(synth.CONFIGS[name].with_rows(rows), weight_format=1)
    _say("mxfp8", name, rows)
    w = synth.make_weights(cfg)
    x, r, _ = gapped_rows(cfg, w)
    o = oracle.moe_tail(x, r, w, cfg)
    dw = {k: dev(v) for k, v in w.items()}
    h = handle_for(cfg)
    g = run(h, cfg, dw, x, r)
    assert h.get_error() == 0
    check_against_oracle(g, o, cfg)
    del dw, h


def _fp4_as_fp8(q):
    """Re-encode packed E2M1 codes (two per byte, low nibble first) as E4M3
    codes, one per byte; every E2M1 value is exact in E4M3."""
    to8 = np.array([0x00, 0x30, 0x38, 0x3C, 0x40, 0x44, 0x48, 0x4C], np.uint8)
    codes = np.stack([q & 0xF, q >> 4], axis=-1).reshape(q.shape[:-1] + (q.shape[-1] * 2,))
    return to8[codes & 7] | ((codes & 8) << 4).astype(np.uint8)


@pytest.mark.parametrize("name,rows", [("c0", 2), ("c1", 8)])
def test_mxfp8_matches_mxfp4_on_reencoded_weights(name, rows):
    """The same weights in both formats give the same GPU outputs bit for bit:
    the MXFP8 loads, strides and decode lane order match the MXFP4 ones."""
    import dataclasses

    from gpu_harness import dev

    cfg = synth.CONFIGS[name].with_rows(rows)
    cfg8 = dataclasses.replace(cfg, weight_format=1)
    _say("fp4-as-fp8", name, rows)
    w = weights(name)
    x, r, _ = gapped_rows(cfg, w)
    g4 = run(handle_for(cfg), cfg, device_weights(name), x, r)
    dw8 = dict(device_weights(name))
    dw8["w13_q"] = dev(_fp4_as_fp8(w["w13_q"]))
    dw8["w2_q"] = dev(_fp4_as_fp8(w["w2_q"]))
    h8 = handle_for(cfg8)
    g8 = run(h8, cfg8, dw8, x, r)
    assert h8.get_error() == 0
    for k in ("ids", "w", "logits", "y_routed", "y_shared", "out", "res_out"):
        np.testing.assert_array_equal(g8[k], g4[k], err_msg=k)


@pytest.mark.parametrize("name,rows", [("c0", 1), ("c1", 1), ("c1", 8), ("c3", 4), ("c4", 16)])
def test_parity_folded_norm(name, rows):
    """The norm folded into the router and shared gate/up sums (rstd applied
    after projecting bf16(h * gamma); "glm53: Long-context indexer ...", PR 85
    commit text) against the oracle's folded form, on every kernel path:
    routed sums by every reader (c0, c1 at 1 row), xn in LDS (c1 at 8 rows,
    c3 with sigmoid keys), xn from global scratch (c4 at 16 rows).  Rows are
    gap-checked on the folded keys."""
    import dataclasses

    cfg = dataclasses.replace(synth.CONFIGS[name].with_rows(rows), fold_norm=1)
    _say("fold", name, rows)
    w = weights(name)
    x, r, _ = gapped_rows(cfg, w)
    o = oracle.moe_tail(x, r, w, cfg)
    h = handle_for(cfg)
    g = run(h, cfg, device_weights(name), x, r)
    assert h.get_error() == 0
    check_against_oracle(g, o, cfg)
    plain = oracle.moe_tail(x, r, w, synth.CONFIGS[name].with_rows(rows))
    assert not np.array_equal(plain["logits"], o["logits"])  # the fold changed the logits


@pytest.mark.parametrize("name,rows,n_group,topk_group", [("c3", 4, 8, 4), ("c1", 8, 8, 3)])
def test_parity_every_option_together(name, rows, n_group, topk_group):
    """MXFP8 experts, the folded norm, group-limited routing with a routed
    scale of 2.5 and a shared gate in one call, against the oracle: the
    optional steps compose (c3: sigmoid keys with a bias, xn in LDS; c1 at 8
    rows: softmax keys)."""
    import dataclasses

    from gpu_harness import dev

    cfg = dataclasses.replace(synth.CONFIGS[name].with_rows(rows), weight_format=1, fold_norm=1, n_group=n_group,
                              topk_group=topk_group, routed_scale=2.5)
    _say("all options", name, rows, n_group, topk_group)
    w = dict(synth.make_weights(cfg))
    w["shared_gate"] = synth.make_shared_gate(cfg)
    x, r = _grouped_rows(cfg, w)
    o = oracle.moe_tail(x, r, w, cfg)
    dw = {k: dev(v) for k, v in w.items()}
    h = handle_for(cfg)
    g = run(h, cfg, dw, x, r)
    assert h.get_error() == 0
    check_against_oracle(g, o, cfg)
    gs = cfg.experts // n_group
    for row in range(rows):
        assert len({int(e) // gs for e in g["ids"][row]}) <= topk_group
    del dw, h


@pytest.mark.parametrize("name,rows,max_rows", [("c1", 32, 32), ("c3", 20, 24), ("c0", 17, 32)])
def test_parity_above_16_rows(name, rows, max_rows):
    """More rows than a narrow launch's 16 MFMA columns (MTP verify batches)
    run as one wide launch: parity with the oracle on every row, and the first
    rows (the first range of the narrow-launch split) equal a call on those
    rows alone, bit for bit."""
    cfg = synth.CONFIGS[name].with_rows(rows)
    _say("rows", name, rows, "max_rows", max_rows)
    w = weights(name)
    x, r, _ = gapped_rows(cfg, w)
    o = oracle_rows(x, r, w, cfg)
    h = handle_for(cfg, max_rows=max_rows)
    g = run(h, cfg, device_weights(name), x, r)
    assert h.get_error() == 0
    check_against_oracle(g, o, cfg)
    n = (rows + 15) // 16
    r1 = rows // n
    g1 = run(h, cfg.with_rows(r1), device_weights(name), x[:r1], r[:r1])
    for k in ("ids", "w", "out", "res_out", "y_routed", "y_shared", "logits"):
        np.testing.assert_array_equal(g[k][:r1], g1[k], err_msg=k)


@pytest.mark.parametrize("name,rows", [("c0", 2), ("c1", 8), ("c3", 4), ("c4", 16), ("c1", 24)])
def test_unit_blocked_w13_matches_row_major(name, rows):
    """The same MXFP4 gate/up codes in the unit-blocked layout give the same
    GPU outputs, bit for bit, as in the row-major one (every kernel path:
    routed sums by every reader, xn in LDS, sigmoid keys, xn from global,
    a wide launch)."""
    from gpu_harness import dev

    cfg = synth.CONFIGS[name].with_rows(rows)
    _say("unit-blocked", name, rows)
    w = weights(name)
    x, r, _ = gapped_rows(cfg, w)
    g0 = run(handle_for(cfg), cfg, device_weights(name), x, r)
    dws = dict(device_weights(name))
    dws["w13_q"] = dev(synth.w13_unit_blocked(w["w13_q"], cfg.inter))
    h = handle_for(cfg, w13_layout=1)
    g1 = run(h, cfg, dws, x, r)
    assert h.get_error() == 0
    for k in ("ids", "w", "logits", "y_routed", "y_shared", "out", "res_out"):
        np.testing.assert_array_equal(g1[k], g0[k], err_msg=k)
    del dws, h
