"""The input generator: reproducible, with the stated shapes, value ranges and row structure."""
import numpy as np
import pytest

import oracle
from cases import GAP_REL, c2_rho, gapped_rows, key_gaps
from decode_moe_layer_amd import synth


def test_reproducible_and_shapes():
    cfg = synth.CONFIGS["c0"]
    a, b = synth.make_weights(cfg), synth.make_weights(cfg)
    for k in a:
        if a[k] is None:
            assert b[k] is None
            continue
        np.testing.assert_array_equal(a[k], b[k])
    E, H, I, Is = cfg.experts, cfg.hidden, cfg.inter, cfg.shared_inter
    assert a["w13_q"].shape == (E, 2 * I, H // 2) and a["w13_s"].shape == (E, 2 * I, H // 32)
    assert a["w2_q"].shape == (E, H, I // 2) and a["w2_s"].shape == (E, H, I // 32)
    assert a["ws13"].shape == (2 * Is, H) and a["ws2"].shape == (H, Is)
    x1, r1 = synth.make_rows(cfg)
    x2, r2 = synth.make_rows(cfg)
    np.testing.assert_array_equal(x1, x2)
    np.testing.assert_array_equal(r1, r2)
    x3, _ = synth.make_rows(cfg, attempts=[1])
    assert not np.array_equal(x1, x3)


def test_value_ranges():
    cfg = synth.CONFIGS["c0"]
    w = synth.make_weights(cfg)
    lo, hi = w["w13_q"] & 0xF, w["w13_q"] >> 4
    counts = np.bincount(np.concatenate([lo.ravel(), hi.ravel()]), minlength=16)
    assert counts.min() > 0.9 * counts.mean()  # every code drawn, about uniformly
    assert w["w13_s"].min() == 121 and w["w13_s"].max() == 124
    assert w["w2_s"].min() == 121 and w["w2_s"].max() == 124
    g = synth.bf16_bits_to_f32(w["gamma"])
    assert g.min() >= 0.5 and g.max() <= 1.5
    std = synth.bf16_bits_to_f32(w["router_w"]).std()
    assert abs(std * np.sqrt(cfg.hidden) - 1) < 0.05


def test_heavy_tail_channels():
    cfg = synth.CONFIGS["c4"]
    ch = synth.heavy_channels(cfg)
    assert ch.size == 82 and len(set(ch.tolist())) == 82
    x, _ = synth.make_rows(cfg.with_rows(2))
    xf = np.abs(synth.bf16_bits_to_f32(x))
    mask = np.zeros(cfg.hidden, bool)
    mask[ch] = True
    assert xf[:, mask].mean() > 10 * xf[:, ~mask].mean()


def test_sigmoid_bias_std():
    cfg = synth.CONFIGS["c3"]
    rw = synth.make_router_weights(cfg)
    assert rw["router_bias"].dtype == np.float32 and abs(rw["router_bias"].std() - 0.1) < 0.02


@pytest.mark.parametrize("name", ["c0", "c1", "c3"])
def test_gapped_rows_pass_the_gap(name):
    cfg = synth.CONFIGS[name]
    rw = synth.make_router_weights(cfg)
    x, r, _ = gapped_rows(cfg, rw)
    _, ky = oracle.router_keys(x, r, rw, cfg)
    assert np.all(key_gaps(ky, cfg.topk) >= GAP_REL)


def test_similar_rows_repeat_about_30_percent():
    cfg = synth.CONFIGS["c2"]
    rw = synth.make_router_weights(cfg)
    x, r, _ = gapped_rows(cfg, rw, rho=c2_rho())
    _, ky = oracle.router_keys(x, r, rw, cfg)
    picks = np.concatenate([oracle.topk(ky[i], cfg.topk) for i in range(cfg.rows)])
    frac = 1 - len(set(picks.tolist())) / picks.size
    assert 0.27 <= frac <= 0.33


def test_mxfp8_codes_are_never_nan_and_cover_every_other_code():
    """MXFP8 expert codes are drawn uniformly over the 254 E4M3 codes that are
    not NaN (0x7F and 0xFF, OCP MX v1.0), in the one-byte-per-element layouts
    [E, 2I, H] and [E, H, I]; the scales keep the MXFP4 shapes."""
    import dataclasses

    cfg = dataclasses.replace(synth.CONFIGS["c0"], weight_format=1)
    w = synth.make_weights(cfg)
    E, H, I = cfg.experts, cfg.hidden, cfg.inter
    assert w["w13_q"].shape == (E, 2 * I, H) and w["w2_q"].shape == (E, H, I)
    assert w["w13_s"].shape == (E, 2 * I, H // 32) and w["w2_s"].shape == (E, H, I // 32)
    codes = np.concatenate([w["w13_q"].ravel(), w["w2_q"].ravel()])
    counts = np.bincount(codes, minlength=256)
    assert counts[0x7F] == 0 and counts[0xFF] == 0
    assert np.count_nonzero(counts) == 254
    assert counts.max() < 2 * counts[counts > 0].min()  # roughly uniform


def test_unit_blocked_w13_is_the_documented_permutation():
    """The unit-blocked layout puts, for every (unit, column group, lane), the
    lane's 16 bytes of its unit row at ((b * H/128 + c) * 64 + l) * 16."""
    cfg = synth.CONFIGS["c0"]
    w = synth.make_weights(cfg)["w13_q"]
    I, H = cfg.inter, cfg.hidden
    s = synth.w13_unit_blocked(w, I).reshape(w.shape[0], -1)
    T2 = H // 128
    for e in (0, w.shape[0] - 1):
        for b in range(I // 8):
            for c in range(T2):
                for lane in (0, 7, 8, 15, 16, 37, 63):
                    i, q = lane & 15, lane >> 4
                    row = b * 8 + i if i < 8 else I + b * 8 + i - 8
                    off = ((b * T2 + c) * 64 + lane) * 16
                    assert np.array_equal(s[e, off:off + 16], w[e, row, c * 64 + q * 16:c * 64 + q * 16 + 16])
    assert sorted(s.ravel().tolist()) == sorted(w.ravel().tolist())
