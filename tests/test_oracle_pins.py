"""Pins of the CPU oracle against facts it does not compute itself.

Each test fixes one part of the oracle by a closed form, a textbook or library
routine, a brute force or an invariant, chosen so that a plausible slip (a
dropped term, a swapped nibble, a transposed operand, a wrong sign) fails.
"""
import itertools
import math

import numpy as np
import pytest
import scipy.special

import oracle
from decode_moe_layer_amd import synth

# ---------------------------------------------------------------- formats ----


def e2m1_from_bits(code: int) -> float:
    """FP4 E2M1 by its bit fields (OCP MX v1.0): 1 sign, 2 exponent (bias 1), 1 mantissa bit."""
    s, e, m = (code >> 3) & 1, (code >> 1) & 3, code & 1
    mag = (m * 0.5) if e == 0 else (2.0 ** (e - 1)) * (1.0 + 0.5 * m)
    return -mag if s else mag


@pytest.mark.parametrize("scale", [0, 121, 122, 123, 124, 127, 254])
def test_mxfp4_dequant_all_16_codes(scale):
    for code in range(16):
        want = e2m1_from_bits(code) * math.ldexp(1.0, scale - 127)
        got = oracle.dequant(code, scale)
        assert got == want, (code, scale, got, want)
    # +0 and -0: distinct bit patterns, equal values
    assert oracle.e2m1(0) == 0.0 and oracle.e2m1(8) == 0.0
    assert math.copysign(1.0, oracle.e2m1(8)) == -1.0
    assert math.isnan(oracle.e8m0(255))


def test_e2m1_magnitudes_are_the_spec_set():
    assert sorted({abs(e2m1_from_bits(c)) for c in range(16)}) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_bf16_round_matches_float32_route():
    """Double -> bf16 (oracle) equals float32 -> bf16 (generator) on float32-exact values."""
    rng = np.random.default_rng(1)
    f = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),  # subnormal range
        np.array([1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, -(1.0 + 2.0**-8), 3.3895313892515355e38, 1e-45], np.float32),
    ])
    # exact ties: bf16 value + half a bf16 ulp
    base = synth.to_bf16_bits(rng.standard_normal(2000).astype(np.float32))
    ties = ((base.astype(np.uint32) << 16) | 0x8000).view(np.float32)
    f = np.concatenate([f, ties])
    want = synth.to_bf16_bits(f)
    got = np.array([oracle.bf16_round(float(v)) for v in f], dtype=np.uint16)
    np.testing.assert_array_equal(got, want)
    assert oracle.bf16_round(1.0 + 2.0**-8) == 0x3F80  # tie to even (down)
    assert oracle.bf16_round(1.0 + 3 * 2.0**-8) == 0x3F82  # tie to even (up)
    assert oracle.bf16_round(2.0**129) == 0x7F80  # overflow


def test_bf16_round_double_rounding_not_used():
    # 1 + 2^-8 + 2^-30 is above the tie: must round up even though float32 would make it a tie
    assert oracle.bf16_round(1.0 + 2.0**-8 + 2.0**-30) == 0x3F81


# ------------------------------------------------------------------ top-k ----


def brute_topk_set(keys, K):
    """The unique K-set S with: every i in S beats every j outside (larger key, or equal and lower id)."""
    E = len(keys)
    found = []
    for S in itertools.combinations(range(E), K):
        Sset = set(S)
        ok = all(keys[i] > keys[j] or (keys[i] == keys[j] and i < j) for i in S for j in range(E) if j not in Sset)
        if ok:
            found.append(S)
    assert len(found) == 1
    return set(found[0])


@pytest.mark.parametrize("E,K", [(4, 1), (5, 2), (8, 3), (10, 4), (12, 4), (6, 6)])
def test_topk_brute_force(E, K):
    rng = np.random.default_rng(E * 100 + K)
    for trial in range(40):
        if trial % 2:
            keys = rng.integers(-2, 3, size=E).astype(np.float64)  # many exact ties
        else:
            keys = rng.standard_normal(E)
        ids = oracle.topk(keys, K)
        assert set(ids.tolist()) == brute_topk_set(keys, K)
        # listed by key descending, id ascending
        for a, b in zip(ids[:-1], ids[1:]):
            assert keys[a] > keys[b] or (keys[a] == keys[b] and a < b)


def test_topk_ties_go_to_lower_id():
    keys = np.array([1.0, 3.0, 3.0, 2.0, 3.0])
    assert oracle.topk(keys, 2).tolist() == [1, 2]
    assert oracle.topk(keys, 3).tolist() == [1, 2, 4]


# ---------------------------------------------------------------- weights ----


def test_softmax_weights_full_k_is_textbook_softmax():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal(16) * 3
    ids = np.arange(16, dtype=np.int32)
    np.testing.assert_allclose(oracle.topk_weights(lg, ids, synth.SOFTMAX), scipy.special.softmax(lg), rtol=1e-14)


def test_weights_sum_to_one_and_k1():
    rng = np.random.default_rng(4)
    for scoring in (synth.SOFTMAX, synth.SIGMOID_BIAS):
        for K in (1, 2, 8, 10):
            lg = rng.standard_normal(64) * 4
            ids = rng.choice(64, K, replace=False).astype(np.int32)
            w = oracle.topk_weights(lg, ids, scoring)
            assert abs(w.sum() - 1.0) < 1e-12
            assert np.all(w > 0)
            if K == 1:
                assert w[0] == 1.0


def test_sigmoid_weights_closed_forms():
    # two experts at +t and -t: sigmoid(t) + sigmoid(-t) = 1, so w = (sigmoid(t), sigmoid(-t))
    for t in (0.0, 0.3, 2.5, -1.7):
        w = oracle.topk_weights(np.array([t, -t]), np.array([0, 1], np.int32), synth.SIGMOID_BIAS)
        assert abs(w[0] - scipy.special.expit(t)) < 1e-15 and abs(w[1] - scipy.special.expit(-t)) < 1e-15
    # equal logits: uniform weights in both modes
    for scoring in (synth.SOFTMAX, synth.SIGMOID_BIAS):
        w = oracle.topk_weights(np.full(8, 0.7), np.arange(5, dtype=np.int32), scoring)
        np.testing.assert_allclose(w, 0.2, rtol=1e-15)


def test_sigmoid_keys_use_bias_for_selection_only():
    lg = np.array([0.0, 0.1, 0.2, 0.3])
    bias = np.array([0.0, 0.0, 0.0, -1.0], np.float32)
    ky = oracle.keys(lg, synth.SIGMOID_BIAS, bias)
    assert oracle.topk(ky, 2).tolist() == [2, 1]  # expert 3 has the largest logit but a -1 bias
    # with zero bias, sigmoid selection equals logit selection (sigmoid is monotone)
    rng = np.random.default_rng(5)
    lg = rng.standard_normal(40)
    ky0 = oracle.keys(lg, synth.SIGMOID_BIAS, np.zeros(40, np.float32))
    assert oracle.topk(ky0, 7).tolist() == oracle.topk(lg, 7).tolist()
    np.testing.assert_allclose(ky0, scipy.special.expit(lg), rtol=1e-15)


# ------------------------------------------------------------------- norm ----


def bf16(v):
    return synth.to_bf16_bits(np.asarray(v, np.float32))


def test_residual_add_rounds_once():
    rng = np.random.default_rng(6)
    H = 256
    x = bf16(rng.standard_normal(H))
    r = bf16(rng.standard_normal(H) * 10 ** rng.uniform(-6, 2, H))
    h, _, _ = oracle.norm_row(x, r, bf16(np.ones(H)), 1e-6)
    # a bf16 + bf16 sum is exact or harmlessly rounded in float32, then rounded to bf16 once
    want = bf16(synth.bf16_bits_to_f32(x) + synth.bf16_bits_to_f32(r))
    np.testing.assert_array_equal(h, want)
    h2, _, _ = oracle.norm_row(x, None, bf16(np.ones(H)), 1e-6)
    np.testing.assert_array_equal(h2, x)


def test_rmsnorm_constant_row_closed_form():
    H = 512
    for c in (1.0, 0.5, 3.0):
        x = bf16(np.full(H, c))
        gamma = bf16(np.linspace(0.5, 1.5, H))
        _, xn, rstd = oracle.norm_row(x, None, gamma, 1e-6)
        assert rstd == 1.0 / math.sqrt(c * c + float(np.float32(1e-6)))
        g = synth.bf16_bits_to_f32(gamma).astype(np.float64)
        want = np.array([oracle.bf16_round(c * rstd * gi) for gi in g], np.uint16)
        np.testing.assert_array_equal(xn, want)


def test_rmsnorm_is_scale_invariant_without_eps():
    rng = np.random.default_rng(7)
    H = 1024
    x = bf16(rng.standard_normal(H))
    gamma = bf16(rng.uniform(0.5, 1.5, H))
    _, xn, _ = oracle.norm_row(x, None, gamma, 0.0)
    for k in (-3, 1, 5):
        xk = bf16(synth.bf16_bits_to_f32(x) * np.float32(2.0**k))
        _, xnk, _ = oracle.norm_row(xk, None, gamma, 0.0)
        np.testing.assert_array_equal(xnk, xn)
    # the normalised row has mean square 1 before the gamma multiply and rounding
    _, xn1, _ = oracle.norm_row(x, None, bf16(np.ones(H)), 0.0)
    ms = np.mean(synth.bf16_bits_to_f32(xn1).astype(np.float64) ** 2)
    assert abs(ms - 1.0) < 1e-2


# --------------------------------------------------------- expert / layer ----


def _cfg(H, E, K, I, Is, scoring=synth.SOFTMAX):
    return synth.Config("pin", 99, 1, H, E, K, I, Is, scoring=scoring)


def _zero_weights(cfg):
    E, H, I, Is = cfg.experts, cfg.hidden, cfg.inter, cfg.shared_inter
    return {
        "gamma": bf16(np.ones(H)),
        "router_w": bf16(np.zeros((E, H))),
        "router_bias": None if cfg.scoring == synth.SOFTMAX else np.zeros(E, np.float32),
        "w13_q": np.zeros((E, 2 * I, H // 2), np.uint8),
        "w13_s": np.full((E, 2 * I, H // 32), 127, np.uint8),
        "w2_q": np.zeros((E, H, I // 2), np.uint8),
        "w2_s": np.full((E, H, I // 32), 127, np.uint8),
        "ws13": bf16(np.zeros((2 * Is, H))) if Is else None,
        "ws2": bf16(np.zeros((H, Is))) if Is else None,
    }


def silu(t):
    return t / (1.0 + math.exp(-t))


def test_one_expert_one_row_closed_form():
    """E = K = 1, no shared expert, x = 1, r = 0, gamma = 1: xn = 1 exactly, so
    g_i = H v_g[i] 2^(s_g-127), u_i = H v_u[i] 2^(s_u-127), out_h = bf16(1 + v_d[h] 2^(s_d-127) sum_i silu(g_i) u_i)."""
    H, I = 256, 64
    cfg = _cfg(H, 1, 1, I, 0)
    w = _zero_weights(cfg)
    rng = np.random.default_rng(8)
    cg = rng.integers(0, 16, I)
    cu = rng.integers(0, 16, I)
    cd = rng.integers(0, 16, H)
    sg, su, sd = 120, 118, 122
    for i in range(I):
        w["w13_q"][0, i, :] = cg[i] | (cg[i] << 4)
        w["w13_q"][0, I + i, :] = cu[i] | (cu[i] << 4)
    w["w13_s"][0, :I, :] = sg
    w["w13_s"][0, I:, :] = su
    for h in range(H):
        w["w2_q"][0, h, :] = cd[h] | (cd[h] << 4)
    w["w2_s"][0] = sd
    x = bf16(np.ones((1, H)))
    o = oracle.moe_tail(x, None, w, cfg)
    assert np.all(o["xn"] == 0x3F80)
    acc = 0.0
    for i in range(I):
        g = H * e2m1_from_bits(cg[i]) * 2.0 ** (sg - 127)
        u = H * e2m1_from_bits(cu[i]) * 2.0 ** (su - 127)
        acc += silu(g) * u
    d = np.array([e2m1_from_bits(cd[h]) * 2.0 ** (sd - 127) * acc for h in range(H)])
    np.testing.assert_allclose(o["y_routed"][0], d, rtol=1e-12, atol=1e-300)
    want = np.array([oracle.bf16_round(1.0 + v) for v in d], np.uint16)
    np.testing.assert_array_equal(o["out"][0], want)
    assert o["ids"][0, 0] == 0 and o["w"][0, 0] == 1.0


@pytest.mark.parametrize("k", [0, 1, 30, 31, 32, 33, 200, 255])
def test_one_hot_probe_pins_nibble_order_and_scale_blocks(k):
    """x = e_k reads column k of W13 only: one nonzero nibble at (row i, column k)
    gives g_i != 0 exactly when the probe hits that column; its block scale is s[i][k//32]."""
    H, I = 256, 32
    cfg = _cfg(H, 1, 1, I, 0)
    w = _zero_weights(cfg)
    i = 5
    code = 6  # 4.0
    byte = code << 4 if (k % 2) else code  # odd columns live in the high nibble
    w["w13_q"][0, i, k // 2] = byte
    w["w13_s"][0, i, :] = 100
    w["w13_s"][0, i, k // 32] = 130  # only the block of column k carries this scale
    w["w13_q"][0, I + i, :] = 0x22  # up row i: every element 1.0 x 2^0
    w["w2_q"][0, :, :] = 0x22  # down: every element 1.0
    for probe in (k, k ^ 1, (k + 32) % H):
        x = np.zeros((1, H), np.uint16)
        x[0, probe] = 0x3F80  # 1.0
        o = oracle.moe_tail(x, None, w, cfg)
        xn_p = synth.bf16_bits_to_f32(o["xn"][0, probe:probe + 1])[0]
        rstd = 1.0 / math.sqrt(1.0 / H + float(np.float32(1e-6)))
        assert xn_p == synth.bf16_bits_to_f32(np.array([oracle.bf16_round(rstd)], np.uint16))[0]
        g = (4.0 * 2.0 ** 3 * xn_p) if probe == k else 0.0
        u = xn_p  # 1.0 * xn_p
        a_i = silu(g) * u
        np.testing.assert_allclose(o["y_routed"][0], np.full(H, a_i), rtol=1e-14, atol=1e-300)


def test_routed_expert_matches_dense_matmul():
    """Dequantise by bit fields, then numpy matmuls: the same expert FFN on random codes."""
    H, I = 256, 64
    cfg = _cfg(H, 3, 1, I, 0)
    rng = np.random.default_rng(9)
    w = _zero_weights(cfg)
    w["w13_q"][:] = rng.integers(0, 256, w["w13_q"].shape, dtype=np.uint8)
    w["w13_s"][:] = rng.integers(121, 125, w["w13_s"].shape, dtype=np.uint8)
    w["w2_q"][:] = rng.integers(0, 256, w["w2_q"].shape, dtype=np.uint8)
    w["w2_s"][:] = rng.integers(121, 125, w["w2_s"].shape, dtype=np.uint8)
    w["router_w"] = bf16(np.zeros((3, H)))
    w["router_w"][2, :] = 0x3F80  # expert 2 wins for a positive row
    x = bf16(np.abs(rng.standard_normal((1, H))) + 0.1)
    o = oracle.moe_tail(x, None, w, cfg)
    assert o["ids"][0, 0] == 2
    lut = np.array([e2m1_from_bits(c) for c in range(16)])

    def deq(q, s):
        lo, hi = lut[q & 0xF], lut[q >> 4]
        v = np.stack([lo, hi], axis=-1).reshape(q.shape[0], -1)
        return v * np.repeat(2.0 ** (s.astype(np.float64) - 127), 32, axis=1)

    W13 = deq(w["w13_q"][2], w["w13_s"][2])
    W2 = deq(w["w2_q"][2], w["w2_s"][2])
    xn = synth.bf16_bits_to_f32(o["xn"][0]).astype(np.float64)
    gu = W13 @ xn
    a = gu[:I] * scipy.special.expit(gu[:I]) * gu[I:]
    np.testing.assert_allclose(o["y_routed"][0], W2 @ a, rtol=1e-10, atol=1e-12)


def test_shared_expert_matches_dense_matmul():
    H, Is = 256, 64
    cfg = _cfg(H, 2, 1, 32, Is)
    rng = np.random.default_rng(10)
    w = _zero_weights(cfg)
    w["ws13"] = bf16(rng.standard_normal((2 * Is, H)) / 16)
    w["ws2"] = bf16(rng.standard_normal((H, Is)) / 8)
    x = bf16(rng.standard_normal((1, H)))
    o = oracle.moe_tail(x, None, w, cfg)
    xn = synth.bf16_bits_to_f32(o["xn"][0]).astype(np.float64)
    Ws13 = synth.bf16_bits_to_f32(w["ws13"]).astype(np.float64)
    Ws2 = synth.bf16_bits_to_f32(w["ws2"]).astype(np.float64)
    gu = Ws13 @ xn
    s = Ws2 @ (gu[:Is] * scipy.special.expit(gu[:Is]) * gu[Is:])
    np.testing.assert_allclose(o["y_shared"][0], s, rtol=1e-10, atol=1e-12)
    np.testing.assert_array_equal(o["y_routed"][0], 0.0)  # all-zero routed codes


def test_router_matches_dense_matmul_and_out_is_h_plus_y():
    cfg = synth.CONFIGS["c0"]
    w = synth.make_weights(cfg)
    x, r = synth.make_rows(cfg)
    o = oracle.moe_tail(x, r, w, cfg)
    xn = synth.bf16_bits_to_f32(o["xn"]).astype(np.float64)
    Wr = synth.bf16_bits_to_f32(w["router_w"]).astype(np.float64)
    np.testing.assert_allclose(o["logits"], xn @ Wr.T, rtol=1e-12, atol=1e-12)
    h = synth.bf16_bits_to_f32(o["h"]).astype(np.float64)
    y = o["y_routed"] + o["y_shared"]
    want = np.array([[oracle.bf16_round(a + b) for a, b in zip(hr, yr)] for hr, yr in zip(h, y)], np.uint16)
    np.testing.assert_array_equal(o["out"], want)
    # the selected ids are the top-k of the logits, weights the softmax over them
    ids = o["ids"][0]
    assert set(ids.tolist()) == set(np.argsort(-o["logits"][0], kind="stable")[: cfg.topk].tolist())
    np.testing.assert_allclose(o["w"][0], scipy.special.softmax(o["logits"][0][ids]), rtol=1e-13)


def test_duplicate_experts_give_one_experts_output():
    """All experts identical: the normalised weights sum to 1, so y_routed equals one expert's output."""
    cfg = synth.Config("dup", 98, 2, 512, 8, 3, 64, 0)
    w = synth.make_weights(cfg)
    for key in ("w13_q", "w13_s", "w2_q", "w2_s"):
        w[key][:] = w[key][0:1]
    x, r = synth.make_rows(cfg)
    o = oracle.moe_tail(x, r, w, cfg)
    one = synth.Config("dup1", 98, 2, 512, 1, 1, 64, 0)
    w1 = dict(w)
    for key in ("w13_q", "w13_s", "w2_q", "w2_s", "router_w"):
        w1[key] = np.ascontiguousarray(w[key][0:1])
    o1 = oracle.moe_tail(x, r, w1, one)
    np.testing.assert_allclose(o["y_routed"], o1["y_routed"], rtol=1e-12, atol=1e-12)


def test_power_of_two_scale_linearity():
    """+1 on every W2 scale byte doubles y_routed exactly; +1 on the up half of W13 does too."""
    cfg = synth.Config("lin", 97, 2, 512, 8, 2, 64, 0)
    w = synth.make_weights(cfg)
    x, r = synth.make_rows(cfg)
    base = oracle.moe_tail(x, r, w, cfg)["y_routed"]
    w2 = dict(w)
    w2["w2_s"] = w["w2_s"] + 1
    np.testing.assert_array_equal(oracle.moe_tail(x, r, w2, cfg)["y_routed"], 2.0 * base)
    wu = dict(w)
    s = w["w13_s"].copy()
    s[:, cfg.inter:, :] += 1
    wu["w13_s"] = s
    np.testing.assert_array_equal(oracle.moe_tail(x, r, wu, cfg)["y_routed"], 2.0 * base)


# ---- the shared expert's sigmoid gate (optional; "[AMD] integrate kimi k3
# monokernel", K2 commit text, "Kernel Replacement") ---------------------------

def _gated(cfg, w, x, r, gate_f32):
    wg = dict(w)
    wg["shared_gate"] = synth.to_bf16_bits(np.asarray(gate_f32, np.float32))
    return oracle.moe_tail(x, r, wg, cfg)


def test_shared_gate_closed_forms():
    """sigmoid(0) = 1/2 halves the shared output exactly; a gate whose dot
    product with xn is about +-200 saturates to exactly 1 (unchanged) or to
    below 1e-80 (gone); the routed part and the routing never change."""
    cfg = synth.CONFIGS["c0"].with_rows(2)
    w = synth.make_weights(cfg)
    x, r = synth.make_rows(cfg)
    o = oracle.moe_tail(x, r, w, cfg)
    H = cfg.hidden
    half = _gated(cfg, w, x, r, np.zeros(H))
    np.testing.assert_array_equal(half["y_shared"], 0.5 * o["y_shared"])
    np.testing.assert_array_equal(half["y_routed"], o["y_routed"])
    np.testing.assert_array_equal(half["ids"], o["ids"])
    for row in range(cfg.rows):
        sgn = np.sign(synth.bf16_bits_to_f32(o["xn"][row]))
        on = _gated(cfg, w, x[row:row + 1], r[row:row + 1], 0.5 * sgn)
        off = _gated(cfg, w, x[row:row + 1], r[row:row + 1], -0.5 * sgn)
        np.testing.assert_array_equal(on["y_shared"][0], o["y_shared"][row])
        assert np.max(np.abs(off["y_shared"][0])) <= 1e-80 * np.max(np.abs(o["y_shared"][row]))


def test_shared_gate_reads_the_normed_row():
    """A one-hot gate e_k picks channel k of xn (not of h or x): the shared
    output is scaled by sigmoid(xn_k), for a few channels k."""
    cfg = synth.CONFIGS["c0"].with_rows(1)
    w = synth.make_weights(cfg)
    x, r = synth.make_rows(cfg)
    o = oracle.moe_tail(x, r, w, cfg)
    xn = synth.bf16_bits_to_f32(o["xn"][0]).astype(np.float64)
    h = synth.bf16_bits_to_f32(o["h"][0]).astype(np.float64)
    for k in (0, 7, 255, 511):
        assert xn[k] != h[k]
        e = np.zeros(cfg.hidden)
        e[k] = 1.0
        g = _gated(cfg, w, x, r, e)
        ratio = g["y_shared"][0] / o["y_shared"][0]
        np.testing.assert_allclose(ratio, 1.0 / (1.0 + np.exp(-xn[k])), rtol=1e-13)


# ---- routing variants: group-limited top-k and a routed scaling factor -----

def test_grouped_topk_reduces_to_plain_topk():
    """One group, or every group kept, is the plain top-k (pinned above)."""
    rng = np.random.default_rng(5)
    for _ in range(20):
        keys = rng.standard_normal(64)
        for k in (1, 3, 8):
            plain = oracle.topk(keys, k)
            np.testing.assert_array_equal(oracle.topk_grouped(keys, k, 1, 1), plain)
            np.testing.assert_array_equal(oracle.topk_grouped(keys, k, 8, 8), plain)


def test_grouped_topk_worked_example():
    """16 experts in 4 groups of 4, keep 2 groups, pick 3.  Group scores (two
    largest keys): g0 0.9+0.1 = 1.0, g1 0.5+0.45 = 0.95, g2 0.8+0 = 0.8, g3 0.6.
    Kept: g0, g1.  Picks: e0 (0.9), e4 (0.5), e5 (0.45); the plain top-3 would
    take e8 (0.8) from g2 instead."""
    keys = np.array([0.9, 0.1, 0.0, 0.0, 0.5, 0.45, 0.0, 0.0, 0.8, 0.0, 0.0, 0.0, 0.3, 0.3, 0.3, 0.3])
    np.testing.assert_array_equal(oracle.topk_grouped(keys, 3, 4, 2), [0, 4, 5])
    np.testing.assert_array_equal(oracle.topk(keys, 3), [0, 8, 4])


def test_grouped_topk_group_ties_go_to_the_lower_group():
    """Groups 1 and 2 score alike (0.5 + 0.25 each); with group 0 first, group 1 is kept."""
    keys = np.array([1.0, 1.0, 0.5, 0.25, 0.5, 0.25, 0.0, 0.0])
    np.testing.assert_array_equal(oracle.topk_grouped(keys, 3, 4, 2), [0, 1, 2])
    keys2 = keys.copy()
    keys2[[2, 3]] = keys[[4, 5]] - np.array([0.0, 1e-9])  # group 1 now a little lower
    np.testing.assert_array_equal(oracle.topk_grouped(keys2, 3, 4, 2), [0, 1, 4])


def test_routed_scale_two_doubles_the_routed_part_exactly():
    import dataclasses

    cfg = synth.CONFIGS["c0"].with_rows(2)
    w = synth.make_weights(cfg)
    x, r = synth.make_rows(cfg)
    o = oracle.moe_tail(x, r, w, cfg)
    o2 = oracle.moe_tail(x, r, w, dataclasses.replace(cfg, routed_scale=2.0))
    np.testing.assert_array_equal(o2["ids"], o["ids"])
    np.testing.assert_array_equal(o2["w"], 2.0 * o["w"])
    np.testing.assert_array_equal(o2["y_routed"], 2.0 * o["y_routed"])
    np.testing.assert_array_equal(o2["y_shared"], o["y_shared"])


def test_grouped_routing_in_the_tail_keeps_picks_inside_the_kept_groups():
    """The whole tail with 4 groups of 4 kept out of 16 experts: every pick's
    group is among the 2 best-scoring groups of its row, and n_group = 1 gives
    the ungrouped tail exactly."""
    import dataclasses

    cfg = synth.CONFIGS["c0"].with_rows(3)
    w = synth.make_weights(cfg)
    x, r = synth.make_rows(cfg)
    g = dataclasses.replace(cfg, n_group=4, topk_group=2)
    og = oracle.moe_tail(x, r, w, g)
    o1 = oracle.moe_tail(x, r, w, dataclasses.replace(cfg, n_group=1, topk_group=1))
    o = oracle.moe_tail(x, r, w, cfg)
    np.testing.assert_array_equal(o1["ids"], o["ids"])
    np.testing.assert_array_equal(o1["out"], o["out"])
    for row in range(cfg.rows):
        ky = og["keys"][row].reshape(4, 4)
        top2 = -np.sort(-ky, axis=1)[:, :2].sum(axis=1)
        kept = set(np.argsort(-top2, kind="stable")[:2].tolist())
        assert {int(e) // 4 for e in og["ids"][row]} <= kept


# ---- a second expert weight format: MXFP8 (E4M3 codes, E8M0 block-32 scales,
# OCP Microscaling Formats v1.0) ---------------------------------------------

def test_e4m3_anchor_values_of_the_spec():
    """OCP MX v1.0 FP8 E4M3: max normal 448 (0x7E), min normal 2^-6 (0x08),
    min subnormal 2^-9 (0x01), 1.0 = 0x38, NaN at S.1111.111, signed zeros."""
    assert oracle.e4m3(0x7E) == 448.0
    assert oracle.e4m3(0xFE) == -448.0
    assert oracle.e4m3(0x08) == 2.0 ** -6
    assert oracle.e4m3(0x01) == 2.0 ** -9
    assert oracle.e4m3(0x38) == 1.0
    assert np.isnan(oracle.e4m3(0x7F)) and np.isnan(oracle.e4m3(0xFF))
    assert oracle.e4m3(0x00) == 0.0 and oracle.e4m3(0x80) == 0.0


def test_e4m3_every_code_from_its_bit_fields():
    """Each non-NaN code rebuilt as an fp32 bit pattern: a normal code moves its
    exponent (bias 7 -> 127) and mantissa (3 -> 23 bits) into place; a
    subnormal one is m * 2^-9."""
    for code in range(256):
        if code & 0x7F == 0x7F:
            continue
        s, e, m = code >> 7, (code >> 3) & 0xF, code & 7
        if e:
            bits = (s << 31) | ((e - 7 + 127) << 23) | (m << 20)
            want = float(np.array([bits], np.uint32).view(np.float32)[0])
        else:
            want = (-1.0) ** s * m * 2.0 ** -9
        assert oracle.e4m3(code) == want, hex(code)


def test_mxfp8_copy_of_mxfp4_weights_gives_the_same_tail():
    """Every E2M1 value is exact in E4M3.  MXFP4 weights re-encoded as MXFP8
    (one byte per element, same scales) give the same tail, bit for bit: this
    pins the MXFP8 layout (row strides, one byte per element) and its decode."""
    import dataclasses

    cfg = synth.CONFIGS["c0"].with_rows(2)
    w = synth.make_weights(cfg)
    x, r = synth.make_rows(cfg)
    o4 = oracle.moe_tail(x, r, w, cfg)
    to8 = np.array([0x00, 0x30, 0x38, 0x3C, 0x40, 0x44, 0x48, 0x4C], np.uint8)  # E2M1 magnitudes as E4M3

    def unpack(q):
        lo, hi = q & 0xF, q >> 4
        codes = np.stack([lo, hi], axis=-1).reshape(q.shape[:-1] + (q.shape[-1] * 2,))
        return to8[codes & 7] | ((codes & 8) << 4).astype(np.uint8)

    w8 = dict(w)
    w8["w13_q"] = unpack(w["w13_q"])
    w8["w2_q"] = unpack(w["w2_q"])
    for c in range(16):  # the re-encoding itself is exact
        assert oracle.e4m3(int(to8[c & 7] | ((c & 8) << 4))) == oracle.e2m1(c)
    o8 = oracle.moe_tail(x, r, w8, dataclasses.replace(cfg, weight_format=1))
    for k in ("ids", "w", "y_routed", "y_shared", "out"):
        np.testing.assert_array_equal(o8[k], o4[k])


# ---- the norm folded into the router and shared projections ------------------------

def _times8(a):
    """bf16 bit patterns times 8 (exact: only the exponent moves)."""
    return (a + np.uint16(3 << 7) * ((a & 0x7F80) != 0)).astype(np.uint16)


def test_folded_norm_with_unit_gamma_is_rstd_times_the_raw_projection():
    """With gamma = 1, bf16(h * gamma) = h exactly, so the folded logits are
    rstd * (h . Wr) and the shared expert's gate/up sums are rstd * (Ws13 . h)
    (the pages' fold of the router norm into its logits and into the next
    projections' activation scales).  x is scaled by 8 so that rstd is far
    from 1 and a missing or inverted rstd is visible."""
    import dataclasses

    cfg = dataclasses.replace(synth.CONFIGS["c0"].with_rows(2), fold_norm=1)
    w = dict(synth.make_weights(cfg))
    w["gamma"] = np.full(cfg.hidden, 0x3F80, np.uint16)
    x, r = synth.make_rows(cfg)
    x = _times8(x)
    o = oracle.moe_tail(x, r, w, cfg)
    Wr = synth.bf16_bits_to_f32(w["router_w"]).astype(np.float64)
    W13 = synth.bf16_bits_to_f32(w["ws13"]).astype(np.float64)
    W2 = synth.bf16_bits_to_f32(w["ws2"]).astype(np.float64)
    Is = cfg.shared_inter
    for row in range(cfg.rows):
        h, xn, rstd = oracle.norm_row(x[row], r[row], w["gamma"], cfg.eps)
        assert rstd < 0.25
        hv = synth.bf16_bits_to_f32(h).astype(np.float64)
        np.testing.assert_allclose(o["logits"][row], rstd * (Wr @ hv), rtol=1e-12, atol=1e-14)
        g, u = rstd * (W13[:Is] @ hv), rstd * (W13[Is:] @ hv)
        np.testing.assert_allclose(o["y_shared"][row], W2 @ (g / (1 + np.exp(-g)) * u), rtol=1e-10, atol=1e-14)
        np.testing.assert_array_equal(o["xn"][row], xn)  # the normed row itself is unchanged


def test_folded_logits_stay_within_two_bf16_roundings_of_the_plain_ones():
    """Folded and plain logits project the same real vector h*rstd*gamma, one
    through bf16(h*gamma) then times rstd, the other through bf16(h*rstd*gamma):
    each rounding is at most 2^-9 relative per element, so the logits differ by
    at most rstd * sum_i |Wr_ei h_i gamma_i| * 2^-8 -- and they do differ."""
    import dataclasses

    cfg = synth.CONFIGS["c3"].with_rows(2)
    w = synth.make_router_weights(cfg)
    x, r = synth.make_rows(cfg)
    x = _times8(x)
    lp, _ = oracle.router_keys(x, r, w, cfg)
    lf, _ = oracle.router_keys(x, r, w, dataclasses.replace(cfg, fold_norm=1))
    Wr = np.abs(synth.bf16_bits_to_f32(w["router_w"]).astype(np.float64))
    gm = synth.bf16_bits_to_f32(w["gamma"]).astype(np.float64)
    for row in range(cfg.rows):
        h, _, rstd = oracle.norm_row(x[row], r[row], w["gamma"], cfg.eps)
        hv = np.abs(synth.bf16_bits_to_f32(h).astype(np.float64) * gm)
        bound = rstd * (Wr @ hv) * 2.0**-8 * (1 + 1e-9)
        d = np.abs(lf[row] - lp[row])
        assert np.all(d <= bound)
        assert np.count_nonzero(d) > cfg.experts // 2


def test_folded_norm_leaves_the_routed_experts_on_xn():
    """With one pick (weight exactly 1) and the same expert chosen, the routed
    output is the same bit for bit with or without the fold: the routed
    experts project xn either way."""
    import dataclasses

    cfg = dataclasses.replace(synth.CONFIGS["c0"].with_rows(4), topk=1)
    w = synth.make_weights(cfg)
    x, r = synth.make_rows(cfg)
    o = oracle.moe_tail(x, r, w, cfg)
    of = oracle.moe_tail(x, r, w, dataclasses.replace(cfg, fold_norm=1))
    same = (o["ids"] == of["ids"]).ravel()
    assert same.sum() >= 3
    np.testing.assert_array_equal(of["w"], 1.0)
    np.testing.assert_array_equal(of["y_routed"][same], o["y_routed"][same])
    np.testing.assert_array_equal(of["xn"], o["xn"])
    np.testing.assert_array_equal(of["h"], o["h"])
    assert not np.array_equal(of["y_shared"], o["y_shared"])


# ---- the out_proj front ----------------------------------------------------------

def test_out_proj_one_hot_row_reads_a_column_exactly():
    """An attention row that is 1 at column a and 0 elsewhere projects to
    column a of w_o, bit for bit (one exact product per output, no rounding)."""
    cfg = synth.CONFIGS["c0"].with_rows(3)
    w_o = synth.make_out_proj(cfg)["w_o"]
    A = w_o.shape[1]
    attn = np.zeros((3, A), np.uint16)
    cols = [0, A // 2 + 1, A - 1]
    for r, a in enumerate(cols):
        attn[r, a] = 0x3F80  # 1.0
    x, _ = oracle.out_proj(attn, w_o)
    for r, a in enumerate(cols):
        np.testing.assert_array_equal(x[r], w_o[:, a])


def test_out_proj_is_the_matrix_product_then_one_rounding():
    """y equals the float64 matrix product (a library routine, another
    summation order), and x is y rounded to bf16 once: it matches the float32
    route wherever float32 holds y exactly enough to round the same way, and
    never misses by more than one bf16 step."""
    cfg = synth.CONFIGS["c3"].with_rows(4)
    f = synth.make_out_proj(cfg)
    x, y = oracle.out_proj(f["attn"], f["w_o"])
    a64 = synth.bf16_bits_to_f32(f["attn"]).astype(np.float64)
    w64 = synth.bf16_bits_to_f32(f["w_o"]).astype(np.float64)
    ref = a64 @ w64.T
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
    for v, b in zip(y.ravel()[:2000], x.ravel()[:2000]):
        assert int(b) == oracle.bf16_round(float(v))
    xf = synth.bf16_bits_to_f32(x).astype(np.float64)
    step = np.abs(xf) * 2.0**-7 + 1e-30
    assert np.all(np.abs(xf - ref) <= step)


def test_out_proj_scales_by_powers_of_two_exactly():
    """Doubling the attention rows doubles every output exactly: the products,
    the sum and the bf16 rounding all commute with a factor of 2."""
    cfg = synth.CONFIGS["c0"].with_rows(2)
    f = synth.make_out_proj(cfg)
    attn2 = (f["attn"] + np.uint16(1 << 7) * ((f["attn"] & 0x7F80) != 0)).astype(np.uint16)
    x1, y1 = oracle.out_proj(f["attn"], f["w_o"])
    x2, y2 = oracle.out_proj(attn2, f["w_o"])
    np.testing.assert_array_equal(y2, 2 * y1)
    np.testing.assert_array_equal(synth.bf16_bits_to_f32(x2), 2 * synth.bf16_bits_to_f32(x1))


def test_out_proj_rounds_once_from_the_exact_sum():
    """y = 1 + 2^-8 + 2^-30 (three exact products) lies just above a bf16
    halfway point: rounded once it is 1 + 2^-7 (0x3F81).  A route through
    float32 would land on the halfway point and round to even (0x3F80)."""
    b = lambda v: int(synth.to_bf16_bits(np.array([v], np.float32))[0])
    attn = np.array([[b(1.0), b(1.0), b(1.0)]], np.uint16)
    w_o = np.array([[b(1.0), b(2.0**-8), b(2.0**-30)]], np.uint16)
    x, y = oracle.out_proj(attn, w_o)
    assert y[0, 0] == 1 + 2.0**-8 + 2.0**-30
    assert int(x[0, 0]) == 0x3F81


def e4m3_from_bits(code: int) -> float:
    """E4M3 from its bit fields (OCP MX v1.0): sign bit 7, exponent bits 6..3
    with bias 7, mantissa bits 2..0; exponent 0 is subnormal (2^-6 m/8)."""
    s = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 0xF, code & 7
    return s * (2.0 ** -6 * m / 8 if e == 0 else 2.0 ** (e - 7) * (1 + m / 8))


def test_one_expert_one_row_closed_form_mxfp8():
    """The same closed form as for MXFP4, with MXFP8 codes drawn from all 254
    non-NaN E4M3 codes (subnormals, both signs, up to 448): xn = 1 exactly, so
    g_i = H v_g[i] 2^(s_g-127), u_i = H v_u[i] 2^(s_u-127) and
    out_h = bf16(1 + v_d[h] 2^(s_d-127) sum_i silu(g_i) u_i)."""
    import dataclasses

    H, I = 256, 64
    cfg = dataclasses.replace(_cfg(H, 1, 1, I, 0), weight_format=1)
    w = _zero_weights(cfg)
    w["w13_q"] = np.zeros((1, 2 * I, H), np.uint8)
    w["w2_q"] = np.zeros((1, H, I), np.uint8)
    rng = np.random.default_rng(9)
    ok = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    cg, cu, cd = rng.choice(ok, I), rng.choice(ok, I), rng.choice(ok, H)
    sg, su, sd = 110, 112, 124
    w["w13_q"][0, :I, :] = cg[:, None]
    w["w13_q"][0, I:, :] = cu[:, None]
    w["w13_s"][0, :I, :] = sg
    w["w13_s"][0, I:, :] = su
    w["w2_q"][0, :, :] = cd[:, None]
    w["w2_s"][0] = sd
    x = bf16(np.ones((1, H)))
    o = oracle.moe_tail(x, None, w, cfg)
    assert np.all(o["xn"] == 0x3F80)
    acc = 0.0
    for i in range(I):
        g = H * e4m3_from_bits(int(cg[i])) * 2.0 ** (sg - 127)
        u = H * e4m3_from_bits(int(cu[i])) * 2.0 ** (su - 127)
        acc += silu(g) * u
    d = np.array([e4m3_from_bits(int(cd[h])) * 2.0 ** (sd - 127) * acc for h in range(H)])
    np.testing.assert_allclose(o["y_routed"][0], d, rtol=1e-12, atol=1e-300)
    want = np.array([oracle.bf16_round(1.0 + v) for v in d], np.uint16)
    np.testing.assert_array_equal(o["out"][0], want)
    assert np.count_nonzero(want != 0x3F80) > H // 2  # the routed part shows in most outputs
