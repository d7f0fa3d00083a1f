"""Determinism under load: one captured graph of calls of mixed widths
(8, 1, 3, 8, 2, 5, 16, 24 and 32 rows on one handle; the last two are wide
launches), replayed until more than 10,000 calls have run.  Every replay is compared with the eager results of
the same calls, element for element, and folded into a digest; the check
stops at the first mismatch and names the replay.  A perturbation control
(one bit of one input changed between replays) must change the digest, so
that the comparison is known to see a difference.

Replay stress with digests and a perturbation control: "[Perf] [MI355X]
glm53: Long-context indexer ...", PR 85, Accuracy (replays with digests,
--perturb); "Split the Kimi3 AttnRes mix across CTAs for decode rows",
validation section (replays that match the eager hash)."""
import numpy as np
import pytest

from cases import gapped_rows, oracle_rows, weights
from decode_moe_layer_amd import binding, synth
from gpu_harness import check_against_oracle, dev, device_weights, handle_for, run

pytestmark = pytest.mark.gpu

WIDTHS = (8, 1, 3, 8, 2, 5, 16, 24, 32)
CALLS = 10_010  # 1113 replays of the 9 calls
CHECK_EVERY = 50  # replays between host checks of the running mismatch flag


def _setup():
    t = pytest.importorskip("torch")
    cfg = synth.CONFIGS["c1"].with_rows(32)
    w = weights("c1")
    x, r, _ = gapped_rows(cfg, w)
    h = handle_for(cfg, max_rows=32)
    dw = device_weights("c1")
    eager = [run(h, cfg, dw, x[:n], r[:n], rows=n) for n in WIDTHS]
    # the eager results themselves meet the parity bar (all 32 rows)
    check_against_oracle(eager[-1], oracle_rows(x, r, w, cfg), cfg)
    xd, rd = dev(x), dev(r)
    outs = [t.empty((n, cfg.hidden), dtype=t.int16, device="cuda") for n in WIDTHS]
    refs = [t.from_numpy(e["out"].view(np.int16)).to("cuda") for e in eager]
    s = t.cuda.Stream()
    g = t.cuda.CUDAGraph()
    with t.cuda.stream(s):
        with t.cuda.graph(g, stream=s):
            for n, o in zip(WIDTHS, outs):
                h.run(n, xd, rd, dw["gamma"], dw["router_w"], None, dw["w13_q"], dw["w13_s"], dw["w2_q"], dw["w2_s"],
                      dw["ws13"], dw["ws2"], o, stream=s.cuda_stream)
    # digest weights: a fixed pseudo-random odd int64 per element (the sum wraps)
    gen = np.random.default_rng(12345)
    wts = [t.from_numpy(gen.integers(1, 2**40, size=n * cfg.hidden, dtype=np.int64) | 1).to("cuda") for n in WIDTHS]
    # every buffer the graph reads or writes stays referenced for as long as it replays
    keep = (xd, rd, dw, outs)
    return t, cfg, h, g, xd, outs, refs, wts, keep


def _digest(t, outs, wts):
    """One int64 per replay: the weighted sum of every output element (on the device)."""
    d = t.zeros((), dtype=t.int64, device="cuda")
    for o, wv in zip(outs, wts):
        d = d * 1000003 + (o.reshape(-1).to(t.int64) * wv).sum()
    return d


def test_replay_stress_matches_eager_every_time():
    t, cfg, h, g, xd, outs, refs, wts, keep = _setup()
    want = _digest(t, refs, wts)
    replays = (CALLS + len(WIDTHS) - 1) // len(WIDTHS)
    bad = t.zeros((), dtype=t.bool, device="cuda")
    digest = t.zeros((), dtype=t.int64, device="cuda")
    expect = t.zeros((), dtype=t.int64, device="cuda")
    first_bad = -1
    for rep in range(replays):
        for o in outs:
            o.fill_(0)
        g.replay()
        for o, e in zip(outs, refs):
            bad |= (o != e).any()
        digest = digest * 31 + _digest(t, outs, wts)
        expect = expect * 31 + want
        if (rep + 1) % CHECK_EVERY == 0 or rep == replays - 1:
            t.cuda.synchronize()
            if bool(bad.item()):
                first_bad = rep
                break
    assert first_bad < 0, "a replay in the %d before replay %d differs from the eager results" % (CHECK_EVERY, first_bad)
    assert int(digest.item()) == int(expect.item())
    assert h.get_error() == binding.OK
    print("replays", replays, "calls", replays * len(WIDTHS), "digest %016x" % (int(digest.item()) & (2**64 - 1)))


def test_replay_stress_perturbation_changes_the_digest():
    """Negative control: one bit of one x element flipped between replays
    changes that replay's outputs and so the digest; restoring it restores both."""
    t, cfg, h, g, xd, outs, refs, wts, keep = _setup()
    want = int(_digest(t, refs, wts).item())
    g.replay()
    assert int(_digest(t, outs, wts).item()) == want
    xv = xd.view(t.int16)
    orig = xv[0, 17].clone()
    xv[0, 17] ^= 1 << 4  # a mantissa bit of row 0, column 17 (in every call: row 0 is in all of them)
    g.replay()
    changed = int(_digest(t, outs, wts).item())
    assert changed != want
    assert any(bool((o != e).any().item()) for o, e in zip(outs, refs))
    xv[0, 17] = orig
    g.replay()
    assert int(_digest(t, outs, wts).item()) == want
    assert h.get_error() == binding.OK
