"""Parity at the edges of the accepted shapes, through the C ABI: no shared
expert, ragged hidden / expert / intermediate sizes (a partial router block, an
odd number of scale bytes per down row), one expert with top-1, and top-k equal
to the expert count, and the largest accepted picks, hidden size and
intermediate sizes."""
import sys

import numpy as np
import pytest

import oracle
from cases import gapped_rows
from decode_moe_layer_amd import synth
from gpu_harness import check_against_oracle, dev, handle_for, run

pytestmark = pytest.mark.gpu

EDGES = {
    # name: (config, max_rows)
    "no_shared": (synth.Config("no_shared", 5, 3, 512, 16, 2, 64, 0), 4),
    "ragged": (synth.Config("ragged", 6, 5, 640, 24, 3, 96, 96, scoring=synth.SIGMOID_BIAS, bias_std=0.1), 7),
    "one_expert": (synth.Config("one_expert", 7, 2, 256, 1, 1, 32, 32), 2),
    "all_experts": (synth.Config("all_experts", 8, 2, 512, 16, 16, 64, 64), 3),
    # the largest accepted sizes, one dimension at a time (all at once would be
    # about 51 GB of expert weights): 16 rows x top-32 of 512 experts = 512
    # picks; hidden 8192 at 16 rows (32 hidden rows per compute unit, xn from
    # global scratch) with few experts; expert and shared intermediate 4096
    "max_picks": (synth.Config("max_picks", 9, 16, 1024, 512, 32, 64, 64), 16),
    "max_hidden": (synth.Config("max_hidden", 10, 16, 8192, 32, 2, 64, 128), 16),
    "max_inter": (synth.Config("max_inter", 11, 1, 512, 16, 4, 4096, 4096), 1),
}


@pytest.mark.parametrize("name", sorted(EDGES))
def test_edge_shapes(name):
    cfg, max_rows = EDGES[name]
    print("edge", name, cfg, "max_rows", max_rows, flush=True)
    sys.stdout.flush()
    w = synth.make_weights(cfg)
    x, r, _ = gapped_rows(cfg, w)
    o = oracle.moe_tail(x, r, w, cfg)
    h = handle_for(cfg, max_rows=max_rows)
    g = run(h, cfg, {k: dev(v) for k, v in w.items()}, x, r)
    assert h.get_error() == 0
    check_against_oracle(g, o, cfg)
    if not cfg.shared_inter:
        assert np.all(g["y_shared"] == 0)
    if cfg.topk == cfg.experts:  # every expert is picked, in key order
        assert sorted(g["ids"][0].tolist()) == list(range(cfg.experts))


def test_hidden_beyond_the_device_is_refused():
    """hidden 16384 passes the device-independent check, but on a 256-CU
    device it is more than 32 hidden rows per compute unit: create refuses it
    with EUNSUPPORTED and a message, and launches nothing."""
    from decode_moe_layer_amd import binding

    c = binding.make_config(16, 16384, 64, 4, 64, 128)
    assert binding.check_config(c) == binding.OK
    with pytest.raises(binding.MoeTailError) as ei:
        binding.MoeTail(c)
    assert ei.value.status == binding.EUNSUPPORTED
    assert "hidden 16384" in str(ei.value)
