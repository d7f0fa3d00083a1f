"""The out_proj front on the GPU: x = bf16(attn . w_o^T) for one rank's
share ("[AMD] integrate kimi k3 monokernel", K2 commit text, Motivation and
Modifications), computed in the same launch as the tail, against the
oracle's out_proj and tail.  x is compared bit for bit (both sides sum in
double and round once); the tail's outputs to the usual bars."""
import dataclasses

import numpy as np
import pytest

import oracle
from cases import GAP_REL, key_gaps, weights
from decode_moe_layer_amd import binding, synth
from gpu_harness import check_against_oracle, dev, device_weights, handle_for, run

pytestmark = pytest.mark.gpu


def _front_rows(cfg, w, A):
    """Attention rows, from a pool drawn once (grown until it is enough),
    whose front output x has a well-posed top-k (oracle keys, 1e-4 relative
    gap), with w_o and x."""
    pool = cfg.rows + 8
    while True:
        big = synth.make_out_proj(cfg.with_rows(pool), attn_dim=A)
        x, _ = oracle.out_proj(big["attn"], big["w_o"])
        _, ky = oracle.router_keys(x, None, w, cfg)
        ok = np.nonzero(key_gaps(ky, cfg.topk) >= GAP_REL)[0][:cfg.rows]
        if len(ok) == cfg.rows:
            return np.ascontiguousarray(big["attn"][ok]), big["w_o"], np.ascontiguousarray(x[ok])
        pool *= 2


@pytest.mark.parametrize("name,rows,A", [("c0", 2, 128), ("c1", 8, 768), ("c3", 4, 896), ("c4", 16, 1024),
                                         ("c1", 20, 768), ("c0", 32, 16384)])
def test_front_parity(name, rows, A):
    """x bit for bit and the whole tail to the usual bars: c0 with A = 128,
    the 512-expert shard at 8 rows, sigmoid keys, 16 rows from global
    scratch, a 20-row call (two tail launches on one front), and the largest
    accepted width A = 16384 at 32 rows (two row blocks in the front)."""
    cfg = synth.CONFIGS[name].with_rows(rows)
    print("front", name, rows, A, flush=True)
    w = weights(name)
    attn, w_o, x = _front_rows(cfg, w, A)
    o = oracle.moe_tail(x, None, w, cfg)
    h = handle_for(cfg, attn_dim=A)
    g = run(h, cfg, device_weights(name), None, None, front=(dev(attn), dev(w_o)))
    assert h.get_error() == 0
    np.testing.assert_array_equal(g["res_out"], x)  # no residual: h = x
    check_against_oracle(g, o, cfg)


def test_front_refusals():
    """x and attn together, attn on a handle without attn_dim, and attn
    without w_o are refused before anything is enqueued."""
    cfg = synth.CONFIGS["c0"].with_rows(2)
    w = weights("c0")
    attn, w_o, x = _front_rows(cfg, w, 128)
    dw = device_weights("c0")
    da, dwo, dx = dev(attn), dev(w_o), dev(x)
    with pytest.raises(binding.MoeTailError) as ei:
        run(handle_for(cfg, attn_dim=128), cfg, dw, x, None, front=(da, dwo), rows=2)
    assert ei.value.status == binding.EINVAL
    with pytest.raises(binding.MoeTailError) as ei:
        run(handle_for(cfg), cfg, dw, None, None, front=(da, dwo))
    assert ei.value.status == binding.EINVAL
    with pytest.raises(binding.MoeTailError) as ei:
        run(handle_for(cfg, attn_dim=128), cfg, dw, None, None, front=(da, None))
    assert ei.value.status == binding.EINVAL
    # the folded norm reads x by K chunks: it takes no attention rows
    folded = dataclasses.replace(cfg, fold_norm=1)
    with pytest.raises(binding.MoeTailError) as ei:
        run(handle_for(folded, attn_dim=128), folded, dw, None, None, front=(da, dwo))
    assert ei.value.status == binding.EUNSUPPORTED
