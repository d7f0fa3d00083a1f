"""The C ABI library: builds, loads, exports every declared symbol, and validates on the host."""
import ctypes
import os
import re

import pytest

from decode_moe_layer_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "moe_tail.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_tail_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = binding.lib()
    names = declared_functions()
    assert set(names) == set(binding.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
        assert ctypes.cast(getattr(L, n), ctypes.c_void_p).value


def test_struct_layout_matches_header():
    # moe_tail_config: 17 x 4-byte integer fields + 2 floats; moe_tail_args: 21 pointers
    assert ctypes.sizeof(binding.Config) == 19 * 4
    assert ctypes.sizeof(binding.Args) == 21 * 8


def good():
    return binding.make_config(8, 6144, 512, 10, 256, 512)


def test_check_config_accepts_the_workloads():
    assert binding.check_config(good()) == binding.OK
    for args in [(1, 512, 16, 2, 64, 64), (4, 7168, 256, 8, 256, 256, binding.SIGMOID_BIAS), (16, 8192, 384, 8, 256, 256),
                 (16, 6144, 512, 10, 256, 512), (3, 1024, 64, 32, 32, 0)]:
        assert binding.check_config(binding.make_config(*args)) == binding.OK, args


@pytest.mark.parametrize("field,value", [
    ("max_rows", 0), ("max_rows", 33), ("hidden", 100), ("hidden", 6000), ("hidden", 32768),
    ("num_experts", 0), ("num_experts", 513), ("top_k", 0), ("top_k", 33), ("inter", 48), ("inter", 0),
    ("shared_inter", 40), ("shared_inter", -32), ("scoring", 2), ("eps", 0.0), ("eps", float("nan")),
    ("debug_flags", 4), ("debug_flags", 6),
    ("n_group", 3), ("n_group", 128), ("n_group", -1),
    ("routed_scale", -1.0), ("routed_scale", float("inf")),
    ("weight_format", 2), ("weight_format", -1), ("fold_norm", 2), ("fold_norm", -1),
    ("attn_dim", -128), ("attn_dim", 100), ("attn_dim", 16512), ("w13_layout", 2), ("w13_layout", -1),
])
def test_check_config_refusals(field, value):
    c = good()
    setattr(c, field, value)
    assert binding.check_config(c) == binding.EINVAL
    assert binding.strerror(None)


def test_grouped_routing_accepted_and_refused():
    c = good()  # 512 experts, top-10
    c.n_group, c.topk_group, c.routed_scale = 8, 4, 2.5
    assert binding.check_config(c) == binding.OK
    c.topk_group = 1  # 64 experts kept >= 10 picks
    assert binding.check_config(c) == binding.OK
    c.n_group, c.topk_group = 64, 1  # 8 experts kept < 10 picks
    assert binding.check_config(c) == binding.EINVAL
    c.n_group, c.topk_group = 8, 0
    assert binding.check_config(c) == binding.EINVAL
    c.topk_group = 9
    assert binding.check_config(c) == binding.EINVAL
    c.n_group, c.topk_group, c.routed_scale = 0, 0, 0.0  # zeroed fields: plain routing, scale 1
    assert binding.check_config(c) == binding.OK


def test_up_to_32_rows_accepted():
    for rows in (16, 17, 32):
        assert binding.check_config(binding.make_config(rows, 6144, 512, 10, 256, 512)) == binding.OK, rows


def test_both_weight_formats_accepted():
    for fmt in (binding.MXFP4, binding.MXFP8):
        c = good()
        c.weight_format = fmt
        c.fold_norm = 1
        assert binding.check_config(c) == binding.OK, fmt


def test_debug_flags_accepted():
    for flags in (binding.DEBUG_STALL, binding.DEBUG_STALL_ONCE, binding.DEBUG_STALL | binding.DEBUG_STALL_ONCE):
        c = good()
        c.debug_flags = flags
        assert binding.check_config(c) == binding.OK, flags


def test_topk_above_experts_refused():
    c = binding.make_config(1, 512, 4, 5, 64, 0)
    assert binding.check_config(c) == binding.EINVAL


def test_create_without_gpu_reports_error():
    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    with pytest.raises(binding.MoeTailError) as ei:
        binding.MoeTail(good())
    assert ei.value.status in (binding.EHIP, binding.EUNSUPPORTED)


def test_noalloc_entry_refuses_bad_configs_on_the_host():
    """moe_tail_run_noalloc validates its config before any GPU call: a bad
    field and the handle-only stall flag are refused synchronously."""
    c = good()
    c.hidden = 100
    a = binding.Args()
    assert binding.lib().moe_tail_run_noalloc(ctypes.byref(c), 1, ctypes.byref(a), None) == binding.EINVAL
    assert "hidden" in binding.strerror(None)
    c = good()
    c.debug_flags = binding.DEBUG_STALL_ONCE
    assert binding.lib().moe_tail_run_noalloc(ctypes.byref(c), 1, ctypes.byref(a), None) == binding.EINVAL
    assert "handle" in binding.strerror(None)
