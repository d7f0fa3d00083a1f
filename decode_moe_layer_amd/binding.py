"""ctypes binding of libmoe_tail.so (the C ABI in include/moe_tail.h).

Argument marshalling only: every step of the tail runs in the HIP kernel.
PyTorch supplies device memory and streams.  When the library is missing this
module raises; there is no other implementation to fall back to.
"""
from __future__ import annotations

import atexit
import ctypes
import os
import weakref

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_tail.so")

OK, EINVAL, EUNSUPPORTED, ENOMEM, EHIP, ETIMEOUT = 0, 1, 2, 3, 4, 5
SOFTMAX, SIGMOID_BIAS = 0, 1
MXFP4, MXFP8 = 0, 1
DEBUG_STALL = 1
DEBUG_STALL_ONCE = 2
STATUS_NAMES = {0: "OK", 1: "EINVAL", 2: "EUNSUPPORTED", 3: "ENOMEM", 4: "EHIP", 5: "ETIMEOUT"}

EXPORTS = ("moe_tail_check_config", "moe_tail_create", "moe_tail_run", "moe_tail_get_error",
           "moe_tail_strerror", "moe_tail_destroy", "moe_tail_run_noalloc")
NOALLOC_SCRATCH_BYTES = 4 << 20


class Config(ctypes.Structure):
    _fields_ = [
        ("max_rows", ctypes.c_int32), ("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("inter", ctypes.c_int32), ("shared_inter", ctypes.c_int32),
        ("scoring", ctypes.c_int32), ("eps", ctypes.c_float), ("device", ctypes.c_int32),
        ("deadline_us", ctypes.c_uint32), ("debug_flags", ctypes.c_uint32), ("debug_block", ctypes.c_int32),
        ("n_group", ctypes.c_int32), ("topk_group", ctypes.c_int32), ("routed_scale", ctypes.c_float),
        ("weight_format", ctypes.c_int32), ("fold_norm", ctypes.c_int32), ("attn_dim", ctypes.c_int32),
        ("w13_layout", ctypes.c_int32),
    ]


class Args(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "x", "residual", "gamma", "router_w", "router_bias", "w13_q", "w13_s", "w2_q", "w2_s", "ws13", "ws2",
        "out", "res_out", "topk_ids", "topk_w", "dbg_logits", "dbg_y_routed", "dbg_y_shared", "shared_gate", "attn",
        "w_o")]


class MoeTailError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), msg))
        self.status = status


_lib = None
_live = weakref.WeakSet()  # open handles, closed at interpreter exit before the HIP runtime tears down


@atexit.register
def _close_live_handles():
    for h in list(_live):
        try:
            h.close()
        except Exception:
            pass


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoeTailError(EHIP, "libmoe_tail.so is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        L.moe_tail_check_config.restype = ctypes.c_int
        L.moe_tail_check_config.argtypes = [ctypes.POINTER(Config)]
        L.moe_tail_create.restype = ctypes.c_int
        L.moe_tail_create.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(vp)]
        L.moe_tail_run.restype = ctypes.c_int
        L.moe_tail_run.argtypes = [vp, ctypes.c_int32, ctypes.POINTER(Args), vp]
        L.moe_tail_get_error.restype = ctypes.c_int
        L.moe_tail_get_error.argtypes = [vp]
        L.moe_tail_strerror.restype = ctypes.c_char_p
        L.moe_tail_strerror.argtypes = [vp]
        L.moe_tail_destroy.restype = None
        L.moe_tail_destroy.argtypes = [vp]
        L.moe_tail_run_noalloc.restype = ctypes.c_int
        L.moe_tail_run_noalloc.argtypes = [ctypes.POINTER(Config), ctypes.c_int32, ctypes.POINTER(Args), vp]
        _lib = L
    return _lib


def make_config(max_rows, hidden, num_experts, top_k, inter, shared_inter, scoring=SOFTMAX, eps=1e-6,
                device=-1, deadline_us=0, debug_flags=0, debug_block=0, n_group=1, topk_group=1,
                routed_scale=1.0, weight_format=MXFP4, fold_norm=0, attn_dim=0, w13_layout=0) -> Config:
    return Config(max_rows, hidden, num_experts, top_k, inter, shared_inter, scoring, eps, device, deadline_us,
                  debug_flags, debug_block, n_group, topk_group, routed_scale, weight_format, fold_norm, attn_dim,
                  w13_layout)


def check_config(cfg: Config) -> int:
    return lib().moe_tail_check_config(ctypes.byref(cfg))


def strerror(handle=None) -> str:
    s = lib().moe_tail_strerror(handle)
    return s.decode() if s else ""


def _args(x, residual, gamma, router_w, router_bias, w13_q, w13_s, w2_q, w2_s, ws13, ws2, out, res_out=None,
          topk_ids=None, topk_w=None, dbg_logits=None, dbg_y_routed=None, dbg_y_shared=None, shared_gate=None,
          attn=None, w_o=None):
    return Args(*[_ptr(t) for t in (x, residual, gamma, router_w, router_bias, w13_q, w13_s, w2_q, w2_s, ws13, ws2,
                                    out, res_out, topk_ids, topk_w, dbg_logits, dbg_y_routed, dbg_y_shared,
                                    shared_gate, attn, w_o)])


def _stream(stream):
    if stream is None:
        import torch

        stream = torch.cuda.current_stream().cuda_stream
    return stream


def run_noalloc(cfg: Config, rows, *tensors, stream=None, **kw):
    """moe_tail_run_noalloc: one call with no handle (the library's static scratch); same
    tensor arguments as MoeTail.run."""
    a = _args(*tensors, **kw)
    st = lib().moe_tail_run_noalloc(ctypes.byref(cfg), rows, ctypes.byref(a), ctypes.c_void_p(_stream(stream)))
    if st != OK:
        raise MoeTailError(st, strerror(None))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


class MoeTail:
    """One handle: create() at construction, run() per call, destroy() on close()."""

    def __init__(self, cfg: Config):
        self.cfg = cfg
        h = ctypes.c_void_p()
        st = lib().moe_tail_create(ctypes.byref(cfg), ctypes.byref(h))
        if st != OK:
            raise MoeTailError(st, strerror(None))
        self.h = h
        _live.add(self)

    def run(self, rows, x, residual, gamma, router_w, router_bias, w13_q, w13_s, w2_q, w2_s, ws13, ws2, out,
            res_out=None, topk_ids=None, topk_w=None, dbg_logits=None, dbg_y_routed=None, dbg_y_shared=None,
            stream=None, shared_gate=None, attn=None, w_o=None):
        """Enqueue one call; tensors are torch device tensors (or raw device addresses).
        With attn (and w_o) the library computes x itself (the out_proj front); pass x=None."""
        a = Args(*[_ptr(t) for t in (x, residual, gamma, router_w, router_bias, w13_q, w13_s, w2_q, w2_s, ws13,
                                     ws2, out, res_out, topk_ids, topk_w, dbg_logits, dbg_y_routed, dbg_y_shared,
                                     shared_gate, attn, w_o)])
        if stream is None:
            import torch

            stream = torch.cuda.current_stream().cuda_stream
        st = lib().moe_tail_run(self.h, rows, ctypes.byref(a), ctypes.c_void_p(stream))
        if st != OK:
            raise MoeTailError(st, strerror(self.h))

    def get_error(self) -> int:
        return lib().moe_tail_get_error(self.h)

    def close(self):
        if getattr(self, "h", None):
            lib().moe_tail_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
