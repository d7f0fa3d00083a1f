"""CPU oracle of the decode MoE layer tail -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never loads it and never falls back to it.

This module is a thin ctypes wrapper over ``moe_oracle.c`` (plain C, IEEE
double).  The C file carries the definition of every step and its sources.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no HIP, no GPU)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        )
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        d, i, p = ctypes.c_double, ctypes.c_int, ctypes.c_void_p
        L.oracle_e2m1.restype = d
        L.oracle_e2m1.argtypes = [i]
        L.oracle_e8m0.restype = d
        L.oracle_e8m0.argtypes = [i]
        L.oracle_dequant.restype = d
        L.oracle_dequant.argtypes = [i, i]
        L.oracle_bf16_round.restype = ctypes.c_uint16
        L.oracle_bf16_round.argtypes = [d]
        L.oracle_bf16_to_double.restype = d
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_topk.restype = None
        L.oracle_topk.argtypes = [i, i, p, p]
        L.oracle_topk_weights.restype = None
        L.oracle_topk_weights.argtypes = [i, i, p, p, p]
        L.oracle_keys.restype = None
        L.oracle_keys.argtypes = [i, i, p, p, p]
        L.oracle_norm_row.restype = None
        L.oracle_norm_row.argtypes = [i, d, p, p, p, p, p, p]
        L.oracle_moe_tail.restype = i
        L.oracle_moe_tail.argtypes = [i, i, i, i, i, i, i, d, i, i, d, i, i] + [p] * 21
        L.oracle_e4m3.restype = d
        L.oracle_e4m3.argtypes = [i]
        L.oracle_topk_grouped.restype = None
        L.oracle_topk_grouped.argtypes = [i, i, p, i, i, p]
        L.oracle_out_proj.restype = None
        L.oracle_out_proj.argtypes = [i, i, i, p, p, p, p]
        L.oracle_router_keys.restype = i
        L.oracle_router_keys.argtypes = [i, i, i, i, d, i] + [p] * 7
        _lib = L
    return _lib


def _ptr(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def e2m1(code: int) -> float:
    return lib().oracle_e2m1(code)


def e8m0(b: int) -> float:
    return lib().oracle_e8m0(b)


def dequant(code: int, scale_byte: int) -> float:
    return lib().oracle_dequant(code, scale_byte)


def bf16_round(v: float) -> int:
    return int(lib().oracle_bf16_round(float(v)))


def bf16_value(bits: int) -> float:
    return lib().oracle_bf16_to_double(int(bits))


def topk(keys: np.ndarray, k: int) -> np.ndarray:
    keys = np.ascontiguousarray(keys, dtype=np.float64)
    ids = np.zeros(k, dtype=np.int32)
    lib().oracle_topk(keys.size, k, _ptr(keys), _ptr(ids))
    return ids


def e4m3(code: int) -> float:
    return lib().oracle_e4m3(code)


def topk_grouped(keys: np.ndarray, k: int, n_group: int, topk_group: int) -> np.ndarray:
    keys = np.ascontiguousarray(keys, dtype=np.float64)
    ids = np.zeros(k, dtype=np.int32)
    lib().oracle_topk_grouped(keys.size, k, _ptr(keys), n_group, topk_group, _ptr(ids))
    return ids


def topk_weights(logits: np.ndarray, ids: np.ndarray, scoring: int) -> np.ndarray:
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.zeros(ids.size, dtype=np.float64)
    lib().oracle_topk_weights(ids.size, scoring, _ptr(logits), _ptr(ids), _ptr(w))
    return w


def keys(logits: np.ndarray, scoring: int, bias: Optional[np.ndarray]) -> np.ndarray:
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    out = np.zeros_like(logits)
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    lib().oracle_keys(logits.size, scoring, _ptr(logits), _ptr(b), _ptr(out))
    return out


def norm_row(x: np.ndarray, r: Optional[np.ndarray], gamma: np.ndarray, eps: float):
    H = x.size
    x = np.ascontiguousarray(x, dtype=np.uint16)
    r = None if r is None else np.ascontiguousarray(r, dtype=np.uint16)
    gamma = np.ascontiguousarray(gamma, dtype=np.uint16)
    h = np.zeros(H, dtype=np.uint16)
    xn = np.zeros(H, dtype=np.uint16)
    rstd = np.zeros(1, dtype=np.float64)
    lib().oracle_norm_row(H, float(np.float32(eps)), _ptr(x), _ptr(r), _ptr(gamma), _ptr(h), _ptr(xn), _ptr(rstd))
    return h, xn, float(rstd[0])


def router_keys(x, r, w: dict, cfg):
    """Logits and selection keys [rows, E] (norm + router only)."""
    R = x.shape[0]
    lg = np.zeros((R, cfg.experts), dtype=np.float64)
    ky = np.zeros((R, cfg.experts), dtype=np.float64)
    bias = w.get("router_bias")
    lib().oracle_router_keys(
        R, cfg.hidden, cfg.experts, cfg.scoring, float(np.float32(cfg.eps)), getattr(cfg, "fold_norm", 0),
        _ptr(np.ascontiguousarray(x)), _ptr(None if r is None else np.ascontiguousarray(r)),
        _ptr(w["gamma"]), _ptr(w["router_w"]), _ptr(bias), _ptr(lg), _ptr(ky),
    )
    return lg, ky


def moe_tail(x, r, w: dict, cfg) -> dict:
    """Run the whole tail on rows x [R, H] (bf16 bits) with residual r (or None).

    Returns a dict with h, xn, out ([R, H] bf16 bits), logits, keys ([R, E]
    float64), ids ([R, K] int32), w ([R, K] float64), y_routed, y_shared
    ([R, H] float64).  w may hold "shared_gate" ([H] bf16 bits): the shared
    output is then scaled by sigmoid(shared_gate . xn); y_shared is gated.
    cfg.fold_norm (if set) folds the norm's rstd into the router and shared
    gate/up sums, which then project bf16(h * gamma).
    """
    R, H = x.shape
    E, K, I, Is = cfg.experts, cfg.topk, cfg.inter, cfg.shared_inter
    o = {
        "h": np.zeros((R, H), np.uint16), "xn": np.zeros((R, H), np.uint16), "out": np.zeros((R, H), np.uint16),
        "logits": np.zeros((R, E)), "keys": np.zeros((R, E)), "ids": np.zeros((R, K), np.int32),
        "w": np.zeros((R, K)), "y_routed": np.zeros((R, H)), "y_shared": np.zeros((R, H)),
    }
    rc = lib().oracle_moe_tail(
        R, H, E, K, I, Is, cfg.scoring, float(np.float32(cfg.eps)), getattr(cfg, "n_group", 1),
        getattr(cfg, "topk_group", 1), float(np.float32(getattr(cfg, "routed_scale", 1.0))),
        getattr(cfg, "weight_format", 0), getattr(cfg, "fold_norm", 0),
        _ptr(np.ascontiguousarray(x)), _ptr(None if r is None else np.ascontiguousarray(r)), _ptr(w["gamma"]),
        _ptr(w["router_w"]), _ptr(w.get("router_bias")), _ptr(w["w13_q"]), _ptr(w["w13_s"]), _ptr(w["w2_q"]),
        _ptr(w["w2_s"]), _ptr(w.get("ws13")), _ptr(w.get("ws2")), _ptr(w.get("shared_gate")), _ptr(o["h"]),
        _ptr(o["xn"]), _ptr(o["logits"]),
        _ptr(o["keys"]), _ptr(o["ids"]), _ptr(o["w"]), _ptr(o["y_routed"]), _ptr(o["y_shared"]), _ptr(o["out"]),
    )
    if rc != 0:
        raise ValueError("oracle_moe_tail rejected its arguments")
    return o


def out_proj(attn: np.ndarray, w_o: np.ndarray):
    """x = bf16(attn . w_o^T) (bf16 bits [rows, H]) and the unrounded y
    (float64), for attn [rows, A] and w_o [H, A] in bf16 bits."""
    attn = np.ascontiguousarray(attn, dtype=np.uint16)
    w_o = np.ascontiguousarray(w_o, dtype=np.uint16)
    R, A = attn.shape
    H = w_o.shape[0]
    assert w_o.shape[1] == A
    y = np.zeros((R, H), dtype=np.float64)
    x = np.zeros((R, H), dtype=np.uint16)
    lib().oracle_out_proj(R, A, H, _ptr(attn), _ptr(w_o), _ptr(y), _ptr(x))
    return x, y
