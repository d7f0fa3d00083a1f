"""Seeded synthetic inputs for the decode MoE layer tail.

This module only draws random numbers and packs them into the storage formats
the layer consumes (bf16 bit patterns, FP4 E2M1 nibbles, E8M0 scale bytes).  It
holds none of the layer's arithmetic: no normalisation, routing, expert or
combine step lives here, so both the CPU oracle and the HIP path can take their
inputs from it without sharing any computation.

Workloads (the decode MoE tail of one tensor-parallel rank, 1 to 16 rows):

* ``c0`` tiny: hidden 512, 16 experts, top-2 softmax, I = Is = 64, 1 row.
* ``c1`` one-rank shard: hidden 6144, 512 MXFP4 experts, top-10 softmax,
  I = 256, shared Is = 512, 1 row.  Shape of the 512-expert / top-10 / one
  bf16 shared expert model of "Qwen3.8 monokernel K2" (sgl-project/sglang
  PR 43481, section Motivation).
* ``c2`` the c1 shard at 8 rows whose rows share a common component, so
  that about 30 % of the 80 picks repeat an expert ("--similar" rows of
  sgl-amd-mono PR 85, commit 19).
* ``c3`` hidden 7168, 256 experts, top-8 by sigmoid score plus a per-expert
  selection bias, I = Is = 256, 4 rows.
* ``c4`` hidden 8192, 384 experts, top-8 softmax, I = Is = 256, 16 rows, 1 %
  of the activation channels scaled by 20.

Value recipe (all seeded from numpy PCG64 SeedSequence([seed, config, stream,
...])): x, residual ~ bf16(N(0,1)); gamma ~ bf16(U(0.5,1.5)); router, shared
gate/up and shared down weights ~ bf16(N(0, 1/hidden)); every FP4 nibble
uniform over its 16 codes; every E8M0 scale byte 127 + U{-6..-3}; selection
bias ~ N(0, 0.1^2) in fp32.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

# stream ids of the seed tree
_S_GAMMA, _S_ROUTER, _S_BIAS, _S_W13Q, _S_W13S, _S_W2Q, _S_W2S = 1, 2, 3, 4, 5, 6, 7
_S_WS13, _S_WS2, _S_ROWS, _S_TAIL, _S_BASE = 8, 9, 10, 11, 12
_S_SGATE = 13
_S_WO, _S_ATTN = 14, 15

SOFTMAX = 0
SIGMOID_BIAS = 1


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    index: int
    rows: int
    hidden: int
    experts: int
    topk: int
    inter: int
    shared_inter: int
    scoring: int = SOFTMAX
    eps: float = 1e-6
    bias_std: float = 0.0
    heavy_frac: float = 0.0
    heavy_scale: float = 1.0
    similar: bool = False  # rows share a common Gaussian component (rho)
    n_group: int = 1  # group-limited routing: expert groups (1: none)
    topk_group: int = 1  # groups kept
    routed_scale: float = 1.0  # routed scaling factor on the top-k weights
    weight_format: int = 0  # routed experts: 0 MXFP4 (E2M1 codes), 1 MXFP8 (E4M3 codes); E8M0 block-32 scales
    fold_norm: int = 0  # 1: rstd multiplies the router and shared gate/up sums over bf16(h * gamma)
    seed: int = 0

    def with_rows(self, rows: int) -> "Config":
        return dataclasses.replace(self, rows=rows)


CONFIGS = {
    "c0": Config("c0", 0, 1, 512, 16, 2, 64, 64),
    "c1": Config("c1", 1, 1, 6144, 512, 10, 256, 512),
    "c2": Config("c2", 2, 8, 6144, 512, 10, 256, 512, similar=True),
    "c3": Config("c3", 3, 4, 7168, 256, 8, 256, 256, scoring=SIGMOID_BIAS, bias_std=0.1),
    "c4": Config("c4", 4, 16, 8192, 384, 8, 256, 256, heavy_frac=0.01, heavy_scale=20.0),
}


def _rng(cfg: Config, *stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, cfg.index, *stream])))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rand_bytes(rng: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    return np.frombuffer(bytearray(rng.bytes(n)), dtype=np.uint8).reshape(shape)


def _e4m3_codes(rng: np.random.Generator, shape) -> np.ndarray:
    v = rng.integers(0, 254, size=shape, dtype=np.uint8)
    v += v >= 0x7F  # skip 0x7F; 0xFF is never drawn
    return v


def make_weights(cfg: Config, experts: Optional[int] = None) -> dict:
    """All weights of one rank's shard, in the layouts the C ABI takes.

    w13_q [E, 2I, H/2]: byte j of a row holds K-elements 2j (low nibble) and 2j+1
    (high nibble); rows [0, I) are the gate projection, rows [I, 2I) the up
    projection.  w13_s [E, 2I, H/32]: one E8M0 byte per 32 consecutive K-elements.
    w2_q [E, H, I/2], w2_s [E, H, I/32] likewise, with K running over I.
    """
    E = cfg.experts if experts is None else experts
    H, I, Is = cfg.hidden, cfg.inter, cfg.shared_inter
    std = 1.0 / math.sqrt(H)
    w = make_router_weights(cfg, experts)
    if cfg.weight_format == 1:  # E4M3 codes uniform over the 254 that are not NaN (0x7F, 0xFF)
        w["w13_q"] = _e4m3_codes(_rng(cfg, _S_W13Q), (E, 2 * I, H))
    else:
        w["w13_q"] = _rand_bytes(_rng(cfg, _S_W13Q), (E, 2 * I, H // 2))
    w["w13_s"] = (127 + _rng(cfg, _S_W13S).integers(-6, -2, size=(E, 2 * I, H // 32))).astype(np.uint8)
    if cfg.weight_format == 1:
        w["w2_q"] = _e4m3_codes(_rng(cfg, _S_W2Q), (E, H, I))
    else:
        w["w2_q"] = _rand_bytes(_rng(cfg, _S_W2Q), (E, H, I // 2))
    w["w2_s"] = (127 + _rng(cfg, _S_W2S).integers(-6, -2, size=(E, H, I // 32))).astype(np.uint8)
    if Is > 0:
        w["ws13"] = to_bf16_bits(_rng(cfg, _S_WS13).standard_normal((2 * Is, H), dtype=np.float32) * std)
        w["ws2"] = to_bf16_bits(_rng(cfg, _S_WS2).standard_normal((H, Is), dtype=np.float32) * std)
    else:
        w["ws13"] = None
        w["ws2"] = None
    return w


def make_out_proj(cfg: Config, attn_dim: Optional[int] = None) -> dict:
    """One rank's share of the attention output projection: w_o [H, A] ~
    bf16(N(0, 1/A)) and attention rows attn [rows, A] ~ bf16(N(0, 1)), with A
    = H / 8 unless given (a square projection split over 8 ranks), each from
    a stream of its own."""
    A = cfg.hidden // 8 if attn_dim is None else attn_dim
    w_o = to_bf16_bits(_rng(cfg, _S_WO).standard_normal((cfg.hidden, A), dtype=np.float32) / np.float32(math.sqrt(A)))
    attn = to_bf16_bits(_rng(cfg, _S_ATTN).standard_normal((cfg.rows, A), dtype=np.float32))
    return {"w_o": w_o, "attn": attn}


def w13_unit_blocked(w13_q: np.ndarray, inter: int) -> np.ndarray:
    """Re-lay MXFP4 w13 codes [E, 2I, H/2] into the unit-blocked layout (same
    shape and bytes, reordered): for unit b (gate rows 8b..8b+7, up rows
    I+8b..I+8b+7), column group c (64 bytes of a row) and lane l = 16 q + i,
    16 bytes at ((b * H/128 + c) * 64 + l) * 16 are bytes 16q..16q+15 of
    column group c of unit row i.  A pure permutation of storage."""
    E, R2, HB = w13_q.shape
    I, T2 = inter, HB // 64
    assert R2 == 2 * I and HB % 64 == 0 and I % 8 == 0
    i16 = np.arange(16)
    rows = np.array([[b * 8 + i if i < 8 else I + b * 8 + i - 8 for i in i16] for b in range(I // 8)])
    x = w13_q[:, rows].reshape(E, I // 8, 16, T2, 4, 16)  # [E, b, i, c, q, byte]
    return np.ascontiguousarray(x.transpose(0, 1, 3, 4, 2, 5)).reshape(E, R2, HB)


def make_shared_gate(cfg: Config) -> np.ndarray:
    """Shared-expert gate weights [H] (bf16 bits) ~ bf16(N(0, 1/hidden)), from a
    stream of their own (the other weights do not change with or without it)."""
    std = 1.0 / math.sqrt(cfg.hidden)
    return to_bf16_bits(_rng(cfg, _S_SGATE).standard_normal(cfg.hidden, dtype=np.float32) * std)


def make_router_weights(cfg: Config, experts: Optional[int] = None) -> dict:
    """gamma [H], router_w [E, H] (bf16 bits) and router_bias [E] fp32 (or None)."""
    E = cfg.experts if experts is None else experts
    H = cfg.hidden
    std = 1.0 / math.sqrt(H)
    w = {}
    w["gamma"] = to_bf16_bits(_rng(cfg, _S_GAMMA).uniform(0.5, 1.5, H).astype(np.float32))
    w["router_w"] = to_bf16_bits((_rng(cfg, _S_ROUTER).standard_normal((E, H), dtype=np.float32) * std))
    if cfg.scoring == SIGMOID_BIAS:
        w["router_bias"] = (_rng(cfg, _S_BIAS).standard_normal(E) * cfg.bias_std).astype(np.float32)
    else:
        w["router_bias"] = None
    return w


def heavy_channels(cfg: Config) -> np.ndarray:
    """Channel indices scaled by cfg.heavy_scale (the same for every row)."""
    if cfg.heavy_frac <= 0.0:
        return np.zeros(0, dtype=np.int64)
    n = int(round(cfg.heavy_frac * cfg.hidden))
    return np.sort(_rng(cfg, _S_TAIL).choice(cfg.hidden, size=n, replace=False))


def make_row(cfg: Config, row: int, attempt: int = 0, rho: float = 0.0):
    """One decode row (x, residual) as bf16 bit patterns [H] each.

    With cfg.similar, x = sqrt(rho) z0 + sqrt(1-rho) z_row (and likewise for the
    residual), where z0 is one Gaussian vector shared by all rows of the step.
    ``attempt`` selects an independent redraw of the row's own part.
    """
    H = cfg.hidden
    g = _rng(cfg, _S_ROWS, row, attempt)
    zx = g.standard_normal(H, dtype=np.float32)
    zr = g.standard_normal(H, dtype=np.float32)
    if cfg.similar and rho > 0.0:
        b = _rng(cfg, _S_BASE)
        bx = b.standard_normal(H, dtype=np.float32)
        br = b.standard_normal(H, dtype=np.float32)
        a, c = np.float32(math.sqrt(rho)), np.float32(math.sqrt(1.0 - rho))
        zx = a * bx + c * zx
        zr = a * br + c * zr
    ch = heavy_channels(cfg)
    if ch.size:
        zx[ch] *= np.float32(cfg.heavy_scale)
    return to_bf16_bits(zx), to_bf16_bits(zr)


def make_rows(cfg: Config, attempts=None, rho: float = 0.0):
    """x, residual [R, H] uint16 for cfg.rows rows; attempts[r] picks each row's redraw."""
    R = cfg.rows
    attempts = [0] * R if attempts is None else list(attempts)
    xs, rs = [], []
    for r in range(R):
        x, res = make_row(cfg, r, attempts[r], rho)
        xs.append(x)
        rs.append(res)
    return np.stack(xs), np.stack(rs)
