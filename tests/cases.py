"""Test inputs: seeded rows from the generator, redrawn until the top-k is well posed.

A row is kept only when its K-th and (K+1)-th selection keys, as the oracle
computes them in double precision, differ by at least 1e-4 relative:
(k_K - k_{K+1}) >= 1e-4 * max(|k_K|, |k_{K+1}|).  A failing row is redrawn
with the next attempt index of its own seed.  Test infrastructure: calls the
oracle.
"""
import functools
import json
import os

import numpy as np

import oracle
from decode_moe_layer_amd import synth

GAP_REL = 1e-4
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def c2_rho() -> float:
    with open(os.path.join(GOLDEN, "c2_rho.json")) as f:
        return float(json.load(f)["rho"])


def rho_for(cfg) -> float:
    return c2_rho() if cfg.similar else 0.0


def key_gaps(keys: np.ndarray, k: int) -> np.ndarray:
    """Relative gap between the k-th and (k+1)-th largest key of each row."""
    if k >= keys.shape[1]:
        return np.full(keys.shape[0], np.inf)
    s = -np.sort(-keys, axis=1)
    a, b = s[:, k - 1], s[:, k]
    return (a - b) / np.maximum(np.maximum(np.abs(a), np.abs(b)), 1e-300)


def gapped_rows(cfg, rw: dict, rho: float = None, max_attempts: int = 64):
    """x, res [R, H] whose every row passes the gap rule; also returns attempts."""
    rho = rho_for(cfg) if rho is None else rho
    attempts = [0] * cfg.rows
    xs, rs = [], []
    for r in range(cfg.rows):
        for a in range(max_attempts):
            x, res = synth.make_row(cfg, r, a, rho)
            _, ky = oracle.router_keys(x[None], res[None], rw, cfg)
            if key_gaps(ky, cfg.topk)[0] >= GAP_REL:
                attempts[r] = a
                break
        else:
            raise RuntimeError("no well-posed row found")
        xs.append(x)
        rs.append(res)
    return np.stack(xs), np.stack(rs), attempts


@functools.lru_cache(maxsize=2)
def weights(name: str):
    return synth.make_weights(synth.CONFIGS[name])


def oracle_rows(x, r, w, cfg):
    """oracle.moe_tail on rows x, r, with the rows split over threads (the
    oracle's C code releases the interpreter lock).  Rows are independent in
    the method, so each thread's rows are whole calls and the results are
    concatenated row by row."""
    from concurrent.futures import ThreadPoolExecutor

    R = x.shape[0]
    nt = max(1, min(R, len(os.sched_getaffinity(0)), 16))
    bounds = [(i * R // nt, (i + 1) * R // nt) for i in range(nt)]
    with ThreadPoolExecutor(max_workers=nt) as pool:
        parts = list(pool.map(lambda b: oracle.moe_tail(x[b[0]:b[1]], None if r is None else r[b[0]:b[1]], w,
                                                        cfg.with_rows(b[1] - b[0])), bounds))
    return {k: (np.concatenate([p[k] for p in parts]) if isinstance(parts[0][k], np.ndarray) and parts[0][k].ndim >= 1
                and parts[0][k].shape[0] == bounds[0][1] - bounds[0][0] else parts[0][k]) for k in parts[0]}

