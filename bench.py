"""Benchmark of the fused decode MoE layer tail on one MI355X.

A step is one call of the tail (norm, router, top-k, de-duplicated MXFP4
routed experts, bf16 shared expert, combine) over one batch of decode rows.
The headline workload is the one-rank shard at 8 rows (hidden 6144, 512
experts, top-10, I 256, shared Is 512, rows drawn so ~30 % of picks repeat).

Timing: L copies of the weights at distinct device addresses (so that the
256 MB Infinity Cache cannot serve a call from a previous call's lines), one
HIP graph of calls rotating over the copies, replayed; HIP events on the
launch stream bracket exactly K calls.  Achieved bandwidth is the algorithmic
bytes of a call (distinct selected experts' codes and scales, router, shared
expert, gamma, activations in and out) over the measured time per call.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--sweep/--no-sweep]
"""
import argparse
import dataclasses
import hashlib
import re
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from decode_moe_layer_amd import binding, synth  # noqa: E402

PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD public specification
METRIC = "µs per MoE-tail call and achieved HBM GB/s (fraction of peak) at 1/8 rows"
MALL_BYTES = 256 * 2**20


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "moe_tail_kernel_c2_8rows_hbm_traffic.txt")
KERNEL_SOURCES = (os.path.join(ROOT, "decode_moe_layer_amd", "csrc", "moe_tail.hip"),
                  os.path.join(ROOT, "decode_moe_layer_amd", "csrc", "moe_tail_device.h"),
                  os.path.join(ROOT, "decode_moe_layer_amd", "csrc", "moe_tail_wide.hip"),
                  os.path.join(ROOT, "include", "moe_tail.h"))


def kernel_source_hash():
    """SHA-256 of the kernel and ABI sources with comments and blank lines
    removed: a comment-only edit keeps the measured traffic valid, any change
    to the code does not."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f) as fh:
            text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
        for line in text.splitlines():
            line = line.split("//", 1)[0].rstrip()
            if line:
                h.update(line.encode() + b"\n")
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE summary.

    Each counter's KiB per dispatch is scaled by what the same counter reads for
    a plain device copy of known size (factors stored in the summary).  Returns
    None when the summary is absent or was taken on a different kernel source.
    """
    try:
        with open(TRAFFIC_SUMMARY) as f:
            kv = dict(l.split(":", 1) for l in f if ":" in l and not l.startswith((" ", "#", "$")))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    try:
        if kv.get("kernel_source_sha256") != kernel_source_hash():
            return None
        fetch = float(kv["fetch_kib_per_dispatch"]) * float(kv["fetch_scale"])
        write = float(kv["write_kib_per_dispatch"]) * float(kv["write_scale"])
    except (KeyError, ValueError):
        return None
    return int(round((fetch + write) * 1024))


def c2_rho():
    with open(os.path.join(ROOT, "tests", "golden", "c2_rho.json")) as f:
        return float(json.load(f)["rho"])


def per_expert_bytes(cfg):
    H, I = cfg.hidden, cfg.inter
    cb = 1 if cfg.weight_format == 1 else 2  # code bytes: MXFP8 one per element, MXFP4 one per two
    return 2 * I * H // cb + 2 * I * H // 32 + H * I // cb + H * I // 32


def alg_bytes(cfg, rows, distinct, attn_dim=0):
    H, E, Is = cfg.hidden, cfg.experts, cfg.shared_inter
    b = distinct * per_expert_bytes(cfg) + E * H * 2 + 3 * Is * H * 2 + H * 2
    if cfg.scoring == synth.SIGMOID_BIAS:
        b += E * 4
    b += rows * H * 2 * 4  # x, residual in; out, res_out out
    if attn_dim:  # the out_proj front: w_o and the attention rows in place of x
        b += H * attn_dim * 2 + rows * attn_dim * 2 - rows * H * 2
    return b


class Workload:
    """Device copies of one config's weights and rows, and a handle."""

    def __init__(self, cfg, rows, copies, torch, front=False, shuf=False):
        self.t = torch
        self.cfg = cfg.with_rows(rows)
        w = synth.make_weights(cfg)
        if shuf:  # the same codes in the unit-blocked gate/up layout
            w["w13_q"] = synth.w13_unit_blocked(w["w13_q"], cfg.inter)
        self.attn_dim = 0
        if front:  # one rank's share of a square out_proj (A = H / 8)
            f = synth.make_out_proj(self.cfg)
            w["w_o"], self.attn_dim = f["w_o"], f["w_o"].shape[1]
        rho = c2_rho() if cfg.similar else 0.0
        x, r = synth.make_rows(self.cfg, rho=rho)
        dev = lambda a: None if a is None else torch.from_numpy(
            np.ascontiguousarray(a).view(np.int16) if a.dtype == np.uint16 else np.ascontiguousarray(a)).cuda()
        base = {k: dev(v) for k, v in w.items()}
        del w
        self.copies = [base] + [{k: (None if v is None else v.clone()) for k, v in base.items()} for _ in range(copies - 1)]
        self.x, self.r = dev(x), dev(r)
        self.attn = dev(f["attn"]) if front else None
        H = cfg.hidden
        self.out = torch.empty((rows, H), dtype=torch.int16, device="cuda")
        self.res_out = torch.empty((rows, H), dtype=torch.int16, device="cuda")
        self.ids = torch.empty((rows, cfg.topk), dtype=torch.int32, device="cuda")
        c = binding.make_config(rows, H, cfg.experts, cfg.topk, cfg.inter, cfg.shared_inter, cfg.scoring, cfg.eps,
                                weight_format=cfg.weight_format, fold_norm=cfg.fold_norm, attn_dim=self.attn_dim,
                                w13_layout=1 if shuf else 0)
        self.h = binding.MoeTail(c)
        self.rows = rows

    def call(self, i, stream, ids=False):
        d = self.copies[i % len(self.copies)]
        self.h.run(self.rows, None if self.attn_dim else self.x, self.r, d["gamma"], d["router_w"], d["router_bias"],
                   d["w13_q"], d["w13_s"], d["w2_q"], d["w2_s"], d["ws13"], d["ws2"], self.out, self.res_out,
                   self.ids if ids else None, None, stream=stream.cuda_stream, attn=self.attn, w_o=d.get("w_o"))

    def distinct(self, stream):
        self.call(0, stream, ids=True)
        stream.synchronize()
        return len(set(self.ids.cpu().numpy().ravel().tolist()))

    def time(self, steps, warmup, per_graph=50):
        """µs per call over exactly `steps` calls (graph replays of `per_graph` calls)."""
        t = self.t
        s = t.cuda.Stream()
        n_full, rem = divmod(steps, per_graph)
        graphs = []
        for n in ([per_graph] if n_full else []) + ([rem] if rem else []):
            g = t.cuda.CUDAGraph()
            with t.cuda.stream(s):
                with t.cuda.graph(g, stream=s):
                    for i in range(n):
                        self.call(i, s)
            graphs.append((n, g))
        big = graphs[0][1]
        with t.cuda.stream(s):  # same stream as the timed replays: calls on one handle never overlap
            for _ in range(max(1, warmup // per_graph)):
                big.replay()
        t.cuda.synchronize()
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        e0.record(s)
        with t.cuda.stream(s):
            for _ in range(n_full):
                graphs[0][1].replay()
            if rem:
                graphs[-1][1].replay()
        e1.record(s)
        s.synchronize()
        if self.h.get_error() != binding.OK:
            raise RuntimeError("device error during timing: " + binding.strerror(self.h.h))
        return e0.elapsed_time(e1) * 1e3 / steps

    def time_eager(self, steps, warmup):
        """µs per call over exactly `steps` direct launches (no graph), for profiler runs."""
        t = self.t
        s = t.cuda.Stream()
        for i in range(warmup):
            self.call(i, s)
        s.synchronize()
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        e0.record(s)
        for i in range(steps):
            self.call(i, s)
        e1.record(s)
        s.synchronize()
        if self.h.get_error() != binding.OK:
            raise RuntimeError("device error during timing: " + binding.strerror(self.h.h))
        return e0.elapsed_time(e1) * 1e3 / steps

    def eager_us(self, reps=20):
        t = self.t
        s = t.cuda.Stream()
        for i in range(3):
            self.call(i, s)
        s.synchronize()
        t0 = time.perf_counter()
        for i in range(reps):
            self.call(i, s)
            s.synchronize()
        return (time.perf_counter() - t0) * 1e6 / reps

    def close(self):
        self.h.close()
        self.copies = None


def copies_for(cfg, rows, distinct_guess):
    b = alg_bytes(cfg, rows, distinct_guess)
    return max(3, int(np.ceil(2 * MALL_BYTES / b)) + 1)


def copy_bandwidth(torch):
    """Device-to-device copy of a 2 GiB buffer: read + write GB/s (context for the peak)."""
    n = 2**31
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    gbps = 2 * n * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    return gbps


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, seconds=10.0):
    """The oracle (plain C, fp64) on full calls of the headline workload, timed
    on this host: once on one thread, once with the rows of each call split
    over min(rows, usable cores) threads (the oracle's C code releases the
    Python lock; its arithmetic is unchanged: each thread runs whole rows)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle  # test infrastructure: only this leg of the benchmark loads it

    w = synth.make_weights(cfg)
    x, r = synth.make_rows(cfg, rho=c2_rho() if cfg.similar else 0.0)
    oracle.lib()

    def timed(fn):
        n, t0 = 0, time.perf_counter()
        while True:
            fn()
            n += 1
            if time.perf_counter() - t0 > seconds:
                return (time.perf_counter() - t0) * 1e6 / n, n

    one_us, n1 = timed(lambda: oracle.moe_tail(x, r, w, cfg))
    avail = len(os.sched_getaffinity(0))
    nt = max(1, min(avail, cfg.rows))
    pool = ThreadPoolExecutor(max_workers=nt)
    bounds = [(i * cfg.rows // nt, (i + 1) * cfg.rows // nt) for i in range(nt)]

    def split_call():
        futs = [pool.submit(oracle.moe_tail, x[a:b], r[a:b], w, cfg) for a, b in bounds]
        for f in futs:
            f.result()

    many_us, nn = timed(split_call)
    pool.shutdown()
    return {"value": round(many_us, 1), "unit": "µs per call", "cores": nt, "kind": "oracle",
            "sample": "%d full %d-row calls of %s, rows split over %d threads (%d usable cores); "
                      "single-thread: %d calls" % (nn, cfg.rows, cfg.name, nt, avail, n1),
            "single_thread_us": round(one_us, 1), "usable_cores": avail, "cpu_model": cpu_model()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--sweep", dest="sweep", action="store_true", default=True)
    ap.add_argument("--no-sweep", dest="sweep", action="store_false")
    ap.add_argument("--no-cpu", dest="cpu", action="store_false", default=True)
    ap.add_argument("--only", default=None, help="time one workload only, e.g. c2 or c1:4")
    ap.add_argument("--eager", action="store_true", help="direct launches instead of graph replay (profiling)")
    ap.add_argument("--fp8", action="store_true", help="with --only: MXFP8 (E4M3) routed experts")
    ap.add_argument("--fold", action="store_true", help="with --only: the norm folded into the router/shared sums")
    ap.add_argument("--shuf", action="store_true", help="with --only: MXFP4 gate/up codes in the unit-blocked layout")
    ap.add_argument("--front", action="store_true", help="with --only: the out_proj front (attention rows in, A = H/8)")
    ap.add_argument("--calib", action="store_true",
                    help="only run a plain 256 MiB device copy 10 times (scale for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU's share of the tail (one tensor-parallel rank); "
              "runs on more than one GPU are not part of this benchmark", file=sys.stderr)
        sys.exit(2)
    import torch

    torch.cuda.set_device(0)
    cfgs = synth.CONFIGS
    if args.calib:
        a = torch.ones(256 * 2**20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        for _ in range(10):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": a.numel(), "copies": 10}))
        return

    def measure(name, rows, fmt=0, fold=0, front=False, shuf=False, extra=False):
        cfg = dataclasses.replace(cfgs[name], weight_format=fmt, fold_norm=fold)
        guess = {1: 10, 2: 20, 4: 39, 8: 56, 16: 139}.get(rows, rows * cfg.topk)
        L = copies_for(cfg, rows, guess)
        wl = Workload(cfg, rows, L, torch, front=front, shuf=shuf)
        s = torch.cuda.Stream()
        dist = wl.distinct(s)
        us = wl.time_eager(args.steps, args.warmup) if args.eager else wl.time(args.steps, args.warmup)
        B = alg_bytes(cfg, rows, dist, wl.attn_dim)
        rec = {"workload": name + ("-mxfp8" if fmt else "") + ("-fold" if fold else "") + ("-front" if front else "") + ("-blocked" if shuf else ""),
               "rows": rows, "copies": L, "distinct_experts": dist, "alg_bytes": B,
               "us_per_call": round(us, 3), "GBps": round(B / (us * 1e-6) / 1e9, 1),
               "frac_of_peak": round(B / (us * 1e-6) / 1e9 / PEAK_GBPS, 4)}
        if extra:  # labelled context figures for the headline workload (never the value)
            e_us = wl.time_eager(args.steps, args.warmup)
            rec["eager"] = {"us_per_call": round(e_us, 3),
                            "what": "the same calls as direct launches on one stream (no graph), HIP events around them"}
            wl.close()
            torch.cuda.empty_cache()
            warm = Workload(cfg, rows, 1, torch, front=front, shuf=shuf)
            w_us = warm.time(args.steps, args.warmup)
            rec["mall_warm"] = {"us_per_call": round(w_us, 3),
                                "what": "one weight copy: every call streams the same %.0f MB, which the 256 MB MALL "
                                        "(Infinity Cache) then serves in part; not an HBM figure" % (B / 1e6)}
            warm.close()
            torch.cuda.empty_cache()
            print(json.dumps(rec), file=sys.stderr, flush=True)
            return rec
        print(json.dumps(rec), file=sys.stderr, flush=True)
        wl.close()
        torch.cuda.empty_cache()
        return rec

    if args.only:
        name, _, rows = args.only.partition(":")
        measure(name, int(rows) if rows else cfgs[name].rows, 1 if args.fp8 else 0, 1 if args.fold else 0, args.front, args.shuf)
        return

    head = measure("c2", 8, shuf=True, extra=True)  # MXFP4 gate/up codes in the unit-blocked layout
    sweep = []
    if args.sweep:
        for rows in (1, 2, 4, 16):
            sweep.append(measure("c1", rows))
        sweep.append(measure("c1", 16, shuf=True))  # 16 rows with the headline's gate/up layout
        sweep.append(head)
        sweep.append(measure("c2", 8))  # the same with row-major gate/up codes
        sweep.append(measure("c3", 4))
        sweep.append(measure("c4", 16))
        sweep.append(measure("c4", 16, shuf=True))
        sweep.append(measure("c2", 8, 1))
        sweep.append(measure("c2", 8, 0, 1))
        sweep.append(measure("c1", 1, 0, 1))
        sweep.append(measure("c1", 32))
        sweep.append(measure("c1", 32, shuf=True))
        sweep.append(measure("c2", 8, front=True))
    copy_gbps = copy_bandwidth(torch)
    cpu = cpu_baseline(cfgs["c2"]) if args.cpu else None
    us = head["us_per_call"]
    line = {
        "metric": METRIC,
        "value": us,
        "unit": "µs",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(us / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "c2: one-rank decode shard, 8 rows, hidden 6144, 512 MXFP4 experts (E2M1, "
                               "E8M0 block-32; gate/up codes in the unit-blocked layout), top-10 softmax, I 256, "
                               "bf16 shared Is 512, ~30% repeated picks",
                   "rows": 8, "distinct_experts": head["distinct_experts"], "weight_copies": head["copies"]},
        "roofline": {"bound": "hbm", "achieved": head["GBps"], "peak": PEAK_GBPS, "unit": "GB/s",
                     "frac": head["frac_of_peak"], "traffic": measured_traffic(),
                     "alg_bytes_per_call": head["alg_bytes"]},
        "cpu_baseline": cpu,
        "eager": head.get("eager"),
        "mall_warm": head.get("mall_warm"),
        "copy_GBps": round(copy_gbps, 1),
        "sweep": sweep,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
