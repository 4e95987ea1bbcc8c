#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

A step is one decode step of the named workload through the HIP library:
  dense61k    (default) Qwen3-4B-shaped layer: 8 KV heads, 32 query heads, d=128,
              n=61,440 bf16, batch 1: cached_attn_lse + lse_merge_local (256 local tokens)
  shared36    36 layers of one shared 61,440-token document, 16 queries, 512 private
              local tokens each: 36 x dense_decode_step (cached_attn_lse + lse_merge_local)
  sparse128k  HashAttention step: 8 KV heads, 32 query heads, n=131,072 bf16, batch 8,
              m = n/32 + 128 sink + 128 recent: sig_score_topk + gather_attn
  quadrature  Nectar's quadrature module as cached_attn_lse: 256 queries against p = 6,144 shared
              (W, Z) pairs per KV head (the 10 % module of a 61,440-token document); MFMA-bound
  sigwidth    sig_score_topk_w on the sparse128k shape with random codes of 32 to 512 bits (value: 256)
  needles512k n=524,288 bf16, batch 4, 64 planted needles per head: the sparse step (m=n/64)
              against cached_attn_lse on the same inputs, with needle recall, attention mass
              captured and the sparse output's error against the dense one

Inputs are synthetic (seeded, drawn on the GPU) and resident in HBM before the timed
region.  Several independent input sets are cycled so that the bytes a cycle touches
exceed the 256 MB last-level cache.  One JSON line is printed.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from long_context_decode_attn_amd import ops, synth, traffic  # noqa: E402
from long_context_decode_attn_amd.profsum import kernel_source_digest  # noqa: E402

HBM_PEAK = 8.0e12   # B/s, MI355X published peak
FP64_PEAK = 78.6e12  # FLOP/s, MI355X published fp64 vector peak
MFMA_BF16_PEAK = 2.5e15   # FLOP/s, MI355X published dense bf16 matrix peak
METRIC = "decode-attention queries/sec + achieved HBM TB/s (KV+sig bytes) vs ~8 TB/s peak"


class Timer:
    """HIP events on torch's current stream (the stream the library launches on)."""

    def __init__(self):
        self.s = torch.cuda.Event(enable_timing=True)
        self.e = torch.cuda.Event(enable_timing=True)

    def start(self):
        self.s.record()

    def stop_ms(self):
        self.e.record()
        self.e.synchronize()
        return self.s.elapsed_time(self.e)


def maybe_graph(fn, use_graph: bool):
    """Capture fn (a sequence of library calls on the current stream) into a HIP graph."""
    if not use_graph:
        return fn
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                          # warm the allocator and the code paths outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g.replay


def run_steps_stats(step_fns, steps: int, warmup: int, use_graph: bool, replays: int = 20) -> dict:
    """Time exactly `steps` steps, step i running step_fns[i % len(step_fns)], as R = min(replays, steps)
    back-to-back replays of steps // R steps (and one replay of the remainder, if any), each bracketed by HIP
    events on the current stream.

    With use_graph the warmup steps, a replay and the remainder are each captured into one HIP graph, so the
    timed region holds exactly `steps` steps and no per-step host launch.  Returns the whole region's time and
    the median, 10th and 90th percentiles of the replays' time per step."""
    R = max(1, min(replays, steps))
    per = steps // R
    rem = steps - per * R

    def seq(count):
        def f():
            for i in range(count):
                step_fns[i % len(step_fns)]()
        return f
    warm = maybe_graph(seq(max(warmup, 1)), use_graph)
    one = maybe_graph(seq(per), use_graph)
    tail = maybe_graph(seq(rem), use_graph) if rem else None
    warm()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(R + 2)]
    ev[0].record()
    for r in range(R):
        one()
        ev[r + 1].record()
    last = R
    if tail is not None:
        tail()
        ev[R + 1].record()
        last = R + 1
    ev[last].synchronize()
    total = ev[0].elapsed_time(ev[last])
    torch.cuda.synchronize()
    per_step = [ev[r].elapsed_time(ev[r + 1]) / per for r in range(R)]
    pct = lambda f: float(np.percentile(per_step, f))
    return {"ms": total, "ms_per_step": total / steps, "replays": R, "steps_per_replay": per,
            "median_ms_per_step": pct(50), "p10_ms_per_step": pct(10), "p90_ms_per_step": pct(90)}


def run_steps(step_fns, steps: int, warmup: int, use_graph: bool) -> float:
    """Time exactly `steps` steps (see run_steps_stats); returns ms."""
    return run_steps_stats(step_fns, steps, warmup, use_graph)["ms"]


def replay_stats(st: dict) -> dict:
    """The per-step spread over the timed replays, in microseconds."""
    return {"replays": st["replays"], "steps_per_replay": st["steps_per_replay"],
            "median_us_per_step": st["median_ms_per_step"] * 1e3, "p10_us_per_step": st["p10_ms_per_step"] * 1e3,
            "p90_us_per_step": st["p90_ms_per_step"] * 1e3}


# ------------------------------------------------------------------ dense ----
class DenseLayer:
    """Preallocated inputs/outputs/workspace of cached_attn_lse + lse_merge_local for one input set."""

    def __init__(self, cfg, rot, layer=0, device="cuda"):
        x = synth.make_inputs(cfg, device=device, rot=rot, layer=layer)
        self.x = x
        B, Hq = x["q"].shape[:2]
        Hkv, n = x["k"].shape[1], x["k"].shape[2]
        stride = 0 if cfg.shared_doc else Hkv * n * 128
        self.a = torch.empty((B, Hq, 128), device=device)
        self.al = torch.empty((B, Hq), device=device)
        self.o = torch.empty((B, Hq, 128), device=device)
        self.oa = torch.empty((B, Hq), device=device)
        nb = max(ops.ws_bytes_cached_attn_lse(B, Hq, Hkv, 128, n, stride),
                 ops.ws_bytes_lse_merge_local(B, Hq, Hkv, 128, x["k_loc"].shape[2]),
                 ops.ws_bytes_dense_decode_step(B, Hq, Hkv, 128, n, stride, x["k_loc"].shape[2]))
        self.ws = torch.empty(nb, dtype=torch.uint8, device=device)

    def attn(self):
        ops.cached_attn_lse(self.x["q"], self.x["k"], self.x["v"], out=self.a, alpha=self.al, ws=self.ws)

    def merge(self):
        ops.lse_merge_local(self.x["q"], self.a, self.al, self.x["k_loc"], self.x["v_loc"], self.x["n_loc"],
                            out=self.o, alpha_out=self.oa, ws=self.ws)

    def step_two_calls(self):
        self.attn()
        self.merge()

    def step(self):
        ops.dense_decode_step(self.x["q"], self.x["k"], self.x["v"], self.x["k_loc"], self.x["v_loc"],
                              self.x["n_loc"], out=self.o, alpha_out=self.oa, ws=self.ws)


def bench_dense(args, cfg, layers=1):
    rot = args.rot if args.rot else (8 if layers == 1 else 1)
    sets = [[DenseLayer(cfg, r, layer=l) for l in range(layers)] for r in range(rot)]
    torch.cuda.synchronize()
    B = cfg.B

    def make(r, what):
        def f():
            for L in sets[r]:
                getattr(L, what)()
        return f

    steps = args.steps
    st = run_steps_stats([make(r, "step") for r in range(rot)], steps, args.warmup, args.graph)
    ms_step = st["ms_per_step"]
    # the same step as the two separate calls, and the dominant call alone
    ms_two = run_steps([make(r, "step_two_calls") for r in range(rot)], steps, args.warmup, args.graph) / steps
    ms_a = run_steps([make(r, "attn") for r in range(rot)], steps, args.warmup, args.graph) / (steps * layers)

    n_loc_total = int(sets[0][0].x["n_loc"].sum().item())
    layer_bytes = traffic.dense_step_bytes(B, cfg.Hq, cfg.Hkv, cfg.d, cfg.n, 2, cfg.shared_doc, n_loc_total,
                                           fused=True)
    two_call_bytes = layers * traffic.dense_step_bytes(B, cfg.Hq, cfg.Hkv, cfg.d, cfg.n, 2, cfg.shared_doc,
                                                       n_loc_total)
    step_bytes = layers * layer_bytes
    attn_bytes = traffic.dense_step_bytes(B, cfg.Hq, cfg.Hkv, cfg.d, cfg.n, 2, cfg.shared_doc, 0)
    # The dominant kernel: one split-KV launch per layer and step (bf16, one cache per batch item:
    # k_split_mfma over cache + local tokens with the LSE combine inside).  Its launches run back to back
    # in the timed graph, so its average launch duration is the per-layer step time.
    fused = not cfg.shared_doc
    launch_us = ms_step * 1e3 / layers
    achieved = layer_bytes / (launch_us * 1e-6)
    res = {
        "value": B / (ms_step * 1e-3),
        "ms_per_step": ms_step,
        "steps": steps,
        "step_bytes": step_bytes,
        "step_tbps": step_bytes / (ms_step * 1e-3) / 1e12,
        "roofline": {"bound": "hbm", "achieved": achieved / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK,
                     "traffic": traffic_from_profile("split_mfma_dense61k", layer_bytes) if fused else
                                traffic_from_profile("split_rows_shared36", layer_bytes, "split_rows"),
                     "kernel": ("k_split_mfma (dense_decode_step: cache + local tokens, LSE combine in-kernel; "
                                "one launch per layer)") if fused else
                               ("k_split_rows_pair + k_combine_small per layer (dense_decode_step on a shared document: "
                                "64-row document pass that also takes each row's local tokens, then the combine; "
                                "avg_launch_us is the per-layer time of the pair)"),
                     "bytes_per_launch": layer_bytes, "avg_launch_us": launch_us},
        "rotations": rot,
        "step_spread": replay_stats(st),
        "two_call_ms_per_step": ms_two,
        "two_call_tbps": two_call_bytes / (ms_two * 1e-3) / 1e12,
        "cached_attn_lse_us": ms_a * 1e3,
        "cached_attn_lse_tbps": attn_bytes / (ms_a * 1e-3) / 1e12,
    }
    return res, sets[0][0]


# ---------------------------------------------------------------- traffic ----
def traffic_from_profile(name: str, algorithmic_bytes: int, kind: str = "split_mfma"):
    """HBM bytes per launch of the dominant kernel from the committed counter summary
    profiles/traffic_<name>.txt (FETCH_SIZE and WRITE_SIZE per dispatch, each scaled by the
    same counter's reading for a copy of known size).  None when there is no summary or the
    kernel sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.txt" % name)
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_digest") != kernel_source_digest(kind):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def hbm_context(nbytes: int = 4 << 30, reps: int = 5, probe_bytes: int = 8 << 30) -> dict:
    """The box's measured read ceiling: the library's streaming-read probe (lcda_stream_read, a hand-written
    kernel in which each workgroup streams one contiguous share with up to sixteen 16-byte nontemporal loads
    per thread in flight) over probe_bytes at several grid sizes, best rate kept; and, as context, a float32
    sum over nbytes (reads nbytes) and a copy of nbytes / 2 (reads and writes it) through plain torch
    kernels."""
    buf = torch.empty(probe_bytes, dtype=torch.uint8, device="cuda").fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    t = Timer()
    probe = {}
    for per_cu in (1, 2, 4, 8):
        wgs = cus * per_cu
        ops.stream_read(buf, wgs, sink)
        torch.cuda.synchronize()
        best = float("inf")
        for _ in range(reps):
            t.start()
            ops.stream_read(buf, wgs, sink)
            best = min(best, t.stop_ms())
        probe["%d_workgroups" % wgs] = probe_bytes / (best * 1e-3) / 1e12
    del buf
    x = torch.ones(nbytes // 4, device="cuda")
    y = torch.empty(nbytes // 8, device="cuda")
    x.sum()
    torch.cuda.synchronize()
    t.start()
    for _ in range(reps):
        x.sum()
    ms_sum = t.stop_ms() / reps
    src = x[: nbytes // 8]
    y.copy_(src)
    torch.cuda.synchronize()
    t.start()
    for _ in range(reps):
        y.copy_(src)
    ms_copy = t.stop_ms() / reps
    del x, y
    torch.cuda.empty_cache()
    return {"stream_read_peak_tbps": max(probe.values()), "stream_read_tbps_by_grid": probe,
            "sum_read_tbps": nbytes / (ms_sum * 1e-3) / 1e12,
            "copy_read_plus_write_tbps": nbytes / (ms_copy * 1e-3) / 1e12,
            "bytes": nbytes, "probe_bytes": probe_bytes,
            "note": "lcda_stream_read over 8 GiB (best of %d per grid, fastest grid); torch.sum and Tensor.copy_ "
                    "over 4 GiB; event-timed" % reps}


def calibrate_copy(nbytes: int, reps: int) -> dict:
    """A plain device-to-device copy of known size (the counter calibration kernel)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t = Timer()
    t.start()
    for _ in range(reps):
        dst.copy_(src)
    ms = t.stop_ms() / reps
    return {"copy_bytes": nbytes, "reps": reps, "read_bytes": nbytes, "write_bytes": nbytes,
            "ms_per_copy": ms, "tbps_read_plus_write": 2 * nbytes / (ms * 1e-3) / 1e12}


# ----------------------------------------------------------------- sparse ----
class SparseSet:
    def __init__(self, cfg, rot, device="cuda", n=None, B=None):
        x = synth.make_inputs(cfg, device=device, rot=rot, n=n, B=B)
        self.x = x
        self.cfg = cfg
        B, Hq = x["q"].shape[:2]
        Hkv, n = x["k"].shape[1], x["k"].shape[2]
        self.cap = ops.capacity(n, cfg.m, cfg.n_sink, cfg.n_recent)
        self.idx = torch.zeros((B, Hq, self.cap), dtype=torch.int32, device=device)
        self.cnt = torch.zeros((B, Hq), dtype=torch.int32, device=device)
        self.o = torch.empty((B, Hq, 128), device=device)
        self.oa = torch.empty((B, Hq), device=device)
        nb = max(ops.ws_bytes_sig_score_topk(B, Hq, Hkv, n), ops.ws_bytes_gather_attn(B, Hq, Hkv, 128, self.cap),
                 ops.ws_bytes_sparse_decode_step(B, Hq, Hkv, 128, n, self.cap))
        self.ws = torch.empty(nb, dtype=torch.uint8, device=device)

    def topk(self):
        c = self.cfg
        ops.sig_score_topk(self.x["key_sigs"], self.x["q_sigs"], c.m, c.n_sink, c.n_recent, cap=self.cap,
                           idx=self.idx, count=self.cnt, ws=self.ws)

    def gather(self):
        ops.gather_attn(self.x["q"], self.x["k"], self.x["v"], self.idx, self.cnt, out=self.o, alpha=self.oa,
                        ws=self.ws)

    def step_two_calls(self):
        self.topk()
        self.gather()

    def step(self):
        c = self.cfg
        ops.sparse_decode_step(self.x["key_sigs"], self.x["q_sigs"], self.x["q"], self.x["k"], self.x["v"], c.m,
                               c.n_sink, c.n_recent, cap=self.cap, idx=self.idx, count=self.cnt, out=self.o,
                               alpha=self.oa, ws=self.ws)

    # T_map (random projection): the query codes, and the codes of one new key per (b, KV head)
    def tmap_setup(self):
        c = self.cfg
        self.R = synth.projection(128, 32, c.cid, device=self.x["q"].device).float()
        self.qs_enc = torch.empty_like(self.x["q_sigs"])
        B, Hkv, n = self.x["key_sigs"].shape
        self.codes_tail = torch.empty((B, Hkv, n), dtype=torch.int32, device=self.x["q"].device)

    def encode_q(self):
        ops.sig_encode(self.x["q"], self.R, codes=self.qs_enc)

    def append_key(self):
        n = self.x["k"].shape[2]
        ops.sig_encode(self.x["k"][:, :, n - 1:n], self.R, codes=self.codes_tail[:, :, n - 1:n])

    def encode_cache(self):
        ops.sig_encode(self.x["k"], self.R, codes=self.codes_tail)

    def topk_q(self):
        c = self.cfg
        ops.sig_score_topk_q(self.x["key_sigs"], self.x["q"], self.R, c.m, c.n_sink, c.n_recent, cap=self.cap,
                             idx=self.idx, count=self.cnt, q_sigs=self.qs_enc, ws=self.ws)


def bench_tmap(args, sets, cfg):
    """Timings of the T_map stage (N2) on the sparse workload's inputs."""
    for s in sets:
        s.tmap_setup()
    torch.cuda.synchronize()
    steps = max(10, args.steps // 2)
    us = lambda fns, k=steps: run_steps(fns, k, max(2, args.warmup // 4), args.graph) / k * 1e3
    rows = cfg.B * cfg.Hkv * cfg.n
    t_cache = us([s.encode_cache for s in sets], 5)
    return {"encode_queries_us": us([s.encode_q for s in sets]),
            "append_one_key_per_head_us": us([s.append_key for s in sets]),
            "sig_score_topk_q_us": us([s.topk_q for s in sets]),
            "encode_whole_cache_us": t_cache,
            "encode_whole_cache_rows_per_s": rows / (t_cache * 1e-6),
            "encode_whole_cache_fp64_tflops": rows * 32 * 128 * 2 / (t_cache * 1e-6) / 1e12,
            "encode_whole_cache_frac_of_fp64_peak": rows * 32 * 128 * 2 / (t_cache * 1e-6) / FP64_PEAK}


def bench_sparse(args, cfg, rot=None):
    rot = rot or args.rot or 2
    sets = [SparseSet(cfg, r) for r in range(rot)]
    torch.cuda.synchronize()

    steps = args.steps
    st = run_steps_stats([s.step for s in sets], steps, args.warmup, args.graph)
    ms_step = st["ms_per_step"]
    ms_two = run_steps([s.step_two_calls for s in sets], steps, args.warmup, args.graph) / steps
    ms_g = run_steps([s.gather for s in sets], steps, args.warmup, args.graph) / steps
    ms_t = run_steps([s.topk for s in sets], steps, args.warmup, args.graph) / steps
    G = cfg.Hq // cfg.Hkv
    uniq = [traffic.unique_rows(s.idx.cpu().numpy(), s.cnt.cpu().numpy(), G) for s in sets]
    per_head_rows = [int(s.cnt.sum().item()) for s in sets]
    step_bytes = float(np.mean([traffic.sparse_step_bytes(cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.n, 2, s.cap, u)
                                for s, u in zip(sets, uniq)]))
    gather_bytes = float(np.mean([u * 2 * cfg.d * 2 for u in uniq]))
    sig_bytes = cfg.B * cfg.Hkv * cfg.n * 4
    res = {
        "value": cfg.B / (ms_step * 1e-3),
        "ms_per_step": ms_step,
        "steps": steps,
        "step_bytes": step_bytes,
        "step_tbps": step_bytes / (ms_step * 1e-3) / 1e12,
        "unique_rows": float(np.mean(uniq)),
        "per_head_rows": float(np.mean(per_head_rows)),
        "two_call_ms_per_step": ms_two,
        "two_call_tbps": step_bytes / (ms_two * 1e-3) / 1e12,
        "sig_score_topk_us": ms_t * 1e3,
        "gather_attn_us": ms_g * 1e3,
        "topk_sig_tbps": sig_bytes / (ms_t * 1e-3) / 1e12,
        "gather_tbps": gather_bytes / (ms_g * 1e-3) / 1e12,
        "gather_bytes": gather_bytes,
        "topk_traffic": traffic_from_profile("topk_unit_sparse128k", sig_bytes, "topk_unit")
                        if cfg.n * cfg.B == 8 * 131072 else None,
        "rotations": rot,
        "step_spread": replay_stats(st),
    }
    if args.tmap:
        res["t_map"] = bench_tmap(args, sets, cfg)
    return res, sets[0]


# ---------------------------------------------------------------- needles ----
class NeedleSet(SparseSet):
    """Config 5 inputs (planted needles) with the buffers of both the dense and the sparse decode."""

    def __init__(self, cfg, rot, device="cuda"):
        super().__init__(cfg, rot, device)
        B, Hq = self.x["q"].shape[:2]
        Hkv, n = self.x["k"].shape[1], self.x["k"].shape[2]
        self.do = torch.empty((B, Hq, 128), device=device)
        self.da = torch.empty((B, Hq), device=device)
        nb = max(self.ws.numel(), ops.ws_bytes_cached_attn_lse(B, Hq, Hkv, 128, n, Hkv * n * 128))
        if nb > self.ws.numel():
            self.ws = torch.empty(nb, dtype=torch.uint8, device=device)

    def dense(self):
        ops.cached_attn_lse(self.x["q"], self.x["k"], self.x["v"], out=self.do, alpha=self.da, ws=self.ws)


def needle_quality(s, cfg) -> dict:
    """Recall of the planted needles in each query head's selected set (over all heads, and over the
    first head of each KV group, along whose query the needles were planted), the attention mass the
    set captures (e^{alpha_I - alpha}), and the sparse output's error against the dense one."""
    G = cfg.Hq // cfg.Hkv
    s.step()
    s.dense()
    torch.cuda.synchronize()
    idx, cnt = s.idx.cpu().numpy(), s.cnt.cpu().numpy()
    pos = s.x["needle_pos"].cpu().numpy()
    B, Hq = cnt.shape
    rec = np.empty((B, Hq))
    for b in range(B):
        for hq in range(Hq):
            rec[b, hq] = np.isin(pos[b, hq // G], idx[b, hq, :cnt[b, hq]]).mean()
    mass = torch.exp(s.oa - s.da).cpu().numpy()
    err = (torch.linalg.vector_norm(s.o - s.do, dim=-1) / torch.linalg.vector_norm(s.do, dim=-1)).cpu().numpy()
    other = np.ones((B, Hq), bool)
    other[:, ::G] = False
    res = {}
    for name, sel in (("planted_head", ~other), ("other_heads", other)):
        res.update({"needle_recall_%s_mean" % name: float(rec[sel].mean()),
                    "needle_recall_%s_min" % name: float(rec[sel].min()),
                    "mass_captured_%s_mean" % name: float(mass[sel].mean()),
                    "mass_captured_%s_min" % name: float(mass[sel].min()),
                    "rel_err_vs_dense_%s_mean" % name: float(err[sel].mean()),
                    "rel_err_vs_dense_%s_max" % name: float(err[sel].max())})
    return res


def bench_needles(args, cfg):
    rot = args.rot or 2
    sets = [NeedleSet(cfg, r) for r in range(rot)]
    torch.cuda.synchronize()
    steps = args.steps
    st = run_steps_stats([s.step for s in sets], steps, args.warmup, args.graph)
    ms_s = st["ms_per_step"]
    ms_g = run_steps([s.gather for s in sets], steps, args.warmup, args.graph) / steps
    ms_t = run_steps([s.topk for s in sets], steps, args.warmup, args.graph) / steps
    ms_d = run_steps([s.dense for s in sets], steps, args.warmup, args.graph) / steps
    G = cfg.Hq // cfg.Hkv
    uniq = [traffic.unique_rows(s.idx.cpu().numpy(), s.cnt.cpu().numpy(), G) for s in sets]
    sparse_bytes = float(np.mean([traffic.sparse_step_bytes(cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.n, 2, s.cap, u)
                                  for s, u in zip(sets, uniq)]))
    gather_bytes = float(np.mean([u * 2 * cfg.d * 2 for u in uniq]))
    sig_bytes = cfg.B * cfg.Hkv * cfg.n * 4
    dense_bytes = traffic.dense_step_bytes(cfg.B, cfg.Hq, cfg.Hkv, cfg.d, cfg.n, 2)
    res = {
        "value": cfg.B / (ms_s * 1e-3),
        "ms_per_step": ms_s,
        "steps": steps,
        "sparse_step_bytes": sparse_bytes,
        "sparse_step_tbps": sparse_bytes / (ms_s * 1e-3) / 1e12,
        "sig_score_topk_us": ms_t * 1e3,
        "topk_sig_tbps": sig_bytes / (ms_t * 1e-3) / 1e12,
        "gather_attn_us": ms_g * 1e3,
        "gather_bytes": gather_bytes,
        "gather_tbps": gather_bytes / (ms_g * 1e-3) / 1e12,
        "dense_queries_per_s": cfg.B / (ms_d * 1e-3),
        "dense_ms_per_step": ms_d,
        "dense_bytes": dense_bytes,
        "dense_tbps": dense_bytes / (ms_d * 1e-3) / 1e12,
        "dense_frac_of_peak": dense_bytes / (ms_d * 1e-3) / HBM_PEAK,
        "speedup_sparse_over_dense": ms_d / ms_s,
        "unique_rows": float(np.mean(uniq)),
        "rotations": rot,
        "step_spread": replay_stats(st),
    }
    res.update(needle_quality(sets[0], cfg))
    return res


# ------------------------------------------------------------- quadrature ----
class QuadSet:
    """One input set of the quadrature workload: q [B, Hq, d] against one shared (W, Z) per KV head."""

    def __init__(self, cfg, rot, device="cuda"):
        self.x = synth.make_inputs(cfg, device=device, rot=rot)
        B, Hq = self.x["q"].shape[:2]
        Hkv, n = self.x["k"].shape[1], self.x["k"].shape[2]
        self.o = torch.empty((B, Hq, 128), device=device)
        self.al = torch.empty((B, Hq), device=device)
        self.ws = torch.empty(ops.ws_bytes_cached_attn_lse(B, Hq, Hkv, 128, n, 0), dtype=torch.uint8, device=device)

    def step(self):
        ops.cached_attn_lse(self.x["q"], self.x["k"], self.x["v"], out=self.o, alpha=self.al, ws=self.ws)


def bench_quadrature(args, cfg):
    rot = args.rot or 2
    sets = [QuadSet(cfg, r) for r in range(rot)]
    torch.cuda.synchronize()
    ms = run_steps([s.step for s in sets], args.steps, args.warmup, args.graph) / args.steps
    flops = 4.0 * cfg.B * cfg.Hq * cfg.n * cfg.d          # q.w and p.z: two multiply-adds per (row, pair, dim)
    bytes_ = 2 * cfg.Hkv * cfg.n * cfg.d * 2 + cfg.B * cfg.Hq * cfg.d * 2 + cfg.B * cfg.Hq * (cfg.d + 1) * 4
    return {"value": cfg.B / (ms * 1e-3), "ms_per_step": ms, "steps": args.steps, "flops": flops,
            "tflops": flops / (ms * 1e-3) / 1e12, "bytes": bytes_, "tbps": bytes_ / (ms * 1e-3) / 1e12,
            "rotations": rot}


# --------------------------------------------------------------- sigwidth ----
def bench_sigwidth(args, cfg):
    """sig_score_topk_w at 32 to 512 bits on config 4's shape (random codes): the code-width sweep."""
    B, Hq, Hkv, n = cfg.B, cfg.Hq, cfg.Hkv, cfg.n
    out = {}
    gen = torch.Generator(device="cuda").manual_seed(4242)
    for W in (1, 2, 4, 8, 16):
        sets = []
        for r in range(2):
            ks = torch.randint(-(1 << 31), 1 << 31, (B, Hkv, n, W), generator=gen, device="cuda", dtype=torch.int64)
            qs = torch.randint(-(1 << 31), 1 << 31, (B, Hq, W), generator=gen, device="cuda", dtype=torch.int64)
            ks, qs = ks.to(torch.int32), qs.to(torch.int32)
            cap = ops.capacity(n, cfg.m, cfg.n_sink, cfg.n_recent)
            idx = torch.empty((B, Hq, cap), dtype=torch.int32, device="cuda")
            cnt = torch.empty((B, Hq), dtype=torch.int32, device="cuda")
            ws = torch.empty(ops.load().lcda_ws_bytes_sig_score_topk_w(B, Hq, n), dtype=torch.uint8, device="cuda")
            sets.append((ks, qs, idx, cnt, ws))
        fns = [lambda s_=s_: ops.sig_score_topk_w(s_[0], s_[1], cfg.m, cfg.n_sink, cfg.n_recent, idx=s_[2],
                                                   count=s_[3], ws=s_[4]) for s_ in sets]
        torch.cuda.synchronize()
        steps = max(20, args.steps // 2)   # 20 replays of several steps: one graph launch shared by several
        ms = run_steps(fns, steps, max(2, args.warmup // 4), args.graph) / steps
        code_bytes = B * Hkv * n * 4 * W
        out["%d_bits" % (32 * W)] = {"us": ms * 1e3, "queries_per_s": B / (ms * 1e-3), "code_bytes": code_bytes,
                                    "code_tbps": code_bytes / (ms * 1e-3) / 1e12}
        del sets, fns
        torch.cuda.empty_cache()
    return out


# -------------------------------------------------------------- CPU oracle ----
def host_copy(x: dict) -> dict:
    """Host copies of an input set's tensors (the very arrays uploaded for the timed steps)."""
    return {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in x.items()}


def cpu_baseline_dense(cfg, seconds: float, threads: int = 0, layers: int = 1, x=None):
    """The oracle (plain C, fp64) on the host's cores (or `threads` of them) over decode steps of the same
    workload: x is the input set the GPU timed (rotation 0; copied to the host here), else one drawn afresh;
    with layers > 1 each timed step is one layer (every layer has the same shape) and the rate is scaled by
    the layer count."""
    from oracle import oracle as orc_mod
    orc = orc_mod.default()
    orc.set_threads(threads or os.cpu_count() or 1)
    x = host_copy(x) if x is not None else synth.make_inputs(cfg, device="cpu")

    def np_(t):
        t = t.contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()
    q, k, v, kl, vl, nl = (np_(x["q"]), np_(x["k"]), np_(x["v"]), np_(x["k_loc"]), np_(x["v_loc"]),
                           x["n_loc"].numpy())
    steps = 0
    t0 = time.perf_counter()
    while True:
        a, al = orc.dense_attn(q, k, v)
        orc.merge_local(q, a, al, kl, vl, nl)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    what = "full decode step(s)" if layers == 1 else "step(s) of one layer"
    tail = "" if layers == 1 else "; the rate is divided by the %d layers of a decode step" % layers
    src = "on host copies of the arrays the GPU timed" if x is not None else "on inputs drawn on the host"
    return {"value": cfg.B * steps / (el * layers), "unit": "queries/s", "cores": orc.get_threads(),
            "kind": "oracle",
            "sample": "%d %s of %s (cached_attn_lse + lse_merge_local definitions, fp64) %s, %.1f s wall%s"
                      % (steps, what, cfg.name, src, el, tail)}


def cpu_baseline_quadrature(cfg, seconds: float, B: int = 4):
    """The oracle's dense attention for B of the queries against the whole shared module."""
    from oracle import oracle as orc_mod
    orc = orc_mod.default()
    orc.set_threads(os.cpu_count() or 1)
    x = synth.make_inputs(cfg, device="cpu")
    q = x["q"][:B].contiguous().view(torch.int16).numpy().view(np.uint16)
    k = x["k"].contiguous().view(torch.int16).numpy().view(np.uint16)
    v = x["v"].contiguous().view(torch.int16).numpy().view(np.uint16)
    steps = 0
    t0 = time.perf_counter()
    while True:
        orc.dense_attn(q, k, v)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": B * steps / el, "unit": "queries/s", "cores": orc.get_threads(), "kind": "oracle",
            "sample": "%d x %d queries against the shared module (cached_attn_lse definition, fp64), %.1f s wall"
                      % (steps, B, el)}


def cpu_baseline_sparse(cfg, seconds: float, B: int = 1, x=None):
    """The oracle's SCORE + TOPK + GATHER-ATT on the first B batch items of x (the input set the GPU timed,
    copied to the host), else of a set drawn on the host."""
    from oracle import oracle as orc_mod
    orc = orc_mod.default()
    orc.set_threads(os.cpu_count() or 1)
    if x is not None:
        x = {k: (v[:B].cpu() if torch.is_tensor(v) and v.dim() > 0 and v.shape[0] == cfg.B else v)
             for k, v in x.items() if k in ("q", "k", "v", "key_sigs", "q_sigs")}
    else:
        x = synth.make_inputs(cfg, device="cpu", B=B)

    def np_(t):
        t = t.contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()
    q, k, v = np_(x["q"]), np_(x["k"]), np_(x["v"])
    ks = x["key_sigs"].numpy().view(np.uint32)
    qs = x["q_sigs"].numpy().view(np.uint32)
    steps = 0
    t0 = time.perf_counter()
    while True:
        idx, cnt, _ = orc.sig_score_topk(ks, qs, cfg.m, cfg.n_sink, cfg.n_recent)
        orc.gather_attn(q, k, v, idx, cnt)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": B * steps / el, "unit": "queries/s", "cores": orc.get_threads(), "kind": "oracle",
            "sample": "%d step(s) of the first %d batch item(s) of the timed input set, copied to the host "
                      "(SCORE+TOPK+GATHER-ATT definitions, fp64), %.1f s wall" % (steps, B, el)}


# ------------------------------------------------------------------- main ----
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dense61k",
                    choices=["dense61k", "shared36", "sparse128k", "needles512k", "quadrature", "sigwidth"])
    ap.add_argument("--rot", type=int, default=0, help="input sets cycled (0: workload default)")
    ap.add_argument("--no-graph", dest="graph", action="store_false", help="launch eagerly instead of a HIP graph")
    ap.add_argument("--no-extra", "--no-sparse", dest="extra", action="store_false",
                    help="skip the sparse128k, shared36 and needles512k entries that ride along with the dense61k line")
    ap.add_argument("--no-tmap", dest="tmap", action="store_false",
                    help="skip the T_map timings that ride along with the sparse measurement")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle sample length (0: skip)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain copy of MIB MiB (--steps times), for counter calibration")
    ap.add_argument("--tuning", action="append", default=[], metavar="KEY=VALUE",
                    help="set a launch-shape knob (lcda_set_tuning) before measuring; may be repeated")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (each GPU would run the same kernels "
              "on its share of KV heads or tokens; see DESIGN.md).  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.calibrate_copy:
        print(json.dumps(calibrate_copy(args.calibrate_copy << 20, args.steps)))
        return
    ops.load()
    for kv in args.tuning:
        key, _, val = kv.partition("=")
        ops.set_tuning(key, int(val))
    dev_name = torch.cuda.get_device_name(0)

    line = {"metric": METRIC, "unit": "queries/s", "n_gpus": 1, "warmup": args.warmup,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) bf16 K/V/q drawn on the GPU)"}
    launch = "hipGraph" if args.graph else "eager"
    if args.workload in ("dense61k", "shared36"):
        cfg = synth.CONFIGS[2 if args.workload == "dense61k" else 3]
        layers = cfg.layers
        res, timed = bench_dense(args, cfg, layers)
        line.update({"value": res["value"], "steps": res["steps"], "ms_per_step": res["ms_per_step"],
                     "roofline": res["roofline"]})
        line["config"] = {"workload": args.workload + ": " + cfg.name, "batch": cfg.B, "n": cfg.n, "layers": layers,
                          "kv_heads": cfg.Hkv, "q_heads": cfg.Hq, "d": cfg.d, "n_loc": cfg.n_loc, "launch": launch,
                          "rotations": res["rotations"]}
        line["step"] = ("dense_decode_step: cached_attn_lse + lse_merge_local as one split-KV launch whose last "
                        "workgroup per (batch, KV head) does the LSE combine" if not cfg.shared_doc else
                        "36 x dense_decode_step over one shared document (cached_attn_lse + lse_merge_local as "
                        "one 64-row split-KV pass that also takes each row's local tokens, then one combine)")
        line["step_spread"] = res["step_spread"]
        line["cached_attn_lse_us"] = res["cached_attn_lse_us"]
        line["two_call_ms_per_step"] = res["two_call_ms_per_step"]
        line["two_call_tbps"] = res["two_call_tbps"]
        line["step_bytes"] = res["step_bytes"]
        line["step_tbps"] = res["step_tbps"]
        line["step_frac_of_peak"] = res["step_tbps"] * 1e12 / HBM_PEAK
        shared_timed = None
        if args.workload == "dense61k" and args.extra:
            # The other target workloads ride along as entries of the same line.
            sres, _ = bench_sparse(args, synth.CONFIGS[4])
            sres["workload"] = "sparse128k: " + synth.CONFIGS[4].name
            sres["step_frac_of_peak"] = sres["step_tbps"] * 1e12 / HBM_PEAK
            line["sparse"] = sres
            torch.cuda.empty_cache()
            c3 = synth.CONFIGS[3]
            dres, shared_timed = bench_dense(args, c3, c3.layers)
            dres["workload"] = "shared36: " + c3.name
            dres["layer_us"] = dres["ms_per_step"] * 1e3 / c3.layers
            dres["step_frac_of_peak"] = dres["step_tbps"] * 1e12 / HBM_PEAK
            line["shared36"] = dres
            shared_timed = host_copy(shared_timed.x)
            torch.cuda.empty_cache()
            nres = bench_needles(args, synth.CONFIGS[5])
            nres["workload"] = "needles512k: " + synth.CONFIGS[5].name
            nres["sparse_step_frac_of_peak"] = nres["sparse_step_tbps"] * 1e12 / HBM_PEAK
            line["needles512k"] = nres
            torch.cuda.empty_cache()
        if args.cpu_seconds > 0:
            line["cpu_baseline"] = cpu_baseline_dense(cfg, args.cpu_seconds, layers=layers, x=timed.x)
            if args.workload == "dense61k":
                # One thread: this workload, the small reference case, and one layer of the shared document.
                short = max(1.0, args.cpu_seconds / 4)
                one = cpu_baseline_dense(cfg, short, threads=1, x=timed.x)
                line["cpu_baseline_one_thread"] = {"value": one["value"], "unit": one["unit"],
                                                   "cores": one["cores"], "sample": one["sample"]}
                c1 = synth.CONFIGS[1]
                tiny = cpu_baseline_dense(c1, short, threads=1, x=synth.make_inputs(c1, device="cuda"))
                line["cpu_baseline_one_thread_tiny"] = {"value": tiny["value"], "unit": tiny["unit"],
                                                        "cores": tiny["cores"], "sample": tiny["sample"]}
                if shared_timed is not None:
                    c3 = synth.CONFIGS[3]
                    lay = cpu_baseline_dense(c3, short, threads=1, x=shared_timed)
                    line["cpu_baseline_one_thread_shared36_layer"] = {
                        "value": lay["value"], "unit": "queries/s through one layer", "cores": lay["cores"],
                        "sample": lay["sample"]}
        if args.workload == "dense61k":
            ctx = hbm_context()
            line["hbm_context"] = ctx
            peak = ctx["stream_read_peak_tbps"] * 1e12
            line["roofline"]["measured_read_peak"] = peak / 1e9
            line["roofline"]["frac_of_measured_read_peak"] = line["roofline"]["achieved"] * 1e9 / peak
    elif args.workload == "sparse128k":
        cfg = synth.CONFIGS[4]
        res, timed = bench_sparse(args, cfg)
        line.update({"value": res["value"], "steps": res["steps"], "ms_per_step": res["ms_per_step"]})
        ach = res["gather_tbps"] * 1e12
        line["roofline"] = {"bound": "hbm", "achieved": ach / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                            "frac": ach / HBM_PEAK,
                            "traffic": traffic_from_profile("split_valu_sparse128k", int(res["gather_bytes"]),
                                                            "split_valu"),
                            "kernel": "gather_attn (k_split_valu in gather mode, one workgroup per query head "
                                      "here, so no combine pass; achieved on unique rows)"}
        line["config"] = {"workload": "sparse128k: " + cfg.name, "launch": launch}
        line["detail"] = res
        if args.cpu_seconds > 0:
            line["cpu_baseline"] = cpu_baseline_sparse(cfg, args.cpu_seconds, x=timed.x)
    elif args.workload == "sigwidth":
        cfg = synth.CONFIGS[4]
        res = bench_sigwidth(args, cfg)
        w8 = res["256_bits"]
        line.update({"value": w8["queries_per_s"], "steps": max(20, args.steps // 2), "ms_per_step": w8["us"] / 1e3})
        line["roofline"] = {"bound": "hbm", "achieved": w8["code_tbps"] * 1e3, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                            "frac": w8["code_tbps"] * 1e12 / HBM_PEAK, "traffic": None,
                            "kernel": "sig_score_topk_w at 256 bits, the whole call (k_wide_hist + k_wide_select + "
                                      "k_wide_compact); achieved on the key-code bytes"}
        # HBM bytes per launch of the histogram pass (key codes read once per KV head, distance bytes written)
        hist_alg = cfg.B * cfg.Hkv * cfg.n * 4 * 8 + cfg.B * cfg.Hq * cfg.n
        line["hist_pass"] = {"algorithmic_bytes": hist_alg,
                             "traffic": traffic_from_profile("wide_hist_sigwidth256", hist_alg, "wide")}
        line["config"] = {"workload": "sigwidth: sig_score_topk_w on " + cfg.name + ", random codes of 32-512 bits",
                          "launch": launch}
        line["step"] = "sig_score_topk_w at 256 bits (value); every width in detail"
        line["detail"] = res
    elif args.workload == "quadrature":
        cfg = synth.QUADRATURE
        res = bench_quadrature(args, cfg)
        line.update({"value": res["value"], "steps": res["steps"], "ms_per_step": res["ms_per_step"]})
        line["roofline"] = {"bound": "mfma", "achieved": res["tflops"], "peak": MFMA_BF16_PEAK / 1e12,
                            "unit": "TFLOP/s", "frac": res["tflops"] * 1e12 / MFMA_BF16_PEAK, "traffic": None,
                            "kernel": "k_split_rows_pair (64-row MFMA pass over the shared module) + k_combine_small"}
        line["config"] = {"workload": "quadrature: " + cfg.name, "launch": launch}
        line["step"] = "cached_attn_lse of 256 queries against p = 6,144 shared (W, Z) pairs per KV head"
        line["detail"] = res
        if args.cpu_seconds > 0:
            line["cpu_baseline"] = cpu_baseline_quadrature(cfg, args.cpu_seconds)
    else:
        cfg = synth.CONFIGS[5]
        res = bench_needles(args, cfg)
        line.update({"value": res["value"], "steps": res["steps"], "ms_per_step": res["ms_per_step"]})
        ach = res["gather_tbps"] * 1e12
        line["roofline"] = {"bound": "hbm", "achieved": ach / 1e9, "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                            "frac": ach / HBM_PEAK, "traffic": None,
                            "kernel": "gather_attn (k_split_valu gather + the combine where a row is split; achieved on "
                                      "unique rows)"}
        line["config"] = {"workload": "needles512k: " + cfg.name, "launch": launch}
        line["step"] = "sig_score_topk + gather_attn (value); cached_attn_lse on the same inputs (dense_*)"
        line["detail"] = res
    line["device"] = dev_name
    line["host"] = platform.node()
    print(json.dumps(line))


if __name__ == "__main__":
    main()
