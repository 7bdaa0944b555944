#!/usr/bin/env python3
"""One sparse prefill attention layer per step on one MI355X.

A step runs the whole path for every head of the layer: vertical-slash heads
(estimate, top-k, sparse format, attention), block-sparse heads (pooling,
block selection, attention) and streaming heads (attention), each call over
its head subset, all writing one output tensor. The block-sparse call runs on
a second stream beside the others (its selection overlaps their work); the
step ends when both streams are done. The one-stream time is reported as
`ms_per_layer_one_stream`. Inputs are
seeded synthetic tensors resident in HBM before timing starts. A layer with
more than one pattern is also timed through the mixed call (the same index
stages, then every head's attention in one launch) and reported as
`one_launch`.

Default workload: the 1M-token Llama-3-8B-shaped mixed layer (the named
workload that runs every step of the path); the other named workloads are
timed beside it under `secondary`, each over at least 300 ms of steps
(`timed_steps`), so that a layer of a fraction of a millisecond is not
timed as host jitter.

Per-stage times (`stages_ms`, and the after-prefill calls) time each call
alone with HIP events after a 512 MiB write that leaves none of its inputs in
the GPU's caches, averaged over the repetitions.

Prints one JSON line. `value` is the effective TFLOP/s of the layer: the
attention FLOPs of the computed key blocks (4 * head_dim * sum over query
blocks of rows x keys, before the causal trim of the diagonal tile) divided by
the measured layer time. `roofline` reports the dominant kernel (the
vertical-slash attention launch) against the bf16 MFMA peak, timed alone with
HIP events on the stream it runs on; its `traffic` comes from the committed
rocprofv3 counter summary when that summary was taken on the current kernel
source. `cpu_baseline` times the CPU oracle on a bounded sample of the same
layer and scales it to the whole layer.

Other modes:
  --copy-probe MIB      also run one plain device copy of MIB MiB (a counter
                        calibration point for rocprofv3 --pmc runs)
  --summarize-pmc DIR   read rocprofv3 --pmc CSVs under DIR (FETCH_SIZE and
                        WRITE_SIZE passes of a run with --copy-probe) and print
                        the per-launch traffic summary as JSON (--record also
                        stores it for --workload in profiles/traffic.json)
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import glob
import hashlib
import json
import math
import os
import re
import subprocess
import sys
import threading
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import dynamic_sparse_attention_slash_amd as dsa  # noqa: E402
import synthetic  # noqa: E402

BLK = 64
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0
# the pages' own figures (other hardware, other metrics): context only
PAGES_CONTEXT = [
    {"figure": "about 10x prefill speedup over dense attention", "hardware": "1x NVIDIA A100",
     "workload": "million-token prompts", "source": "MInference 1.0 article, preface"},
    {"figure": "18.95x attention decoding speedup", "hardware": "1x NVIDIA L40s 48GB",
     "workload": "1M-token context", "source": "InfiniteHiP summary, introduction"},
    {"figure": "about 1.58x serving throughput over vLLM 0.6.1", "hardware": "RTX 4090",
     "workload": "4000 input / 500 output tokens", "source": "Novita AI KV-sparsity blog, results"},
]
ATTN_SRC = os.path.join(ROOT, "dynamic_sparse_attention_slash_amd", "csrc", "sparse_attention.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
DOMINANT = "attn_vs_single_kernel"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(path=ATTN_SRC):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


# ----------------------------------------------------------------------------
# device facts and the clock under load
# ----------------------------------------------------------------------------
def device_info():
    """Compute units and peak shader clock of device 0 from the HIP runtime
    (hipDeviceAttributeMultiprocessorCount / hipDeviceAttributeClockRate)."""
    info = {"name": torch.cuda.get_device_properties(0).name,
            "gcn_arch": torch.cuda.get_device_properties(0).gcnArchName}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        val = ctypes.c_int(0)
        for key, attr in (("compute_units", 63), ("peak_clock_mhz", 5)):
            if hip.hipDeviceGetAttribute(ctypes.byref(val), attr, 0) == 0:
                info[key] = val.value if key == "compute_units" else val.value / 1000.0
    except OSError as e:
        info["error"] = str(e)
    if "compute_units" in info and "peak_clock_mhz" in info:
        # dense bf16 MFMA: 4 SIMDs x 1024 FLOP per clock per CU
        info["bf16_peak_tflops_at_peak_clock"] = info["compute_units"] * 4096 * info["peak_clock_mhz"] * 1e6 / 1e12
    return info


class ClockSampler:
    """Samples the GPU's current shader clock with rocm-smi (a child process)
    while the timed steps run."""

    enabled = True  # --no-clock: no child processes (e.g. under a counter profiler)

    def __init__(self, period=0.3):
        self.period, self.samples, self._stop = period, [], threading.Event()
        self._thr = None

    def _one(self):
        try:
            out = subprocess.run(["rocm-smi", "-d", "0", "--showclocks"], capture_output=True, text=True,
                                 timeout=5).stdout
        except (OSError, subprocess.SubprocessError):
            return None
        m = re.search(r"sclk[^\n]*?\((\d+)\s*Mhz\)", out, re.I)
        return float(m.group(1)) if m else None

    def _sample(self):
        v = self._one()
        if v is not None:
            self.samples.append(v)

    def _run(self):
        while not self._stop.wait(self.period):
            self._sample()

    def __enter__(self):
        # The first sample is taken here, before the timed region: starting a
        # child process from this (large) process can stall its launches for
        # milliseconds, which a layer of a fraction of a millisecond would show.
        if ClockSampler.enabled:
            self._sample()
            self._thr = threading.Thread(target=self._run, daemon=True)
            self._thr.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thr is not None:
            self._thr.join(timeout=10)

    def summary(self):
        if not self.samples:
            return None
        v = sorted(self.samples)
        return {"median_mhz": v[len(v) // 2], "min_mhz": v[0], "max_mhz": v[-1], "samples": len(v),
                "tool": "rocm-smi --showclocks (sclk), sampled during the timed steps"}


# ----------------------------------------------------------------------------
# FLOP accounting from the indices
# ----------------------------------------------------------------------------
def rows_per_block(n):
    nb = (n + BLK - 1) // BLK
    r = np.full(nb, BLK, np.int64)
    r[-1] = n - BLK * (nb - 1)
    return r


def vs_keys_per_block(iv, n_iv, n_cols, n):
    """keys(a) of every (row, block): clipped range lengths + columns."""
    iv, n_iv, n_cols = iv.cpu().numpy(), n_iv.cpu().numpy(), n_cols.cpu().numpy().astype(np.int64)
    nb = (n + BLK - 1) // BLK
    r0 = np.arange(nb, dtype=np.int64) * BLK
    keys = n_cols.copy()
    for r in range(iv.shape[0]):
        for t in range(int(n_iv[r])):
            d_lo, d_hi = int(iv[r, t, 0]), int(iv[r, t, 1])
            lo = np.maximum(0, r0 - d_hi)
            hi = np.minimum(n, r0 + BLK - d_lo)
            keys[r] += np.where(d_lo < r0 + BLK, np.maximum(0, hi - lo), 0)
    return keys


def bs_keys_per_block(sel, n_sel, n):
    sel, n_sel = sel.cpu().numpy(), n_sel.cpu().numpy().astype(np.int64)
    rows, nb, kmax = sel.shape
    last = n - BLK * (nb - 1)
    valid = np.arange(kmax)[None, None, :] < n_sel[:, :, None]
    has_last = ((sel == nb - 1) & valid).sum(axis=2)
    return BLK * n_sel - (BLK - last) * has_last


def st_keys_per_block(n, init_blocks, local_blocks):
    nb = (n + BLK - 1) // BLK
    last = n - BLK * (nb - 1)
    a = np.arange(nb)
    sink = np.minimum(init_blocks, a + 1)
    local_start = np.maximum(a - local_blocks + 1, sink)
    nblk = sink + np.maximum(0, a - local_start + 1)
    has_last = (nb - 1 < sink) | ((nb - 1 >= local_start) & (nb - 1 <= a))
    return BLK * nblk - (BLK - last) * has_last


def attn_flops(keys_rows_blocks, n, D):
    """4*D * sum_a rows(a) * keys(a): QK^T and PV over the computed key blocks."""
    return float(4 * D * (np.asarray(keys_rows_blocks) * rows_per_block(n)).sum())


# ----------------------------------------------------------------------------
# layer
# ----------------------------------------------------------------------------
class Layer:
    def __init__(self, w, x):
        self.w, self.x = w, x
        self.q, self.k, self.v = x.q, x.k, x.v
        self.o = torch.zeros_like(self.q)
        all_vs = len(x.heads["vs"]) == w.q_heads
        self.vs_heads = None if all_vs else x.heads["vs"]
        self.ws_vs = self.ws_bs = self.ws_mixed = None
        self.side = torch.cuda.Stream()  # default priority
        self.patterns = synthetic.pattern_list(w)
        if x.heads["vs"]:
            nbytes = dsa.vertical_slash_workspace_bytes(self.q, self.k, w.vertical_topk, w.slash_topk,
                                                        self.vs_heads)
            self.ws_vs = torch.empty(nbytes, dtype=torch.uint8, device=self.q.device)
        if x.heads["bs"]:
            nbytes = dsa.block_sparse_workspace_bytes(self.q, self.k, w.topk, x.heads["bs"])
            self.ws_bs = torch.empty(nbytes, dtype=torch.uint8, device=self.q.device)

    def _bs(self):
        dsa.block_sparse_attention(self.q, self.k, self.v, self.w.topk, heads=self.x.heads["bs"], out=self.o,
                                   workspace=self.ws_bs)

    def step(self, serial=False):
        """One layer. The block-sparse call (pooling, block selection,
        attention) runs on a second stream beside the streaming and
        vertical-slash calls, so its selection stages overlap the other heads'
        work (the streaming heads need no index and go first); the main stream
        waits for it before the step ends. The calls write disjoint heads of
        one output with their own workspaces, so the result is the same bits
        as the serial order (serial=True)."""
        w, x = self.w, self.x
        side = x.heads["bs"] and (x.heads["vs"] or x.heads["st"]) and not serial
        main = torch.cuda.current_stream()
        if side:
            self.side.wait_stream(main)
            with torch.cuda.stream(self.side):
                self._bs()
        if x.heads["st"]:
            dsa.streaming_attention(self.q, self.k, self.v, w.init_blocks, w.local_blocks,
                                    heads=x.heads["st"], out=self.o)
        if x.heads["vs"]:
            dsa.vertical_slash_sparse_attention(self.q, self.k, self.v, w.vertical_topk, w.slash_topk,
                                                last_q=w.last_q, heads=self.vs_heads, out=self.o,
                                                workspace=self.ws_vs)
        if x.heads["bs"] and not side:
            self._bs()
        if side:
            main.wait_stream(self.side)

    def one_launch(self):
        """The same layer through the mixed call: every head's attention in one
        launch (index stages as above)."""
        w = self.w
        if self.ws_mixed is None:
            nbytes = dsa.mixed_workspace_bytes(self.q, self.k, self.patterns, w.vertical_topk,
                                               w.slash_topk, w.topk)
            self.ws_mixed = torch.empty(max(1, nbytes), dtype=torch.uint8, device=self.q.device)
        return lambda: dsa.mixed_sparse_attention(
            self.q, self.k, self.v, self.patterns, vertical_topk=w.vertical_topk, slash_topk=w.slash_topk,
            topk=w.topk, init_blocks=w.init_blocks, local_blocks=w.local_blocks, last_q=w.last_q,
            out=self.o, workspace=self.ws_mixed)


def time_events(fn, reps):
    """Average ms per call of fn over back-to-back calls, HIP events on
    torch's current stream (the stream every library call is enqueued on)."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    e0.record(s)
    for _ in range(reps):
        fn()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


FLUSH_BYTES = 512 << 20  # twice the 256 MB last-level (MALL) cache
_flush_buf = None


def flush_caches():
    """Write 512 MiB so that no input of the next call is left in the GPU's
    caches from the previous one."""
    global _flush_buf
    if _flush_buf is None:
        _flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    _flush_buf.fill_(1)


def time_stage(fn, reps):
    """Average ms of one call of fn, each timed alone with HIP events on
    torch's current stream after a cache flush (one untimed call first)."""
    s = torch.cuda.current_stream()
    fn()
    ev = []
    for _ in range(reps):
        flush_caches()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        fn()
        e1.record(s)
        ev.append((e0, e1))
    ev[-1][1].synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / reps


def stages(layer, reps):
    """Each stage of the layer through the stage calls, timed alone; also
    returns the indices (for the FLOP accounting)."""
    w, x = layer.w, layer.x
    q, k, v, o = layer.q, layer.k, layer.v, layer.o
    t, idx = {}, {}
    if x.heads["vs"]:
        hs = x.heads["vs"]
        vg, sg = dsa.vs_estimate(q, k, last_q=w.last_q, heads=hs)
        t["vs_estimate_ms"] = time_stage(lambda: dsa.vs_estimate(q, k, last_q=w.last_q, heads=hs), reps)
        V = dsa.topk(vg, w.vertical_topk)
        S = dsa.topk(sg, w.slash_topk, 0)
        t["vs_topk_ms"] = time_stage(lambda: (dsa.topk(vg, w.vertical_topk), dsa.topk(sg, w.slash_topk, 0)), reps)
        ix = dsa.vs_build_index(V, S, w.seq_len)
        t["vs_index_ms"] = time_stage(lambda: dsa.vs_build_index(V, S, w.seq_len), reps)
        t["vs_attention_ms"] = time_stage(lambda: dsa.sparse_attention_vs(q, k, v, *ix, heads=hs, out=o), reps)
        idx["vs"] = ix
        del vg, sg
    if x.heads["bs"]:
        hs = x.heads["bs"]
        G = w.q_heads // w.kv_heads
        sel_rows = torch.tensor([b * w.kv_heads + h // G for b in range(w.batch) for h in hs], device=q.device)
        qp = dsa.bs_pool(q, hs)
        kp_all = dsa.bs_pool(k)
        t["bs_pool_ms"] = time_stage(lambda: (dsa.bs_pool(q, hs), dsa.bs_pool(k)), reps)
        kp = kp_all[sel_rows].contiguous()
        sel, n_sel = dsa.bs_select(qp, kp, w.topk)
        t["bs_select_ms"] = time_stage(lambda: dsa.bs_select(qp, kp, w.topk), reps)
        t["bs_attention_ms"] = time_stage(lambda: dsa.sparse_attention_blocks(q, k, v, sel, n_sel, heads=hs, out=o), reps)
        idx["bs"] = (sel, n_sel)
        del qp, kp, kp_all
    if x.heads["st"]:
        hs = x.heads["st"]
        t["st_attention_ms"] = time_stage(lambda: dsa.streaming_attention(q, k, v, w.init_blocks, w.local_blocks, heads=hs, out=o), reps)
    return t, idx


def layer_flops(w, x, idx):
    n, D = w.seq_len, w.head_dim
    fl = {}
    if "vs" in idx:
        iv, n_iv, cols, n_cols = idx["vs"]
        fl["vs"] = attn_flops(vs_keys_per_block(iv, n_iv, n_cols, n), n, D)
    if "bs" in idx:
        fl["bs"] = attn_flops(bs_keys_per_block(*idx["bs"], n), n, D)
    if x.heads["st"]:
        fl["st"] = attn_flops(st_keys_per_block(n, w.init_blocks, w.local_blocks), n, D) \
            * w.batch * len(x.heads["st"])
    return fl


KV_WINDOW, KV_KEEP = 256, 4096
# decode over pruned keys after prefill: 256 chunks of 4096 keys keep 16, their
# 128 chunks of 512 keep 32, their 256 blocks of 64 keep 64 (4096 keys per
# head, the retention budget); each stage keeps fewer chunks than the next, so
# the hierarchy is not a flat selection
HIER_DECODE_STAGES = [(4096, 16), (512, 32), (64, 64)]


def hier_prefill_stages(topk):
    """Pruning stages for a block-sparse layer with the same budget: topk key
    blocks per query block after a 1024- and a 256-key stage."""
    return [(1024, max(1, topk // 8)), (256, max(2, topk // 2)), (64, topk)]


def kv_retention_timing(layer, reps):
    """The steps after prefill, outside the layer step: KV-retention scores of
    every query head over the last 256 query rows and the 4096 kept keys per
    head (algorithmic bytes: K of every kv head once per pass, two passes for
    the softmax statistics and the scores; the scores written and read back by
    the top-k; the kept indices), then one decode step over the kept keys and
    one over the whole cache."""
    w, q, k, v = layer.w, layer.q, layer.k, layer.v
    torch.cuda.synchronize()
    ms = time_stage(lambda: dsa.kv_retention(q, k, KV_WINDOW, KV_KEEP), reps)
    n, D, B = w.seq_len, w.head_dim, w.batch
    rows = B * w.q_heads
    nbytes = 2 * B * w.kv_heads * n * D * 2 + 2 * rows * n * 4 + rows * min(KV_KEEP, n) * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    out = {"kv_retention_ms": ms, "window": KV_WINDOW, "keep": KV_KEEP, "heads": w.q_heads,
           "bytes": nbytes, "gbs": gbs, "frac_hbm": gbs / PEAK_HBM_GBS}
    # One decode step after prefill: a new row per head over the kept keys, and
    # over the whole cache. Bytes: the K and V rows read once (whole cache:
    # once per kv head, the heads of a group share them in L2; kept keys: per
    # head), the key lists, q and o.
    _, kept = dsa.kv_retention(q, k, KV_WINDOW, KV_KEEP)
    kk = kept.shape[1]
    n_keys = torch.full((rows,), kk, dtype=torch.int32, device=q.device)
    g = torch.Generator(device=q.device).manual_seed(7)
    qd = torch.randn(B, w.q_heads, D, generator=g, device=q.device).to(q.dtype)
    eb = 2 if w.dtype == "bf16" else 4
    qo = 2 * rows * D * eb
    ms_k = time_stage(lambda: dsa.sparse_decode(qd, k, v, kept, n_keys), 20)
    b_k = rows * kk * D * eb * 2 + rows * kk * 4 + qo
    ms_a = time_stage(lambda: dsa.sparse_decode(qd, k, v), 10)
    b_a = 2 * B * w.kv_heads * n * D * eb + qo
    for name, t, nb in (("decode_kept", ms_k, b_k), ("decode_all", ms_a, b_a)):
        out[name] = {"ms": t, "keys_per_head": kk if name == "decode_kept" else n, "bytes": nb,
                     "gbs": nb / (t * 1e-3) / 1e9, "frac_hbm": nb / (t * 1e-3) / 1e9 / PEAK_HBM_GBS}
    # the retention passes are bound by their products and exponentials, not
    # by memory: two passes of the window's rows against every key
    wr = min(KV_WINDOW, n)
    fl = 2 * 2.0 * rows * wr * n * D
    out["compute"] = {"flops": fl, "exp": 2.0 * rows * wr * n, "tflops": fl / (ms * 1e-3) / 1e12,
                      "frac_bf16_peak": fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    # decode over keys chosen per query by hierarchical chunk pruning: the
    # block-maximum pass streams K once per kv head (the heads of a group share
    # it in L2), then the decode reads the kept rows
    ms_h = time_stage(lambda: dsa.hier_sparse_decode(qd, k, v, HIER_DECODE_STAGES), 10)
    qu = qd.reshape(rows, 1, D).contiguous()
    ms_p = time_stage(lambda: dsa.hier_prune(qu, k, HIER_DECODE_STAGES, q_heads=w.q_heads), 10)
    kh = HIER_DECODE_STAGES[-1][0] * HIER_DECODE_STAGES[-1][1]
    b_p = B * w.kv_heads * n * D * eb + rows * D * eb
    b_h = b_p + rows * kh * D * eb * 2 + qo
    out["hier_decode"] = {"stages": HIER_DECODE_STAGES, "ms": ms_h, "prune_ms": ms_p, "keys_per_head": kh,
                          "bytes": b_h, "gbs": b_h / (ms_h * 1e-3) / 1e9,
                          "frac_hbm": b_h / (ms_h * 1e-3) / 1e9 / PEAK_HBM_GBS,
                          "prune_bytes": b_p, "prune_frac_hbm": b_p / (ms_p * 1e-3) / 1e9 / PEAK_HBM_GBS,
                          "speedup_vs_decode_all": ms_a / ms_h}
    del kept, n_keys, qd, qu
    return out


def hier_prefill_timing(layer, reps):
    """The block-sparse heads of a layer with the hierarchical pruning as their
    block estimator (same key-block budget), beside the mean-pooled block
    estimator. The pruning's block maxima score every visible key against
    every query block's pooled row: 2·D FLOP per pair, two bf16 MFMA products
    per fp32 product (the pooled row's hi and lo halves), so its peak is half
    the bf16 peak."""
    w, x = layer.w, layer.x
    hb = x.heads["bs"]
    st = hier_prefill_stages(w.topk)
    ms = time_stage(lambda: dsa.hier_block_sparse_attention(layer.q, layer.k, layer.v, st, heads=hb,
                                                           out=layer.o), reps)
    ms_bs = time_stage(layer._bs, reps)
    n, D, nb = w.seq_len, w.head_dim, (w.seq_len + 63) // 64
    rows = w.batch * len(hb)
    qp = dsa.bs_pool(layer.q, hb)
    ms_p = time_stage(lambda: dsa.hier_prune(qp, layer.k, st, q_heads=w.q_heads, heads=hb, unit_rows=64), reps)
    fma = rows * sum(min(n, 64 * (a + 1)) for a in range(nb)) * D
    del qp
    return {"stages": st, "ms": ms, "block_sparse_ms": ms_bs, "prune_ms": ms_p,
            "prune_flops": 2 * fma, "prune_tflops": 2 * fma / (ms_p * 1e-3) / 1e12,
            "prune_peak_tflops": PEAK_BF16_TFLOPS / 2,
            "prune_frac": 2 * fma / (ms_p * 1e-3) / 1e12 / (PEAK_BF16_TFLOPS / 2)}


def stage_bytes(w, x, idx):
    """Algorithmic HBM bytes of the memory-side stages (what each stage must
    read and write once), for the fraction of HBM peak next to its time:
    VS estimate: K of each involved kv head once per pass (two passes), the
    window rows of Q, the v and s vectors; VS top-k: v and s in, the indices
    out; VS index: the indices in, intervals, column lists and counts out;
    BS pool: Q of the block-sparse heads and all of K in, the pooled rows out."""
    n, D, B = w.seq_len, w.head_dim, w.batch
    eb = 2 if w.dtype == "bf16" else 4
    G = w.q_heads // w.kv_heads
    nb = (n + 63) // 64
    out = {}
    if "vs" in idx:
        hs = x.heads["vs"]
        kv = {h // G for h in hs}
        lq = min(w.last_q, n)
        out["vs_estimate_ms"] = (2 * B * len(kv) * n * D * eb + B * len(hs) * lq * D * eb
                                 + 2 * B * len(hs) * n * 4)
        vk, sk = min(w.vertical_topk, n), min(w.slash_topk, n)
        out["vs_topk_ms"] = B * len(hs) * (2 * n * 4 + (vk + sk) * 4)
        iv, n_iv, cols, n_cols = idx["vs"]
        out["vs_index_ms"] = (B * len(hs) * (vk + sk) * 4 + int(n_iv.sum()) * 8
                              + int(n_cols.sum()) * 4 + n_cols.numel() * 4 + n_iv.numel() * 4)
    if "bs" in idx:
        hs = x.heads["bs"]
        out["bs_pool_ms"] = B * (len(hs) + w.kv_heads) * (n * D * eb + nb * D * 4)
    return out


def bs_select_roofline(w, x, ms):
    """Block select against its own roofline: D * nb * (nb + 1) FLOP per head
    (one D-long dot per block pair of the causal triangle), each fp32 product
    taken as three bf16 MFMA products, so the peak is a third of the bf16
    MFMA peak; bytes are the pooled rows read, the logits written once and read
    twice by the select, and the selections written."""
    n, D, B = w.seq_len, w.head_dim, w.batch
    nb = (n + BLK - 1) // BLK
    rows = B * len(x.heads["bs"])
    flops = float(D * nb * (nb + 1)) * rows
    tri = nb * (nb + 1) // 2
    nbytes = rows * (2 * nb * D * 4 + 3 * tri * 4 + nb * min(w.topk, nb) * 4 + nb * 4)
    ach = flops / (ms * 1e-3) / 1e12
    return {"bound": "mfma (three bf16 products per fp32 product)", "flops": flops, "achieved": ach,
            "peak": PEAK_BF16_TFLOPS / 3, "unit": "TFLOP/s", "frac": ach / (PEAK_BF16_TFLOPS / 3),
            "bytes": nbytes, "gbs": nbytes / (ms * 1e-3) / 1e9,
            "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "ms": ms}


# ----------------------------------------------------------------------------
# CPU oracle on a bounded sample
# ----------------------------------------------------------------------------
def _sampled_blocks(nb, rng, seconds, max_blocks, fn):
    """Run fn(a) on random query blocks until `seconds` of CPU time are spent
    (at least two blocks, at most max_blocks); returns (seconds, rows x keys,
    blocks)."""
    t_sum, rk_sum, done = 0.0, 0, 0
    for a in rng.permutation(nb)[:max_blocks]:
        t0 = time.perf_counter()
        rk_sum += fn(int(a))
        t_sum += time.perf_counter() - t0
        done += 1
        if done >= 2 and t_sum >= seconds:
            break
    return t_sum, rk_sum, done


def cpu_baseline(layer, idx, flops_total, seconds=(12.0, 5.0, 1.0), full=False):
    """The oracle on the host's cores: the whole layer (full=True; only for
    layers it finishes in seconds), or a bounded sample scaled to the layer.
    `cores` is the threads it actually kept busy: process CPU time over wall
    time (numpy's BLAS threads; the oracle's own loops are serial)."""
    c0, t0 = os.times(), time.perf_counter()
    res = _cpu_full(layer) if full else _cpu_sampled(layer, idx, flops_total, seconds)
    c1, wall = os.times(), time.perf_counter() - t0
    cpu_s = (c1.user - c0.user) + (c1.system - c0.system)
    res["value"] = flops_total / (res.pop("t_layer") ) / 1e12
    res["cores"] = round(cpu_s / wall, 1) if wall > 0 else 1.0
    res["affinity_cpus"] = len(os.sched_getaffinity(0))
    res["wall_s"] = round(wall, 2)
    return res


def _cpu_full(layer):
    """The oracle's three pipelines over every head of the layer."""
    from oracle import dsa_oracle as O
    w, x = layer.w, layer.x
    f = lambda t: t.detach().float().cpu().numpy().astype(np.float64)  # noqa: E731
    q, k, v = f(layer.q), f(layer.k), f(layer.v)
    t0 = time.perf_counter()
    if x.heads["vs"]:
        O.vertical_slash_sparse_attention(q, k, v, w.vertical_topk, w.slash_topk, last_q=w.last_q,
                                          heads=x.heads["vs"])
    if x.heads["bs"]:
        O.block_sparse_attention(q, k, v, w.topk, heads=x.heads["bs"])
    if x.heads["st"]:
        O.streaming_attention(q, k, v, w.init_blocks, w.local_blocks, heads=x.heads["st"])
    t = time.perf_counter() - t0
    return {"unit": "TFLOP/s (effective, computed blocks)", "kind": "oracle", "t_layer": t,
            "sample": "the whole layer: every head's estimate, selection and attention (float64 numpy "
                      "oracle, not a tuned CPU implementation)",
            "ms_per_layer": t * 1e3}


def _cpu_sampled(layer, idx, flops_total, seconds):
    from oracle import dsa_oracle as O
    w, x = layer.w, layer.x
    n, D = w.seq_len, w.head_dim
    nb = (n + BLK - 1) // BLK
    G = w.q_heads // w.kv_heads
    sc = 1.0 / math.sqrt(D)
    f = lambda t: t.detach().float().cpu().numpy().astype(np.float64)  # noqa: E731
    rng = np.random.default_rng(0)
    t_total = 0.0
    parts = []
    if x.heads["vs"]:
        h = x.heads["vs"][0]
        qh, kh, vh = f(layer.q[0, h]), f(layer.k[0, h // G]), f(layer.v[0, h // G])
        t0 = time.perf_counter()
        v64, s64 = O.vs_scores(qh, kh, w.last_q, sc)
        V, S = O.vs_select(O.to_f32(v64), O.to_f32(s64), w.vertical_topk, w.slash_topk)
        iv = O.merge_offsets(S)
        t_est = time.perf_counter() - t0

        def vs_block(a):
            keys = O.vs_block_keys(iv, V, a, n)
            rows = np.arange(a * BLK, min(n, a * BLK + BLK))
            O.masked_attention(qh[rows], rows, keys, kh, vh, sc)
            return len(keys) * len(rows)
        t_att, keys_s, nblk = _sampled_blocks(nb, rng, seconds[0], 64, vs_block)
        iv_g, n_iv_g, cols_g, n_cols_g = idx["vs"]
        rk_all = float((vs_keys_per_block(iv_g, n_iv_g, n_cols_g, n) * rows_per_block(n)).sum())
        t_total += t_est * w.batch * len(x.heads["vs"]) + t_att * rk_all / keys_s
        parts.append(f"one vertical-slash head: full estimate, top-k and intervals; "
                     f"attention of {nblk} sampled query blocks")
    if x.heads["bs"]:
        h = x.heads["bs"][0]
        qh, kh, vh = f(layer.q[0, h]), f(layer.k[0, h // G]), f(layer.v[0, h // G])
        t0 = time.perf_counter()
        qp, kp = O.mean_pool(qh), O.mean_pool(kh)
        t_pool = time.perf_counter() - t0

        def bs_block(a):
            L = O.to_f32(O.block_logits(qp[a:a + 1], kp[: a + 1], sc))[0]
            keys = O.blocks_to_keys(O.topk_indices(L, w.topk, forced=(a,)), n)
            rows = np.arange(a * BLK, min(n, a * BLK + BLK))
            O.masked_attention(qh[rows], rows, keys, kh, vh, sc)
            return len(keys) * len(rows)
        t_blk, keys_s, nblk = _sampled_blocks(nb, rng, seconds[1], 64, bs_block)
        rk_all = float((bs_keys_per_block(*idx["bs"], n) * rows_per_block(n)).sum())
        t_total += t_pool * w.batch * len(x.heads["bs"]) + t_blk * rk_all / keys_s
        parts.append(f"one block-sparse head: pooling; block scores, selection and attention of "
                     f"{nblk} sampled query blocks")
    if x.heads["st"]:
        h = x.heads["st"][0]
        qh, kh, vh = f(layer.q[0, h]), f(layer.k[0, h // G]), f(layer.v[0, h // G])

        def st_block(a):
            keys = O.blocks_to_keys(O.streaming_blocks(a, w.init_blocks, w.local_blocks), n)
            rows = np.arange(a * BLK, min(n, a * BLK + BLK))
            O.masked_attention(qh[rows], rows, keys, kh, vh, sc)
            return len(keys) * len(rows)
        t_att, keys_s, nblk = _sampled_blocks(nb, rng, seconds[2], 64, st_block)
        rk = float((st_keys_per_block(n, w.init_blocks, w.local_blocks) * rows_per_block(n)).sum())
        t_total += t_att * rk / keys_s * w.batch * len(x.heads["st"])
        parts.append(f"one streaming head: attention of {nblk} sampled query blocks")
    return {"unit": "TFLOP/s (effective, computed blocks)", "kind": "oracle", "t_layer": t_total,
            "sample": "; ".join(parts) + "; times scaled to the whole layer by head count and by "
                      "row x key count (float64 numpy oracle, not a tuned CPU implementation)",
            "extrapolated_ms_per_layer": t_total * 1e3}


# ----------------------------------------------------------------------------
# counter traffic
# ----------------------------------------------------------------------------
def summarize_pmc(directory, copy_mib):
    """Per-launch HBM bytes of the dominant kernel from FETCH_SIZE / WRITE_SIZE
    passes, each scaled by what the counter reads for the plain copy probe."""
    def per_kernel(counter):
        vals = {}
        for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(path)):
                if r["Counter_Name"] != counter:
                    continue
                name = r["Kernel_Name"]
                key = ("dominant" if DOMINANT in name else
                       "copy" if "copyBuffer" in name else "neg" if "neg_kernel" in name else None)
                if key:
                    vals.setdefault(key, []).append(float(r["Counter_Value"]))
        return vals
    nbytes = copy_mib * 2 ** 20
    out = {"kernel": DOMINANT, "source_sha256_16": source_hash(), "copy_probe_bytes": nbytes}
    for counter, role in (("FETCH_SIZE", "read"), ("WRITE_SIZE", "write")):
        v = per_kernel(counter)
        probe = "copy" if "copy" in v else "neg"
        if "dominant" not in v or probe not in v:
            raise SystemExit(f"{counter}: dominant or probe kernel missing in {directory}")
        copy_kib = max(v[probe])                  # the probe is the largest copy
        out["probe_kernel"] = probe
        factor = nbytes / (copy_kib * 1024.0)
        dom_kib = float(np.median(v["dominant"]))
        out[f"{counter}_kib_per_launch"] = dom_kib
        out[f"{counter}_copy_kib"] = copy_kib
        out[f"{role}_scale"] = factor
        out[f"{role}_bytes_per_launch"] = dom_kib * 1024.0 * factor
    out["traffic_bytes_per_launch"] = out["read_bytes_per_launch"] + out["write_bytes_per_launch"]
    return out


def committed_traffic(workload):
    if not os.path.exists(TRAFFIC_FILE):
        return None
    t = json.load(open(TRAFFIC_FILE)).get(workload)
    if not t or t.get("source_sha256_16") != source_hash():
        return None                               # kernel changed since the counters
    return t["traffic_bytes_per_launch"]


# ----------------------------------------------------------------------------
def run_layer(w, steps, warmup, with_cpu, cpu_full=False, after_prefill=True, cpu_seconds=(12.0, 5.0, 1.0),
              min_timed_ms=None):
    """One workload's record. steps: the timed steps; with min_timed_ms, at
    least as many as fill that many milliseconds (short layers, whose few
    steps would otherwise time host jitter)."""
    dev = torch.device("cuda:0")
    log(f"[bench] workload {w.name}: generating inputs on {dev}")
    x = synthetic.make_inputs(w, device=dev)
    torch.cuda.synchronize()
    layer = Layer(w, x)
    log(f"[bench] {w.name}: stages and indices")
    st, idx = stages(layer, reps=max(2, min(5, steps)))
    flops = layer_flops(w, x, idx)
    f_total = sum(flops.values())
    n, D = w.seq_len, w.head_dim
    dense = 4.0 * D * (n * (n + 1) / 2) * w.batch * w.q_heads
    log(f"[bench] {w.name}: warmup {warmup}, timing {steps} steps")
    for _ in range(warmup):
        layer.step()
    torch.cuda.synchronize()
    if min_timed_ms:
        est = time_events(layer.step, 3)
        steps = max(steps, int(math.ceil(min_timed_ms / max(est, 1e-3))))
        log(f"[bench] {w.name}: {steps} timed steps (about {est:.3f} ms each)")
    s = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    with ClockSampler() as clk:
        ev[0].record(s)
        for i in range(steps):
            layer.step()
            ev[i + 1].record(s)
        torch.cuda.synchronize()
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    ms = ev[0].elapsed_time(ev[-1]) / steps
    log(f"[bench] {w.name}: {ms:.3f} ms/layer; stages {st}")
    res = {
        "ms_per_layer": ms, "tflops": f_total / (ms * 1e-3) / 1e12,
        "ms_per_layer_median": per_step[len(per_step) // 2], "ms_per_layer_min": per_step[0],
        "steps": steps, "dtype": w.dtype,
        "clock_during_steps": clk.summary(),
        "flops_computed_blocks": f_total, "flops_per_pattern": flops,
        "flops_dense_causal": dense, "density_vs_dense": f_total / dense,
        "stages_ms": st,
    }
    if sum(1 for p in ("vs", "bs", "st") if x.heads[p]) > 1:
        res["ms_per_layer_one_stream"] = time_events(lambda: layer.step(serial=True), steps)
        one = layer.one_launch()
        ms1 = time_events(one, steps)
        res["one_launch"] = {"ms_per_layer": ms1, "tflops": f_total / (ms1 * 1e-3) / 1e12,
                             "vs_three_calls": ms / ms1}
        log(f"[bench] {w.name}: one-launch mixed layer {ms1:.3f} ms")
    sb = stage_bytes(w, x, idx)
    res["stages_hbm"] = {k.replace("_ms", ""): {"bytes": v, "gbs": v / (st[k] * 1e-3) / 1e9,
                                                "frac_hbm": v / (st[k] * 1e-3) / 1e9 / PEAK_HBM_GBS}
                         for k, v in sb.items() if k in st}
    dom = "vs" if "vs" in flops else "bs" if "bs" in flops else None
    if dom:
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
        launch_ms = st[f"{dom}_attention_ms"]
        ach = flops[dom] / (launch_ms * 1e-3) / 1e12
        kernel = {("vs", "bf16"): DOMINANT, ("bs", "bf16"): "attn_blocks_single_kernel",
                  ("vs", "f32"): "attn_vs_f32_kernel", ("bs", "f32"): "attn_blocks_f32_kernel"}[(dom, w.dtype)]
        res["roofline"] = {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                           "frac": ach / peak,
                           "traffic": committed_traffic(w.name) if kernel == DOMINANT else None,
                           "kernel": kernel, "flops_per_launch": flops[dom], "launch_ms": launch_ms}
    if "bs" in idx and "bs_select_ms" in st:
        res["bs_select_roofline"] = bs_select_roofline(w, x, st["bs_select_ms"])
    if w.dtype == "bf16" and after_prefill:
        res["after_prefill"] = kv_retention_timing(layer, reps=3)
    if w.dtype == "bf16" and x.heads["bs"] and w.seq_len <= 32768:
        res["hier_prefill"] = hier_prefill_timing(layer, reps=3)
    if with_cpu:
        log(f"[bench] {w.name}: cpu baseline (oracle, {'whole layer' if cpu_full else 'bounded sample'})")
        res["cpu_baseline"] = cpu_baseline(layer, idx, f_total, seconds=cpu_seconds, full=cpu_full)
    del layer, x, idx
    torch.cuda.empty_cache()
    return res


# the secondary workloads are timed over at least this long (their own step
# count, reported as timed_steps)
SECONDARY_MIN_MS = 300.0

# layers whose whole-layer oracle finishes in seconds (timed in full)
FULL_ORACLE = ("vs_head_4k_f32", "bs_mha4_32k_bf16")


def workload_config(w):
    return {"workload": w.name, "batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
            "seq_len": w.seq_len, "head_dim": w.head_dim,
            "heads_per_pattern": {p: len(hs) for p, hs in synthetic.head_patterns(w).items()},
            "vertical_topk": w.vertical_topk, "slash_topk": w.slash_topk, "topk": w.topk,
            "init_blocks": w.init_blocks, "local_blocks": w.local_blocks}


def layer_record(r):
    """The per-layer fields of the JSON line for one timed workload."""
    peak = PEAK_BF16_TFLOPS if r["dtype"] == "bf16" else PEAK_F32_TFLOPS
    out = {
        "ms_per_layer": round(r["ms_per_layer"], 4),
        "ms_per_layer_median": round(r["ms_per_layer_median"], 4),
        "ms_per_layer_min": round(r["ms_per_layer_min"], 4),
        "timed_steps": r["steps"],
        "tflops": round(r["tflops"], 3),
        "pct_peak": round(100 * r["tflops"] / peak, 2),
        "peak_tflops": peak,
        "clock_during_steps": r.get("clock_during_steps"),
        "flops_computed_blocks": r["flops_computed_blocks"],
        "flops_per_pattern": r["flops_per_pattern"],
        "density_vs_dense": r["density_vs_dense"],
        "stages_ms": {k: round(v, 4) for k, v in r["stages_ms"].items()},
        "stages_hbm": {k: {kk: (round(vv, 4) if kk != "bytes" else vv) for kk, vv in v.items()}
                       for k, v in r["stages_hbm"].items()},
        "roofline": r.get("roofline"),
    }
    for key in ("bs_select_roofline", "after_prefill", "hier_prefill", "ms_per_layer_one_stream", "one_launch"):
        if r.get(key) is not None:
            out[key] = r[key]
    if r["dtype"] == "bf16":
        out["pct_bf16_peak"] = out["pct_peak"]
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b_1m_mixed_bf16",
                    choices=[w.name for w in synthetic.WORKLOADS])
    ap.add_argument("--secondary", default="all",
                    help="workloads timed beside the first: 'all' (every other named workload), "
                         "a comma-separated list, or 'none'")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB")
    ap.add_argument("--no-clock", action="store_true",
                    help="do not sample the clock with rocm-smi child processes")
    ap.add_argument("--summarize-pmc", metavar="DIR")
    ap.add_argument("--record", action="store_true",
                    help="with --summarize-pmc: store the summary for --workload in the traffic file")
    args = ap.parse_args()
    ClockSampler.enabled = not args.no_clock
    if args.summarize_pmc:
        summ = summarize_pmc(args.summarize_pmc, args.copy_probe or 1024)
        summ["workload"] = args.workload
        print(json.dumps(summ, indent=1))
        if args.record:
            allt = json.load(open(TRAFFIC_FILE)) if os.path.exists(TRAFFIC_FILE) else {}
            allt[args.workload] = summ
            json.dump(allt, open(TRAFFIC_FILE, "w"), indent=1)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer shards by "
              "(batch, kv-head group) with no exchange, which this benchmark does not launch.",
              file=sys.stderr)
        sys.exit(2)
    torch.cuda.set_device(0)
    if args.copy_probe:
        src = torch.empty(args.copy_probe * 2 ** 18, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)                            # device-to-device copy (blit kernel)
        torch.neg(src, out=dst)                   # the same bytes through an elementwise kernel
        torch.cuda.synchronize()
        del src, dst
    w = synthetic.BY_NAME[args.workload]
    dev_info = device_info()
    log(f"[bench] device {dev_info}")
    prim = run_layer(w, args.steps, args.warmup, not args.no_cpu_baseline,
                     cpu_full=w.name in FULL_ORACLE)
    res = {
        "metric": "sparse prefill attention ms/layer + effective TFLOP/s (% bf16 peak) at 128K/1M",
        "value": round(prim["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(prim["ms_per_layer"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic (seeded; planted sink/slash structure)",
        "config": workload_config(w),
        "device": dev_info,
    }
    res.update(layer_record(prim))
    if "cpu_baseline" in prim:
        res["cpu_baseline"] = prim["cpu_baseline"]
    res["pages_context"] = PAGES_CONTEXT
    if args.secondary == "all":
        names = [x.name for x in synthetic.WORKLOADS if x.name != w.name]
    elif args.secondary == "none":
        names = []
    else:
        names = [x for x in args.secondary.split(",") if x and x != w.name]
    res["secondary"] = []
    for name in names:
        w2 = synthetic.BY_NAME[name]
        sec = run_layer(w2, args.steps, args.warmup, not args.no_cpu_baseline,
                        cpu_full=w2.name in FULL_ORACLE, after_prefill=False, cpu_seconds=(5.0, 3.0, 1.0),
                        min_timed_ms=SECONDARY_MIN_MS)
        rec = {"workload": w2.name, "config": workload_config(w2), "dtype": w2.dtype}
        rec.update(layer_record(sec))
        if "cpu_baseline" in sec:
            rec["cpu_baseline"] = sec["cpu_baseline"]
        res["secondary"].append(rec)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
