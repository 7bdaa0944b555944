#!/usr/bin/env python3
"""One sparse prefill attention layer per step on one MI355X.

A step runs the whole path for every head of the layer: vertical-slash heads
(estimate, top-k, sparse format, attention), block-sparse heads (pooling,
block selection, attention) and streaming heads (attention), each call over
its head subset, all writing one output tensor, on one stream. Inputs are
seeded synthetic tensors resident in HBM before timing starts.

Prints one JSON line. `value` is the effective TFLOP/s of the layer: the
attention FLOPs of the computed key blocks (4 * head_dim * sum over query
blocks of rows x keys, before the causal trim of the diagonal tile) divided by
the measured layer time. `roofline` reports the dominant kernel (the
vertical-slash attention launch) against the bf16 MFMA peak, timed alone with
HIP events on the stream it runs on. `cpu_baseline` times the CPU oracle on a
bounded sample of the same layer and scales it to the whole layer.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


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
    sel, n_sel = sel.cpu().numpy(), n_sel.cpu().numpy()
    rows, nb, _ = sel.shape
    last = n - BLK * (nb - 1)
    keys = np.zeros((rows, nb), np.int64)
    for r in range(rows):
        for a in range(nb):
            cs = sel[r, a, : n_sel[r, a]]
            keys[r, a] = BLK * len(cs) - (BLK - last) * int((cs == nb - 1).sum())
    return keys


def st_keys_per_block(n, init_blocks, local_blocks):
    nb = (n + BLK - 1) // BLK
    last = n - BLK * (nb - 1)
    keys = np.zeros(nb, np.int64)
    for a in range(nb):
        cs = [c for c in range(a + 1) if c < init_blocks or a - c < local_blocks]
        keys[a] = BLK * len(cs) - (BLK - last) * (nb - 1 in cs)
    return keys


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
        self.hp = {p: (hs if hs else None) for p, hs in x.heads.items()}
        all_vs = len(x.heads["vs"]) == w.q_heads
        self.vs_heads = None if all_vs else x.heads["vs"]
        self.ws_vs = self.ws_bs = None
        if x.heads["vs"]:
            nbytes = dsa.vertical_slash_workspace_bytes(self.q, self.k, w.vertical_topk, w.slash_topk,
                                                        self.vs_heads)
            self.ws_vs = torch.empty(nbytes, dtype=torch.uint8, device=self.q.device)
        if x.heads["bs"]:
            nbytes = dsa.block_sparse_workspace_bytes(self.q, self.k, w.topk, x.heads["bs"])
            self.ws_bs = torch.empty(nbytes, dtype=torch.uint8, device=self.q.device)

    def step(self):
        w, x = self.w, self.x
        if x.heads["vs"]:
            dsa.vertical_slash_sparse_attention(self.q, self.k, self.v, w.vertical_topk, w.slash_topk,
                                                last_q=w.last_q, heads=self.vs_heads, out=self.o,
                                                workspace=self.ws_vs)
        if x.heads["bs"]:
            dsa.block_sparse_attention(self.q, self.k, self.v, w.topk, heads=x.heads["bs"], out=self.o,
                                       workspace=self.ws_bs)
        if x.heads["st"]:
            dsa.streaming_attention(self.q, self.k, self.v, w.init_blocks, w.local_blocks,
                                    heads=x.heads["st"], out=self.o)

    # indices of the vertical-slash and block-sparse heads through the stage calls
    def indices(self):
        w, x = self.w, self.x
        out = {}
        if x.heads["vs"]:
            vg, sg = dsa.vs_estimate(self.q, self.k, last_q=w.last_q, heads=x.heads["vs"])
            V = dsa.topk(vg, w.vertical_topk)
            S = dsa.topk(sg, w.slash_topk, 0)
            out["vs"] = dsa.vs_build_index(V, S, w.seq_len)
            del vg, sg
        if x.heads["bs"]:
            qp = dsa.bs_pool(self.q, x.heads["bs"])
            kp_all = dsa.bs_pool(self.k)
            G = w.q_heads // w.kv_heads
            idx = torch.tensor([b * w.kv_heads + h // G for b in range(w.batch) for h in x.heads["bs"]],
                               device=self.q.device)
            out["bs"] = dsa.bs_select(qp, kp_all[idx].contiguous(), w.topk)
        return out


def time_events(fn, reps):
    """Average ms per call of fn, HIP events on torch's current stream (the
    stream every library call is enqueued on)."""
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    fn()
    e0.record(s)
    for _ in range(reps):
        fn()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


# ----------------------------------------------------------------------------
# CPU oracle on a bounded sample
# ----------------------------------------------------------------------------
def cpu_baseline(layer, idx, flops_total, budget_blocks=6):
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
        blocks = rng.choice(nb, budget_blocks, replace=False)
        t0 = time.perf_counter()
        keys_s = 0
        for a in blocks:
            keys = O.vs_block_keys(iv, V, int(a), n)
            rows = np.arange(a * BLK, min(n, a * BLK + BLK))
            O.masked_attention(qh[rows], rows, keys, kh, vh, sc)
            keys_s += len(keys) * len(rows)
        t_att = time.perf_counter() - t0
        # scale: estimate per head, attention per (row x key) of all VS heads
        iv_g, n_iv_g, cols_g, n_cols_g = idx["vs"]
        keys_all = vs_keys_per_block(iv_g, n_iv_g, n_cols_g, n)
        rk_all = float((keys_all * rows_per_block(n)).sum())
        rows_vs = w.batch * len(x.heads["vs"])
        t_total += t_est * rows_vs + t_att * rk_all / keys_s
        parts.append(f"vs head {h}: full estimate+top-k+intervals, attention of {budget_blocks} blocks")
    if x.heads["bs"]:
        h = x.heads["bs"][0]
        qh, kh, vh = f(layer.q[0, h]), f(layer.k[0, h // G]), f(layer.v[0, h // G])
        t0 = time.perf_counter()
        qp, kp = O.mean_pool(qh), O.mean_pool(kh)
        t_pool = time.perf_counter() - t0
        blocks = rng.choice(nb, budget_blocks, replace=False)
        t0 = time.perf_counter()
        keys_s = 0
        sel_rows = 0
        for a in blocks:
            L = O.to_f32(O.block_logits(qp[a:a + 1], kp[: a + 1], sc))[0]
            sel = O.topk_indices(L, w.topk, forced=(int(a),))
            keys = O.blocks_to_keys(sel, n)
            rows = np.arange(a * BLK, min(n, a * BLK + BLK))
            O.masked_attention(qh[rows], rows, keys, kh, vh, sc)
            keys_s += len(keys) * len(rows)
            sel_rows += 1
        t_blk = time.perf_counter() - t0
        sel_g, n_sel_g = idx["bs"]
        keys_all = bs_keys_per_block(sel_g, n_sel_g, n)
        rk_all = float((keys_all * rows_per_block(n)).sum())
        rows_bs = w.batch * len(x.heads["bs"])
        t_total += t_pool * rows_bs + t_blk * rk_all / keys_s
        parts.append(f"bs head {h}: pooling, select+attention of {budget_blocks} blocks")
    if x.heads["st"]:
        h = x.heads["st"][0]
        qh, kh, vh = f(layer.q[0, h]), f(layer.k[0, h // G]), f(layer.v[0, h // G])
        blocks = rng.choice(nb, budget_blocks, replace=False)
        t0 = time.perf_counter()
        keys_s = 0
        for a in blocks:
            keys = O.blocks_to_keys(O.streaming_blocks(int(a), w.init_blocks, w.local_blocks), n)
            rows = np.arange(a * BLK, min(n, a * BLK + BLK))
            O.masked_attention(qh[rows], rows, keys, kh, vh, sc)
            keys_s += len(keys) * len(rows)
        t_att = time.perf_counter() - t0
        rk = float((st_keys_per_block(n, w.init_blocks, w.local_blocks) * rows_per_block(n)).sum())
        t_total += t_att * rk / keys_s * w.batch * len(x.heads["st"])
        parts.append(f"st head {h}: attention of {budget_blocks} blocks")
    cores = len(os.sched_getaffinity(0))
    return {"value": flops_total / t_total / 1e12, "unit": "TFLOP/s (effective, computed blocks)",
            "cores": cores, "kind": "oracle",
            "sample": "; ".join(parts) + "; scaled to the whole layer by head count and row x key count",
            "extrapolated_ms_per_layer": t_total * 1e3}


# ----------------------------------------------------------------------------
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_8b_128k_vs_bf16",
                    choices=[w.name for w in synthetic.WORKLOADS])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer shards by "
              "(batch, kv-head group) with no exchange, which this benchmark does not launch.",
              file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = synthetic.BY_NAME[args.workload]
    log(f"[bench] workload {w.name}: generating inputs on {dev}")
    x = synthetic.make_inputs(w, device=dev)
    torch.cuda.synchronize()
    layer = Layer(w, x)
    n, D = w.seq_len, w.head_dim

    log("[bench] indices for FLOP accounting")
    idx = layer.indices()
    flops = {}
    if "vs" in idx:
        iv, n_iv, cols, n_cols = idx["vs"]
        flops["vs"] = attn_flops(vs_keys_per_block(iv, n_iv, n_cols, n), n, D)
    if "bs" in idx:
        flops["bs"] = attn_flops(bs_keys_per_block(*idx["bs"], n), n, D)
    if x.heads["st"]:
        flops["st"] = attn_flops(st_keys_per_block(n, w.init_blocks, w.local_blocks), n, D) \
            * w.batch * len(x.heads["st"])
    f_total = sum(flops.values())
    dense = 4.0 * D * (n * (n + 1) / 2) * w.batch * w.q_heads

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        layer.step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record(s)
    for _ in range(args.steps):
        layer.step()
    e1.record(s)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1) / args.steps
    log(f"[bench] {ms:.3f} ms/layer (wall {t_wall / args.steps * 1e3:.3f})")

    # per-stage times and the dominant kernel, each timed alone
    stages = {}
    reps = max(2, min(10, args.steps))
    roof = None
    if "vs" in idx:
        iv, n_iv, cols, n_cols = idx["vs"]
        t_attn = time_events(lambda: dsa.sparse_attention_vs(
            layer.q, layer.k, layer.v, iv, n_iv, cols, n_cols, heads=x.heads["vs"], out=layer.o), reps)
        stages["vs_attention_ms"] = t_attn
        stages["vs_estimate_ms"] = time_events(lambda: dsa.vs_estimate(layer.q, layer.k, heads=x.heads["vs"]), reps)
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
        ach = flops["vs"] / (t_attn * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": ach, "peak": peak, "unit": "TFLOP/s", "frac": ach / peak,
                "traffic": None, "kernel": "attn_vs_kernel",
                "flops_per_launch": flops["vs"]}
    if "bs" in idx:
        sel, n_sel = idx["bs"]
        stages["bs_attention_ms"] = time_events(lambda: dsa.sparse_attention_blocks(
            layer.q, layer.k, layer.v, sel, n_sel, heads=x.heads["bs"], out=layer.o), reps)
    if x.heads["st"]:
        stages["st_attention_ms"] = time_events(lambda: dsa.streaming_attention(
            layer.q, layer.k, layer.v, w.init_blocks, w.local_blocks, heads=x.heads["st"], out=layer.o), reps)
    log(f"[bench] stages {stages}")

    value = f_total / (ms * 1e-3) / 1e12
    res = {
        "metric": "sparse prefill attention ms/layer + effective TFLOP/s (% bf16 peak) at 128K/1M",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "q_heads": w.q_heads, "kv_heads": w.kv_heads,
                   "seq_len": n, "head_dim": D,
                   "heads_per_pattern": {p: len(hs) for p, hs in x.heads.items()},
                   "vertical_topk": w.vertical_topk, "slash_topk": w.slash_topk, "topk": w.topk,
                   "init_blocks": w.init_blocks, "local_blocks": w.local_blocks},
        "ms_per_layer": round(ms, 4),
        "pct_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "flops_computed_blocks": f_total, "flops_dense_causal": dense,
        "density_vs_dense": f_total / dense,
        "stages_ms": {k: round(v, 4) for k, v in stages.items()},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle, bounded sample)")
        res["cpu_baseline"] = cpu_baseline(layer, idx, f_total)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
