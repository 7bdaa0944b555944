"""Seeded synthetic inputs shaped like the long-context prefill workloads.

This module only draws inputs. It holds none of the attention method's
arithmetic, so both the GPU path and the CPU oracle may be fed from it.

The recipe:

* Base: Q, K, V ~ N(0, 1) i.i.d., drawn in float32 with a seeded
  ``torch.Generator`` on the generation device, then cast to the workload
  dtype (round to nearest even for bf16).
* "vs" structure (planted sinks and slashes): per (batch, kv head) a smooth
  positional component P(t)[m] = alpha*sqrt(2/D)*cos(w_m*t + phi_m) with
  w_m ~ N(0, 1/sigma^2), phi_m ~ U[0, 2pi) (random Fourier features of a
  Gaussian kernel, so P(i).P(j) ~ alpha^2 exp(-(i-j)^2 / (2 sigma^2))) is added
  to K and to the Q of every query head of the group: attention then favours
  nearby diagonals. alpha = 8, sigma = the workload's slash_topk. Then key row
  0 and 8 further random key rows (distinct, from [1, n)) are scaled by 8:
  vertical lines (an attention sink and scattered heavy keys).
* "bs" structure (planted block clusters): per (batch, head) 16 clusters; each
  picks a key block kb uniformly (without replacement) and 4 query blocks
  uniformly from [kb, nb) (causal side, without replacement); a mean vector
  mu ~ N(0, I_D) is added to the 64 K rows of kb and the 64 Q rows of each
  chosen query block.
* Head patterns of mixed layers: 60/30/10 % of the heads vertical-slash /
  block-sparse / streaming by largest remainder under a seeded permutation, or
  seeded round-robin (head perm[t] gets pattern t mod 3).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import Dict, List, Optional

import torch

BLOCK = 64


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    seq_len: int
    head_dim: int
    dtype: str                      # "bf16" or "f32"
    structure: str                  # "vs" or "bs"
    assignment: str                 # "vs", "bs", "mixed-remainder", "mixed-roundrobin"
    vertical_topk: int = 0
    slash_topk: int = 0
    last_q: int = 64
    topk: int = 0
    init_blocks: int = 0
    local_blocks: int = 0
    seed: int = 0

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads, in order: a small fp32 vertical-slash head; a block-sparse
# MHA layer at 32K; a Llama-3-8B-shaped layer at 128K (all vertical-slash); the
# same layer at 1M tokens with mixed patterns; a batched Qwen2-7B-shaped mixed
# layer at 32K.
WORKLOADS: List[Workload] = [
    Workload("vs_head_4k_f32", 1, 1, 1, 4096, 64, "f32", "vs", "vs",
             vertical_topk=256, slash_topk=256, last_q=64, seed=0),
    Workload("bs_mha4_32k_bf16", 1, 4, 4, 32768, 128, "bf16", "bs", "bs",
             topk=100, seed=1),
    Workload("llama3_8b_128k_vs_bf16", 1, 32, 8, 131072, 128, "bf16", "vs", "vs",
             vertical_topk=1000, slash_topk=6096, last_q=64, seed=2),
    Workload("llama3_8b_1m_mixed_bf16", 1, 32, 8, 1048576, 128, "bf16", "vs",
             "mixed-remainder", vertical_topk=1000, slash_topk=6096, last_q=64,
             topk=256, init_blocks=1, local_blocks=64, seed=3),
    Workload("qwen2_7b_32k_b4_mixed_bf16", 4, 28, 4, 32768, 128, "bf16", "vs",
             "mixed-roundrobin", vertical_topk=500, slash_topk=3000, last_q=64,
             topk=64, init_blocks=1, local_blocks=32, seed=4),
]
BY_NAME: Dict[str, Workload] = {w.name: w for w in WORKLOADS}


def torch_dtype(name: str) -> torch.dtype:
    return {"bf16": torch.bfloat16, "f32": torch.float32}[name]


def head_patterns(w: Workload) -> Dict[str, List[int]]:
    """Query heads per pattern ("vs", "bs", "st"), each list ascending."""
    H = w.q_heads
    if w.assignment in ("vs", "bs"):
        return {"vs": list(range(H)) if w.assignment == "vs" else [],
                "bs": list(range(H)) if w.assignment == "bs" else [], "st": []}
    g = torch.Generator(device="cpu").manual_seed(10_000 + w.seed)
    perm = torch.randperm(H, generator=g).tolist()
    if w.assignment == "mixed-remainder":
        quotas = [0.6 * H, 0.3 * H, 0.1 * H]
        counts = [int(math.floor(x)) for x in quotas]
        order = sorted(range(3), key=lambda t: -(quotas[t] - counts[t]))
        for t in order[: H - sum(counts)]:
            counts[t] += 1
        vs = perm[: counts[0]]
        bs = perm[counts[0]: counts[0] + counts[1]]
        st = perm[counts[0] + counts[1]:]
    elif w.assignment == "mixed-roundrobin":
        vs = [perm[t] for t in range(H) if t % 3 == 0]
        bs = [perm[t] for t in range(H) if t % 3 == 1]
        st = [perm[t] for t in range(H) if t % 3 == 2]
    else:
        raise ValueError(w.assignment)
    return {"vs": sorted(vs), "bs": sorted(bs), "st": sorted(st)}


def pattern_list(w: Workload) -> List[Optional[str]]:
    """The same assignment as one pattern name per query head."""
    out: List[Optional[str]] = [None] * w.q_heads
    for pat, heads in head_patterns(w).items():
        for h in heads:
            out[h] = pat
    return out


@dataclass
class Inputs:
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    heads: Dict[str, List[int]] = field(default_factory=dict)
    workload: Optional[Workload] = None
    # (batch, head) -> planted (key block, [query blocks]) pairs ("bs" structure)
    planted: Dict[tuple, list] = field(default_factory=dict)


def _vs_structure(q, k, b, kvh, G, n, D, sigma, g, dev):
    alpha = 8.0
    w = torch.randn(D, generator=g, device=dev, dtype=torch.float64) / sigma
    phi = torch.rand(D, generator=g, device=dev, dtype=torch.float64) * (2 * math.pi)
    amp = alpha * math.sqrt(2.0 / D)
    step = 1 << 16
    for t0 in range(0, n, step):
        t = torch.arange(t0, min(n, t0 + step), device=dev, dtype=torch.float64)
        P = (amp * torch.cos(t[:, None] * w[None, :] + phi[None, :])).float()
        k[b, kvh, t0:t0 + P.shape[0]] += P
        for h in range(kvh * G, (kvh + 1) * G):
            q[b, h, t0:t0 + P.shape[0]] += P
    heavy = torch.randperm(n - 1, generator=g, device=dev)[:8] + 1 if n > 1 else \
        torch.zeros(0, dtype=torch.long, device=dev)
    k[b, kvh, 0] *= 8.0
    k[b, kvh, heavy] *= 8.0


def _bs_structure(q, k, b, h, n, D, g, dev):
    """Returns the planted (key block, [query blocks]) pairs."""
    nb = (n + BLOCK - 1) // BLOCK
    ncl = min(16, nb)
    kbs = torch.randperm(nb, generator=g, device=dev)[:ncl].tolist()
    planted = []
    for kb in kbs:
        mu = torch.randn(D, generator=g, device=dev, dtype=torch.float32)
        cand = nb - kb
        qbs = (torch.randperm(cand, generator=g, device=dev)[: min(4, cand)] + kb).tolist()
        k[b, h, kb * BLOCK: (kb + 1) * BLOCK] += mu
        for qa in qbs:
            q[b, h, qa * BLOCK: (qa + 1) * BLOCK] += mu
        planted.append((kb, sorted(qbs)))
    return planted


def make_inputs(w: Workload, device="cpu") -> Inputs:
    """Draw q [B,Hq,n,D], k/v [B,Hkv,n,D] for workload ``w`` on ``device``."""
    dev = torch.device(device)
    g = torch.Generator(device=dev).manual_seed(w.seed)
    B, Hq, Hkv, n, D = w.batch, w.q_heads, w.kv_heads, w.seq_len, w.head_dim
    G = Hq // Hkv
    out_dt = torch_dtype(w.dtype)
    q = torch.empty((B, Hq, n, D), dtype=out_dt, device=dev)
    k = torch.empty((B, Hkv, n, D), dtype=out_dt, device=dev)
    v = torch.empty((B, Hkv, n, D), dtype=out_dt, device=dev)
    planted = {}
    for b in range(B):
        for kvh in range(Hkv):
            # one kv group at a time, in float32, to bound peak memory
            qg = torch.randn((1, G, n, D), generator=g, device=dev, dtype=torch.float32)
            kg = torch.randn((1, 1, n, D), generator=g, device=dev, dtype=torch.float32)
            vg = torch.randn((1, 1, n, D), generator=g, device=dev, dtype=torch.float32)
            if w.structure == "vs":
                _vs_structure(qg, kg, 0, 0, G, n, D, float(max(1, w.slash_topk)), g, dev)
            elif w.structure == "bs":
                if G != 1:
                    raise ValueError("block-cluster structure is drawn per MHA head")
                planted[(b, kvh)] = _bs_structure(qg, kg, 0, 0, n, D, g, dev)
            q[b, kvh * G:(kvh + 1) * G] = qg[0].to(out_dt)
            k[b, kvh] = kg[0, 0].to(out_dt)
            v[b, kvh] = vg[0, 0].to(out_dt)
            del qg, kg, vg
    return Inputs(q, k, v, head_patterns(w), w, planted)
