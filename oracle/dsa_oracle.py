"""CPU oracle for dynamic sparse attention in the long-context prefill phase.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The GPU
library never imports it and shares no code with it.

Everything here is plain numpy in float64: slow, direct and meant to be checked
by eye against the pages it follows. Sources, cited by page title and section:

* [MInf] "MInference 1.0" summary article (developer.volcengine.com), §1
  "Problem Formulation", §2.2 "Sparsity Indices Approximation and Dynamic
  Sparse Attention Calculation" (Vertical-Slash Head, Block-Sparse Head), and
  the kernel-only usage listing at the end of the article.
* [Novita] "How KV sparsity achieves 1.5x acceleration for vLLM" (Novita AI
  blog), §2 "Modificación de Atención": softmax statistics (rowmax, l) reused to
  score keys over a window of the last queries, with the q start/end
  restriction.
* [IHiP] InfiniteHiP summary (www.dtcms.com), section "模块化分层令牌剪枝算法"
  (modular hierarchical token pruning): fixed-length chunks, the
  highest-scoring token of each chunk, only the best chunks go on to the next
  stage, stacked stages refine a block-sparse mask per query block.

Readings taken where the pages are silent or garbled:

R1  Mask semantics [MInf §1]: the constant c of A(M) = softmax(QK^T/sqrt(d) -
    c(1-M)) is taken to infinity, so masked entries are excluded exactly. The
    scale is 1/sqrt(head_dim). The mask is always intersected with causality
    (prefill). A row with no allowed key outputs zeros.
R2  VS estimate [MInf §2.2 VS head; Novita §2]: the estimated attention is the
    causal softmax of the last ``last_q`` query rows against all keys, each row
    normalised over its whole causal range. Vertical score v[j] = sum over
    those rows of p[r, j]; slash score s[d] = sum over those rows of
    p[r, i_r - d] (i_r is the row's position; partial diagonals are not
    renormalised). Both are rounded to float32.
R3  Top-k: forced indices rank first, then larger score, then smaller index;
    -0.0 counts as +0.0 and NaN as -inf; k is clamped to the candidate count;
    the result is returned in ascending index order.
R4  VS forced entries: slash offset 0 (the main diagonal) is always selected
    and takes one of the slash_topk slots; no vertical is forced.
R5  VS sparse format [MInf §2.2 "convert to sparse format"]: query block a
    covers rows [64a, 64a+64) of the 64-row grid. Slash offset d covers, in
    that block, the key rectangle [64a - d, 64a + 64 - d), clipped to [0, n).
    Offsets whose gap is <= 64 give touching rectangles and are merged into
    one interval [d_lo, d_hi], which covers keys
    [max(0, 64a - d_hi), min(n, 64a + 64 - d_lo)). Verticals not already inside
    one of the block's ranges and below the block's end form the block's
    column list. The element mask is (range or column) and causal.
R6  Block-sparse [MInf §2.2 BS head]: Q and K are mean-pooled over 64-row
    blocks (a ragged last block averages its actual rows). The block logit is
    L[a, c] = scale * Qp[a] . Kp[c] for c <= a, rounded to float32; selection
    ranks logits (softmax is monotone per row, so the set is the same) with the
    diagonal block forced.
R7  Streaming / A-shape [MInf usage listing, streaming_forward(init_num,
    local_window_num)]: key block c is kept for query block a iff c <= a and
    (c < init_blocks or a - c < local_blocks); the local window counts the
    diagonal block.
R8  GQA: query head h reads kv head h // (q_heads / kv_heads).
R10 Sparse decode [Novita §2: decoding uses only the kept KV entries; MInf §1]:
    one new query row per head, placed after the whole cache, attends over a
    set of cached key positions (every position when none is given) with the
    softmax of R1; an empty set gives zeros. Each head has its own set (GQA
    heads share the cache, not the set).
R9  KV retention [Novita §2, the PyramidKV score; the formula itself is lost
    from the page text]: a key's retention score is the sum of its softmax
    probabilities over the window of the last ``window`` query rows (each row
    normalised over its whole causal range, as in R2), rounded to float32;
    per head the ``keep`` highest-scoring keys are kept (R3, no forced entry).
    A window longer than the prompt is clamped to it. Not taken: also keeping
    the window's own tokens whatever their score (the page does not say so).
R11 Hierarchical chunk pruning [IHiP, modular hierarchical token pruning]: a
    query vector sees the keys j < limit. A token's score is its logit
    scale * q . k_j. Stage s has a chunk length c_s and a keep count k_s; the
    lengths decrease and each divides the one before. Stage 1's candidates are
    the chunks [x c_1, (x+1) c_1) that hold a visible key; stage s > 1 splits
    each chunk kept by stage s-1 into chunks of c_s and takes those holding a
    visible key. A candidate's score is the largest score of its visible
    tokens (the chunk's highest-scoring token, found exactly); the k_s best
    candidates are kept (R3), with the chunk holding key limit - 1 forced, so
    the query's own neighbourhood is never pruned. The result is the last
    stage's kept chunk ids, ascending. Decode: the query is the new row and
    limit = n; the row then attends over the keys of the kept chunks (R10).
    Prefill (an alternative block-sparse estimator): the query of block a is
    its mean-pooled row (R6) and limit = min(n, 64 (a + 1)); with a last chunk
    length of 64 the kept chunks are key blocks, attended as in R6. Not taken:
    an approximate search for the highest-scoring token (the page says that it
    is found in parallel and efficiently, not how).
"""
from __future__ import annotations

import math
from typing import Dict, List, Sequence, Tuple

import numpy as np

BLOCK = 64


# ----------------------------------------------------------------------------
# helpers
# ----------------------------------------------------------------------------
def f64(x) -> np.ndarray:
    """Any array-like (numpy or a CPU torch tensor) as float64 numpy."""
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def default_scale(head_dim: int) -> float:
    """R1: the softmax scale is 1/sqrt(head_dim) [MInf §1]."""
    return 1.0 / math.sqrt(head_dim)


def num_blocks(n: int) -> int:
    return (n + BLOCK - 1) // BLOCK


def kv_head_of(h: int, q_heads: int, kv_heads: int) -> int:
    """R8: consecutive grouping of query heads onto kv heads."""
    return h // (q_heads // kv_heads)


# ----------------------------------------------------------------------------
# attention under an explicit mask  [MInf §1, R1]
# ----------------------------------------------------------------------------
def masked_attention(q_rows: np.ndarray, row_pos: np.ndarray, keys: np.ndarray,
                     k: np.ndarray, v: np.ndarray, scale: float) -> np.ndarray:
    """Softmax attention of query rows over the key positions ``keys``.

    q_rows [R, D] are the queries at sequence positions ``row_pos`` [R];
    ``keys`` is an ascending array of allowed key positions (the row's mask
    before causality); k, v [n, D]. Causality keeps key j for row i iff j <= i.
    Two-pass softmax: max, then the exponential sum. Returns [R, D] float64.
    """
    q_rows = f64(q_rows)
    out = np.zeros((q_rows.shape[0], v.shape[1]), dtype=np.float64)
    if len(keys) == 0:
        return out
    kk = k[keys]
    vv = v[keys]
    logits = scale * (q_rows @ kk.T)                     # [R, |keys|]
    for r in range(q_rows.shape[0]):
        allowed = keys <= row_pos[r]
        if not allowed.any():
            continue
        lr = logits[r, allowed]
        m = lr.max()
        e = np.exp(lr - m)
        p = e / e.sum()
        out[r] = p @ vv[allowed]
    return out


def dense_causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                           scale: float) -> np.ndarray:
    """Full causal attention of one head (every key allowed), [n, D]."""
    n = q.shape[0]
    return masked_attention(q, np.arange(n), np.arange(n), f64(k), f64(v), scale)


# ----------------------------------------------------------------------------
# vertical-slash estimate  [MInf §2.2 VS head; Novita §2; R2]
# ----------------------------------------------------------------------------
def vs_scores(q: np.ndarray, k: np.ndarray, last_q: int, scale: float
              ) -> Tuple[np.ndarray, np.ndarray]:
    """Vertical and slash scores of one query head, float64 [n] each.

    The window is the last ``min(last_q, n)`` query rows [Novita §2, q
    start/end restriction]; each row's softmax runs over its whole causal range
    (R2). v[j] sums p over rows; s[d] sums p over the diagonal i - j = d.
    """
    q = f64(q)
    k = f64(k)
    n = q.shape[0]
    lq = min(last_q, n)
    rows = np.arange(n - lq, n)
    logits = scale * (q[rows] @ k.T)                      # [lq, n]
    v = np.zeros(n, dtype=np.float64)
    s = np.zeros(n, dtype=np.float64)
    for r, i in enumerate(rows):
        lr = logits[r, : i + 1]
        m = lr.max()
        e = np.exp(lr - m)
        p = e / e.sum()
        v[: i + 1] += p
        s[: i + 1] += p[::-1]          # s[d] += p[i - d] for d = 0..i
    return v, s


def to_f32(x: np.ndarray) -> np.ndarray:
    """Round to float32 (round to nearest even), the stored score precision."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


# ----------------------------------------------------------------------------
# top-k  [MInf §2.2 "top-k vertical / slash indices", "top-k blocks"; R3]
# ----------------------------------------------------------------------------
def canonical_scores(x) -> np.ndarray:
    """R3: -0.0 -> +0.0 and NaN -> -inf, compared as float64."""
    y = np.asarray(x, dtype=np.float64).copy()
    y[np.isnan(y)] = -np.inf
    y[y == 0.0] = 0.0
    return y


def topk_indices(x, k: int, forced: Sequence[int] = ()) -> np.ndarray:
    """Indices of the top min(k, len(x)) entries, ascending (R3).

    Rank order: forced entries first, then score descending, then index
    ascending (a strict total order, so the selected set is unique).
    """
    key = canonical_scores(x)
    n = key.shape[0]
    k = max(0, min(int(k), n))
    is_forced = np.zeros(n, dtype=bool)
    if len(forced):
        is_forced[np.asarray(list(forced), dtype=np.int64)] = True
    # np.lexsort: the last key is the primary one.
    order = np.lexsort((np.arange(n), -key, ~is_forced))
    return np.sort(order[:k]).astype(np.int64)


# ----------------------------------------------------------------------------
# KV retention after prefill  [Novita §2; R9]
# ----------------------------------------------------------------------------
def kv_retention_scores(q: np.ndarray, k: np.ndarray, window: int, scale: float) -> np.ndarray:
    """Retention score of every key of one query head, float64 [n]: the sum of
    the key's softmax probabilities over the last min(window, n) query rows
    [Novita §2: scores from the window of the last queries, each row's
    probabilities p = exp(qk - rowmax) / l]."""
    q = f64(q)
    k = f64(k)
    n = q.shape[0]
    w = min(int(window), n)
    S = np.zeros(n, dtype=np.float64)
    for i in range(n - w, n):
        lr = scale * (k[: i + 1] @ q[i])
        e = np.exp(lr - lr.max())
        S[: i + 1] += e / e.sum()
    return S


def decode_attention(q_row, k, v, keys=None, scale: float | None = None) -> np.ndarray:
    """One decode row over the cached keys ``keys`` (all when None), float64
    [D] (R10): the masked attention of R1 for a row after the whole cache."""
    k = f64(k)
    v = f64(v)
    n = k.shape[0]
    scale = default_scale(k.shape[1]) if scale is None else scale
    keys = np.arange(n) if keys is None else np.asarray(keys, dtype=np.int64)
    return masked_attention(f64(q_row)[None, :], np.array([n]), keys, k, v, scale)[0]


def kv_retention(q, k, window: int, keep: int, scale: float | None = None
                 ) -> Tuple[np.ndarray, np.ndarray]:
    """(float32 scores, kept keys ascending) of one query head (R9)."""
    scale = default_scale(np.shape(q)[1]) if scale is None else scale
    S32 = to_f32(kv_retention_scores(q, k, window, scale))
    return S32, topk_indices(S32, keep)


# ----------------------------------------------------------------------------
# vertical-slash sparse format  [MInf §2.2 "convert to sparse format"; R4, R5]
# ----------------------------------------------------------------------------
def vs_select(v32: np.ndarray, s32: np.ndarray, vertical_topk: int,
              slash_topk: int) -> Tuple[np.ndarray, np.ndarray]:
    """V = TopK(v, vk) and S = TopK(s, sk) with offset 0 forced (R4)."""
    V = topk_indices(v32, vertical_topk)
    S = topk_indices(s32, slash_topk, forced=(0,))
    return V, S


def merge_offsets(S: Sequence[int], block: int = BLOCK) -> List[Tuple[int, int]]:
    """R5: ascending offsets merged into [d_lo, d_hi] while the gap <= block."""
    intervals: List[List[int]] = []
    for d in sorted(int(x) for x in S):
        if intervals and d - intervals[-1][1] <= block:
            intervals[-1][1] = d
        else:
            intervals.append([d, d])
    return [(a, b) for a, b in intervals]


def vs_block_ranges(intervals: Sequence[Tuple[int, int]], a: int, n: int
                    ) -> List[Tuple[int, int]]:
    """R5: half-open key ranges of query block a, one per non-empty interval,
    in interval order (which is descending key order)."""
    r0 = a * BLOCK
    out = []
    for d_lo, d_hi in intervals:
        lo = max(0, r0 - d_hi)
        hi = min(n, r0 + BLOCK - d_lo)
        if lo < hi:
            out.append((lo, hi))
    return out


def vs_block_cols(V: Sequence[int], ranges: Sequence[Tuple[int, int]], a: int,
                  n: int) -> np.ndarray:
    """R5: verticals below the block's end and outside every range, ascending."""
    end = min(n, (a + 1) * BLOCK)
    cols = [int(j) for j in sorted(V)
            if j < end and not any(lo <= j < hi for lo, hi in ranges)]
    return np.asarray(cols, dtype=np.int64)


def vs_block_keys(intervals, V, a: int, n: int) -> np.ndarray:
    """All key positions of block a before causality, ascending."""
    ranges = vs_block_ranges(intervals, a, n)
    parts = [np.arange(lo, hi) for lo, hi in ranges]
    parts.append(vs_block_cols(V, ranges, a, n))
    keys = np.concatenate(parts) if parts else np.zeros(0, np.int64)
    return np.unique(keys.astype(np.int64))


# ----------------------------------------------------------------------------
# block-sparse estimate  [MInf §2.2 BS head; R6]
# ----------------------------------------------------------------------------
def mean_pool(x: np.ndarray) -> np.ndarray:
    """Mean of each 64-row block (a ragged last block averages its rows)."""
    x = f64(x)
    n = x.shape[0]
    return np.stack([x[a * BLOCK: min(n, (a + 1) * BLOCK)].mean(axis=0)
                     for a in range(num_blocks(n))])


def block_logits(qp: np.ndarray, kp: np.ndarray, scale: float) -> np.ndarray:
    """L[a, c] = scale * Qp[a] . Kp[c], float64 [nb, nb] (only c <= a is used)."""
    return scale * (f64(qp) @ f64(kp).T)


def block_select(L32: np.ndarray, topk: int) -> List[np.ndarray]:
    """Sel(a) = TopK(L[a, 0..a], topk) with c = a forced, ascending (R6)."""
    nb = L32.shape[0]
    return [topk_indices(L32[a, : a + 1], topk, forced=(a,)) for a in range(nb)]


def blocks_to_keys(blocks: Sequence[int], n: int) -> np.ndarray:
    parts = [np.arange(c * BLOCK, min(n, (c + 1) * BLOCK)) for c in sorted(blocks)]
    return np.concatenate(parts).astype(np.int64) if parts else np.zeros(0, np.int64)


# ----------------------------------------------------------------------------
# streaming / A-shape  [MInf usage listing; R7]
# ----------------------------------------------------------------------------
def streaming_blocks(a: int, init_blocks: int, local_blocks: int) -> np.ndarray:
    return np.asarray([c for c in range(a + 1)
                       if c < init_blocks or a - c < local_blocks], dtype=np.int64)


# ----------------------------------------------------------------------------
# multi-stage hierarchical chunk pruning  [IHiP modular hierarchical token
# pruning; R11]
# ----------------------------------------------------------------------------
def token_scores(q_vec, k, limit: int, scale: float) -> np.ndarray:
    """scale * q . k_j of the visible keys j < limit, float64 [limit]."""
    return scale * (f64(k)[:limit] @ f64(q_vec))


def hier_prune(q_vec, k, limit: int, stages: Sequence[Tuple[int, int]], scale: float,
               fine_max=None) -> np.ndarray:
    """Chunk ids (of the last stage's length) kept by the stages, ascending.

    ``stages``: (chunk length, keep count) per stage, outermost first.
    ``fine_max`` (optional float32 [ceil(limit / 64)]): the largest token score
    of every 64-key block, as another implementation computed it; a chunk's
    score is then the largest of its blocks' values, which is the same
    quantity, so the selection steps can be run on that implementation's
    scores. Otherwise the token scores are computed here (float64).
    """
    if fine_max is None:
        s = token_scores(q_vec, k, limit, scale)

        def chunk_score(x, c):
            return s[x * c: min(limit, (x + 1) * c)].max()
    else:
        fm = np.asarray(fine_max, dtype=np.float32)

        def chunk_score(x, c):
            return fm[x * c // BLOCK: (min(limit, (x + 1) * c) + BLOCK - 1) // BLOCK].max()

    kept = None
    prev_c = None
    for c, keep in stages:
        if kept is None:   # stage 1: every chunk holding a visible key
            cand = list(range((limit + c - 1) // c))
        else:              # the sub-chunks of the chunks the last stage kept
            r = prev_c // c
            cand = [y for x in kept for y in range(x * r, (x + 1) * r) if y * c < limit]
        scores = np.array([chunk_score(x, c) for x in cand])
        forced = cand.index((limit - 1) // c)
        pick = topk_indices(scores, keep, forced=(forced,))
        kept = [cand[i] for i in pick]
        prev_c = c
    return np.asarray(kept, dtype=np.int64)


def chunks_to_keys(chunks: Sequence[int], c: int, limit: int) -> np.ndarray:
    """Key positions (< limit) of the chunks of length c, ascending."""
    parts = [np.arange(x * c, min(limit, (x + 1) * c)) for x in sorted(chunks)]
    return np.concatenate(parts).astype(np.int64) if parts else np.zeros(0, np.int64)


def hier_decode(q_row, k, v, stages, scale: float | None = None, fine_max=None) -> dict:
    """Decode row over the keys the pruning keeps (R11, R10)."""
    k, v = f64(k), f64(v)
    n, D = k.shape
    scale = default_scale(D) if scale is None else scale
    chunks = hier_prune(q_row, k, n, stages, scale, fine_max)
    keys = chunks_to_keys(chunks, stages[-1][0], n)
    return dict(chunks=chunks, keys=keys, out=decode_attention(q_row, k, v, keys, scale))


# ----------------------------------------------------------------------------
# per-head pipelines (one query head; q [n, D], k/v its kv head [n, D])
# ----------------------------------------------------------------------------
def _attend_blocks(q, k, v, scale, block_keys, blocks=None) -> Dict[int, np.ndarray]:
    """Attention output of the listed query blocks (all by default)."""
    q = f64(q)
    k = f64(k)
    v = f64(v)
    n = q.shape[0]
    blocks = range(num_blocks(n)) if blocks is None else blocks
    out = {}
    for a in blocks:
        rows = np.arange(a * BLOCK, min(n, (a + 1) * BLOCK))
        out[a] = masked_attention(q[rows], rows, block_keys(a), k, v, scale)
    return out


def vs_head(q, k, v, vertical_topk: int, slash_topk: int, last_q: int = 64,
            scale: float | None = None, blocks=None, scores=None) -> dict:
    """Whole vertical-slash path for one head.

    ``scores`` (optional float32 (v, s)) replaces the oracle's own estimate, so
    the index steps and attention can be run on another implementation's
    scores. Returns the scores, V, S, merged intervals and the per-block
    outputs.
    """
    n, D = q.shape
    scale = default_scale(D) if scale is None else scale
    if scores is None:
        v64, s64 = vs_scores(q, k, last_q, scale)
        v32, s32 = to_f32(v64), to_f32(s64)
    else:
        v32, s32 = (np.asarray(x, np.float32) for x in scores)
    V, S = vs_select(v32, s32, vertical_topk, slash_topk)
    intervals = merge_offsets(S)
    out = _attend_blocks(q, k, v, scale,
                         lambda a: vs_block_keys(intervals, V, a, n), blocks)
    return dict(v=v32, s=s32, V=V, S=S, intervals=intervals, out=out)


def bs_head(q, k, v, topk: int, scale: float | None = None, blocks=None,
            logits=None) -> dict:
    """Whole block-sparse path for one head (``logits`` as in vs_head)."""
    n, D = q.shape
    scale = default_scale(D) if scale is None else scale
    qp, kp = mean_pool(q), mean_pool(k)
    L32 = to_f32(block_logits(qp, kp, scale)) if logits is None \
        else np.asarray(logits, np.float32)
    sel = block_select(L32, topk)
    out = _attend_blocks(q, k, v, scale, lambda a: blocks_to_keys(sel[a], n), blocks)
    return dict(qp=qp, kp=kp, logits=L32, sel=sel, out=out)


def hier_head(q, k, v, stages, scale: float | None = None, blocks=None, fine_max=None) -> dict:
    """Prefill head with the hierarchical pruning as its block estimator
    (R11): block a's query is its mean-pooled row, its keys those before its
    end; the last stage's chunk length must be 64 (key blocks). ``fine_max``
    (optional, float32 [nb][nb]) as in hier_prune, row a per query block."""
    n, D = q.shape
    assert stages[-1][0] == BLOCK
    scale = default_scale(D) if scale is None else scale
    qp = mean_pool(q)
    sel = [hier_prune(qp[a], k, min(n, (a + 1) * BLOCK), stages, scale,
                      None if fine_max is None else fine_max[a])
           for a in range(num_blocks(n))]
    out = _attend_blocks(q, k, v, scale, lambda a: blocks_to_keys(sel[a], n), blocks)
    return dict(qp=qp, sel=sel, out=out)


def streaming_head(q, k, v, init_blocks: int, local_blocks: int,
                   scale: float | None = None, blocks=None) -> dict:
    n, D = q.shape
    scale = default_scale(D) if scale is None else scale
    out = _attend_blocks(
        q, k, v, scale,
        lambda a: blocks_to_keys(streaming_blocks(a, init_blocks, local_blocks), n),
        blocks)
    return dict(out=out)


def assemble(out_blocks: Dict[int, np.ndarray], n: int, D: int) -> np.ndarray:
    """Per-block outputs into one [n, D] array (missing blocks stay NaN)."""
    o = np.full((n, D), np.nan)
    for a, ob in out_blocks.items():
        o[a * BLOCK: a * BLOCK + ob.shape[0]] = ob
    return o


# ----------------------------------------------------------------------------
# the three calls of the kernel-only API  [MInf usage listing]
# q [B, Hq, n, D], k/v [B, Hkv, n, D]; results float64 [B, Hq, n, D]
# ----------------------------------------------------------------------------
def _per_head(q, k, v, heads, fn):
    q, k, v = f64(q), f64(k), f64(v)
    B, Hq, n, D = q.shape
    Hkv = k.shape[1]
    o = np.zeros((B, Hq, n, D))
    for b in range(B):
        for h in (range(Hq) if heads is None else heads):
            g = kv_head_of(h, Hq, Hkv)
            res = fn(q[b, h], k[b, g], v[b, g])
            o[b, h] = assemble(res["out"], n, D)
    return o


def vertical_slash_sparse_attention(q, k, v, vertical_topk, slash_topk,
                                    last_q=64, scale=None, heads=None):
    return _per_head(q, k, v, heads, lambda qq, kk, vv: vs_head(
        qq, kk, vv, vertical_topk, slash_topk, last_q, scale))


def block_sparse_attention(q, k, v, topk, scale=None, heads=None):
    return _per_head(q, k, v, heads, lambda qq, kk, vv: bs_head(qq, kk, vv, topk, scale))


def streaming_attention(q, k, v, init_blocks, local_blocks, scale=None, heads=None):
    return _per_head(q, k, v, heads, lambda qq, kk, vv: streaming_head(
        qq, kk, vv, init_blocks, local_blocks, scale))
