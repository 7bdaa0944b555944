"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against brute force written independently in pure
Python (element-wise mask predicates, explicit loops with math.exp), closed
forms, a library special case (torch's scaled_dot_product_attention in float64)
or figures printed on the pages (tests/golden/). No GPU is involved.
"""
import json
import math
import os
import random

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BLK = 64


# ---------------------------------------------------------------------------
# independent brute force (pure Python)
# ---------------------------------------------------------------------------
def bf_attention(q, k, v, scale, allowed):
    """Row-by-row softmax attention; allowed(i, j) is the full element mask."""
    n, D = len(q), len(v[0])
    out = []
    for i in range(n):
        js = [j for j in range(n) if allowed(i, j)]
        if not js:
            out.append([0.0] * D)
            continue
        lg = [scale * sum(q[i][t] * k[j][t] for t in range(len(q[i]))) for j in js]
        m = max(lg)
        e = [math.exp(x - m) for x in lg]
        z = sum(e)
        out.append([sum(e[u] / z * v[js[u]][t] for u in range(len(js))) for t in range(D)])
    return np.array(out)


def bf_vs_scores(q, k, lq, scale):
    n = len(q)
    vs = [0.0] * n
    ss = [0.0] * n
    for i in range(n - min(lq, n), n):
        lg = [scale * sum(a * b for a, b in zip(q[i], k[j])) for j in range(i + 1)]
        m = max(lg)
        e = [math.exp(x - m) for x in lg]
        z = sum(e)
        for j in range(i + 1):
            vs[j] += e[j] / z
            ss[i - j] += e[j] / z
    return np.array(vs), np.array(ss)


def bf_topk(x, k, forced=()):
    def key(a):
        y = float(x[a])
        if math.isnan(y):
            return -math.inf
        return 0.0 if y == 0.0 else y

    n = len(x)
    forced = set(int(f) for f in forced)

    def before(b, a):  # does b rank strictly before a?
        fb, fa = b in forced, a in forced
        if fb != fa:
            return fb
        if key(b) != key(a):
            return key(b) > key(a)
        return b < a

    return [a for a in range(n) if sum(before(b, a) for b in range(n)) < k]


def vs_pred(V, S):
    Vs = set(int(j) for j in V)

    def allowed(i, j):
        if j > i:
            return False
        if j in Vs:
            return True
        r0 = (i // BLK) * BLK
        return any(r0 - d <= j < r0 + BLK - d for d in S)
    return allowed


def rnd(n, D, seed):
    r = np.random.default_rng(seed)
    return r.standard_normal((n, D)), r.standard_normal((n, D)), r.standard_normal((n, D))


# ---------------------------------------------------------------------------
# vertical-slash scores
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,lq", [(1, 64), (5, 3), (70, 64), (130, 64), (200, 17)])
def test_vs_scores_bruteforce(n, lq):
    q, k, _ = rnd(n, 6, n + lq)
    q *= 2.0  # peakier softmax: a reversed diagonal would show
    v, s = O.vs_scores(q, k, lq, 0.4)
    bv, bs = bf_vs_scores(q.tolist(), k.tolist(), lq, 0.4)
    np.testing.assert_allclose(v, bv, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(s, bs, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("n,lq", [(1, 64), (64, 64), (300, 64), (1000, 16)])
def test_vs_scores_identical_keys_closed_form(n, lq):
    """All keys equal: row i attends uniformly, p = 1/(i+1) on j <= i."""
    r = np.random.default_rng(0)
    q = r.standard_normal((n, 8))
    k = np.tile(r.standard_normal((1, 8)), (n, 1))
    v, s = O.vs_scores(q, k, lq, 0.3)
    lqe = min(lq, n)
    rows = range(n - lqe, n)
    ev = np.array([sum(1.0 / (i + 1) for i in rows if i >= j) for j in range(n)])
    es = np.array([sum(1.0 / (i + 1) for i in rows if i >= d) for d in range(n)])
    np.testing.assert_allclose(v, ev, rtol=1e-12)
    np.testing.assert_allclose(s, es, rtol=1e-12)


def test_vs_scores_mass():
    """Each window row is a probability distribution: sum v = sum s = lq."""
    q, k, _ = rnd(3000, 32, 7)
    v, s = O.vs_scores(q * 3, k, 64, 1 / math.sqrt(32))
    assert abs(v.sum() - 64) < 1e-9 and abs(s.sum() - 64) < 1e-9
    assert (v >= 0).all() and (s >= 0).all()


def test_window_worked_example():
    """Novita §2 q start/end restriction: prompt 5000, window 256 -> only
    5000*256 query-key products, not 5000*5000."""
    g = json.load(open(os.path.join(GOLDEN, "novita_window_example.json")))
    n, win = g["prompt_len"], g["window"]
    assert n * win == g["ops_window"] and n * n == g["ops_full"]
    q, k, _ = rnd(n, 4, 3)
    v, s = O.vs_scores(q, k, win, 0.5)
    q2 = q.copy()
    q2[: n - win] += 5.0          # rows before the window do not matter
    v2, s2 = O.vs_scores(q2, k, win, 0.5)
    assert np.array_equal(v, v2) and np.array_equal(s, s2)
    q3 = q.copy()
    q3[n - win] += 5.0            # the first window row does
    v3, _ = O.vs_scores(q3, k, win, 0.5)
    assert not np.array_equal(v, v3)
    k2 = k.copy()
    k2[0] += 5.0                  # and every key does
    v4, _ = O.vs_scores(q, k2, win, 0.5)
    assert not np.array_equal(v, v4)


# ---------------------------------------------------------------------------
# KV-retention scores (the vertical score over a window of any length)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,window", [(1, 5), (9, 3), (70, 70), (150, 100), (200, 400)])
def test_kv_retention_bruteforce(n, window):
    q, k, _ = rnd(n, 6, 3 * n + window)
    q *= 2.0
    S = O.kv_retention_scores(q, k, window, 0.4)
    bv, _ = bf_vs_scores(q.tolist(), k.tolist(), window, 0.4)
    np.testing.assert_allclose(S, bv, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("n,window", [(300, 256), (1000, 130), (50, 1000)])
def test_kv_retention_uniform_closed_form(n, window):
    """q = 0: every row attends uniformly, so S[j] = sum over window rows
    i >= j of 1/(i+1): a difference of harmonic numbers."""
    k = np.random.default_rng(1).standard_normal((n, 8))
    S = O.kv_retention_scores(np.zeros((n, 8)), k, window, 0.3)
    w = min(window, n)
    H = np.concatenate([[0.0], np.cumsum(1.0 / np.arange(1, n + 1))])
    want = np.array([H[n] - H[max(j, n - w)] for j in range(n)])
    np.testing.assert_allclose(S, want, rtol=1e-12)
    assert abs(S.sum() - w) < 1e-9


def test_kv_retention_last_row_is_softmax():
    """A window of one row is that row's causal softmax (scipy's)."""
    from scipy.special import softmax
    q, k, _ = rnd(500, 16, 11)
    S = O.kv_retention_scores(q, k, 1, 0.25)
    np.testing.assert_allclose(S, softmax(0.25 * (k @ q[-1])), rtol=1e-12)


def test_kv_retention_keeps_heaviest_keys():
    """Kept keys are the brute-force top-k of the float32 scores, and a key
    made to dominate the window's attention is kept."""
    q, k, _ = rnd(400, 16, 13)
    u = q[-64:].mean(axis=0)
    k[123] = 30.0 * u / (u @ u)   # mean window logit 30 * 0.25 = 7.5
    S32, kept = O.kv_retention(q, k, 64, 20, 0.25)
    assert S32.dtype == np.float32 and 123 in kept
    assert list(kept) == bf_topk(S32.tolist(), 20)


# ---------------------------------------------------------------------------
# sparse decode (one row after the whole cache)
# ---------------------------------------------------------------------------
def test_decode_bruteforce_and_sdpa():
    """A key subset matches the pure-Python brute force; the whole cache
    matches torch's scaled_dot_product_attention (float64, no mask)."""
    q, k, v = rnd(300, 16, 21)
    qd = 2.0 * q[0]
    keys = np.array([0, 3, 17, 100, 101, 250, 299])
    got = O.decode_attention(qd, k, v, keys, 0.3)
    Q = np.vstack([k, qd[None, :]])                       # row 300 sees keys 0..299
    bf = bf_attention(Q.tolist(), np.vstack([k, k[:1]]).tolist(), np.vstack([v, v[:1]]).tolist(), 0.3,
                      lambda i, j: i == 300 and j in set(keys.tolist()))
    np.testing.assert_allclose(got, bf[300], rtol=1e-12, atol=1e-14)
    full = O.decode_attention(qd, k, v, None, 0.25)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.tensor(qd)[None, None, None], torch.tensor(k)[None, None], torch.tensor(v)[None, None],
        scale=0.25)[0, 0, 0].numpy()
    np.testing.assert_allclose(full, ref, rtol=1e-12, atol=1e-14)


def test_decode_closed_forms():
    """One key gives its value row; q = 0 gives the mean of the listed
    value rows; no key gives zeros."""
    _, k, v = rnd(50, 8, 22)
    np.testing.assert_allclose(O.decode_attention(np.ones(8), k, v, [7], 0.5), v[7], rtol=1e-15)
    keys = [1, 4, 9, 30]
    np.testing.assert_allclose(O.decode_attention(np.zeros(8), k, v, keys, 0.5), v[keys].mean(0), rtol=1e-13)
    assert not O.decode_attention(np.ones(8), k, v, [], 0.5).any()


# ---------------------------------------------------------------------------
# top-k
# ---------------------------------------------------------------------------
def test_topk_bruteforce_random():
    rng = random.Random(5)
    pool = [0.0, -0.0, 1.0, -1.0, 2.5, float("nan"), float("inf"), -float("inf"), 1e-30]
    for trial in range(300):
        n = rng.randint(1, 24)
        x = np.array([rng.choice(pool) if rng.random() < 0.5 else rng.uniform(-3, 3)
                      for _ in range(n)], dtype=np.float32)
        k = rng.randint(0, n + 2)
        forced = rng.sample(range(n), rng.randint(0, min(2, n)))
        got = O.topk_indices(x, k, forced).tolist()
        assert got == bf_topk(x, k, forced), (x, k, forced)


def test_topk_ties_lowest_index():
    assert O.topk_indices(np.zeros(10, np.float32), 4).tolist() == [0, 1, 2, 3]
    x = np.array([1, 5, 5, 0, 5, 5], np.float32)
    assert O.topk_indices(x, 3).tolist() == [1, 2, 4]
    assert O.topk_indices(x, 3, forced=[3]).tolist() == [1, 2, 3]
    assert O.topk_indices(x, 100).tolist() == list(range(6))


# ---------------------------------------------------------------------------
# vertical-slash sparse format
# ---------------------------------------------------------------------------
def test_merge_offsets_cases():
    assert O.merge_offsets([300, 0, 64, 129]) == [(0, 64), (129, 129), (300, 300)]
    assert O.merge_offsets([0, 65]) == [(0, 0), (65, 65)]
    assert O.merge_offsets(list(range(0, 1000, 64))) == [(0, 960)]


@pytest.mark.parametrize("n", [1, 63, 64, 65, 200, 257, 390])
def test_vs_mask_bruteforce(n):
    rng = random.Random(n)
    for trial in range(6):
        V = rng.sample(range(n), rng.randint(0, min(n, 12)))
        S = sorted(set([0] + rng.sample(range(n), rng.randint(0, min(n, 10)))))
        iv = O.merge_offsets(S)
        pred = vs_pred(V, S)
        for a in range(O.num_blocks(n)):
            keys = set(O.vs_block_keys(iv, V, a, n).tolist())
            for i in range(a * BLK, min(n, (a + 1) * BLK)):
                got = {j for j in keys if j <= i}
                want = {j for j in range(n) if pred(i, j)}
                assert got == want, (n, a, i, V, S)
        # canonical form: ranges disjoint and non-adjacent; the column list is
        # exactly the verticals the block's last row may see that no offset
        # rectangle covers, ascending
        for a in range(O.num_blocks(n)):
            rg = sorted(O.vs_block_ranges(iv, a, n))
            for (l0, h0), (l1, h1) in zip(rg, rg[1:]):
                assert h0 < l1
            cols = O.vs_block_cols(V, rg, a, n)
            last = min(n, (a + 1) * BLK) - 1
            r0 = a * BLK
            want = sorted(j for j in set(V) if j <= last and
                          not any(r0 - d <= j < r0 + BLK - d for d in S))
            assert cols.tolist() == want


def test_vs_all_offsets_is_one_range():
    n = 300
    iv = O.merge_offsets(range(n))
    assert iv == [(0, n - 1)]
    for a in range(O.num_blocks(n)):
        assert O.vs_block_ranges(iv, a, n) == [(0, min(n, a * BLK + BLK))]


def test_vs_planted_col_inside_range_removed():
    n = 512
    iv = O.merge_offsets([0])
    # block 3 covers keys [192, 256) through offset 0; verticals 10 and 200
    rg = O.vs_block_ranges(iv, 3, n)
    assert rg == [(192, 256)]
    assert O.vs_block_cols([10, 200, 300], rg, 3, n).tolist() == [10]


# ---------------------------------------------------------------------------
# block-sparse estimate
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n", [64, 100, 257])
def test_pool_closed_form(n):
    x = np.tile(np.arange(n, dtype=np.float64)[:, None], (1, 4))
    p = O.mean_pool(x)
    for a in range(O.num_blocks(n)):
        last = min(n, (a + 1) * BLK) - 1
        assert np.allclose(p[a], (a * BLK + last) / 2.0)


@pytest.mark.parametrize("n,topk", [(64 * 7 + 5, 3), (64 * 5, 1), (64 * 4, 9)])
def test_block_select_bruteforce(n, topk):
    q, k, _ = rnd(n, 8, n)
    L = O.to_f32(O.block_logits(O.mean_pool(q), O.mean_pool(k), 0.7))
    sel = O.block_select(L, topk)
    nb = O.num_blocks(n)
    ql, kl = q.tolist(), k.tolist()
    for a in range(nb):
        qa = [sum(ql[i][t] for i in range(a * BLK, min(n, a * BLK + BLK))) /
              (min(n, a * BLK + BLK) - a * BLK) for t in range(8)]
        row = []
        for c in range(a + 1):
            kc = [sum(kl[i][t] for i in range(c * BLK, min(n, c * BLK + BLK))) /
                  (min(n, c * BLK + BLK) - c * BLK) for t in range(8)]
            row.append(np.float32(0.7 * sum(x * y for x, y in zip(qa, kc))))
        assert abs(float(L[a, a]) - float(row[a])) <= 1e-6 * (1 + abs(float(row[a])))
        assert sel[a].tolist() == bf_topk(np.array(row, np.float32), topk, [a])
        assert a in sel[a].tolist()


def test_block_select_finds_planted_clusters():
    w = synthetic.BY_NAME["bs_mha4_32k_bf16"].scaled(seq_len=4096)
    x = synthetic.make_inputs(w)
    for h in range(w.q_heads):
        res = O.bs_head(x.q[0, h], x.k[0, h], x.v[0, h], topk=8, blocks=[])
        for kb, qbs in x.planted[(0, h)]:
            for qa in qbs:
                assert kb in res["sel"][qa].tolist(), (h, kb, qa)


# ---------------------------------------------------------------------------
# streaming mask
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("init,local", [(0, 1), (1, 1), (1, 3), (2, 2), (5, 1)])
def test_streaming_bruteforce(init, local):
    n = 64 * 6 + 11
    for a in range(O.num_blocks(n)):
        keys = set(O.blocks_to_keys(O.streaming_blocks(a, init, local), n).tolist())
        for i in range(a * BLK, min(n, a * BLK + BLK)):
            want = {j for j in range(n)
                    if j <= i and (j // BLK < init or i // BLK - j // BLK < local)}
            assert {j for j in keys if j <= i} == want


# ---------------------------------------------------------------------------
# attention under the mask
# ---------------------------------------------------------------------------
def test_attention_bruteforce_all_patterns():
    n, D = 64 * 3 + 9, 4
    q, k, v = rnd(n, D, 11)
    q *= 2
    sc = 0.5
    ql, kl, vl = q.tolist(), k.tolist(), v.tolist()
    # vertical-slash with fixed indices
    V, S = [3, 70, 150], [0, 40, 130]
    iv = O.merge_offsets(S)
    out = O._attend_blocks(q, k, v, sc, lambda a: O.vs_block_keys(iv, V, a, n))
    want = bf_attention(ql, kl, vl, sc, vs_pred(V, S))
    np.testing.assert_allclose(O.assemble(out, n, D), want, rtol=1e-10, atol=1e-12)
    # block-sparse with the oracle's own selection
    res = O.bs_head(q, k, v, topk=2, scale=sc)
    sel = res["sel"]
    want = bf_attention(ql, kl, vl, sc,
                        lambda i, j: j <= i and (j // BLK) in sel[i // BLK].tolist())
    np.testing.assert_allclose(O.assemble(res["out"], n, D), want, rtol=1e-10, atol=1e-12)
    # streaming
    res = O.streaming_head(q, k, v, 1, 2, scale=sc)
    want = bf_attention(ql, kl, vl, sc,
                        lambda i, j: j <= i and (j // BLK < 1 or i // BLK - j // BLK < 2))
    np.testing.assert_allclose(O.assemble(res["out"], n, D), want, rtol=1e-10, atol=1e-12)


def _sdpa(q, k, v):
    Hq, Hkv = q.shape[1], k.shape[1]
    kk = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=1)
    vv = torch.from_numpy(v).repeat_interleave(Hq // Hkv, dim=1)
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), kk, vv, is_causal=True).numpy()


@pytest.mark.parametrize("n", [100, 64 * 4])
def test_full_selection_equals_dense_causal(n):
    """Full selection in any pattern is dense causal attention (library case,
    with the GQA map of consecutive query heads per kv head)."""
    r = np.random.default_rng(n)
    B, Hq, Hkv, D = 2, 4, 2, 16
    q = r.standard_normal((B, Hq, n, D)) * 2
    k = r.standard_normal((B, Hkv, n, D))
    v = r.standard_normal((B, Hkv, n, D))
    ref = _sdpa(q, k, v)
    nb = O.num_blocks(n)
    for o in (O.vertical_slash_sparse_attention(q, k, v, n, 1),
              O.vertical_slash_sparse_attention(q, k, v, 0, n),
              O.block_sparse_attention(q, k, v, nb),
              O.streaming_attention(q, k, v, 1, nb - 1),
              O.streaming_attention(q, k, v, nb, 1)):
        np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-12)


def test_attention_large_logits_stay_finite():
    """Logits in the thousands: the softmax must not overflow; in the limit each
    row returns the value of its best allowed key."""
    n, D = 130, 8
    r = np.random.default_rng(4)
    q, k, v = r.standard_normal((n, D)) * 300, r.standard_normal((n, D)), r.standard_normal((n, D))
    res = O.streaming_head(q, k, v, 1, 1, scale=1.0)
    o = O.assemble(res["out"], n, D)
    assert np.isfinite(o).all()
    for i in (5, 70, 129):
        js = [j for j in range(n) if j <= i and (j // BLK < 1 or i // BLK == j // BLK)]
        best = max(js, key=lambda j: float(q[i] @ k[j]))
        assert np.allclose(o[i], v[best], atol=1e-6)
    vv, ss = O.vs_scores(q, k, 64, 1.0)
    assert np.isfinite(vv).all() and abs(vv.sum() - 64) < 1e-9


def test_attention_closed_forms():
    n, D = 150, 8
    r = np.random.default_rng(1)
    q, k, v = r.standard_normal((n, D)), r.standard_normal((n, D)), r.standard_normal((n, D))
    V, S = [5, 90], [0, 70]
    iv = O.merge_offsets(S)
    keys = lambda a: O.vs_block_keys(iv, V, a, n)  # noqa: E731
    o = O.assemble(O._attend_blocks(q, k, v, 0.3, keys), n, D)
    assert np.allclose(o[0], v[0])                       # row 0 sees only key 0
    o0 = O.assemble(O._attend_blocks(np.zeros_like(q), k, v, 0.3, keys), n, D)
    pred = vs_pred(V, S)
    for i in (0, 64, 100, 149):                          # Q = 0: plain mean
        js = [j for j in range(n) if pred(i, j)]
        assert np.allclose(o0[i], v[js].mean(axis=0))
    oc = O.assemble(O._attend_blocks(q, k, np.ones_like(v) * 3.5, 0.3, keys), n, D)
    assert np.allclose(oc, 3.5)                          # constant V
    # one-hot V recovers the probabilities: support = mask, rows sum to 1
    n2 = 96
    q2, k2 = r.standard_normal((n2, n2)), r.standard_normal((n2, n2))
    iv2 = O.merge_offsets([0, 80])
    P = O.assemble(O._attend_blocks(q2, k2, np.eye(n2), 0.1,
                                    lambda a: O.vs_block_keys(iv2, [7], a, n2)), n2, n2)
    pred2 = vs_pred([7], [0, 80])
    for i in range(n2):
        assert abs(P[i].sum() - 1) < 1e-12
        assert set(np.nonzero(P[i])[0].tolist()) == {j for j in range(n2) if pred2(i, j)}


def test_vs_structure_selects_sink():
    w = synthetic.BY_NAME["vs_head_4k_f32"].scaled(seq_len=2048)
    x = synthetic.make_inputs(w)
    res = O.vs_head(x.q[0, 0], x.k[0, 0], x.v[0, 0], 64, 64, blocks=[])
    assert 0 in res["V"].tolist() and 0 in res["S"].tolist()
    assert abs(float(res["v"].astype(np.float64).sum()) - 64) < 1e-3


# ---------------------------------------------------------------------------
# hierarchical chunk pruning (R11)
# ---------------------------------------------------------------------------
def bf_hier(q, k, limit, stages, scale):
    """The stages written out with explicit loops: token scores, chunk maxima
    by scanning tokens, ranks by pairwise comparison (bf_topk)."""
    s = [scale * sum(a * b for a, b in zip(q, k[j])) for j in range(limit)]
    kept, prev = None, None
    for c, keep in stages:
        if kept is None:
            cand = [x for x in range(limit) if x * c < limit]
        else:
            cand = []
            for x in kept:
                for y in range(x * (prev // c), (x + 1) * (prev // c)):
                    if y * c < limit:
                        cand.append(y)
        scores = []
        for x in cand:
            best = -math.inf
            for j in range(x * c, min(limit, (x + 1) * c)):
                best = max(best, s[j])
            scores.append(best)
        forced = [i for i, x in enumerate(cand) if x * c <= limit - 1 < (x + 1) * c]
        kept = [cand[i] for i in bf_topk(scores, keep, forced)]
        prev = c
    return sorted(kept)


def test_hier_worked_examples():
    """Hand-worked: 512 keys, scores are the keys' only entry (q = 1). Token 10
    scores 5, token 300 scores 3, all others 0; key 511 lies in the forced
    chunks. Keeping one 256-chunk keeps only the forced one (tokens 256..511),
    whose best 64-chunk besides the forced one (7) is chunk 4 (token 300).
    Keeping two 256-chunks lets chunk 0 (token 10) win the second slot."""
    k = np.zeros((512, 1))
    k[10, 0], k[300, 0] = 5.0, 3.0
    q = np.ones(1)
    assert O.hier_prune(q, k, 512, [(256, 1), (64, 2)], 1.0).tolist() == [4, 7]
    assert O.hier_prune(q, k, 512, [(256, 2), (64, 2)], 1.0).tolist() == [0, 7]
    # a visible limit cuts the candidates: keys below 300 only, key 299 forced
    assert O.hier_prune(q, k, 300, [(256, 1), (64, 1)], 1.0).tolist() == [4]
    assert O.hier_prune(q, k, 300, [(128, 2), (64, 2)], 1.0).tolist() == [0, 4]
    # the chunk score is the chunk's largest token, not its mean: one token of
    # 2.0 beats sixty-four tokens of 1.5
    k2 = np.zeros((256, 1))
    k2[0:64, 0] = 1.5
    k2[100, 0] = 2.0
    assert O.hier_prune(q, k2, 256, [(64, 2)], 1.0).tolist() == [1, 3]


@pytest.mark.parametrize("limit,stages", [(300, [(64, 3)]), (1000, [(256, 2), (64, 3)]),
                                          (1000, [(512, 1), (128, 3), (64, 2)]), (64, [(128, 1), (64, 1)]),
                                          (777, [(256, 9), (64, 50)]), (450, [(192, 2), (64, 4)])])
def test_hier_bruteforce(limit, stages):
    r = np.random.default_rng(limit)
    D = 4
    k = r.standard_normal((limit + 37, D))
    q = r.standard_normal(D)
    k[r.integers(0, limit, 5)] *= 3.0      # a few dominant tokens
    assert O.hier_prune(q, k, limit, stages, 0.5).tolist() == bf_hier(q, k, limit, stages, 0.5)


@pytest.mark.parametrize("seed", range(8))
def test_hier_equals_flat_selection_when_outer_keeps_enough(seed):
    """Closed form: with exact chunk maxima, two stages whose first keeps at
    least as many chunks as the second select exactly the flat top-k of the
    fine chunks (every chunk ranked above a selected fine chunk's parent holds
    a fine chunk ranked above it). A mean instead of the max, or a dropped
    forced chunk, breaks this."""
    r = np.random.default_rng(seed)
    limit = int(r.integers(200, 3000))
    k = r.standard_normal((limit, 8))
    q = r.standard_normal(8)
    c1 = int(r.choice([128, 256, 512]))
    k2 = int(r.integers(1, 12))
    k1 = k2 + int(r.integers(0, 4))
    hier = O.hier_prune(q, k, limit, [(c1, k1), (64, k2)], 0.3)
    flat = O.hier_prune(q, k, limit, [(64, k2)], 0.3)
    assert hier.tolist() == flat.tolist()
    # and the flat selection is the top-k of the 64-key maxima (R3)
    s = 0.3 * (k @ q)
    m = np.array([s[x * 64: min(limit, x * 64 + 64)].max() for x in range((limit + 63) // 64)])
    assert flat.tolist() == O.topk_indices(m, k2, forced=((limit - 1) // 64,)).tolist()


def test_hier_properties():
    """Keep-all keeps every visible chunk; the forced chunk survives even when
    it scores lowest; each kept chunk lies inside a chunk every earlier stage
    kept; a planted dominant token's chunks survive every stage."""
    r = np.random.default_rng(3)
    n = 4096
    k = r.standard_normal((n, 16))
    q = r.standard_normal(16)
    assert O.hier_prune(q, k, n, [(1024, 4), (64, 64)], 1.0).tolist() == list(range(64))
    k_low = k.copy()
    k_low[n - 64:] = -10 * q / np.linalg.norm(q)      # the forced chunk scores lowest
    res = O.hier_prune(q, k_low, n, [(1024, 1), (256, 1), (64, 1)], 1.0)
    assert res.tolist() == [63]
    k_pl = k.copy()
    k_pl[1234] = 20 * q / np.linalg.norm(q)
    st = [(1024, 2), (256, 2), (64, 2)]
    res = O.hier_prune(q, k_pl, n, st, 1.0)
    assert 1234 // 64 in res.tolist() and 63 in res.tolist()
    for c, keep in [(1024, 2), (256, 2)]:
        outer = set(O.hier_prune(q, k_pl, n, st[: [s[0] for s in st].index(c) + 1], 1.0).tolist())
        assert all(x * 64 // c in outer for x in res.tolist())


def test_hier_fine_max_route_agrees():
    """The selection run on 64-key block maxima (rounded to float32) equals
    the one on float64 token scores when no two candidates are within float32
    rounding of each other (random Gaussian data)."""
    r = np.random.default_rng(11)
    n = 3000
    k = r.standard_normal((n, 8))
    q = r.standard_normal(8)
    s = 0.25 * (k @ q)
    fm = np.array([s[x * 64: min(n, x * 64 + 64)].max() for x in range((n + 63) // 64)], np.float32)
    st = [(512, 3), (128, 4), (64, 5)]
    assert O.hier_prune(q, k, n, st, 0.25).tolist() == O.hier_prune(q, k, n, st, 0.25, fine_max=fm).tolist()


def test_hier_decode_and_head():
    """Decode over the kept keys is R10's decode over exactly those keys, and
    the prefill head attends each block over its kept key blocks (brute-force
    attention with the element mask)."""
    q, k, v = rnd(300, 8, 4)
    res = O.hier_decode(q[5], k, v, [(128, 2), (64, 2)], 0.4)
    keys = O.chunks_to_keys(res["chunks"], 64, 300)
    assert set(keys.tolist()) == {j for x in res["chunks"].tolist() for j in range(x * 64, min(300, x * 64 + 64))}
    np.testing.assert_allclose(res["out"], O.decode_attention(q[5], k, v, keys, 0.4), rtol=0, atol=1e-12)
    st = [(128, 1), (64, 2)]
    h = O.hier_head(q, k, v, st, 0.4)
    qp = O.mean_pool(q)
    for a, sel in enumerate(h["sel"]):
        assert sel.tolist() == bf_hier(qp[a], k, min(300, 64 * (a + 1)), st, 0.4)
    sets = {a: set(h["sel"][a].tolist()) for a in range(len(h["sel"]))}
    bf = bf_attention(q.tolist(), k.tolist(), v.tolist(), 0.4,
                      lambda i, j: j <= i and (j // 64) in sets[i // 64])
    np.testing.assert_allclose(O.assemble(h["out"], 300, 8), bf, rtol=1e-10, atol=1e-12)
