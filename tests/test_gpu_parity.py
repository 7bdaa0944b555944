"""GPU path against the CPU oracle, stage by stage and end to end.

Every call goes through the C ABI (ctypes binding). Inputs are seeded; the
oracle sees exactly the GPU's input values (bf16/fp32 -> float64). Bars:
index construction bit-exact given the GPU's own fp32 scores; estimator scores
within 1e-3 relative; attention within max-abs 2e-2 and mean-abs 2e-3 against
the unrounded float64 oracle.
"""
import math
import sys

import numpy as np
import pytest
import torch

import dynamic_sparse_attention_slash_amd as dsa
import synthetic
from oracle import dsa_oracle as O
from tests.gpu_util import (BLK, check_attention, check_scores, gpu_cols, host64,
                            oracle_vs_index)

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rand_qkv(B, Hq, Hkv, n, D, dt, seed, amp=1.0):
    g = torch.Generator().manual_seed(seed)
    q = (torch.randn(B, Hq, n, D, generator=g) * amp).to(DT[dt])
    k = torch.randn(B, Hkv, n, D, generator=g).to(DT[dt])
    v = torch.randn(B, Hkv, n, D, generator=g).to(DT[dt])
    return q.cuda(), k.cuda(), v.cuda()


def kvh(h, Hq, Hkv):
    return h // (Hq // Hkv)


# ---------------------------------------------------------------------------
# estimator scores
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,D,dt,lq", [(1000, 128, "bf16", 64), (64 * 3 + 17, 64, "f32", 64),
                                       (333, 128, "bf16", 16), (40, 128, "bf16", 64),
                                       (1, 64, "f32", 64), (2049, 64, "bf16", 64)])
def test_vs_estimate(n, D, dt, lq):
    say(f"vs_estimate n={n} D={D} {dt} lq={lq}")
    q, k, _ = rand_qkv(2, 4, 2, n, D, dt, seed=n + D, amp=2.0)
    heads = [3, 0]
    vg, sg = dsa.vs_estimate(q, k, last_q=lq, heads=heads)
    torch.cuda.synchronize()
    qh, kh = host64(q), host64(k)
    sc = 1.0 / math.sqrt(D)
    for b in range(2):
        for t, h in enumerate(heads):
            v, s = O.vs_scores(qh[b, h], kh[b, kvh(h, 4, 2)], lq, sc)
            row = b * len(heads) + t
            check_scores(vg[row].cpu().numpy(), v, f"v row {row}")
            check_scores(sg[row].cpu().numpy(), s, f"s row {row}")


@pytest.mark.parametrize("n,dt", [(3000, "bf16"), (20000, "bf16"), (70000, "bf16"), (777, "f32")])
def test_vs_estimate_same_bits_for_any_head_list(n, dt):
    """A head's scores do not depend on the batch or head list of the call:
    the key chunking (and so the fp32 summation order) depends on seq_len only."""
    say(f"vs_estimate head-list independence n={n} {dt}")
    q, k, _ = rand_qkv(2, 8, 2, n, 64, dt, seed=n, amp=2.0)
    v_all, s_all = dsa.vs_estimate(q, k)
    v_one, s_one = dsa.vs_estimate(q[1:2], k[1:2], heads=[5])
    torch.cuda.synchronize()
    assert torch.equal(v_one[0], v_all[8 + 5]) and torch.equal(s_one[0], s_all[8 + 5])


def test_empty_calls_through_the_binding():
    """batch 0 or seq_len 0 (zero-size tensors, whose data pointers are NULL)
    return without work through every wrapper."""
    say("empty calls")
    for B, n in ((0, 256), (1, 0)):
        q, k, v = rand_qkv(B, 4, 2, n, 64, "bf16", seed=1)
        o = dsa.vertical_slash_sparse_attention(q, k, v, 8, 8)
        o = dsa.block_sparse_attention(q, k, v, 4, out=o)
        o = dsa.streaming_attention(q, k, v, 1, 2, out=o)
        o = dsa.mixed_sparse_attention(q, k, v, ["vs", "bs", "st", None], vertical_topk=8, slash_topk=8,
                                       topk=4, init_blocks=1, local_blocks=2, out=o)
        assert o.shape == q.shape
        vg, sg = dsa.vs_estimate(q, k)
        sc, kept = dsa.kv_retention(q, k, 64, 8)
        assert vg.numel() == sg.numel() == sc.numel() == kept.numel() == 0
        assert dsa.bs_pool(q).numel() == 0
        rows, nb = B * 4, (n + 63) // 64
        i32 = dict(dtype=torch.int32, device="cuda")
        dsa.sparse_attention_vs(q, k, v, torch.zeros(rows, 1, 2, **i32), torch.zeros(rows, **i32),
                                torch.zeros(rows, nb, 1, **i32), torch.zeros(rows, nb, **i32), out=o)
        dsa.sparse_attention_blocks(q, k, v, torch.zeros(rows, nb, 1, **i32), torch.zeros(rows, nb, **i32), out=o)
    qd = torch.zeros(0, 4, 64, dtype=torch.bfloat16, device="cuda")
    kd = torch.zeros(0, 2, 100, 64, dtype=torch.bfloat16, device="cuda")
    assert dsa.sparse_decode(qd, kd, kd).numel() == 0
    assert dsa.hier_sparse_decode(qd, kd, kd, [(128, 1), (64, 1)]).numel() == 0
    # an empty cache: every decode row comes out as zeros
    q1 = torch.randn(2, 4, 64, device="cuda").to(torch.bfloat16)
    k0 = torch.zeros(2, 2, 0, 64, dtype=torch.bfloat16, device="cuda")
    for out in (dsa.sparse_decode(q1, k0, k0, out=torch.full_like(q1, 3.0)),
                dsa.hier_sparse_decode(q1, k0, k0, [(128, 1), (64, 1)], out=torch.full_like(q1, 3.0))):
        torch.cuda.synchronize()
        assert not out.float().any()
    torch.cuda.synchronize()


def test_vs_estimate_planted_structure_and_mass():
    w = synthetic.BY_NAME["llama3_8b_128k_vs_bf16"].scaled(seq_len=8192, q_heads=4, kv_heads=1,
                                                            slash_topk=512)
    x = synthetic.make_inputs(w)
    q, k = x.q.cuda(), x.k.cuda()
    vg, sg = dsa.vs_estimate(q, k)
    torch.cuda.synchronize()
    assert torch.allclose(vg.double().sum(1), torch.full((4,), 64.0, dtype=torch.float64, device="cuda"), rtol=1e-4)
    assert torch.allclose(sg.double().sum(1), torch.full((4,), 64.0, dtype=torch.float64, device="cuda"), rtol=1e-4)
    qh, kh = host64(x.q), host64(x.k)
    v, s = O.vs_scores(qh[0, 2], kh[0, 0], 64, 1 / math.sqrt(128))
    check_scores(vg[2].cpu().numpy(), v, "planted v")
    check_scores(sg[2].cpu().numpy(), s, "planted s")


# ---------------------------------------------------------------------------
# top-k
# ---------------------------------------------------------------------------
def _special_scores(rows, n, seed):
    r = np.random.default_rng(seed)
    x = r.standard_normal((rows, n)).astype(np.float32)
    x[:, ::7] = np.round(x[:, ::7])            # many exact ties
    x[0, : n // 2] = 0.0                       # a run of zeros
    if n > 10:
        x[1 % rows, 3] = -0.0
        x[1 % rows, 5] = np.nan
        x[1 % rows, 7] = np.inf
        x[1 % rows, 9] = -np.inf
    return x


@pytest.mark.parametrize("n,k,forced", [(100, 7, -1), (100, 7, 0), (100, 100, -1), (100, 150, 0),
                                        (1, 1, 0), (5000, 256, 0), (5000, 1, -1), (131072, 6096, 0),
                                        (131072, 1000, -1), (4097, 4096, 4096),
                                        # one work-group per row: many kept entries written from
                                        # the bitmap (up to its 65535-entry rows), and k above its
                                        # 8192 kept entries (radix select)
                                        (65535, 8192, 65534), (30000, 3000, 0), (50000, 9000, -1),
                                        # rows of 64K entries or more take the row-parallel path
                                        (200001, 1000, 200000), (300000, 6096, 0), (70000, 16384, 5),
                                        (1 << 20, 6096, 123457), (1 << 20, 1000, -1),
                                        # k above 16384: one work-group per row, or chunks + merge
                                        (70000, 20000, 7), (300000, 17000, -1)])
def test_topk(n, k, forced):
    say(f"topk n={n} k={k} forced={forced}")
    x = _special_scores(3, n, n + k)
    out = dsa.topk(torch.from_numpy(x).cuda(), k, forced).cpu().numpy()
    for r in range(3):
        want = O.topk_indices(x[r], k, [forced] if forced >= 0 else [])
        assert np.array_equal(out[r], want), (r, out[r][:10], want[:10])


@pytest.mark.parametrize("n,k,forced", [(100000, 8000, -1), (100000, 16384, 99999), (65536, 7000, 3)])
def test_topk_ties_across_chunks(n, k, forced):
    # the k-th largest key is an exact tie shared by entries in many 16K-entry
    # chunks: the tied entries kept are the first ones in index order, across
    # chunk boundaries (rows of 64K entries or more are selected row-parallel)
    say(f"topk ties across chunks n={n} k={k} forced={forced}")
    r = np.random.default_rng(n + k)
    x = -np.abs(r.standard_normal((2, n))).astype(np.float32) - 1.0
    x[:, ::10] = 0.0
    pos = r.choice(n, size=(3000,), replace=False)
    x[0, pos] = np.abs(r.standard_normal(3000)).astype(np.float32) + 0.5
    x[1, pos[:200]] = 1.0                      # ties above the boundary too
    out = dsa.topk(torch.from_numpy(x).cuda(), k, forced).cpu().numpy()
    for row in range(2):
        want = O.topk_indices(x[row], k, [forced] if forced >= 0 else [])
        assert np.array_equal(out[row], want), (row, out[row][:10], want[:10])


@pytest.mark.parametrize("n", [70000, 300000])
def test_topk_all_ties(n):
    x = torch.zeros(2, n, device="cuda")
    out = dsa.topk(x, 300, 0).cpu().numpy()
    assert (out[0] == np.arange(300)).all() and (out[1] == np.arange(300)).all()
    out = dsa.topk(x, 300, n - 1).cpu().numpy()
    want = np.concatenate([np.arange(299), [n - 1]])
    assert (out[0] == want).all() and (out[1] == want).all()


# ---------------------------------------------------------------------------
# vertical-slash index builder
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,nv,ns,with0", [(1, 1, 1, True), (65, 5, 9, True), (1000, 30, 40, True),
                                           (1000, 30, 40, False), (4096 + 13, 200, 300, True),
                                           (20000, 1000, 600, True)])
def test_vs_build_index(n, nv, ns, with0):
    say(f"vs_build_index n={n} nv={nv} ns={ns}")
    rng = np.random.default_rng(n + nv)
    rows = 3
    Vs, Ss = [], []
    for r in range(rows):
        V = np.sort(rng.choice(n, size=min(nv, n), replace=False))
        pool = np.arange(1, n) if with0 else np.arange(n)
        S = rng.choice(pool, size=min(ns, len(pool)) - (1 if with0 else 0), replace=False) if len(pool) else np.zeros(0, int)
        if with0:
            S = np.concatenate([[0], S])
        if r == 1 and len(S) > 8:   # a dense run of nearby offsets, same count
            run = np.arange(0, min(n, 200), 3)
            rest = np.setdiff1d(np.arange(n), run)
            extra = rng.choice(rest, size=max(0, len(S) - len(run)), replace=False)
            S = np.concatenate([run, extra])[: len(S)]
        Ss.append(np.sort(S).astype(np.int32))
        Vs.append(V.astype(np.int32))
    nvv, nss = len(Vs[0]), len(Ss[0])
    assert all(len(x) == nvv for x in Vs) and all(len(x) == nss for x in Ss)
    Vt = torch.from_numpy(np.stack(Vs)).cuda()
    St = torch.from_numpy(np.stack(Ss)).cuda()
    iv, n_iv, cols, n_cols = dsa.vs_build_index(Vt, St, n)
    torch.cuda.synchronize()
    iv, n_iv = iv.cpu().numpy(), n_iv.cpu().numpy()
    for r in range(rows):
        want = O.merge_offsets(Ss[r])
        assert n_iv[r] == len(want)
        assert [tuple(x) for x in iv[r, : n_iv[r]].tolist()] == want
        for a in range(O.num_blocks(n)):
            c = O.vs_block_cols(Vs[r], O.vs_block_ranges(want, a, n), a, n)
            assert np.array_equal(gpu_cols(cols, n_cols, r, a), c), (r, a)


# ---------------------------------------------------------------------------
# attention from given indices
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,D,dt,with0", [(1000, 128, "bf16", True), (64 * 5 + 3, 64, "f32", True),
                                          (777, 128, "bf16", False), (300, 64, "bf16", True),
                                          (64 * 4, 128, "f32", False), (64 * 5 + 29, 128, "f32", True)])
def test_attention_vs_given_indices(n, D, dt, with0):
    say(f"attention_vs n={n} D={D} {dt}")
    B, Hq, Hkv = 1, 4, 2
    q, k, v = rand_qkv(B, Hq, Hkv, n, D, dt, seed=7 * n, amp=1.5)
    heads = [1, 2, 3]
    rng = np.random.default_rng(n)
    nv, ns = min(40, n), min(30, n)
    rows = B * len(heads)
    ivs, nivs, colss, ncolss, Vs, Ss = [], [], [], [], [], []
    for r in range(rows):
        V = np.sort(rng.choice(n, nv, replace=False))
        S = np.sort(rng.choice(np.arange(1, n), ns - 1, replace=False)) if n > 1 else np.zeros(0, int)
        S = np.concatenate([[0], S]) if with0 else np.sort(rng.choice(n, ns, replace=False))
        iv, ivarr, cols, ncols = oracle_vs_index(V, S, n)
        ivs.append(ivarr); nivs.append(len(iv)); colss.append(cols); ncolss.append(ncols)
        Vs.append(V); Ss.append(S)
    o = dsa.sparse_attention_vs(q, k, v, torch.from_numpy(np.stack(ivs)).cuda(),
                                torch.tensor(nivs, dtype=torch.int32).cuda(),
                                torch.from_numpy(np.stack(colss)).cuda(),
                                torch.from_numpy(np.stack(ncolss)).cuda(), heads=heads)
    torch.cuda.synchronize()
    qh, kh, vh, oh = host64(q), host64(k), host64(v), host64(o)
    sc = 1 / math.sqrt(D)
    for t, h in enumerate(heads):
        g = kvh(h, Hq, Hkv)
        ivl = O.merge_offsets(Ss[t])
        ref = O._attend_blocks(qh[0, h], kh[0, g], vh[0, g], sc,
                               lambda a: O.vs_block_keys(ivl, Vs[t], a, n))
        check_attention(oh[0, h], O.assemble(ref, n, D), f"head {h}")
    # heads not listed are untouched (zeros)
    assert float(np.abs(oh[0, 0]).max()) == 0.0


@pytest.mark.parametrize("n,D,dt", [(1000, 128, "bf16"), (64 * 6 + 1, 64, "f32"), (64 * 6 + 40, 128, "f32")])
def test_attention_blocks_given_indices(n, D, dt):
    say(f"attention_blocks n={n} D={D} {dt}")
    q, k, v = rand_qkv(2, 2, 1, n, D, dt, seed=3 * n)
    nb = O.num_blocks(n)
    rng = np.random.default_rng(n)
    kmax = 5
    sel = np.zeros((4, nb, kmax), np.int32)
    nsel = np.zeros((4, nb), np.int32)
    sets = {}
    for r in range(4):
        for a in range(nb):
            cand = rng.choice(nb, size=min(kmax, nb), replace=False)   # may hold c > a
            cs = np.unique(np.concatenate([[a], cand]))[:kmax]
            sel[r, a, : len(cs)] = cs
            nsel[r, a] = len(cs)
            sets[(r, a)] = cs
    o = dsa.sparse_attention_blocks(q, k, v, torch.from_numpy(sel).cuda(), torch.from_numpy(nsel).cuda())
    torch.cuda.synchronize()
    qh, kh, vh, oh = host64(q), host64(k), host64(v), host64(o)
    for b in range(2):
        for h in range(2):
            r = b * 2 + h
            ref = O._attend_blocks(qh[b, h], kh[b, 0], vh[b, 0], 1 / math.sqrt(D),
                                   lambda a: O.blocks_to_keys(sets[(r, a)], n))
            check_attention(oh[b, h], O.assemble(ref, n, D), f"b{b} h{h}")


@pytest.mark.parametrize("D", [64, 128])
def test_attention_blocks_f32_long_rows(D):
    """fp32 query blocks with more than 1024 key sub-blocks: every key block up
    to the diagonal is listed, so the last query blocks of a 19211-token head
    hold up to 1201 sub-blocks, more than one refill of the descriptor array
    that the work-group's four waves share (at D = 128 two waves per query
    half split the keys). Sampled query blocks (both sides of the
    1024-sub-block line, the ragged last one) against the oracle; every output
    row finite."""
    n = 64 * 300 + 11
    say(f"attention_blocks f32 long rows n={n} D={D}")
    q, k, v = rand_qkv(1, 1, 1, n, D, "f32", seed=77)
    nb = O.num_blocks(n)
    sel = np.zeros((1, nb, nb), np.int32)
    nsel = np.zeros((1, nb), np.int32)
    for a in range(nb):
        sel[0, a, : a + 1] = np.arange(a + 1)
        nsel[0, a] = a + 1
    o = dsa.sparse_attention_blocks(q, k, v, torch.from_numpy(sel).cuda(), torch.from_numpy(nsel).cuda())
    torch.cuda.synchronize()
    oh = host64(o)
    assert np.isfinite(oh).all()
    blocks = [0, 1, 200, 255, 256, 257, 299, 300]
    ref = O._attend_blocks(host64(q)[0, 0], host64(k)[0, 0], host64(v)[0, 0], 1 / math.sqrt(D),
                           lambda a: O.blocks_to_keys(np.arange(a + 1), n), blocks=blocks)
    for a in blocks:
        rows = slice(a * 64, min(n, (a + 1) * 64))
        check_attention(oh[0, 0, rows], ref[a], f"block {a}")


@pytest.mark.parametrize("n,D,dt,init,local", [(1000, 128, "bf16", 1, 2), (1000, 128, "bf16", 0, 1),
                                               (64 * 9 + 5, 64, "f32", 2, 3), (500, 128, "bf16", 3, 64),
                                               (64 * 8 + 50, 128, "f32", 1, 3),
                                               # bf16 panels at head_dim 64: an even and an odd
                                               # block count, windows crossing panel edges
                                               (1000, 64, "bf16", 1, 3), (64 * 7 + 33, 64, "bf16", 2, 2)])
def test_streaming(n, D, dt, init, local):
    say(f"streaming n={n} init={init} local={local}")
    q, k, v = rand_qkv(1, 4, 4, n, D, dt, seed=n + init, amp=2.0)
    o = dsa.streaming_attention(q, k, v, init, local, heads=[0, 2])
    torch.cuda.synchronize()
    qh, kh, vh, oh = host64(q), host64(k), host64(v), host64(o)
    for h in (0, 2):
        ref = O.streaming_head(qh[0, h], kh[0, h], vh[0, h], init, local)
        check_attention(oh[0, h], O.assemble(ref["out"], n, D), f"h{h}")
    assert float(np.abs(oh[0, 1]).max()) == 0.0


# ---------------------------------------------------------------------------
# block-sparse estimate
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("n,D,dt,topk", [(64 * 40 + 9, 128, "bf16", 6), (64 * 20, 64, "f32", 3),
                                         (64 * 70, 128, "bf16", 100)])
def test_bs_pool_select(n, D, dt, topk):
    say(f"bs_pool_select n={n} D={D} {dt} topk={topk}")
    q, k, _ = rand_qkv(1, 4, 2, n, D, dt, seed=n, amp=1.0)
    heads = [0, 3]
    qp = dsa.bs_pool(q, heads)
    kp_all = dsa.bs_pool(k)
    kp = kp_all[torch.tensor([kvh(h, 4, 2) for h in heads], device="cuda")].contiguous()
    sel, n_sel, lg = dsa.bs_select(qp, kp, topk, return_logits=True)
    torch.cuda.synchronize()
    qh, kh = host64(q), host64(k)
    nb = O.num_blocks(n)
    sc = 1 / math.sqrt(D)
    for t, h in enumerate(heads):
        qpo, kpo = O.mean_pool(qh[0, h]), O.mean_pool(kh[0, kvh(h, 4, 2)])
        np.testing.assert_allclose(qp[t].cpu().numpy(), qpo, rtol=2e-6, atol=2e-6)
        np.testing.assert_allclose(kp[t].cpu().numpy(), kpo, rtol=2e-6, atol=2e-6)
        L = O.block_logits(qpo, kpo, sc)
        Lg = lg[t].cpu().numpy()
        cs = sc * np.linalg.norm(qpo, axis=1)[:, None] * np.linalg.norm(kpo, axis=1)[None, :]
        tri = np.tril(np.ones((nb, nb), bool))
        assert (np.abs(Lg - L)[tri] <= 1e-3 * cs[tri] + 1e-12).all()
        want = O.block_select(Lg, topk)                     # bit-exact on the GPU's logits
        for a in range(nb):
            assert int(n_sel[t, a]) == min(topk, a + 1)
            assert np.array_equal(sel[t, a, : int(n_sel[t, a])].cpu().numpy(), want[a]), (t, a)
    # the scratch-buffer path gives the same selection (entries past the
    # counts are unwritten, so only the counted prefixes are compared)
    sel2, n_sel2 = dsa.bs_select(qp, kp, topk)
    assert torch.equal(n_sel2, n_sel)
    valid = torch.arange(sel.shape[-1], device=sel.device) < n_sel[..., None]
    assert torch.equal(sel2[valid], sel[valid])


@pytest.mark.parametrize("case", ["ties", "wide_topk", "few_values"])
def test_bs_select_bin_and_radix_paths(case):
    """Rows of 1100 blocks through both selection paths: all-equal logits (the
    whole row shares one key bin, which the bin path ranks while the row holds
    at most 1024 entries and the radix select takes beyond), a topk above 1024
    (radix select), and logits with few distinct values (large tied bins).
    Indices bit-exact against the oracle on the GPU's logits."""
    say(f"bs_select paths case={case}")
    nb, D = 1100, 64
    g = torch.Generator(device="cuda").manual_seed(5)
    kp = torch.randn(1, nb, D, generator=g, device="cuda")
    qp = torch.randn(1, nb, D, generator=g, device="cuda")
    topk = 40
    if case == "ties":
        qp.zero_()
    elif case == "wide_topk":
        topk = 1050
    else:
        qp = torch.randint(-1, 2, (1, nb, D), generator=g, device="cuda").float()
        kp = torch.randint(-1, 2, (1, nb, D), generator=g, device="cuda").float()
        topk = 300
    sel, n_sel, lg = dsa.bs_select(qp, kp, topk, return_logits=True)
    torch.cuda.synchronize()
    Lg = lg[0].cpu().numpy()
    want = O.block_select(Lg, topk)
    s_h, n_h = sel[0].cpu().numpy(), n_sel[0].cpu().numpy()
    for a in range(nb):
        assert int(n_h[a]) == min(topk, a + 1)
        assert np.array_equal(s_h[a, : int(n_h[a])], want[a]), (case, a)


# ---------------------------------------------------------------------------
# the three public calls end to end
# ---------------------------------------------------------------------------
def _vs_stage_pipeline(q, k, v, vk, sk, heads):
    vg, sg = dsa.vs_estimate(q, k, heads=heads)
    V = dsa.topk(vg, vk)
    S = dsa.topk(sg, sk, 0)
    iv, niv, cols, ncols = dsa.vs_build_index(V, S, q.shape[2])
    o = dsa.sparse_attention_vs(q, k, v, iv, niv, cols, ncols, heads=heads)
    return vg, sg, V, S, iv, niv, cols, ncols, o


def check_vs_end_to_end(q, k, v, vk, sk, heads, blocks=None, tag=""):
    """Fused call == stage pipeline (bitwise); indices == oracle on the GPU's
    scores (bitwise); attention == oracle within tolerance. ``blocks``: query
    blocks the oracle checks (all when None)."""
    B, Hq, n, D = q.shape
    Hkv = k.shape[1]
    o_fused = dsa.vertical_slash_sparse_attention(q, k, v, vk, sk, heads=heads)
    vg, sg, V, S, iv, niv, cols, ncols, o = _vs_stage_pipeline(q, k, v, vk, sk, heads)
    torch.cuda.synchronize()
    assert torch.equal(o_fused, o), tag
    qh = host64(q)
    kh, vh = host64(k), host64(v)
    oh = host64(o)
    stats = []
    for b in range(B):
        for t, h in enumerate(heads):
            row = b * len(heads) + t
            g = kvh(h, Hq, Hkv)
            res = O.vs_head(qh[b, h], kh[b, g], vh[b, g], vk, sk, blocks=blocks,
                            scores=(vg[row].cpu().numpy(), sg[row].cpu().numpy()))
            assert np.array_equal(V[row].cpu().numpy(), res["V"]), (tag, row)
            assert np.array_equal(S[row].cpu().numpy(), res["S"]), (tag, row)
            assert int(niv[row]) == len(res["intervals"])
            assert [tuple(x) for x in iv[row, : int(niv[row])].cpu().tolist()] == res["intervals"]
            for a in res["out"]:
                c = O.vs_block_cols(res["V"], O.vs_block_ranges(res["intervals"], a, n), a, n)
                assert np.array_equal(gpu_cols(cols, ncols, row, a), c), (tag, row, a)
                r0 = a * BLK
                stats.append(check_attention(oh[b, h, r0: r0 + res["out"][a].shape[0]], res["out"][a],
                                             f"{tag} row {row} block {a}"))
    return stats


def test_vs_end_to_end_small():
    say("vs end to end small")
    for n, D, dt in [(1000, 128, "bf16"), (64 * 7 + 30, 64, "f32")]:
        q, k, v = rand_qkv(2, 4, 2, n, D, dt, seed=n, amp=2.0)
        check_vs_end_to_end(q, k, v, 30, 20, [2, 0, 1], tag=f"n{n}")


def test_bs_end_to_end_small():
    say("bs end to end small")
    for n, D, dt, topk in [(64 * 30 + 7, 128, "bf16", 5), (64 * 12, 64, "f32", 4)]:
        q, k, v = rand_qkv(2, 4, 2, n, D, dt, seed=n + 1, amp=2.0)
        heads = [1, 2]
        o = dsa.block_sparse_attention(q, k, v, topk, heads=heads)
        qp = dsa.bs_pool(q, heads)
        kp_all = dsa.bs_pool(k)
        idx = torch.tensor([b * 2 + kvh(h, 4, 2) for b in range(2) for h in heads], device="cuda")
        sel, n_sel, lg = dsa.bs_select(qp, kp_all[idx].contiguous(), topk, return_logits=True)
        o2 = dsa.sparse_attention_blocks(q, k, v, sel, n_sel, heads=heads)
        torch.cuda.synchronize()
        assert torch.equal(o, o2)
        qh, kh, vh, oh = host64(q), host64(k), host64(v), host64(o)
        for b in range(2):
            for t, h in enumerate(heads):
                row = b * 2 + t
                g = kvh(h, 4, 2)
                res = O.bs_head(qh[b, h], kh[b, g], vh[b, g], topk, logits=lg[row].cpu().numpy())
                for a in range(O.num_blocks(n)):
                    assert np.array_equal(sel[row, a, : int(n_sel[row, a])].cpu().numpy(), res["sel"][a])
                check_attention(oh[b, h], O.assemble(res["out"], n, D), f"bs b{b} h{h}")


@pytest.mark.parametrize("n,D,dt,window,keep", [(1000, 128, "bf16", 256, 100), (777, 64, "f32", 64, 50),
                                                 (300, 128, "bf16", 100, 300), (70, 128, "bf16", 500, 20),
                                                 (5000, 128, "bf16", 130, 2000), (129, 64, "bf16", 1, 5),
                                                 (400, 128, "bf16", 64, 0)])
def test_kv_retention(n, D, dt, window, keep):
    """Retention scores within the estimator bar of the oracle; kept keys
    bit-exact against the oracle's top-k of the GPU's own scores."""
    say(f"kv retention n={n} D={D} {dt} window={window} keep={keep}")
    q, k, _ = rand_qkv(2, 4, 2, n, D, dt, seed=n + window, amp=2.0)
    heads = [3, 1]
    sc, kept = dsa.kv_retention(q, k, window, keep, heads=heads)
    torch.cuda.synchronize()
    assert kept.shape == (4, min(keep, n))
    qh, kh = host64(q), host64(k)
    for b in range(2):
        for t, h in enumerate(heads):
            row = b * 2 + t
            S = O.kv_retention_scores(qh[b, h], kh[b, kvh(h, 4, 2)], window, 1.0 / math.sqrt(D))
            g = sc[row].cpu().numpy()
            check_scores(g, S, f"kv retention row {row}")
            assert abs(float(g.astype(np.float64).sum()) - min(window, n)) < 1e-3 * min(window, n)
            assert np.array_equal(kept[row].cpu().numpy(), O.topk_indices(g, keep))


def test_kv_retention_128k_planted():
    """At 128K with a 256-row window: scores of two heads against the oracle,
    kept keys against the oracle's top-k of the GPU scores, and the planted
    sink key (row 0, scaled up) is kept."""
    say("kv retention 128K")
    w = synthetic.BY_NAME["llama3_8b_128k_vs_bf16"].scaled(q_heads=4, kv_heads=1)
    x = synthetic.make_inputs(w)
    q, k = x.q.cuda(), x.k.cuda()
    heads = [0, 3]
    sc, kept = dsa.kv_retention(q, k, 256, 4096, heads=heads)
    torch.cuda.synchronize()
    qh, kh = host64(x.q), host64(x.k)
    for t, h in enumerate(heads):
        S = O.kv_retention_scores(qh[0, h], kh[0, 0], 256, 1.0 / math.sqrt(w.head_dim))
        g = sc[t].cpu().numpy()
        check_scores(g, S, f"kv retention 128K head {h}")
        kt = kept[t].cpu().numpy()
        assert np.array_equal(kt, O.topk_indices(g, 4096))
        assert 0 in kt


@pytest.mark.parametrize("n,D,dt,counts", [(10000, 128, "bf16", [0, 1, 7, 100, 5000, 257]),
                                           (777, 64, "f32", [3, 777, 64, 0, 500, 31]),
                                           (4096, 128, "bf16", None), (1, 64, "bf16", None),
                                           (300, 128, "f32", None), (70000, 128, "bf16", None)])
def test_sparse_decode(n, D, dt, counts):
    """One decode row per listed head over a key list (or the whole cache)
    against the oracle on the attention bar; unlisted heads stay zero."""
    say(f"sparse decode n={n} D={D} {dt} counts={counts}")
    B, Hq, Hkv, heads = 2, 4, 2, [3, 0, 2]
    g = torch.Generator().manual_seed(n + D)
    q = (torch.randn(B, Hq, D, generator=g) * 2.0).to(DT[dt]).cuda()
    k = torch.randn(B, Hkv, n, D, generator=g).to(DT[dt]).cuda()
    v = torch.randn(B, Hkv, n, D, generator=g).to(DT[dt]).cuda()
    rng = np.random.default_rng(n)
    lists = None
    if counts is None:
        o = dsa.sparse_decode(q, k, v, heads=heads)
    else:
        width = max(counts) + 3
        keys = np.full((B * len(heads), width), -7, np.int32)   # entries past a count are never read
        lists = []
        for r, c in enumerate(counts):
            sel = np.sort(rng.choice(n, size=min(c, n), replace=False)).astype(np.int32)
            keys[r, : len(sel)] = sel
            lists.append(sel)
        n_keys = torch.tensor([len(x) for x in lists], dtype=torch.int32).cuda()
        o = dsa.sparse_decode(q, k, v, torch.from_numpy(keys).cuda(), n_keys, heads=heads)
    torch.cuda.synchronize()
    qh, kh, vh, oh = host64(q), host64(k), host64(v), host64(o)
    sc = 1.0 / math.sqrt(D)
    for b in range(B):
        for t, h in enumerate(heads):
            r = b * len(heads) + t
            want = O.decode_attention(qh[b, h], kh[b, kvh(h, Hq, Hkv)], vh[b, kvh(h, Hq, Hkv)],
                                      None if lists is None else lists[r], sc)
            check_attention(oh[b, h][None], want[None], f"decode b{b} h{h}")
        assert not oh[b, 1].any()


def test_decode_over_retained_keys_1m():
    """The after-prefill chain at 1M tokens: retention scores over the last
    256 rows keep 4096 keys per head, then a new row decodes over exactly
    those keys; checked against the oracle (scores of the kept set, attention
    over it), and decoding over all keys is checked too."""
    say("decode over retained keys 1M")
    w = synthetic.BY_NAME["llama3_8b_1m_mixed_bf16"].scaled(q_heads=4, kv_heads=1)
    x = synthetic.make_inputs(w, device="cuda")
    heads = [1, 2]
    sc_, kept = dsa.kv_retention(x.q, x.k, 256, 4096, heads=heads)
    g = torch.Generator().manual_seed(5)
    qd = torch.randn(1, 4, w.head_dim, generator=g).to(torch.bfloat16).cuda()
    n_keys = torch.full((2,), 4096, dtype=torch.int32, device="cuda")
    o = dsa.sparse_decode(qd, x.k, x.v, kept, n_keys, heads=heads)
    o_all = dsa.sparse_decode(qd, x.k, x.v, heads=heads)
    torch.cuda.synchronize()
    kh = x.k[0, 0].float().cpu().numpy().astype(np.float64)
    vh = x.v[0, 0].float().cpu().numpy().astype(np.float64)
    qh = host64(qd)
    sc = 1.0 / math.sqrt(w.head_dim)
    for t, h in enumerate(heads):
        kt = kept[t].cpu().numpy()
        assert np.array_equal(kt, O.topk_indices(sc_[t].cpu().numpy(), 4096))
        want = O.decode_attention(qh[0, h], kh, vh, kt, sc)
        check_attention(host64(o)[0, h][None], want[None], f"decode retained h{h}")
        want_all = O.decode_attention(qh[0, h], kh, vh, None, sc)
        check_attention(host64(o_all)[0, h][None], want_all[None], f"decode all h{h}")


def test_repeat_launch_bitwise():
    """Two launches on the same inputs give the same bits for every pattern: a
    kernel that read an MFMA result before it is complete, or raced on LDS,
    would change the lazy-max decisions and with them the last bits."""
    say("repeat launch bitwise")
    w = synthetic.BY_NAME["qwen2_7b_32k_b4_mixed_bf16"].scaled(batch=1, seq_len=8192, slash_topk=600,
                                                                vertical_topk=100, topk=16, local_blocks=8)
    x = synthetic.make_inputs(w)
    q, k, v = x.q.cuda(), x.k.cuda(), x.v.cuda()
    hp = x.heads
    outs = []
    for _ in range(2):
        o = torch.zeros_like(q)
        dsa.vertical_slash_sparse_attention(q, k, v, w.vertical_topk, w.slash_topk, heads=hp["vs"], out=o)
        dsa.block_sparse_attention(q, k, v, w.topk, heads=hp["bs"], out=o)
        dsa.streaming_attention(q, k, v, w.init_blocks, w.local_blocks, heads=hp["st"], out=o)
        outs.append(o)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


def test_layer_two_streams_bitwise():
    """The block-sparse call on a second stream beside the other calls (the
    benchmark's layer step) writes the same bits as the serial order."""
    say("layer on two streams")
    w = synthetic.BY_NAME["qwen2_7b_32k_b4_mixed_bf16"].scaled(batch=2, seq_len=4096 + 77, slash_topk=500,
                                                                vertical_topk=60, topk=12, local_blocks=6)
    x = synthetic.make_inputs(w)
    q, k, v = x.q.cuda(), x.k.cuda(), x.v.cuda()
    hp = x.heads
    calls = [lambda o: dsa.vertical_slash_sparse_attention(q, k, v, w.vertical_topk, w.slash_topk, heads=hp["vs"], out=o),
             lambda o: dsa.block_sparse_attention(q, k, v, w.topk, heads=hp["bs"], out=o),
             lambda o: dsa.streaming_attention(q, k, v, w.init_blocks, w.local_blocks, heads=hp["st"], out=o)]
    ref = torch.zeros_like(q)
    for c in calls:
        c(ref)
    side = torch.cuda.Stream()
    for _ in range(2):
        o = torch.zeros_like(q)
        main = torch.cuda.current_stream()
        side.wait_stream(main)
        with torch.cuda.stream(side):
            calls[1](o)
        calls[0](o)
        calls[2](o)
        main.wait_stream(side)
        torch.cuda.synchronize()
        assert torch.equal(o, ref)


def test_mixed_layer_small():
    """Three calls over head subsets fill one output, as a mixed layer does."""
    say("mixed layer small")
    w = synthetic.BY_NAME["qwen2_7b_32k_b4_mixed_bf16"].scaled(batch=1, seq_len=2048, slash_topk=300,
                                                                vertical_topk=50, topk=8, local_blocks=4)
    x = synthetic.make_inputs(w)
    q, k, v = x.q.cuda(), x.k.cuda(), x.v.cuda()
    hp = x.heads
    o = torch.zeros_like(q)
    dsa.vertical_slash_sparse_attention(q, k, v, w.vertical_topk, w.slash_topk, heads=hp["vs"], out=o)
    dsa.block_sparse_attention(q, k, v, w.topk, heads=hp["bs"], out=o)
    dsa.streaming_attention(q, k, v, w.init_blocks, w.local_blocks, heads=hp["st"], out=o)
    torch.cuda.synchronize()
    oh = host64(o)
    assert np.isfinite(oh).all()
    qh, kh, vh = host64(q), host64(k), host64(v)
    n, D = w.seq_len, w.head_dim
    for h in hp["st"][:2]:
        g = kvh(h, w.q_heads, w.kv_heads)
        ref = O.streaming_head(qh[0, h], kh[0, g], vh[0, g], w.init_blocks, w.local_blocks)
        check_attention(oh[0, h], O.assemble(ref["out"], n, D), f"st h{h}")
    for h in hp["vs"][:2]:
        row_o = dsa.vertical_slash_sparse_attention(q, k, v, w.vertical_topk, w.slash_topk, heads=[h])
        assert torch.equal(row_o[0, h], o[0, h])
    for h in hp["bs"][:2]:
        row_o = dsa.block_sparse_attention(q, k, v, w.topk, heads=[h])
        assert torch.equal(row_o[0, h], o[0, h])


@pytest.mark.parametrize("n,D,dt", [(1, 128, "bf16"), (2, 64, "f32"), (63, 128, "bf16"), (64, 64, "bf16")])
def test_one_block_layers(n, D, dt):
    """Sequences of at most one 64-key block through the three public calls,
    estimation included: every pattern's key set is then the whole causal
    range (the forced diagonal offset, the forced diagonal block, the window
    that holds the diagonal block), so each head equals dense causal attention;
    a single token returns its own value row."""
    say(f"one-block layer n={n} D={D} {dt}")
    q, k, v = rand_qkv(1, 6, 2, n, D, dt, seed=40 + n)
    o = torch.zeros_like(q)
    dsa.vertical_slash_sparse_attention(q, k, v, 3, 2, heads=[0, 3], out=o)
    dsa.block_sparse_attention(q, k, v, 1, heads=[1, 4], out=o)
    dsa.streaming_attention(q, k, v, 0, 1, heads=[2, 5], out=o)
    torch.cuda.synchronize()
    oh, qh, kh, vh = host64(o), host64(q), host64(k), host64(v)
    for h in range(6):
        g = kvh(h, 6, 2)
        ref = O.dense_causal_attention(qh[0, h], kh[0, g], vh[0, g], 1 / math.sqrt(D))
        check_attention(oh[0, h], ref, f"h{h}")
        if n == 1:
            assert np.array_equal(oh[0, h, 0], vh[0, g, 0]), h


def _streaming_vs_oracle(o, q, k, v, heads, init_blocks, local_blocks, tag, blocks=None):
    Hq, Hkv, n, D = q.shape[1], k.shape[1], q.shape[2], q.shape[3]
    oh, qh, kh, vh = host64(o), host64(q), host64(k), host64(v)
    for b in range(q.shape[0]):
        for h in heads:
            g = kvh(h, Hq, Hkv)
            res = O.streaming_head(qh[b, h], kh[b, g], vh[b, g], init_blocks, local_blocks, blocks=blocks)
            for a, ref in res["out"].items():
                check_attention(oh[b, h, a * BLK: a * BLK + ref.shape[0]], ref, f"{tag} st b{b} h{h} block {a}")


@pytest.mark.parametrize("D,dt,n,B", [(128, "bf16", 2048 + 37, 2), (64, "bf16", 1500, 1),
                                      (64, "f32", 700, 2), (128, "bf16", 64, 1), (128, "bf16", 5, 2)])
def test_mixed_one_launch(D, dt, n, B):
    """The mixed layer as one attention launch: VS and BS heads bit-identical
    to the per-pattern calls (which the oracle checks above), streaming heads
    against the oracle, heads without a pattern left untouched."""
    say(f"mixed one launch D={D} {dt} n={n} B={B}")
    Hq, Hkv = 8, 2
    q, k, v = rand_qkv(B, Hq, Hkv, n, D, dt, seed=100 + n)
    pats = ["vs", "bs", "st", "vs", "st", None, "bs", "vs"]
    vk, sk, tk, ib, lb = 40, 200, 6, 1, 3
    hv = [h for h, p in enumerate(pats) if p == "vs"]
    hb = [h for h, p in enumerate(pats) if p == "bs"]
    hs = [h for h, p in enumerate(pats) if p == "st"]
    o = torch.full_like(q, 7.0)
    dsa.mixed_sparse_attention(q, k, v, pats, vertical_topk=vk, slash_topk=sk, topk=tk, init_blocks=ib,
                               local_blocks=lb, out=o)
    ref = torch.zeros_like(q)
    dsa.vertical_slash_sparse_attention(q, k, v, vk, sk, heads=hv, out=ref)
    dsa.block_sparse_attention(q, k, v, tk, heads=hb, out=ref)
    dsa.streaming_attention(q, k, v, ib, lb, heads=hs, out=ref)
    torch.cuda.synchronize()
    for h in hv + hb:
        assert torch.equal(o[:, h], ref[:, h]), h
    assert (o[:, 5] == 7.0).all()
    if dt == "f32":  # fp32 launches per pattern: the streaming kernel itself
        for h in hs:
            assert torch.equal(o[:, h], ref[:, h]), h
    _streaming_vs_oracle(o, q, k, v, hs, ib, lb, "mixed")


def test_sparse_attention_mixed_given_indices():
    """The one-launch stage call over indices from the stage calls equals the
    per-pattern stage calls bit for bit (VS, BS heads)."""
    say("mixed given indices")
    B, Hq, Hkv, n, D = 2, 6, 2, 1300, 128
    q, k, v = rand_qkv(B, Hq, Hkv, n, D, "bf16", seed=5)
    pats = ["st", "vs", "bs", "bs", "vs", "st"]
    hv = [h for h, p in enumerate(pats) if p == "vs"]
    hb = [h for h, p in enumerate(pats) if p == "bs"]
    hs = [h for h, p in enumerate(pats) if p == "st"]
    vg, sg = dsa.vs_estimate(q, k, heads=hv)
    ix = dsa.vs_build_index(dsa.topk(vg, 30), dsa.topk(sg, 150, 0), n)
    G = Hq // Hkv
    kp = dsa.bs_pool(k)[torch.tensor([b * Hkv + h // G for b in range(B) for h in hb], device=q.device)]
    sel, n_sel = dsa.bs_select(dsa.bs_pool(q, hb), kp.contiguous(), 5)
    o = dsa.sparse_attention_mixed(q, k, v, pats, vs_index=ix, bs_index=(sel, n_sel), init_blocks=2,
                                   local_blocks=4)
    ref = dsa.sparse_attention_vs(q, k, v, *ix, heads=hv)
    dsa.sparse_attention_blocks(q, k, v, sel, n_sel, heads=hb, out=ref)
    torch.cuda.synchronize()
    for h in hv + hb:
        assert torch.equal(o[:, h], ref[:, h]), h
    _streaming_vs_oracle(o, q, k, v, hs, 2, 4, "mixed stage")


# ---------------------------------------------------------------------------
# workload-shaped cases
# ---------------------------------------------------------------------------
def test_workload_vs_head_4k_f32():
    """Full 4K fp32 vertical-slash head, every row checked."""
    w = synthetic.BY_NAME["vs_head_4k_f32"]
    say(f"workload {w.name}")
    x = synthetic.make_inputs(w)
    q, k, v = x.q.cuda(), x.k.cuda(), x.v.cuda()
    vg, sg = dsa.vs_estimate(q, k)
    v64, s64 = O.vs_scores(host64(x.q)[0, 0], host64(x.k)[0, 0], 64, 1 / 8.0)
    check_scores(vg[0].cpu().numpy(), v64, "v")
    check_scores(sg[0].cpu().numpy(), s64, "s")
    check_vs_end_to_end(q, k, v, w.vertical_topk, w.slash_topk, [0], tag=w.name)
    # independent end to end: the oracle's own estimate gives the same indices
    # up to score gaps below the estimator tolerance
    res = O.vs_head(host64(x.q)[0, 0], host64(x.k)[0, 0], host64(x.v)[0, 0], 256, 256, blocks=[])
    V = dsa.topk(vg, 256)[0].cpu().numpy()
    jac = len(set(V) & set(res["V"])) / len(set(V) | set(res["V"]))
    say(f"  vertical Jaccard GPU vs oracle-estimated: {jac:.4f}")
    assert jac > 0.95


def test_workload_bs_32k():
    """The 32K block-sparse MHA layer, all heads, sampled query blocks."""
    w = synthetic.BY_NAME["bs_mha4_32k_bf16"]
    say(f"workload {w.name}")
    x = synthetic.make_inputs(w)
    q, k, v = x.q.cuda(), x.k.cuda(), x.v.cuda()
    o = dsa.block_sparse_attention(q, k, v, w.topk)
    qp = dsa.bs_pool(q)
    kp = dsa.bs_pool(k)
    sel, n_sel, lg = dsa.bs_select(qp, kp, w.topk, return_logits=True)
    torch.cuda.synchronize()
    nb = O.num_blocks(w.seq_len)
    rng = np.random.default_rng(0)
    blocks = sorted(set([0, nb - 1] + rng.choice(nb, 24, replace=False).tolist()))
    qh, kh, vh, oh = host64(x.q), host64(x.k), host64(x.v), host64(o)
    for h in range(w.q_heads):
        L = lg[h].cpu().numpy()
        res = O.bs_head(qh[0, h], kh[0, h], vh[0, h], w.topk, logits=L, blocks=blocks)
        for a in range(nb):
            assert np.array_equal(sel[h, a, : int(n_sel[h, a])].cpu().numpy(), res["sel"][a])
        for kb, qbs in x.planted[(0, h)]:
            for qa in qbs:
                assert kb in res["sel"][qa].tolist()
        for a in blocks:
            check_attention(oh[0, h, a * BLK:(a + 1) * BLK], res["out"][a], f"h{h} a{a}")


def test_workload_llama_128k_sampled():
    """The 128K Llama-3-8B-shaped layer at full size: every head runs on the
    GPU; the oracle checks two heads' scores and indices and a sample of query
    blocks' attention."""
    w = synthetic.BY_NAME["llama3_8b_128k_vs_bf16"]
    say(f"workload {w.name}")
    x = synthetic.make_inputs(w, device="cuda")
    q, k, v = x.q, x.k, x.v
    heads = list(range(w.q_heads))
    o = dsa.vertical_slash_sparse_attention(q, k, v, w.vertical_topk, w.slash_topk)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
    n = w.seq_len
    nb = O.num_blocks(n)
    rng = np.random.default_rng(2)
    blocks = sorted(set([0, 1, nb - 1] + rng.choice(nb, 12, replace=False).tolist()))
    for h in (5, 30):
        g = kvh(h, w.q_heads, w.kv_heads)
        qs, ks, vs = q[:, h:h + 1].contiguous(), k[:, g:g + 1].contiguous(), v[:, g:g + 1].contiguous()
        vg, sg = dsa.vs_estimate(qs, ks)
        qh, kh = host64(qs)[0, 0], host64(ks)[0, 0]
        v64, s64 = O.vs_scores(qh, kh, 64, 1 / math.sqrt(128))
        check_scores(vg[0].cpu().numpy(), v64, f"v h{h}")
        check_scores(sg[0].cpu().numpy(), s64, f"s h{h}")
        # per-head call reproduces the layer call bit for bit
        o1 = dsa.vertical_slash_sparse_attention(qs, ks, vs, w.vertical_topk, w.slash_topk)
        assert torch.equal(o1[0, 0], o[0, h])
        stats = check_vs_end_to_end(qs, ks, vs, w.vertical_topk, w.slash_topk, [0], blocks=blocks,
                                    tag=f"h{h}")
        say(f"  h{h}: worst max-abs {max(s[0] for s in stats):.2e}, mean {np.mean([s[1] for s in stats]):.2e}")


# Every head of the two mixed layers at full size, one test per (batch,
# head), on one module-scoped run of each layer (three calls into one output,
# as the benchmark times them, and the one-launch call beside it).
_LAYERS = {}


def _mixed_layer(name):
    if name not in _LAYERS:
        _LAYERS.clear()
        torch.cuda.empty_cache()
        w = synthetic.BY_NAME[name]
        say(f"workload {w.name} (mixed layer, full size)")
        x = synthetic.make_inputs(w, device="cuda")
        q, k, v = x.q, x.k, x.v
        o = torch.zeros_like(q)
        dsa.vertical_slash_sparse_attention(q, k, v, w.vertical_topk, w.slash_topk, last_q=w.last_q,
                                            heads=x.heads["vs"], out=o)
        dsa.block_sparse_attention(q, k, v, w.topk, heads=x.heads["bs"], out=o)
        dsa.streaming_attention(q, k, v, w.init_blocks, w.local_blocks, heads=x.heads["st"], out=o)
        o_one = dsa.mixed_sparse_attention(q, k, v, synthetic.pattern_list(w), vertical_topk=w.vertical_topk,
                                           slash_topk=w.slash_topk, topk=w.topk, init_blocks=w.init_blocks,
                                           local_blocks=w.local_blocks, last_q=w.last_q)
        torch.cuda.synchronize()
        assert torch.isfinite(o.float()).all() and torch.isfinite(o_one.float()).all()
        _LAYERS[name] = dict(w=w, x=x, o=o, o_one=o_one)
    return _LAYERS[name]


def _check_mixed_head(name, b, h, n_sample, seed):
    """One head of a full-size mixed layer: the head alone reproduces the
    layer's output bit for bit; its scores or logits match the oracle; its
    indices are the oracle's on the GPU's own scores or logits; and sampled
    query blocks of both the three-call output and the one-launch output match
    the oracle's attention."""
    L = _mixed_layer(name)
    w, x, o, o_one = L["w"], L["x"], L["o"], L["o_one"]
    pat = next(p for p in ("vs", "bs", "st") if h in x.heads[p])
    q, k, v = x.q, x.k, x.v
    n, D = w.seq_len, w.head_dim
    nb = O.num_blocks(n)
    sc = 1 / math.sqrt(D)
    rng = np.random.default_rng(seed)
    blocks = sorted(set([0, 1, nb - 1] + rng.choice(nb, n_sample, replace=False).tolist()))
    g = kvh(h, w.q_heads, w.kv_heads)
    qs, ks, vs = (q[b:b + 1, h:h + 1].contiguous(), k[b:b + 1, g:g + 1].contiguous(),
                  v[b:b + 1, g:g + 1].contiguous())
    tag = f"{w.name} {pat} b{b} h{h}"
    say(f"  {tag}")
    qh, kh, vh = host64(qs)[0, 0], host64(ks)[0, 0], host64(vs)[0, 0]
    outs = {"three calls": o[b, h], "one launch": o_one[b, h]}

    def check_blocks(ref_blocks):
        for label, oh in outs.items():
            for a, ref in ref_blocks.items():
                check_attention(host64(oh[a * BLK: a * BLK + ref.shape[0]]), ref, f"{tag} {label} block {a}")

    if pat == "vs":
        o1 = dsa.vertical_slash_sparse_attention(qs, ks, vs, w.vertical_topk, w.slash_topk, last_q=w.last_q)
        assert torch.equal(o1[0, 0], o[b, h]), tag
        vg, sg = dsa.vs_estimate(qs, ks, last_q=w.last_q)
        torch.cuda.synchronize()
        v64, s64 = O.vs_scores(qh, kh, w.last_q, sc)
        check_scores(vg[0].cpu().numpy(), v64, f"v {tag}")
        check_scores(sg[0].cpu().numpy(), s64, f"s {tag}")
        del v64, s64
        # indices: the oracle's top-k, intervals and column lists on the GPU's scores
        V = dsa.topk(vg, w.vertical_topk)
        S = dsa.topk(sg, w.slash_topk, 0)
        iv, niv, cols, ncols = dsa.vs_build_index(V, S, n)
        torch.cuda.synchronize()
        res = O.vs_head(qh, kh, vh, w.vertical_topk, w.slash_topk, last_q=w.last_q, blocks=blocks,
                        scores=(vg[0].cpu().numpy(), sg[0].cpu().numpy()))
        assert np.array_equal(V[0].cpu().numpy(), res["V"]), tag
        assert np.array_equal(S[0].cpu().numpy(), res["S"]), tag
        assert [tuple(t) for t in iv[0, : int(niv[0])].cpu().tolist()] == res["intervals"], tag
        for a in blocks:
            c = O.vs_block_cols(res["V"], O.vs_block_ranges(res["intervals"], a, n), a, n)
            assert np.array_equal(gpu_cols(cols, ncols, 0, a), c), (tag, a)
        check_blocks(res["out"])
    elif pat == "bs":
        o1 = dsa.block_sparse_attention(qs, ks, vs, w.topk)
        assert torch.equal(o1[0, 0], o[b, h]), tag
        qp, kp = dsa.bs_pool(qs), dsa.bs_pool(ks)
        sel, n_sel, lg = dsa.bs_select(qp, kp, w.topk, return_logits=True)
        torch.cuda.synchronize()
        qpo, kpo = O.mean_pool(qh), O.mean_pool(kh)
        np.testing.assert_allclose(qp[0].cpu().numpy(), qpo, rtol=2e-6, atol=2e-6)
        np.testing.assert_allclose(kp[0].cpu().numpy(), kpo, rtol=2e-6, atol=2e-6)
        ref = {}
        for a in blocks:
            L32 = O.block_logits(qpo[a:a + 1], kpo[: a + 1], sc)[0]
            la = lg[0, a, : a + 1].cpu().numpy()
            bound = sc * np.linalg.norm(qpo[a]) * np.linalg.norm(kpo[: a + 1], axis=1)
            assert (np.abs(la - L32) <= 1e-3 * bound + 1e-12).all(), (tag, a)
            want = O.topk_indices(la, w.topk, forced=(a,))
            assert int(n_sel[0, a]) == len(want), (tag, a)
            assert np.array_equal(sel[0, a, : len(want)].cpu().numpy(), want), (tag, a)
            rows = np.arange(a * BLK, min(n, (a + 1) * BLK))
            ref[a] = O.masked_attention(qh[rows], rows, O.blocks_to_keys(want, n), kh, vh, sc)
        check_blocks(ref)
        del lg
    else:
        o1 = dsa.streaming_attention(qs, ks, vs, w.init_blocks, w.local_blocks)
        assert torch.equal(o1[0, 0], o[b, h]), tag
        res = O.streaming_head(qh, kh, vh, w.init_blocks, w.local_blocks, blocks=blocks)
        check_blocks(res["out"])


_W1M = synthetic.BY_NAME["llama3_8b_1m_mixed_bf16"]
_WQW = synthetic.BY_NAME["qwen2_7b_32k_b4_mixed_bf16"]


@pytest.mark.parametrize("h", range(_W1M.q_heads))
def test_workload_llama_1m_mixed_every_head(h):
    """The headline 1M-token layer (19 VS, 10 BS, 3 streaming heads), every head."""
    _check_mixed_head(_W1M.name, 0, h, 16, seed=7 + h)


@pytest.mark.parametrize("b,h", [(b, h) for b in range(_WQW.batch) for h in range(_WQW.q_heads)])
def test_workload_qwen2_32k_b4_mixed_every_head(b, h):
    """The Qwen2-7B-shaped 32K layer, batch 4 (10 VS, 9 BS, 9 streaming heads), every (batch, head)."""
    _check_mixed_head(_WQW.name, b, h, 8, seed=8 + 28 * b + h)


# ---------------------------------------------------------------------------
# hierarchical chunk pruning
# ---------------------------------------------------------------------------
def _block_max_oracle(qv, kh, limit, scale):
    """float64 largest token score of each visible 64-key block."""
    s = O.token_scores(qv, kh, limit, scale)
    return np.array([s[b * BLK: min(limit, (b + 1) * BLK)].max() for b in range((limit + BLK - 1) // BLK)])


def _check_block_max(bm_gpu, qv, kh, limit, scale, tag):
    """GPU block maxima within fp32 dot-product rounding of the float64 ones:
    |error| <= 1e-4 * scale * |q| * max |k_j| over the block."""
    ref = _block_max_oracle(qv, kh, limit, scale)
    g = np.asarray(bm_gpu[: len(ref)], np.float64)
    kn = np.linalg.norm(kh[:limit], axis=1)
    kmax = np.array([kn[b * BLK: min(limit, (b + 1) * BLK)].max() for b in range(len(ref))])
    bound = 1e-4 * scale * np.linalg.norm(qv) * kmax + 1e-6
    bad = np.abs(g - ref) > bound
    assert not bad.any(), (tag, np.flatnonzero(bad)[:5], g[bad][:5], ref[bad][:5])


@pytest.mark.parametrize("n,D,dt,qdt,stages,unit_rows", [
    (5000, 128, "bf16", "bf16", [(1024, 2), (256, 3), (64, 4)], 0),
    (4096, 64, "f32", "f32", [(512, 3), (64, 5)], 0),
    (777, 128, "bf16", "f32", [(256, 9), (64, 50)], 0),        # keep-all stages
    (64, 128, "bf16", "bf16", [(128, 1), (64, 1)], 0),          # one block
    (1, 64, "bf16", "bf16", [(64, 1)], 0),                      # one key
    (70000, 128, "bf16", "bf16", [(4096, 4), (512, 8), (64, 16)], 0),
    (1000, 128, "bf16", "f32", [(256, 2), (64, 3)], 64),        # prefill units (pooled blocks)
    (64 * 9 + 5, 64, "f32", "f32", [(192, 1), (64, 2)], 64),
])
def test_hier_prune_stage_call(n, D, dt, qdt, stages, unit_rows):
    """Block maxima against the float64 oracle; chunk ids bit-exact against the
    oracle's stages on the GPU's own block maxima (GQA, a head subset)."""
    say(f"hier prune n={n} D={D} {dt}/{qdt} stages={stages} unit_rows={unit_rows}")
    B, Hq, Hkv, heads = 2, 4, 2, [3, 0]
    g = torch.Generator().manual_seed(n + D)
    k = torch.randn(B, Hkv, n, D, generator=g).to(DT[dt])
    k[:, :, torch.randint(0, n, (5,), generator=g)] *= 4.0   # a few dominant keys
    units = 1 if unit_rows == 0 else O.num_blocks(n)
    qu = (torch.randn(B * len(heads), units, D, generator=g) * 0.7).to(DT[qdt])
    sel, n_sel, bm = dsa.hier_prune(qu.cuda(), k.cuda(), stages, q_heads=Hq, heads=heads, unit_rows=unit_rows,
                                    return_block_max=True)
    torch.cuda.synchronize()
    kh, quh = host64(k), host64(qu)
    sc = 1 / math.sqrt(D)
    sel, n_sel, bm = sel.cpu().numpy(), n_sel.cpu().numpy(), bm.cpu().numpy()
    for b in range(B):
        for t, h in enumerate(heads):
            r = b * len(heads) + t
            kk = kh[b, kvh(h, Hq, Hkv)]
            for u in range(units):
                limit = n if unit_rows == 0 else min(n, (u + 1) * unit_rows)
                if u < 3 or u % 5 == 0 or u == units - 1:
                    _check_block_max(bm[r, u], quh[r, u], kk, limit, sc, (r, u))
                nv = O.num_blocks(limit)
                want = O.hier_prune(quh[r, u], kk, limit, stages, sc, fine_max=bm[r, u, :nv])
                assert int(n_sel[r, u]) == len(want), (r, u)
                assert np.array_equal(sel[r, u, : len(want)], want), (r, u, sel[r, u, : len(want)], want)


@pytest.mark.parametrize("n,D,dt,stages", [(5000, 128, "bf16", [(1024, 2), (256, 3), (64, 4)]),
                                           (3000, 64, "f32", [(512, 2), (64, 3)]),
                                           (2000, 64, "bf16", [(512, 2), (128, 3), (64, 5)]),
                                           (100, 128, "bf16", [(128, 1), (64, 2)])])
def test_hier_sparse_decode(n, D, dt, stages):
    """Decode over pruned keys: the chunks equal the oracle's stages on the
    GPU's block maxima, the key lists are those chunks' keys, and the output
    matches the oracle's decode over them."""
    say(f"hier decode n={n} D={D} {dt} stages={stages}")
    B, Hq, Hkv, heads = 2, 4, 2, [2, 1, 3]
    g = torch.Generator().manual_seed(n)
    q = (torch.randn(B, Hq, D, generator=g) * 1.5).to(DT[dt]).cuda()
    k = torch.randn(B, Hkv, n, D, generator=g).to(DT[dt]).cuda()
    v = torch.randn(B, Hkv, n, D, generator=g).to(DT[dt]).cuda()
    o = dsa.hier_sparse_decode(q, k, v, stages, heads=heads)
    qu = q[:, heads].reshape(B * len(heads), 1, D).contiguous()
    sel, n_sel, bm = dsa.hier_prune(qu, k, stages, q_heads=Hq, heads=heads, return_block_max=True)
    keys, n_keys = dsa.chunks_to_keys(sel[:, 0].contiguous(), n_sel[:, 0].contiguous(), stages[-1][0], n)
    o2 = dsa.sparse_decode(q, k, v, keys, n_keys, heads=heads)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)   # the composite call is the three stage calls
    qh, kh, vh, oh = host64(q), host64(k), host64(v), host64(o)
    sc = 1 / math.sqrt(D)
    for b in range(B):
        for t, h in enumerate(heads):
            r = b * len(heads) + t
            gk = kvh(h, Hq, Hkv)
            res = O.hier_decode(qh[b, h], kh[b, gk], vh[b, gk], stages, sc,
                                fine_max=bm[r, 0].cpu().numpy())
            assert np.array_equal(sel[r, 0, : int(n_sel[r, 0])].cpu().numpy(), res["chunks"])
            nk = int(n_keys[r])
            assert np.array_equal(keys[r, :nk].cpu().numpy(), res["keys"])
            check_attention(oh[b, h][None], res["out"][None], f"hier decode b{b} h{h}")
        assert not oh[b, 0].any()


@pytest.mark.parametrize("n,D,dt,stages", [(1000, 128, "bf16", [(256, 2), (64, 3)]),
                                           (64 * 12 + 7, 64, "f32", [(384, 1), (128, 2), (64, 3)]),
                                           (64 * 70 + 9, 64, "bf16", [(1024, 1), (256, 2), (64, 6)])])
def test_hier_block_sparse_attention(n, D, dt, stages):
    """Prefill heads with the pruning as block estimator: every query block
    against the oracle (blocks chosen by the oracle's stages on the GPU's
    block maxima of the pooled queries)."""
    say(f"hier prefill n={n} D={D} {dt} stages={stages}")
    q, k, v = rand_qkv(1, 4, 2, n, D, dt, seed=n, amp=1.5)
    heads = [1, 2]
    o = dsa.hier_block_sparse_attention(q, k, v, stages, heads=heads)
    qp = dsa.bs_pool(q, heads)
    sel, n_sel, bm = dsa.hier_prune(qp, k, stages, q_heads=4, heads=heads, unit_rows=BLK, return_block_max=True)
    o2 = dsa.sparse_attention_blocks(q, k, v, sel, n_sel, heads=heads)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    qh, kh, vh, oh = host64(q), host64(k), host64(v), host64(o)
    nb = O.num_blocks(n)
    for t, h in enumerate(heads):
        fm = np.full((nb, nb), np.nan, np.float32)
        b_np = bm[t].cpu().numpy()
        for a in range(nb):
            fm[a, : a + 1] = b_np[a, : a + 1]
        res = O.hier_head(qh[0, h], kh[0, kvh(h, 4, 2)], vh[0, kvh(h, 4, 2)], stages, 1 / math.sqrt(D),
                          fine_max=fm)
        for a in range(nb):
            assert np.array_equal(sel[t, a, : int(n_sel[t, a])].cpu().numpy(), res["sel"][a]), (h, a)
        check_attention(oh[0, h], O.assemble(res["out"], n, D), f"hier prefill h{h}")
    assert float(np.abs(oh[0, 0]).max()) == 0.0


HIER_DECODE_STAGES = [(4096, 16), (512, 32), (64, 64)]


def test_hier_decode_1m_every_head():
    """Decode after a 1M-token prefill (Llama-3-8B shape, 32 query heads):
    every head's chunks against the oracle's stages on the GPU's block maxima,
    four heads' block maxima against float64, every head's output against the
    oracle's decode over its kept keys."""
    w = synthetic.BY_NAME["llama3_8b_1m_mixed_bf16"]
    say(f"hier decode 1M ({w.name})")
    x = synthetic.make_inputs(w, device="cuda")
    g = torch.Generator().manual_seed(21)
    qd = torch.randn(1, w.q_heads, w.head_dim, generator=g).to(torch.bfloat16).cuda()
    o = dsa.hier_sparse_decode(qd, x.k, x.v, HIER_DECODE_STAGES)
    sel, n_sel, bm = dsa.hier_prune(qd.reshape(w.q_heads, 1, w.head_dim).contiguous(), x.k, HIER_DECODE_STAGES,
                                    q_heads=w.q_heads, return_block_max=True)
    torch.cuda.synchronize()
    n, D = w.seq_len, w.head_dim
    sc = 1 / math.sqrt(D)
    qh, oh = host64(qd), host64(o)
    bm_h, sel_h, ns_h = bm.cpu().numpy(), sel.cpu().numpy(), n_sel.cpu().numpy()
    for kv in range(w.kv_heads):
        kh = host64(x.k[0, kv])
        vh = host64(x.v[0, kv])
        for h in range(kv * (w.q_heads // w.kv_heads), (kv + 1) * (w.q_heads // w.kv_heads)):
            if h % 8 == 0:
                _check_block_max(bm_h[h, 0], qh[0, h], kh, n, sc, f"1M h{h}")
            res = O.hier_decode(qh[0, h], kh, vh, HIER_DECODE_STAGES, sc, fine_max=bm_h[h, 0])
            assert np.array_equal(sel_h[h, 0, : int(ns_h[h, 0])], res["chunks"]), h
            check_attention(oh[0, h][None], res["out"][None], f"1M hier decode h{h}")
        del kh, vh


def test_hier_prefill_qwen2_32k_b4_sampled():
    """The pruning as block estimator on the Qwen2-shaped 32K batch-4 layer's
    block-sparse heads at full size, with the benchmark's stages: every
    (batch, head)'s chunk ids bit-exact against the oracle's stages on the
    GPU's block maxima for sampled query blocks, block maxima of those blocks
    against float64, and their attention against the oracle."""
    w = synthetic.BY_NAME["qwen2_7b_32k_b4_mixed_bf16"]
    say(f"hier prefill {w.name}")
    x = synthetic.make_inputs(w, device="cuda")
    hb = x.heads["bs"]
    st = [(1024, max(1, w.topk // 8)), (256, max(2, w.topk // 2)), (64, w.topk)]
    o = dsa.hier_block_sparse_attention(x.q, x.k, x.v, st, heads=hb)
    qp = dsa.bs_pool(x.q, hb)
    sel, n_sel, bm = dsa.hier_prune(qp, x.k, st, q_heads=w.q_heads, heads=hb, unit_rows=BLK, return_block_max=True)
    torch.cuda.synchronize()
    n, D = w.seq_len, w.head_dim
    nb = O.num_blocks(n)
    sc = 1 / math.sqrt(D)
    rng = np.random.default_rng(31)
    for b in range(w.batch):
        for t, h in enumerate(hb):
            r = b * len(hb) + t
            g = kvh(h, w.q_heads, w.kv_heads)
            kh, vh = host64(x.k[b, g]), host64(x.v[b, g])
            qh = host64(x.q[b, h])
            qpo = O.mean_pool(qh)
            blocks = sorted(set([0, nb - 1] + rng.choice(nb, 3, replace=False).tolist()))
            bm_r = bm[r].cpu().numpy()
            for a in blocks:
                limit = min(n, BLK * (a + 1))
                _check_block_max(bm_r[a], qpo[a], kh, limit, sc, (b, h, a))
                want = O.hier_prune(qpo[a], kh, limit, st, sc, fine_max=bm_r[a, : a + 1])
                assert int(n_sel[r, a]) == len(want), (b, h, a)
                assert np.array_equal(sel[r, a, : len(want)].cpu().numpy(), want), (b, h, a)
                rows = np.arange(a * BLK, min(n, (a + 1) * BLK))
                ref = O.masked_attention(qh[rows], rows, O.blocks_to_keys(want, n), kh, vh, sc)
                check_attention(host64(o[b, h, a * BLK: a * BLK + len(rows)]), ref, f"hier prefill b{b} h{h} a{a}")
