"""C-ABI checks that need no GPU: the library loads, exports every function
include/dsa.h declares, and rejects bad arguments on the host before any HIP
call (no compute calls here)."""
import ctypes
import os
import re

import pytest

import dynamic_sparse_attention_slash_amd as dsa
from dynamic_sparse_attention_slash_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return dsa.load()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) >= 15
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(B.EXPORTED)


def test_status_strings(lib):
    for code in range(5):
        assert lib.dsa_status_string(code)


def shape(b=1, hq=4, hkv=2, n=256, d=128, dt=0):
    return B.Shape(b, hq, hkv, n, d, dt)


P = ctypes.c_void_p(16)  # a non-NULL pointer that is never dereferenced


def vs_call(lib, sh, vk=8, sk=8, lq=64, heads=None, nh=0, ws=P, wsb=1 << 40, q=P):
    return lib.dsa_vertical_slash_sparse_attention(q, P, P, P, ctypes.byref(sh), vk, sk, lq, 0.0,
                                                   heads, nh, ws, wsb, None)


def test_vs_argument_errors(lib):
    assert vs_call(lib, shape(), q=None) == INVALID
    assert vs_call(lib, shape(hq=3, hkv=2)) == INVALID
    assert vs_call(lib, shape(d=96)) == UNSUPPORTED
    assert vs_call(lib, shape(dt=7)) == UNSUPPORTED
    assert vs_call(lib, shape(n=-1)) == INVALID
    assert vs_call(lib, shape(), vk=-1) == INVALID
    assert vs_call(lib, shape(), sk=0) == INVALID
    assert vs_call(lib, shape(), lq=0) == UNSUPPORTED
    assert vs_call(lib, shape(), lq=65) == UNSUPPORTED
    dup = (ctypes.c_int32 * 2)(1, 1)
    assert vs_call(lib, shape(), heads=dup, nh=2) == INVALID
    bad = (ctypes.c_int32 * 1)(4)
    assert vs_call(lib, shape(), heads=bad, nh=1) == INVALID
    assert vs_call(lib, shape(), wsb=10) == WORKSPACE
    assert vs_call(lib, shape(), ws=None) == WORKSPACE
    # nothing to do: zero batch or empty head list succeed without touching memory
    assert vs_call(lib, shape(b=0), ws=None, wsb=0) == OK
    assert vs_call(lib, shape(), heads=(ctypes.c_int32 * 1)(0), nh=0, ws=None, wsb=0) == OK
    # an empty sequence: no workspace asked for, nothing enqueued
    assert vs_call(lib, shape(n=0), ws=None, wsb=0) == OK
    assert lib.dsa_vertical_slash_workspace_bytes(ctypes.byref(shape(n=0)), 8, 8, 4) == 0
    assert lib.dsa_block_sparse_workspace_bytes(ctypes.byref(shape(n=0)), 4, 4) == 0
    assert lib.dsa_vs_estimate(P, P, ctypes.byref(shape(n=0)), 64, 0.0, None, 0, P, P, None, 0, None) == OK


def test_workspace_sizes(lib):
    sh = shape(n=4096)
    w4 = lib.dsa_vertical_slash_workspace_bytes(ctypes.byref(sh), 256, 256, 4)
    w2 = lib.dsa_vertical_slash_workspace_bytes(ctypes.byref(sh), 256, 256, 2)
    assert w4 > w2 > 0
    # per-block column lists dominate: rows * nb * vk int32
    assert w4 >= 4 * 64 * 256 * 4
    assert lib.dsa_vertical_slash_workspace_bytes(ctypes.byref(shape(d=96)), 1, 1, 1) == 0
    assert lib.dsa_block_sparse_workspace_bytes(ctypes.byref(sh), 8, 4) > 0
    # block select: one group's fp32 logits plus its bf16 hi / lo splits of the
    # pooled Q and K (four arrays, sized for head_dim 128)
    assert lib.dsa_bs_select_workspace_bytes(3, 512) == 3 * 512 * 512 * 4 + 4 * 3 * 512 * 128 * 2
    # top-k: no scratch for rows shorter than 65536 entries (one work-group
    # each); longer rows: per row three key histograms (4096 + 4096 + 256
    # bins), K and its count, and (above K, equal to K) per 16K-entry chunk
    # and wave
    assert lib.dsa_topk_workspace_bytes(4, 65535, 1000) == 0
    assert lib.dsa_topk_workspace_bytes(4, 65536, 65536) == 0   # k >= n: every index
    assert lib.dsa_topk_workspace_bytes(4, 131072, 1000) == 4 * (8450 + 8 * 8) * 4
    assert lib.dsa_topk_workspace_bytes(2, 1 << 20, 20000) == 2 * (8450 + 8 * 64) * 4
    assert lib.dsa_topk_workspace_bytes(1, 70000, 5) == (8450 + 8 * 5) * 4


def test_other_argument_errors(lib):
    sh = shape()
    assert lib.dsa_block_sparse_attention(P, P, P, P, ctypes.byref(sh), 0, 0.0, None, 0, P, 1 << 40, None) == INVALID
    assert lib.dsa_block_sparse_attention(P, P, P, P, ctypes.byref(sh), 4, 0.0, None, 0, P, 8, None) == WORKSPACE
    assert lib.dsa_streaming_attention(P, P, P, P, ctypes.byref(sh), -1, 1, 0.0, None, 0, None) == INVALID
    assert lib.dsa_streaming_attention(P, P, P, P, ctypes.byref(sh), 1, 0, 0.0, None, 0, None) == INVALID
    assert lib.dsa_streaming_attention(P, None, P, P, ctypes.byref(sh), 1, 1, 0.0, None, 0, None) == INVALID
    assert lib.dsa_topk(P, 1, 10, -1, -1, P, None, 0, None) == INVALID
    assert lib.dsa_topk(P, 1, 10, 3, 10, P, None, 0, None) == INVALID
    assert lib.dsa_topk(None, 1, 10, 3, -1, P, None, 0, None) == INVALID
    assert lib.dsa_topk(None, 0, 10, 3, -1, None, None, 0, None) == OK
    assert lib.dsa_topk(P, 2, 1 << 20, 1000, -1, P, P, 8, None) == WORKSPACE
    assert lib.dsa_vs_build_index(P, -1, P, 1, 1, 10, P, P, P, P, None) == INVALID
    assert lib.dsa_bs_pool(P, 0, 1, 2, 100, 80, None, 0, P, None) == UNSUPPORTED
    assert lib.dsa_bs_select(P, P, 1, 4, 128, 0.1, 0, P, P, None, P, 1 << 30, None) == INVALID
    assert lib.dsa_bs_select(P, P, 1, 4, 128, 0.1, 2, P, P, None, P, 4, None) == WORKSPACE
    assert lib.dsa_vs_estimate(P, P, ctypes.byref(sh), 64, 0.0, None, 0, P, P, P, 4, None) == WORKSPACE
    assert lib.dsa_sparse_attention_vs(P, P, P, P, ctypes.byref(sh), 0.0, None, 0, P, None, 1, P, P, 1, None) == INVALID
    assert lib.dsa_sparse_attention_blocks(P, P, P, P, ctypes.byref(sh), 0.0, None, 0, P, P, -1, None) == INVALID
    # KV retention: window >= 1, keep >= 0, kept needed when keep > 0, workspace checked
    kv = lambda win, keep, kept=P, ws=P, wsb=1 << 40, q=P: lib.dsa_kv_retention(
        q, P, ctypes.byref(sh), win, keep, 0.0, None, 0, P, kept, ws, wsb, None)
    assert kv(0, 4) == INVALID
    assert kv(64, -1) == INVALID
    assert kv(64, 4, kept=None) == INVALID
    assert kv(64, 4, q=None) == INVALID
    assert kv(64, 4, wsb=8) == WORKSPACE
    assert lib.dsa_kv_retention_workspace_bytes(ctypes.byref(sh), 4, 4) > 0
    assert lib.dsa_kv_retention_workspace_bytes(ctypes.byref(sh), -1, 4) == 0
    # sparse decode: q/k/v/o required, a key list needs its counts and a width >= 0
    dec = lambda keys=None, mk=0, nk=None, wsb=1 << 40, q=P: lib.dsa_sparse_decode(
        q, P, P, P, ctypes.byref(sh), 0.0, None, 0, keys, mk, nk, P, wsb, None)
    assert dec(q=None) == INVALID
    assert dec(keys=P, mk=4, nk=None) == INVALID
    assert dec(keys=P, mk=-1, nk=P) == INVALID
    assert dec(wsb=8) == WORKSPACE
    assert lib.dsa_sparse_decode_workspace_bytes(ctypes.byref(sh), -1, 4) > 0
    assert lib.dsa_sparse_decode_workspace_bytes(ctypes.byref(sh), -2, 4) == 0
    many = (ctypes.c_int32 * 300)(*range(300))
    big = shape(hq=300, hkv=300)
    assert lib.dsa_streaming_attention(P, P, P, P, ctypes.byref(big), 1, 1, 0.0, many, 300, None) == UNSUPPORTED


def test_mixed_argument_errors(lib):
    sh = shape(hq=4, hkv=2)
    pats = lambda *p: (ctypes.c_int32 * len(p))(*p)
    good = pats(0, 1, 2, -1)
    mixed = lambda p=good, vk=8, sk=8, lq=64, tk=4, ib=1, lb=2, wsb=1 << 40, q=P: lib.dsa_mixed_sparse_attention(
        q, P, P, P, ctypes.byref(sh), p, vk, sk, lq, tk, ib, lb, 0.0, P, wsb, None)
    assert mixed(p=None) == INVALID
    assert mixed(p=pats(0, 1, 3, -1)) == INVALID
    assert mixed(p=pats(0, -2, 2, 1)) == INVALID
    assert mixed(q=None) == INVALID
    assert mixed(sk=0) == INVALID
    assert mixed(tk=0) == INVALID
    assert mixed(ib=-1) == INVALID
    assert mixed(lb=0) == INVALID
    assert mixed(lq=65) == UNSUPPORTED
    assert mixed(wsb=8) == WORKSPACE
    # no head processed, or no tokens: nothing to enqueue
    assert mixed(p=pats(-1, -1, -1, -1), wsb=0) == OK
    empty = shape(hq=4, hkv=2, n=0)
    assert lib.dsa_mixed_sparse_attention(P, P, P, P, ctypes.byref(empty), good, 8, 8, 64, 4, 1, 2, 0.0,
                                          None, 0, None) == OK
    # workspace: the VS part for the VS heads plus the BS part for the BS heads
    big = shape(hq=4, hkv=2, n=4096)
    wm = lib.dsa_mixed_sparse_attention_workspace_bytes
    vs1 = lib.dsa_vertical_slash_workspace_bytes(ctypes.byref(big), 64, 64, 1)
    bs2 = lib.dsa_block_sparse_workspace_bytes(ctypes.byref(big), 8, 2)
    assert wm(ctypes.byref(big), pats(0, 1, 1, 2), 64, 64, 8) == vs1 + bs2
    assert wm(ctypes.byref(big), pats(2, 2, -1, 2), 64, 64, 8) == 0
    assert wm(ctypes.byref(big), pats(2, 2, 5, 2), 64, 64, 8) == 0
    assert wm(ctypes.byref(big), None, 64, 64, 8) == 0
    # the stage call: index pointers required only for patterns some head follows
    stage = lambda p, iv=P, niv=P, cols=P, ncols=P, sel=P, nsel=P: lib.dsa_sparse_attention_mixed(
        P, P, P, P, ctypes.byref(sh), 0.0, p, iv, niv, 4, cols, ncols, 4, sel, nsel, 4, 1, 2, None)
    assert stage(good, niv=None) == INVALID
    assert stage(good, nsel=None) == INVALID
    assert stage(pats(-1, -1, -1, -1), None, None, None, None, None, None) == OK
    assert stage(pats(0, 1, 9, -1)) == INVALID


# ---- the binding refuses index arrays whose extents do not match the call ----
# (meta tensors: the extents are checked before any pointer is taken, so these
# run without a GPU; a correct call gets as far as the GPU-tensor check)
def _meta(*shape, dtype=None):
    import torch
    return torch.empty(shape, dtype=dtype or torch.bfloat16, device="meta")


def test_binding_rejects_mismatched_vs_index():
    import torch
    i32 = torch.int32
    q, k, v = _meta(2, 4, 300, 64), _meta(2, 2, 300, 64), _meta(2, 2, 300, 64)
    nb = 5
    good = dict(intervals=_meta(8, 6, 2, dtype=i32), n_intervals=_meta(8, dtype=i32),
                cols=_meta(8, nb, 7, dtype=i32), n_cols=_meta(8, nb, dtype=i32))
    with pytest.raises(ValueError, match="GPU tensor"):
        dsa.sparse_attention_vs(q, k, v, **good)
    bad = [("intervals", _meta(6, 6, 2, dtype=i32)),     # rows for another head list
           ("intervals", _meta(8, 6, 3, dtype=i32)),
           ("n_intervals", _meta(7, dtype=i32)),
           ("cols", _meta(8, nb + 1, 7, dtype=i32)),     # index of another seq_len
           ("n_cols", _meta(8, nb - 1, dtype=i32))]
    for name, t in bad:
        args = dict(good, **{name: t})
        with pytest.raises(ValueError, match="must have shape"):
            dsa.sparse_attention_vs(q, k, v, **args)
    # with a head subset the rows are batch * len(heads)
    sub = dict(intervals=_meta(2, 6, 2, dtype=i32), n_intervals=_meta(2, dtype=i32),
               cols=_meta(2, nb, 7, dtype=i32), n_cols=_meta(2, nb, dtype=i32))
    with pytest.raises(ValueError, match="GPU tensor"):
        dsa.sparse_attention_vs(q, k, v, heads=[3], **sub)
    with pytest.raises(ValueError, match="must have shape"):
        dsa.sparse_attention_vs(q, k, v, heads=[1, 3], **sub)


def test_binding_rejects_mismatched_block_lists():
    import torch
    i32 = torch.int32
    q, k, v = _meta(1, 4, 200, 128), _meta(1, 1, 200, 128), _meta(1, 1, 200, 128)
    with pytest.raises(ValueError, match="GPU tensor"):
        dsa.sparse_attention_blocks(q, k, v, _meta(4, 4, 3, dtype=i32), _meta(4, 4, dtype=i32))
    for sel, n_sel in ((_meta(4, 3, 3, dtype=i32), _meta(4, 4, dtype=i32)),
                       (_meta(5, 4, 3, dtype=i32), _meta(4, 4, dtype=i32)),
                       (_meta(4, 4, 3, dtype=i32), _meta(4, 3, dtype=i32))):
        with pytest.raises(ValueError, match="must have shape"):
            dsa.sparse_attention_blocks(q, k, v, sel, n_sel)
    # the one-launch call checks each pattern's index against that pattern's heads
    pats = ["vs", "bs", "st", None]
    vs_ix = (_meta(1, 4, 2, dtype=i32), _meta(1, dtype=i32), _meta(1, 4, 5, dtype=i32), _meta(1, 4, dtype=i32))
    bs_ix = (_meta(1, 4, 3, dtype=i32), _meta(1, 4, dtype=i32))
    with pytest.raises(ValueError, match="GPU tensor"):
        dsa.sparse_attention_mixed(q, k, v, pats, vs_index=vs_ix, bs_index=bs_ix)
    with pytest.raises(ValueError, match="must have shape"):
        dsa.sparse_attention_mixed(q, k, v, pats, vs_index=vs_ix, bs_index=(_meta(2, 4, 3, dtype=i32),
                                                                            _meta(2, 4, dtype=i32)))
    with pytest.raises(ValueError, match="required"):
        dsa.sparse_attention_mixed(q, k, v, pats, vs_index=vs_ix)


def test_binding_rejects_mismatched_q_k():
    q = _meta(1, 4, 256, 64)
    for k in (_meta(2, 2, 256, 64), _meta(1, 2, 255, 64), _meta(1, 2, 256, 128)):
        with pytest.raises(ValueError, match="shape mismatch"):
            dsa.vs_estimate(q, k)
        with pytest.raises(ValueError, match="shape mismatch"):
            dsa.kv_retention(q, k, 64, 8)
    with pytest.raises(ValueError, match="batch and head_dim"):
        dsa.sparse_decode(_meta(1, 4, 128), _meta(1, 2, 256, 64), _meta(1, 2, 256, 64))


def test_empty_work_accepts_null_pointers(lib):
    """batch 0 or seq_len 0: nothing is read, so NULL data pointers are fine
    (zero-size tensors have no address); scalar arguments are still checked."""
    for sh in (shape(b=0), shape(n=0)):
        s = ctypes.byref(sh)
        assert lib.dsa_vertical_slash_sparse_attention(None, None, None, None, s, 8, 8, 64, 0.0, None, 0,
                                                       None, 0, None) == OK
        assert lib.dsa_vertical_slash_sparse_attention(None, None, None, None, s, 8, 0, 64, 0.0, None, 0,
                                                       None, 0, None) == INVALID
        assert lib.dsa_block_sparse_attention(None, None, None, None, s, 4, 0.0, None, 0, None, 0, None) == OK
        assert lib.dsa_streaming_attention(None, None, None, None, s, 1, 2, 0.0, None, 0, None) == OK
        assert lib.dsa_streaming_attention(None, None, None, None, s, 1, 0, 0.0, None, 0, None) == INVALID
        assert lib.dsa_vs_estimate(None, None, s, 64, 0.0, None, 0, None, None, None, 0, None) == OK
        assert lib.dsa_kv_retention(None, None, s, 64, 8, 0.0, None, 0, None, None, None, 0, None) == OK
        assert lib.dsa_sparse_attention_vs(None, None, None, None, s, 0.0, None, 0, None, None, 0, None, None,
                                           0, None) == OK
        assert lib.dsa_sparse_attention_blocks(None, None, None, None, s, 0.0, None, 0, None, None, 0,
                                               None) == OK
        pats = (ctypes.c_int32 * 4)(0, 1, 2, -1)
        assert lib.dsa_mixed_sparse_attention(None, None, None, None, s, pats, 8, 8, 64, 4, 1, 2, 0.0, None,
                                              0, None) == OK
        assert lib.dsa_sparse_attention_mixed(None, None, None, None, s, 0.0, pats, None, None, 0, None, None,
                                              0, None, None, 0, 1, 2, None) == OK
    assert lib.dsa_bs_pool(None, 0, 0, 2, 100, 64, None, 0, None, None) == OK
    assert lib.dsa_bs_pool(None, 0, 1, 2, 0, 64, None, 0, None, None) == OK
    assert lib.dsa_sparse_decode(None, None, None, None, ctypes.byref(shape(b=0)), 0.0, None, 0, None, 0,
                                 None, None, 0, None) == OK


def test_noalloc_decode_argument_errors(lib):
    """The allocation-free decode refuses, on the host, a call whose split
    partials exceed its static scratch (no HIP call is made)."""
    need = lib.dsa_sparse_decode_workspace_bytes(ctypes.byref(shape(b=200, hq=256, hkv=256, n=64)), -1, 256)
    assert need > 16 << 20
    big = shape(b=200, hq=256, hkv=256, n=64)
    assert lib.dsa_sparse_decode_noalloc(P, P, P, P, ctypes.byref(big), 0.0, None, 0, None, 0, None,
                                         None) == WORKSPACE
    sh = shape()
    assert lib.dsa_sparse_decode_noalloc(None, P, P, P, ctypes.byref(sh), 0.0, None, 0, None, 0, None,
                                         None) == INVALID
    assert lib.dsa_sparse_decode_noalloc(P, P, P, P, ctypes.byref(sh), 0.0, None, 0, P, -1, P, None) == INVALID
    assert lib.dsa_sparse_decode_noalloc(None, None, None, None, ctypes.byref(shape(b=0)), 0.0, None, 0, None,
                                         0, None, None) == OK


def stages(*pairs):
    return B._stages(list(pairs))


def prune_call(lib, sh, st, units=0, unit_rows=0, qd=0, qu=P, sel=P):
    # units = 0 by default: every check runs, and a call that passes them has
    # no work, so nothing is launched
    return lib.dsa_hier_prune(qu, qd, units, unit_rows, P, ctypes.byref(sh), ctypes.byref(st), 0.0, None, 0,
                              P, sel, P, None, 0, None)


def test_prune_stage_checks(lib):
    """Stage lists are checked on the host: lengths multiples of 64, strictly
    decreasing and nested, keep >= 1, at most 4 stages; candidate counts
    capped at 4096 (unsupported beyond). No call here launches anything."""
    sh = shape(n=1 << 20)
    assert prune_call(lib, sh, stages((4096, 16), (512, 32), (64, 64))) == OK
    assert prune_call(lib, sh, stages((4096, 16), (1000, 4))) == INVALID      # not a multiple of 64
    assert prune_call(lib, sh, stages((512, 4), (512, 4))) == INVALID         # not decreasing
    assert prune_call(lib, sh, stages((512, 4), (192, 4))) == INVALID         # does not divide
    assert prune_call(lib, sh, stages((512, 0))) == INVALID                   # keep 0
    assert prune_call(lib, sh, stages((32, 4))) == INVALID                    # below 64
    st = stages((4096, 1))
    st.n_stages = 5
    assert prune_call(lib, sh, st) == INVALID
    st.n_stages = 0
    assert prune_call(lib, sh, st) == INVALID
    assert prune_call(lib, sh, stages((128, 4))) == UNSUPPORTED               # 8192 stage-1 candidates
    assert prune_call(lib, sh, stages((4096, 100), (64, 10))) == UNSUPPORTED  # 6400 stage-2 candidates
    assert prune_call(lib, sh, stages((4096, 4)), qd=5) == UNSUPPORTED
    assert prune_call(lib, sh, stages((4096, 4)), units=1, qu=None) == INVALID
    assert prune_call(lib, sh, stages((4096, 4)), units=1, sel=None) == INVALID
    assert prune_call(lib, sh, stages((4096, 4)), units=-1) == INVALID
    assert prune_call(lib, sh, stages((4096, 4)), unit_rows=-1) == INVALID
    assert prune_call(lib, sh, stages((4096, 4)), qu=None, sel=None) == OK   # no unit: nothing to do
    assert lib.dsa_hier_prune(P, 0, 1, 0, P, ctypes.byref(sh), None, 0.0, None, 0, P, P, P, None, 0, None) == INVALID
    # no block_max output and too small a workspace
    assert lib.dsa_hier_prune(P, 0, 1, 0, P, ctypes.byref(sh), ctypes.byref(stages((4096, 4))), 0.0, None, 0,
                              None, P, P, P, 16, None) == WORKSPACE


def test_prune_composite_calls_checks(lib):
    sh = shape(n=5000)
    st = stages((1024, 2), (64, 8))
    assert lib.dsa_hier_sparse_decode_workspace_bytes(ctypes.byref(sh), ctypes.byref(st), 4) > 0
    assert lib.dsa_hier_block_sparse_workspace_bytes(ctypes.byref(sh), ctypes.byref(st), 4) > 0
    assert lib.dsa_hier_sparse_decode_workspace_bytes(ctypes.byref(sh), None, 4) == 0
    assert lib.dsa_hier_sparse_decode(P, P, P, P, ctypes.byref(sh), ctypes.byref(st), 0.0, None, 0, P, 8,
                                      None) == WORKSPACE
    assert lib.dsa_hier_sparse_decode(None, P, P, P, ctypes.byref(sh), ctypes.byref(st), 0.0, None, 0, P,
                                      1 << 40, None) == INVALID
    # the prefill form needs 64-key blocks at the last stage
    st2 = stages((1024, 2), (128, 8))
    assert lib.dsa_hier_block_sparse_attention(P, P, P, P, ctypes.byref(sh), ctypes.byref(st2), 0.0, None, 0,
                                               P, 1 << 40, None) == INVALID
    assert lib.dsa_hier_block_sparse_attention(P, P, P, P, ctypes.byref(shape(b=0)), ctypes.byref(st), 0.0,
                                               None, 0, None, 0, None) == OK
    assert lib.dsa_chunks_to_keys(P, P, 4, 8, 0, 100, P, P, None) == INVALID
    assert lib.dsa_chunks_to_keys(P, P, 0, 8, 64, 100, P, P, None) == OK
    assert lib.dsa_chunks_to_keys(None, P, 4, 8, 64, 100, P, P, None) == INVALID
