"""ctypes binding of libdsa.so (include/dsa.h).

Argument marshalling only: tensors are checked for device, dtype and layout,
turned into raw pointers, and handed to the library together with torch's
current HIP stream. Every step of the computation runs in the library's
kernels. When the library is missing, import succeeds but every call raises
``RuntimeError``: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdsa.so")
BLOCK = 64
MAX_HEADS = 256

BF16, F32 = 0, 1
_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace too small", 4: "HIP error"}

_lib: Optional[ctypes.CDLL] = None
_load_error: Optional[str] = None


class DsaError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} failed: {_STATUS.get(code, code)} (status {code})")
        self.code = code


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("q_heads", ctypes.c_int32),
                ("kv_heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32)]


PRUNE_MAX_STAGES = 4


class PruneStages(ctypes.Structure):
    _fields_ = [("n_stages", ctypes.c_int32), ("chunk", ctypes.c_int32 * PRUNE_MAX_STAGES),
                ("keep", ctypes.c_int32 * PRUNE_MAX_STAGES)]


_vp, _i32, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
_ip = ctypes.POINTER(ctypes.c_int32)
_SIGS = {
    "dsa_status_string": ([_i32], ctypes.c_char_p),
    "dsa_vertical_slash_sparse_attention": ([_vp, _vp, _vp, _vp, ctypes.POINTER(Shape), _i32, _i32, _i32, _f32, _ip, _i32, _vp, _sz, _vp], _i32),
    "dsa_vertical_slash_workspace_bytes": ([ctypes.POINTER(Shape), _i32, _i32, _i32], _sz),
    "dsa_block_sparse_attention": ([_vp, _vp, _vp, _vp, ctypes.POINTER(Shape), _i32, _f32, _ip, _i32, _vp, _sz, _vp], _i32),
    "dsa_block_sparse_workspace_bytes": ([ctypes.POINTER(Shape), _i32, _i32], _sz),
    "dsa_streaming_attention": ([_vp, _vp, _vp, _vp, ctypes.POINTER(Shape), _i32, _i32, _f32, _ip, _i32, _vp], _i32),
    "dsa_vs_estimate": ([_vp, _vp, ctypes.POINTER(Shape), _i32, _f32, _ip, _i32, _vp, _vp, _vp, _sz, _vp], _i32),
    "dsa_vs_estimate_workspace_bytes": ([ctypes.POINTER(Shape), _i32], _sz),
    "dsa_kv_retention": ([_vp, _vp, ctypes.POINTER(Shape), _i32, _i32, _f32, _ip, _i32, _vp, _vp, _vp, _sz, _vp], _i32),
    "dsa_kv_retention_workspace_bytes": ([ctypes.POINTER(Shape), _i32, _i32], _sz),
    "dsa_sparse_decode": ([_vp, _vp, _vp, _vp, ctypes.POINTER(Shape), _f32, _ip, _i32, _vp, _i32, _vp, _vp, _sz, _vp], _i32),
    "dsa_sparse_decode_workspace_bytes": ([ctypes.POINTER(Shape), _i32, _i32], _sz),
    "dsa_sparse_decode_noalloc": ([_vp, _vp, _vp, _vp, ctypes.POINTER(Shape), _f32, _ip, _i32, _vp, _i32, _vp, _vp], _i32),
    "dsa_topk": ([_vp, _i32, _i32, _i32, _i32, _vp, _vp, _sz, _vp], _i32),
    "dsa_topk_workspace_bytes": ([_i32, _i32, _i32], _sz),
    "dsa_vs_build_index": ([_vp, _i32, _vp, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp], _i32),
    "dsa_bs_pool": ([_vp, _i32, _i32, _i32, _i32, _i32, _ip, _i32, _vp, _vp], _i32),
    "dsa_bs_select": ([_vp, _vp, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _vp, _vp, _sz, _vp], _i32),
    "dsa_bs_select_workspace_bytes": ([_i32, _i32], _sz),
    "dsa_sparse_attention_vs": ([_vp, _vp, _vp, _vp, ctypes.POINTER(Shape), _f32, _ip, _i32, _vp, _vp, _i32, _vp, _vp, _i32, _vp], _i32),
    "dsa_sparse_attention_blocks": ([_vp, _vp, _vp, _vp, ctypes.POINTER(Shape), _f32, _ip, _i32, _vp, _vp, _i32, _vp], _i32),
    "dsa_mixed_sparse_attention": ([_vp, _vp, _vp, _vp, ctypes.POINTER(Shape), _ip, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _vp, _sz, _vp], _i32),
    "dsa_mixed_sparse_attention_workspace_bytes": ([ctypes.POINTER(Shape), _ip, _i32, _i32, _i32], _sz),
    "dsa_sparse_attention_mixed": ([_vp, _vp, _vp, _vp, ctypes.POINTER(Shape), _f32, _ip, _vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _vp], _i32),
    "dsa_hier_prune": ([_vp, _i32, _i32, _i32, _vp, ctypes.POINTER(Shape), ctypes.POINTER(PruneStages), _f32, _ip, _i32, _vp, _vp, _vp, _vp, _sz, _vp], _i32),
    "dsa_hier_prune_workspace_bytes": ([ctypes.POINTER(Shape), _i32, _i32], _sz),
    "dsa_chunks_to_keys": ([_vp, _vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp], _i32),
    "dsa_hier_sparse_decode": ([_vp, _vp, _vp, _vp, ctypes.POINTER(Shape), ctypes.POINTER(PruneStages), _f32, _ip, _i32, _vp, _sz, _vp], _i32),
    "dsa_hier_sparse_decode_workspace_bytes": ([ctypes.POINTER(Shape), ctypes.POINTER(PruneStages), _i32], _sz),
    "dsa_hier_block_sparse_attention": ([_vp, _vp, _vp, _vp, ctypes.POINTER(Shape), ctypes.POINTER(PruneStages), _f32, _ip, _i32, _vp, _sz, _vp], _i32),
    "dsa_hier_block_sparse_workspace_bytes": ([ctypes.POINTER(Shape), ctypes.POINTER(PruneStages), _i32], _sz),
}
EXPORTED = tuple(_SIGS)


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdsa.so (once) and attach the C signatures."""
    global _lib, _load_error
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        _load_error = f"{path} is not built (run dynamic_sparse_attention_slash_amd.build)"
        raise RuntimeError(_load_error)
    lib = ctypes.CDLL(path)
    for name, (args, res) in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _call(name: str, *args) -> None:
    code = getattr(load(), name)(*args)
    if code != 0:
        raise DsaError(name, code)


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------
def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype} (bf16 or fp32)")


def _dev(t: torch.Tensor, name: str, dtype=None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _shape_qkv(q, k, v) -> Shape:
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [batch, heads, seq_len, head_dim]")
    if k.shape != v.shape or q.shape[0] != k.shape[0] or q.shape[2:] != k.shape[2:]:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k, v must share one dtype")
    B, Hq, n, D = q.shape
    return Shape(B, Hq, k.shape[1], n, D, _dtype_code(q))


def _expect(name: str, t: torch.Tensor, shape: Tuple[int, ...]) -> None:
    """The kernels read an index array as [rows, ...] of the call's extents
    with no bound of their own: an array of any other shape is refused here."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _check_qk(q: torch.Tensor, k: torch.Tensor) -> None:
    """q [B, Hq, n, D] and k [B, Hkv, n, D] with equal batch, seq_len and head_dim."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k must be [batch, heads, seq_len, head_dim]")
    if q.shape[0] != k.shape[0] or q.shape[2:] != k.shape[2:]:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)}")
    if q.dtype != k.dtype:
        raise TypeError("q and k must share one dtype")


def _index_rows(sh: Shape, heads: Optional[Sequence[int]]) -> Tuple[int, int]:
    """(rows, nb) of an explicit-index call: rows = batch * listed heads."""
    nh = sh.q_heads if heads is None else len(heads)
    return sh.batch * nh, (sh.seq_len + BLOCK - 1) // BLOCK


def check_vs_index(sh: Shape, heads, intervals, n_intervals, cols, n_cols) -> None:
    """Extents of a vertical-slash index for the call's rows: intervals
    [rows, max_iv, 2], n_intervals [rows], cols [rows, nb, max_cols], n_cols
    [rows, nb]."""
    rows, nb = _index_rows(sh, heads)
    if intervals.dim() != 3 or cols.dim() != 3:
        raise ValueError("intervals must be [rows, max_iv, 2] and cols [rows, nb, max_cols]")
    _expect("intervals", intervals, (rows, intervals.shape[1], 2))
    _expect("n_intervals", n_intervals, (rows,))
    _expect("cols", cols, (rows, nb, cols.shape[2]))
    _expect("n_cols", n_cols, (rows, nb))


def check_block_index(sh: Shape, heads, sel, n_sel) -> None:
    """Extents of block lists for the call's rows: sel [rows, nb, max_sel],
    n_sel [rows, nb]."""
    rows, nb = _index_rows(sh, heads)
    if sel.dim() != 3:
        raise ValueError("sel must be [rows, nb, max_sel]")
    _expect("sel", sel, (rows, nb, sel.shape[2]))
    _expect("n_sel", n_sel, (rows, nb))


def _heads(heads: Optional[Sequence[int]]) -> Tuple[Optional[ctypes.Array], int]:
    if heads is None:
        return None, 0
    arr = (ctypes.c_int32 * max(1, len(heads)))(*[int(h) for h in heads])
    return arr, len(heads)


def _scale(scale: Optional[float]) -> float:
    return 0.0 if scale is None else float(scale)


def _workspace(nbytes: int, device, given: Optional[torch.Tensor] = None) -> torch.Tensor:
    """A caller-supplied uint8 workspace when it is large enough, else a new one."""
    if given is not None:
        if given.dtype != torch.uint8 or not given.is_cuda or given.numel() < nbytes:
            raise ValueError(f"workspace must be a uint8 GPU tensor of >= {nbytes} bytes")
        return given
    return torch.empty(max(1, int(nbytes)), dtype=torch.uint8, device=device)


def vertical_slash_workspace_bytes(q, k, vertical_topk: int, slash_topk: int,
                                   heads: Optional[Sequence[int]] = None) -> int:
    sh = Shape(q.shape[0], q.shape[1], k.shape[1], q.shape[2], q.shape[3], _dtype_code(q))
    nh = sh.q_heads if heads is None else len(heads)
    return int(load().dsa_vertical_slash_workspace_bytes(ctypes.byref(sh), vertical_topk, slash_topk, nh))


def block_sparse_workspace_bytes(q, k, topk: int, heads: Optional[Sequence[int]] = None) -> int:
    sh = Shape(q.shape[0], q.shape[1], k.shape[1], q.shape[2], q.shape[3], _dtype_code(q))
    nh = sh.q_heads if heads is None else len(heads)
    return int(load().dsa_block_sparse_workspace_bytes(ctypes.byref(sh), topk, nh))


def _out_like(q: torch.Tensor, out: Optional[torch.Tensor]) -> torch.Tensor:
    if out is None:
        return torch.zeros_like(q)
    if out.shape != q.shape or out.dtype != q.dtype or out.device != q.device:
        raise ValueError("out must match q")
    return out


# ----------------------------------------------------------------------------
# the three calls of the kernel-only API
# ----------------------------------------------------------------------------
def vertical_slash_sparse_attention(q, k, v, vertical_topk: int, slash_topk: int, *,
                                    last_q: int = 64, scale: Optional[float] = None,
                                    heads: Optional[Sequence[int]] = None,
                                    out: Optional[torch.Tensor] = None,
                                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    sh = _shape_qkv(q, k, v)
    o = _out_like(q, out)
    ha, hn = _heads(heads)
    nh = sh.q_heads if heads is None else hn
    ws = _workspace(load().dsa_vertical_slash_workspace_bytes(ctypes.byref(sh), vertical_topk,
                                                              slash_topk, nh), q.device, workspace)
    _call("dsa_vertical_slash_sparse_attention", _dev(q, "q"), _dev(k, "k"), _dev(v, "v"),
          _dev(o, "out"), ctypes.byref(sh), vertical_topk, slash_topk, last_q, _scale(scale),
          ha, hn, ws.data_ptr(), ws.numel(), _stream(q))
    return o


def block_sparse_attention(q, k, v, topk: int, *, scale: Optional[float] = None,
                           heads: Optional[Sequence[int]] = None,
                           out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    sh = _shape_qkv(q, k, v)
    o = _out_like(q, out)
    ha, hn = _heads(heads)
    nh = sh.q_heads if heads is None else hn
    ws = _workspace(load().dsa_block_sparse_workspace_bytes(ctypes.byref(sh), topk, nh), q.device,
                    workspace)
    _call("dsa_block_sparse_attention", _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "out"),
          ctypes.byref(sh), topk, _scale(scale), ha, hn, ws.data_ptr(), ws.numel(), _stream(q))
    return o


def streaming_attention(q, k, v, init_blocks: int, local_blocks: int, *,
                        scale: Optional[float] = None, heads: Optional[Sequence[int]] = None,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    sh = _shape_qkv(q, k, v)
    o = _out_like(q, out)
    ha, hn = _heads(heads)
    _call("dsa_streaming_attention", _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "out"),
          ctypes.byref(sh), init_blocks, local_blocks, _scale(scale), ha, hn, _stream(q))
    return o


PATTERN_CODES = {None: -1, "vs": 0, "bs": 1, "st": 2}


def _patterns(patterns: Sequence[Optional[str]], q_heads: int) -> ctypes.Array:
    """Per-query-head pattern names ("vs", "bs", "st" or None) -> int32 array."""
    if len(patterns) != q_heads:
        raise ValueError(f"patterns must name one pattern per query head ({q_heads})")
    try:
        codes = [PATTERN_CODES[p] for p in patterns]
    except KeyError as e:
        raise ValueError(f"unknown pattern {e.args[0]!r}; use 'vs', 'bs', 'st' or None") from None
    return (ctypes.c_int32 * q_heads)(*codes)


def mixed_workspace_bytes(q, k, patterns: Sequence[Optional[str]], vertical_topk: int,
                          slash_topk: int, topk: int) -> int:
    sh = Shape(q.shape[0], q.shape[1], k.shape[1], q.shape[2], q.shape[3], _dtype_code(q))
    return int(load().dsa_mixed_sparse_attention_workspace_bytes(
        ctypes.byref(sh), _patterns(patterns, sh.q_heads), vertical_topk, slash_topk, topk))


def mixed_sparse_attention(q, k, v, patterns: Sequence[Optional[str]], *, vertical_topk: int,
                           slash_topk: int, topk: int, init_blocks: int, local_blocks: int,
                           last_q: int = 64, scale: Optional[float] = None,
                           out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """A layer whose query head h follows patterns[h]; every head's attention
    runs in one launch (heads with pattern None are left untouched in out)."""
    sh = _shape_qkv(q, k, v)
    o = _out_like(q, out)
    pa = _patterns(patterns, sh.q_heads)
    ws = _workspace(load().dsa_mixed_sparse_attention_workspace_bytes(
        ctypes.byref(sh), pa, vertical_topk, slash_topk, topk), q.device, workspace)
    _call("dsa_mixed_sparse_attention", _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "out"),
          ctypes.byref(sh), pa, vertical_topk, slash_topk, last_q, topk, init_blocks, local_blocks,
          _scale(scale), ws.data_ptr(), ws.numel(), _stream(q))
    return o


# ----------------------------------------------------------------------------
# stage calls
# ----------------------------------------------------------------------------
def vs_estimate(q, k, *, last_q: int = 64, scale: Optional[float] = None,
                heads: Optional[Sequence[int]] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Vertical and slash scores, fp32 [batch * n_heads, seq_len] each."""
    _check_qk(q, k)
    B, Hq, n, D = q.shape
    sh = Shape(B, Hq, k.shape[1], n, D, _dtype_code(q))
    ha, hn = _heads(heads)
    nh = Hq if heads is None else hn
    rows = B * nh
    vsc = torch.empty((rows, n), dtype=torch.float32, device=q.device)
    ssc = torch.empty((rows, n), dtype=torch.float32, device=q.device)
    ws = _workspace(load().dsa_vs_estimate_workspace_bytes(ctypes.byref(sh), nh), q.device)
    _call("dsa_vs_estimate", _dev(q, "q"), _dev(k, "k", q.dtype), ctypes.byref(sh), last_q,
          _scale(scale), ha, hn, vsc.data_ptr(), ssc.data_ptr(), ws.data_ptr(), ws.numel(), _stream(q))
    return vsc, ssc


def kv_retention(q, k, window: int, keep: int, *, scale: Optional[float] = None,
                 heads: Optional[Sequence[int]] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """KV-retention scores fp32 [batch * n_heads, seq_len] (softmax mass of each
    key over the last `window` query rows) and the kept keys int32
    [batch * n_heads, min(keep, seq_len)], ascending."""
    _check_qk(q, k)
    B, Hq, n, D = q.shape
    sh = Shape(B, Hq, k.shape[1], n, D, _dtype_code(q))
    ha, hn = _heads(heads)
    nh = Hq if heads is None else hn
    rows = B * nh
    scores = torch.empty((rows, n), dtype=torch.float32, device=q.device)
    kept = torch.empty((rows, max(0, min(keep, n))), dtype=torch.int32, device=q.device)
    ws = _workspace(load().dsa_kv_retention_workspace_bytes(ctypes.byref(sh), keep, nh), q.device)
    _call("dsa_kv_retention", _dev(q, "q"), _dev(k, "k", q.dtype), ctypes.byref(sh), window, keep,
          _scale(scale), ha, hn, scores.data_ptr(), kept.data_ptr() if kept.numel() else None,
          ws.data_ptr(), ws.numel(), _stream(q))
    return scores, kept


def sparse_decode(q, k, v, keys: Optional[torch.Tensor] = None, n_keys: Optional[torch.Tensor] = None, *,
                  scale: Optional[float] = None, heads: Optional[Sequence[int]] = None,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode attention of one new row per head over cached keys: q [batch,
    q_heads, head_dim] (or [batch, q_heads, 1, head_dim]), k, v the cache
    [batch, kv_heads, seq_len, head_dim]; keys int32 [batch * n_heads,
    max_keys] with counts n_keys [batch * n_heads], or None for the whole
    cache. Returns o shaped like q (listed heads written)."""
    return _decode(q, k, v, keys, n_keys, scale, heads, out, False)


def sparse_decode_noalloc(q, k, v, keys: Optional[torch.Tensor] = None,
                          n_keys: Optional[torch.Tensor] = None, *, scale: Optional[float] = None,
                          heads: Optional[Sequence[int]] = None,
                          out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """sparse_decode through the allocation-free entry point (split partials in
    the library's static device scratch, no workspace). Pass `out` to keep the
    call free of allocations on this side too."""
    return _decode(q, k, v, keys, n_keys, scale, heads, out, True)


def _decode(q, k, v, keys, n_keys, scale, heads, out, noalloc: bool) -> torch.Tensor:
    if k.dim() != 4 or v.shape != k.shape:
        raise ValueError("k, v must be [batch, kv_heads, seq_len, head_dim]")
    B, Hkv, n, D = k.shape
    if q.dim() == 4:
        if q.shape[2] != 1:
            raise ValueError("decode takes one query row per head")
    elif q.dim() != 3:
        raise ValueError("q must be [batch, q_heads, head_dim]")
    if q.shape[0] != B or q.shape[-1] != D:
        raise ValueError(f"q{tuple(q.shape)} must match the cache's batch and head_dim {tuple(k.shape)}")
    Hq = q.shape[1]
    sh = Shape(B, Hq, Hkv, n, D, _dtype_code(q))
    ha, hn = _heads(heads)
    nh = Hq if heads is None else hn
    o = torch.zeros_like(q) if out is None else out
    if keys is not None:
        if keys.dtype != torch.int32 or n_keys is None or n_keys.dtype != torch.int32:
            raise ValueError("keys and n_keys must be int32 tensors")
        if keys.dim() != 2 or keys.shape[0] != B * nh or n_keys.numel() != B * nh:
            raise ValueError("keys must be [batch * n_heads, max_keys], n_keys [batch * n_heads]")
        kp, mk, nkp = _dev(keys, "keys"), keys.shape[1], _dev(n_keys, "n_keys")
    else:
        kp, mk, nkp = None, -1, None
    if noalloc:
        _call("dsa_sparse_decode_noalloc", _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype),
              _dev(o, "out"), ctypes.byref(sh), _scale(scale), ha, hn, kp, max(mk, 0), nkp, _stream(q))
        return o
    ws = _workspace(load().dsa_sparse_decode_workspace_bytes(ctypes.byref(sh), mk, nh), q.device)
    _call("dsa_sparse_decode", _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype), _dev(o, "out"),
          ctypes.byref(sh), _scale(scale), ha, hn, kp, max(mk, 0), nkp, ws.data_ptr(), ws.numel(),
          _stream(q))
    return o


def topk(scores: torch.Tensor, k: int, forced_index: int = -1) -> torch.Tensor:
    """Row-wise top-k of fp32 [rows, n] -> int32 [rows, min(k, n)], ascending."""
    rows, n = scores.shape
    kk = min(k, n)
    out = torch.empty((rows, kk), dtype=torch.int32, device=scores.device)
    ws = _workspace(load().dsa_topk_workspace_bytes(rows, n, k), scores.device)
    _call("dsa_topk", _dev(scores, "scores", torch.float32), rows, n, k, forced_index,
          out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(scores))
    return out


def vs_build_index(V: torch.Tensor, S: torch.Tensor, seq_len: int):
    """(intervals [rows, ns, 2], n_intervals [rows], cols [rows, nb, nv], n_cols [rows, nb]);
    entries past the counts are left unwritten."""
    rows, nv = V.shape
    ns = S.shape[1]
    nb = (seq_len + BLOCK - 1) // BLOCK
    dev = V.device
    iv = torch.empty((rows, ns, 2), dtype=torch.int32, device=dev)
    n_iv = torch.empty((rows,), dtype=torch.int32, device=dev)
    cols = torch.empty((rows, nb, nv), dtype=torch.int32, device=dev)
    n_cols = torch.empty((rows, nb), dtype=torch.int32, device=dev)
    _call("dsa_vs_build_index", _dev(V, "V", torch.int32), nv, _dev(S, "S", torch.int32), ns, rows,
          seq_len, iv.data_ptr(), n_iv.data_ptr(), cols.data_ptr(), n_cols.data_ptr(), _stream(V))
    return iv, n_iv, cols, n_cols


def bs_pool(x: torch.Tensor, heads: Optional[Sequence[int]] = None) -> torch.Tensor:
    """Block means of x [B, H, n, D] -> fp32 [B * n_heads, nb, D]."""
    B, H, n, D = x.shape
    ha, hn = _heads(heads)
    rows = B * (H if heads is None else hn)
    nb = (n + BLOCK - 1) // BLOCK
    out = torch.empty((rows, nb, D), dtype=torch.float32, device=x.device)
    _call("dsa_bs_pool", _dev(x, "x"), _dtype_code(x), B, H, n, D, ha, hn, out.data_ptr(), _stream(x))
    return out


def bs_select(qp: torch.Tensor, kp: torch.Tensor, topk: int, *, scale: Optional[float] = None,
              return_logits: bool = False):
    """(sel [rows, nb, min(topk, nb)], n_sel [rows, nb][, logits [rows, nb, nb]]); entries of
    sel past n_sel are left unwritten."""
    rows, nb, D = qp.shape
    if kp.shape != qp.shape:
        raise ValueError("qp and kp must have equal shapes")
    ke = min(topk, nb)
    sel = torch.empty((rows, nb, ke), dtype=torch.int32, device=qp.device)
    n_sel = torch.empty((rows, nb), dtype=torch.int32, device=qp.device)
    ws = _workspace(load().dsa_bs_select_workspace_bytes(rows, nb), qp.device)
    if return_logits:
        lg = torch.full((rows, nb, nb), float("nan"), dtype=torch.float32, device=qp.device)
        _call("dsa_bs_select", _dev(qp, "qp", torch.float32), _dev(kp, "kp", torch.float32), rows, nb, D,
              _scale(scale), topk, sel.data_ptr(), n_sel.data_ptr(), lg.data_ptr(), ws.data_ptr(), ws.numel(),
              _stream(qp))
        return sel, n_sel, lg
    _call("dsa_bs_select", _dev(qp, "qp", torch.float32), _dev(kp, "kp", torch.float32), rows, nb, D,
          _scale(scale), topk, sel.data_ptr(), n_sel.data_ptr(), None, ws.data_ptr(), ws.numel(), _stream(qp))
    return sel, n_sel


def sparse_attention_vs(q, k, v, intervals, n_intervals, cols, n_cols, *,
                        scale: Optional[float] = None, heads: Optional[Sequence[int]] = None,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    sh = _shape_qkv(q, k, v)
    check_vs_index(sh, heads, intervals, n_intervals, cols, n_cols)
    o = _out_like(q, out)
    ha, hn = _heads(heads)
    _call("dsa_sparse_attention_vs", _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "out"),
          ctypes.byref(sh), _scale(scale), ha, hn, _dev(intervals, "intervals", torch.int32),
          _dev(n_intervals, "n_intervals", torch.int32), intervals.shape[1],
          _dev(cols, "cols", torch.int32), _dev(n_cols, "n_cols", torch.int32), cols.shape[2],
          _stream(q))
    return o


def sparse_attention_blocks(q, k, v, sel, n_sel, *, scale: Optional[float] = None,
                            heads: Optional[Sequence[int]] = None,
                            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    sh = _shape_qkv(q, k, v)
    check_block_index(sh, heads, sel, n_sel)
    o = _out_like(q, out)
    ha, hn = _heads(heads)
    _call("dsa_sparse_attention_blocks", _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "out"),
          ctypes.byref(sh), _scale(scale), ha, hn, _dev(sel, "sel", torch.int32),
          _dev(n_sel, "n_sel", torch.int32), sel.shape[2], _stream(q))
    return o


def sparse_attention_mixed(q, k, v, patterns: Sequence[Optional[str]], *, vs_index=None, bs_index=None,
                           init_blocks: int = 1, local_blocks: int = 1, scale: Optional[float] = None,
                           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The one-launch attention over given indices: vs_index = (intervals,
    n_intervals, cols, n_cols) for the VS heads in ascending order, bs_index =
    (sel, n_sel) for the BS heads in ascending order."""
    sh = _shape_qkv(q, k, v)
    pa = _patterns(patterns, sh.q_heads)
    n_vs = sum(1 for p in patterns if p == "vs")
    n_bs = sum(1 for p in patterns if p == "bs")
    if n_vs and vs_index is None:
        raise ValueError("vs_index is required when a head follows the vertical-slash pattern")
    if n_bs and bs_index is None:
        raise ValueError("bs_index is required when a head follows the block-sparse pattern")
    if vs_index is not None:
        check_vs_index(sh, [0] * n_vs, *vs_index)
    if bs_index is not None:
        check_block_index(sh, [0] * n_bs, *bs_index)
    o = _out_like(q, out)
    iv = niv = cols = ncols = sel = nsel = None
    max_iv = max_cols = max_sel = 0
    if vs_index is not None:
        intervals, n_intervals, c, nc = vs_index
        iv, niv = _dev(intervals, "intervals", torch.int32), _dev(n_intervals, "n_intervals", torch.int32)
        cols, ncols = _dev(c, "cols", torch.int32), _dev(nc, "n_cols", torch.int32)
        max_iv, max_cols = intervals.shape[1], c.shape[2]
    if bs_index is not None:
        s_, ns = bs_index
        sel, nsel = _dev(s_, "sel", torch.int32), _dev(ns, "n_sel", torch.int32)
        max_sel = s_.shape[2]
    _call("dsa_sparse_attention_mixed", _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "out"),
          ctypes.byref(sh), _scale(scale), pa, iv, niv, max_iv, cols, ncols, max_cols, sel, nsel,
          max_sel, init_blocks, local_blocks, _stream(q))
    return o


# ----------------------------------------------------------------------------
# hierarchical chunk pruning
# ----------------------------------------------------------------------------
def _stages(stages: Sequence[Tuple[int, int]]) -> PruneStages:
    """[(chunk length, keep count), ...] outermost first -> the C struct (the
    library checks the values)."""
    st = PruneStages()
    st.n_stages = len(stages)
    if not 1 <= len(stages) <= PRUNE_MAX_STAGES:
        raise ValueError(f"1 to {PRUNE_MAX_STAGES} stages")
    for i, (c, k) in enumerate(stages):
        st.chunk[i], st.keep[i] = int(c), int(k)
    return st


def hier_prune(qu: torch.Tensor, k: torch.Tensor, stages: Sequence[Tuple[int, int]], *, q_heads: int,
               heads: Optional[Sequence[int]] = None, unit_rows: int = 0, scale: Optional[float] = None,
               return_block_max: bool = False):
    """Pruning stages for query vectors qu [batch * n_heads, units, head_dim]
    (bf16 or fp32) over the cache k [batch, kv_heads, seq_len, head_dim]:
    (sel [rows, units, keep_last], n_sel [rows, units][, block_max
    [rows, units, ceil(seq_len / 64)]]). Entries past the counts (and blocks a
    unit does not see) are left unwritten."""
    B, Hkv, n, D = k.shape
    rows, units, Dq = qu.shape
    ha, hn = _heads(heads)
    nh = q_heads if heads is None else hn
    if rows != B * nh or Dq != D:
        raise ValueError(f"qu must be [batch * n_heads, units, head_dim] = [{B * nh}, *, {D}]")
    sh = Shape(B, q_heads, Hkv, n, D, _dtype_code(k))
    st = _stages(stages)
    ks = stages[-1][1]
    sel = torch.empty((rows, units, ks), dtype=torch.int32, device=k.device)
    n_sel = torch.empty((rows, units), dtype=torch.int32, device=k.device)
    bm, ws = None, None
    if return_block_max:
        bm = torch.full((rows, units, (n + BLOCK - 1) // BLOCK), float("nan"), dtype=torch.float32,
                        device=k.device)
    else:
        ws = _workspace(load().dsa_hier_prune_workspace_bytes(ctypes.byref(sh), units, nh), k.device)
    _call("dsa_hier_prune", _dev(qu, "qu"), _dtype_code(qu), units, unit_rows, _dev(k, "k"), ctypes.byref(sh),
          ctypes.byref(st), _scale(scale), ha, hn, None if bm is None else bm.data_ptr(), sel.data_ptr(),
          n_sel.data_ptr(), None if ws is None else ws.data_ptr(), 0 if ws is None else ws.numel(), _stream(k))
    return (sel, n_sel, bm) if return_block_max else (sel, n_sel)


def chunks_to_keys(sel: torch.Tensor, n_sel: torch.Tensor, chunk: int, seq_len: int):
    """Key lists of kept chunks: (keys [rows, max_sel * chunk], n_keys [rows]); sel [rows, max_sel]."""
    rows, max_sel = sel.shape
    keys = torch.empty((rows, max_sel * chunk), dtype=torch.int32, device=sel.device)
    n_keys = torch.empty((rows,), dtype=torch.int32, device=sel.device)
    _call("dsa_chunks_to_keys", _dev(sel, "sel", torch.int32), _dev(n_sel, "n_sel", torch.int32), rows,
          max_sel, chunk, seq_len, keys.data_ptr(), n_keys.data_ptr(), _stream(sel))
    return keys, n_keys


def hier_sparse_decode(q, k, v, stages: Sequence[Tuple[int, int]], *, scale: Optional[float] = None,
                       heads: Optional[Sequence[int]] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode rows (q [batch, q_heads, head_dim]) over the keys the pruning
    stages keep for them; k, v the cache [batch, kv_heads, seq_len, head_dim]."""
    if k.dim() != 4 or v.shape != k.shape:
        raise ValueError("k, v must be [batch, kv_heads, seq_len, head_dim]")
    B, Hkv, n, D = k.shape
    if q.dim() != 3 or q.shape[0] != B or q.shape[2] != D:
        raise ValueError("q must be [batch, q_heads, head_dim]")
    sh = Shape(B, q.shape[1], Hkv, n, D, _dtype_code(q))
    st = _stages(stages)
    ha, hn = _heads(heads)
    nh = q.shape[1] if heads is None else hn
    o = torch.zeros_like(q) if out is None else out
    ws = _workspace(load().dsa_hier_sparse_decode_workspace_bytes(ctypes.byref(sh), ctypes.byref(st), nh),
                    q.device)
    _call("dsa_hier_sparse_decode", _dev(q, "q"), _dev(k, "k", q.dtype), _dev(v, "v", q.dtype), _dev(o, "out"),
          ctypes.byref(sh), ctypes.byref(st), _scale(scale), ha, hn, ws.data_ptr(), ws.numel(), _stream(q))
    return o


def hier_block_sparse_attention(q, k, v, stages: Sequence[Tuple[int, int]], *, scale: Optional[float] = None,
                                heads: Optional[Sequence[int]] = None,
                                out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Prefill heads whose key blocks the pruning stages choose (last chunk
    length 64), q, k, v as in block_sparse_attention."""
    sh = _shape_qkv(q, k, v)
    st = _stages(stages)
    o = _out_like(q, out)
    ha, hn = _heads(heads)
    nh = sh.q_heads if heads is None else hn
    ws = _workspace(load().dsa_hier_block_sparse_workspace_bytes(ctypes.byref(sh), ctypes.byref(st), nh),
                    q.device)
    _call("dsa_hier_block_sparse_attention", _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "out"),
          ctypes.byref(sh), ctypes.byref(st), _scale(scale), ha, hn, ws.data_ptr(), ws.numel(), _stream(q))
    return o
