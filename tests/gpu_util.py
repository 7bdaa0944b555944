"""Shared helpers of the GPU parity tests: conversions between the GPU's index
layouts and the oracle's, and the tolerances of the parity contract."""
import numpy as np
import torch

from oracle import dsa_oracle as O

BLK = 64
ATTN_MAX_ABS = 2e-2     # attention output, max |gpu - oracle|
ATTN_MEAN_ABS = 2e-3    # attention output, mean |gpu - oracle|
SCORE_REL = 1e-3        # estimator scores, relative


def host64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a bf16/fp32 tensor."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_scores(gpu: np.ndarray, ref: np.ndarray, what: str):
    gpu = np.asarray(gpu, np.float64)
    bad = np.abs(gpu - ref) > SCORE_REL * np.abs(ref) + 1e-12
    assert not bad.any(), (what, int(bad.sum()), np.flatnonzero(bad)[:5],
                           gpu[bad][:5], ref[bad][:5])


def check_attention(gpu_rows: np.ndarray, ref_rows: np.ndarray, what: str):
    d = np.abs(np.asarray(gpu_rows, np.float64) - ref_rows)
    assert np.isfinite(gpu_rows).all(), what
    mx, mean = float(d.max()), float(d.mean())
    assert mx <= ATTN_MAX_ABS and mean <= ATTN_MEAN_ABS, (what, mx, mean)
    return mx, mean


def oracle_vs_index(V, S, n):
    """Oracle sparse format in the GPU layout: intervals [ns, 2] + count,
    cols [nb, nv] + counts."""
    iv = O.merge_offsets(S)
    nb = O.num_blocks(n)
    ivs = np.zeros((max(1, len(S)), 2), np.int32)
    ivs[: len(iv)] = np.asarray(iv, np.int32).reshape(-1, 2) if iv else 0
    cols = np.zeros((nb, max(1, len(V))), np.int32)
    ncols = np.zeros(nb, np.int32)
    for a in range(nb):
        c = O.vs_block_cols(V, O.vs_block_ranges(iv, a, n), a, n)
        cols[a, : len(c)] = c
        ncols[a] = len(c)
    return iv, ivs, cols, ncols


def gpu_cols(cols: torch.Tensor, ncols: torch.Tensor, row: int, a: int):
    k = int(ncols[row, a])
    return cols[row, a, :k].cpu().numpy().astype(np.int64)


def block_rows(out_blocks: dict, a: int):
    return out_blocks[a]
