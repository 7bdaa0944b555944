"""The allocation-free decode entry point (dsa_sparse_decode_noalloc) against
dsa_sparse_decode: same kernels and split partials, so the outputs must be the
same bits. Two calls in a row, the second with a smaller input, so that the
static scratch holds the first call's partials when the second one runs."""
import pytest
import torch

import dynamic_sparse_attention_slash_amd as dsa

pytestmark = pytest.mark.gpu
DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _inputs(B, Hq, Hkv, n, D, dt, n_list, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, Hq, D, generator=g).to(DT[dt]).cuda()
    k = torch.randn(B, Hkv, n, D, generator=g).to(DT[dt]).cuda()
    v = torch.randn(B, Hkv, n, D, generator=g).to(DT[dt]).cuda()
    rows = B * Hq
    keys = torch.stack([torch.randperm(n, generator=g)[:n_list] for _ in range(rows)]).to(torch.int32).cuda()
    counts = torch.randint(0, n_list + 1, (rows,), generator=g).to(torch.int32)
    counts[0] = n_list
    return q, k, v, keys, counts.cuda()


@pytest.mark.parametrize("first,second", [
    ((2, 8, 2, 20000, 128, "bf16", 4000), (1, 4, 1, 3000, 64, "bf16", 700)),
    ((1, 32, 8, 65536, 128, "bf16", 4096), (1, 4, 2, 500, 128, "f32", 100)),
])
def test_noalloc_decode_matches_workspace_decode(first, second):
    for case, (B, Hq, Hkv, n, D, dt, n_list) in (("first", first), ("second", second)):
        print(f"noalloc decode {case}: B={B} Hq={Hq} Hkv={Hkv} n={n} D={D} {dt} list={n_list}", flush=True)
        q, k, v, keys, counts = _inputs(B, Hq, Hkv, n, D, dt, n_list, seed=n + D)
        for kk, nk in ((keys, counts), (None, None)):
            ref = dsa.sparse_decode(q, k, v, kk, nk)
            out = torch.full_like(q, float("nan"))
            got = dsa.sparse_decode_noalloc(q, k, v, kk, nk, out=out)
            torch.cuda.synchronize()
            assert got.data_ptr() == out.data_ptr()
            assert torch.equal(got, ref), (case, kk is None)
            # a head subset writes only its heads
            hs = [Hq - 1, 0]
            sub_keys = None if kk is None else torch.cat([kk[b * Hq + h][None] for b in range(B) for h in hs])
            sub_n = None if nk is None else torch.cat([nk[b * Hq + h][None] for b in range(B) for h in hs])
            out2 = torch.zeros_like(q)
            dsa.sparse_decode_noalloc(q, k, v, sub_keys, sub_n, heads=hs, out=out2)
            torch.cuda.synchronize()
            for h in range(Hq):
                if h in hs:
                    assert torch.equal(out2[:, h], ref[:, h]), (case, h)
                else:
                    assert float(out2[:, h].abs().max()) == 0.0


def test_noalloc_decode_refuses_oversized_partials():
    # 200 x 256 decode rows need more partials than the static scratch holds;
    # refused on the host before any device work
    q = torch.zeros(200, 256, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(200, 256, 64, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dsa.DsaError) as e:
        dsa.sparse_decode_noalloc(q, k, k)
    assert e.value.code == 3
    torch.cuda.synchronize()
