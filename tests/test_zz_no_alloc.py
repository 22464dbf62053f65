"""The mask entry point that allocates nothing (nabla_build_mask_raster_noalloc) against
the workspace entry point it mirrors (nabla_build_mask_raster), through the C ABI: counts,
lists, bitmap and start order must agree bit for bit, on calls in a row whose second and
third inputs are smaller than the first (the device array keeps the previous call's
contents, which must not leak into the next)."""
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_blockmean_amd as nab
from parity import lists_to_mask

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def structured(B, heads, T, H, W, d, dtype, seed):
    """Seeded inputs with spatial structure on the GPU: a smooth random field over the
    8 x 8 patches shared by Q and K, plus per-token noise."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    nH, nW = H // 8, W // 8
    field = torch.randn((B, heads, T, nH, 1, nW, 1, d), device="cuda", generator=g)
    field = field.expand(B, heads, T, nH, 8, nW, 8, d).reshape(B, heads, T * H * W, d)
    q = (field + 0.5 * torch.randn(field.shape, device="cuda", generator=g)) * 0.6
    k = (field + 0.5 * torch.randn(field.shape, device="cuda", generator=g)) * 0.6
    return q.to(dtype).contiguous(), k.to(dtype).contiguous()


CASES = [
    # 2 x 11 heads of 2048 blocks at d = 128: the pooled Q and K of 16 heads fill the
    # 32 MiB array, so this call runs in two chunks
    dict(B=2, heads=11, T=16, H=64, W=128, d=128, dtype=torch.bfloat16, thr=0.2, sta=None),
    # smaller: 75 blocks per head (ragged against 16-row and 64-column tiles), window
    dict(B=1, heads=3, T=5, H=24, W=40, d=64, dtype=torch.bfloat16, thr=0.2, sta=(3, 3, 3)),
    # smaller still, float32
    dict(B=1, heads=2, T=4, H=16, W=16, d=128, dtype=torch.float32, thr=0.1, sta=None),
]


def test_noalloc_matches_workspace_entry():
    for n, c in enumerate(CASES):
        B, NH, T, H, W, d = c["B"], c["heads"], c["T"], c["H"], c["W"], c["d"]
        nb = T * H * W // 64
        words = (nb + 31) // 32
        say(f"call {n}: B{B} heads{NH} {T}x{H}x{W} d{d} {c['dtype']} nb {nb} thr {c['thr']} sta {c['sta']}")
        q, k = structured(B, NH, T, H, W, d, c["dtype"], seed=100 + n)
        ref_cnt, ref_idx, ref_bm, ref_sched = nab.build_mask(q, k, T, H, W, 8, 64, c["thr"], c["sta"],
                                                             with_bitmap=True, with_schedule=True, raster=True)
        # outputs filled with garbage first: only what the call writes may be compared
        cnt = torch.full((B, NH, nb), -7, dtype=torch.int32, device="cuda")
        idx = torch.full((B, NH, nb, nb), -7, dtype=torch.int32, device="cuda")
        bm = torch.full((B, NH, nb, words), -7, dtype=torch.int32, device="cuda")
        sched = torch.full((B * NH * nb,), -7, dtype=torch.int32, device="cuda")
        nab.build_mask_raster_noalloc(q, k, T, H, W, 8, cnt, idx, 64, c["thr"], c["sta"], bitmap=bm,
                                      schedule=sched)
        torch.cuda.synchronize()
        assert torch.equal(cnt, ref_cnt), "counts differ"
        G = B * NH
        cn = cnt.cpu().numpy().reshape(G, nb)
        m = lists_to_mask(cn, idx.cpu().numpy().reshape(G, nb, nb))
        m_ref = lists_to_mask(ref_cnt.cpu().numpy().reshape(G, nb), ref_idx.cpu().numpy().reshape(G, nb, nb))
        assert np.array_equal(m, m_ref), "lists differ"
        assert torch.equal(bm, ref_bm), "bitmaps differ"
        # the start order: each head's blocks once, by non-increasing count (ties in any order)
        s = sched.cpu().numpy().reshape(G, nb)
        s_ref = ref_sched.cpu().numpy().reshape(G, nb)
        for g in range(G):
            assert np.array_equal(np.sort(s[g]), np.sort(s_ref[g]))
            assert np.array_equal(cn.reshape(-1)[s[g]], cn.reshape(-1)[s_ref[g]])
        say(f"  kept {m.mean():.4f}: counts, lists, bitmap and order agree")
        del q, k, ref_idx, idx
        torch.cuda.empty_cache()
