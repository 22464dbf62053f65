"""The mask entry point that allocates nothing (nabla_build_mask_raster_noalloc) against
the workspace entry point it mirrors (nabla_build_mask_raster), through the C ABI: counts,
lists, bitmap and start order must agree bit for bit, on calls in a row each smaller than
the one before (the device array keeps the previous call's contents, which must not leak
into the next); the first runs in two chunks of heads."""
import sys

import numpy as np
import pytest
import torch

import block_sparse_attention_blockmean_amd as nab

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
    # 2 x 8 heads of 4096 blocks at d = 128 (the longest rows): one head's pooled K takes
    # 2.1 MB of the 32 MiB array, 15 heads fit, so this call runs in two chunks
    dict(B=2, heads=8, T=64, H=64, W=64, d=128, dtype=torch.bfloat16, thr=0.2, sta=None),
    # 2 x 11 heads of 2048 blocks, window: one chunk of 22 heads
    dict(B=2, heads=11, T=16, H=64, W=128, d=128, dtype=torch.bfloat16, thr=0.2, sta=(3, 3, 3)),
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
        # the lists are ascending and duplicate-free, so equal masks mean equal written
        # prefixes; compared on the GPU (a list holds only its first count entries)
        valid = torch.arange(nb, device="cuda")[None, None, None, :] < cnt[..., None]
        assert torch.equal(idx[valid], ref_idx[valid]), "lists differ"
        assert torch.equal(bm, ref_bm), "bitmaps differ"
        # the start order: each head's blocks once, by non-increasing count (ties in any order)
        s = sched.cpu().numpy().reshape(G, nb)
        s_ref = ref_sched.cpu().numpy().reshape(G, nb)
        for g in range(G):
            assert np.array_equal(np.sort(s[g]), np.sort(s_ref[g]))
            assert np.array_equal(cn.reshape(-1)[s[g]], cn.reshape(-1)[s_ref[g]])
        say(f"  kept {cn.sum() / (G * nb * nb):.4f}: counts, lists, bitmap and order agree")
        del q, k, ref_idx, idx, valid
        torch.cuda.empty_cache()
