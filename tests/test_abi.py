"""The C ABI on the CPU: the library loads without a GPU, exports every symbol the
header declares, and rejects bad arguments before any HIP call (no kernel runs)."""
import ctypes
import os
import re
import subprocess

import pytest

from conftest import ROOT
import block_sparse_attention_blockmean_amd as nb_lib
from block_sparse_attention_blockmean_amd._binding import (
    NABLA_BF16, NABLA_E_INVAL, NABLA_E_UNSUPPORTED, NABLA_E_WORKSPACE, NABLA_F32, StaWindow,
)

HEADER = os.path.join(ROOT, "include", "nabla.h")

# Fake, 256-byte aligned device addresses: validation rejects every call below before
# anything dereferences them.
A, B_, C, D_, E, F_, G = (ctypes.c_void_p(0x100000 * (i + 1)) for i in range(7))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)) - {"if"})


@pytest.fixture(scope="module")
def lib():
    return nb_lib.load_library()


def test_library_loads_without_gpu(lib):
    assert lib is not None


def test_every_declared_symbol_is_exported(lib):
    decl = declared_functions()
    assert sorted(decl) == sorted(nb_lib.EXPORTS), decl
    out = subprocess.run(["nm", "-D", "--defined-only", nb_lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in decl:
        assert name in exported, name
        assert hasattr(lib, name)


def test_status_strings(lib):
    names = [lib.nabla_status_string(i).decode() for i in range(5)]
    assert names == ["NABLA_OK", "NABLA_E_INVAL", "NABLA_E_UNSUPPORTED", "NABLA_E_HIP",
                     "NABLA_E_WORKSPACE"]


def up256(n):
    return (n + 255) // 256 * 256


def test_workspace_size(lib):
    # pooled K in the split half form (4 d bytes per block, blocks padded to a multiple
    # of 16 per head), then one 4-byte exponent per block, each part rounded up to 256
    assert lib.nabla_build_mask_workspace_size(1, 12, 32256, 128, 64) == 12 * 512 * 128 * 4 + up256(12 * 504 * 4)
    assert lib.nabla_build_mask_workspace_size(1, 2, 1024, 64, 64) == 2 * 16 * 64 * 4 + up256(2 * 16 * 4)
    # 3 blocks (padded to 16), d = 16: 1024 B, and 12 B rounded up to 256
    assert lib.nabla_build_mask_workspace_size(1, 1, 192, 16, 64) == 16 * 16 * 4 + 256
    assert lib.nabla_build_mask_workspace_size(1, 1, 1000, 64, 64) == 0
    assert lib.nabla_build_mask_workspace_size(0, 1, 1024, 64, 64) == 0


# ------------------------------------------------------------- nabla_reorder

def reorder(lib, src=A, dst=B_, batch=1, heads=2, T=4, H=16, W=16, d=64, P=8, dt=NABLA_F32,
            inverse=0):
    return lib.nabla_reorder(src, dst, batch, heads, T, H, W, d, P, dt, inverse, None)


@pytest.mark.parametrize("kw,status", [
    (dict(src=None), NABLA_E_INVAL),
    (dict(dst=None), NABLA_E_INVAL),
    (dict(dst=A), NABLA_E_INVAL),
    (dict(src=ctypes.c_void_p(0x100008)), NABLA_E_INVAL),
    (dict(batch=0), NABLA_E_INVAL),
    (dict(T=-1), NABLA_E_INVAL),
    (dict(H=12), NABLA_E_INVAL),
    (dict(W=20), NABLA_E_INVAL),
    (dict(inverse=2), NABLA_E_INVAL),
    (dict(dt=7), NABLA_E_INVAL),
    (dict(d=2), NABLA_E_UNSUPPORTED),
    (dict(d=24), NABLA_E_UNSUPPORTED),
])
def test_reorder_validation(lib, kw, status):
    assert reorder(lib, **kw) == status
    assert lib.nabla_last_error().decode().startswith("nabla_reorder")


# ------------------------------------------------------------- nabla_build_mask

def build_mask(lib, q=A, k=B_, batch=1, heads=2, T=4, H=16, W=16, d=64, P=8, N=64, thr=0.1,
               sta=None, scale=0.0, dt=NABLA_F32, cnt=C, idx=D_, bitmap=None, schedule=None, ws=E,
               ws_bytes=1 << 30):
    win = None if sta is None else ctypes.byref(StaWindow(*sta))
    return lib.nabla_build_mask(q, k, batch, heads, T, H, W, d, P, N, thr, win, scale, dt, cnt,
                                idx, bitmap, schedule, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), NABLA_E_INVAL),
    (dict(k=None), NABLA_E_INVAL),
    (dict(cnt=None), NABLA_E_INVAL),
    (dict(idx=None), NABLA_E_INVAL),
    (dict(q=ctypes.c_void_p(0x100004)), NABLA_E_INVAL),
    (dict(heads=0), NABLA_E_INVAL),
    (dict(H=20), NABLA_E_INVAL),
    (dict(T=3, H=8, W=8, P=8, thr=2.0), NABLA_E_INVAL),  # valid shape, bad thr
    (dict(T=1, H=8, W=12, P=4), NABLA_E_INVAL),         # L = 96 not a multiple of 64
    (dict(thr=1.0), NABLA_E_INVAL),
    (dict(thr=-0.1), NABLA_E_INVAL),
    (dict(thr=float("nan")), NABLA_E_INVAL),
    (dict(scale=float("nan")), NABLA_E_INVAL),
    (dict(scale=float("inf")), NABLA_E_INVAL),
    (dict(sta=(2, 3, 3)), NABLA_E_INVAL),
    (dict(sta=(3, 0, 3)), NABLA_E_INVAL),
    (dict(sta=(3, 3, 3), P=4, H=16, W=16), NABLA_E_INVAL),  # N != P*P
    (dict(dt=5), NABLA_E_INVAL),
    (dict(N=32, T=4), NABLA_E_UNSUPPORTED),
    (dict(d=96), NABLA_E_UNSUPPORTED),
    (dict(T=257, H=32, W=32), NABLA_E_UNSUPPORTED),     # 4112 blocks > NABLA_MAX_BLOCKS
    (dict(schedule=ctypes.c_void_p(0x100002)), NABLA_E_INVAL),
    (dict(ws=None), NABLA_E_WORKSPACE),
    (dict(ws_bytes=100), NABLA_E_WORKSPACE),
])
def test_build_mask_validation(lib, kw, status):
    assert build_mask(lib, **kw) == status
    assert lib.nabla_last_error().decode().startswith("nabla_build_mask")


# ------------------------------------------------------------- block_sparse_attn_fwd

def attn(lib, q=A, k=B_, v=C, o=D_, batch=1, heads=2, L=1024, d=64, N=64, cnt=E, idx=F_,
         schedule=None, scale=0.0, dt=NABLA_BF16):
    return lib.block_sparse_attn_fwd(q, k, v, o, batch, heads, L, d, N, cnt, idx, schedule, scale,
                                     dt, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), NABLA_E_INVAL),
    (dict(v=None), NABLA_E_INVAL),
    (dict(o=None), NABLA_E_INVAL),
    (dict(cnt=None), NABLA_E_INVAL),
    (dict(idx=None), NABLA_E_INVAL),
    (dict(o=ctypes.c_void_p(0x100002)), NABLA_E_INVAL),
    (dict(schedule=ctypes.c_void_p(0x100001)), NABLA_E_INVAL),
    (dict(L=1000), NABLA_E_INVAL),
    (dict(L=0), NABLA_E_INVAL),
    (dict(scale=float("nan")), NABLA_E_INVAL),
    (dict(dt=3), NABLA_E_INVAL),
    (dict(N=128), NABLA_E_UNSUPPORTED),
    (dict(d=256), NABLA_E_UNSUPPORTED),
    (dict(L=1 << 23, d=128), NABLA_E_UNSUPPORTED),       # one head = 2^31 bytes of bf16
    (dict(L=1 << 22, d=128, dt=NABLA_F32), NABLA_E_UNSUPPORTED),
])
def test_attn_validation(lib, kw, status):
    assert attn(lib, **kw) == status
    assert lib.nabla_last_error().decode().startswith("block_sparse_attn_fwd")


def attn_lse(lib, lse=G, **kw):
    a = dict(q=A, k=B_, v=C, o=D_, batch=1, heads=2, L=1024, d=64, N=64, cnt=E, idx=F_,
             schedule=None, scale=0.0, dt=NABLA_BF16)
    a.update(kw)
    return lib.block_sparse_attn_fwd_lse(a["q"], a["k"], a["v"], a["o"], a["batch"], a["heads"], a["L"],
                                         a["d"], a["N"], a["cnt"], a["idx"], a["schedule"], a["scale"],
                                         a["dt"], lse, None)


@pytest.mark.parametrize("kw,status", [
    (dict(lse=None), NABLA_E_INVAL),
    (dict(lse=ctypes.c_void_p(0x100004)), NABLA_E_INVAL),
    (dict(q=None), NABLA_E_INVAL),
    (dict(L=1000), NABLA_E_INVAL),
    (dict(d=96), NABLA_E_UNSUPPORTED),
])
def test_attn_lse_validation(lib, kw, status):
    assert attn_lse(lib, **kw) == status
    assert lib.nabla_last_error().decode().startswith("block_sparse_attn_fwd_lse")


# ------------------------------------------------------------- block_sparse_attn_bwd

H_, I_, J_, K_, M_ = (ctypes.c_void_p(0x1000000 * (i + 1)) for i in range(5))


def test_bwd_workspace_size(lib):
    # D, bitmap, counts, lists, two orders; each rounded up to 256 bytes
    BH, L, nb = 12, 32256, 504
    up = lambda b: (b + 255) // 256 * 256
    want = up(BH * L * 4) + up(BH * nb * 16 * 4) + up(BH * nb * 4) + up(BH * nb * nb * 4) + 2 * up(BH * nb * 4)
    assert lib.nabla_attn_bwd_workspace_size(1, 12, L, 64) == want
    assert lib.nabla_attn_bwd_workspace_size(1, 1, 1000, 64) == 0
    assert lib.nabla_attn_bwd_workspace_size(1, 0, 1024, 64) == 0


def attn_bwd(lib, **kw):
    a = dict(q=A, k=B_, v=C, o=D_, dout=E, lse=F_, dq=G, dk=H_, dv=I_, batch=1, heads=2, L=1024, d=64,
             N=64, cnt=J_, idx=K_, scale=0.0, dt=NABLA_BF16, ws=M_, ws_bytes=1 << 30)
    a.update(kw)
    return lib.block_sparse_attn_bwd(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"],
                                     a["dv"], a["batch"], a["heads"], a["L"], a["d"], a["N"], a["cnt"],
                                     a["idx"], a["scale"], a["dt"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), NABLA_E_INVAL),
    (dict(dout=None), NABLA_E_INVAL),
    (dict(lse=None), NABLA_E_INVAL),
    (dict(dk=None), NABLA_E_INVAL),
    (dict(lse=ctypes.c_void_p(0x100008)), NABLA_E_INVAL),
    (dict(dq=A), NABLA_E_INVAL),            # output aliases q
    (dict(dv=E), NABLA_E_INVAL),            # output aliases dout
    (dict(dk=G), NABLA_E_INVAL),            # dk == dq
    (dict(L=1000), NABLA_E_INVAL),
    (dict(scale=float("inf")), NABLA_E_INVAL),
    (dict(dt=4), NABLA_E_INVAL),
    (dict(N=32), NABLA_E_UNSUPPORTED),
    (dict(d=32), NABLA_E_UNSUPPORTED),
    (dict(L=64 * 4097), NABLA_E_UNSUPPORTED),          # nb > NABLA_MAX_BLOCKS
    (dict(L=1 << 23, d=128), NABLA_E_UNSUPPORTED),
    (dict(ws=None), NABLA_E_WORKSPACE),
    (dict(ws_bytes=1000), NABLA_E_WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x100010)), NABLA_E_INVAL),
])
def test_attn_bwd_validation(lib, kw, status):
    assert attn_bwd(lib, **kw) == status
    assert lib.nabla_last_error().decode().startswith("block_sparse_attn_bwd")


# ------------------------------------------------------------- raster-order entry points

def test_build_mask_raster_validation(lib):
    win = None
    def call(**kw):
        a = dict(q=A, k=B_, batch=1, heads=2, T=4, H=16, W=16, d=64, P=8, N=64, thr=0.1, scale=0.0,
                 dt=NABLA_F32, cnt=C, idx=D_, ws=E, ws_bytes=1 << 30)
        a.update(kw)
        return lib.nabla_build_mask_raster(a["q"], a["k"], a["batch"], a["heads"], a["T"], a["H"], a["W"],
                                           a["d"], a["P"], a["N"], a["thr"], win, a["scale"], a["dt"], a["cnt"],
                                           a["idx"], None, None, a["ws"], a["ws_bytes"], None)
    for kw, st in ((dict(q=None), NABLA_E_INVAL), (dict(P=4, H=16, W=16), NABLA_E_INVAL),
                   (dict(thr=1.5), NABLA_E_INVAL), (dict(d=96), NABLA_E_UNSUPPORTED),
                   (dict(ws_bytes=10), NABLA_E_WORKSPACE)):
        assert call(**kw) == st, kw
        assert lib.nabla_last_error().decode().startswith("nabla_build_mask_raster")


def test_attn_raster_validation(lib):
    def call(**kw):
        a = dict(q=A, k=B_, v=C, o=D_, batch=1, heads=2, T=4, H=16, W=16, d=64, P=8, N=64, cnt=E, idx=F_,
                 scale=0.0, dt=NABLA_BF16)
        a.update(kw)
        return lib.block_sparse_attn_fwd_raster(a["q"], a["k"], a["v"], a["o"], a["batch"], a["heads"], a["T"],
                                                a["H"], a["W"], a["d"], a["P"], a["N"], a["cnt"], a["idx"], None,
                                                a["scale"], a["dt"], None)
    for kw, st in ((dict(o=None), NABLA_E_INVAL), (dict(P=4), NABLA_E_INVAL), (dict(H=20), NABLA_E_INVAL),
                   (dict(T=0), NABLA_E_INVAL), (dict(d=32), NABLA_E_UNSUPPORTED),
                   (dict(scale=float("nan")), NABLA_E_INVAL)):
        assert call(**kw) == st, kw
        assert lib.nabla_last_error().decode().startswith("block_sparse_attn_fwd_raster")


def test_attn_lse_raster_validation(lib):
    def call(**kw):
        a = dict(q=A, k=B_, v=C, o=D_, batch=1, heads=2, T=4, H=16, W=16, d=64, P=8, N=64, cnt=E, idx=F_,
                 scale=0.0, dt=NABLA_BF16, lse=G)
        a.update(kw)
        return lib.block_sparse_attn_fwd_lse_raster(a["q"], a["k"], a["v"], a["o"], a["batch"], a["heads"],
                                                    a["T"], a["H"], a["W"], a["d"], a["P"], a["N"], a["cnt"],
                                                    a["idx"], None, a["scale"], a["dt"], a["lse"], None)
    for kw, st in ((dict(lse=None), NABLA_E_INVAL), (dict(lse=ctypes.c_void_p(0x100008)), NABLA_E_INVAL),
                   (dict(o=None), NABLA_E_INVAL), (dict(P=4), NABLA_E_INVAL), (dict(W=12), NABLA_E_INVAL),
                   (dict(T=0), NABLA_E_INVAL), (dict(d=96), NABLA_E_UNSUPPORTED)):
        assert call(**kw) == st, kw
        assert lib.nabla_last_error().decode().startswith("block_sparse_attn_fwd_lse_raster")


def test_attn_bwd_raster_validation(lib):
    need = lib.nabla_attn_bwd_workspace_size(1, 2, 4 * 16 * 16, 64)
    def call(**kw):
        a = dict(q=A, k=B_, v=C, o=D_, dout=E, lse=F_, dq=G, dk=H_, dv=I_, batch=1, heads=2, T=4, H=16, W=16,
                 d=64, P=8, N=64, cnt=J_, idx=K_, scale=0.0, dt=NABLA_BF16, ws=M_, ws_bytes=need)
        a.update(kw)
        return lib.block_sparse_attn_bwd_raster(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"],
                                                a["dk"], a["dv"], a["batch"], a["heads"], a["T"], a["H"], a["W"],
                                                a["d"], a["P"], a["N"], a["cnt"], a["idx"], a["scale"], a["dt"],
                                                a["ws"], a["ws_bytes"], None)
    for kw, st in ((dict(q=None), NABLA_E_INVAL), (dict(lse=None), NABLA_E_INVAL), (dict(dq=A), NABLA_E_INVAL),
                   (dict(P=4), NABLA_E_INVAL), (dict(N=32), NABLA_E_INVAL), (dict(H=20), NABLA_E_INVAL),
                   (dict(T=-1), NABLA_E_INVAL), (dict(d=32), NABLA_E_UNSUPPORTED),
                   (dict(ws_bytes=need - 1), NABLA_E_WORKSPACE), (dict(ws=None), NABLA_E_WORKSPACE)):
        assert call(**kw) == st, kw
        assert lib.nabla_last_error().decode().startswith("block_sparse_attn_bwd_raster")


# ------------------------------------------------------------- SIP entry points

def test_build_mask_sip_validation(lib):
    def call(**kw):
        a = dict(q=A, k=B_, batch=1, heads=2, T=4, H=16, W=16, d=64, P=8, N=64, budget=4, u=G, scale=0.0,
                 dt=NABLA_BF16, cnt=C, idx=D_, logw=E, ws=F_, ws_bytes=1 << 30)
        a.update(kw)
        return lib.nabla_build_mask_sip(a["q"], a["k"], a["batch"], a["heads"], a["T"], a["H"], a["W"], a["d"],
                                        a["P"], a["N"], a["budget"], a["u"], a["scale"], a["dt"], a["cnt"],
                                        a["idx"], a["logw"], None, None, a["ws"], a["ws_bytes"], None)
    for kw, st in ((dict(u=None), NABLA_E_INVAL), (dict(logw=None), NABLA_E_INVAL), (dict(budget=0), NABLA_E_INVAL),
                   (dict(u=ctypes.c_void_p(0x100002)), NABLA_E_INVAL), (dict(q=None), NABLA_E_INVAL),
                   (dict(d=96), NABLA_E_UNSUPPORTED), (dict(ws=None), NABLA_E_WORKSPACE)):
        assert call(**kw) == st, kw
        assert lib.nabla_last_error().decode().startswith("nabla_build_mask_sip")


def test_attn_weighted_validation(lib):
    def call(**kw):
        a = dict(q=A, k=B_, v=C, o=D_, batch=1, heads=2, L=1024, d=64, N=64, cnt=E, idx=F_, logw=G, scale=0.0,
                 dt=NABLA_BF16)
        a.update(kw)
        return lib.block_sparse_attn_fwd_weighted(a["q"], a["k"], a["v"], a["o"], a["batch"], a["heads"], a["L"],
                                                  a["d"], a["N"], a["cnt"], a["idx"], a["logw"], None, a["scale"],
                                                  a["dt"], None)
    for kw, st in ((dict(logw=None), NABLA_E_INVAL), (dict(logw=ctypes.c_void_p(0x100001)), NABLA_E_INVAL),
                   (dict(L=1000), NABLA_E_INVAL), (dict(N=32), NABLA_E_UNSUPPORTED)):
        assert call(**kw) == st, kw
        assert lib.nabla_last_error().decode().startswith("block_sparse_attn_fwd_weighted")


# ------------------------------------------------------------- IBCS entry points

def test_ibcs_workspace_size(lib):
    # pooled K per block (blocks padded to a multiple of 16 per head); 8 centroids, 8
    # weights and one nb-long score row per query group; sections rounded up to 256
    blocks = 12 * 504
    for qg in (64, 128):
        groups = blocks * 64 // qg
        want = 12 * 512 * 128 * 4 + groups * 8 * 128 * 4 + groups * 8 * 4 + groups * 504 * 4
        assert lib.nabla_build_mask_ibcs_workspace_size(1, 12, 32256, 128, 64, qg) == want
    # 3 blocks (padded to 16), d = 64, one block per group: 4096 B, 6144 B, 96 B, 36 B
    assert lib.nabla_build_mask_ibcs_workspace_size(1, 1, 192, 64, 64, 64) == 4096 + 6144 + 256 + 256
    assert lib.nabla_build_mask_ibcs_workspace_size(1, 1, 192, 64, 64, 128) == 0     # 192 % 128
    assert lib.nabla_build_mask_ibcs_workspace_size(1, 1, 256, 64, 64, 96) == 0      # 96 % 64
    assert lib.nabla_build_mask_ibcs_workspace_size(1, 1, 1000, 64, 64, 64) == 0
    assert lib.nabla_build_mask_ibcs_workspace_size(1, -1, 1024, 64, 64, 64) == 0


def test_build_mask_ibcs_validation(lib):
    def call(**kw):
        a = dict(q=A, k=B_, batch=1, heads=2, T=4, H=16, W=16, d=64, P=8, N=64, qg=128, thr=0.1, sta=None,
                 scale=0.0, dt=NABLA_BF16, cnt=C, idx=D_, ws=E, ws_bytes=1 << 30)
        a.update(kw)
        win = None if a["sta"] is None else ctypes.byref(StaWindow(*a["sta"]))
        return lib.nabla_build_mask_ibcs(a["q"], a["k"], a["batch"], a["heads"], a["T"], a["H"], a["W"], a["d"],
                                         a["P"], a["N"], a["qg"], a["thr"], win, a["scale"], a["dt"], a["cnt"],
                                         a["idx"], None, None, a["ws"], a["ws_bytes"], None)
    # the plain mask's workspace is too small for the centroids
    small_ws = lib.nabla_build_mask_workspace_size(1, 2, 1024, 64, 64)
    for kw, st in ((dict(q=None), NABLA_E_INVAL), (dict(thr=1.0), NABLA_E_INVAL), (dict(sta=(2, 3, 3)), NABLA_E_INVAL),
                   (dict(T=1, H=8, W=12, P=4), NABLA_E_INVAL), (dict(d=96), NABLA_E_UNSUPPORTED),
                   (dict(N=32, qg=64), NABLA_E_UNSUPPORTED), (dict(ws=None), NABLA_E_WORKSPACE),
                   (dict(ws_bytes=small_ws), NABLA_E_WORKSPACE),
                   (dict(qg=0), NABLA_E_INVAL), (dict(qg=96), NABLA_E_INVAL),
                   (dict(T=3, H=8, W=8), NABLA_E_INVAL),          # 3 blocks: L = 192 not a multiple of 128
                   (dict(qg=256), NABLA_E_UNSUPPORTED),
                   (dict(T=129, H=32, W=32), NABLA_E_UNSUPPORTED)):   # 2064 blocks > NABLA_IBCS_MAX_BLOCKS
        assert call(**kw) == st, kw
        assert lib.nabla_last_error().decode().startswith("nabla_build_mask_ibcs")


def test_build_mask_ibcs_raster_validation(lib):
    def call(**kw):
        a = dict(q=A, k=B_, batch=1, heads=2, T=4, H=16, W=16, d=64, P=8, N=64, qg=128, thr=0.1, dt=NABLA_BF16,
                 ws_bytes=1 << 30)
        a.update(kw)
        return lib.nabla_build_mask_ibcs_raster(a["q"], a["k"], a["batch"], a["heads"], a["T"], a["H"], a["W"],
                                                a["d"], a["P"], a["N"], a["qg"], a["thr"], None, 0.0, a["dt"], C, D_,
                                                None, None, E, a["ws_bytes"], None)
    for kw, st in ((dict(q=None), NABLA_E_INVAL), (dict(P=4, H=16, W=16), NABLA_E_INVAL),   # N != P*P
                   (dict(qg=96), NABLA_E_INVAL), (dict(qg=256), NABLA_E_UNSUPPORTED), (dict(ws_bytes=64), NABLA_E_WORKSPACE)):
        assert call(**kw) == st, kw
        assert lib.nabla_last_error().decode().startswith("nabla_build_mask_ibcs_raster")


def test_build_mask_ibcs_sip_validation(lib):
    def call(**kw):
        a = dict(q=A, k=B_, batch=1, heads=2, T=4, H=16, W=16, d=64, P=8, N=64, qg=128, budget=4, u=G, scale=0.0,
                 dt=NABLA_BF16, cnt=C, idx=D_, logw=E, ws=F_, ws_bytes=1 << 30)
        a.update(kw)
        return lib.nabla_build_mask_ibcs_sip(a["q"], a["k"], a["batch"], a["heads"], a["T"], a["H"], a["W"],
                                             a["d"], a["P"], a["N"], a["qg"], a["budget"], a["u"], a["scale"],
                                             a["dt"], a["cnt"], a["idx"], a["logw"], None, None, a["ws"],
                                             a["ws_bytes"], None)
    small_ws = lib.nabla_build_mask_workspace_size(1, 2, 1024, 64, 64)
    for kw, st in ((dict(u=None), NABLA_E_INVAL), (dict(logw=None), NABLA_E_INVAL), (dict(budget=0), NABLA_E_INVAL),
                   (dict(qg=96), NABLA_E_INVAL), (dict(T=3, H=8, W=8), NABLA_E_INVAL), (dict(qg=256), NABLA_E_UNSUPPORTED),
                   (dict(d=96), NABLA_E_UNSUPPORTED), (dict(ws_bytes=small_ws), NABLA_E_WORKSPACE)):
        assert call(**kw) == st, kw
        assert lib.nabla_last_error().decode().startswith("nabla_build_mask_ibcs_sip")


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 1, 1024, 64)
    with pytest.raises(ValueError):
        nb_lib.reorder(x, 4, 16, 16, 8)


def test_binding_checks_mask_shapes_before_pointers():
    """The mask wrappers check the token count against T*H*W and the caller's output
    buffers (dtype, size) before taking any pointer: the library sizes its lists from
    T*H*W, so a mismatch would write lists with another stride into q-sized buffers."""
    import torch
    q = torch.zeros(1, 2, 1024, 64)
    with pytest.raises(ValueError, match="does not match T\\*H\\*W"):
        nb_lib.build_mask(q, q, 4, 16, 8, 8)                       # T*H*W = 512
    with pytest.raises(ValueError, match="does not match T\\*H\\*W"):
        nb_lib.build_mask_sip(q, q, 2, 16, 16, 8, 4, torch.zeros(1, 2, 16, 16))
    with pytest.raises(ValueError, match="same shape"):
        nb_lib.build_mask(q, torch.zeros(1, 2, 1024, 32), 4, 16, 16, 8)
    with pytest.raises(TypeError, match="kv_count must be int32"):
        nb_lib.build_mask(q, q, 4, 16, 16, 8, kv_count=torch.zeros(1, 2, 16, dtype=torch.int64))
    with pytest.raises(ValueError, match="kv_index holds"):
        nb_lib.build_mask(q, q, 4, 16, 16, 8, kv_index=torch.zeros(1, 2, 16, 15, dtype=torch.int32))
    with pytest.raises(ValueError, match="schedule holds"):
        nb_lib.build_mask(q, q, 4, 16, 16, 8, schedule=torch.zeros(31, dtype=torch.int32))
    with pytest.raises(ValueError, match="sizes do not match"):
        nb_lib.attn_fwd_raster(q, q, q, torch.zeros(1, 2, 16, dtype=torch.int32),
                               torch.zeros(1, 2, 16, 16, dtype=torch.int32)[..., :8].contiguous(), 4, 16, 16, 8)


def test_build_mask_raster_noalloc_validation(lib):
    """The allocation-free entry validates like nabla_build_mask_raster (it has no
    workspace) before any HIP call."""
    win = None

    def call(**kw):
        a = dict(q=A, k=B_, batch=1, heads=2, T=4, H=16, W=16, d=64, P=8, N=64, thr=0.1, scale=0.0,
                 dt=NABLA_F32, cnt=C, idx=D_)
        a.update(kw)
        return lib.nabla_build_mask_raster_noalloc(a["q"], a["k"], a["batch"], a["heads"], a["T"], a["H"], a["W"],
                                                   a["d"], a["P"], a["N"], a["thr"], win, a["scale"], a["dt"],
                                                   a["cnt"], a["idx"], None, None, None)
    for kw, st in ((dict(q=None), NABLA_E_INVAL), (dict(idx=None), NABLA_E_INVAL), (dict(thr=1.5), NABLA_E_INVAL),
                   (dict(P=4, H=16, W=16), NABLA_E_INVAL), (dict(H=20), NABLA_E_INVAL),
                   (dict(d=96), NABLA_E_UNSUPPORTED), (dict(T=257, H=32, W=32), NABLA_E_UNSUPPORTED)):
        assert call(**kw) == st, kw
        assert lib.nabla_last_error().decode().startswith("nabla_build_mask_raster_noalloc")
