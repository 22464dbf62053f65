"""ctypes binding of libnabla.so: marshals torch device tensors into the C ABI.

Every function passes raw device pointers and torch's current HIP stream; all
computation happens in the library's kernels.  There is no fallback: if the
library is missing or a tensor is not on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnabla.so")

NABLA_OK, NABLA_E_INVAL, NABLA_E_UNSUPPORTED, NABLA_E_HIP, NABLA_E_WORKSPACE = range(5)
NABLA_F32, NABLA_BF16 = 0, 1

# Every symbol that include/nabla.h declares.
EXPORTS = (
    "nabla_reorder",
    "nabla_build_mask_workspace_size",
    "nabla_build_mask",
    "nabla_build_mask_raster",
    "nabla_build_mask_raster_noalloc",
    "nabla_build_mask_sip",
    "nabla_build_mask_ibcs_workspace_size",
    "nabla_build_mask_ibcs",
    "nabla_build_mask_ibcs_raster",
    "nabla_build_mask_ibcs_sip",
    "block_sparse_attn_fwd_weighted",
    "block_sparse_attn_fwd",
    "block_sparse_attn_fwd_raster",
    "block_sparse_attn_fwd_lse",
    "block_sparse_attn_fwd_lse_raster",
    "nabla_attn_bwd_workspace_size",
    "block_sparse_attn_bwd",
    "block_sparse_attn_bwd_raster",
    "nabla_status_string",
    "nabla_last_error",
)


class NablaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class StaWindow(ctypes.Structure):
    _fields_ = [("wt", ctypes.c_int), ("wh", ctypes.c_int), ("ww", ctypes.c_int)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libnabla.so and declare its signatures (no GPU needed to load)."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m block_sparse_attention_blockmean_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.nabla_reorder.argtypes = [vp, vp, i, i, i, i, i, i, i, i, i, vp]
    lib.nabla_reorder.restype = i
    lib.nabla_build_mask_workspace_size.argtypes = [i, i, i, i, i]
    lib.nabla_build_mask_workspace_size.restype = sz
    lib.nabla_build_mask.argtypes = [vp, vp, i, i, i, i, i, i, i, i, f, ctypes.POINTER(StaWindow),
                                     f, i, vp, vp, vp, vp, vp, sz, vp]
    lib.nabla_build_mask.restype = i
    lib.nabla_build_mask_raster.argtypes = lib.nabla_build_mask.argtypes
    lib.nabla_build_mask_raster.restype = i
    lib.nabla_build_mask_raster_noalloc.argtypes = [vp, vp, i, i, i, i, i, i, i, i, f, ctypes.POINTER(StaWindow),
                                                    f, i, vp, vp, vp, vp, vp]
    lib.nabla_build_mask_raster_noalloc.restype = i
    lib.nabla_build_mask_ibcs.argtypes = [vp, vp, i, i, i, i, i, i, i, i, i, f, ctypes.POINTER(StaWindow),
                                          f, i, vp, vp, vp, vp, vp, sz, vp]
    lib.nabla_build_mask_ibcs.restype = i
    lib.nabla_build_mask_ibcs_raster.argtypes = lib.nabla_build_mask_ibcs.argtypes
    lib.nabla_build_mask_ibcs_raster.restype = i
    lib.nabla_build_mask_ibcs_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.nabla_build_mask_ibcs_sip.argtypes = [vp, vp, i, i, i, i, i, i, i, i, i, i, vp, f, i, vp, vp, vp, vp, vp, vp,
                                              sz, vp]
    lib.nabla_build_mask_ibcs_sip.restype = i
    lib.nabla_build_mask_ibcs_workspace_size.restype = sz
    lib.block_sparse_attn_fwd_raster.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, vp, vp, f, i, vp]
    lib.block_sparse_attn_fwd_raster.restype = i
    lib.nabla_build_mask_sip.argtypes = [vp, vp, i, i, i, i, i, i, i, i, i, vp, f, i, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.nabla_build_mask_sip.restype = i
    lib.block_sparse_attn_fwd_weighted.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, vp, vp, vp, f, i, vp]
    lib.block_sparse_attn_fwd_weighted.restype = i
    lib.block_sparse_attn_fwd.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, vp, vp, f, i, vp]
    lib.block_sparse_attn_fwd.restype = i
    lib.block_sparse_attn_fwd_lse.argtypes = [vp, vp, vp, vp, i, i, i, i, i, vp, vp, vp, f, i, vp, vp]
    lib.block_sparse_attn_fwd_lse.restype = i
    lib.block_sparse_attn_fwd_lse_raster.argtypes = [vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, vp, vp, f, i, vp,
                                                     vp]
    lib.block_sparse_attn_fwd_lse_raster.restype = i
    lib.nabla_attn_bwd_workspace_size.argtypes = [i, i, i, i]
    lib.nabla_attn_bwd_workspace_size.restype = sz
    lib.block_sparse_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, f, i,
                                          vp, sz, vp]
    lib.block_sparse_attn_bwd.restype = i
    lib.block_sparse_attn_bwd_raster.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i, vp, vp,
                                                 f, i, vp, sz, vp]
    lib.block_sparse_attn_bwd_raster.restype = i
    lib.nabla_status_string.argtypes = [i]
    lib.nabla_status_string.restype = ctypes.c_char_p
    lib.nabla_last_error.argtypes = []
    lib.nabla_last_error.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(status: int, lib) -> None:
    if status != NABLA_OK:
        name = lib.nabla_status_string(status).decode()
        msg = lib.nabla_last_error().decode()
        raise NablaError(status, f"{name}: {msg}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return NABLA_BF16
    if t.dtype == torch.float32:
        return NABLA_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use bfloat16 or float32")


def _dev(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def reorder(x: torch.Tensor, T: int, H: int, W: int, P: int, inverse: bool = False,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Raster <-> fractal token order of a [B, heads, T*H*W, d] tensor."""
    lib = load_library()
    if x.dim() != 4:
        raise ValueError("x must be [batch, heads, L, d]")
    B, NH, L, d = x.shape
    if L != T * H * W:
        raise ValueError(f"L={L} does not match T*H*W={T * H * W}")
    if out is None:
        out = torch.empty_like(x)
    _check(lib.nabla_reorder(_dev(x, "x"), _dev(out, "out"), B, NH, T, H, W, d, P,
                             _dtype_code(x), int(bool(inverse)), _stream()), lib)
    return out


def build_mask_workspace_size(batch: int, heads: int, L: int, d: int, N: int = 64,
                              ibcs: bool = False, ibcs_group: int = 128) -> int:
    lib = load_library()
    if ibcs:
        return int(lib.nabla_build_mask_ibcs_workspace_size(batch, heads, L, d, N, ibcs_group))
    return int(lib.nabla_build_mask_workspace_size(batch, heads, L, d, N))


def build_mask(q: torch.Tensor, k: torch.Tensor, T: int, H: int, W: int, P: int, N: int = 64,
               thr: float = 0.1, sta: Optional[Tuple[int, int, int]] = None,
               scale: Optional[float] = None, with_bitmap: bool = False,
               with_schedule: bool = False, workspace: Optional[torch.Tensor] = None,
               kv_count: Optional[torch.Tensor] = None, kv_index: Optional[torch.Tensor] = None,
               schedule: Optional[torch.Tensor] = None, raster: bool = False,
               ibcs: bool = False, ibcs_group: int = 128):
    """NABLA block mask of fractal-ordered Q, K (``raster=True``: Q, K in raster order,
    the fractal flattening applied in the addressing; needs N == P*P; ``ibcs=True``: the
    block scores come from 8 clusters of each group of ``ibcs_group`` queries, 128 as on
    the AB-Attention page or 64, instead of the mean query).

    Returns (kv_count, kv_index), plus the bitmap and/or the longest-first
    schedule when asked for (in that order)."""
    lib = load_library()
    _check_mask_inputs(q, k, T, H, W, N)
    B, NH, L, d = q.shape
    nb = L // N
    _check_int32(kv_count, "kv_count", B * NH * nb)
    _check_int32(kv_index, "kv_index", B * NH * nb * nb)
    _check_int32(schedule, "schedule", B * NH * nb)
    dev = q.device
    if kv_count is None:
        kv_count = torch.empty((B, NH, nb), dtype=torch.int32, device=dev)
    if kv_index is None:
        kv_index = torch.empty((B, NH, nb, nb), dtype=torch.int32, device=dev)
    bitmap = None
    if with_bitmap:
        bitmap = torch.empty((B, NH, nb, (nb + 31) // 32), dtype=torch.int32, device=dev)
    if with_schedule and schedule is None:
        schedule = torch.empty((B * NH * nb,), dtype=torch.int32, device=dev)
    ws_bytes = build_mask_workspace_size(B, NH, L, d, N, ibcs=ibcs, ibcs_group=ibcs_group)
    if workspace is None:
        workspace = torch.empty(max(int(ws_bytes), 1), dtype=torch.uint8, device=dev)
    win = None if sta is None else ctypes.byref(StaWindow(*sta))
    # the IBCS entry takes the query-group size right after N
    shape = (B, NH, T, H, W, d, P, N) + ((int(ibcs_group),) if ibcs else ())
    if ibcs:
        entry = lib.nabla_build_mask_ibcs_raster if raster else lib.nabla_build_mask_ibcs
    else:
        entry = lib.nabla_build_mask_raster if raster else lib.nabla_build_mask
    _check(entry(
        _dev(q, "q"), _dev(k, "k"), *shape, float(thr), win,
        float(scale) if scale is not None else 0.0, _dtype_code(q),
        _dev(kv_count, "kv_count"), _dev(kv_index, "kv_index"),
        _dev(bitmap, "bitmap") if bitmap is not None else None,
        _dev(schedule, "schedule") if schedule is not None else None,
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream()), lib)
    out = [kv_count, kv_index]
    if with_bitmap:
        out.append(bitmap)
    if with_schedule or schedule is not None:
        out.append(schedule)
    return tuple(out)


def build_mask_raster_noalloc(q: torch.Tensor, k: torch.Tensor, T: int, H: int, W: int, P: int,
                              kv_count: torch.Tensor, kv_index: torch.Tensor, N: int = 64, thr: float = 0.1,
                              sta: Optional[Tuple[int, int, int]] = None, scale: Optional[float] = None,
                              bitmap: Optional[torch.Tensor] = None, schedule: Optional[torch.Tensor] = None):
    """The NABLA mask of raster-order Q, K through the entry point that allocates nothing:
    the caller passes every output (int32 kv_count [B, heads, nb], kv_index
    [B, heads, nb, nb], optional int32 bitmap [B, heads, nb, ceil(nb/32)] and schedule
    [B*heads*nb]); the pooled means live in the library's own device array.  Calls that
    overlap on one GPU race on that array."""
    lib = load_library()
    _check_mask_inputs(q, k, T, H, W, N)
    B, NH, L, d = q.shape
    nb = L // N
    _check_int32(kv_count, "kv_count", B * NH * nb)
    _check_int32(kv_index, "kv_index", B * NH * nb * nb)
    _check_int32(bitmap, "bitmap", B * NH * nb * ((nb + 31) // 32))
    _check_int32(schedule, "schedule", B * NH * nb)
    win = None if sta is None else ctypes.byref(StaWindow(*sta))
    _check(lib.nabla_build_mask_raster_noalloc(
        _dev(q, "q"), _dev(k, "k"), B, NH, T, H, W, d, P, N, float(thr), win,
        float(scale) if scale is not None else 0.0, _dtype_code(q),
        _dev(kv_count, "kv_count"), _dev(kv_index, "kv_index"),
        _dev(bitmap, "bitmap") if bitmap is not None else None,
        _dev(schedule, "schedule") if schedule is not None else None, _stream()), lib)


def _check_mask_inputs(q: torch.Tensor, k: torch.Tensor, T: int, H: int, W: int, N: int) -> None:
    """Shape checks shared by the mask entry points, before any pointer is taken: the
    library sizes its outputs from T*H*W, so q's token count must equal it."""
    if q.dim() != 4:
        raise ValueError("q must be [batch, heads, L, d]")
    if k.shape != q.shape or k.dtype != q.dtype:
        raise ValueError("q and k must have the same shape and dtype")
    L = q.shape[2]
    if L != T * H * W:
        raise ValueError(f"L={L} does not match T*H*W={T * H * W}")
    if N <= 0 or L % N:
        raise ValueError(f"L={L} is not a multiple of N={N}")


def _check_int32(t: Optional[torch.Tensor], name: str, numel: int) -> None:
    """A caller-supplied int32 output or list must hold exactly ``numel`` entries."""
    if t is None:
        return
    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32")
    if t.numel() != numel:
        raise ValueError(f"{name} holds {t.numel()} entries, {numel} needed")


def _check_lists(q: torch.Tensor, kv_count: torch.Tensor, kv_index: torch.Tensor, N: int) -> None:
    B, NH, L, d = q.shape
    nb = L // N
    if kv_count.dtype != torch.int32 or kv_index.dtype != torch.int32:
        raise TypeError("kv_count and kv_index must be int32")
    if kv_count.numel() != B * NH * nb or kv_index.numel() != B * NH * nb * nb:
        raise ValueError("kv_count / kv_index sizes do not match q")
    if L % N:
        raise ValueError(f"L={L} is not a multiple of N={N}")


def attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_count: torch.Tensor,
             kv_index: torch.Tensor, N: int = 64, scale: Optional[float] = None,
             out: Optional[torch.Tensor] = None,
             schedule: Optional[torch.Tensor] = None, with_lse: bool = False,
             lse: Optional[torch.Tensor] = None):
    """Block-sparse attention over the kept N x N tiles listed in kv_count/kv_index.

    With ``with_lse`` (or an ``lse`` tensor) it also returns the float32 [B, heads, L]
    log-sum-exp of every query row, as (out, lse), which ``attn_bwd`` needs."""
    if with_lse or lse is not None:
        lib = load_library()
        B, NH, L, d = q.shape
        if lse is None:
            lse = torch.empty((B, NH, L), dtype=torch.float32, device=q.device)
        if lse.dtype != torch.float32 or lse.numel() != B * NH * L:
            raise ValueError("lse must hold batch*heads*L float32 values")
        for name, t in (("k", k), ("v", v)):
            if t.shape != q.shape or t.dtype != q.dtype:
                raise ValueError(f"{name} must match q in shape and dtype")
        _check_lists(q, kv_count, kv_index, N)
        if out is None:
            out = torch.empty_like(q)
        _check(lib.block_sparse_attn_fwd_lse(
            _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"), B, NH, L, d, N,
            _dev(kv_count, "kv_count"), _dev(kv_index, "kv_index"),
            _dev(schedule, "schedule") if schedule is not None else None,
            float(scale) if scale is not None else 0.0, _dtype_code(q), _dev(lse, "lse"), _stream()), lib)
        return out, lse
    lib = load_library()
    B, NH, L, d = q.shape
    for name, t in (("k", k), ("v", v)):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    nb = L // N
    if kv_count.dtype != torch.int32 or kv_index.dtype != torch.int32:
        raise TypeError("kv_count and kv_index must be int32")
    if kv_count.numel() != B * NH * nb or kv_index.numel() != B * NH * nb * nb:
        raise ValueError("kv_count / kv_index sizes do not match q")
    if schedule is not None:
        if schedule.dtype != torch.int32 or schedule.numel() != B * NH * nb:
            raise ValueError("schedule must hold batch*heads*nb int32 entries")
    if out is None:
        out = torch.empty_like(q)
    _check(lib.block_sparse_attn_fwd(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"), B, NH, L, d, N,
        _dev(kv_count, "kv_count"), _dev(kv_index, "kv_index"),
        _dev(schedule, "schedule") if schedule is not None else None,
        float(scale) if scale is not None else 0.0, _dtype_code(q), _stream()), lib)
    return out


def build_mask_sip(q: torch.Tensor, k: torch.Tensor, T: int, H: int, W: int, P: int, budget: int,
                   uniforms: torch.Tensor, N: int = 64, scale: Optional[float] = None,
                   with_bitmap: bool = False, with_schedule: bool = False,
                   workspace: Optional[torch.Tensor] = None, ibcs: bool = False, ibcs_group: int = 128):
    """SIP block selection of fractal-ordered Q, K: returns (kv_count, kv_index, kv_logw),
    plus the bitmap and/or schedule when asked for.  ``uniforms`` is a float32
    [B, heads, nb, nb] tensor of draws in [0, 1).  The scores sampled from are NABLA's
    pooled map, or with ``ibcs=True`` the IBCS scores of ``ibcs_group``-query clusters."""
    lib = load_library()
    _check_mask_inputs(q, k, T, H, W, N)
    B, NH, L, d = q.shape
    nb = L // N
    if uniforms.dtype != torch.float32 or uniforms.numel() != B * NH * nb * nb:
        raise ValueError("uniforms must hold batch*heads*nb*nb float32 values")
    dev = q.device
    kv_count = torch.empty((B, NH, nb), dtype=torch.int32, device=dev)
    kv_index = torch.empty((B, NH, nb, nb), dtype=torch.int32, device=dev)
    kv_logw = torch.empty((B, NH, nb, nb), dtype=torch.float32, device=dev)
    bitmap = torch.empty((B, NH, nb, (nb + 31) // 32), dtype=torch.int32, device=dev) if with_bitmap else None
    schedule = torch.empty((B * NH * nb,), dtype=torch.int32, device=dev) if with_schedule else None
    ws_bytes = build_mask_workspace_size(B, NH, L, d, N, ibcs=ibcs, ibcs_group=ibcs_group)
    if workspace is None:
        workspace = torch.empty(max(int(ws_bytes), 1), dtype=torch.uint8, device=dev)
    # the IBCS entry takes the query-group size right after N
    shape = (B, NH, T, H, W, d, P, N) + ((int(ibcs_group),) if ibcs else ())
    entry = lib.nabla_build_mask_ibcs_sip if ibcs else lib.nabla_build_mask_sip
    _check(entry(
        _dev(q, "q"), _dev(k, "k"), *shape, int(budget), _dev(uniforms, "uniforms"),
        float(scale) if scale is not None else 0.0, _dtype_code(q), _dev(kv_count, "kv_count"),
        _dev(kv_index, "kv_index"), _dev(kv_logw, "kv_logw"),
        _dev(bitmap, "bitmap") if bitmap is not None else None,
        _dev(schedule, "schedule") if schedule is not None else None,
        _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream()), lib)
    out = [kv_count, kv_index, kv_logw]
    if with_bitmap:
        out.append(bitmap)
    if with_schedule:
        out.append(schedule)
    return tuple(out)


def attn_fwd_weighted(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_count: torch.Tensor,
                      kv_index: torch.Tensor, kv_logw: torch.Tensor, N: int = 64,
                      scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                      schedule: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Block-sparse attention with the per-tile logit shifts ``kv_logw`` (SIP weights)."""
    lib = load_library()
    B, NH, L, d = q.shape
    for name, t in (("k", k), ("v", v)):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    _check_lists(q, kv_count, kv_index, N)
    if kv_logw.dtype != torch.float32 or kv_logw.numel() != kv_index.numel():
        raise ValueError("kv_logw must be float32 shaped like kv_index")
    if out is None:
        out = torch.empty_like(q)
    _check(lib.block_sparse_attn_fwd_weighted(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"), B, NH, L, d, N,
        _dev(kv_count, "kv_count"), _dev(kv_index, "kv_index"), _dev(kv_logw, "kv_logw"),
        _dev(schedule, "schedule") if schedule is not None else None,
        float(scale) if scale is not None else 0.0, _dtype_code(q), _stream()), lib)
    return out


def attn_fwd_raster(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_count: torch.Tensor,
                    kv_index: torch.Tensor, T: int, H: int, W: int, P: int, N: int = 64,
                    scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                    schedule: Optional[torch.Tensor] = None, with_lse: bool = False,
                    lse: Optional[torch.Tensor] = None):
    """Block-sparse attention of raster-ordered Q, K, V (output in raster order) under
    lists that number blocks in fractal order (``build_mask(..., raster=True)``).

    With ``with_lse`` (or an ``lse`` tensor) it also returns the float32 [B, heads, L]
    log-sum-exp of every query row in raster order, as (out, lse), which
    ``attn_bwd_raster`` needs."""
    lib = load_library()
    B, NH, L, d = q.shape
    if L != T * H * W:
        raise ValueError(f"L={L} does not match T*H*W={T * H * W}")
    for name, t in (("k", k), ("v", v)):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    _check_lists(q, kv_count, kv_index, N)
    if schedule is not None and (schedule.dtype != torch.int32 or schedule.numel() != B * NH * (L // N)):
        raise ValueError("schedule must hold batch*heads*nb int32 entries")
    if out is None:
        out = torch.empty_like(q)
    sched = _dev(schedule, "schedule") if schedule is not None else None
    scale_arg = float(scale) if scale is not None else 0.0
    if with_lse or lse is not None:
        if lse is None:
            lse = torch.empty((B, NH, L), dtype=torch.float32, device=q.device)
        if lse.dtype != torch.float32 or lse.numel() != B * NH * L:
            raise ValueError("lse must hold batch*heads*L float32 values")
        _check(lib.block_sparse_attn_fwd_lse_raster(
            _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"), B, NH, T, H, W, d, P, N,
            _dev(kv_count, "kv_count"), _dev(kv_index, "kv_index"), sched, scale_arg, _dtype_code(q),
            _dev(lse, "lse"), _stream()), lib)
        return out, lse
    _check(lib.block_sparse_attn_fwd_raster(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(out, "out"), B, NH, T, H, W, d, P, N,
        _dev(kv_count, "kv_count"), _dev(kv_index, "kv_index"), sched, scale_arg, _dtype_code(q), _stream()), lib)
    return out


def attn_bwd_workspace_size(batch: int, heads: int, L: int, N: int = 64) -> int:
    return int(load_library().nabla_attn_bwd_workspace_size(batch, heads, L, N))


def attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, dout: torch.Tensor,
             lse: torch.Tensor, kv_count: torch.Tensor, kv_index: torch.Tensor, N: int = 64,
             scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
             dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
             dv: Optional[torch.Tensor] = None, raster: Optional[tuple] = None):
    """Gradients (dq, dk, dv) of sum(o * dout) for o = attn_fwd(q, k, v, ...) under the
    same lists; ``o`` and ``lse`` come from ``attn_fwd(..., with_lse=True)``.

    ``raster=(T, H, W, P)``: every tensor (gradients too) is in raster order, ``o`` and
    ``lse`` from ``attn_fwd_raster(..., with_lse=True)``."""
    lib = load_library()
    B, NH, L, d = q.shape
    if raster is not None:
        T, H, W, P = (int(x) for x in raster)
        if L != T * H * W:
            raise ValueError(f"L={L} does not match T*H*W={T * H * W}")
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout)):
        if t.shape != q.shape or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in shape and dtype")
    if lse.dtype != torch.float32 or lse.numel() != B * NH * L:
        raise ValueError("lse must hold batch*heads*L float32 values")
    _check_lists(q, kv_count, kv_index, N)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    ws_bytes = int(lib.nabla_attn_bwd_workspace_size(B, NH, L, N))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    ptrs = (_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(o, "o"), _dev(dout, "dout"), _dev(lse, "lse"),
            _dev(dq, "dq"), _dev(dk, "dk"), _dev(dv, "dv"))
    rest = (_dev(kv_count, "kv_count"), _dev(kv_index, "kv_index"),
            float(scale) if scale is not None else 0.0, _dtype_code(q),
            _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(), _stream())
    if raster is not None:
        _check(lib.block_sparse_attn_bwd_raster(*ptrs, B, NH, T, H, W, d, P, N, *rest), lib)
    else:
        _check(lib.block_sparse_attn_bwd(*ptrs, B, NH, L, d, N, *rest), lib)
    return dq, dk, dv
