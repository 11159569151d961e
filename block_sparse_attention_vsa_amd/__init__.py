"""Block-sparse attention over a 3D video token grid on AMD MI355X (gfx950).

Thin Python binding of libvsa.so: every function has the name of the C entry
point it calls and does argument marshalling only (shape checks, output
allocation through torch, the current HIP stream). Every step of the path runs
in the library's HIP kernels; there is no fallback: if libvsa.so is missing or
fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
# VSA_LIBRARY names another build of the same library (the host-sanitized one
# the CPU tests load); by default the in-tree libvsa.so
LIB_PATH = os.environ.get("VSA_LIBRARY") or os.path.join(HERE, "libvsa.so")

VSA_OK, VSA_ERR_INVALID, VSA_ERR_UNSUPPORTED, VSA_ERR_LAUNCH, VSA_ERR_WORKSPACE = range(5)
VSA_BF16, VSA_F32 = 0, 1
VSA_PERM_FRAME_MAJOR, VSA_PERM_CUBE4 = 0, 1
VSA_PATTERN_SPATIAL, VSA_PATTERN_TEMPORAL = 0, 1
VSA_FP8_ROWS, VSA_FP8_VT = 0, 1
VSA_SKIPARSE_TOKEN, VSA_SKIPARSE_GROUP = 0, 1


class vsa_grid(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("Hh", ctypes.c_int32), ("W", ctypes.c_int32)]


class vsa_blocks(ctypes.Structure):
    _fields_ = [("mask", ctypes.c_void_p), ("kv_idx", ctypes.c_void_p), ("kv_cnt", ctypes.c_void_p),
                ("max_kv", ctypes.c_int32)]


class VsaError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        super().__init__(f"{func}: status {status}: {msg}")
        self.status = status


_P, _I, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
_SIGNATURES = {
    "vsa_status_string": (ctypes.c_char_p, [_I]),
    "vsa_last_error": (ctypes.c_char_p, []),
    "vsa_version": (_I, []),
    "vsa_selftest_host": (_I, []),
    "vsa_cube_dims": (_I, [vsa_grid, _P, _P]),
    "vsa_pattern_mask": (_I, [vsa_grid, _I, _I, _I, _P, _P]),
    "vsa_cube_block_len": (_I, [vsa_grid, _P, _P]),
    "vsa_permute": (_I, [_P, _P, _I, _I, vsa_grid, _I, _I, _I, _I, _P, _P]),
    "vsa_skiparse_dims": (_I, [vsa_grid, _I, _I, _I, _P, _P]),
    "vsa_skiparse_block_len": (_I, [vsa_grid, _I, _I, _I, _P, _P]),
    "vsa_skiparse_mask": (_I, [vsa_grid, _I, _I, _I, _P, _P]),
    "vsa_skiparse_permute": (_I, [_P, _P, _I, _I, vsa_grid, _I, _I, _I, _I, _I, _I, _P]),
    "vsa_block_scores": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, _F, _P, _P, _P, _P]),
    "vsa_select_topk": (_I, [_P, _I, _I, _I, _I, _P, _I, _F, _P, _P, _P]),
    "vsa_profile_workspace_bytes": (_SZ, [_I, _I, vsa_grid, _I, _I, _I]),
    "vsa_profile_heads": (_I, [_P, _P, _P, _I, _I, vsa_grid, _I, _I, _I, _P, _I, _P, _P, _I, _F,
                               _P, _P, _P, _SZ, _P]),
    "vsa_profile_scratch_capacity": (_SZ, []),
    "vsa_profile_heads_noalloc": (_I, [_P, _P, _P, _I, _I, vsa_grid, _I, _I, _I, _P, _I, _P, _P, _I, _F,
                                       _P, _P, _P]),
    "vsa_mask_to_list": (_I, [_P, _I, _I, _I, _I, _P, _I, _I, _P, _P, _P]),
    "vsa_attn_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "vsa_block_sparse_attn_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P,
                                       ctypes.POINTER(vsa_blocks), _F, _P, _SZ, _P]),
    "vsa_block_sparse_attn_fwd_permuted": (_I, [_P, _P, _P, _P, _P, _I, _I, vsa_grid, _I, _I, _I, _P, _P,
                                                ctypes.POINTER(vsa_blocks), _F, _P]),
    "vsa_block_sparse_attn_fwd_chosen": (_I, [_P, _P, _P, _P, _P, _I, _I, vsa_grid, _I, _I, _I, _P, _P, _I, _P,
                                              _P, _F, _P]),
    "vsa_attn_bwd_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "vsa_block_sparse_attn_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P,
                                       ctypes.POINTER(vsa_blocks), _F, _P, _SZ, _P]),
    "vsa_kmeans_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "vsa_kmeans": (_I, [_P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _SZ, _P]),
    "vsa_cluster_order_workspace_bytes": (_SZ, [_I, _I, _I, _I]),
    "vsa_cluster_order": (_I, [_P, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "vsa_gather_rows": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _I, _P]),
    "vsa_cluster_scores": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _F, _P, _P]),
    "vsa_varlen_attn_workspace_bytes": (_SZ, [_I, _I, _I, _I]),
    "vsa_varlen_sparse_attn_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _I, _P, _I,
                                        ctypes.POINTER(vsa_blocks), _F, _P, _SZ, _P]),
    "vsa_fp8_quantize": (_I, [_P, _I, _I, _I, _I, _I, _I, _P, _P, _P]),
    "vsa_block_sparse_attn_fwd_fp8": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P,
                                           ctypes.POINTER(vsa_blocks), _F, _P]),
    "vsa_check_block_list_host": (_I, [_P, _P, _I64, _I, _I]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libvsa.so (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m block_sparse_attention_vsa_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def _check(status: int, func: str):
    if status != VSA_OK:
        raise VsaError(status, func, lib().vsa_last_error().decode())


# ---------------------------------------------------------------- helpers ----
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return VSA_BF16
    if t.dtype == torch.float32:
        return VSA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _expect(t, name, shape=None, dtype=None, ndim=None):
    """Type, dtype, exact shape and layout of a tensor argument. The kernels
    index every buffer from the sizes alone, so a tensor of the wrong shape is
    rejected here, before any call. Devices are checked separately
    (_on_device), after every shape."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if shape is not None:
        want = tuple(int(x) for x in shape)
        if tuple(t.shape) != want:
            raise ValueError(f"{name} must have shape {want}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _expect_workspace(ws, name, need: int):
    torch = _torch()
    _expect(ws, name, dtype=torch.uint8, ndim=1)
    if ws.numel() < need:
        raise ValueError(f"{name} needs at least {need} bytes, got {ws.numel()}")


def _on_device(first, **others):
    """Every tensor argument lives on the GPU, on `first`'s device."""
    if not first.is_cuda:
        raise ValueError("tensors must be device tensors")
    for name, t in others.items():
        if t is not None and t.device != first.device:
            raise ValueError(f"{name} must be on {first.device}, got {t.device}")


def _grid(grid) -> vsa_grid:
    T, Hh, W = (int(x) for x in grid)
    return vsa_grid(T, Hh, W)


def _nb(N: int, bs: int) -> int:
    if bs <= 0:
        raise ValueError("block size must be positive")
    return -(-N // bs)


def _same_shape(ref, **ts):
    for name, t in ts.items():
        if tuple(t.shape) != tuple(ref.shape):
            raise ValueError(f"{name} must have shape {tuple(ref.shape)}, got {tuple(t.shape)}")


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)


def _blocks_arg(B, H, nqb, nkb, mask, kv_idx, kv_cnt):
    """The block set (exactly one form): mask uint8 [B, H, nqb, nkb], or kv_idx
    int32 [B, H, nqb, max_kv] with kv_cnt int32 [B, H, nqb]."""
    torch = _torch()
    blocks = vsa_blocks()
    if (mask is None) == (kv_idx is None and kv_cnt is None):
        raise ValueError("give exactly one of mask or (kv_idx, kv_cnt)")
    if mask is not None:
        _expect(mask, "mask", (B, H, nqb, nkb), torch.uint8)
        blocks.mask = mask.data_ptr()
    else:
        if kv_idx is None or kv_cnt is None:
            raise ValueError("the list form needs both kv_idx and kv_cnt")
        _expect(kv_idx, "kv_idx", dtype=torch.int32, ndim=4)
        _expect(kv_idx, "kv_idx", (B, H, nqb, kv_idx.shape[-1]))
        if kv_idx.shape[-1] < 1:
            raise ValueError("kv_idx needs max_kv >= 1")
        _expect(kv_cnt, "kv_cnt", (B, H, nqb), torch.int32)
        blocks.kv_idx = kv_idx.data_ptr()
        blocks.kv_cnt = kv_cnt.data_ptr()
        blocks.max_kv = kv_idx.shape[-1]
    return blocks


def _qkv(q, k, v):
    _expect(q, "q", ndim=4)
    _expect(k, "k", q.shape, q.dtype)
    _expect(v, "v", q.shape, q.dtype)
    return q.shape


def _outputs(q, out, lse, return_lse, B, H, N, D, dtype=None):
    """O (allocated like q unless given) and LSE [B, H, N] fp32 (allocated when
    asked for unless given), both shape-checked."""
    torch = _torch()
    dtype = q.dtype if dtype is None else dtype
    if out is None:
        out = torch.empty((B, H, N, D), dtype=dtype, device=q.device)
    _expect(out, "out", (B, H, N, D), dtype)
    if return_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if lse is not None:
        _expect(lse, "lse", (B, H, N), torch.float32)
    return out, lse


# ------------------------------------------------------------- entry points --
def vsa_status_string(status: int) -> str:
    return lib().vsa_status_string(status).decode()


def vsa_last_error() -> str:
    return lib().vsa_last_error().decode()


def vsa_version() -> int:
    return lib().vsa_version()


def vsa_selftest_host() -> None:
    _check(lib().vsa_selftest_host(), "vsa_selftest_host")


def vsa_cube_dims(grid):
    nc, ns = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().vsa_cube_dims(_grid(grid), ctypes.byref(nc), ctypes.byref(ns)), "vsa_cube_dims")
    return nc.value, ns.value


def vsa_pattern_mask(grid, bs: int, pattern: int, w: int, device="cuda", out=None):
    torch = _torch()
    nb = _nb(int(np.prod(grid)), bs)
    if out is None:
        out = torch.empty((nb, nb), dtype=torch.uint8, device=device)
    _expect(out, "out", (nb, nb), torch.uint8)
    _on_device(out)
    _check(lib().vsa_pattern_mask(_grid(grid), bs, pattern, w, _ptr(out), _stream(out.device)), "vsa_pattern_mask")
    return out


def vsa_cube_block_len(grid, device="cuda", out=None):
    torch = _torch()
    nc, _ = vsa_cube_dims(grid)
    if out is None:
        out = torch.empty((nc,), dtype=torch.int32, device=device)
    _expect(out, "out", (nc,), torch.int32)
    _on_device(out)
    _check(lib().vsa_cube_block_len(_grid(grid), _ptr(out), _stream(out.device)), "vsa_cube_block_len")
    return out


def vsa_permute(src, grid, kind: int, inverse: bool = False, head_sel=None, out=None):
    torch = _torch()
    _expect(src, "src", ndim=4)
    B, H, rows_in, D = src.shape
    N = int(np.prod(grid))
    rows_out = N
    if kind == VSA_PERM_CUBE4:
        n_slots = vsa_cube_dims(grid)[1]
        rows_in_want, rows_out = (n_slots, N) if inverse else (N, n_slots)
    else:
        rows_in_want = N
    if rows_in != rows_in_want:
        raise ValueError(f"src must hold {rows_in_want} rows per head for this grid, got {rows_in}")
    if out is None:
        out = torch.empty((B, H, rows_out, D), dtype=src.dtype, device=src.device)
    _expect(out, "out", (B, H, rows_out, D), src.dtype)
    hs = None
    if head_sel is not None:
        if len(head_sel) != H:
            raise ValueError("head_sel needs one flag per head")
        hs_arr = (ctypes.c_uint8 * H)(*[1 if x else 0 for x in head_sel])
        hs = ctypes.cast(hs_arr, ctypes.c_void_p)
    _on_device(src, out=out)
    _check(lib().vsa_permute(_ptr(src), _ptr(out), B, H, _grid(grid), D, _dtype_code(src), kind, int(bool(inverse)),
                             hs, _stream(src.device)), "vsa_permute")
    return out


def vsa_skiparse_dims(grid, mode: int, k: int, bs: int):
    """(n_slots, n_blocks) of the padded Skiparse-2D layout."""
    ns, nb = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().vsa_skiparse_dims(_grid(grid), mode, k, bs, ctypes.byref(ns), ctypes.byref(nb)), "vsa_skiparse_dims")
    return ns.value, nb.value


def vsa_skiparse_block_len(grid, mode: int, k: int, bs: int, device="cuda", out=None):
    torch = _torch()
    _, nb = vsa_skiparse_dims(grid, mode, k, bs)
    if out is None:
        out = torch.empty((nb,), dtype=torch.int32, device=device)
    _expect(out, "out", (nb,), torch.int32)
    _on_device(out)
    _check(lib().vsa_skiparse_block_len(_grid(grid), mode, k, bs, _ptr(out), _stream(out.device)),
           "vsa_skiparse_block_len")
    return out


def vsa_skiparse_mask(grid, mode: int, k: int, bs: int, device="cuda", out=None):
    torch = _torch()
    _, nb = vsa_skiparse_dims(grid, mode, k, bs)
    if out is None:
        out = torch.empty((nb, nb), dtype=torch.uint8, device=device)
    _expect(out, "out", (nb, nb), torch.uint8)
    _on_device(out)
    _check(lib().vsa_skiparse_mask(_grid(grid), mode, k, bs, _ptr(out), _stream(out.device)), "vsa_skiparse_mask")
    return out


def vsa_skiparse_permute(src, grid, mode: int, k: int, bs: int, inverse: bool = False, out=None):
    torch = _torch()
    _expect(src, "src", ndim=4)
    B, H, rows_in, D = src.shape
    N = int(np.prod(grid))
    n_slots, _ = vsa_skiparse_dims(grid, mode, k, bs)
    want_in, rows_out = (n_slots, N) if inverse else (N, n_slots)
    if rows_in != want_in:
        raise ValueError(f"src must hold {want_in} rows per head for this layout, got {rows_in}")
    if out is None:
        out = torch.empty((B, H, rows_out, D), dtype=src.dtype, device=src.device)
    _expect(out, "out", (B, H, rows_out, D), src.dtype)
    _on_device(src, out=out)
    _check(lib().vsa_skiparse_permute(_ptr(src), _ptr(out), B, H, _grid(grid), D, _dtype_code(src), mode, k, bs,
                                      int(bool(inverse)), _stream(src.device)), "vsa_skiparse_permute")
    return out


def vsa_block_scores(q, k, bs: int, blk_len=None, scale=None, out=None):
    torch = _torch()
    _expect(q, "q", ndim=4)
    _expect(k, "k", q.shape, q.dtype)
    B, H, N, D = q.shape
    nb = _nb(N, bs)
    scale = default_scale(D) if scale is None else scale
    if out is None:
        out = (torch.empty((B, H, nb, nb), dtype=torch.float32, device=q.device),
               torch.empty((B, H, nb, D), dtype=torch.float32, device=q.device),
               torch.empty((B, H, nb, D), dtype=torch.float32, device=q.device))
    s, qp, kp = out
    _expect(s, "scores", (B, H, nb, nb), torch.float32)
    _expect(qp, "qpool", (B, H, nb, D), torch.float32)
    _expect(kp, "kpool", (B, H, nb, D), torch.float32)
    if blk_len is not None:
        _expect(blk_len, "blk_len", (nb,), torch.int32)
    _on_device(q, k=k, scores=s, qpool=qp, kpool=kp, blk_len=blk_len)
    _check(lib().vsa_block_scores(_ptr(q), _ptr(k), B, H, N, D, _dtype_code(q), bs, _ptr(blk_len), scale, _ptr(s),
                                  _ptr(qp), _ptr(kp), _stream(q.device)), "vsa_block_scores")
    return s, qp, kp


def vsa_select_topk(scores, k_max: int, top_p: float = 1.0, forced=None, out=None):
    torch = _torch()
    _expect(scores, "scores", dtype=torch.float32, ndim=4)
    B, H, nqb, nkb = scores.shape
    if forced is not None:
        _expect(forced, "forced", (nqb, nkb), torch.uint8)
    if out is None:
        out = (torch.empty((B, H, nqb, k_max), dtype=torch.int32, device=scores.device),
               torch.empty((B, H, nqb), dtype=torch.int32, device=scores.device))
    idx, cnt = out
    _expect(idx, "kv_idx", (B, H, nqb, k_max), torch.int32)
    _expect(cnt, "kv_cnt", (B, H, nqb), torch.int32)
    _on_device(scores, forced=forced, kv_idx=idx, kv_cnt=cnt)
    _check(lib().vsa_select_topk(_ptr(scores), B, H, nqb, nkb, _ptr(forced), k_max, top_p, _ptr(idx), _ptr(cnt),
                                 _stream(scores.device)), "vsa_select_topk")
    return idx, cnt


def vsa_profile_workspace_bytes(B, H, grid, D, R, P) -> int:
    return lib().vsa_profile_workspace_bytes(B, H, _grid(grid), D, R, P)


def _profile_args(q, k, v, grid, bs, rows, cand_masks, cand_layout, out):
    torch = _torch()
    B, H, N, D = _qkv(q, k, v)
    if N != int(np.prod(grid)):
        raise ValueError("N must equal T*Hh*W")
    nb = _nb(N, bs)
    _expect(rows, "rows", dtype=torch.int32, ndim=1)
    _expect(cand_masks, "cand_masks", dtype=torch.uint8, ndim=3)
    P = cand_masks.shape[0]
    _expect(cand_masks, "cand_masks", (P, nb, nb))
    if len(cand_layout) != P:
        raise ValueError("cand_layout needs one entry per candidate")
    if out is None:
        out = (torch.empty((B, H, P), dtype=torch.float32, device=q.device),
               torch.empty((B, H), dtype=torch.int32, device=q.device))
    err, choice = out
    _expect(err, "err", (B, H, P), torch.float32)
    _expect(choice, "choice", (B, H), torch.int32)
    lay = (ctypes.c_int32 * P)(*[int(x) for x in cand_layout])
    return B, H, N, D, P, rows.shape[0], err, choice, lay


def vsa_profile_heads(q, k, v, grid, bs: int, rows, cand_masks, cand_layout, scale=None, workspace=None, out=None):
    torch = _torch()
    B, H, N, D, P, R, err, choice, lay = _profile_args(q, k, v, grid, bs, rows, cand_masks, cand_layout, out)
    scale = default_scale(D) if scale is None else scale
    ws = vsa_profile_workspace_bytes(B, H, grid, D, R, P)
    if workspace is None:
        workspace = torch.empty((max(ws, 1),), dtype=torch.uint8, device=q.device)
    _expect_workspace(workspace, "workspace", ws)
    _on_device(q, k=k, v=v, rows=rows, cand_masks=cand_masks, err=err, choice=choice, workspace=workspace)
    _check(lib().vsa_profile_heads(_ptr(q), _ptr(k), _ptr(v), B, H, _grid(grid), D, _dtype_code(q), bs, _ptr(rows), R,
                                   _ptr(cand_masks), ctypes.cast(lay, ctypes.c_void_p), P, scale, _ptr(err),
                                   _ptr(choice), _ptr(workspace), workspace.numel(), _stream(q.device)),
           "vsa_profile_heads")
    return err, choice


def vsa_profile_scratch_capacity() -> int:
    return lib().vsa_profile_scratch_capacity()


def vsa_profile_heads_noalloc(q, k, v, grid, bs: int, rows, cand_masks, cand_layout, scale=None, out=None):
    """vsa_profile_heads with the library's static scratch instead of a
    workspace; pass `out` = (err [B, H, P] fp32, choice [B, H] int32) to make the
    call allocate nothing at all."""
    B, H, N, D, P, R, err, choice, lay = _profile_args(q, k, v, grid, bs, rows, cand_masks, cand_layout, out)
    scale = default_scale(D) if scale is None else scale
    _on_device(q, k=k, v=v, rows=rows, cand_masks=cand_masks, err=err, choice=choice)
    _check(lib().vsa_profile_heads_noalloc(_ptr(q), _ptr(k), _ptr(v), B, H, _grid(grid), D, _dtype_code(q), bs,
                                           _ptr(rows), R, _ptr(cand_masks), ctypes.cast(lay, ctypes.c_void_p), P,
                                           scale, _ptr(err), _ptr(choice), _stream(q.device)),
           "vsa_profile_heads_noalloc")
    return err, choice


def vsa_mask_to_list(mask, max_kv=None, head_mask_idx=None, B=None, H=None, out=None):
    """mask [B,H,nqb,nkb]; or mask [P,nqb,nkb] with head_mask_idx (length H) and B given."""
    torch = _torch()
    if head_mask_idx is None:
        _expect(mask, "mask", dtype=torch.uint8, ndim=4)
        B, H, nqb, nkb = mask.shape
        P = 0
        sel = None
    else:
        _expect(mask, "mask", dtype=torch.uint8, ndim=3)
        P, nqb, nkb = mask.shape
        H = len(head_mask_idx)
        B = 1 if B is None else B
        if any(not 0 <= int(x) < P for x in head_mask_idx):
            raise ValueError(f"head_mask_idx entries must lie in [0, {P})")
        arr = (ctypes.c_int32 * H)(*[int(x) for x in head_mask_idx])
        sel = ctypes.cast(arr, ctypes.c_void_p)
    max_kv = nkb if max_kv is None else max_kv
    if out is None:
        out = (torch.empty((B, H, nqb, max_kv), dtype=torch.int32, device=mask.device),
               torch.empty((B, H, nqb), dtype=torch.int32, device=mask.device))
    idx, cnt = out
    _expect(idx, "kv_idx", (B, H, nqb, max_kv), torch.int32)
    _expect(cnt, "kv_cnt", (B, H, nqb), torch.int32)
    _on_device(mask, kv_idx=idx, kv_cnt=cnt)
    _check(lib().vsa_mask_to_list(_ptr(mask), B, H, nqb, nkb, sel, P, max_kv, _ptr(idx), _ptr(cnt),
                                  _stream(mask.device)), "vsa_mask_to_list")
    return idx, cnt


def vsa_attn_workspace_bytes(B, H, N, bs, max_kv) -> int:
    return lib().vsa_attn_workspace_bytes(B, H, N, bs, max_kv)


def vsa_block_sparse_attn_fwd(q, k, v, bs: int, mask=None, kv_idx=None, kv_cnt=None, blk_len=None, scale=None,
                              return_lse=False, out=None, lse=None, workspace=None):
    torch = _torch()
    B, H, N, D = _qkv(q, k, v)
    nb = _nb(N, bs)
    scale = default_scale(D) if scale is None else scale
    blocks = _blocks_arg(B, H, nb, nb, mask, kv_idx, kv_cnt)
    if blk_len is not None:
        _expect(blk_len, "blk_len", (nb,), torch.int32)
    out, lse = _outputs(q, out, lse, return_lse, B, H, N, D)
    max_kv = blocks.max_kv if kv_idx is not None else nb
    ws = vsa_attn_workspace_bytes(B, H, N, bs, max_kv)
    if ws and workspace is None:
        workspace = torch.empty((ws,), dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _expect_workspace(workspace, "workspace", ws)
    _on_device(q, k=k, v=v, mask=mask, kv_idx=kv_idx, kv_cnt=kv_cnt, blk_len=blk_len, out=out, lse=lse,
               workspace=workspace)
    _check(lib().vsa_block_sparse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, D,
                                           _dtype_code(q), bs, _ptr(blk_len), ctypes.byref(blocks), scale,
                                           _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                           _stream(q.device)), "vsa_block_sparse_attn_fwd")
    return (out, lse) if return_lse else out


def vsa_block_sparse_attn_fwd_permuted(q, k, v, grid, bs: int, head_fm=None, mask=None, kv_idx=None, kv_cnt=None,
                                       blk_len=None, scale=None, return_lse=False, out=None, lse=None):
    """Attention with the frame-major permutation of the heads in `head_fm`
    (host sequence of H flags) folded into the kernel's loads and stores; q, k,
    v and the result are in natural order."""
    torch = _torch()
    B, H, N, D = _qkv(q, k, v)
    if N != int(np.prod(grid)):
        raise ValueError("N must equal T*Hh*W")
    nb = _nb(N, bs)
    scale = default_scale(D) if scale is None else scale
    blocks = _blocks_arg(B, H, nb, nb, mask, kv_idx, kv_cnt)
    if blk_len is not None:
        _expect(blk_len, "blk_len", (nb,), torch.int32)
    out, lse = _outputs(q, out, lse, return_lse, B, H, N, D)
    hf = None
    if head_fm is not None:
        if len(head_fm) != H:
            raise ValueError("head_fm needs one flag per head")
        hf_arr = (ctypes.c_uint8 * H)(*[1 if x else 0 for x in head_fm])
        hf = ctypes.cast(hf_arr, ctypes.c_void_p)
    _on_device(q, k=k, v=v, mask=mask, kv_idx=kv_idx, kv_cnt=kv_cnt, blk_len=blk_len, out=out, lse=lse)
    _check(lib().vsa_block_sparse_attn_fwd_permuted(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H,
                                                    _grid(grid), D, _dtype_code(q), bs, hf, _ptr(blk_len),
                                                    ctypes.byref(blocks), scale, _stream(q.device)),
           "vsa_block_sparse_attn_fwd_permuted")
    return (out, lse) if return_lse else out


def vsa_block_sparse_attn_fwd_chosen(q, k, v, grid, bs: int, cand_masks, cand_layout, choice, blk_len=None,
                                     scale=None, return_lse=False, out=None, lse=None):
    """Attention with head (b, h) using candidate mask cand_masks[choice[b, h]]
    in layout cand_layout[choice[b, h]]; `choice` is a device int32 [B, H]
    tensor (e.g. vsa_profile_heads' output), read by the kernel."""
    torch = _torch()
    B, H, N, D = _qkv(q, k, v)
    if N != int(np.prod(grid)):
        raise ValueError("N must equal T*Hh*W")
    nb = _nb(N, bs)
    _expect(cand_masks, "cand_masks", dtype=torch.uint8, ndim=3)
    P = cand_masks.shape[0]
    _expect(cand_masks, "cand_masks", (P, nb, nb))
    _expect(choice, "choice", dtype=torch.int32)
    if choice.numel() != B * H:
        raise ValueError("choice needs B*H entries")
    if len(cand_layout) != P:
        raise ValueError("cand_layout needs one entry per candidate")
    lay = (ctypes.c_int32 * P)(*[int(x) for x in cand_layout])
    scale = default_scale(D) if scale is None else scale
    if blk_len is not None:
        _expect(blk_len, "blk_len", (nb,), torch.int32)
    out, lse = _outputs(q, out, lse, return_lse, B, H, N, D)
    _on_device(q, k=k, v=v, cand_masks=cand_masks, choice=choice, blk_len=blk_len, out=out, lse=lse)
    _check(lib().vsa_block_sparse_attn_fwd_chosen(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, _grid(grid),
                                                  D, _dtype_code(q), bs, _ptr(cand_masks),
                                                  ctypes.cast(lay, ctypes.c_void_p), P, _ptr(choice), _ptr(blk_len),
                                                  scale, _stream(q.device)),
           "vsa_block_sparse_attn_fwd_chosen")
    return (out, lse) if return_lse else out


def vsa_attn_bwd_workspace_bytes(B, H, N, bs, list_form) -> int:
    return lib().vsa_attn_bwd_workspace_bytes(B, H, N, bs, int(bool(list_form)))


def vsa_block_sparse_attn_bwd(q, k, v, o, lse, dout, bs: int, mask=None, kv_idx=None, kv_cnt=None, blk_len=None,
                              scale=None, dq=None, dk=None, dv=None, workspace=None):
    """(dq, dk, dv) of the forward with the same block set; o and lse are the
    forward's outputs, dout the upstream gradient."""
    torch = _torch()
    B, H, N, D = _qkv(q, k, v)
    _expect(o, "o", q.shape, q.dtype)
    _expect(dout, "dout", q.shape, q.dtype)
    _expect(lse, "lse", (B, H, N), torch.float32)
    nb = _nb(N, bs)
    if blk_len is not None:
        _expect(blk_len, "blk_len", (nb,), torch.int32)
    blocks = _blocks_arg(B, H, nb, nb, mask, kv_idx, kv_cnt)
    scale = default_scale(D) if scale is None else scale
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _expect(t, name, q.shape, q.dtype)
    ws = vsa_attn_bwd_workspace_bytes(B, H, N, bs, kv_idx is not None)
    if workspace is None and ws:
        workspace = torch.empty((ws,), dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _expect_workspace(workspace, "workspace", ws)
    _on_device(q, k=k, v=v, o=o, dout=dout, lse=lse, mask=mask, kv_idx=kv_idx, kv_cnt=kv_cnt, blk_len=blk_len,
               dq=dq, dk=dk, dv=dv, workspace=workspace)
    _check(lib().vsa_block_sparse_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                                           _ptr(dk), _ptr(dv), B, H, N, D, _dtype_code(q), bs, _ptr(blk_len),
                                           ctypes.byref(blocks), scale, _ptr(workspace),
                                           0 if workspace is None else workspace.numel(), _stream(q.device)),
           "vsa_block_sparse_attn_bwd")
    return dq, dk, dv


def vsa_kmeans_workspace_bytes(B, H, N, C, D) -> int:
    return lib().vsa_kmeans_workspace_bytes(B, H, N, C, D)


def vsa_kmeans(x, C: int, iters: int, out=None, workspace=None):
    """Lloyd's k-means of every (b, h) of x [B, H, N, D] (bf16): returns
    (centroids fp32 [B, H, C, D], labels int32 [B, H, N], counts int32 [B, H, C])."""
    torch = _torch()
    _expect(x, "x", ndim=4)
    B, H, N, D = x.shape
    if out is None:
        out = (torch.empty((B, H, C, D), dtype=torch.float32, device=x.device),
               torch.empty((B, H, N), dtype=torch.int32, device=x.device),
               torch.empty((B, H, C), dtype=torch.int32, device=x.device))
    cent, lab, cnt = out
    _expect(cent, "centroids", (B, H, C, D), torch.float32)
    _expect(lab, "labels", (B, H, N), torch.int32)
    _expect(cnt, "counts", (B, H, C), torch.int32)
    ws = vsa_kmeans_workspace_bytes(B, H, N, C, D)
    if workspace is None:
        workspace = torch.empty((max(1, ws),), dtype=torch.uint8, device=x.device)
    _expect_workspace(workspace, "workspace", ws)
    _on_device(x, centroids=cent, labels=lab, counts=cnt, workspace=workspace)
    _check(lib().vsa_kmeans(_ptr(x), B, H, N, D, _dtype_code(x), C, iters, _ptr(cent), _ptr(lab), _ptr(cnt),
                            _ptr(workspace), workspace.numel(), _stream(x.device)), "vsa_kmeans")
    return cent, lab, cnt


def vsa_cluster_order_workspace_bytes(B, H, N, C) -> int:
    return lib().vsa_cluster_order_workspace_bytes(B, H, N, C)


def vsa_cluster_order(labels, C: int, out=None, workspace=None):
    """Stable cluster-major order: (perm int32 [B, H, N], offsets int32 [B, H, C + 1])."""
    torch = _torch()
    _expect(labels, "labels", dtype=torch.int32, ndim=3)
    B, H, N = labels.shape
    if out is None:
        out = (torch.empty((B, H, N), dtype=torch.int32, device=labels.device),
               torch.empty((B, H, C + 1), dtype=torch.int32, device=labels.device))
    perm, off = out
    _expect(perm, "perm", (B, H, N), torch.int32)
    _expect(off, "offsets", (B, H, C + 1), torch.int32)
    ws = vsa_cluster_order_workspace_bytes(B, H, N, C)
    if workspace is None:
        workspace = torch.empty((max(1, ws),), dtype=torch.uint8, device=labels.device)
    _expect_workspace(workspace, "workspace", ws)
    _on_device(labels, perm=perm, offsets=off, workspace=workspace)
    _check(lib().vsa_cluster_order(_ptr(labels), B, H, N, C, _ptr(perm), _ptr(off), _ptr(workspace),
                                   workspace.numel(), _stream(labels.device)), "vsa_cluster_order")
    return perm, off


def vsa_gather_rows(src, perm, inverse: bool = False, out=None):
    torch = _torch()
    _expect(src, "src", ndim=4)
    B, H, N, D = src.shape
    _expect(perm, "perm", (B, H, N), torch.int32)
    if out is None:
        out = torch.empty_like(src)
    _expect(out, "out", src.shape, src.dtype)
    _on_device(src, perm=perm, out=out)
    _check(lib().vsa_gather_rows(_ptr(src), _ptr(out), B, H, N, D, _dtype_code(src), _ptr(perm), int(bool(inverse)),
                                 _stream(src.device)), "vsa_gather_rows")
    return out


def vsa_cluster_scores(cq, ck, k_counts, scale=None, out=None):
    torch = _torch()
    _expect(cq, "cq", dtype=torch.float32, ndim=4)
    B, H, Cq, D = cq.shape
    _expect(ck, "ck", dtype=torch.float32, ndim=4)
    Ck = ck.shape[2]
    _expect(ck, "ck", (B, H, Ck, D))
    _expect(k_counts, "k_counts", (B, H, Ck), torch.int32)
    scale = default_scale(D) if scale is None else scale
    if out is None:
        out = torch.empty((B, H, Cq, Ck), dtype=torch.float32, device=cq.device)
    _expect(out, "out", (B, H, Cq, Ck), torch.float32)
    _on_device(cq, ck=ck, k_counts=k_counts, out=out)
    _check(lib().vsa_cluster_scores(_ptr(cq), _ptr(ck), _ptr(k_counts), B, H, Cq, Ck, D, scale, _ptr(out),
                                    _stream(cq.device)), "vsa_cluster_scores")
    return out


def vsa_varlen_attn_workspace_bytes(B, H, N, Cq) -> int:
    return lib().vsa_varlen_attn_workspace_bytes(B, H, N, Cq)


def vsa_varlen_sparse_attn_fwd(q, k, v, q_off, k_off, mask=None, kv_idx=None, kv_cnt=None, scale=None,
                               return_lse=False, out=None, lse=None, workspace=None):
    """Attention over clusters in cluster-major storage (q by query cluster, k / v
    by key cluster; q_off [B, H, Cq + 1], k_off [B, H, Ck + 1])."""
    torch = _torch()
    B, H, N, D = _qkv(q, k, v)
    _expect(q_off, "q_off", dtype=torch.int32, ndim=3)
    _expect(k_off, "k_off", dtype=torch.int32, ndim=3)
    Cq, Ck = q_off.shape[-1] - 1, k_off.shape[-1] - 1
    _expect(q_off, "q_off", (B, H, Cq + 1))
    _expect(k_off, "k_off", (B, H, Ck + 1))
    scale = default_scale(D) if scale is None else scale
    blocks = _blocks_arg(B, H, Cq, Ck, mask, kv_idx, kv_cnt)
    out, lse = _outputs(q, out, lse, return_lse, B, H, N, D)
    ws = vsa_varlen_attn_workspace_bytes(B, H, N, Cq)
    if workspace is None:
        workspace = torch.empty((max(1, ws),), dtype=torch.uint8, device=q.device)
    _expect_workspace(workspace, "workspace", ws)
    _on_device(q, k=k, v=v, q_off=q_off, k_off=k_off, mask=mask, kv_idx=kv_idx, kv_cnt=kv_cnt, out=out, lse=lse,
               workspace=workspace)
    _check(lib().vsa_varlen_sparse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, D,
                                            _dtype_code(q), _ptr(q_off), Cq, _ptr(k_off), Ck, ctypes.byref(blocks),
                                            scale, _ptr(workspace), workspace.numel(), _stream(q.device)),
           "vsa_varlen_sparse_attn_fwd")
    return (out, lse) if return_lse else out


def vsa_fp8_quantize(x, kind: int, out=None, scales=None):
    """e4m3 codes and scales of x [B, H, N, D] (bf16): kind VSA_FP8_ROWS gives
    ([B, H, N, D], [B, H, ceil(N/64)]), VSA_FP8_VT ([B, H, ceil(N/64), D, 64], [B, H, D])."""
    torch = _torch()
    _expect(x, "x", ndim=4)
    B, H, N, D = x.shape
    nt = -(-N // 64)
    if kind not in (VSA_FP8_ROWS, VSA_FP8_VT):
        raise ValueError(f"unknown fp8 layout {kind}")
    shape = (B, H, N, D) if kind == VSA_FP8_ROWS else (B, H, nt, D, 64)
    sshape = (B, H, nt) if kind == VSA_FP8_ROWS else (B, H, D)
    if out is None:
        out = torch.empty(shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(sshape, dtype=torch.float32, device=x.device)
    _expect(out, "out", shape, torch.uint8)
    _expect(scales, "scales", sshape, torch.float32)
    _on_device(x, out=out, scales=scales)
    _check(lib().vsa_fp8_quantize(_ptr(x), B, H, N, D, _dtype_code(x), kind, _ptr(out), _ptr(scales),
                                  _stream(x.device)), "vsa_fp8_quantize")
    return out, scales


def vsa_block_sparse_attn_fwd_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, bs: int, mask=None, kv_idx=None,
                                  kv_cnt=None, blk_len=None, scale=None, return_lse=False, out=None, lse=None):
    torch = _torch()
    _expect(q8, "q8", dtype=torch.uint8, ndim=4)
    B, H, N, D = q8.shape
    nt = -(-N // 64)
    _expect(k8, "k8", q8.shape, torch.uint8)
    _expect(vt8, "vt8", (B, H, nt, D, 64), torch.uint8)
    _expect(q_scale, "q_scale", (B, H, nt), torch.float32)
    _expect(k_scale, "k_scale", (B, H, nt), torch.float32)
    _expect(v_scale, "v_scale", (B, H, D), torch.float32)
    nb = _nb(N, bs)
    scale = default_scale(D) if scale is None else scale
    blocks = _blocks_arg(B, H, nb, nb, mask, kv_idx, kv_cnt)
    if blk_len is not None:
        _expect(blk_len, "blk_len", (nb,), torch.int32)
    out, lse = _outputs(q8, out, lse, return_lse, B, H, N, D, dtype=torch.bfloat16)
    _on_device(q8, k8=k8, vt8=vt8, q_scale=q_scale, k_scale=k_scale, v_scale=v_scale, mask=mask, kv_idx=kv_idx,
               kv_cnt=kv_cnt, blk_len=blk_len, out=out, lse=lse)
    _check(lib().vsa_block_sparse_attn_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(vt8), _ptr(q_scale), _ptr(k_scale),
                                               _ptr(v_scale), _ptr(out), _ptr(lse), B, H, N, D, bs, _ptr(blk_len),
                                               ctypes.byref(blocks), scale, _stream(q8.device)),
           "vsa_block_sparse_attn_fwd_fp8")
    return (out, lse) if return_lse else out


def vsa_check_block_list_host(kv_idx: np.ndarray, kv_cnt: np.ndarray, nkb: int) -> None:
    idx = np.ascontiguousarray(kv_idx, np.int32)
    cnt = np.ascontiguousarray(kv_cnt, np.int32)
    max_kv = idx.shape[-1]
    rows = cnt.size
    if idx.size != rows * max_kv:
        raise ValueError("kv_idx and kv_cnt shapes disagree")
    _check(lib().vsa_check_block_list_host(idx.ctypes.data, cnt.ctypes.data, rows, nkb, max_kv),
           "vsa_check_block_list_host")
