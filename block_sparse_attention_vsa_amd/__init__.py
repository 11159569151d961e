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
LIB_PATH = os.path.join(HERE, "libvsa.so")

VSA_OK, VSA_ERR_INVALID, VSA_ERR_UNSUPPORTED, VSA_ERR_LAUNCH, VSA_ERR_WORKSPACE = range(5)
VSA_BF16, VSA_F32 = 0, 1
VSA_PERM_FRAME_MAJOR, VSA_PERM_CUBE4 = 0, 1
VSA_PATTERN_SPATIAL, VSA_PATTERN_TEMPORAL = 0, 1
VSA_FP8_ROWS, VSA_FP8_VT = 0, 1


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
    "vsa_block_scores": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, _F, _P, _P, _P, _P]),
    "vsa_select_topk": (_I, [_P, _I, _I, _I, _I, _P, _I, _F, _P, _P, _P]),
    "vsa_profile_workspace_bytes": (_SZ, [_I, _I, vsa_grid, _I, _I, _I]),
    "vsa_profile_heads": (_I, [_P, _P, _P, _I, _I, vsa_grid, _I, _I, _I, _P, _I, _P, _P, _I, _F,
                               _P, _P, _P, _SZ, _P]),
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


def _need(t, name, dtype=None, ndim=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")


def _grid(grid) -> vsa_grid:
    T, Hh, W = (int(x) for x in grid)
    return vsa_grid(T, Hh, W)


def default_scale(D: int) -> float:
    return 1.0 / math.sqrt(D)


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
    N = int(np.prod(grid))
    nb = -(-N // bs)
    if out is None:
        out = torch.empty((nb, nb), dtype=torch.uint8, device=device)
    _need(out, "out", torch.uint8)
    _check(lib().vsa_pattern_mask(_grid(grid), bs, pattern, w, _ptr(out), _stream(out.device)), "vsa_pattern_mask")
    return out


def vsa_cube_block_len(grid, device="cuda", out=None):
    torch = _torch()
    nc, _ = vsa_cube_dims(grid)
    if out is None:
        out = torch.empty((nc,), dtype=torch.int32, device=device)
    _need(out, "out", torch.int32)
    _check(lib().vsa_cube_block_len(_grid(grid), _ptr(out), _stream(out.device)), "vsa_cube_block_len")
    return out


def vsa_permute(src, grid, kind: int, inverse: bool = False, head_sel=None, out=None):
    torch = _torch()
    _need(src, "src", ndim=4)
    B, H, _, D = src.shape
    N = int(np.prod(grid))
    if kind == VSA_PERM_CUBE4 and not inverse:
        rows = vsa_cube_dims(grid)[1]
    else:
        rows = N
    if out is None:
        out = torch.empty((B, H, rows, D), dtype=src.dtype, device=src.device)
    _need(out, "out", src.dtype)
    hs = None
    if head_sel is not None:
        hs_arr = (ctypes.c_uint8 * H)(*[1 if x else 0 for x in head_sel])
        hs = ctypes.cast(hs_arr, ctypes.c_void_p)
    _check(lib().vsa_permute(_ptr(src), _ptr(out), B, H, _grid(grid), D, _dtype_code(src), kind, int(bool(inverse)),
                             hs, _stream(src.device)), "vsa_permute")
    return out


def vsa_block_scores(q, k, bs: int, blk_len=None, scale=None, out=None):
    torch = _torch()
    _need(q, "q", ndim=4)
    _need(k, "k", q.dtype, 4)
    B, H, N, D = q.shape
    nb = -(-N // bs)
    scale = default_scale(D) if scale is None else scale
    if out is None:
        out = (torch.empty((B, H, nb, nb), dtype=torch.float32, device=q.device),
               torch.empty((B, H, nb, D), dtype=torch.float32, device=q.device),
               torch.empty((B, H, nb, D), dtype=torch.float32, device=q.device))
    s, qp, kp = out
    if blk_len is not None:
        _need(blk_len, "blk_len", torch.int32)
    _check(lib().vsa_block_scores(_ptr(q), _ptr(k), B, H, N, D, _dtype_code(q), bs, _ptr(blk_len), scale, _ptr(s),
                                  _ptr(qp), _ptr(kp), _stream(q.device)), "vsa_block_scores")
    return s, qp, kp


def vsa_select_topk(scores, k_max: int, top_p: float = 1.0, forced=None, out=None):
    torch = _torch()
    _need(scores, "scores", torch.float32, 4)
    B, H, nqb, nkb = scores.shape
    if forced is not None:
        _need(forced, "forced", torch.uint8)
    if out is None:
        out = (torch.empty((B, H, nqb, k_max), dtype=torch.int32, device=scores.device),
               torch.empty((B, H, nqb), dtype=torch.int32, device=scores.device))
    idx, cnt = out
    _check(lib().vsa_select_topk(_ptr(scores), B, H, nqb, nkb, _ptr(forced), k_max, top_p, _ptr(idx), _ptr(cnt),
                                 _stream(scores.device)), "vsa_select_topk")
    return idx, cnt


def vsa_profile_workspace_bytes(B, H, grid, D, R, P) -> int:
    return lib().vsa_profile_workspace_bytes(B, H, _grid(grid), D, R, P)


def vsa_profile_heads(q, k, v, grid, bs: int, rows, cand_masks, cand_layout, scale=None, workspace=None, out=None):
    torch = _torch()
    _need(q, "q", ndim=4)
    _need(k, "k", q.dtype, 4)
    _need(v, "v", q.dtype, 4)
    _need(rows, "rows", torch.int32, 1)
    _need(cand_masks, "cand_masks", torch.uint8, 3)
    B, H, N, D = q.shape
    P = cand_masks.shape[0]
    R = rows.shape[0]
    scale = default_scale(D) if scale is None else scale
    ws = vsa_profile_workspace_bytes(B, H, grid, D, R, P)
    if workspace is None:
        workspace = torch.empty((max(ws, 1),), dtype=torch.uint8, device=q.device)
    if out is None:
        out = (torch.empty((B, H, P), dtype=torch.float32, device=q.device),
               torch.empty((B, H), dtype=torch.int32, device=q.device))
    err, choice = out
    lay = (ctypes.c_int32 * P)(*[int(x) for x in cand_layout])
    _check(lib().vsa_profile_heads(_ptr(q), _ptr(k), _ptr(v), B, H, _grid(grid), D, _dtype_code(q), bs, _ptr(rows), R,
                                   _ptr(cand_masks), ctypes.cast(lay, ctypes.c_void_p), P, scale, _ptr(err),
                                   _ptr(choice), _ptr(workspace), workspace.numel(), _stream(q.device)),
           "vsa_profile_heads")
    return err, choice


def vsa_mask_to_list(mask, max_kv=None, head_mask_idx=None, B=None, H=None, out=None):
    """mask [B,H,nqb,nkb]; or mask [P,nqb,nkb] with head_mask_idx (length H) and B given."""
    torch = _torch()
    _need(mask, "mask", torch.uint8)
    if head_mask_idx is None:
        B, H, nqb, nkb = mask.shape
        P = 0
        sel = None
    else:
        P, nqb, nkb = mask.shape
        H = len(head_mask_idx)
        B = 1 if B is None else B
        arr = (ctypes.c_int32 * H)(*[int(x) for x in head_mask_idx])
        sel = ctypes.cast(arr, ctypes.c_void_p)
    max_kv = nkb if max_kv is None else max_kv
    if out is None:
        out = (torch.empty((B, H, nqb, max_kv), dtype=torch.int32, device=mask.device),
               torch.empty((B, H, nqb), dtype=torch.int32, device=mask.device))
    idx, cnt = out
    _check(lib().vsa_mask_to_list(_ptr(mask), B, H, nqb, nkb, sel, P, max_kv, _ptr(idx), _ptr(cnt),
                                  _stream(mask.device)), "vsa_mask_to_list")
    return idx, cnt


def vsa_attn_workspace_bytes(B, H, N, bs, max_kv) -> int:
    return lib().vsa_attn_workspace_bytes(B, H, N, bs, max_kv)


def vsa_block_sparse_attn_fwd(q, k, v, bs: int, mask=None, kv_idx=None, kv_cnt=None, blk_len=None, scale=None,
                              return_lse=False, out=None, lse=None, workspace=None):
    torch = _torch()
    _need(q, "q", ndim=4)
    _need(k, "k", q.dtype, 4)
    _need(v, "v", q.dtype, 4)
    B, H, N, D = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    scale = default_scale(D) if scale is None else scale
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    blocks = vsa_blocks()
    if mask is not None:
        _need(mask, "mask", torch.uint8)
        blocks.mask = mask.data_ptr()
    if kv_idx is not None:
        _need(kv_idx, "kv_idx", torch.int32, 4)
        _need(kv_cnt, "kv_cnt", torch.int32, 3)
        blocks.kv_idx = kv_idx.data_ptr()
        blocks.kv_cnt = kv_cnt.data_ptr()
        blocks.max_kv = kv_idx.shape[-1]
    if blk_len is not None:
        _need(blk_len, "blk_len", torch.int32, 1)
    max_kv = blocks.max_kv if kv_idx is not None else -(-N // bs)
    ws = vsa_attn_workspace_bytes(B, H, N, bs, max_kv)
    if ws and workspace is None:
        workspace = torch.empty((ws,), dtype=torch.uint8, device=q.device)
    _check(lib().vsa_block_sparse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, D,
                                           _dtype_code(q), bs, _ptr(blk_len), ctypes.byref(blocks), scale,
                                           _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                           _stream(q.device)), "vsa_block_sparse_attn_fwd")
    return (out, lse) if return_lse else out


def _blocks_arg(q, bs, mask, kv_idx, kv_cnt):
    torch = _torch()
    blocks = vsa_blocks()
    if mask is not None:
        _need(mask, "mask", torch.uint8)
        blocks.mask = mask.data_ptr()
    if kv_idx is not None:
        _need(kv_idx, "kv_idx", torch.int32, 4)
        _need(kv_cnt, "kv_cnt", torch.int32, 3)
        blocks.kv_idx = kv_idx.data_ptr()
        blocks.kv_cnt = kv_cnt.data_ptr()
        blocks.max_kv = kv_idx.shape[-1]
    return blocks


def vsa_block_sparse_attn_fwd_permuted(q, k, v, grid, bs: int, head_fm=None, mask=None, kv_idx=None, kv_cnt=None,
                                       blk_len=None, scale=None, return_lse=False, out=None, lse=None):
    """Attention with the frame-major permutation of the heads in `head_fm`
    (host sequence of H flags) folded into the kernel's loads and stores; q, k,
    v and the result are in natural order."""
    torch = _torch()
    _need(q, "q", ndim=4)
    _need(k, "k", q.dtype, 4)
    _need(v, "v", q.dtype, 4)
    B, H, N, D = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    if N != int(np.prod(grid)):
        raise ValueError("N must equal T*Hh*W")
    scale = default_scale(D) if scale is None else scale
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    blocks = _blocks_arg(q, bs, mask, kv_idx, kv_cnt)
    if blk_len is not None:
        _need(blk_len, "blk_len", torch.int32, 1)
    hf = None
    if head_fm is not None:
        if len(head_fm) != H:
            raise ValueError("head_fm needs one flag per head")
        hf_arr = (ctypes.c_uint8 * H)(*[1 if x else 0 for x in head_fm])
        hf = ctypes.cast(hf_arr, ctypes.c_void_p)
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
    _need(q, "q", ndim=4)
    _need(k, "k", q.dtype, 4)
    _need(v, "v", q.dtype, 4)
    B, H, N, D = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    if N != int(np.prod(grid)):
        raise ValueError("N must equal T*Hh*W")
    _need(cand_masks, "cand_masks", torch.uint8, 3)
    _need(choice, "choice", torch.int32)
    if choice.numel() != B * H:
        raise ValueError("choice needs B*H entries")
    P = cand_masks.shape[0]
    if len(cand_layout) != P:
        raise ValueError("cand_layout needs one entry per candidate")
    lay = (ctypes.c_int32 * P)(*[int(x) for x in cand_layout])
    scale = default_scale(D) if scale is None else scale
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if blk_len is not None:
        _need(blk_len, "blk_len", torch.int32, 1)
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
    _need(q, "q", ndim=4)
    for t, name in ((k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _need(t, name, q.dtype, 4)
        if t.shape != q.shape:
            raise ValueError(f"{name} must have the shape of q")
    B, H, N, D = q.shape
    _need(lse, "lse", torch.float32, 3)
    if tuple(lse.shape) != (B, H, N):
        raise ValueError("lse must be [B, H, N]")
    if blk_len is not None:
        _need(blk_len, "blk_len", torch.int32, 1)
    scale = default_scale(D) if scale is None else scale
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _need(t, name, q.dtype, 4)
    blocks = _blocks_arg(q, bs, mask, kv_idx, kv_cnt)
    ws = vsa_attn_bwd_workspace_bytes(B, H, N, bs, kv_idx is not None)
    if workspace is None and ws:
        workspace = torch.empty((ws,), dtype=torch.uint8, device=q.device)
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
    _need(x, "x", ndim=4)
    B, H, N, D = x.shape
    if out is None:
        out = (torch.empty((B, H, C, D), dtype=torch.float32, device=x.device),
               torch.empty((B, H, N), dtype=torch.int32, device=x.device),
               torch.empty((B, H, C), dtype=torch.int32, device=x.device))
    cent, lab, cnt = out
    if workspace is None:
        workspace = torch.empty((max(1, vsa_kmeans_workspace_bytes(B, H, N, C, D)),), dtype=torch.uint8,
                                device=x.device)
    _check(lib().vsa_kmeans(_ptr(x), B, H, N, D, _dtype_code(x), C, iters, _ptr(cent), _ptr(lab), _ptr(cnt),
                            _ptr(workspace), workspace.numel(), _stream(x.device)), "vsa_kmeans")
    return cent, lab, cnt


def vsa_cluster_order_workspace_bytes(B, H, N, C) -> int:
    return lib().vsa_cluster_order_workspace_bytes(B, H, N, C)


def vsa_cluster_order(labels, C: int, out=None, workspace=None):
    """Stable cluster-major order: (perm int32 [B, H, N], offsets int32 [B, H, C + 1])."""
    torch = _torch()
    _need(labels, "labels", torch.int32, 3)
    B, H, N = labels.shape
    if out is None:
        out = (torch.empty((B, H, N), dtype=torch.int32, device=labels.device),
               torch.empty((B, H, C + 1), dtype=torch.int32, device=labels.device))
    perm, off = out
    if workspace is None:
        workspace = torch.empty((max(1, vsa_cluster_order_workspace_bytes(B, H, N, C)),), dtype=torch.uint8,
                                device=labels.device)
    _check(lib().vsa_cluster_order(_ptr(labels), B, H, N, C, _ptr(perm), _ptr(off), _ptr(workspace),
                                   workspace.numel(), _stream(labels.device)), "vsa_cluster_order")
    return perm, off


def vsa_gather_rows(src, perm, inverse: bool = False, out=None):
    torch = _torch()
    _need(src, "src", ndim=4)
    _need(perm, "perm", torch.int32, 3)
    B, H, N, D = src.shape
    if out is None:
        out = torch.empty_like(src)
    _check(lib().vsa_gather_rows(_ptr(src), _ptr(out), B, H, N, D, _dtype_code(src), _ptr(perm), int(bool(inverse)),
                                 _stream(src.device)), "vsa_gather_rows")
    return out


def vsa_cluster_scores(cq, ck, k_counts, scale=None, out=None):
    torch = _torch()
    _need(cq, "cq", torch.float32, 4)
    _need(ck, "ck", torch.float32, 4)
    _need(k_counts, "k_counts", torch.int32, 3)
    B, H, Cq, D = cq.shape
    Ck = ck.shape[2]
    scale = default_scale(D) if scale is None else scale
    if out is None:
        out = torch.empty((B, H, Cq, Ck), dtype=torch.float32, device=cq.device)
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
    _need(q, "q", ndim=4)
    _need(k, "k", q.dtype, 4)
    _need(v, "v", q.dtype, 4)
    _need(q_off, "q_off", torch.int32, 3)
    _need(k_off, "k_off", torch.int32, 3)
    B, H, N, D = q.shape
    Cq, Ck = q_off.shape[-1] - 1, k_off.shape[-1] - 1
    scale = default_scale(D) if scale is None else scale
    if out is None:
        out = torch.empty_like(q)
    if return_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    blocks = _blocks_arg(q, 0, mask, kv_idx, kv_cnt)
    if workspace is None:
        workspace = torch.empty((vsa_varlen_attn_workspace_bytes(B, H, N, Cq),), dtype=torch.uint8, device=q.device)
    _check(lib().vsa_varlen_sparse_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, D,
                                            _dtype_code(q), _ptr(q_off), Cq, _ptr(k_off), Ck, ctypes.byref(blocks),
                                            scale, _ptr(workspace), workspace.numel(), _stream(q.device)),
           "vsa_varlen_sparse_attn_fwd")
    return (out, lse) if return_lse else out


def vsa_fp8_quantize(x, kind: int, out=None, scales=None):
    """e4m3 codes and scales of x [B, H, N, D] (bf16): kind VSA_FP8_ROWS gives
    ([B, H, N, D], [B, H, ceil(N/64)]), VSA_FP8_VT ([B, H, ceil(N/64), D, 64], [B, H, D])."""
    torch = _torch()
    _need(x, "x", ndim=4)
    B, H, N, D = x.shape
    nt = -(-N // 64)
    if out is None:
        shape = (B, H, N, D) if kind == VSA_FP8_ROWS else (B, H, nt, D, 64)
        out = torch.empty(shape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((B, H, nt) if kind == VSA_FP8_ROWS else (B, H, D), dtype=torch.float32, device=x.device)
    _check(lib().vsa_fp8_quantize(_ptr(x), B, H, N, D, _dtype_code(x), kind, _ptr(out), _ptr(scales),
                                  _stream(x.device)), "vsa_fp8_quantize")
    return out, scales


def vsa_block_sparse_attn_fwd_fp8(q8, k8, vt8, q_scale, k_scale, v_scale, bs: int, mask=None, kv_idx=None,
                                  kv_cnt=None, blk_len=None, scale=None, return_lse=False, out=None, lse=None):
    torch = _torch()
    _need(q8, "q8", torch.uint8, 4)
    _need(k8, "k8", torch.uint8, 4)
    _need(vt8, "vt8", torch.uint8, 5)
    B, H, N, D = q8.shape
    scale = default_scale(D) if scale is None else scale
    if out is None:
        out = torch.empty((B, H, N, D), dtype=torch.bfloat16, device=q8.device)
    if return_lse and lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    if blk_len is not None:
        _need(blk_len, "blk_len", torch.int32, 1)
    blocks = _blocks_arg(q8, bs, mask, kv_idx, kv_cnt)
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
