"""Python binding of libbsa: block-sparse attention with NABLA / sliding-tile masks on MI355X.

Argument marshalling only. Every step runs in the HIP kernels of libbsa.so; torch is
used for device memory (outputs, workspaces) and for the current HIP stream. If the
library is not built, every call raises.

    mask = nabla_build_mask(q, k, thr=0.2)                   # [B,H,nb,nb] uint8
    sta  = sta_build_mask(S, S_valid, grid, tile, window)    # [nb,nb] uint8
    out  = block_sparse_attn_fwd(q, k, v, mask)              # [B,H,S,D]
"""
import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbsa.so")
# the checked build (-DBSA_CHECKED): same entry points, list indices tested in the kernels
CHECKED_LIB_PATH = os.path.join(_PKG, "libbsa_checked.so")

BSA_F32, BSA_BF16, BSA_FP8_E4M3FN = 0, 1, 2
_STATUS = {0: "BSA_OK", 1: "BSA_EINVAL", 2: "BSA_EUNSUPPORTED", 3: "BSA_EWORKSPACE", 4: "BSA_EHIP"}

# every function the C header declares, in declaration order
EXPORTS = ["nabla_workspace_size", "nabla_build_mask", "nabla_build_mask_noalloc", "nabla_build_mask_topk",
           "quantize_fp8_blocks",
           "nabla_build_mask_fp8", "quantize_fp8_blocks_rotated", "nabla_build_mask_fp8_rotated",
           "sta_workspace_size", "sta_build_mask", "nabla_sta_workspace_size", "nabla_build_mask_sta",
           "nabla_lists_workspace_size", "nabla_build_mask_lists", "mask_or",
           "csr_workspace_size", "bsa_mask_to_csr", "bsa_mask_to_csr_ordered", "attn_workspace_size",
           "block_sparse_attn_fwd", "bsa_set_attn_kv_chunk", "attn_pair_workspace_size", "attn_pair_offsets",
           "attn_csr_workspace_size", "block_sparse_attn_fwd_csr", "block_sparse_attn_fwd_lists",
           "attn_work_order_slots", "attn_work_order",
           "attn_bwd_workspace_size", "block_sparse_attn_bwd", "token_reorder", "bsa_last_error",
           "bsa_abi_version", "bsa_checked_build", "bsa_check_flags"]


class BsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class Tensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("dtype", ctypes.c_int), ("sb", ctypes.c_int64),
                ("sh", ctypes.c_int64), ("ss", ctypes.c_int64)]


class Shape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int), ("H", ctypes.c_int), ("S", ctypes.c_int), ("S_valid", ctypes.c_int),
                ("D", ctypes.c_int), ("N", ctypes.c_int)]


_lib = None
_lib_path = None


def load(path: Optional[str] = None):
    """Load libbsa.so (or the library at `path`, e.g. CHECKED_LIB_PATH, which then serves
    every call of this module) and declare its signatures; raises if it is not built."""
    global _lib, _lib_path
    p = path or _lib_path or LIB_PATH
    if _lib is not None and p == _lib_path:
        return _lib
    if not os.path.exists(p):
        raise RuntimeError(f"libbsa.so not found at {p}; build it with "
                           "`python -m block_sparse_attention_mask_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i64, i32, dbl, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double, ctypes.c_size_t
    PT, PS = ctypes.POINTER(Tensor), ctypes.POINTER(Shape)
    i3 = ctypes.POINTER(ctypes.c_int)
    sig = {
        "nabla_workspace_size": (sz, [PS]),
        "nabla_build_mask": (i32, [PT, PT, PS, dbl, dbl, vp, i64, i64, vp, vp, vp, sz, vp]),
        "nabla_build_mask_noalloc": (i32, [PT, PT, PS, dbl, dbl, vp, i64, i64, vp, vp, vp]),
        "nabla_build_mask_topk": (i32, [PT, PT, PS, i32, dbl, vp, i64, i64, vp, vp, sz, vp]),
        "quantize_fp8_blocks": (i32, [PT, PS, PT, vp, vp]),
        "nabla_build_mask_fp8": (i32, [PT, PT, PS, dbl, dbl, vp, i64, i64, vp, vp, PT, vp, PT, vp, vp, sz, vp]),
        "quantize_fp8_blocks_rotated": (i32, [PT, PS, vp, i32, PT, vp, vp]),
        "nabla_build_mask_fp8_rotated": (i32, [PT, PT, PS, dbl, dbl, vp, i64, i64, vp, vp, vp, PT, vp, PT, vp, vp,
                                               sz, vp]),
        "sta_workspace_size": (sz, [PS]),
        "sta_build_mask": (i32, [PS, i3, i3, i3, i32, i3, vp, vp, sz, vp]),
        "nabla_sta_workspace_size": (sz, [PS]),
        "nabla_build_mask_sta": (i32, [PT, PT, PS, dbl, dbl, i3, i3, i3, i32, i3, vp, vp, vp, sz, vp]),
        "nabla_lists_workspace_size": (sz, [PS]),
        "nabla_build_mask_lists": (i32, [PT, PT, PS, dbl, dbl, i3, i3, i3, i32, i3, vp, vp, vp, vp, vp, vp, sz,
                                         vp]),
        "mask_or": (i32, [vp, vp, i64, vp, i64, vp]),
        "csr_workspace_size": (sz, [i32, i32, i32]),
        "bsa_mask_to_csr": (i32, [vp, i64, i64, i32, i32, i32, vp, vp, vp, vp, sz, vp]),
        "bsa_mask_to_csr_ordered": (i32, [vp, i64, i64, i32, i32, i32, vp, vp, vp, vp, sz, vp]),
        "attn_workspace_size": (sz, [PS, i32]),
        "block_sparse_attn_fwd": (i32, [PT, PT, PT, PS, vp, i64, i64, vp, vp, dbl, PT, vp, vp, sz, vp]),
        "attn_csr_workspace_size": (sz, [PS, i32]),
        "block_sparse_attn_fwd_csr": (i32, [PT, PT, PT, PS, vp, vp, vp, vp, vp, dbl, PT, vp, vp, sz, vp]),
        "block_sparse_attn_fwd_lists": (i32, [PT, PT, PT, PS, vp, vp, vp, vp, vp, dbl, PT, vp, vp, sz, vp]),
        "bsa_set_attn_kv_chunk": (i32, [i32]),
        "attn_pair_workspace_size": (sz, [PS]),
        "attn_pair_offsets": (i32, [PS, vp, vp, vp, vp, vp, sz, vp]),
        "attn_work_order_slots": (i32, [PS]),
        "attn_work_order": (i32, [PS, vp, vp, vp]),
        "attn_bwd_workspace_size": (sz, [PS]),
        "token_reorder": (i32, [PT, PS, i3, i32, i3, i32, PT, vp]),
        "block_sparse_attn_bwd": (i32, [PT, PT, PT, PT, PT, vp, PS, vp, i64, i64, dbl, PT, PT, PT, vp, sz, vp]),
        "bsa_last_error": (ctypes.c_char_p, []),
        "bsa_abi_version": (i32, []),
        "bsa_checked_build": (i32, []),
        "bsa_check_flags": (ctypes.c_uint, [i32]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    _lib, _lib_path = lib, p
    return lib


def _check(status: int):
    if status != 0:
        raise BsaError(status, _lib.bsa_last_error().decode())


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return BSA_F32
    if t.dtype == torch.bfloat16:
        return BSA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return BSA_FP8_E4M3FN
    raise TypeError(f"unsupported dtype {t.dtype}")


def _tensor(t: torch.Tensor) -> Tensor:
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B, H, S, D] tensor with contiguous D")
    return Tensor(t.data_ptr(), _dtype_code(t), t.stride(0), t.stride(1), t.stride(2))


def _shape(t: torch.Tensor, s_valid: Optional[int]) -> Shape:
    B, H, S, D = t.shape
    return Shape(B, H, S, S if s_valid is None else int(s_valid), D, 64)


def _ws(nbytes: int, dev) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=dev)


def _mask_strides(mask: torch.Tensor):
    """(ptr, sb, sh) of a [B,H,nb,nb] or [nb,nb] uint8 mask (bytes; 0 = broadcast)."""
    if mask.dtype not in (torch.uint8, torch.bool):
        raise TypeError("mask must be uint8 or bool")
    if mask.dim() == 2:
        mask = mask[None, None]
    if mask.stride(3) != 1 or mask.stride(2) != mask.shape[3]:
        raise ValueError("mask rows must be contiguous")
    sb = mask.stride(0) if mask.shape[0] > 1 else 0
    sh = mask.stride(1) if mask.shape[1] > 1 else 0
    return mask.data_ptr(), sb, sh, mask


def _near_buffer(q, near):
    """near: False (no flags), True (a new [B,H,nb,nb] uint8 buffer) or a tensor to fill."""
    if near is None or near is False:
        return None
    if near is True:
        B, H, S, _ = q.shape
        return torch.empty(B, H, S // 64, S // 64, dtype=torch.uint8, device=q.device)
    if near.dtype != torch.uint8 or not near.is_contiguous():
        raise ValueError("near-threshold flags must be a contiguous uint8 [B, H, nb, nb] tensor")
    return near


def nabla_build_mask(q: torch.Tensor, k: torch.Tensor, thr: float, scale: Optional[float] = None,
                     or_mask: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                     near=False):
    """NABLA adaptive block mask of q, k [B,H,S,D] (bf16 or f32) -> uint8 [B,H,S/64,S/64].

    near=True (or a uint8 [B,H,nb,nb] tensor): also the near-threshold flags (1 where the
    block's exclusive cumulative mass lies within 1e-6 of 1 - thr); returns (mask, flags)."""
    lib = load()
    B, H, S, D = q.shape
    nb = S // 64
    shp = _shape(q, None)
    if out is None:
        out = torch.empty(B, H, nb, nb, dtype=torch.uint8, device=q.device)
    nf = _near_buffer(q, near)
    ws = _ws(lib.nabla_workspace_size(ctypes.byref(shp)), q.device)
    om, osb, osh = None, 0, 0
    if or_mask is not None:
        om, osb, osh, _keep = _mask_strides(or_mask)
    tq, tk = _tensor(q), _tensor(k)
    _check(lib.nabla_build_mask(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(shp), float(thr),
                                float(scale) if scale else 0.0, om, osb, osh, out.data_ptr(),
                                nf.data_ptr() if nf is not None else None, ws.data_ptr(), ws.numel(),
                                _stream(q.device)))
    return (out, nf) if nf is not None else out


def nabla_build_mask_noalloc(q: torch.Tensor, k: torch.Tensor, thr: float, scale: Optional[float] = None,
                             or_mask: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                             near=False):
    """nabla_build_mask with the library's static scratch as workspace (no device allocation
    inside the call; pass `out` (and a `near` tensor) to allocate nothing here either).
    Calls on one GPU must not overlap in time."""
    lib = load()
    B, H, S, D = q.shape
    nb = S // 64
    shp = _shape(q, None)
    if out is None:
        out = torch.empty(B, H, nb, nb, dtype=torch.uint8, device=q.device)
    nf = _near_buffer(q, near)
    om, osb, osh = None, 0, 0
    if or_mask is not None:
        om, osb, osh, _keep = _mask_strides(or_mask)
    tq, tk = _tensor(q), _tensor(k)
    _check(lib.nabla_build_mask_noalloc(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(shp), float(thr),
                                        float(scale) if scale else 0.0, om, osb, osh, out.data_ptr(),
                                        nf.data_ptr() if nf is not None else None, _stream(q.device)))
    return (out, nf) if nf is not None else out


def nabla_build_mask_topk(q: torch.Tensor, k: torch.Tensor, topk: int, scale: Optional[float] = None,
                          or_mask: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Top-k block mask on NABLA's reduced map: each row keeps its topk most probable blocks."""
    lib = load()
    B, H, S, D = q.shape
    nb = S // 64
    shp = _shape(q, None)
    if out is None:
        out = torch.empty(B, H, nb, nb, dtype=torch.uint8, device=q.device)
    ws = _ws(lib.nabla_workspace_size(ctypes.byref(shp)), q.device)
    om, osb, osh = None, 0, 0
    if or_mask is not None:
        om, osb, osh, _keep = _mask_strides(or_mask)
    tq, tk = _tensor(q), _tensor(k)
    _check(lib.nabla_build_mask_topk(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(shp), int(topk),
                                     float(scale) if scale else 0.0, om, osb, osh, out.data_ptr(), ws.data_ptr(),
                                     ws.numel(), _stream(q.device)))
    return out


def _fp8_buffers(x: torch.Tensor, out=None):
    if out is not None:
        return out
    B, H, S, _ = x.shape
    return (torch.empty(x.shape, dtype=torch.uint8, device=x.device),
            torch.empty(B, H, S // 64, dtype=torch.float32, device=x.device))


def quantize_fp8_blocks(x: torch.Tensor, out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """fp8 e4m3fn codes (uint8 [B,H,S,D]) and per-block scales (float32 [B,H,S/64]) of x."""
    lib = load()
    shp = _shape(x, None)
    codes, scales = _fp8_buffers(x, out)
    if not scales.is_contiguous() or scales.dtype != torch.float32:
        raise ValueError("scales must be contiguous float32 [B, H, S/64]")
    tx, tc = _tensor(x), _tensor(codes)
    _check(lib.quantize_fp8_blocks(ctypes.byref(tx), ctypes.byref(shp), ctypes.byref(tc), scales.data_ptr(),
                                   _stream(x.device)))
    return codes, scales


def nabla_build_mask_fp8(q: torch.Tensor, k: torch.Tensor, thr: float, scale: Optional[float] = None,
                         or_mask: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                         q8_out=None, k8_out=None, near=False):
    """nabla_build_mask plus the fp8 block quantisation of q and k from the same read.

    Returns (mask, (q codes, q scales), (k codes, k scales)), with near also the flags
    (mask, flags, (q codes, q scales), (k codes, k scales))."""
    lib = load()
    B, H, S, D = q.shape
    nb = S // 64
    shp = _shape(q, None)
    if out is None:
        out = torch.empty(B, H, nb, nb, dtype=torch.uint8, device=q.device)
    q8, qs = _fp8_buffers(q, q8_out)
    k8, ks = _fp8_buffers(k, k8_out)
    ws = _ws(lib.nabla_workspace_size(ctypes.byref(shp)), q.device)
    om, osb, osh = None, 0, 0
    if or_mask is not None:
        om, osb, osh, _keep = _mask_strides(or_mask)
    nf = _near_buffer(q, near)
    tq, tk, tq8, tk8 = _tensor(q), _tensor(k), _tensor(q8), _tensor(k8)
    _check(lib.nabla_build_mask_fp8(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(shp), float(thr),
                                    float(scale) if scale else 0.0, om, osb, osh, out.data_ptr(),
                                    nf.data_ptr() if nf is not None else None,
                                    ctypes.byref(tq8), qs.data_ptr(), ctypes.byref(tk8), ks.data_ptr(),
                                    ws.data_ptr(), ws.numel(), _stream(q.device)))
    if nf is not None:
        return out, nf, (q8, qs), (k8, ks)
    return out, (q8, qs), (k8, ks)


def _sign_words(signs, D: int):
    """Random signs s (+1 / -1, length D) -> the header's host bit words (bit set where s = -1)."""
    s = [float(x) for x in (signs.tolist() if hasattr(signs, "tolist") else signs)]
    if len(s) != D or any(x not in (1.0, -1.0) for x in s):
        raise ValueError(f"signs must be {D} values of +1 or -1")
    words = (ctypes.c_uint64 * max(1, D // 64))()
    for d, x in enumerate(s):
        if x < 0:
            words[d // 64] |= 1 << (d % 64)
    return words


def quantize_fp8_blocks_rotated(x: torch.Tensor, signs, key_side: bool,
                                out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None):
    """Incoherent processing, then fp8 block quantisation: codes and scales of the rows
    H (s . x); with key_side the scales also carry 1/D."""
    lib = load()
    shp = _shape(x, None)
    codes, scales = _fp8_buffers(x, out)
    if not scales.is_contiguous() or scales.dtype != torch.float32:
        raise ValueError("scales must be contiguous float32 [B, H, S/64]")
    words = _sign_words(signs, x.shape[3])
    tx, tc = _tensor(x), _tensor(codes)
    _check(lib.quantize_fp8_blocks_rotated(ctypes.byref(tx), ctypes.byref(shp), words, 1 if key_side else 0,
                                           ctypes.byref(tc), scales.data_ptr(), _stream(x.device)))
    return codes, scales


def nabla_build_mask_fp8_rotated(q: torch.Tensor, k: torch.Tensor, thr: float, signs,
                                 scale: Optional[float] = None, or_mask: Optional[torch.Tensor] = None,
                                 out: Optional[torch.Tensor] = None, q8_out=None, k8_out=None):
    """nabla_build_mask plus the rotated fp8 quantisation of q (query side) and k (key side)
    from the same read. Returns (mask, (q codes, q scales), (k codes, k scales))."""
    lib = load()
    B, H, S, D = q.shape
    nb = S // 64
    shp = _shape(q, None)
    if out is None:
        out = torch.empty(B, H, nb, nb, dtype=torch.uint8, device=q.device)
    q8, qs = _fp8_buffers(q, q8_out)
    k8, ks = _fp8_buffers(k, k8_out)
    ws = _ws(lib.nabla_workspace_size(ctypes.byref(shp)), q.device)
    om, osb, osh = None, 0, 0
    if or_mask is not None:
        om, osb, osh, _keep = _mask_strides(or_mask)
    words = _sign_words(signs, D)
    tq, tk, tq8, tk8 = _tensor(q), _tensor(k), _tensor(q8), _tensor(k8)
    _check(lib.nabla_build_mask_fp8_rotated(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(shp), float(thr),
                                            float(scale) if scale else 0.0, om, osb, osh, out.data_ptr(), None,
                                            words, ctypes.byref(tq8), qs.data_ptr(), ctypes.byref(tk8),
                                            ks.data_ptr(), ws.data_ptr(), ws.numel(), _stream(q.device)))
    return out, (q8, qs), (k8, ks)


def sta_build_mask(S: int, S_valid: int, grid: Sequence[int], tile: Sequence[int], window: Sequence[int],
                   order: str = "row", order_tile: Optional[Sequence[int]] = None, device="cuda",
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Sliding-tile block mask -> uint8 [S/64, S/64] (shared by all heads)."""
    lib = load()
    nb = S // 64
    shp = Shape(1, 1, S, S_valid, 64, 64)
    dev = torch.device(device)
    if out is None:
        out = torch.empty(nb, nb, dtype=torch.uint8, device=dev)
    ws = _ws(lib.sta_workspace_size(ctypes.byref(shp)), dev)
    arr = ctypes.c_int * 3
    ot = arr(*order_tile) if order_tile is not None else None
    _check(lib.sta_build_mask(ctypes.byref(shp), arr(*grid), arr(*tile), arr(*window),
                              0 if order == "row" else 1, ot, out.data_ptr(), ws.data_ptr(), ws.numel(),
                              _stream(dev)))
    return out


def nabla_build_mask_sta(q: torch.Tensor, k: torch.Tensor, thr: float, grid: Sequence[int], tile: Sequence[int],
                         window: Sequence[int], order: str = "row", order_tile: Optional[Sequence[int]] = None,
                         s_valid: Optional[int] = None, scale: Optional[float] = None,
                         out: Optional[torch.Tensor] = None, near=False):
    """NABLA mask of q, k OR'd with the sliding-tile mask of the grid in one call
    -> uint8 [B,H,S/64,S/64] (equal to nabla_build_mask(..., or_mask=sta_build_mask(...)));
    with near, (mask, near-threshold flags of the adaptive rule)."""
    lib = load()
    B, H, S, D = q.shape
    nb = S // 64
    shp = _shape(q, s_valid)
    if out is None:
        out = torch.empty(B, H, nb, nb, dtype=torch.uint8, device=q.device)
    ws = _ws(lib.nabla_sta_workspace_size(ctypes.byref(shp)), q.device)
    arr = ctypes.c_int * 3
    ot = arr(*order_tile) if order_tile is not None else None
    nf = _near_buffer(q, near)
    tq, tk = _tensor(q), _tensor(k)
    _check(lib.nabla_build_mask_sta(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(shp), float(thr),
                                    float(scale) if scale else 0.0, arr(*grid), arr(*tile), arr(*window),
                                    0 if order == "row" else 1, ot, out.data_ptr(),
                                    nf.data_ptr() if nf is not None else None, ws.data_ptr(), ws.numel(),
                                    _stream(q.device)))
    return (out, nf) if nf is not None else out


def nabla_lists_workspace(q: torch.Tensor, s_valid: Optional[int] = None) -> torch.Tensor:
    """A workspace for nabla_build_mask_lists on tensors shaped like q (reusable by calls
    that do not overlap in time)."""
    lib = load()
    shp = _shape(q, s_valid)
    return _ws(lib.nabla_lists_workspace_size(ctypes.byref(shp)), q.device)


def nabla_build_mask_lists(q: torch.Tensor, k: torch.Tensor, thr: float, grid: Optional[Sequence[int]] = None,
                           tile: Optional[Sequence[int]] = None, window: Optional[Sequence[int]] = None,
                           order: str = "row", order_tile: Optional[Sequence[int]] = None,
                           s_valid: Optional[int] = None, scale: Optional[float] = None, work_order: bool = True,
                           out=None, ws: Optional[torch.Tensor] = None, near=None):
    """The mask of nabla_build_mask_sta (grid None: of nabla_build_mask) with, from the same
    launch, the kv lists -> (mask uint8 [B,H,nb,nb], kv_len int32 [B*H*nb], kv_idx int32
    [B*H*nb, nb] (row r's kept blocks, ascending, in kv_idx[r, :kv_len[r]]), work order
    int32 [slots] or None when the shape runs in the default order). nb <= 256. near: an
    optional uint8 [B,H,nb,nb] tensor filled with the near-threshold flags (not returned)."""
    lib = load()
    B, H, S, D = q.shape
    nb = S // 64
    shp = _shape(q, s_valid)
    if out is None:
        out = (torch.empty(B, H, nb, nb, dtype=torch.uint8, device=q.device),
               torch.empty(B * H * nb, dtype=torch.int32, device=q.device),
               torch.empty(B * H * nb, nb, dtype=torch.int32, device=q.device), None)
        n = lib.attn_work_order_slots(ctypes.byref(shp))
        if work_order and n > 0:
            out = out[:3] + (torch.empty(n, dtype=torch.int32, device=q.device),)
    mask, kv_len, kv_idx, wo = out
    if ws is None:
        ws = nabla_lists_workspace(q, s_valid)
    arr = ctypes.c_int * 3
    g3 = arr(*grid) if grid is not None else None
    t3 = arr(*tile) if tile is not None else None
    w3 = arr(*window) if window is not None else None
    ot = arr(*order_tile) if order_tile is not None else None
    nf = _near_buffer(q, near)
    tq, tk = _tensor(q), _tensor(k)
    _check(lib.nabla_build_mask_lists(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(shp), float(thr),
                                      float(scale) if scale else 0.0, g3, t3, w3, 0 if order == "row" else 1, ot,
                                      mask.data_ptr(), nf.data_ptr() if nf is not None else None,
                                      kv_len.data_ptr(), kv_idx.data_ptr(),
                                      wo.data_ptr() if wo is not None else None, ws.data_ptr(), ws.numel(),
                                      _stream(q.device)))
    return mask, kv_len, kv_idx, wo


def mask_or(a: torch.Tensor, b: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """a | b elementwise; b may be one [nb, nb] plane broadcast over a [B,H,nb,nb] mask."""
    lib = load()
    if not (a.is_contiguous() and b.is_contiguous()):
        raise ValueError("mask_or needs contiguous masks")
    if out is None:
        out = torch.empty_like(a, dtype=torch.uint8)
    _check(lib.mask_or(out.data_ptr(), a.data_ptr(), a.numel(), b.data_ptr(), b.numel(), _stream(a.device)))
    return out


def mask_to_csr(mask: torch.Tensor, B: Optional[int] = None, H: Optional[int] = None,
                row_ptr: Optional[torch.Tensor] = None, col_idx: Optional[torch.Tensor] = None,
                ws: Optional[torch.Tensor] = None, order: Optional[torch.Tensor] = None,
                return_order: bool = False, work_order: Optional[torch.Tensor] = None):
    """Per-query-block kv lists of a [B,H,nb,nb] mask (or one [nb,nb] plane broadcast
    over B, H) -> (row_ptr int32 [B*H*nb+1], col_idx int32 [B*H*nb*nb]); with
    return_order (or an `order` buffer) also the rows sorted by kept count,
    descending, ties by row index (int32 [B*H*nb]). With `work_order` (int32
    [attn_work_order_slots]) the attention work order of the lists is written into it
    in the same call (bsa_mask_to_csr_ordered); it cannot be combined with `order`."""
    lib = load()
    ptr, sb, sh, m = _mask_strides(mask)
    B = B or m.shape[0]
    H = H or m.shape[1]
    nb = m.shape[-1]
    rows = B * H * nb
    if row_ptr is None:
        row_ptr = torch.empty(rows + 1, dtype=torch.int32, device=m.device)
    if col_idx is None:
        col_idx = torch.empty(rows * nb, dtype=torch.int32, device=m.device)
    if ws is None:
        ws = _ws(lib.csr_workspace_size(B, H, nb), m.device)
    if work_order is not None:
        if order is not None or return_order:
            raise ValueError("work_order cannot be combined with order")
        _check(lib.bsa_mask_to_csr_ordered(ptr, sb, sh, B, H, nb, row_ptr.data_ptr(), col_idx.data_ptr(),
                                           work_order.data_ptr(), ws.data_ptr(), ws.numel(), _stream(m.device)))
        return row_ptr, col_idx
    if return_order and order is None:
        order = torch.empty(rows, dtype=torch.int32, device=m.device)
    _check(lib.bsa_mask_to_csr(ptr, sb, sh, B, H, nb, row_ptr.data_ptr(), col_idx.data_ptr(),
                               order.data_ptr() if order is not None else None, ws.data_ptr(), ws.numel(),
                               _stream(m.device)))
    if order is not None:
        return row_ptr, col_idx, order
    return row_ptr, col_idx


class AttnPlan:
    """Reusable output and workspace buffers for repeated block_sparse_attn_fwd calls."""

    def __init__(self, q: torch.Tensor, v: torch.Tensor, s_valid: Optional[int] = None, lse: bool = False):
        lib = load()
        self.shape = _shape(q, s_valid)
        self.qk_code = _dtype_code(q)
        self.ws = _ws(lib.attn_workspace_size(ctypes.byref(self.shape), self.qk_code), q.device)
        odt = torch.float32 if q.dtype == torch.float32 else torch.bfloat16
        self.out = torch.empty(q.shape, dtype=odt, device=q.device)
        self.lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if lse else None


def block_sparse_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mask: torch.Tensor,
                          scale: Optional[float] = None, s_valid: Optional[int] = None,
                          q_scale: Optional[torch.Tensor] = None, k_scale: Optional[torch.Tensor] = None,
                          return_lse: bool = False, plan: Optional[AttnPlan] = None):
    """Attention over the kept 64x64 tiles of `mask` ([B,H,nb,nb] or one [nb,nb] plane).

    q, k: bf16, f32, or fp8 e4m3 codes (uint8 / float8_e4m3fn, then q_scale, k_scale
    are float32 [B,H,nb]); v bf16 (f32 for f32 q, k). Returns O (and lse if asked).
    """
    lib = load()
    if plan is None:
        plan = AttnPlan(q, v, s_valid, lse=return_lse)
    ptr, sb, sh, _m = _mask_strides(mask)
    tq, tk, tv, to = _tensor(q), _tensor(k), _tensor(v), _tensor(plan.out)
    qs = q_scale.data_ptr() if q_scale is not None else None
    ks = k_scale.data_ptr() if k_scale is not None else None
    lse_ptr = plan.lse.data_ptr() if (return_lse and plan.lse is not None) else None
    _check(lib.block_sparse_attn_fwd(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), ctypes.byref(plan.shape),
                                     ptr, sb, sh, qs, ks, float(scale) if scale else 0.0, ctypes.byref(to), lse_ptr,
                                     plan.ws.data_ptr(), plan.ws.numel(), _stream(q.device)))
    if return_lse:
        return plan.out, plan.lse
    return plan.out


def set_attn_kv_chunk(kv_chunk: int) -> int:
    """Chunk width (key blocks) of the attention's kv-chunked walk for the whole process:
    > 0 that width for every shape, < 0 never chunk, 0 the automatic choice. Returns the
    previous setting; workspaces sized before a change do not follow it."""
    return int(load().bsa_set_attn_kv_chunk(int(kv_chunk)))


def attn_pair_offsets(q: torch.Tensor, row_ptr: Optional[torch.Tensor], col_idx: torch.Tensor,
                      kv_len: Optional[torch.Tensor] = None, s_valid: Optional[int] = None) -> torch.Tensor:
    """Pairing offset of each head (int32 [B*H]) that the attention picks for these kv lists:
    CSR (row_ptr, col_idx), or with row_ptr None the fixed-stride lists (kv_len, col_idx)."""
    lib = load()
    shp = _shape(q, s_valid)
    out = torch.empty(q.shape[0] * q.shape[1], dtype=torch.int32, device=q.device)
    ws = _ws(lib.attn_pair_workspace_size(ctypes.byref(shp)), q.device)
    _check(lib.attn_pair_offsets(ctypes.byref(shp), row_ptr.data_ptr() if row_ptr is not None else None,
                                 col_idx.data_ptr(), kv_len.data_ptr() if kv_len is not None else None,
                                 out.data_ptr(), ws.data_ptr(), ws.numel(), _stream(q.device)))
    return out


def attn_work_order_slots(q: torch.Tensor, s_valid: Optional[int] = None) -> int:
    """Length of the attention work order for tensors shaped like q (0: the shape runs in
    the default order, each workgroup deriving its item in the kernel)."""
    lib = load()
    shp = _shape(q, s_valid)
    n = lib.attn_work_order_slots(ctypes.byref(shp))
    if n < 0:
        raise BsaError(1, lib.bsa_last_error().decode())
    return int(n)


def attn_work_order(q: torch.Tensor, row_ptr: torch.Tensor, s_valid: Optional[int] = None,
                    out: Optional[torch.Tensor] = None) -> Optional[torch.Tensor]:
    """Work order of the attention kernel for the kv lists row_ptr (int32 [slots], -1 =
    no item), or None when the shape runs in the default order."""
    lib = load()
    shp = _shape(q, s_valid)
    n = lib.attn_work_order_slots(ctypes.byref(shp))
    if n < 0:
        raise BsaError(1, lib.bsa_last_error().decode())
    if n == 0:
        return None
    if out is None:
        out = torch.empty(n, dtype=torch.int32, device=q.device)
    _check(lib.attn_work_order(ctypes.byref(shp), row_ptr.data_ptr(), out.data_ptr(), _stream(q.device)))
    return out


def block_sparse_attn_fwd_csr(q, k, v, row_ptr, col_idx, scale=None, s_valid=None, q_scale=None, k_scale=None,
                              return_lse=False, out=None, lse=None, ws=None, work_order=None):
    """Attention over prebuilt kv lists (see mask_to_csr), optionally with a work order
    from attn_work_order (computed internally when None)."""
    lib = load()
    shp = _shape(q, s_valid)
    code = _dtype_code(q)
    if ws is None:
        ws = _ws(lib.attn_csr_workspace_size(ctypes.byref(shp), code), q.device)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32 if q.dtype == torch.float32 else torch.bfloat16,
                          device=q.device)
    if return_lse and lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    tq, tk, tv, to = _tensor(q), _tensor(k), _tensor(v), _tensor(out)
    _check(lib.block_sparse_attn_fwd_csr(
        ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), ctypes.byref(shp), row_ptr.data_ptr(),
        col_idx.data_ptr(), work_order.data_ptr() if work_order is not None else None,
        q_scale.data_ptr() if q_scale is not None else None,
        k_scale.data_ptr() if k_scale is not None else None, float(scale) if scale else 0.0, ctypes.byref(to),
        lse.data_ptr() if return_lse else None, ws.data_ptr(), ws.numel(), _stream(q.device)))
    return (out, lse) if return_lse else out


def block_sparse_attn_fwd_lists(q, k, v, kv_len, kv_idx, scale=None, s_valid=None, q_scale=None, k_scale=None,
                                return_lse=False, out=None, lse=None, ws=None, work_order=None):
    """Attention over the fixed-stride kv lists of nabla_build_mask_lists, optionally with
    its work order (computed internally when None)."""
    lib = load()
    shp = _shape(q, s_valid)
    code = _dtype_code(q)
    if ws is None:
        ws = _ws(lib.attn_csr_workspace_size(ctypes.byref(shp), code), q.device)
    if out is None:
        out = torch.empty(q.shape, dtype=torch.float32 if q.dtype == torch.float32 else torch.bfloat16,
                          device=q.device)
    if return_lse and lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    tq, tk, tv, to = _tensor(q), _tensor(k), _tensor(v), _tensor(out)
    _check(lib.block_sparse_attn_fwd_lists(
        ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), ctypes.byref(shp), kv_len.data_ptr(),
        kv_idx.data_ptr(), work_order.data_ptr() if work_order is not None else None,
        q_scale.data_ptr() if q_scale is not None else None,
        k_scale.data_ptr() if k_scale is not None else None, float(scale) if scale else 0.0, ctypes.byref(to),
        lse.data_ptr() if return_lse else None, ws.data_ptr(), ws.numel(), _stream(q.device)))
    return (out, lse) if return_lse else out


def block_sparse_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, do: torch.Tensor,
                          lse: torch.Tensor, mask: torch.Tensor, scale: Optional[float] = None,
                          s_valid: Optional[int] = None, grad_dtype: Optional[torch.dtype] = None,
                          out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None,
                          ws: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv) of block_sparse_attn_fwd for the upstream gradient `do`.

    q, k, v, o, do: bf16 [B,H,S,D]; lse: the forward's float32 [B,H,S] output; mask and
    scale as in the forward. Gradients are bf16 (default) or float32 (grad_dtype).
    """
    lib = load()
    shape = _shape(q, s_valid)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != tuple(q.shape[:3]):
        raise ValueError("lse must be a contiguous float32 [B, H, S] tensor")
    gdt = grad_dtype or torch.bfloat16
    if out is None:
        out = tuple(torch.empty(q.shape, dtype=gdt, device=q.device) for _ in range(3))
    if ws is None:
        ws = _ws(lib.attn_bwd_workspace_size(ctypes.byref(shape)), q.device)
    ptr, sb, sh, _m = _mask_strides(mask)
    t = [_tensor(x) for x in (q, k, v, o, do) + tuple(out)]
    _check(lib.block_sparse_attn_bwd(*(ctypes.byref(x) for x in t[:5]), lse.data_ptr(), ctypes.byref(shape),
                                     ptr, sb, sh, float(scale) if scale else 0.0,
                                     *(ctypes.byref(x) for x in t[5:]), ws.data_ptr(), ws.numel(),
                                     _stream(q.device)))
    return out


ORDER_CODES = {"row": 0, "tile": 1, "spatial": 2}


def token_reorder(x: torch.Tensor, grid: Sequence[int], order: str, tile: Optional[Sequence[int]] = None,
                  inverse: bool = False, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Permute the T*H*W token rows of x [B,H,S,D] from row-major (t, h, w) to `order`
    ("tile" with `tile`, e.g. (1, P, P) for fractal flattening; "spatial"; "row"), or
    back with inverse=True. Rows >= T*H*W of the result are zero."""
    lib = load()
    if out is None:
        out = torch.empty_like(x)
    shp = _shape(x, int(grid[0]) * int(grid[1]) * int(grid[2]))
    a3 = ctypes.c_int * 3
    t = a3(*tile) if tile is not None else None
    tx, to = _tensor(x), _tensor(out)
    _check(lib.token_reorder(ctypes.byref(tx), ctypes.byref(shp), a3(*grid), ORDER_CODES[order], t, int(inverse),
                             ctypes.byref(to), _stream(x.device)))
    return out
