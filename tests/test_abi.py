"""The C-ABI library loads, exports every declared symbol, and rejects bad arguments
on the host before any launch (CPU only: no compute call reaches the GPU)."""
import ctypes
import os
import re

import pytest

import block_sparse_attention_mask_amd as bsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "bsa.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return bsa.load()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) >= 13
    assert sorted(names) == sorted(bsa.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version(lib):
    assert lib.bsa_abi_version() == 13


def _t(ptr=256, dtype=bsa.BSA_BF16, ss=128):
    return bsa.Tensor(ptr, dtype, 0, 0, ss)


def _nabla(lib, shape, thr=0.2, q=None, k=None, mask=4096, ws=8192, ws_bytes=1 << 40, near=None):
    q = q or _t()
    k = k or _t()
    return lib.nabla_build_mask(ctypes.byref(q), ctypes.byref(k), ctypes.byref(shape), thr, 0.0, None, 0, 0, mask,
                                near, ws, ws_bytes, None)


@pytest.mark.parametrize("shape,thr,msg", [
    (bsa.Shape(1, 2, 256, 256, 128, 64), 1.0, "thr"),
    (bsa.Shape(1, 2, 256, 256, 128, 64), -0.1, "thr"),
    (bsa.Shape(1, 2, 250, 250, 128, 64), 0.2, "multiple of 64"),
    (bsa.Shape(1, 2, 256, 300, 128, 64), 0.2, "S_valid"),
    (bsa.Shape(0, 2, 256, 256, 128, 64), 0.2, "B="),
    (bsa.Shape(1, 2, 256, 256, 96, 64), 0.2, "head dim"),
    (bsa.Shape(1, 2, 256, 256, 128, 32), 0.2, "block size"),
    (bsa.Shape(1, 1, 64 * 2049, 64 * 2049, 128, 64), 0.2, "2048"),
])
def test_nabla_rejects_bad_arguments(lib, shape, thr, msg):
    st = _nabla(lib, shape, thr)
    assert st in (1, 2)
    assert msg in lib.bsa_last_error().decode()


def test_nabla_rejects_misaligned_and_mixed(lib):
    shape = bsa.Shape(1, 2, 256, 256, 128, 64)
    assert _nabla(lib, shape, q=_t(ptr=258)) == 1
    assert _nabla(lib, shape, q=_t(ss=100)) == 1
    assert _nabla(lib, shape, k=_t(dtype=bsa.BSA_F32)) == 2
    assert _nabla(lib, shape, ws_bytes=16) == 3
    assert "workspace" in lib.bsa_last_error().decode()
    assert _nabla(lib, shape, near=4096) == 1                 # flags may not alias the mask
    assert "alias" in lib.bsa_last_error().decode()
    assert _nabla(lib, shape, mask=None) == 1


def test_sta_rejects_bad_geometry(lib):
    shape = bsa.Shape(1, 1, 256, 256, 64, 64)
    a3 = ctypes.c_int * 3
    st = lib.sta_build_mask(ctypes.byref(shape), a3(4, 8, 8), a3(4, 8, 8), a3(3, 2, 3), 0, None, 4096, 8192,
                            1 << 20, None)
    assert st == 1 and "odd" in lib.bsa_last_error().decode()
    st = lib.sta_build_mask(ctypes.byref(shape), a3(4, 8, 9), a3(4, 8, 8), a3(3, 3, 3), 0, None, 4096, 8192,
                            1 << 20, None)
    assert st == 1 and "S_valid" in lib.bsa_last_error().decode()
    st = lib.sta_build_mask(ctypes.byref(shape), a3(4, 8, 8), a3(4, 8, 8), a3(3, 3, 3), 1, None, 4096, 8192,
                            1 << 20, None)
    assert st == 1


def test_nabla_sta_rejects(lib):
    # NABLA OR sliding tiles in one call: the checks of both calls, before any launch
    shape = bsa.Shape(1, 2, 256, 256, 128, 64)
    a3 = ctypes.c_int * 3
    q, k = _t(), _t(4096)
    f = lib.nabla_build_mask_sta
    need = lib.nabla_sta_workspace_size(ctypes.byref(shape))
    assert need >= lib.nabla_workspace_size(ctypes.byref(shape)) + 16
    st = f(ctypes.byref(q), ctypes.byref(k), ctypes.byref(shape), 0.1, 0.0, a3(4, 8, 8), a3(4, 8, 8), a3(3, 2, 3), 0,
           None, 8192, None, 1 << 16, need, None)
    assert st == 1 and "odd" in lib.bsa_last_error().decode()
    st = f(ctypes.byref(q), ctypes.byref(k), ctypes.byref(shape), 0.1, 0.0, a3(4, 8, 9), a3(4, 8, 8), a3(3, 3, 3), 0,
           None, 8192, None, 1 << 16, need, None)
    assert st == 1 and "S_valid" in lib.bsa_last_error().decode()
    st = f(ctypes.byref(q), ctypes.byref(k), ctypes.byref(shape), 0.1, 0.0, a3(4, 8, 8), a3(4, 8, 8), a3(3, 3, 3), 0,
           None, 8192, None, 1 << 16, need - 1, None)
    assert st == 3
    st = f(ctypes.byref(q), ctypes.byref(k), ctypes.byref(shape), 1.5, 0.0, a3(4, 8, 8), a3(4, 8, 8), a3(3, 3, 3), 0,
           None, 8192, None, 1 << 16, need, None)
    assert st == 1 and "thr" in lib.bsa_last_error().decode()


def test_nabla_lists_rejects(lib):
    # mask + kv lists in one call: every check before any launch
    a3 = ctypes.c_int * 3
    q, k = _t(), _t(4096)
    f = lib.nabla_build_mask_lists

    def call(shape, kv_len=8192, kv_idx=16384, order=None, ws_bytes=None, thr=0.1, grid=None):
        need = lib.nabla_lists_workspace_size(ctypes.byref(shape))
        return f(ctypes.byref(q), ctypes.byref(k), ctypes.byref(shape), thr, 0.0, grid, a3(4, 8, 8) if grid else None,
                 a3(3, 3, 3) if grid else None, 0, None, 32768, None, kv_len, kv_idx, order, 1 << 16,
                 need if ws_bytes is None else ws_bytes, None)
    small = bsa.Shape(1, 2, 256, 256, 128, 64)
    assert lib.nabla_lists_workspace_size(ctypes.byref(small)) >= lib.nabla_sta_workspace_size(ctypes.byref(small))
    assert call(bsa.Shape(1, 1, 64 * 257, 64 * 257, 128, 64)) == 2          # nb > 256
    assert "nb <= 256" in lib.bsa_last_error().decode()
    assert call(small, kv_len=None) == 1
    assert call(small, kv_idx=None) == 1
    assert call(small, ws_bytes=100) == 3
    assert call(small, thr=1.0) == 1 and "thr" in lib.bsa_last_error().decode()
    assert call(small, grid=a3(4, 8, 9)) == 1 and "S_valid" in lib.bsa_last_error().decode()
    # 64 heads x 128 pairs = 8192 items: more than four rounds, no work order for this shape
    assert call(bsa.Shape(1, 64, 64 * 256, 64 * 256, 128, 64), order=8192) == 2
    assert "default order" in lib.bsa_last_error().decode()


def test_attention_lists_rejects(lib):
    shape = bsa.Shape(1, 2, 256, 256, 128, 64)
    q, k, v, o = _t(), _t(), _t(), _t()
    f = lib.block_sparse_attn_fwd_lists
    need = lib.attn_csr_workspace_size(ctypes.byref(shape), bsa.BSA_BF16)

    def call(kv_len=8192, kv_idx=16384, ws_bytes=need, vv=v):
        return f(ctypes.byref(q), ctypes.byref(k), ctypes.byref(vv), ctypes.byref(shape), kv_len, kv_idx, None, None,
                 None, 0.0, ctypes.byref(o), None, 32768, ws_bytes, None)
    assert call(kv_len=None) == 1
    assert call(kv_idx=None) == 1
    assert call(vv=_t(dtype=bsa.BSA_F32)) == 1
    if need:
        assert call(ws_bytes=need - 1) == 3


def test_mask_or_and_csr_reject(lib):
    assert lib.mask_or(4096, 4096, 10, 8192, 3, None) == 1
    assert lib.mask_or(None, 4096, 10, 8192, 10, None) == 1
    assert lib.bsa_mask_to_csr(4096, -1, 0, 1, 1, 4, 8192, 8192, None, 8192, 1 << 20, None) == 1
    assert lib.bsa_mask_to_csr(4096, 0, 0, 1, 1, 4, 8192, 8192, None, 8192, 0, None) == 3
    # kv lists with the attention work order: NULL order, bad stride, a shape that runs in
    # the default order (64 heads x 64 pairs = 4096 items > 4 rounds), too small a workspace
    f = lib.bsa_mask_to_csr_ordered
    assert f(4096, 0, 0, 1, 16, 128, 8192, 8192, None, 8192, 1 << 20, None) == 1
    assert f(4096, -1, 0, 1, 16, 128, 8192, 8192, 8192, 8192, 1 << 20, None) == 1
    assert f(4096, 0, 0, 1, 64, 128, 8192, 8192, 8192, 8192, 1 << 20, None) == 2
    assert "default order" in lib.bsa_last_error().decode()
    assert f(4096, 0, 0, 1, 16, 128, 8192, 8192, 8192, 8192, 0, None) == 3


def test_attention_rejects(lib):
    shape = bsa.Shape(1, 2, 256, 256, 128, 64)
    q, k, v, o = _t(), _t(), _t(), _t()
    ws = lib.attn_workspace_size(ctypes.byref(shape), bsa.BSA_BF16)
    assert ws > 0
    args = lambda **kw: dict(dict(q=q, k=k, v=v, o=o, mask=4096, qs=None, ks=None, ws=4096, wsb=ws), **kw)

    def call(a):
        return lib.block_sparse_attn_fwd(ctypes.byref(a["q"]), ctypes.byref(a["k"]), ctypes.byref(a["v"]),
                                         ctypes.byref(shape), a["mask"], 0, 0, a["qs"], a["ks"], 0.0,
                                         ctypes.byref(a["o"]), None, a["ws"], a["wsb"], None)
    assert call(args(v=_t(dtype=bsa.BSA_F32))) == 1
    assert call(args(q=_t(dtype=bsa.BSA_FP8_E4M3FN, ss=128), k=_t(dtype=bsa.BSA_FP8_E4M3FN))) == 1   # no scales
    assert "scale" in lib.bsa_last_error().decode()
    assert call(args(mask=None)) == 1
    assert call(args(wsb=ws - 1)) == 3
    assert call(args(ws=4097)) == 1
    f32 = lib.attn_workspace_size(ctypes.byref(shape), bsa.BSA_F32)
    assert f32 > ws            # f32 inputs need room for their bf16 hi/lo copies


def _bwd(lib, shape, q=None, o=None, dq=None, dk=None, lse=4096, mask=4096, ws_bytes=1 << 40):
    t = [q or _t(), _t(), _t(), o or _t(), _t()]
    g = [dq or _t(), dk or _t(), _t()]
    return lib.block_sparse_attn_bwd(*(ctypes.byref(x) for x in t), lse, ctypes.byref(shape), mask, 0, 0, 0.0,
                                     *(ctypes.byref(x) for x in g), 8192, ws_bytes, None)


def test_backward_rejects_bad_arguments(lib):
    shape = bsa.Shape(1, 2, 256, 256, 128, 64)
    assert _bwd(lib, shape, q=_t(dtype=bsa.BSA_FP8_E4M3FN)) == 2
    assert "bf16" in lib.bsa_last_error().decode()
    assert _bwd(lib, shape, o=_t(ptr=258)) == 1
    assert _bwd(lib, shape, dq=_t(dtype=bsa.BSA_F32)) == 1              # dq f32, dk bf16
    assert "all three" in lib.bsa_last_error().decode() or "all f32" in lib.bsa_last_error().decode()
    assert _bwd(lib, shape, lse=None) == 1
    assert _bwd(lib, shape, mask=None) == 1
    assert _bwd(lib, shape, ws_bytes=16) == 3
    assert _bwd(lib, bsa.Shape(1, 2, 256, 256, 96, 64)) == 2
    assert lib.attn_bwd_workspace_size(ctypes.byref(shape)) > 0


def test_fp8_entry_points_reject_bad_arguments(lib):
    shape = bsa.Shape(1, 2, 256, 256, 128, 64)
    x, codes = _t(), _t(dtype=bsa.BSA_FP8_E4M3FN)
    assert lib.quantize_fp8_blocks(ctypes.byref(x), ctypes.byref(shape), ctypes.byref(_t()), 4096, None) == 1
    assert "fp8" in lib.bsa_last_error().decode()
    assert lib.quantize_fp8_blocks(ctypes.byref(x), ctypes.byref(shape), ctypes.byref(codes), 4098, None) == 1
    assert lib.quantize_fp8_blocks(ctypes.byref(codes), ctypes.byref(shape), ctypes.byref(codes), 4096, None) == 2
    st = lib.nabla_build_mask_fp8(ctypes.byref(x), ctypes.byref(x), ctypes.byref(shape), 0.2, 0.0, None, 0, 0, 4096,
                                  None, ctypes.byref(codes), None, ctypes.byref(codes), 4096, 8192, 1 << 40, None)
    assert st == 1 and "scales" in lib.bsa_last_error().decode()


def test_topk_rejects_bad_arguments(lib):
    shape = bsa.Shape(1, 2, 256, 256, 128, 64)
    q = _t()
    st = lib.nabla_build_mask_topk(ctypes.byref(q), ctypes.byref(q), ctypes.byref(shape), 0, 0.0, None, 0, 0, 4096,
                                   8192, 1 << 40, None)
    assert st == 1 and "topk" in lib.bsa_last_error().decode()


def test_noalloc_rejects_before_touching_the_device(lib):
    # more scratch than the library's static array holds: rejected on the host, no HIP call
    big = bsa.Shape(1, 100, 64 * 2048, 64 * 2048, 128, 64)
    assert lib.nabla_workspace_size(ctypes.byref(big)) > (128 << 20)
    q = _t()
    st = lib.nabla_build_mask_noalloc(ctypes.byref(q), ctypes.byref(q), ctypes.byref(big), 0.2, 0.0, None, 0, 0,
                                      4096, None, None)
    assert st == 2 and "scratch" in lib.bsa_last_error().decode()
    # the 40-head 14B 720p shape fits
    cfg3 = bsa.Shape(1, 40, 75648, 75600, 128, 64)
    assert lib.nabla_workspace_size(ctypes.byref(cfg3)) <= (128 << 20)
    bad = bsa.Shape(1, 2, 250, 250, 128, 64)
    assert lib.nabla_build_mask_noalloc(ctypes.byref(q), ctypes.byref(q), ctypes.byref(bad), 0.2, 0.0, None, 0, 0,
                                        4096, None, None) == 1


def test_rotated_quantisation_rejects_bad_arguments(lib):
    """Incoherent processing: the sign words are required and key_side is 0 or 1; both are
    checked on the host before any launch."""
    shape = bsa.Shape(1, 2, 256, 256, 128, 64)
    x, codes = _t(), _t(dtype=bsa.BSA_FP8_E4M3FN)
    words = (ctypes.c_uint64 * 2)(0x5, 0x3)
    assert lib.quantize_fp8_blocks_rotated(ctypes.byref(x), ctypes.byref(shape), None, 0, ctypes.byref(codes),
                                           4096, None) == 1
    assert "sign_bits" in lib.bsa_last_error().decode()
    assert lib.quantize_fp8_blocks_rotated(ctypes.byref(x), ctypes.byref(shape), words, 2, ctypes.byref(codes),
                                           4096, None) == 1
    assert "key_side" in lib.bsa_last_error().decode()
    q8, k8 = _t(dtype=bsa.BSA_FP8_E4M3FN), _t(dtype=bsa.BSA_FP8_E4M3FN)
    st = lib.nabla_build_mask_fp8_rotated(ctypes.byref(_t()), ctypes.byref(_t()), ctypes.byref(shape), 0.2, 0.0,
                                          None, 0, 0, 4096, None, None, ctypes.byref(q8), 8192,
                                          ctypes.byref(k8), 12288, 16384, 1 << 40, None)
    assert st == 1 and "sign_bits" in lib.bsa_last_error().decode()
    with pytest.raises(ValueError):
        bsa._sign_words([1.0, -1.0, 0.5] + [1.0] * 125, 128)
    w = bsa._sign_words([-1.0 if d in (0, 63, 64, 127) else 1.0 for d in range(128)], 128)
    assert list(w) == [(1 << 0) | (1 << 63), (1 << 0) | (1 << 63)]


def test_checked_build_exports_the_same_calls():
    """The checked library (built beside the production one) exports every declared call,
    reports itself as checked and starts with no flag set (reading the flags needs no GPU
    work: both calls are host-side in the production library)."""
    lib = bsa.load()
    assert lib.bsa_checked_build() == 0
    assert lib.bsa_check_flags(0) == 0
    assert os.path.exists(bsa.CHECKED_LIB_PATH), "libbsa_checked.so is not built"
    chk = ctypes.CDLL(bsa.CHECKED_LIB_PATH)
    for n in _declared():
        assert hasattr(chk, n), n
    assert chk.bsa_checked_build() == 1
    assert chk.bsa_abi_version() == lib.bsa_abi_version()
