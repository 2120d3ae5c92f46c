"""The C-ABI library on the CPU: it loads, exports every declared symbol, and
rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

import block_sparse_masked_amd as lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            names += re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\**\s*(flexattn_[a-z_]+)\s*\(",
                                text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    return lib.load_library()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("flexattn_create_block_mask", "flexattn_fwd", "flexattn_bwd",
                     "flexattn_block_mask_sizes", "flexattn_last_error", "flexattn_version"):
        assert required in names


def test_library_exports_every_declared_symbol(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_version_and_last_error(L):
    assert lib.version().startswith("flexattn-gfx950")
    assert isinstance(L.flexattn_last_error(), bytes)


def test_block_mask_sizes(L):
    assert lib.block_mask_sizes(4, 16, 4096, 4096) == (4 * 16 * 32, 4 * 16 * 32 * 32, 4 * 16 * 32)
    assert lib.block_mask_sizes(1, 1, 300, 129) == (3, 3 * 2, 3)
    with pytest.raises(NotImplementedError, match="block must be 128"):
        lib.block_mask_sizes(1, 1, 256, 256, 64)
    # multiples of 128 up to 512
    assert lib.block_mask_sizes(2, 3, 1000, 700, 256) == (2 * 3 * 4, 2 * 3 * 4 * 3, 2 * 3 * 4)
    # the tuple form (KV_BLOCK_SIZE, Q_BLOCK_SIZE)
    assert lib.block_mask_sizes(2, 3, 1000, 700, (256, 128)) == (2 * 3 * 8, 2 * 3 * 8 * 3, 2 * 3 * 8)
    for bad in (192, 640):
        with pytest.raises(NotImplementedError, match="block must be 128"):
            lib.block_mask_sizes(1, 1, 256, 256, bad)
    with pytest.raises(ValueError, match="must be >= 1"):
        lib.block_mask_sizes(0, 1, 256, 256)


def _bm_struct(ptr=16):
    c = lib._BlockMask()
    for f in ("kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices", "schedule"):
        setattr(c, f, ptr)
    return c


def _create(L, kind, params, B=1, H=1, Q=256, K=256, block=128, bm=None):
    bm = _bm_struct() if bm is None else bm
    p = ctypes.byref(params) if params is not None else None
    return L.flexattn_create_block_mask(kind, p, B, H, Q, K, block, 1, ctypes.byref(bm), None)


def test_create_block_mask_rejects_bad_arguments(L):
    mp = lib._MaskParams(0, 0, None, 0, 0)
    assert _create(L, 9, mp) == lib._UNSUPPORTED
    assert b"mask_kind" in L.flexattn_last_error()
    assert _create(L, 1, mp, block=64) == lib._UNSUPPORTED
    assert _create(L, 1, mp, Q=0) == lib._INVALID
    assert _create(L, 1, mp, bm=_bm_struct(ptr=0)) == lib._INVALID
    assert L.flexattn_create_block_mask(1, None, 1, 1, 256, 256, 128, 1, None, None) == lib._INVALID
    # sliding window needs window >= 1 and sinks >= 0
    assert _create(L, 2, lib._MaskParams(0, 0, None, 0, 0)) == lib._INVALID
    assert b"window" in L.flexattn_last_error()
    assert _create(L, 2, lib._MaskParams(4, -1, None, 0, 0)) == lib._INVALID
    assert _create(L, 2, None) == lib._INVALID
    # documents need ids, a long enough row and a valid batch count
    assert _create(L, 3, lib._MaskParams(0, 0, None, 1, 256)) == lib._INVALID
    assert _create(L, 3, lib._MaskParams(0, 0, 64, 1, 100)) == lib._INVALID
    assert b"doc_len" in L.flexattn_last_error()
    assert _create(L, 3, lib._MaskParams(0, 0, 64, 3, 256), B=2) == lib._INVALID
    # PrefixLM needs params with prefix_len >= 0
    assert _create(L, 4, None) == lib._INVALID
    assert _create(L, 4, lib._MaskParams(0, 0, None, 0, 0, -1)) == lib._INVALID
    assert b"prefix_len" in L.flexattn_last_error()
    # builder limit on KV length
    assert _create(L, 1, mp, K=128 * 5000) == lib._UNSUPPORTED


def _tensor(dtype=1, B=1, H=2, L_=256, D=64, data=4096, strides=None):
    if strides is None:
        strides = (H * L_ * D, L_ * D, D, 1)
    return lib._Tensor(data, dtype, B, H, L_, D, (ctypes.c_int64 * 4)(*strides))


def _good_bm():
    c = _bm_struct(ptr=4096)
    c.B, c.H, c.Q_LEN, c.KV_LEN, c.BLOCK_SIZE = 1, 1, 256, 256, 128
    c.num_q_blocks, c.num_kv_blocks = 2, 2
    c.mask_kind = 1
    return c


def _fwd(L, q=None, k=None, v=None, o=None, bm=None, score=0, sp=None, scale=0.125, lse=4096):
    q = _tensor() if q is None else q
    k = _tensor() if k is None else k
    v = _tensor() if v is None else v
    o = _tensor() if o is None else o
    bm = _good_bm() if bm is None else bm
    sp = lib._ScoreParams(0.0, None) if sp is None else sp
    return L.flexattn_fwd(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(bm),
                          score, ctypes.byref(sp), scale, ctypes.byref(o),
                          ctypes.c_void_p(lse), None)


@pytest.mark.parametrize("case,expect,msg", [
    (dict(q=_tensor(data=0)), lib._INVALID, b"q->data is NULL"),
    (dict(k=_tensor(dtype=7)), lib._UNSUPPORTED, b"dtype"),
    (dict(q=_tensor(D=96), k=_tensor(D=96), v=_tensor(D=96), o=_tensor(D=96)),
     lib._UNSUPPORTED, b"head dim"),
    # 256 is a 16-bit kernel head dim only
    (dict(q=_tensor(dtype=0, D=256), k=_tensor(dtype=0, D=256), v=_tensor(dtype=0, D=256),
          o=_tensor(dtype=0, D=256)), lib._UNSUPPORTED, b"head dim"),
    (dict(v=_tensor(D=128)), lib._INVALID, b"head dims differ"),
    (dict(k=_tensor(H=3), v=_tensor(H=3)), lib._INVALID, b"multiple"),
    (dict(k=_tensor(dtype=0)), lib._INVALID, b"one dtype"),
    (dict(q=_tensor(strides=(2 * 256 * 64, 256 * 64, 64, 2))), lib._INVALID, b"contiguous"),
    (dict(q=_tensor(strides=(2 * 256 * 64, 256 * 64, 60, 1))), lib._INVALID, b"16 bytes"),
    (dict(q=_tensor(data=4098)), lib._INVALID, b"aligned"),
    (dict(lse=0), lib._INVALID, b"lse"),
    (dict(scale=float("nan")), lib._INVALID, b"scale"),
    (dict(score=9), lib._UNSUPPORTED, b"score_kind"),
    (dict(score=2, sp=lib._ScoreParams(0.0, None)), lib._INVALID, b"softcap"),
    (dict(score=3, sp=lib._ScoreParams(float("inf"), None)), lib._INVALID, b"softcap"),
    # bf16 k/v rows more than 2^22 elements apart (a [B][L][H][D] view with H*D > 2^22)
    (dict(k=_tensor(strides=(256 * (1 << 22 + 3), 64, (1 << 22) + 64, 1)),
          v=_tensor(strides=(256 * (1 << 22 + 3), 64, (1 << 22) + 64, 1))),
     lib._UNSUPPORTED, b"row stride"),
])
def test_fwd_rejects_bad_arguments(L, case, expect, msg):
    assert _fwd(L, **case) == expect
    assert msg in L.flexattn_last_error()


def test_fwd_rejects_mismatched_block_mask(L):
    bm = _good_bm()
    bm.Q_LEN = 512
    assert _fwd(L, bm=bm) == lib._INVALID
    bm = _good_bm()
    bm.BLOCK_SIZE = 64
    assert _fwd(L, bm=bm) == lib._UNSUPPORTED
    bm = _good_bm()
    bm.H = 3
    assert _fwd(L, bm=bm) == lib._INVALID
    bm = _good_bm()
    bm.num_kv_blocks = 5
    assert _fwd(L, bm=bm) == lib._INVALID
    bm = _good_bm()
    bm.schedule = 0
    assert _fwd(L, bm=bm) == lib._INVALID


def test_python_wrapper_maps_errors():
    import torch
    with pytest.raises(NotImplementedError):
        lib.create_block_mask("dilated", 1, 1, 128, 128, device="cpu")
    q = torch.zeros(1, 1, 128, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        lib._tensor(q, "q")
    with pytest.raises(NotImplementedError):
        lib._tensor(q.double(), "q")


def test_library_has_no_undefined_internal_symbols():
    """Every kernel the dispatcher launches has its host stub in the library
    (a missing stub only shows up when the library is loaded)."""
    import subprocess
    out = subprocess.run(["nm", "-D", "--undefined-only", lib.library_path()],
                         capture_output=True, text=True, check=True).stdout
    bad = [line for line in out.splitlines() if "_ZN2fa" in line]
    assert not bad, bad[:5]


def _bwd(L, tensors, bm, lse=16, ws=16, score=0):
    t = [ctypes.byref(x) if x is not None else None for x in tensors]
    sp = lib._ScoreParams(0.0, None)
    return L.flexattn_bwd(t[0], t[1], t[2], ctypes.c_void_p(lse), t[3], ctypes.byref(bm),
                          score, ctypes.byref(sp), 0.125, t[4], t[5], t[6],
                          ctypes.c_void_p(ws), None)


def test_bwd_rejects_bad_arguments(L):
    """Host-side checks of the backward (no launch happens)."""
    def tens(dtype=1, H=2, Lq=256, D=128):
        st = (H * Lq * D, Lq * D, D, 1)
        return lib._Tensor(16, dtype, 1, H, Lq, D, (ctypes.c_int64 * 4)(*st))
    bm = _bm_struct()
    bm.B, bm.H, bm.Q_LEN, bm.KV_LEN, bm.BLOCK_SIZE = 1, 1, 256, 256, 128
    bm.num_q_blocks, bm.num_kv_blocks, bm.mask_kind = 2, 2, 1
    good = [tens() for _ in range(7)]
    # no backward lists
    assert _bwd(L, good, bm) == lib._INVALID
    assert b"q_*" in L.flexattn_last_error()
    bm.q_num_blocks = bm.q_indices = bm.full_q_num_blocks = bm.full_q_indices = 16
    # fp32 tensors are not supported by the backward
    f32 = [tens(dtype=0) for _ in range(7)]
    assert _bwd(L, f32, bm) == lib._UNSUPPORTED
    assert b"16-bit" in L.flexattn_last_error()
    # fp16 is accepted, but every tensor must share q's dtype
    mixed = [tens(dtype=2)] + good[1:]
    assert _bwd(L, mixed, bm) == lib._INVALID
    assert b"dtype differs" in L.flexattn_last_error()
    assert _bwd(L, [tens(dtype=2) for _ in range(7)], bm, ws=0) == lib._INVALID
    assert b"workspace" in L.flexattn_last_error()
    # head dim, NULL workspace, NULL tensor, mismatched shapes
    assert _bwd(L, [tens(D=96) for _ in range(7)], bm) == lib._UNSUPPORTED
    assert _bwd(L, good, bm, ws=0) == lib._INVALID
    assert _bwd(L, [None] + good[1:], bm) == lib._INVALID
    bad = list(good)
    bad[4] = tens(Lq=128)
    assert _bwd(L, bad, bm) == lib._INVALID
    assert b"shaped like q" in L.flexattn_last_error()
    # row strides past 2^22 elements (32-bit tile offsets) for q, k, v, d_out
    big = (1 << 22) + 128
    wide = lib._Tensor(16, 1, 1, 2, 256, 128, (ctypes.c_int64 * 4)(2 * 256 * big, 256 * big, big, 1))
    for i in (0, 1, 2, 3):
        bad = list(good)
        bad[i] = wide
        assert _bwd(L, bad, bm) == lib._UNSUPPORTED, i
        assert b"row stride" in L.flexattn_last_error()


def test_from_kv_blocks_rejects_bad_arguments(L):
    """Host-side checks of from_kv_blocks (no launch happens)."""
    fn = L.flexattn_block_mask_from_kv_blocks
    bm = _bm_struct()
    bm.B, bm.H, bm.Q_LEN, bm.KV_LEN, bm.BLOCK_SIZE = 1, 1, 256, 256, 128
    bm.num_q_blocks, bm.num_kv_blocks, bm.mask_kind = 2, 2, 0
    assert fn(ctypes.byref(bm), None, None) == lib._INVALID          # NULL status
    assert b"status" in L.flexattn_last_error()
    assert fn(None, ctypes.c_void_p(16), None) == lib._INVALID       # NULL bm
    bm.num_kv_blocks = 3                                              # inconsistent tile count
    assert fn(ctypes.byref(bm), ctypes.c_void_p(16), None) == lib._INVALID
    bm.num_kv_blocks, bm.BLOCK_SIZE = 2, 64
    assert fn(ctypes.byref(bm), ctypes.c_void_p(16), None) == lib._UNSUPPORTED
    bm.BLOCK_SIZE, bm.mask_kind = 128, 2                              # sliding window, window 0
    assert fn(ctypes.byref(bm), ctypes.c_void_p(16), None) == lib._INVALID


def _fwd_split(L, splits, ws=4096, ws_bytes=1 << 30, q=None, k=None, v=None, o=None):
    q = _tensor() if q is None else q
    k = _tensor() if k is None else k
    v = _tensor() if v is None else v
    o = _tensor() if o is None else o
    bm = _good_bm()
    sp = lib._ScoreParams(0.0, None)
    return L.flexattn_fwd_splitkv(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v),
                                  ctypes.byref(bm), 0, ctypes.byref(sp), 0.125, splits,
                                  ctypes.c_void_p(ws), ws_bytes, ctypes.byref(o),
                                  ctypes.c_void_p(4096), None)


def test_splitkv_workspace_bytes(L):
    fn = L.flexattn_fwd_splitkv_workspace_bytes
    fn.restype = ctypes.c_size_t
    # fp32 partial O [splits][B][Hq][Q_LEN][D] then partial LSE [splits][B][Hq][Q_LEN]
    assert fn(2, 8, 16, 128, 4) == 4 * (4 * 2 * 8 * 16 * 128 + 4 * 2 * 8 * 16)
    assert fn(1, 1, 1, 64, 1) == 4 * (64 + 1)
    assert fn(0, 1, 1, 64, 2) == 0 and fn(1, 1, 1, 64, 0) == 0


@pytest.mark.parametrize("case,expect,msg", [
    (dict(splits=0), lib._INVALID, b"num_splits"),
    (dict(splits=257), lib._INVALID, b"above 256"),
    (dict(splits=2, ws=0), lib._INVALID, b"workspace"),
    (dict(splits=2, ws=4100), lib._INVALID, b"16-byte"),
    (dict(splits=2, ws_bytes=1000), lib._INVALID, b"below"),
])
def test_splitkv_rejects_bad_arguments(L, case, expect, msg):
    # the default tensors are bf16 (dtype 1): the checks past the dtype run
    assert _fwd_split(L, **case) == expect
    assert msg in L.flexattn_last_error()


def test_splitkv_is_bf16_only(L):
    t = [_tensor(dtype=0) for _ in range(4)]
    assert _fwd_split(L, 2, q=t[0], k=t[1], v=t[2], o=t[3]) == lib._UNSUPPORTED
    assert b"bf16" in L.flexattn_last_error()


def _fwd_paged(L, pages=True, table=4096, max_pages=2, page=128, dtype=1, splits=1):
    q = _tensor(dtype=dtype)
    kc = _tensor(dtype=dtype, B=5, H=2, L_=page)
    vc = _tensor(dtype=dtype, B=5, H=2, L_=page)
    o = _tensor(dtype=dtype)
    bm = _good_bm()
    sp = lib._ScoreParams(0.0, None)
    pt = lib._PageTable(table, max_pages)
    return L.flexattn_fwd_paged(ctypes.byref(q), ctypes.byref(kc), ctypes.byref(vc),
                                ctypes.byref(pt) if pages else None, ctypes.byref(bm), 0,
                                ctypes.byref(sp), 0.125, splits, None, 0, ctypes.byref(o),
                                ctypes.c_void_p(4096), None)


@pytest.mark.parametrize("case,expect,msg", [
    (dict(pages=False), lib._INVALID, b"pages is NULL"),
    (dict(table=0), lib._INVALID, b"page_table"),
    (dict(table=4098), lib._INVALID, b"aligned"),
    (dict(max_pages=1), lib._INVALID, b"do not cover"),
    (dict(page=64), lib._UNSUPPORTED, b"multiple of 128"),
    (dict(dtype=0), lib._UNSUPPORTED, b"16-bit"),
    (dict(splits=0), lib._INVALID, b"num_splits"),
    (dict(splits=2), lib._INVALID, b"workspace"),
    (dict(dtype=2, splits=0), lib._INVALID, b"num_splits"),
])
def test_fwd_paged_rejects_bad_arguments(L, case, expect, msg):
    # the BlockMask is for KV_LEN 256: two pages of 128 keys cover it
    assert _fwd_paged(L, **case) == expect
    assert msg in L.flexattn_last_error()


def _composite_params(terms, window=0, sinks=0, prefix=0, doc=None, doc_len=0):
    mp = lib._MaskParams(window, sinks, doc, 1 if doc else 0, doc_len, prefix)
    mp.num_terms = len(terms)
    for i, t in enumerate(terms):
        mp.terms[i] = t
    return mp


def test_create_composite_rejects_bad_arguments(L):
    """COMPOSITE: 1..4 terms of 5-bit primitive sets, each used primitive's
    parameter present (all checked before any launch)."""
    assert _create(L, 5, None) == lib._INVALID
    assert _create(L, 5, _composite_params([])) == lib._INVALID
    assert b"num_terms" in L.flexattn_last_error()
    mp = _composite_params([1, 1, 1, 1])
    mp.num_terms = 5
    assert _create(L, 5, mp) == lib._INVALID
    assert _create(L, 5, _composite_params([32])) == lib._INVALID
    assert b"bits" in L.flexattn_last_error()
    assert _create(L, 5, _composite_params([2], window=0)) == lib._INVALID
    assert b"window" in L.flexattn_last_error()
    assert _create(L, 5, _composite_params([4], sinks=-1)) == lib._INVALID
    assert _create(L, 5, _composite_params([8], prefix=-1)) == lib._INVALID
    assert _create(L, 5, _composite_params([16])) == lib._INVALID
    assert b"doc_ids" in L.flexattn_last_error()
    assert _create(L, 5, _composite_params([16], doc=4096, doc_len=100)) == lib._INVALID
    assert b"doc_len" in L.flexattn_last_error()


def test_training_pair_rejects_bad_arguments(L):
    q, k, v, o = _tensor(), _tensor(), _tensor(), _tensor()
    bm = _good_bm()
    sp = lib._ScoreParams(0.0, None)
    assert L.flexattn_fwd_train(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(bm),
                                0, ctypes.byref(sp), 0.125, ctypes.byref(o), ctypes.c_void_p(4096),
                                None, None) == lib._INVALID
    assert b"out_f32" in L.flexattn_last_error()
    assert L.flexattn_fwd_train(ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), ctypes.byref(bm),
                                0, ctypes.byref(sp), 0.125, ctypes.byref(o), ctypes.c_void_p(4096),
                                ctypes.c_void_p(4100), None) == lib._INVALID
    f = [_tensor(dtype=0) for _ in range(4)]
    assert L.flexattn_fwd_train(ctypes.byref(f[0]), ctypes.byref(f[1]), ctypes.byref(f[2]),
                                ctypes.byref(bm), 0, ctypes.byref(sp), 0.125, ctypes.byref(f[3]),
                                ctypes.c_void_p(4096), ctypes.c_void_p(8192), None) == lib._INVALID
    assert b"16-bit" in L.flexattn_last_error()
    t = [_tensor() for _ in range(7)]
    assert L.flexattn_bwd_from_out(*(ctypes.byref(x) for x in t[:3]), ctypes.c_void_p(4096), None,
                                   ctypes.byref(t[3]), ctypes.byref(bm), 0, ctypes.byref(sp),
                                   0.125, *(ctypes.byref(x) for x in t[4:]),
                                   ctypes.c_void_p(4096), None) == lib._INVALID
    assert b"out_f32" in L.flexattn_last_error()
    # out_f32 must be 16-byte aligned (Delta reads it in 16-byte pieces)
    assert L.flexattn_bwd_from_out(*(ctypes.byref(x) for x in t[:3]), ctypes.c_void_p(4096),
                                   ctypes.c_void_p(4100), ctypes.byref(t[3]), ctypes.byref(bm), 0,
                                   ctypes.byref(sp), 0.125, *(ctypes.byref(x) for x in t[4:]),
                                   ctypes.c_void_p(4096), None) == lib._INVALID
    assert b"16-byte aligned" in L.flexattn_last_error()


def test_create_rejects_block_sizes(L):
    assert _create(L, 1, lib._MaskParams(0, 0, None, 0, 0), block=640) == lib._UNSUPPORTED
    assert _create(L, 1, lib._MaskParams(0, 0, None, 0, 0), block=192) == lib._UNSUPPORTED


def test_noalloc_rejects_oversized_partials_on_the_host(L):
    """The allocation-free split-KV entry point refuses, before any HIP call,
    a request whose partials exceed the library's fixed scratch, and a slice
    count below 1; the message names the scratch size."""
    q = _tensor(B=8, H=32, L_=64, D=128)
    k = _tensor(B=8, H=8, L_=4096, D=128)
    bm = _good_bm()
    sp = lib._ScoreParams(0.0, None)
    o = _tensor(B=8, H=32, L_=64, D=128)
    fn = L.flexattn_fwd_splitkv_noalloc
    need = L.flexattn_fwd_splitkv_workspace_bytes(8, 32, 64, 128, 32)
    assert need > 32 * 1024 * 1024
    assert fn(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), ctypes.byref(bm), 0,
              ctypes.byref(sp), 0.125, 32, ctypes.byref(o), ctypes.c_void_p(4096),
              None) == lib._INVALID
    assert b"scratch" in L.flexattn_last_error() and str(32 * 1024 * 1024).encode() in \
        L.flexattn_last_error()
    assert fn(ctypes.byref(q), ctypes.byref(k), ctypes.byref(k), ctypes.byref(bm), 0,
              ctypes.byref(sp), 0.125, 0, ctypes.byref(o), ctypes.c_void_p(4096),
              None) == lib._INVALID
