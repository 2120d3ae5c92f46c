"""MI355X (gfx950) FlexAttention-style block-sparse attention forward.

A thin ctypes binding over ``libflexattn.so`` (C ABI in ``include/flexattn.h``).
Python only marshals arguments: every step of the BlockMask build and the
forward runs in the library's HIP kernels. PyTorch provides device memory and
the current stream. There is no CPU fallback: without the built library on a
GPU machine, every call raises.

    bm = create_block_mask("causal", B=1, H=1, Q_LEN=4096, KV_LEN=4096)
    out, lse = flex_attention(q, k, v, bm, score="softcap_alibi", softcap=50.0)
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

__all__ = [
    "BlockMask", "FlexAttnError", "MASK_KINDS", "SCORE_KINDS", "create_block_mask",
    "flex_attention", "flex_attention_backward", "block_mask_from_kv_blocks", "library_path",
    "auto_splits", "fwd_plan", "flex_attention_noalloc", "flex_attention_train",
    "load_library",
    "block_mask_sizes", "version",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libflexattn.so")

MASK_KINDS = {"noop": 0, "causal": 1, "sliding_sink": 2, "document_causal": 3, "prefix_lm": 4,
              "composite": 5}
# primitives of a composite mask's terms (and_masks inside, or_masks across terms)
MASK_PRIMS = {"causal": 1, "window": 2, "sink": 4, "prefix": 8, "document": 16}
SCORE_KINDS = {"none": 0, "alibi": 1, "softcap": 2, "softcap_alibi": 3}
_F32, _BF16, _F16 = 0, 1, 2
_OK, _INVALID, _UNSUPPORTED, _HIP = 0, 1, 2, 3


class FlexAttnError(RuntimeError):
    """A launch or runtime failure reported by the library."""


class _MaskParams(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int32), ("num_sinks", ctypes.c_int32),
                ("doc_ids", ctypes.c_void_p), ("doc_batch", ctypes.c_int32),
                ("doc_len", ctypes.c_int32), ("prefix_len", ctypes.c_int32),
                ("num_terms", ctypes.c_int32), ("terms", ctypes.c_int32 * 4)]


class _ScoreParams(ctypes.Structure):
    _fields_ = [("softcap", ctypes.c_float), ("alibi_slopes", ctypes.c_void_p)]


class _Tensor(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("dtype", ctypes.c_int),
                ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("L", ctypes.c_int32),
                ("D", ctypes.c_int32), ("stride", ctypes.c_int64 * 4)]


class _BlockMask(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Q_LEN", ctypes.c_int32),
                ("KV_LEN", ctypes.c_int32), ("BLOCK_SIZE", ctypes.c_int32),
                ("num_q_blocks", ctypes.c_int32), ("num_kv_blocks", ctypes.c_int32),
                ("kv_num_blocks", ctypes.c_void_p), ("kv_indices", ctypes.c_void_p),
                ("full_kv_num_blocks", ctypes.c_void_p), ("full_kv_indices", ctypes.c_void_p),
                ("schedule", ctypes.c_void_p), ("mask_kind", ctypes.c_int),
                ("mask_params", _MaskParams),
                ("q_num_blocks", ctypes.c_void_p), ("q_indices", ctypes.c_void_p),
                ("full_q_num_blocks", ctypes.c_void_p), ("full_q_indices", ctypes.c_void_p),
                ("Q_BLOCK_SIZE", ctypes.c_int32)]


class _FwdPlan(ctypes.Structure):
    _fields_ = [("waves_per_head", ctypes.c_int32), ("heads_per_workgroup", ctypes.c_int32),
                ("row16", ctypes.c_int32), ("num_splits", ctypes.c_int32),
                ("work_items", ctypes.c_int64)]


class _PageTable(ctypes.Structure):
    _fields_ = [("page_table", ctypes.c_void_p), ("max_pages", ctypes.c_int32)]


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load ``libflexattn.so`` (built in-tree by ``block_sparse_masked_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: build it with `python -m block_sparse_masked_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(_LIB_PATH)
    lib.flexattn_last_error.restype = ctypes.c_char_p
    lib.flexattn_version.restype = ctypes.c_char_p
    lib.flexattn_block_mask_sizes_2d.restype = ctypes.c_int
    lib.flexattn_block_mask_sizes_2d.argtypes = [ctypes.c_int32] * 6 + [
        ctypes.POINTER(ctypes.c_size_t)] * 3
    lib.flexattn_block_mask_sizes.restype = ctypes.c_int
    lib.flexattn_block_mask_sizes.argtypes = [ctypes.c_int32] * 5 + [
        ctypes.POINTER(ctypes.c_size_t)] * 3
    lib.flexattn_create_block_mask.restype = ctypes.c_int
    lib.flexattn_create_block_mask.argtypes = [
        ctypes.c_int, ctypes.POINTER(_MaskParams), ctypes.c_int32, ctypes.c_int32,
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
        ctypes.POINTER(_BlockMask), ctypes.c_void_p]
    lib.flexattn_fwd_splitkv_workspace_bytes.restype = ctypes.c_size_t
    lib.flexattn_fwd_splitkv_workspace_bytes.argtypes = [ctypes.c_int32] * 5
    lib.flexattn_fwd_splitkv.restype = ctypes.c_int
    lib.flexattn_fwd_splitkv.argtypes = [
        ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor),
        ctypes.POINTER(_BlockMask), ctypes.c_int, ctypes.POINTER(_ScoreParams), ctypes.c_float,
        ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(_Tensor),
        ctypes.c_void_p, ctypes.c_void_p]
    lib.flexattn_fwd_splitkv_noalloc.restype = ctypes.c_int
    lib.flexattn_fwd_splitkv_noalloc.argtypes = [
        ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor),
        ctypes.POINTER(_BlockMask), ctypes.c_int, ctypes.POINTER(_ScoreParams), ctypes.c_float,
        ctypes.c_int32, ctypes.POINTER(_Tensor), ctypes.c_void_p, ctypes.c_void_p]
    lib.flexattn_fwd_paged.restype = ctypes.c_int
    lib.flexattn_fwd_paged.argtypes = [
        ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor),
        ctypes.POINTER(_PageTable), ctypes.POINTER(_BlockMask), ctypes.c_int,
        ctypes.POINTER(_ScoreParams), ctypes.c_float, ctypes.c_int32, ctypes.c_void_p,
        ctypes.c_size_t, ctypes.POINTER(_Tensor), ctypes.c_void_p, ctypes.c_void_p]
    lib.flexattn_block_mask_from_kv_blocks.restype = ctypes.c_int
    lib.flexattn_block_mask_from_kv_blocks.argtypes = [ctypes.POINTER(_BlockMask), ctypes.c_void_p,
                                                       ctypes.c_void_p]
    lib.flexattn_fwd_train.restype = ctypes.c_int
    lib.flexattn_fwd_train.argtypes = [
        ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor),
        ctypes.POINTER(_BlockMask), ctypes.c_int, ctypes.POINTER(_ScoreParams), ctypes.c_float,
        ctypes.POINTER(_Tensor), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.flexattn_bwd_from_out.restype = ctypes.c_int
    lib.flexattn_bwd_from_out.argtypes = [
        ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor),
        ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(_Tensor),
        ctypes.POINTER(_BlockMask), ctypes.c_int, ctypes.POINTER(_ScoreParams), ctypes.c_float,
        ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor),
        ctypes.c_void_p, ctypes.c_void_p]
    lib.flexattn_bwd.restype = ctypes.c_int
    lib.flexattn_bwd.argtypes = [
        ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor),
        ctypes.c_void_p, ctypes.POINTER(_Tensor),
        ctypes.POINTER(_BlockMask), ctypes.c_int, ctypes.POINTER(_ScoreParams), ctypes.c_float,
        ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor),
        ctypes.c_void_p, ctypes.c_void_p]
    lib.flexattn_fwd_make_plan.restype = ctypes.c_int
    lib.flexattn_fwd_make_plan.argtypes = [ctypes.c_int32] * 5 + [
        ctypes.c_int, ctypes.POINTER(_BlockMask), ctypes.c_int32, ctypes.POINTER(_FwdPlan)]
    lib.flexattn_fwd.restype = ctypes.c_int
    lib.flexattn_fwd.argtypes = [
        ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor), ctypes.POINTER(_Tensor),
        ctypes.POINTER(_BlockMask), ctypes.c_int, ctypes.POINTER(_ScoreParams), ctypes.c_float,
        ctypes.POINTER(_Tensor), ctypes.c_void_p, ctypes.c_void_p]
    _lib = lib
    return lib


def version() -> str:
    return load_library().flexattn_version().decode()


def _check(status: int, what: str):
    if status == _OK:
        return
    msg = load_library().flexattn_last_error().decode() or what
    if status == _INVALID:
        raise ValueError(msg)
    if status == _UNSUPPORTED:
        raise NotImplementedError(msg)
    raise FlexAttnError(msg)


def _stream_handle(device: torch.device, stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


def _blocks(block):
    """(kv_block, q_block) from an int or the page's (KV_BLOCK_SIZE,
    Q_BLOCK_SIZE) tuple."""
    if isinstance(block, (tuple, list)):
        return int(block[0]), int(block[1])
    return int(block), int(block)


def block_mask_sizes(B: int, H: int, Q_LEN: int, KV_LEN: int, block=128):
    """(num_elems, idx_elems, sched_elems) of the BlockMask buffers."""
    lib = load_library()
    kb, qb = _blocks(block)
    a, b, c = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib.flexattn_block_mask_sizes_2d(B, H, Q_LEN, KV_LEN, kb, qb, ctypes.byref(a),
                                            ctypes.byref(b), ctypes.byref(c)),
           "flexattn_block_mask_sizes")
    return a.value, b.value, c.value


@dataclass
class BlockMask:
    """Device BlockMask tensors plus the C struct that points at them."""

    kind: str
    B: int
    H: int
    Q_LEN: int
    KV_LEN: int
    BLOCK_SIZE: int
    kv_num_blocks: torch.Tensor       # int32 [B, H, NQB]
    kv_indices: torch.Tensor          # int32 [B, H, NQB, NKB]
    full_kv_num_blocks: torch.Tensor  # int32 [B, H, NQB]
    full_kv_indices: torch.Tensor     # int32 [B, H, NQB, NKB]
    schedule: torch.Tensor            # int32 [B*H*NQB]
    doc_ids: Optional[torch.Tensor]
    _c: _BlockMask
    # per-KV-tile query lists for the backward (built on request)
    q_num_blocks: Optional[torch.Tensor] = None       # int32 [B, H, NKB]
    q_indices: Optional[torch.Tensor] = None          # int32 [B, H, NKB, NQB]
    full_q_num_blocks: Optional[torch.Tensor] = None  # int32 [B, H, NKB]
    full_q_indices: Optional[torch.Tensor] = None     # int32 [B, H, NKB, NQB]
    status: Optional[torch.Tensor] = None             # int32 [1]: from_kv_blocks check flags
    Q_BLOCK_SIZE: int = 0  # query rows per tile (0: BLOCK_SIZE, square tiles)

    @property
    def q_block(self) -> int:
        return self.Q_BLOCK_SIZE or self.BLOCK_SIZE

    @property
    def num_q_blocks(self) -> int:
        return self.kv_num_blocks.shape[-1]

    @property
    def num_kv_blocks(self) -> int:
        return self.kv_indices.shape[-1]

    # Inspection helpers (page "tensorplay.nn.attention API", BlockMask:
    # to_dense, to_string, sparsity). They read the lists back to the host;
    # nothing on the attention path uses them.

    def to_dense(self) -> np.ndarray:
        """Tile classes [B, H, NQB, NKB] on the host: 0 empty, 1 partial,
        2 full."""
        out = np.zeros(tuple(self.kv_indices.shape), dtype=np.int8)
        for lists, cls in (((self.kv_num_blocks, self.kv_indices), 1),
                           ((self.full_kv_num_blocks, self.full_kv_indices), 2)):
            num, idx = (t.cpu().numpy() for t in lists)
            for pos in np.ndindex(*num.shape):
                out[pos + (idx[pos][:int(num[pos])],)] = cls
        return out

    def to_string(self, grid_size=(20, 20), limit: int = 4) -> str:
        """A character picture of the tile grid of the first `limit` (b, h)
        rows of the BlockMask: '#' full, '+' partial, '.' empty. The grid is
        reduced to at most grid_size cells (rows, columns) by grouping
        tiles; a cell is '#' when all its tiles are full, '.' when all are
        empty, '+' otherwise. grid_size=-1 prints every tile."""
        dense = self.to_dense()
        B, H, nqb, nkb = dense.shape
        if grid_size == -1:
            gr, gc = nqb, nkb
        else:
            gr, gc = (grid_size, grid_size) if isinstance(grid_size, int) else grid_size
            gr, gc = min(gr, nqb), min(gc, nkb)
        rows = np.array_split(np.arange(nqb), gr)
        cols = np.array_split(np.arange(nkb), gc)
        out = [f"BlockMask(B={self.B}, H={self.H}, Q_LEN={self.Q_LEN}, KV_LEN={self.KV_LEN}, "
               f"BLOCK_SIZE={self.BLOCK_SIZE if self.q_block == self.BLOCK_SIZE else (self.BLOCK_SIZE, self.q_block)}, "
               f"kind={self.kind}, sparsity={self.sparsity():.2f}%)"]
        for n, (b, h) in enumerate(np.ndindex(B, H)):
            if n >= limit:
                out.append(f"... {B * H - limit} more (b, h)")
                break
            out.append(f"(b={b}, h={h})")
            for r in rows:
                line = ""
                for c in cols:
                    cell = dense[b, h][np.ix_(r, c)]
                    line += "#" if (cell == 2).all() else "." if (cell == 0).all() else "+"
                out.append(line)
        return "\n".join(out)

    def numel(self) -> int:
        """Dense element count of the mask (sparsity ignored)."""
        return self.B * self.H * self.Q_LEN * self.KV_LEN

    def sparsity(self) -> float:
        """Percentage of tiles that are not computed (empty), over all (b, h)
        (reads the counts back)."""
        nonempty = int(self.kv_num_blocks.sum().item()) + int(self.full_kv_num_blocks.sum().item())
        total = self.B * self.H * self.num_q_blocks * self.num_kv_blocks
        return 100.0 * (1.0 - nonempty / total)


def _mask_params(kind, window, num_sinks, prefix_len, terms) -> _MaskParams:
    mp = _MaskParams(window, num_sinks, None, 0, 0, prefix_len)
    if kind == "composite":
        if not terms or len(terms) > 4:
            raise ValueError("a composite mask needs 1 to 4 terms")
        mp.num_terms = len(terms)
        for i, term in enumerate(terms):
            bits = 0
            for name in term:
                if name not in MASK_PRIMS:
                    raise ValueError(f"unknown mask primitive {name!r} (one of {sorted(MASK_PRIMS)})")
                bits |= MASK_PRIMS[name]
            mp.terms[i] = bits
    return mp


def create_block_mask(kind: str, B: int, H: int, Q_LEN: int, KV_LEN: int, block: int = 128,
                      window: int = 0, num_sinks: int = 0,
                      doc_ids: Optional[torch.Tensor] = None,
                      device="cuda", stream=None, separate_full_blocks: bool = True,
                      backward_lists: bool = False, prefix_len: int = 0,
                      terms=None) -> BlockMask:
    """Build the BlockMask of a mask kind on the GPU (the library's builder
    kernels). B and H may be 1 to broadcast over batch / query heads.
    kind="composite" takes `terms`: up to 4 iterables of primitive names
    (MASK_PRIMS); the mask is the OR of the terms and each term the AND of
    its primitives (an empty term allows every pair), with the primitives'
    parameters window, num_sinks, prefix_len and doc_ids.
    separate_full_blocks=False lists every non-empty tile as partial, so the
    forward applies the mask on every tile. backward_lists=True also builds
    the per-KV-tile query lists (q_num_blocks, q_indices, full_q_*) that
    flex_attention_backward needs."""
    lib = load_library()
    if kind not in MASK_KINDS:
        raise NotImplementedError(f"mask kind {kind!r} is not one of {sorted(MASK_KINDS)}")
    device = torch.device(device)
    n_num, n_idx, n_sched = block_mask_sizes(B, H, Q_LEN, KV_LEN, block)
    block, q_block = _blocks(block)
    nqb = -(-Q_LEN // q_block)
    nkb = -(-KV_LEN // block)
    kv_num = torch.empty((B, H, nqb), dtype=torch.int32, device=device)
    kv_idx = torch.empty((B, H, nqb, nkb), dtype=torch.int32, device=device)
    full_num = torch.empty((B, H, nqb), dtype=torch.int32, device=device)
    full_idx = torch.empty((B, H, nqb, nkb), dtype=torch.int32, device=device)
    sched = torch.empty((n_sched,), dtype=torch.int32, device=device)
    assert kv_num.numel() == n_num and kv_idx.numel() == n_idx
    mp = _mask_params(kind, window, num_sinks, prefix_len, terms)
    if kind == "document_causal" or (kind == "composite" and any(t & 16 for t in mp.terms)):
        if doc_ids is None:
            raise ValueError(f"{kind} needs doc_ids")
        doc_ids = doc_ids.to(device=device, dtype=torch.int32)
        if doc_ids.dim() == 1:
            doc_ids = doc_ids.unsqueeze(0)
        doc_ids = doc_ids.contiguous()
        mp.doc_ids = doc_ids.data_ptr()
        mp.doc_batch = doc_ids.shape[0]
        mp.doc_len = doc_ids.shape[1]
    c = _BlockMask()
    c.Q_BLOCK_SIZE = q_block
    c.kv_num_blocks = kv_num.data_ptr()
    c.kv_indices = kv_idx.data_ptr()
    c.full_kv_num_blocks = full_num.data_ptr()
    c.full_kv_indices = full_idx.data_ptr()
    c.schedule = sched.data_ptr()
    qlists = [None] * 4
    if backward_lists:
        qlists = [torch.empty((B, H, nkb), dtype=torch.int32, device=device),
                  torch.empty((B, H, nkb, nqb), dtype=torch.int32, device=device),
                  torch.empty((B, H, nkb), dtype=torch.int32, device=device),
                  torch.empty((B, H, nkb, nqb), dtype=torch.int32, device=device)]
        c.q_num_blocks, c.q_indices, c.full_q_num_blocks, c.full_q_indices = (
            t.data_ptr() for t in qlists)
    st = lib.flexattn_create_block_mask(MASK_KINDS[kind], ctypes.byref(mp), B, H, Q_LEN, KV_LEN,
                                        block, int(bool(separate_full_blocks)), ctypes.byref(c),
                                        _stream_handle(device, stream))
    _check(st, "flexattn_create_block_mask")
    return BlockMask(kind, B, H, Q_LEN, KV_LEN, block, kv_num, kv_idx, full_num, full_idx, sched,
                     doc_ids, c, *qlists, Q_BLOCK_SIZE=q_block)


def _tensor(t: torch.Tensor, name: str) -> _Tensor:
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D [B, H, L, D]")
    if t.dtype == torch.float32:
        dt = _F32
    elif t.dtype == torch.bfloat16:
        dt = _BF16
    elif t.dtype == torch.float16:
        dt = _F16
    else:
        raise NotImplementedError(f"{name} dtype {t.dtype} is not float32, bfloat16 or float16")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    st = (ctypes.c_int64 * 4)(*t.stride())
    return _Tensor(t.data_ptr(), dt, *t.shape, st)


def fwd_plan(q: torch.Tensor, k: torch.Tensor, block_mask: BlockMask,
             target_workgroups: int = 512) -> dict:
    """The library's launch plan for a forward of these shapes
    (flexattn_fwd_make_plan): waves_per_head, heads_per_workgroup, row16,
    num_splits (slices that fill target_workgroups once when work items are
    few) and work_items."""
    lib = load_library()
    dt = {torch.float32: _F32, torch.bfloat16: _BF16, torch.float16: _F16}.get(q.dtype)
    if dt is None:
        raise NotImplementedError(f"q dtype {q.dtype} is not float32, bfloat16 or float16")
    B, Hq, M, D = q.shape
    plan = _FwdPlan()
    _check(lib.flexattn_fwd_make_plan(B, Hq, k.shape[1], M, D, dt, ctypes.byref(block_mask._c),
                                      int(target_workgroups), ctypes.byref(plan)),
           "flexattn_fwd_make_plan")
    return {name: getattr(plan, name) for name, _ in _FwdPlan._fields_}


def auto_splits(q: torch.Tensor, k: torch.Tensor, block_mask: BlockMask,
                target_workgroups: int = 512) -> int:
    """Split count for a call: enough workgroups to fill the chip once
    (target_workgroups, two per CU, the forward's occupancy) when there are
    few work items, and 1 (no split) otherwise; the library's plan decides.
    Measured on the decode shape (64 items): 8 slices (512 workgroups) beat
    16 (two rounds) and the 10 and 12 of a ragged round."""
    return fwd_plan(q, k, block_mask, target_workgroups)["num_splits"]


def flex_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_mask: BlockMask,
                   score: str = "none", softcap: float = 0.0,
                   alibi_slopes: Optional[torch.Tensor] = None, scale: Optional[float] = None,
                   out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                   stream=None, num_splits: Optional[int] = 1,
                   workspace: Optional[torch.Tensor] = None,
                   page_table: Optional[torch.Tensor] = None):
    """Block-sparse attention forward. q [B,Hq,M,D]; k, v [B,Hkv,N,D].

    With page_table (int32 [B, max_pages]; bf16 or fp16): k and v are paged caches
    [num_pages, Hkv, page_size, D] (page_size a multiple of 128) and key j of
    batch b is row j % page_size of page page_table[b, j // page_size]; the
    sequence length is block_mask.KV_LEN.

    num_splits > 1 (bf16) cuts each query tile's KV tiles into that many
    slices run by separate workgroups and merged afterwards (split-KV, for
    decode-like calls with few query tiles); None picks a count from the
    shapes. The workspace (fp32, flexattn_fwd_splitkv_workspace_bytes) is
    allocated when not given.
    Returns (out [B,Hq,M,D] in q's dtype, lse [B,Hq,M] float32)."""
    lib = load_library()
    if score not in SCORE_KINDS:
        raise NotImplementedError(f"score kind {score!r} is not one of {sorted(SCORE_KINDS)}")
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != tuple(q.shape[:3]):
        raise ValueError("lse must be a contiguous float32 tensor of shape [B, Hq, M]")
    sp = _ScoreParams(float(softcap), None)
    if alibi_slopes is not None:
        alibi_slopes = alibi_slopes.to(device=q.device, dtype=torch.float32).contiguous()
        sp.alibi_slopes = alibi_slopes.data_ptr()
    tq, tk, tv, to = _tensor(q, "q"), _tensor(k, "k"), _tensor(v, "v"), _tensor(out, "out")
    if num_splits is None:
        num_splits = auto_splits(q, k, block_mask)
    if page_table is not None:
        if page_table.dtype != torch.int32 or page_table.dim() != 2 or not page_table.is_cuda:
            raise ValueError("page_table must be a GPU int32 tensor [B, max_pages]")
        if page_table.shape[0] != q.shape[0]:
            raise ValueError("page_table must have one row per batch")
        page_table = page_table.contiguous()
        pt = _PageTable(page_table.data_ptr(), page_table.shape[1])
        B, Hq, M, D = q.shape
        need = lib.flexattn_fwd_splitkv_workspace_bytes(B, Hq, M, D, max(num_splits, 1))
        if num_splits > 1 and workspace is None:
            workspace = torch.empty((need + 3) // 4, dtype=torch.float32, device=q.device)
        ws_ptr = workspace.data_ptr() if num_splits > 1 else None
        ws_bytes = workspace.numel() * workspace.element_size() if num_splits > 1 else 0
        st = lib.flexattn_fwd_paged(
            ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), ctypes.byref(pt),
            ctypes.byref(block_mask._c), SCORE_KINDS[score], ctypes.byref(sp), float(scale),
            int(num_splits), ctypes.c_void_p(ws_ptr), ws_bytes, ctypes.byref(to),
            ctypes.c_void_p(lse.data_ptr()), _stream_handle(q.device, stream))
        _check(st, "flexattn_fwd_paged")
        return out, lse
    if num_splits > 1:
        B, Hq, M, D = q.shape
        need = lib.flexattn_fwd_splitkv_workspace_bytes(B, Hq, M, D, num_splits)
        if workspace is None:
            workspace = torch.empty((need + 3) // 4, dtype=torch.float32, device=q.device)
        st = lib.flexattn_fwd_splitkv(
            ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), ctypes.byref(block_mask._c),
            SCORE_KINDS[score], ctypes.byref(sp), float(scale), int(num_splits),
            ctypes.c_void_p(workspace.data_ptr()), workspace.numel() * workspace.element_size(),
            ctypes.byref(to), ctypes.c_void_p(lse.data_ptr()), _stream_handle(q.device, stream))
        _check(st, "flexattn_fwd_splitkv")
        return out, lse
    st = lib.flexattn_fwd(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv),
                          ctypes.byref(block_mask._c), SCORE_KINDS[score], ctypes.byref(sp),
                          float(scale), ctypes.byref(to), ctypes.c_void_p(lse.data_ptr()),
                          _stream_handle(q.device, stream))
    _check(st, "flexattn_fwd")
    return out, lse


def flex_attention_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                           block_mask: BlockMask, out: torch.Tensor, lse: torch.Tensor,
                           num_splits: int, score: str = "none", softcap: float = 0.0,
                           alibi_slopes: Optional[torch.Tensor] = None,
                           scale: Optional[float] = None, stream=None):
    """The split-KV forward with its partials in the library's own scratch
    (flexattn_fwd_splitkv_noalloc): nothing is allocated, so out, lse and (for
    ALiBi with explicit slopes) a contiguous float32 alibi_slopes on the
    device must be given. Calls that overlap on one GPU race on the scratch."""
    lib = load_library()
    if score not in SCORE_KINDS:
        raise NotImplementedError(f"score kind {score!r} is not one of {sorted(SCORE_KINDS)}")
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != tuple(q.shape[:3]):
        raise ValueError("lse must be a contiguous float32 tensor of shape [B, Hq, M]")
    sp = _ScoreParams(float(softcap), None)
    if alibi_slopes is not None:
        if (alibi_slopes.dtype != torch.float32 or not alibi_slopes.is_contiguous()
                or alibi_slopes.device != q.device):
            raise ValueError("alibi_slopes must be a contiguous float32 tensor on q's device")
        sp.alibi_slopes = alibi_slopes.data_ptr()
    tq, tk, tv, to = _tensor(q, "q"), _tensor(k, "k"), _tensor(v, "v"), _tensor(out, "out")
    st = lib.flexattn_fwd_splitkv_noalloc(
        ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv), ctypes.byref(block_mask._c),
        SCORE_KINDS[score], ctypes.byref(sp), float(scale), int(num_splits), ctypes.byref(to),
        ctypes.c_void_p(lse.data_ptr()), _stream_handle(q.device, stream))
    _check(st, "flexattn_fwd_splitkv_noalloc")
    return out, lse


def flex_attention_train(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_mask: BlockMask,
                         score: str = "none", softcap: float = 0.0,
                         alibi_slopes: Optional[torch.Tensor] = None,
                         scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                         lse: Optional[torch.Tensor] = None,
                         out_f32: Optional[torch.Tensor] = None, stream=None):
    """flex_attention (16-bit inputs, no split) that also returns O in fp32
    for flex_attention_backward(..., out_f32=...). Returns (out, lse,
    out_f32)."""
    lib = load_library()
    if score not in SCORE_KINDS:
        raise NotImplementedError(f"score kind {score!r} is not one of {sorted(SCORE_KINDS)}")
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    out = torch.empty_like(q, memory_format=torch.contiguous_format) if out is None else out
    if lse is None:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if out_f32 is None:
        out_f32 = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if (out_f32.dtype != torch.float32 or not out_f32.is_contiguous()
            or tuple(out_f32.shape) != tuple(q.shape)):
        raise ValueError("out_f32 must be a contiguous float32 tensor shaped like q")
    sp = _ScoreParams(float(softcap), None)
    if alibi_slopes is not None:
        alibi_slopes = alibi_slopes.to(device=q.device, dtype=torch.float32).contiguous()
        sp.alibi_slopes = alibi_slopes.data_ptr()
    tq, tk, tv, to = _tensor(q, "q"), _tensor(k, "k"), _tensor(v, "v"), _tensor(out, "out")
    st = lib.flexattn_fwd_train(ctypes.byref(tq), ctypes.byref(tk), ctypes.byref(tv),
                                ctypes.byref(block_mask._c), SCORE_KINDS[score], ctypes.byref(sp),
                                float(scale), ctypes.byref(to), ctypes.c_void_p(lse.data_ptr()),
                                ctypes.c_void_p(out_f32.data_ptr()),
                                _stream_handle(q.device, stream))
    _check(st, "flexattn_fwd_train")
    return out, lse, out_f32


def flex_attention_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                            lse: torch.Tensor, d_out: torch.Tensor,
                            block_mask: BlockMask, score: str = "none", softcap: float = 0.0,
                            alibi_slopes: Optional[torch.Tensor] = None,
                            scale: Optional[float] = None, dq: Optional[torch.Tensor] = None,
                            dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None, stream=None,
                            out_f32: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv) of flex_attention's output for the upstream
    gradient d_out. With out_f32 (the fp32 O of flex_attention_train) the
    row sums Delta = dO . O come from one pass over it instead of a
    recompute. bf16 or fp16 tensors (one dtype for all; the gradients come
    back in it); lse is the forward's and the BlockMask must
    carry the backward lists (create_block_mask(..., backward_lists=True)).
    dk / dv sum the query heads of each KV head."""
    lib = load_library()
    if score not in SCORE_KINDS:
        raise NotImplementedError(f"score kind {score!r} is not one of {sorted(SCORE_KINDS)}")
    if block_mask.q_num_blocks is None:
        raise ValueError("the BlockMask has no backward lists: build it with backward_lists=True")
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != tuple(q.shape[:3]):
        raise ValueError("lse must be a contiguous float32 tensor of shape [B, Hq, M]")
    dq = torch.empty_like(q, memory_format=torch.contiguous_format) if dq is None else dq
    dk = torch.empty_like(k, memory_format=torch.contiguous_format) if dk is None else dk
    dv = torch.empty_like(v, memory_format=torch.contiguous_format) if dv is None else dv
    if workspace is None:
        workspace = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    if workspace.dtype != torch.float32 or workspace.numel() < q.shape[0] * q.shape[1] * q.shape[2]:
        raise ValueError("workspace must be float32 with at least B * Hq * M elements")
    sp = _ScoreParams(float(softcap), None)
    if alibi_slopes is not None:
        alibi_slopes = alibi_slopes.to(device=q.device, dtype=torch.float32).contiguous()
        sp.alibi_slopes = alibi_slopes.data_ptr()
    t = {n: _tensor(x, n) for n, x in (("q", q), ("k", k), ("v", v), ("d_out", d_out),
                                       ("dq", dq), ("dk", dk), ("dv", dv))}
    tail = (ctypes.byref(t["d_out"]), ctypes.byref(block_mask._c), SCORE_KINDS[score],
            ctypes.byref(sp), float(scale), ctypes.byref(t["dq"]), ctypes.byref(t["dk"]),
            ctypes.byref(t["dv"]), ctypes.c_void_p(workspace.data_ptr()),
            _stream_handle(q.device, stream))
    if out_f32 is not None:
        if (out_f32.dtype != torch.float32 or not out_f32.is_contiguous()
                or tuple(out_f32.shape) != tuple(q.shape)):
            raise ValueError("out_f32 must be the contiguous float32 O of flex_attention_train")
        st = lib.flexattn_bwd_from_out(ctypes.byref(t["q"]), ctypes.byref(t["k"]),
                                       ctypes.byref(t["v"]), ctypes.c_void_p(lse.data_ptr()),
                                       ctypes.c_void_p(out_f32.data_ptr()), *tail)
        _check(st, "flexattn_bwd_from_out")
        return dq, dk, dv
    st = lib.flexattn_bwd(ctypes.byref(t["q"]), ctypes.byref(t["k"]), ctypes.byref(t["v"]),
                          ctypes.c_void_p(lse.data_ptr()), *tail)
    _check(st, "flexattn_bwd")
    return dq, dk, dv


FROM_KV_BLOCKS_FLAGS = {1: "a count outside [0, NKB]", 2: "an index outside [0, NKB)",
                        4: "a list that is not strictly ascending",
                        8: "a tile in both the partial and the full list of a row",
                        16: "a full tile that crosses Q_LEN or KV_LEN"}


def block_mask_from_kv_blocks(kv_num_blocks: torch.Tensor, kv_indices: torch.Tensor,
                              full_kv_num_blocks: Optional[torch.Tensor] = None,
                              full_kv_indices: Optional[torch.Tensor] = None,
                              Q_LEN: Optional[int] = None, KV_LEN: Optional[int] = None,
                              kind: str = "noop", window: int = 0, num_sinks: int = 0,
                              doc_ids: Optional[torch.Tensor] = None,
                              backward_lists: bool = False, validate: bool = True,
                              stream=None, prefix_len: int = 0, terms=None) -> BlockMask:
    """A BlockMask from caller-given tile lists (BlockMask.from_kv_blocks):
    kv_num_blocks [B, H, NQB] and kv_indices [B, H, NQB, NKB] list the
    partial tiles (evaluated with the mask `kind`; "noop" makes them dense),
    the optional full_* lists the tiles computed without the mask. The GPU
    computes the schedule (and the backward lists) and checks the lists;
    with validate=True the check is read back (a synchronisation) and bad
    lists raise RuntimeError."""
    lib = load_library()
    if kind not in MASK_KINDS:
        raise NotImplementedError(f"mask kind {kind!r} is not one of {sorted(MASK_KINDS)}")
    if kv_num_blocks.dim() != 3 or kv_indices.dim() != 4:
        raise RuntimeError("kv_num_blocks must be [B, H, NQB] and kv_indices [B, H, NQB, NKB]")
    device = kv_indices.device
    B, H, nqb, nkb = kv_indices.shape
    if tuple(kv_num_blocks.shape) != (B, H, nqb):
        raise RuntimeError("kv_num_blocks and kv_indices disagree on [B, H, NQB]")
    Q_LEN = nqb * 128 if Q_LEN is None else Q_LEN
    KV_LEN = nkb * 128 if KV_LEN is None else KV_LEN
    as_i32 = lambda t: t.to(device=device, dtype=torch.int32).contiguous()  # noqa: E731
    kv_num, kv_idx = as_i32(kv_num_blocks), as_i32(kv_indices)
    if full_kv_num_blocks is None:
        full_num = torch.zeros_like(kv_num)
        full_idx = torch.zeros_like(kv_idx)
    else:
        full_num, full_idx = as_i32(full_kv_num_blocks), as_i32(full_kv_indices)
        if full_num.shape != kv_num.shape or full_idx.shape != kv_idx.shape:
            raise RuntimeError("full_* lists must have the shapes of the partial lists")
    sched = torch.empty((B * H * nqb,), dtype=torch.int32, device=device)
    status = torch.empty((1,), dtype=torch.int32, device=device)
    c = _BlockMask()
    c.B, c.H, c.Q_LEN, c.KV_LEN, c.BLOCK_SIZE = B, H, Q_LEN, KV_LEN, 128
    c.num_q_blocks, c.num_kv_blocks = -(-Q_LEN // 128), -(-KV_LEN // 128)
    c.kv_num_blocks, c.kv_indices = kv_num.data_ptr(), kv_idx.data_ptr()
    c.full_kv_num_blocks, c.full_kv_indices = full_num.data_ptr(), full_idx.data_ptr()
    c.schedule = sched.data_ptr()
    c.mask_kind = MASK_KINDS[kind]
    mp = _mask_params(kind, window, num_sinks, prefix_len, terms)
    if kind == "document_causal" or (kind == "composite" and any(t & 16 for t in mp.terms)):
        if doc_ids is None:
            raise ValueError(f"{kind} needs doc_ids")
        doc_ids = doc_ids.to(device=device, dtype=torch.int32)
        doc_ids = (doc_ids.unsqueeze(0) if doc_ids.dim() == 1 else doc_ids).contiguous()
        mp.doc_ids, mp.doc_batch, mp.doc_len = doc_ids.data_ptr(), doc_ids.shape[0], doc_ids.shape[1]
    c.mask_params = mp
    qlists = [None] * 4
    if backward_lists:
        qlists = [torch.empty((B, H, nkb), dtype=torch.int32, device=device),
                  torch.empty((B, H, nkb, nqb), dtype=torch.int32, device=device),
                  torch.empty((B, H, nkb), dtype=torch.int32, device=device),
                  torch.empty((B, H, nkb, nqb), dtype=torch.int32, device=device)]
        c.q_num_blocks, c.q_indices, c.full_q_num_blocks, c.full_q_indices = (
            t.data_ptr() for t in qlists)
    st = lib.flexattn_block_mask_from_kv_blocks(ctypes.byref(c), ctypes.c_void_p(status.data_ptr()),
                                                _stream_handle(device, stream))
    _check(st, "flexattn_block_mask_from_kv_blocks")
    bm = BlockMask(kind, B, H, Q_LEN, KV_LEN, 128, kv_num, kv_idx, full_num, full_idx, sched,
                   doc_ids, c, *qlists, status=status)
    if validate:
        flags = int(status.item())
        if flags:
            reasons = [text for bit, text in FROM_KV_BLOCKS_FLAGS.items() if flags & bit]
            raise RuntimeError("invalid kv block lists: " + "; ".join(reasons))
    return bm
