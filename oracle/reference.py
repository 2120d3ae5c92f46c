"""Plain fp64 CPU oracle for FlexAttention-style block-sparse attention.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package's smoke check and
the bench's CPU-baseline leg may import this module. The GPU product path never
calls it and shares no code with it.

It is written to be checked by eye against the pages, not to be fast:

* mask_mod semantics (``(b, h, q_idx, kv_idx) -> bool``, True = may attend),
  ``create_mask`` (a dense ``(B, H, M, N)`` mask), ``create_block_mask`` and the
  combinators ``and_masks`` / ``or_masks`` / ``noop_mask``: page
  "tensorplay.nn.attention API", sections create_block_mask, create_mask,
  and_masks, or_masks, noop_mask.
* The BlockMask format (a tile is skipped only when every element in it is
  masked; fully unmasked tiles are listed apart so mask_mod can be skipped on
  them; per query row-tile a count plus a list of KV tile positions; the dense
  reconstruction loop; ``numel``; ``sparsity``): same page, section BlockMask
  ("Basics", "Details", numel, sparsity, to_dense).
* score_mod changes a score before the softmax: page "attention-gym: examples,
  masks and kernels for FlexAttention", section "A gallery that grew into a
  toolkit".
* ALiBi adds the per-head linear distance penalty m_h * (j - i); sink tokens
  plus a sliding window (StreamingLLM): page "transformerlab", section
  "Attention variants".
* Block-diagonal attention over packed variable-length sequences and tanh
  soft-capping as variants needing custom kernels: page "Attention Backends"
  (L-GATr), section "Why care about Attention Kernels?".
* Query heads map to KV heads in contiguous groups (GQA/MQA, K/V stored before
  the head broadcast): page "FlagAttention", section "Operator overview"
  (layout ``q [B,Hq,M,D]``, ``k/v [B,Hkv,N,D]``), and page "transformerlab",
  sections "Adding a new attention variant" and "Decode / KV cache".

Readings taken where the pages are silent:
the score passed to score_mod already carries the ``scale`` factor; softcap is
``c * tanh(s / c)`` applied before the ALiBi bias; a query row with no allowed
key yields O = 0 and LSE = -inf; LSE is the natural-log log-sum-exp; KV tile
indices are ascending with the unused tail filled with 0; out-of-range
elements of a tail tile count as masked, so a tail tile is never full.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Optional, Sequence

import numpy as np

MaskMod = Callable[[int, int, np.ndarray, np.ndarray], np.ndarray]
ScoreMod = Callable[[np.ndarray, int, int, np.ndarray, np.ndarray], np.ndarray]


# --------------------------------------------------------------------------
# mask_mods (page "tensorplay.nn.attention API": create_block_mask's mask_mod
# parameter; noop_mask; and_masks; or_masks)
# --------------------------------------------------------------------------

def noop_mask(b, h, q_idx, kv_idx):
    """Every (q, kv) pair may attend."""
    return np.ones(np.broadcast_shapes(np.shape(q_idx), np.shape(kv_idx)), dtype=bool)


def causal_mask(b, h, q_idx, kv_idx):
    """The page's causal example: a query attends to keys at or before it."""
    return q_idx >= kv_idx


def and_masks(*mods: MaskMod) -> MaskMod:
    """Intersection of mask_mods."""
    def mod(b, h, q_idx, kv_idx):
        out = noop_mask(b, h, q_idx, kv_idx)
        for m in mods:
            out = out & m(b, h, q_idx, kv_idx)
        return out
    return mod


def or_masks(*mods: MaskMod) -> MaskMod:
    """Union of mask_mods."""
    def mod(b, h, q_idx, kv_idx):
        out = ~noop_mask(b, h, q_idx, kv_idx)
        for m in mods:
            out = out | m(b, h, q_idx, kv_idx)
        return out
    return mod


def window_mask(window: int) -> MaskMod:
    """Keys fewer than ``window`` positions behind the query (page
    "transformerlab": ``local`` / ``local_flex`` sliding window)."""
    def mod(b, h, q_idx, kv_idx):
        return (q_idx - kv_idx) < window
    return mod


def sink_mask(num_sinks: int) -> MaskMod:
    """The first ``num_sinks`` keys (page "transformerlab": ``sink``,
    StreamingLLM first-k sink tokens)."""
    def mod(b, h, q_idx, kv_idx):
        return kv_idx < num_sinks
    return mod


def sliding_sink_mask(window: int, num_sinks: int) -> MaskMod:
    """Causal AND (inside the window OR a sink token)."""
    return and_masks(causal_mask, or_masks(window_mask(window), sink_mask(num_sinks)))


def prefix_lm_mask(prefix_len: int) -> MaskMod:
    """PrefixLM (named on page "Attention Backends", section "Why care about
    Attention Kernels?"): every query sees the first prefix_len keys, and
    causally after them: or_masks(kv_idx < prefix_len, causal_mask)."""
    prefix_len = int(prefix_len)

    def in_prefix(b, h, q_idx, kv_idx):
        return kv_idx < prefix_len
    return or_masks(in_prefix, causal_mask)


def prefix_mask(prefix_len: int) -> MaskMod:
    """The first ``prefix_len`` keys, whatever the query."""
    prefix_len = int(prefix_len)

    def mod(b, h, q_idx, kv_idx):
        return kv_idx < prefix_len
    return mod


def document_mask(doc_ids: np.ndarray) -> MaskMod:
    """Pairs whose positions carry the same document id (``doc_ids`` ``[L]``
    or ``[B, L]``, indexed by q_idx and kv_idx), in either direction."""
    doc = np.asarray(doc_ids)

    def mod(b, h, q_idx, kv_idx):
        d = doc if doc.ndim == 1 else doc[b]
        return d[q_idx] == d[kv_idx]
    return mod


def composite_mask(terms, window: int = 0, num_sinks: int = 0, prefix_len: int = 0,
                   doc_ids=None) -> MaskMod:
    """Runtime composition (page "tensorplay.nn.attention API": or_masks is
    the union and and_masks the intersection of mask_mods): or_masks over the
    terms of and_masks over each term's primitives, named "causal",
    "window", "sink", "prefix", "document"; an empty term is noop_mask."""
    prims = {"causal": lambda: causal_mask, "window": lambda: window_mask(window),
             "sink": lambda: sink_mask(num_sinks), "prefix": lambda: prefix_mask(prefix_len),
             "document": lambda: document_mask(doc_ids)}
    return or_masks(*[and_masks(*[prims[name]() for name in term]) for term in terms])


def document_causal_mask(doc_ids: np.ndarray) -> MaskMod:
    """Block-diagonal causal mask over packed documents.

    ``doc_ids`` is ``[L]`` (shared by every batch entry) or ``[B, L]``; both
    q_idx and kv_idx index it. A pair may attend when both positions carry the
    same document id and the key is not after the query (page "Attention
    Backends": block-diagonal mask over concatenated events, here made causal).
    """
    doc = np.asarray(doc_ids)

    def mod(b, h, q_idx, kv_idx):
        d = doc if doc.ndim == 1 else doc[b]
        return (d[q_idx] == d[kv_idx]) & (q_idx >= kv_idx)
    return mod


# --------------------------------------------------------------------------
# score_mods (page "attention-gym ...": a score mod changes the score before
# the softmax; page "transformerlab": ALiBi m_h * (j - i); page "Attention
# Backends": tanh soft-capping)
# --------------------------------------------------------------------------

def alibi_slopes(num_heads: int) -> np.ndarray:
    """Geometric per-head slopes 2^(-8 (h + 1) / H), h = query head."""
    h = np.arange(num_heads, dtype=np.float64)
    return np.power(2.0, -8.0 * (h + 1.0) / num_heads)


def alibi_score(slopes: Sequence[float]) -> ScoreMod:
    """score + m_h * (kv_idx - q_idx)."""
    slopes = np.asarray(slopes, dtype=np.float64)

    def mod(score, b, h, q_idx, kv_idx):
        return score + slopes[h] * (kv_idx - q_idx).astype(np.float64)
    return mod


def softcap_score(cap: float) -> ScoreMod:
    """cap * tanh(score / cap)."""
    cap = float(cap)

    def mod(score, b, h, q_idx, kv_idx):
        return cap * np.tanh(score / cap)
    return mod


def softcap_alibi_score(cap: float, slopes: Sequence[float]) -> ScoreMod:
    """Soft-cap first, then add the ALiBi bias."""
    cap_mod = softcap_score(cap)
    bias_mod = alibi_score(slopes)

    def mod(score, b, h, q_idx, kv_idx):
        return bias_mod(cap_mod(score, b, h, q_idx, kv_idx), b, h, q_idx, kv_idx)
    return mod


# --------------------------------------------------------------------------
# create_mask / create_block_mask / to_dense / sparsity / numel
# (page "tensorplay.nn.attention API")
# --------------------------------------------------------------------------

def create_mask(mask_mod: MaskMod, B: int, H: int, Q_LEN: int, KV_LEN: int) -> np.ndarray:
    """Dense boolean mask of shape (B, H, Q_LEN, KV_LEN), one mask_mod call
    per (b, h) over the whole index grid."""
    q_idx = np.arange(Q_LEN, dtype=np.int64)[:, None]
    kv_idx = np.arange(KV_LEN, dtype=np.int64)[None, :]
    out = np.empty((B, H, Q_LEN, KV_LEN), dtype=bool)
    for b in range(B):
        for h in range(H):
            out[b, h] = np.broadcast_to(mask_mod(b, h, q_idx, kv_idx), (Q_LEN, KV_LEN))
    return out


@dataclass
class BlockMask:
    """The BlockMask tensors for one (mask_mod, B, H, Q_LEN, KV_LEN, block).

    kv_num_blocks / full_kv_num_blocks: int32 [B, H, NQB]
    kv_indices / full_kv_indices:       int32 [B, H, NQB, NKB]
    ``kv_*`` lists the partial tiles, ``full_kv_*`` the full tiles; the two
    are disjoint; lists are ascending and padded with 0.
    """

    Q_LEN: int
    KV_LEN: int
    BLOCK_SIZE: int
    kv_num_blocks: np.ndarray
    kv_indices: np.ndarray
    full_kv_num_blocks: np.ndarray
    full_kv_indices: np.ndarray
    tile_counts: np.ndarray  # int64 [B, H, NQB, NKB]: allowed in-range elements per tile

    @property
    def shape(self):
        return self.kv_num_blocks.shape

    def numel(self) -> int:
        """Element count of the dense mask, sparsity ignored."""
        B, H, _ = self.kv_num_blocks.shape
        return B * H * self.Q_LEN * self.KV_LEN

    def to_dense(self) -> np.ndarray:
        """Dense tile grid [B, H, NQB, NKB]: 1 where a tile is computed."""
        nkb = self.kv_indices.shape[-1]
        part = to_dense(self.kv_num_blocks, self.kv_indices, nkb)
        full = to_dense(self.full_kv_num_blocks, self.full_kv_indices, nkb)
        return np.maximum(part, full)

    def sparsity(self) -> float:
        """Percentage of tiles that are not computed."""
        dense = self.to_dense()
        return 100.0 * (1.0 - dense.sum() / dense.size)


def classify_tiles(counts: np.ndarray, q_len: int, kv_len: int, block):
    """Tile classes from per-tile allowed counts: 0 empty, 1 partial, 2 full.

    `block` is an int or (kv_block, q_block). A tile is full only when all of
    its q_block x kv_block elements exist and are allowed; a tail tile has
    fewer in-range elements, so it is never full."""
    kblk, qblk = (block, block) if np.isscalar(block) else block
    cls = np.where(counts == 0, 0, np.where(counts == kblk * qblk, 2, 1))
    return cls.astype(np.int8)


def create_block_mask(mask_mod: MaskMod, B: int, H: int, Q_LEN: int, KV_LEN: int,
                      BLOCK_SIZE: int = 128, separate_full_blocks: bool = True) -> BlockMask:
    """Reduce the element mask to tiles and list them. BLOCK_SIZE is one
    int (square tiles) or the page's tuple (KV_BLOCK_SIZE, Q_BLOCK_SIZE).

    For each (b, h, q-tile) the element mask rows of that tile are evaluated
    over every key, allowed elements are counted per KV tile, and the tile is
    empty (count 0), full (count block^2) or partial. With
    separate_full_blocks=True partial tiles go to ``kv_*`` and full tiles to
    ``full_kv_*``, each as a count plus an ascending index list; with False
    every non-empty tile is listed in ``kv_*`` and ``full_kv_*`` is empty
    (page "tensorplay.nn.attention API", create_block_mask parameters).
    """
    kblk, qblk = (BLOCK_SIZE, BLOCK_SIZE) if np.isscalar(BLOCK_SIZE) else BLOCK_SIZE
    kblk, qblk = int(kblk), int(qblk)
    nqb = -(-Q_LEN // qblk)
    nkb = -(-KV_LEN // kblk)
    counts = np.zeros((B, H, nqb, nkb), dtype=np.int64)
    kv_idx = np.arange(KV_LEN, dtype=np.int64)[None, :]
    for b in range(B):
        for h in range(H):
            for i in range(nqb):
                q_idx = np.arange(i * qblk, min((i + 1) * qblk, Q_LEN), dtype=np.int64)[:, None]
                rows = np.broadcast_to(mask_mod(b, h, q_idx, kv_idx), (q_idx.shape[0], KV_LEN))
                per_col = rows.sum(axis=0, dtype=np.int64)
                padded = np.zeros(nkb * kblk, dtype=np.int64)
                padded[:KV_LEN] = per_col
                counts[b, h, i] = padded.reshape(nkb, kblk).sum(axis=1)
    cls = classify_tiles(counts, Q_LEN, KV_LEN, (kblk, qblk))
    if not separate_full_blocks:
        cls = np.where(cls == 0, 0, 1).astype(np.int8)
    kv_num = np.zeros((B, H, nqb), dtype=np.int32)
    kv_ind = np.zeros((B, H, nqb, nkb), dtype=np.int32)
    full_num = np.zeros((B, H, nqb), dtype=np.int32)
    full_ind = np.zeros((B, H, nqb, nkb), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(nqb):
                part = np.nonzero(cls[b, h, i] == 1)[0]
                full = np.nonzero(cls[b, h, i] == 2)[0]
                kv_num[b, h, i] = len(part)
                kv_ind[b, h, i, :len(part)] = part
                full_num[b, h, i] = len(full)
                full_ind[b, h, i, :len(full)] = full
    blk = kblk if kblk == qblk else (kblk, qblk)
    return BlockMask(Q_LEN, KV_LEN, blk, kv_num, kv_ind, full_num, full_ind, counts)


def from_kv_blocks_mask(kv_num_blocks: np.ndarray, kv_indices: np.ndarray,
                        full_kv_num_blocks: Optional[np.ndarray] = None,
                        full_kv_indices: Optional[np.ndarray] = None, BLOCK_SIZE: int = 128,
                        mask_mod: Optional[MaskMod] = None) -> MaskMod:
    """The element mask that tile lists given directly stand for (page
    "tensorplay.nn.attention API", BlockMask.from_kv_blocks, with "Details"
    items 1 and 2): an element is computed only inside a listed tile; inside
    a partial tile where mask_mod allows it, inside a full tile always.
    Lists with extent 1 over batch or heads broadcast."""
    mask_mod = noop_mask if mask_mod is None else mask_mod
    blk = int(BLOCK_SIZE)
    B, H, nqb, nkb = kv_indices.shape
    cls = np.zeros((B, H, nqb, nkb), dtype=np.int8)
    for pos in np.ndindex(B, H, nqb):
        for t in range(int(kv_num_blocks[pos])):
            cls[pos + (int(kv_indices[pos + (t,)]),)] = 1
        if full_kv_num_blocks is not None:
            for t in range(int(full_kv_num_blocks[pos])):
                cls[pos + (int(full_kv_indices[pos + (t,)]),)] = 2

    def mod(b, h, q_idx, kv_idx):
        c = cls[b if B > 1 else 0, h if H > 1 else 0][np.asarray(q_idx) // blk,
                                                       np.asarray(kv_idx) // blk]
        return np.where(c == 2, True, np.where(c == 1, mask_mod(b, h, q_idx, kv_idx), False))
    return mod


def to_dense(num_blocks: np.ndarray, indices: np.ndarray, num_cols: int) -> np.ndarray:
    """The page's reconstruction loop: mark (row, indices[row, i]) for
    i < num_blocks[row]; leading dims are batch dims."""
    lead = num_blocks.shape
    out = np.zeros(lead + (num_cols,), dtype=np.int32)
    for pos in np.ndindex(*lead):
        for i in range(int(num_blocks[pos])):
            out[pos + (int(indices[pos + (i,)]),)] = 1
    return out


# --------------------------------------------------------------------------
# Attention (the plain definition: full score matrix, mods per element,
# standard softmax; rows are independent, so they may be taken in chunks)
# --------------------------------------------------------------------------

def gather_paged(cache: np.ndarray, page_table: np.ndarray, kv_len: int) -> np.ndarray:
    """Keys (or values) of each sequence from a paged KV cache: row j of
    batch b is row j mod P of cache page page_table[b, j div P], P the page
    size (page "FlagAttention", operator overview: a KV cache kept in pages).
    cache [num_pages, H, P, D] -> [B, H, kv_len, D]."""
    P = cache.shape[2]
    j = np.arange(kv_len)
    pages = np.asarray(page_table)[:, j // P]                    # [B, kv_len]
    out = cache[pages, :, (j % P)[None, :], :]                   # [B, kv_len, H, D]
    return np.ascontiguousarray(np.swapaxes(out, 1, 2))


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
              mask_mod: Optional[MaskMod] = None,
              score_mod: Optional[ScoreMod] = None,
              scale: Optional[float] = None,
              batches: Optional[Sequence[int]] = None,
              heads: Optional[Sequence[int]] = None,
              rows: Optional[Sequence[int]] = None,
              row_chunk: int = 1024):
    """O and LSE of masked, score-modified softmax attention in fp64.

    q: [B, Hq, M, D]; k, v: [B, Hkv, N, D] (Dv may differ from D); Hq is a
    multiple of Hkv and query head h reads KV head h // (Hq // Hkv).
    Returns O [B, Hq, M, Dv] and LSE [B, Hq, M] (float64). Only the selected
    batches / heads / rows are computed; the others stay NaN.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, M, D = q.shape
    Bk, Hkv, N, Dk = k.shape
    if Bk != B or Dk != D or v.shape[:3] != (B, Hkv, N):
        raise ValueError("q/k/v shapes do not match")
    if Hq % Hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    mask_mod = noop_mask if mask_mod is None else mask_mod
    out = np.full((B, Hq, M, v.shape[-1]), np.nan)
    lse = np.full((B, Hq, M), np.nan)
    batches = range(B) if batches is None else batches
    heads = range(Hq) if heads is None else heads
    rows = np.arange(M) if rows is None else np.asarray(rows, dtype=np.int64)
    kv_idx = np.arange(N, dtype=np.int64)[None, :]
    for b in batches:
        for h in heads:
            hk = h // group
            for c in range(0, len(rows), row_chunk):
                r = rows[c:c + row_chunk]
                q_idx = r[:, None]
                s = scale * (q[b, h, r] @ k[b, hk].T)
                if score_mod is not None:
                    s = score_mod(s, b, h, q_idx, kv_idx)
                allowed = np.broadcast_to(mask_mod(b, h, q_idx, kv_idx), s.shape)
                s = np.where(allowed, s, -np.inf)
                m = s.max(axis=1)
                live = np.isfinite(m)
                m_safe = np.where(live, m, 0.0)
                e = np.exp(s - m_safe[:, None])
                denom = e.sum(axis=1)
                with np.errstate(divide="ignore"):
                    row_lse = np.where(live, m_safe + np.log(denom), -np.inf)
                p = np.where(live[:, None], e / np.where(live, denom, 1.0)[:, None], 0.0)
                out[b, h, r] = p @ v[b, hk]
                lse[b, h, r] = row_lse
    return out, lse


def unmasked_pairs(bm: BlockMask) -> int:
    """Allowed (q, kv) pairs summed over the BlockMask's (b, h)."""
    return int(bm.tile_counts.sum())
