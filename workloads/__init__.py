"""Seeded synthetic inputs for the block-sparse attention workloads.

This module only *generates inputs*: shapes, seeded normal draws, rounding of
those draws to bfloat16, and the packed document layout of the varlen case.
It holds none of the attention arithmetic. Both the fp64 oracle (through the
tests and the bench) and the GPU path consume what it returns, so that the two
sides see bit-identical inputs.

Workload recipe (the pages publish no dataset for this path, so every input is
synthetic):

* q, k, v are drawn in that order with ``numpy.random.default_rng(seed)`` as
  float32 standard normals of shape ``[B, H, L, D]`` (``H`` = query heads for
  q, KV heads for k and v), multiplied by ``value_scale`` (2 for the softcap
  case, 1 otherwise).
* bf16 workloads round each float32 draw to the nearest bfloat16, ties to
  even, and f16 workloads to the nearest IEEE half (NumPy's conversion, ties
  to even); the rounded values (held exactly in float32) are what both
  sides use.
* The document (packed varlen) workload draws document lengths uniformly in
  ``[lo, hi]`` until the remainder fits in one document, and lays the documents
  out as contiguous runs of ids, the packed layout the L-GATr "Attention
  Backends" page describes for block-diagonal attention over events of
  different lengths.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple

import numpy as np

MASK_KINDS = ("noop", "causal", "sliding_sink", "document_causal", "prefix_lm", "composite")
SCORE_KINDS = ("none", "alibi", "softcap", "softcap_alibi")


@dataclass(frozen=True)
class Workload:
    """One attention workload: shapes, dtype, seeds, mask and score kinds."""

    name: str
    B: int
    Hq: int
    Hkv: int
    Q_LEN: int
    KV_LEN: int
    D: int
    dtype: str  # "f32", "bf16" or "f16"
    seed: int
    mask: str = "causal"
    window: int = 0
    sinks: int = 0
    doc_seed: Optional[int] = None
    doc_len_range: Tuple[int, int] = (128, 4096)
    score: str = "none"
    softcap: float = 0.0
    value_scale: float = 1.0
    block: int = 128
    prefix: int = 0  # prefix_lm: keys [0, prefix) visible to every query
    terms: Optional[tuple] = None  # composite: tuples of primitive names
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def scale(self) -> float:
        # 1/sqrt(D) unless a test sets extra["scale"].
        return float(self.extra.get("scale", 1.0 / np.sqrt(self.D)))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads the hot path is measured and checked on. Seeds 1-5 for
# q/k/v; seed 1004 for the document lengths.
TINY_CAUSAL = Workload("tiny_causal_f32", B=1, Hq=2, Hkv=2, Q_LEN=256, KV_LEN=256,
                       D=64, dtype="f32", seed=1, mask="causal")
DENSE_CAUSAL_GQA = Workload("dense_causal_gqa_bf16", B=4, Hq=16, Hkv=4, Q_LEN=4096,
                            KV_LEN=4096, D=128, dtype="bf16", seed=2, mask="causal")
SLIDING_SINKS = Workload("sliding_window_sinks_bf16", B=2, Hq=32, Hkv=8, Q_LEN=8192,
                         KV_LEN=8192, D=128, dtype="bf16", seed=3, mask="sliding_sink",
                         window=1024, sinks=4)
DOCUMENT = Workload("document_causal_bf16", B=1, Hq=16, Hkv=16, Q_LEN=16384,
                    KV_LEN=16384, D=64, dtype="bf16", seed=4, mask="document_causal",
                    doc_seed=1004, doc_len_range=(128, 4096))
ALIBI_SOFTCAP = Workload("alibi_softcap_bf16", B=2, Hq=16, Hkv=16, Q_LEN=8192,
                         KV_LEN=8192, D=128, dtype="bf16", seed=5, mask="causal",
                         score="softcap_alibi", softcap=50.0, value_scale=2.0)
# Decode-shaped calls (few queries, long KV): not a headline configuration;
# measured on the HBM roofline with the split-KV path.
DECODE_GQA = Workload("decode_gqa_bf16", B=8, Hq=32, Hkv=8, Q_LEN=16, KV_LEN=32768, D=128,
                      dtype="bf16", seed=6, mask="noop")

WORKLOADS = (TINY_CAUSAL, DENSE_CAUSAL_GQA, SLIDING_SINKS, DOCUMENT, ALIBI_SOFTCAP)
BY_NAME = {w.name: w for w in WORKLOADS}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even).

    Returns float32 values that are exactly representable in bfloat16.
    Inputs here are finite normals, so NaN handling is not needed.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are exact bfloat16 values."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    if np.any(u & 0xFFFF):
        raise ValueError("values are not exactly representable in bfloat16")
    return (u >> 16).astype(np.uint16)


def document_lengths(total: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Seeded document lengths in ``[lo, hi]`` that sum to ``total``.

    While more than ``hi`` tokens remain, draw a length uniformly from
    ``[lo, min(hi, remaining - lo)]`` (so the remainder never drops below
    ``lo``); the last document takes the remainder.
    """
    if total < lo:
        raise ValueError("total shorter than the minimum document length")
    rng = np.random.default_rng(seed)
    lens = []
    rem = total
    while rem > hi:
        x = int(rng.integers(lo, min(hi, rem - lo) + 1))
        lens.append(x)
        rem -= x
    lens.append(rem)
    return np.asarray(lens, dtype=np.int64)


def document_ids(lengths) -> np.ndarray:
    """int32 document id per position: contiguous runs 0, 0, ..., 1, 1, ..."""
    lengths = np.asarray(lengths, dtype=np.int64)
    return np.repeat(np.arange(len(lengths), dtype=np.int32), lengths)


@dataclass
class Inputs:
    """Generated inputs: float32 arrays (bf16-exact for bf16 workloads)."""

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    doc_ids: Optional[np.ndarray]
    doc_lengths: Optional[np.ndarray]


def generate(w: Workload) -> Inputs:
    """Draw q, k, v (and document ids) for a workload."""
    rng = np.random.default_rng(w.seed)
    q = rng.standard_normal((w.B, w.Hq, w.Q_LEN, w.D), dtype=np.float32)
    k = rng.standard_normal((w.B, w.Hkv, w.KV_LEN, w.D), dtype=np.float32)
    v = rng.standard_normal((w.B, w.Hkv, w.KV_LEN, w.D), dtype=np.float32)
    if w.value_scale != 1.0:
        s = np.float32(w.value_scale)
        q, k, v = q * s, k * s, v * s
    if w.dtype == "bf16":
        q, k, v = round_to_bf16(q), round_to_bf16(k), round_to_bf16(v)
    elif w.dtype == "f16":
        q, k, v = (x.astype(np.float16).astype(np.float32) for x in (q, k, v))
    elif w.dtype != "f32":
        raise ValueError(f"unknown dtype {w.dtype!r}")
    doc_ids = doc_lengths = None
    if w.mask == "document_causal" or (w.mask == "composite"
                                       and any("document" in t for t in w.terms)):
        L = max(w.Q_LEN, w.KV_LEN)
        if w.doc_seed is None:
            raise ValueError("document workload needs doc_seed")
        lo, hi = w.doc_len_range
        doc_lengths = document_lengths(L, lo, hi, w.doc_seed)
        doc_ids = document_ids(doc_lengths)
    return Inputs(q, k, v, doc_ids, doc_lengths)


def generate_upstream(w: Workload) -> np.ndarray:
    """Upstream gradient dO for the backward: standard normal, shaped like
    the output [B, Hq, Q_LEN, D], from its own stream (seed + 7919) so the
    forward's inputs do not change; rounded to the workload's 16-bit type
    (bf16 or IEEE half) as its inputs are."""
    rng = np.random.default_rng(w.seed + 7919)
    g = rng.standard_normal((w.B, w.Hq, w.Q_LEN, w.D), dtype=np.float32)
    if w.dtype == "bf16":
        return round_to_bf16(g)
    if w.dtype == "f16":
        return g.astype(np.float16).astype(np.float32)
    return g


def paged_cache(k: np.ndarray, v: np.ndarray, page_size: int, seed: int, spare_pages: int = 3,
                extra_columns: int = 1):
    """Lay k and v [B, H, N, D] out in a paged KV cache: pages of page_size
    key rows per head, placed at a seeded random permutation of the cache's
    pages, with `spare_pages` pages no sequence uses.

    Returns (k_cache, v_cache [P, H, page_size, D], page_table int32
    [B, ceil(N / page_size) + extra_columns]). Cache rows that hold no key
    (spare pages, the rows past N in a sequence's last page) are NaN, and
    the page table's extra columns hold an index past the cache, so a read
    of anything outside the sequence shows up in the output."""
    B, H, N, D = k.shape
    per_seq = -(-N // page_size)
    P = B * per_seq + spare_pages
    rng = np.random.default_rng(seed)
    order = rng.permutation(P)[:B * per_seq].reshape(B, per_seq)
    k_cache = np.full((P, H, page_size, D), np.nan, dtype=k.dtype)
    v_cache = np.full((P, H, page_size, D), np.nan, dtype=v.dtype)
    for b in range(B):
        for j in range(per_seq):
            rows = min(page_size, N - j * page_size)
            k_cache[order[b, j], :, :rows] = k[b, :, j * page_size:j * page_size + rows]
            v_cache[order[b, j], :, :rows] = v[b, :, j * page_size:j * page_size + rows]
    table = np.full((B, per_seq + extra_columns), P + 1000, dtype=np.int32)
    table[:, :per_seq] = order
    return k_cache, v_cache, table


def small(w: Workload, **kw) -> Workload:
    """A reduced copy of a workload (same kinds and dtype), for quick checks."""
    return w.with_(**kw)
