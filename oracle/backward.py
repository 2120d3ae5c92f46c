"""Plain fp64 CPU oracle for the backward of the block-sparse attention.

TEST INFRASTRUCTURE ONLY (like ``oracle/reference.py``): imported by the test
suite and the bench's CPU-baseline leg, never by the GPU product path.

What it follows on the pages:

* The backward needs, per KV tile, the query tiles that attend to it, listed
  apart for partial and full tiles and derived from the forward's lists:
  page "tensorplay.nn.attention API", section BlockMask ("Details", items 3
  and 4: q_num_blocks / q_indices and full_q_num_blocks / full_q_indices).
  ``transpose_block_mask`` builds them from the per-tile classes.
* The gradients themselves are the plain chain rule through the forward's
  definition (score = scale * q.k, then score_mod, then the mask, softmax,
  P.V), written out with the whole score matrix of a row chunk, as in
  ``reference.attention``. For an upstream gradient dO:

    dV_j  = sum_i P_ij dO_i
    dP_ij = dO_i . v_j
    dS'_ij = P_ij (dP_ij - sum_l P_il dP_il)        (softmax backward)
    dS_ij = dS'_ij * d score_mod / d s               (1 - tanh^2(s/c) for the
                                                      soft-cap, 1 for ALiBi)
    dQ_i  = scale * sum_j dS_ij k_j
    dK_j  = scale * sum_i dS_ij q_i

  Masked entries have P = 0 and so contribute nothing; a row with no allowed
  key has zero gradient. Query heads of one GQA group add their dK and dV
  into the shared KV head.
"""
from __future__ import annotations

from typing import Callable, Optional, Sequence

import numpy as np

from .reference import BlockMask, MaskMod, ScoreMod, noop_mask

# d score_mod(s) / d s at the scaled score s (elementwise)
ScoreGrad = Callable[[np.ndarray, int, int, np.ndarray, np.ndarray], np.ndarray]


def softcap_grad(cap: float) -> ScoreGrad:
    """Derivative of cap * tanh(s / cap): 1 - tanh(s / cap)^2. An added ALiBi
    bias does not depend on s, so the soft-capped kinds share it."""
    cap = float(cap)

    def grad(score, b, h, q_idx, kv_idx):
        t = np.tanh(score / cap)
        return 1.0 - t * t
    return grad


def score_grad_for(kind: str, softcap: float = 0.0) -> Optional[ScoreGrad]:
    """d score_mod / d s for a score kind name (None: the identity's 1)."""
    if kind in ("none", "alibi"):
        return None
    if kind in ("softcap", "softcap_alibi"):
        return softcap_grad(softcap)
    raise ValueError(f"unknown score kind {kind!r}")


def attention_backward(q: np.ndarray, k: np.ndarray, v: np.ndarray, d_out: np.ndarray,
                       mask_mod: Optional[MaskMod] = None,
                       score_mod: Optional[ScoreMod] = None,
                       score_grad: Optional[ScoreGrad] = None,
                       scale: Optional[float] = None,
                       batches: Optional[Sequence[int]] = None,
                       heads: Optional[Sequence[int]] = None,
                       rows: Optional[Sequence[int]] = None,
                       row_chunk: int = 1024):
    """dQ [B, Hq, M, D], dK [B, Hkv, N, D], dV [B, Hkv, N, Dv] in fp64.

    Only the selected batches / query heads / query rows contribute (dQ rows
    not selected stay NaN; dK / dV collect only the selected rows, so they
    are the full gradients only when every row of a head is selected)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    d_out = np.asarray(d_out, dtype=np.float64)
    B, Hq, M, D = q.shape
    _, Hkv, N, _ = k.shape
    if d_out.shape != (B, Hq, M, v.shape[-1]):
        raise ValueError("d_out must have the shape of the output")
    group = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    mask_mod = noop_mask if mask_mod is None else mask_mod
    dq = np.full(q.shape, np.nan)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    batches = range(B) if batches is None else batches
    heads = range(Hq) if heads is None else heads
    rows = np.arange(M, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    kv_idx = np.arange(N, dtype=np.int64)[None, :]
    for b in batches:
        for h in heads:
            hk = h // group
            for c in range(0, len(rows), row_chunk):
                r = rows[c:c + row_chunk]
                q_idx = r[:, None]
                s = scale * (q[b, h, r] @ k[b, hk].T)
                s_mod = score_mod(s, b, h, q_idx, kv_idx) if score_mod is not None else s
                allowed = np.broadcast_to(mask_mod(b, h, q_idx, kv_idx), s.shape)
                s_mod = np.where(allowed, s_mod, -np.inf)
                m = s_mod.max(axis=1)
                live = np.isfinite(m)
                e = np.exp(s_mod - np.where(live, m, 0.0)[:, None])
                p = np.where(live[:, None], e / np.where(live, e.sum(axis=1), 1.0)[:, None], 0.0)
                dv[b, hk] += p.T @ d_out[b, h, r]
                dp = d_out[b, h, r] @ v[b, hk].T
                ds = p * (dp - (p * dp).sum(axis=1)[:, None])
                if score_grad is not None:
                    ds = ds * np.where(allowed, score_grad(s, b, h, q_idx, kv_idx), 0.0)
                dq[b, h, r] = scale * (ds @ k[b, hk])
                dk[b, hk] += scale * (ds.T @ q[b, h, r])
    return dq, dk, dv


def transpose_block_mask(bm: BlockMask):
    """Per KV tile, the ascending query tiles whose tile is partial
    (q_num_blocks [B, H, NKB], q_indices [B, H, NKB, NQB]) and full
    (full_q_num_blocks, full_q_indices), from the tile classes the forward
    lists encode; unused tails are 0."""
    B, H, nqb = bm.kv_num_blocks.shape
    nkb = bm.kv_indices.shape[-1]
    part = np.zeros((B, H, nqb, nkb), dtype=np.int32)
    full = np.zeros((B, H, nqb, nkb), dtype=np.int32)
    for b in range(B):
        for h in range(H):
            for i in range(nqb):
                for t in range(int(bm.kv_num_blocks[b, h, i])):
                    part[b, h, i, int(bm.kv_indices[b, h, i, t])] = 1
                for t in range(int(bm.full_kv_num_blocks[b, h, i])):
                    full[b, h, i, int(bm.full_kv_indices[b, h, i, t])] = 1
    out = []
    for grid in (part, full):
        num = np.zeros((B, H, nkb), dtype=np.int32)
        idx = np.zeros((B, H, nkb, nqb), dtype=np.int32)
        for b in range(B):
            for h in range(H):
                for j in range(nkb):
                    rows = np.nonzero(grid[b, h, :, j])[0]
                    num[b, h, j] = len(rows)
                    idx[b, h, j, :len(rows)] = rows
        out += [num, idx]
    return tuple(out)  # q_num, q_idx, full_q_num, full_q_idx
