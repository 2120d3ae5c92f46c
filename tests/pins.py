"""Pins for the oracle: checks against things other than the oracle itself.

Each check takes the oracle function under test as an argument, so the
mutation tests can run the same check on a copy of the oracle with a planted
mistake and show that the check catches it.
"""
from __future__ import annotations

import math

import numpy as np
import torch


# ---------------------------------------------------------------- BlockMask

def brute_force_tiles(allowed, B, H, Q_LEN, KV_LEN, blk, q_blk=None):
    """Per-element pure-Python loop: class of every tile (0 empty, 1 partial,
    2 full) straight from the definitions (a tile is skipped only if every
    element is masked; full means every one of its blk*blk elements exists and
    is allowed)."""
    qb_ = blk if q_blk is None else q_blk  # query rows per tile (blk: keys)
    nqb = -(-Q_LEN // qb_)
    nkb = -(-KV_LEN // blk)
    cls = np.zeros((B, H, nqb, nkb), dtype=np.int8)
    for b in range(B):
        for h in range(H):
            for i in range(nqb):
                for j in range(nkb):
                    n_allowed = 0
                    for q in range(i * qb_, min((i + 1) * qb_, Q_LEN)):
                        for kv in range(j * blk, min((j + 1) * blk, KV_LEN)):
                            if allowed(b, h, q, kv):
                                n_allowed += 1
                    if n_allowed == 0:
                        cls[b, h, i, j] = 0
                    elif n_allowed == blk * qb_:
                        cls[b, h, i, j] = 2
                    else:
                        cls[b, h, i, j] = 1
    return cls


def lists_from_classes(cls):
    """Expected (kv_num, kv_ind, full_num, full_ind) from a class grid:
    ascending lists, tail 0 (the reading of the 'undefined' tail)."""
    B, H, nqb, nkb = cls.shape
    out = [np.zeros((B, H, nqb), np.int32), np.zeros((B, H, nqb, nkb), np.int32),
           np.zeros((B, H, nqb), np.int32), np.zeros((B, H, nqb, nkb), np.int32)]
    for b in range(B):
        for h in range(H):
            for i in range(nqb):
                p = [j for j in range(nkb) if cls[b, h, i, j] == 1]
                f = [j for j in range(nkb) if cls[b, h, i, j] == 2]
                out[0][b, h, i] = len(p)
                out[1][b, h, i, :len(p)] = p
                out[2][b, h, i] = len(f)
                out[3][b, h, i, :len(f)] = f
    return out


def block_mask_matches(bm, expected_lists) -> bool:
    got = [bm.kv_num_blocks, bm.kv_indices, bm.full_kv_num_blocks, bm.full_kv_indices]
    return all(np.array_equal(g, e) for g, e in zip(got, expected_lists))


def causal_closed_form(nb):
    """Causal at Q_LEN = KV_LEN = nb*blk: row i has partial {i}, full {0..i-1}."""
    kv_num = np.ones(nb, np.int32)
    kv_ind = np.zeros((nb, nb), np.int32)
    kv_ind[:, 0] = np.arange(nb)
    full_num = np.arange(nb, dtype=np.int32)
    full_ind = np.zeros((nb, nb), np.int32)
    for i in range(nb):
        full_ind[i, :i] = np.arange(i)
    return kv_num, kv_ind, full_num, full_ind


def sliding_sink_closed_form(nb, window_blocks):
    """Sliding window of window_blocks*blk keys plus 1..blk sink tokens,
    causal, Q_LEN = KV_LEN = nb*blk (derived from the definition):
    j > i empty; j = i partial (diagonal); i-w < j < i full (the whole tile is
    within the window); j = i-w partial (the window edge crosses it); j < i-w
    only the sinks: tile 0 partial, other tiles empty."""
    w = window_blocks
    part = [[] for _ in range(nb)]
    full = [[] for _ in range(nb)]
    for i in range(nb):
        for j in range(nb):
            if j > i:
                continue
            if j == i or j == i - w:
                part[i].append(j)
            elif j > i - w:
                full[i].append(j)
            elif j == 0:
                part[i].append(j)
    kv_num = np.array([len(p) for p in part], np.int32)
    full_num = np.array([len(f) for f in full], np.int32)
    kv_ind = np.zeros((nb, nb), np.int32)
    full_ind = np.zeros((nb, nb), np.int32)
    for i in range(nb):
        kv_ind[i, :len(part[i])] = part[i]
        full_ind[i, :len(full[i])] = full[i]
    return kv_num, kv_ind, full_num, full_ind


# ---------------------------------------------------------------- attention

def sdpa_reference(q, k, v, allowed, scale, bias=None):
    """torch.nn.functional.scaled_dot_product_attention on the CPU in fp64.

    allowed: bool [B, Hq, M, N] (True = may attend); bias: optional float
    additive [B, Hq, M, N]; GQA by repeating each KV head over its group."""
    qt = torch.from_numpy(np.asarray(q, np.float64))
    kt = torch.from_numpy(np.asarray(k, np.float64))
    vt = torch.from_numpy(np.asarray(v, np.float64))
    g = qt.shape[1] // kt.shape[1]
    kt = kt.repeat_interleave(g, dim=1).contiguous()
    vt = vt.repeat_interleave(g, dim=1).contiguous()
    if bias is None:
        mask = torch.from_numpy(np.asarray(allowed, bool))
    else:
        mask = torch.from_numpy(np.where(allowed, np.asarray(bias, np.float64), -np.inf))
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o.numpy()


def loop_attention(q, k, v, allowed_fn, score_fn, scale):
    """Second, independent formulation with scalar Python loops and the math
    module (no NumPy vectorisation): for each row, scores, mods, masked
    softmax, weighted sum of V rows. Tiny shapes only."""
    B, Hq, M, D = q.shape
    _, Hkv, N, Dv = v.shape
    g = Hq // Hkv
    O = np.zeros((B, Hq, M, Dv))
    L = np.zeros((B, Hq, M))
    for b in range(B):
        for h in range(Hq):
            hk = h // g
            for i in range(M):
                scores = []
                for j in range(N):
                    if not allowed_fn(b, h, i, j):
                        continue
                    s = 0.0
                    for d in range(D):
                        s += float(q[b, h, i, d]) * float(k[b, hk, j, d])
                    s *= scale
                    if score_fn is not None:
                        s = score_fn(s, b, h, i, j)
                    scores.append((j, s))
                if not scores:
                    L[b, h, i] = -math.inf
                    continue
                mx = max(s for _, s in scores)
                tot = math.fsum(math.exp(s - mx) for _, s in scores)
                L[b, h, i] = mx + math.log(tot)
                for j, s in scores:
                    w = math.exp(s - mx) / tot
                    for d in range(Dv):
                        O[b, h, i, d] += w * float(v[b, hk, j, d])
    return O, L
