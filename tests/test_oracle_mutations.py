"""Plant plausible mistakes in a copy of the oracle and show the pins fail.

Each case edits the oracle's source text, executes the edited copy as a
separate module (on the CPU), and runs one of the pin checks against it. The
real oracle is untouched.
"""
import inspect
import itertools
import math
import sys
import types

import numpy as np
import pytest

import oracle
import workloads as W
from oracle import reference
from tests import pins

SOURCE = inspect.getsource(reference)
_COUNTER = itertools.count()


def mutated(old: str, new: str):
    assert SOURCE.count(old) >= 1, f"mutation anchor not found: {old!r}"
    name = f"oracle_mutant_{next(_COUNTER)}"
    mod = types.ModuleType(name)
    sys.modules[name] = mod  # dataclasses look the module up while executing it
    try:
        exec(compile(SOURCE.replace(old, new), name, "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    return mod


def _qkv(B, Hq, Hkv, M, N, D, seed):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, Hq, M, D)), r.standard_normal((B, Hkv, N, D)),
            r.standard_normal((B, Hkv, N, D)))


def sdpa_pin_error(ref_mod, kind="causal", score=False):
    """Max |O - SDPA| for a GQA case (Hq=4, Hkv=2, M != N)."""
    B, Hq, Hkv, M, N, D = 1, 4, 2, 21, 27, 8
    q, k, v = _qkv(B, Hq, Hkv, M, N, D, seed=99)
    mask = {"causal": ref_mod.causal_mask, "noop": ref_mod.noop_mask}[kind]
    allowed = oracle.create_mask(oracle.causal_mask if kind == "causal" else oracle.noop_mask,
                                 B, Hq, M, N)
    bias = None
    smod = None
    if score:
        slopes = np.array([0.5, 0.25, 0.125, 0.0625])
        smod = ref_mod.alibi_score(slopes)
        i = np.arange(M)[:, None]
        j = np.arange(N)[None, :]
        bias = np.broadcast_to(slopes[None, :, None, None] * (j - i)[None, None], (B, Hq, M, N))
    o, _ = ref_mod.attention(q, k, v, mask, smod, 0.45)
    ref = pins.sdpa_reference(q, k, v, allowed, 0.45, bias=bias)
    live = allowed.any(-1)
    return float(np.max(np.abs(o[live] - ref[live])))


def lse_pin_error(ref_mod):
    """Max |LSE - (s_ij - log P_ij)| with P from the library softmax."""
    q, k, _ = _qkv(1, 1, 1, 12, 12, 8, seed=5)
    v = np.eye(12)[None, None]
    allowed = oracle.create_mask(oracle.causal_mask, 1, 1, 12, 12)
    P = pins.sdpa_reference(q, k, v, allowed, 0.5)
    _, lse = ref_mod.attention(q, k, v, ref_mod.causal_mask, None, 0.5)
    err = 0.0
    for i in range(12):
        j = int(np.argmax(P[0, 0, i]))
        s = 0.5 * float(q[0, 0, i] @ k[0, 0, j])
        err = max(err, abs(lse[0, 0, i] - (s - math.log(P[0, 0, i, j]))))
    return err


def loop_pin_error(ref_mod):
    """Max error vs the scalar-loop formulation with softcap then ALiBi."""
    q, k, v = _qkv(1, 2, 1, 7, 9, 4, seed=6)
    q, k = 4 * q, 4 * k
    cap = 3.0
    slopes = [0.5, 0.25]

    def score_fn(s, b, h, i, j):
        return cap * math.tanh(s / cap) + slopes[h] * (j - i)

    o, lse = ref_mod.attention(q, k, v, ref_mod.causal_mask,
                               ref_mod.softcap_alibi_score(cap, slopes), 0.6)
    o2, lse2 = pins.loop_attention(q, k, v, lambda b, h, i, j: j <= i, score_fn, 0.6)
    return max(float(np.max(np.abs(o - o2))), float(np.max(np.abs(lse - lse2))))


def brute_force_pin_ok(ref_mod, kind="causal"):
    """Brute-force tile classes at shapes chosen so that each class boundary
    is exercised: a one-column tail tile (KV_LEN = 49, block 16), a tile with
    a single masked element, and a window edge (31) that ends exactly at a
    tile's far corner."""
    if kind == "causal":
        cases = [(ref_mod.causal_mask, lambda b, h, q, kv: kv <= q, 70, 49)]
        hole = lambda b, h, q, kv: ~((q == 5) & (kv == 7))  # noqa: E731
        cases.append((hole, lambda b, h, q, kv: not (q == 5 and kv == 7), 40, 40))
    else:
        cases = [(ref_mod.sliding_sink_mask(31, 2),
                  lambda b, h, q, kv: kv <= q and (q - kv < 31 or kv < 2), 70, 53)]
    ok = True
    for mod, scalar, M, N in cases:
        bm = ref_mod.create_block_mask(mod, 1, 1, M, N, 16)
        cls = pins.brute_force_tiles(scalar, 1, 1, M, N, 16)
        ok = ok and pins.block_mask_matches(bm, pins.lists_from_classes(cls))
    return ok


def test_unmutated_oracle_passes_every_pin():
    assert sdpa_pin_error(reference) < 1e-12
    assert sdpa_pin_error(reference, score=True) < 1e-12
    assert lse_pin_error(reference) < 1e-12
    assert loop_pin_error(reference) < 1e-12
    assert brute_force_pin_ok(reference, "causal")
    assert brute_force_pin_ok(reference, "sliding")


@pytest.mark.parametrize("old,new,check", [
    # GQA: wrong head mapping (modulo instead of contiguous groups)
    ("hk = h // group", "hk = h % Hkv", "sdpa"),
    # dropped scale factor
    ("s = scale * (q[b, h, r] @ k[b, hk].T)", "s = (q[b, h, r] @ k[b, hk].T)", "sdpa"),
    # wrong V row index (rows reversed)
    ("out[b, h, r] = p @ v[b, hk]", "out[b, h, r] = p @ v[b, hk][::-1]", "sdpa"),
    # causal off by one
    ("return q_idx >= kv_idx", "return q_idx > kv_idx", "sdpa"),
    # ALiBi sign flipped
    ("slopes[h] * (kv_idx - q_idx)", "slopes[h] * (q_idx - kv_idx)", "sdpa_alibi"),
    # ALiBi slope indexed by the KV-head-like modulo
    ("return score + slopes[h] *", "return score + slopes[h % 2] *", "sdpa_alibi"),
    # LSE missing the running max
    ("m_safe + np.log(denom)", "np.log(denom)", "lse"),
    # softcap and ALiBi in the other order
    ("return bias_mod(cap_mod(score, b, h, q_idx, kv_idx), b, h, q_idx, kv_idx)",
     "return cap_mod(bias_mod(score, b, h, q_idx, kv_idx), b, h, q_idx, kv_idx)", "loop"),
    # tanh softcap without the outer factor
    ("return cap * np.tanh(score / cap)", "return np.tanh(score / cap)", "loop"),
    # full-tile threshold off by one element
    ("counts == kblk * qblk", "counts >= kblk * qblk - 1", "brute_causal"),
    # tail tiles dropped from the count
    ("padded[:KV_LEN] = per_col", "padded[:KV_LEN - 1] = per_col[:-1]", "brute_causal"),
    # sink term lost
    ("return kv_idx < num_sinks", "return kv_idx < 0", "brute_sliding"),
    # window edge off by one
    ("return (q_idx - kv_idx) < window", "return (q_idx - kv_idx) <= window", "brute_sliding"),
])
def test_planted_mistake_is_caught(old, new, check):
    m = mutated(old, new)
    if check == "sdpa":
        assert sdpa_pin_error(m) > 1e-6
    elif check == "sdpa_alibi":
        assert sdpa_pin_error(m, score=True) > 1e-6
    elif check == "lse":
        assert lse_pin_error(m) > 1e-6
    elif check == "loop":
        assert loop_pin_error(m) > 1e-6
    elif check == "brute_causal":
        assert not brute_force_pin_ok(m, "causal")
    elif check == "brute_sliding":
        assert not brute_force_pin_ok(m, "sliding")
    else:
        raise AssertionError(check)


def test_document_mutation_caught_by_closed_form():
    """Document mask that forgets causality changes the full-length tiles."""
    m = mutated("return (d[q_idx] == d[kv_idx]) & (q_idx >= kv_idx)",
                "return (d[q_idx] == d[kv_idx])")
    doc = W.document_ids([30, 2, 50])
    bm = m.create_block_mask(m.document_causal_mask(doc), 1, 1, 82, 82, 16)
    scalar = lambda b, h, q, kv: doc[q] == doc[kv] and kv <= q  # noqa: E731
    cls = pins.brute_force_tiles(scalar, 1, 1, 82, 82, 16)
    assert not pins.block_mask_matches(bm, pins.lists_from_classes(cls))
