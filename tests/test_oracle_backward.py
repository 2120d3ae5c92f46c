"""Pins of the fp64 backward oracle (CPU only).

The gradients are pinned by central finite differences of the forward
oracle's output (itself pinned against SDPA, brute force and closed forms in
test_oracle_pins.py), by invariants that follow from the softmax, and by
mutations that each pin must catch. The transposed tile lists are pinned by a
per-element brute force of the tile classes.
"""
import inspect
import itertools
import sys
import types

import numpy as np
import pytest

import oracle
import workloads as W
from oracle import backward as bwd_module
from tests import pins

SCALAR_MASKS = {
    "noop": lambda doc: (lambda b, h, q, kv: True),
    "causal": lambda doc: (lambda b, h, q, kv: kv <= q),
    "sliding_sink": lambda doc: (lambda b, h, q, kv: kv <= q and (q - kv < 3 or kv < 1)),
    "document_causal": lambda doc: (lambda b, h, q, kv: doc[q] == doc[kv] and kv <= q),
}
DOC = W.document_ids([2, 1, 4, 3, 6])  # 16 ids


def _mods(mask, score, Hq):
    mask_mod = oracle.mask_mod_for(mask, window=3, sinks=1, doc_ids=DOC)
    score_mod = oracle.score_mod_for(score, Hq, softcap=1.5)
    grad = oracle.score_grad_for(score, softcap=1.5)
    return mask_mod, score_mod, grad


def _inputs(B, Hq, Hkv, M, N, D, seed):
    r = np.random.default_rng(seed)
    q = r.standard_normal((B, Hq, M, D))
    k = r.standard_normal((B, Hkv, N, D))
    v = r.standard_normal((B, Hkv, N, D))
    do = r.standard_normal((B, Hq, M, D))
    return q, k, v, do


def _loss(q, k, v, do, mask_mod, score_mod, scale):
    o, _ = oracle.attention(q, k, v, mask_mod, score_mod, scale)
    return float(np.nansum(o * do))


def _finite_difference(x, f, eps=1e-6):
    g = np.zeros_like(x)
    for idx in np.ndindex(*x.shape):
        old = x[idx]
        x[idx] = old + eps
        up = f()
        x[idx] = old - eps
        dn = f()
        x[idx] = old
        g[idx] = (up - dn) / (2 * eps)
    return g


@pytest.mark.parametrize("mask", list(SCALAR_MASKS))
@pytest.mark.parametrize("score", ["none", "alibi", "softcap", "softcap_alibi"])
def test_gradients_match_finite_differences(mask, score):
    """dQ, dK, dV equal central differences of sum(O * dO) (GQA: 2 query
    heads per KV head; M != N so the index roles cannot be swapped)."""
    B, Hq, Hkv, M, N, D = 1, 2, 1, 7, 9, 3
    q, k, v, do = _inputs(B, Hq, Hkv, M, N, D, seed=5)
    mask_mod, score_mod, grad = _mods(mask, score, Hq)
    scale = 0.7
    dq, dk, dv = oracle.attention_backward(q, k, v, do, mask_mod, score_mod, grad, scale)
    f = lambda: _loss(q, k, v, do, mask_mod, score_mod, scale)  # noqa: E731
    for name, x, g in (("dq", q, dq), ("dk", k, dk), ("dv", v, dv)):
        fd = _finite_difference(x, f)
        assert np.allclose(np.nan_to_num(g), fd, rtol=1e-5, atol=1e-7), (name, np.abs(g - fd).max())


def test_empty_rows_have_zero_gradient():
    """Rows with no allowed key (sliding window, no sinks, query beyond the
    keys) give dQ = 0 and add nothing to dK / dV."""
    B, Hq, Hkv, M, N, D = 1, 1, 1, 6, 3, 4
    q, k, v, do = _inputs(B, Hq, Hkv, M, N, D, seed=8)
    mask_mod = oracle.sliding_sink_mask(2, 0)  # q >= 5 sees no key < 3
    dq, dk, dv = oracle.attention_backward(q, k, v, do, mask_mod, None, None, 0.5)
    assert np.all(dq[0, 0, 5] == 0.0)
    do2 = do.copy()
    do2[0, 0, 5] = 100.0
    _, dk2, dv2 = oracle.attention_backward(q, k, v, do2, mask_mod, None, None, 0.5)
    assert np.array_equal(dk, dk2) and np.array_equal(dv, dv2)


def test_value_shift_leaves_dq_dk_and_dv():
    """Each row's probabilities sum to 1, so adding one vector to every value
    row changes O by that vector and leaves all three gradients alone."""
    q, k, v, do = _inputs(1, 2, 2, 8, 8, 4, seed=11)
    mask_mod = oracle.causal_mask
    a = oracle.attention_backward(q, k, v, do, mask_mod, None, None, 0.6)
    b = oracle.attention_backward(q, k, v + np.array([1.0, -2.0, 0.5, 3.0]), do, mask_mod,
                                  None, None, 0.6)
    for x, y in zip(a, b):
        assert np.allclose(x, y, rtol=1e-12, atol=1e-12)


def test_single_key_rows_have_zero_dq():
    """A row that sees one key has P = 1 there whatever q is, so dQ = 0 and
    dV of that key is dO (causal row 0)."""
    q, k, v, do = _inputs(1, 1, 1, 4, 4, 3, seed=2)
    dq, _, dv = oracle.attention_backward(q, k, v, do, oracle.causal_mask, None, None, 0.9)
    assert np.allclose(dq[0, 0, 0], 0.0, atol=1e-15)
    # key 3 is seen only by row 3 (with weight P_33)
    _, lse = oracle.attention(q, k, v, oracle.causal_mask, None, 0.9)
    p33 = np.exp(0.9 * q[0, 0, 3] @ k[0, 0, 3] - lse[0, 0, 3])
    assert np.allclose(dv[0, 0, 3], p33 * do[0, 0, 3], rtol=1e-12)


def test_gqa_gradients_sum_over_the_group():
    """GQA dK / dV equal the per-head gradients of the repeated-KV (MHA)
    problem summed over each group."""
    q, k, v, do = _inputs(1, 4, 2, 6, 5, 3, seed=4)
    g = oracle.attention_backward(q, k, v, do, oracle.causal_mask, None, None, 0.8)
    k_rep = np.repeat(k, 2, axis=1)
    v_rep = np.repeat(v, 2, axis=1)
    m = oracle.attention_backward(q, k_rep, v_rep, do, oracle.causal_mask, None, None, 0.8)
    assert np.allclose(g[0], m[0], rtol=1e-12)
    assert np.allclose(g[1], m[1].reshape(1, 2, 2, 5, 3).sum(axis=2), rtol=1e-12)
    assert np.allclose(g[2], m[2].reshape(1, 2, 2, 5, 3).sum(axis=2), rtol=1e-12)


# ---------------------------------------------------------- transposed lists

@pytest.mark.parametrize("kind", list(SCALAR_MASKS))
@pytest.mark.parametrize("q_len,kv_len", [(16, 16), (17, 33), (40, 23)])
def test_transposed_lists_brute_force(kind, q_len, kv_len):
    """q_* / full_q_* list, per KV tile, the query tiles of each class in
    ascending order (block 8 so tiny shapes span several tiles)."""
    blk = 8
    doc = W.document_ids([5, 1, 20, 13, 61])
    scalar = SCALAR_MASKS[kind](doc)
    mask_mod = oracle.mask_mod_for(kind, window=3, sinks=1, doc_ids=doc)
    bm = oracle.create_block_mask(mask_mod, 1, 1, q_len, kv_len, blk)
    cls = pins.brute_force_tiles(scalar, 1, 1, q_len, kv_len, blk)
    qn, qi, fqn, fqi = oracle.transpose_block_mask(bm)
    # the transposed class grid through the same list builder
    expected = pins.lists_from_classes(np.swapaxes(cls, 2, 3))
    for got, exp in zip((qn, qi, fqn, fqi), expected):
        assert np.array_equal(got, exp)


# ---------------------------------------------------------------- mutations

SOURCE = inspect.getsource(bwd_module)
_COUNTER = itertools.count()


def _mutant(old, new):
    assert SOURCE.count(old) >= 1, old
    name = f"oracle_bwd_mutant_{next(_COUNTER)}"
    mod = types.ModuleType(name)
    mod.__package__ = "oracle"
    sys.modules[name] = mod
    try:
        exec(compile(SOURCE.replace(old, new), name, "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    return mod


@pytest.mark.parametrize("old,new", [
    ("ds = p * (dp - (p * dp).sum(axis=1)[:, None])", "ds = p * dp"),
    ("ds = p * (dp - (p * dp).sum(axis=1)[:, None])", "ds = p * (dp + (p * dp).sum(axis=1)[:, None])"),
    ("dq[b, h, r] = scale * (ds @ k[b, hk])", "dq[b, h, r] = ds @ k[b, hk]"),
    ("dk[b, hk] += scale * (ds.T @ q[b, h, r])", "dk[b, hk] = scale * (ds.T @ q[b, h, r])"),
    ("dv[b, hk] += p.T @ d_out[b, h, r]", "dv[b, hk] += p @ d_out[b, h, r][:p.shape[1]]"),
    ("return 1.0 - t * t", "return 1.0 + t * t"),
    ("hk = h // group", "hk = h % Hkv"),
])
def test_mutations_fail_the_finite_difference_pin(old, new):
    mod = _mutant(old, new)
    B, Hq, Hkv, M, N, D = 1, 4, 2, 7, 7, 3
    q, k, v, do = _inputs(B, Hq, Hkv, M, N, D, seed=5)
    mask_mod, score_mod, _ = _mods("causal", "softcap_alibi", Hq)
    grad = mod.softcap_grad(1.5)
    try:
        dq, dk, dv = mod.attention_backward(q, k, v, do, mask_mod, score_mod, grad, 0.7)
    except (ValueError, IndexError):
        return  # the mutant cannot even run
    f = lambda: _loss(q, k, v, do, mask_mod, score_mod, 0.7)  # noqa: E731
    ok = all(np.allclose(np.nan_to_num(g), _finite_difference(x, f), rtol=1e-5, atol=1e-7)
             for x, g in ((q, dq), (k, dk), (v, dv)))
    assert not ok
