"""Pins of the fp64 oracle against the pages and the mathematics (CPU only)."""
import math
import os

import numpy as np
import pytest

import oracle
import workloads as W
from tests import pins

RNG = np.random.default_rng(12345)


def _qkv(B, Hq, Hkv, M, N, D, Dv=None, scale=1.0, seed=0):
    r = np.random.default_rng(seed)
    Dv = D if Dv is None else Dv
    q = r.standard_normal((B, Hq, M, D)) * scale
    k = r.standard_normal((B, Hkv, N, D)) * scale
    v = r.standard_normal((B, Hkv, N, Dv))
    return q, k, v


# ------------------------------------------------------------ BlockMask pins

SCALAR_MASKS = {
    "noop": lambda doc: (lambda b, h, q, kv: True),
    "causal": lambda doc: (lambda b, h, q, kv: kv <= q),
    "sliding_sink": lambda doc: (lambda b, h, q, kv: kv <= q and (q - kv < 40 or kv < 3)),
    "document_causal": lambda doc: (lambda b, h, q, kv: doc[q] == doc[kv] and kv <= q),
    "prefix_lm": lambda doc: (lambda b, h, q, kv: kv <= q or kv < 10),
}


def _oracle_mask(kind, doc):
    return oracle.mask_mod_for(kind, window=40, sinks=3, doc_ids=doc, prefix=10)


@pytest.mark.parametrize("kind", list(SCALAR_MASKS))
@pytest.mark.parametrize("q_len,kv_len", [(1, 1), (15, 16), (16, 16), (17, 33), (64, 64),
                                          (77, 50), (50, 77), (100, 100)])
def test_block_mask_brute_force(kind, q_len, kv_len):
    """Tile classes and lists equal a per-element Python loop (block 16, so
    tiny shapes span many tiles and ragged tails)."""
    blk = 16
    L = max(q_len, kv_len)
    doc = W.document_ids([5, 1, 20, 13, 61])[:L] if L <= 100 else None
    scalar = SCALAR_MASKS[kind](doc)
    bm = oracle.create_block_mask(_oracle_mask(kind, doc), 1, 1, q_len, kv_len, blk)
    cls = pins.brute_force_tiles(scalar, 1, 1, q_len, kv_len, blk)
    assert pins.block_mask_matches(bm, pins.lists_from_classes(cls))


@pytest.mark.parametrize("kind", list(SCALAR_MASKS))
@pytest.mark.parametrize("q_len,kv_len", [(16, 16), (17, 33), (77, 50), (100, 100)])
def test_block_mask_unseparated_brute_force(kind, q_len, kv_len):
    """separate_full_blocks=False (page "tensorplay.nn.attention API",
    create_block_mask parameters): every non-empty tile of the per-element
    loop is listed as partial, in ascending order, and no tile as full."""
    blk = 16
    L = max(q_len, kv_len)
    doc = W.document_ids([5, 1, 20, 13, 61])[:L]
    scalar = SCALAR_MASKS[kind](doc)
    bm = oracle.create_block_mask(_oracle_mask(kind, doc), 1, 1, q_len, kv_len, blk,
                                  separate_full_blocks=False)
    cls = pins.brute_force_tiles(scalar, 1, 1, q_len, kv_len, blk)
    merged = np.where(cls == 0, 0, 1)
    assert pins.block_mask_matches(bm, pins.lists_from_classes(merged))
    assert int(bm.full_kv_num_blocks.sum()) == 0 and not bm.full_kv_indices.any()
    split = oracle.create_block_mask(_oracle_mask(kind, doc), 1, 1, q_len, kv_len, blk)
    assert np.array_equal(bm.to_dense(), split.to_dense())


def test_block_mask_brute_force_batched_heads():
    """(b, h)-dependent mask_mod: each (b, h) gets its own lists."""
    def mod(b, h, q, kv):
        return (q - kv) <= 7 * (h + 1) + 3 * b

    def scalar(b, h, q, kv):
        return (q - kv) <= 7 * (h + 1) + 3 * b

    bm = oracle.create_block_mask(mod, 2, 3, 40, 37, 8)
    cls = pins.brute_force_tiles(scalar, 2, 3, 40, 37, 8)
    assert pins.block_mask_matches(bm, pins.lists_from_classes(cls))


def test_block_mask_class_boundaries():
    """Shapes where a tile sits exactly on each class boundary: one masked
    element in an otherwise full tile, a one-column tail tile, and a window
    edge landing on a tile's far corner."""
    hole = lambda b, h, q, kv: ~((q == 5) & (kv == 7))  # noqa: E731
    cases = [
        (hole, lambda b, h, q, kv: not (q == 5 and kv == 7), 40, 40),
        (oracle.noop_mask, lambda b, h, q, kv: True, 33, 49),
        (oracle.sliding_sink_mask(31, 0), lambda b, h, q, kv: kv <= q and q - kv < 31, 70, 70),
        (oracle.sliding_sink_mask(32, 0), lambda b, h, q, kv: kv <= q and q - kv < 32, 70, 70),
    ]
    for mod, scalar, M, N in cases:
        bm = oracle.create_block_mask(mod, 1, 1, M, N, 16)
        cls = pins.brute_force_tiles(scalar, 1, 1, M, N, 16)
        assert pins.block_mask_matches(bm, pins.lists_from_classes(cls))


def _read_golden(path):
    vals = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, shape, *nums = line.split()
            arr = np.array([float(x) for x in nums])
            if shape != "-":
                arr = arr.astype(np.int32).reshape([int(s) for s in shape.split(",")])
            vals[name] = arr
    return vals


def test_tiny_causal_golden(golden_dir):
    """The tiny causal workload's BlockMask, derived by hand from the page's
    causal example (stored in tests/golden with its derivation)."""
    g = _read_golden(os.path.join(golden_dir, "tiny_causal_block_mask.txt"))
    w = W.TINY_CAUSAL
    bm = oracle.create_block_mask(oracle.causal_mask, w.B, w.Hq, w.Q_LEN, w.KV_LEN, 128)
    for name in ("kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices"):
        assert np.array_equal(getattr(bm, name), g[name]), name
    assert bm.sparsity() == pytest.approx(float(g["sparsity_percent"][0]))


@pytest.mark.parametrize("L", [4096, 8192])
def test_causal_closed_form(L):
    """Causal at full length (the page's 8192 example and the 4096 workload):
    row i lists partial {i} and full {0..i-1}; sparsity = 1 - (n+1)/(2n)."""
    bm = oracle.create_block_mask(oracle.causal_mask, 1, 1, L, L, 128)
    nb = L // 128
    exp = [x[None, None] for x in pins.causal_closed_form(nb)]
    assert pins.block_mask_matches(bm, exp)
    assert bm.sparsity() == pytest.approx(100.0 * (1 - (nb + 1) / (2 * nb)))


def test_sliding_sink_closed_form():
    """Sliding window 1024 + 4 sinks at L = 8192 matches the closed form
    (175 partial and 420 full tiles per head)."""
    w = W.SLIDING_SINKS
    bm = oracle.create_block_mask(oracle.sliding_sink_mask(w.window, w.sinks), 1, 1,
                                  w.Q_LEN, w.KV_LEN, 128)
    exp = [x[None, None] for x in pins.sliding_sink_closed_form(64, 8)]
    assert pins.block_mask_matches(bm, exp)
    assert int(bm.kv_num_blocks.sum()) == 175
    assert int(bm.full_kv_num_blocks.sum()) == 420


def test_document_tiles_against_runs():
    """Document mask at the full packed length: a tile is full iff one
    document covers all its rows and columns and it lies strictly below the
    diagonal; empty iff no row of it reaches back into it; checked from the
    document boundaries directly."""
    w = W.DOCUMENT
    inp_lens = W.document_lengths(w.Q_LEN, *w.doc_len_range, w.doc_seed)
    doc = W.document_ids(inp_lens)
    starts = np.concatenate([[0], np.cumsum(inp_lens)[:-1]])
    start_of = np.repeat(starts, inp_lens)  # first position of each row's doc
    bm = oracle.create_block_mask(oracle.document_causal_mask(doc), 1, 1, w.Q_LEN, w.KV_LEN, 128)
    nb = w.Q_LEN // 128
    cls = np.zeros((nb, nb), np.int8)
    for i in range(nb):
        r0, r1 = 128 * i, 128 * i + 127
        for j in range(nb):
            c0, c1 = 128 * j, 128 * j + 127
            if j > i:
                continue
            # any row q in [r0, r1] with allowed interval [start_of[q], q] meeting [c0, c1]
            rows = np.arange(r0, r1 + 1)
            meets = (start_of[rows] <= c1) & (rows >= c0)
            if not meets.any():
                continue
            same_doc = doc[r0] == doc[r1] == doc[c0] == doc[c1]
            cls[i, j] = 2 if (same_doc and j < i) else 1
    assert pins.block_mask_matches(bm, pins.lists_from_classes(cls[None, None]))


def test_to_dense_round_trip():
    """The page's dense reconstruction loop over both lists gives back the
    set of non-empty tiles."""
    doc = W.document_ids([40, 3, 90, 17])
    for mod in (oracle.causal_mask, oracle.sliding_sink_mask(33, 2),
                oracle.document_causal_mask(doc)):
        bm = oracle.create_block_mask(mod, 1, 1, 150, 150, 16)
        grid = bm.to_dense()
        assert np.array_equal(grid, (bm.tile_counts > 0).astype(np.int32))
        part = oracle.to_dense(bm.kv_num_blocks, bm.kv_indices, grid.shape[-1])
        full = oracle.to_dense(bm.full_kv_num_blocks, bm.full_kv_indices, grid.shape[-1])
        assert not np.any(part & full)


def test_broadcast_build_equals_full_build():
    """A (b, h)-independent mask built at B = H = 1 equals the full build."""
    mod = oracle.sliding_sink_mask(21, 2)
    one = oracle.create_block_mask(mod, 1, 1, 70, 70, 16)
    full = oracle.create_block_mask(mod, 2, 3, 70, 70, 16)
    for name in ("kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices"):
        assert np.array_equal(np.broadcast_to(getattr(one, name), getattr(full, name).shape),
                              getattr(full, name))


def test_numel_and_sparsity_definitions():
    bm = oracle.create_block_mask(oracle.noop_mask, 2, 3, 40, 24, 8)
    assert bm.numel() == 2 * 3 * 40 * 24
    assert bm.sparsity() == 0.0
    assert int(bm.full_kv_num_blocks.sum()) == 2 * 3 * 5 * 3


def test_tail_tile_is_never_full():
    """With lengths not a multiple of the block, the tail tile is partial
    even under the all-true mask."""
    bm = oracle.create_block_mask(oracle.noop_mask, 1, 1, 20, 20, 16)
    assert bm.full_kv_num_blocks[0, 0].tolist() == [1, 0]
    assert bm.kv_num_blocks[0, 0].tolist() == [1, 2]
    assert bm.kv_indices[0, 0].tolist() == [[1, 0], [0, 1]]


# ------------------------------------------------------------ attention pins

MASK_CASES = ["noop", "causal", "sliding_sink", "document_causal"]


@pytest.mark.parametrize("kind", MASK_CASES)
@pytest.mark.parametrize("shape", [(2, 4, 2, 37, 37, 16), (1, 3, 1, 20, 45, 8), (1, 2, 2, 45, 45, 32)])
def test_attention_matches_sdpa(kind, shape):
    """O equals torch's scaled_dot_product_attention (fp64, CPU) with the
    boolean mask; GQA by repeating KV heads over contiguous query groups."""
    B, Hq, Hkv, M, N, D = shape
    q, k, v = _qkv(B, Hq, Hkv, M, N, D, seed=hash((kind,) + shape) % 1000)
    doc = W.document_ids([7, 1, 12, 30])[: max(M, N)]
    mod = oracle.mask_mod_for(kind, window=9, sinks=2, doc_ids=doc)
    allowed = oracle.create_mask(mod, B, Hq, M, N)
    live = allowed.any(axis=-1)
    scale = 0.37
    o, lse = oracle.attention(q, k, v, mod, None, scale)
    ref = pins.sdpa_reference(q, k, v, allowed, scale)
    np.testing.assert_allclose(o[live], ref[live], rtol=0, atol=1e-12)


def test_lse_matches_sdpa_probabilities():
    """With V = identity the library's output is the probability matrix P;
    then LSE = s_ij - log P_ij for any allowed j."""
    B, Hq, Hkv, M, N, D = 1, 2, 1, 30, 30, 16
    q, k, _ = _qkv(B, Hq, Hkv, M, N, D, seed=7)
    v = np.broadcast_to(np.eye(N), (B, Hkv, N, N)).copy()
    mod = oracle.causal_mask
    allowed = oracle.create_mask(mod, B, Hq, M, N)
    scale = 0.25
    P = pins.sdpa_reference(q, k, v, allowed, scale)
    o, lse = oracle.attention(q, k, v, mod, None, scale)
    np.testing.assert_allclose(o, P, atol=1e-13)
    for h in range(Hq):
        for i in range(M):
            j = int(np.argmax(P[0, h, i]))
            s = scale * float(np.dot(q[0, h, i], k[0, 0, j]))
            assert lse[0, h, i] == pytest.approx(s - math.log(P[0, h, i, j]), abs=1e-12)


def test_alibi_matches_sdpa_with_additive_bias():
    """ALiBi equals SDPA with the float bias m_h (j - i) as attn_mask."""
    B, Hq, Hkv, M, N, D = 2, 4, 2, 33, 33, 16
    q, k, v = _qkv(B, Hq, Hkv, M, N, D, seed=11)
    slopes = oracle.alibi_slopes(Hq)
    assert slopes.tolist() == [2.0 ** -2, 2.0 ** -4, 2.0 ** -6, 2.0 ** -8]
    allowed = oracle.create_mask(oracle.causal_mask, B, Hq, M, N)
    i = np.arange(M)[:, None]
    j = np.arange(N)[None, :]
    bias = np.broadcast_to(slopes[None, :, None, None] * (j - i)[None, None], (B, Hq, M, N))
    o, _ = oracle.attention(q, k, v, oracle.causal_mask, oracle.alibi_score(slopes), 0.3)
    ref = pins.sdpa_reference(q, k, v, allowed, 0.3, bias=bias)
    np.testing.assert_allclose(o, ref, atol=1e-12)


def test_alibi_zero_slope_is_identity():
    q, k, v = _qkv(1, 2, 2, 20, 20, 8, seed=3)
    a, la = oracle.attention(q, k, v, oracle.causal_mask, oracle.alibi_score([0.0, 0.0]), 0.5)
    b, lb = oracle.attention(q, k, v, oracle.causal_mask, None, 0.5)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(la, lb)


def test_softcap_limit_and_bound():
    """cap -> infinity reduces to no score_mod; |capped| < cap."""
    q, k, v = _qkv(1, 2, 1, 25, 25, 16, scale=3.0, seed=5)
    a, la = oracle.attention(q, k, v, oracle.causal_mask, oracle.softcap_score(1e9), 0.7)
    b, lb = oracle.attention(q, k, v, oracle.causal_mask, None, 0.7)
    np.testing.assert_allclose(a, b, atol=1e-9)
    np.testing.assert_allclose(la, lb, atol=1e-9)
    s = np.linspace(-500, 500, 1001)
    capped = oracle.softcap_score(50.0)(s, 0, 0, None, None)
    assert np.all(np.abs(capped) < 50.0 + 1e-12)
    assert np.all(np.diff(capped) > 0)


@pytest.mark.parametrize("kind", MASK_CASES)
@pytest.mark.parametrize("score", ["none", "alibi", "softcap", "softcap_alibi"])
def test_attention_matches_loop_formulation(kind, score):
    """A scalar-loop formulation (math module, no NumPy) agrees to 1e-12 for
    every mask kind x score kind, with GQA and Q_LEN != KV_LEN."""
    B, Hq, Hkv, M, N, D = 1, 4, 2, 11, 13, 6
    q, k, v = _qkv(B, Hq, Hkv, M, N, D, scale=4.0, seed=21)
    doc = W.document_ids([3, 1, 5, 4])
    mod = oracle.mask_mod_for(kind, window=4, sinks=2, doc_ids=doc)
    cap = 5.0
    slopes = oracle.alibi_slopes(Hq)
    smod = oracle.score_mod_for(score, Hq, softcap=cap)

    def allowed_fn(b, h, i, j):
        if kind == "noop":
            return True
        if kind == "causal":
            return j <= i
        if kind == "sliding_sink":
            return j <= i and (i - j < 4 or j < 2)
        return int(doc[i]) == int(doc[j]) and j <= i

    def score_fn(s, b, h, i, j):
        if score in ("softcap", "softcap_alibi"):
            s = cap * math.tanh(s / cap)
        if score in ("alibi", "softcap_alibi"):
            s = s + float(slopes[h]) * (j - i)
        return s

    o, lse = oracle.attention(q, k, v, mod, smod, 0.41)
    o2, lse2 = pins.loop_attention(q, k, v, allowed_fn, None if score == "none" else score_fn, 0.41)
    np.testing.assert_allclose(o, o2, atol=1e-12)
    np.testing.assert_allclose(lse, lse2, atol=1e-12)


def test_constant_v_gives_constant_output():
    q, k, _ = _qkv(1, 2, 1, 30, 30, 8, seed=9)
    v = np.full((1, 1, 30, 5), 3.25)
    o, _ = oracle.attention(q, k, v, oracle.sliding_sink_mask(5, 1), oracle.softcap_score(2.0))
    np.testing.assert_allclose(o, 3.25, atol=1e-13)


def test_rows_sum_to_one():
    q, k, _ = _qkv(2, 4, 2, 24, 40, 8, seed=10)
    v = np.ones((2, 2, 40, 1))
    o, _ = oracle.attention(q, k, v, oracle.causal_mask, oracle.alibi_score([0.5, 0.1, 1.0, 2.0]))
    live = oracle.create_mask(oracle.causal_mask, 2, 4, 24, 40).any(-1)
    np.testing.assert_allclose(o[live][..., 0], 1.0, atol=1e-13)


def test_causal_row_zero_is_first_value():
    q, k, v = _qkv(1, 2, 2, 16, 16, 8, seed=12)
    o, lse = oracle.attention(q, k, v, oracle.causal_mask, None, 0.5)
    np.testing.assert_allclose(o[:, :, 0], v[:, :, 0], atol=1e-15)
    for h in range(2):
        assert lse[0, h, 0] == pytest.approx(0.5 * float(q[0, h, 0] @ k[0, h, 0]), abs=1e-14)


def test_single_key_masks_return_that_value_row():
    """Window 1 without sinks, and documents of length 1, leave one key per
    row: O = V (row i gets v_i) and LSE = the diagonal score."""
    q, k, v = _qkv(1, 2, 2, 20, 20, 8, seed=13)
    diag = 0.3 * np.einsum("bhid,bhid->bhi", q, k)
    for mod in (oracle.sliding_sink_mask(1, 0), oracle.document_causal_mask(np.arange(20))):
        o, lse = oracle.attention(q, k, v, mod, None, 0.3)
        np.testing.assert_allclose(o, v, atol=1e-15)
        np.testing.assert_allclose(lse, diag, atol=1e-14)


def test_reductions_to_causal():
    """Window >= L without sinks, and one document covering everything, are
    the causal mask."""
    q, k, v = _qkv(1, 2, 1, 30, 30, 8, seed=14)
    ref = oracle.attention(q, k, v, oracle.causal_mask, None, 0.5)
    for mod in (oracle.sliding_sink_mask(30, 0), oracle.document_causal_mask(np.zeros(30, np.int32))):
        got = oracle.attention(q, k, v, mod, None, 0.5)
        np.testing.assert_array_equal(got[0], ref[0])
        np.testing.assert_array_equal(got[1], ref[1])


def test_empty_rows_give_zero_and_minus_inf():
    """Rows with no allowed key: O = 0 and LSE = -inf."""
    q, k, v = _qkv(1, 1, 1, 40, 16, 8, seed=15)
    o, lse = oracle.attention(q, k, v, oracle.sliding_sink_mask(4, 0), None, 0.5)
    dead = np.arange(40) >= 16 + 4 - 1
    assert np.all(o[0, 0, dead] == 0.0)
    assert np.all(np.isneginf(lse[0, 0, dead]))
    assert np.all(np.isfinite(lse[0, 0, ~dead]))


def test_single_query_noop_is_softmax_weighted_mean():
    """One query over all keys: O is the softmax-weighted mean of V rows."""
    q, k, v = _qkv(1, 1, 1, 1, 50, 8, seed=16)
    o, lse = oracle.attention(q, k, v, None, None, 1.0)
    s = [float(q[0, 0, 0] @ k[0, 0, j]) for j in range(50)]
    mx = max(s)
    w = [math.exp(x - mx) for x in s]
    tot = math.fsum(w)
    mean = sum(wj * v[0, 0, j] for j, wj in enumerate(w)) / tot
    np.testing.assert_allclose(o[0, 0, 0], mean, atol=1e-13)
    assert lse[0, 0, 0] == pytest.approx(mx + math.log(tot), abs=1e-13)


def test_row_subset_equals_full_computation():
    q, k, v = _qkv(2, 4, 2, 64, 64, 8, seed=17)
    full = oracle.attention(q, k, v, oracle.causal_mask, oracle.alibi_score(oracle.alibi_slopes(4)))
    part = oracle.attention(q, k, v, oracle.causal_mask, oracle.alibi_score(oracle.alibi_slopes(4)),
                            batches=[1], heads=[2, 3], rows=[0, 5, 63], row_chunk=2)
    for h in (2, 3):
        # equal up to the BLAS summation order of different row blocks
        np.testing.assert_allclose(part[0][1, h, [0, 5, 63]], full[0][1, h, [0, 5, 63]],
                                   rtol=0, atol=1e-14)
        np.testing.assert_allclose(part[1][1, h, [0, 5, 63]], full[1][1, h, [0, 5, 63]],
                                   rtol=0, atol=1e-14)
    assert np.isnan(part[0][0]).all()


# ------------------------------------------------------------ from_kv_blocks

@pytest.mark.parametrize("kind", list(SCALAR_MASKS))
def test_from_kv_blocks_round_trip(kind):
    """Lists built from a mask_mod, read back through from_kv_blocks with the
    same mask_mod on partial tiles, give the same element mask."""
    doc = W.document_ids([5, 1, 20, 13, 61])
    mm = _oracle_mask(kind, doc)
    bm = oracle.create_block_mask(mm, 1, 1, 77, 90, 16)
    back = oracle.from_kv_blocks_mask(bm.kv_num_blocks, bm.kv_indices, bm.full_kv_num_blocks,
                                      bm.full_kv_indices, 16, mm)
    assert np.array_equal(oracle.create_mask(back, 1, 1, 77, 90), oracle.create_mask(mm, 1, 1, 77, 90))


def test_from_kv_blocks_hand_example():
    """Block 2, 3 x 3 tiles: row 0 lists tile 1 partial (causal inside) and
    tile 0 full; row 1 nothing; row 2 tile 2 full. Checked element by
    element against the definition."""
    kv_num = np.array([[[1, 0, 0]]])
    kv_idx = np.array([[[[1, 0, 0], [0, 0, 0], [0, 0, 0]]]])
    full_num = np.array([[[1, 0, 1]]])
    full_idx = np.array([[[[0, 0, 0], [0, 0, 0], [2, 0, 0]]]])
    mod = oracle.from_kv_blocks_mask(kv_num, kv_idx, full_num, full_idx, 2, oracle.causal_mask)
    got = oracle.create_mask(mod, 1, 1, 6, 6)[0, 0]
    exp = np.zeros((6, 6), dtype=bool)
    exp[0:2, 0:2] = True                        # full tile (0, 0)
    for q in range(2):
        for kv in range(2, 4):
            exp[q, kv] = kv <= q                # partial tile (0, 1): causal -> none
    exp[4:6, 4:6] = True                        # full tile (2, 2)
    assert np.array_equal(got, exp)


@pytest.mark.parametrize("N,page", [(300, 128), (256, 128), (1000, 256), (128, 512)])
def test_gather_paged_round_trip(N, page):
    """The oracle's paged gather undoes the generator's page-by-page scatter
    (written separately, as a loop over pages) for full and partial last
    pages; cache rows outside the sequences are NaN and never gathered."""
    rng = np.random.default_rng(N + page)
    k = rng.standard_normal((2, 3, N, 16)).astype(np.float32)
    v = rng.standard_normal((2, 3, N, 16)).astype(np.float32)
    kc, vc, table = W.paged_cache(k, v, page, seed=N)
    assert np.array_equal(oracle.gather_paged(kc, table, N), k)
    assert np.array_equal(oracle.gather_paged(vc, table, N), v)


def test_gather_paged_identity_layout():
    """One page per sequence holding it whole, page b for batch b: the cache
    is the contiguous tensor itself."""
    rng = np.random.default_rng(5)
    k = rng.standard_normal((3, 2, 256, 8))
    assert np.array_equal(oracle.gather_paged(k, np.arange(3, dtype=np.int32)[:, None], 256), k)


def _prim_truth(name, q, kv, W_, S, P, doc):
    """One primitive by its definition, for a single (q, kv) pair."""
    return {"causal": kv <= q, "window": q - kv < W_, "sink": kv < S, "prefix": kv < P,
            "document": doc[q] == doc[kv]}[name]


@pytest.mark.parametrize("terms", [
    [("causal", "window"), ("causal", "sink")], [("causal", "document", "window")],
    [("prefix",), ("causal", "window")], [("document",)], [("window", "sink")], [()],
    [("causal", "window"), ("sink",), ("prefix", "document"), ("causal", "document")]])
def test_composite_mask_brute_force(terms):
    """The composite oracle against a pure-Python truth table: any() over the
    terms of all() over each term's primitives, pair by pair."""
    L_, W_, S, P = 23, 5, 2, 4
    doc = np.repeat(np.arange(5), [4, 6, 1, 7, 5])
    mod = oracle.composite_mask(terms, W_, S, P, doc)
    q = np.arange(L_)[:, None]
    kv = np.arange(L_)[None, :]
    got = np.broadcast_to(mod(0, 0, q, kv), (L_, L_))
    want = np.array([[any(all(_prim_truth(n, i, j, W_, S, P, doc) for n in t) for t in terms)
                      for j in range(L_)] for i in range(L_)])
    assert np.array_equal(got, want)


def test_composite_mask_reduces_to_the_fixed_kinds():
    """Compositions that spell the fixed kinds give their element masks:
    (causal AND window) OR (causal AND sink) is the sliding window with sinks
    (distributivity), causal OR prefix is PrefixLM, causal AND document is the
    causal document mask."""
    L_ = 300
    doc = np.repeat(np.arange(6), [40, 70, 10, 90, 50, 40])
    q = np.arange(L_)[:, None]
    kv = np.arange(L_)[None, :]
    pairs = [
        (oracle.composite_mask([("causal", "window"), ("causal", "sink")], 50, 3),
         oracle.sliding_sink_mask(50, 3)),
        (oracle.composite_mask([("causal",), ("prefix",)], prefix_len=70), oracle.prefix_lm_mask(70)),
        (oracle.composite_mask([("causal", "document")], doc_ids=doc),
         oracle.document_causal_mask(doc)),
        (oracle.composite_mask([()]), oracle.noop_mask),
    ]
    for a, b in pairs:
        assert np.array_equal(np.broadcast_to(a(0, 0, q, kv), (L_, L_)),
                              np.broadcast_to(b(0, 0, q, kv), (L_, L_)))


@pytest.mark.parametrize("kind", list(SCALAR_MASKS))
@pytest.mark.parametrize("kblk,qblk", [(16, 8), (8, 24), (32, 16)])
def test_block_mask_non_square_brute_force(kind, kblk, qblk):
    """Non-square tiles (page "tensorplay.nn.attention API": BLOCK_SIZE may be
    the tuple (KV_BLOCK_SIZE, Q_BLOCK_SIZE)) against the per-element loop."""
    q_len, kv_len = 77, 50
    doc = W.document_ids([5, 1, 20, 13, 61])[:max(q_len, kv_len)]
    bm = oracle.create_block_mask(_oracle_mask(kind, doc), 1, 1, q_len, kv_len, (kblk, qblk))
    cls = pins.brute_force_tiles(SCALAR_MASKS[kind](doc), 1, 1, q_len, kv_len, kblk, qblk)
    assert pins.block_mask_matches(bm, pins.lists_from_classes(cls))


@pytest.mark.parametrize("B,H", [(1, 1), (2, 3)])
def test_unmasked_pairs_closed_forms(B, H):
    """unmasked_pairs counts the allowed (q, kv) elements of every (b, h):
    closed forms for noop (M N), causal (L (L + 1) / 2), the document mask
    (sum over documents of n (n + 1) / 2) and the sliding window with sinks
    (row q sees min(q + 1, W) window keys plus the sinks below the window),
    and brute force over the dense mask on a ragged shape."""
    L = 1000
    scale = B * H
    assert oracle.unmasked_pairs(oracle.create_block_mask(oracle.noop_mask, B, H, 300, 700,
                                                          128)) == scale * 300 * 700
    assert oracle.unmasked_pairs(oracle.create_block_mask(oracle.causal_mask, B, H, L, L,
                                                          128)) == scale * L * (L + 1) // 2
    lens = np.array([123, 1, 400, 476])
    doc = W.document_ids(lens)
    bm = oracle.create_block_mask(oracle.document_causal_mask(doc), B, H, L, L, 128)
    assert oracle.unmasked_pairs(bm) == scale * int((lens * (lens + 1) // 2).sum())
    Wn, S = 64, 4
    bm = oracle.create_block_mask(oracle.sliding_sink_mask(Wn, S), B, H, L, L, 128)
    q = np.arange(L)
    per_row = np.minimum(q + 1, Wn) + np.clip(np.minimum(S, q - Wn + 1), 0, None)
    assert oracle.unmasked_pairs(bm) == scale * int(per_row.sum())
    dense = oracle.create_mask(oracle.prefix_lm_mask(37), B, H, 150, 211)
    bm = oracle.create_block_mask(oracle.prefix_lm_mask(37), B, H, 150, 211, 128)
    assert oracle.unmasked_pairs(bm) == int(dense.sum())
