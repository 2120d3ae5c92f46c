"""GPU forward vs the fp64 oracle, element by element, through the C ABI."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_masked_amd as m
    m.load_library()
    return m


def tiny(dtype, D, mask, score, B=2, Hq=4, Hkv=2, Q_LEN=300, KV_LEN=300, seed=0, **kw):
    return W.Workload(f"tiny_{dtype}_{D}_{mask}_{score}", B=B, Hq=Hq, Hkv=Hkv, Q_LEN=Q_LEN,
                      KV_LEN=KV_LEN, D=D, dtype=dtype, seed=seed, mask=mask,
                      window=kw.get("window", 100), sinks=kw.get("sinks", 3),
                      doc_seed=kw.get("doc_seed", 77), doc_len_range=kw.get("doc_len_range", (20, 150)),
                      score=score, softcap=kw.get("softcap", 20.0),
                      value_scale=kw.get("value_scale", 1.0), prefix=kw.get("prefix", 170),
                      terms=kw.get("terms"))


def check_full(lib, w, B_mask=1, H_mask=1):
    inp = W.generate(w)
    bm = G.build_gpu_mask(lib, w, inp, B_mask, H_mask)
    o, lse, _ = G.run_gpu(lib, w, inp, bm)
    o_ref, lse_ref = G.oracle_rows(w, inp)
    res = G.compare(w, o, lse, o_ref, lse_ref)
    assert res["ok"], G.summary(res)
    return res


TINY_MASKS = ["noop", "causal", "sliding_sink", "document_causal", "prefix_lm"]
TINY_SCORES = ["none", "alibi", "softcap", "softcap_alibi"]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", TINY_MASKS)
@pytest.mark.parametrize("score", TINY_SCORES)
def test_fwd_tiny_grid(lib, dtype, D, mask, score):
    """Every dtype x head dim x mask x score kind, with GQA, 3 query tiles and a
    ragged tail (300 = 2*128 + 44). bf16 softcap cases scale the inputs by 2
    (cap 20); fp32 cases keep unit-variance inputs, where the 1e-5 bound is
    stated, and use cap 2 so tanh is far from linear. fp16 runs the 16-bit
    kernel with fp16 MFMA under the bf16 bounds."""
    if dtype == "f32":
        w = tiny(dtype, D, mask, score, softcap=2.0)
    else:
        w = tiny(dtype, D, mask, score, value_scale=2.0 if "softcap" in score else 1.0)
    check_full(lib, w)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mask", ["noop", "causal", "sliding_sink", "document_causal"])
def test_fwd_unseparated_mask(lib, dtype, mask):
    """A BlockMask built with separate_full_blocks=False (mask_mod on every
    tile) gives the same attention as the oracle."""
    w = tiny(dtype, 128, mask, "softcap_alibi" if dtype == "bf16" else "alibi", Q_LEN=520,
             KV_LEN=520, value_scale=2.0 if dtype == "bf16" else 1.0)
    inp = W.generate(w)
    bm = G.build_gpu_mask(lib, w, inp, separate_full_blocks=False)
    assert int(bm.full_kv_num_blocks.sum().item()) == 0
    o, lse, _ = G.run_gpu(lib, w, inp, bm)
    o_ref, lse_ref = G.oracle_rows(w, inp)
    res = G.compare(w, o, lse, o_ref, lse_ref)
    assert res["ok"], G.summary(res)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("scale", [-0.125, 0.0])
@pytest.mark.parametrize("mask", ["causal", "sliding_sink"])
def test_fwd_nonpositive_scale(lib, dtype, scale, mask):
    """scale <= 0 is a plain multiplier on q.k (page "tensorplay.nn.attention
    API", flex_attention's scale argument); the bf16 fast path takes the row
    max before scaling, so these scales go through the scaled-score path."""
    w = tiny(dtype, 128, mask, "none", B=1, Hq=2, Hkv=1)
    w = w.with_(extra={"scale": scale})
    check_full(lib, w)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("q_len,kv_len", [(1, 1), (1, 200), (200, 1), (129, 257), (257, 129),
                                          (128, 128), (513, 200)])
def test_fwd_ragged_lengths(lib, dtype, q_len, kv_len):
    check_full(lib, tiny(dtype, 64, "causal", "none", Q_LEN=q_len, KV_LEN=kv_len, B=1, Hq=2))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fwd_mqa_and_per_head_mask(lib, dtype):
    """One KV head for eight query heads; BlockMask built per (b, h)."""
    w = tiny(dtype, 128, "sliding_sink", "alibi", B=2, Hq=8, Hkv=1, Q_LEN=260, KV_LEN=260)
    check_full(lib, w, B_mask=2, H_mask=8)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fwd_empty_rows(lib, dtype):
    """Rows with no allowed key (window 8, no sinks, queries past the keys):
    O = 0 and LSE = -inf."""
    w = tiny(dtype, 64, "sliding_sink", "none", B=1, Hq=2, Hkv=2, Q_LEN=300, KV_LEN=140,
             window=8, sinks=0)
    res = check_full(lib, w)
    assert res["dead_rows"] > 0 and res["dead_ok"]


def test_fwd_document_not_sorted(lib):
    """Document ids that are not contiguous runs (the general definition)."""
    w = tiny("bf16", 64, "document_causal", "none", B=1, Hq=2, Hkv=1, Q_LEN=400, KV_LEN=400)
    inp = W.generate(w)
    inp.doc_ids = np.random.default_rng(3).integers(0, 4, size=400).astype(np.int32)
    o, lse, _ = G.run_gpu(lib, w, inp)
    o_ref, lse_ref = G.oracle_rows(w, inp)
    res = G.compare(w, o, lse, o_ref, lse_ref)
    assert res["ok"], G.summary(res)


def test_fwd_explicit_slopes_and_strided_q(lib):
    """Caller-given ALiBi slopes, and q / out as views of [B, L, H, D] memory."""
    w = tiny("bf16", 128, "causal", "alibi", B=2, Hq=4, Hkv=2, Q_LEN=256, KV_LEN=256)
    inp = W.generate(w)
    slopes = np.array([0.3, 0.05, 0.0, 1.5], dtype=np.float32)
    qd = G.to_device(inp.q.transpose(0, 2, 1, 3), "bf16").transpose(1, 2)  # strided view
    assert not qd.is_contiguous()
    k = G.to_device(inp.k, "bf16")
    v = G.to_device(inp.v, "bf16")
    bm = lib.create_block_mask("causal", 1, 1, 256, 256)
    out = torch.empty((2, 256, 4, 128), dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    o, lse = lib.flex_attention(qd, k, v, bm, score="alibi",
                                alibi_slopes=torch.from_numpy(slopes), out=out)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(inp.q, inp.k, inp.v, oracle.causal_mask,
                                      oracle.alibi_score(slopes.astype(np.float64)), w.scale)
    res = G.compare(w, o.float().cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref)
    assert res["ok"], G.summary(res)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fwd_invariants(lib, dtype):
    """V = 1 gives O = 1 (rows sum to 1); causal row 0 returns V[0]; window 1
    without sinks returns V row by row."""
    B, H, L, D = 1, 2, 256, 64
    rng = np.random.default_rng(9)
    q = rng.standard_normal((B, H, L, D)).astype(np.float32)
    k = rng.standard_normal((B, H, L, D)).astype(np.float32)
    v = rng.standard_normal((B, H, L, D)).astype(np.float32)
    if dtype == "bf16":
        q, k, v = W.round_to_bf16(q), W.round_to_bf16(k), W.round_to_bf16(v)
    qd, kd, vd = (G.to_device(x, dtype) for x in (q, k, v))
    ones = torch.ones_like(vd)
    bm = lib.create_block_mask("causal", 1, 1, L, L)
    o1, _ = lib.flex_attention(qd, kd, ones, bm)
    o, lse = lib.flex_attention(qd, kd, vd, bm)
    bm1 = lib.create_block_mask("sliding_sink", 1, 1, L, L, window=1, num_sinks=0)
    ow, lsew = lib.flex_attention(qd, kd, vd, bm1)
    torch.cuda.synchronize()
    # V = 1: the P.V product uses bf16-rounded probabilities, the sum uses fp32
    tol_ones = 1e-6 if dtype == "f32" else 1e-2
    assert torch.allclose(o1.float(), torch.ones_like(o1.float()), atol=tol_ones, rtol=0)
    # a single allowed key has probability exactly 1: O is that V row exactly
    assert torch.equal(o[:, :, 0].float(), vd[:, :, 0].float())
    assert torch.equal(ow.float(), vd.float())
    diag = (q.astype(np.float64) * k.astype(np.float64)).sum(-1) / math.sqrt(D)
    np.testing.assert_allclose(lsew.cpu().numpy(), diag, atol=1e-5)


def test_fwd_deterministic(lib):
    w = W.DENSE_CAUSAL_GQA.with_(B=1, Q_LEN=1024, KV_LEN=1024)
    inp = W.generate(w)
    bm = G.build_gpu_mask(lib, w, inp)
    q, k, v = (G.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    o1, l1 = lib.flex_attention(q, k, v, bm)
    o2, l2 = lib.flex_attention(q, k, v, bm)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_tiny_causal_workload_full(lib):
    """The tiny fp32 causal workload, every output element."""
    res = check_full(lib, W.TINY_CAUSAL)
    assert res["o_max_abs"] <= 1e-5 and res["lse_max_abs"] <= 1e-5


@pytest.mark.parametrize("splits", [2, 3, 7])
@pytest.mark.parametrize("mask,score", [("noop", "none"), ("sliding_sink", "alibi"),
                                        ("document_causal", "softcap_alibi"),
                                        ("prefix_lm", "none")])
@pytest.mark.parametrize("q_len,kv_len", [(1, 2000), (16, 1000), (130, 700)])
def test_fwd_splitkv(lib, splits, mask, score, q_len, kv_len):
    """Split-KV forward (slices of each row's KV tiles merged by LSE) against
    the oracle: decode-like lengths, GQA, every slice count including slices
    with no tiles (7 slices of 6 tiles)."""
    w = tiny("bf16", 128, mask, score, B=2, Hq=4, Hkv=2, Q_LEN=q_len, KV_LEN=kv_len,
             window=300, prefix=50, value_scale=2.0 if "softcap" in score else 1.0)
    inp = W.generate(w)
    bm = G.build_gpu_mask(lib, w, inp)
    q, k, v = (G.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    out, lse = lib.flex_attention(q, k, v, bm, score=w.score, softcap=w.softcap, scale=w.scale,
                                  num_splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = G.oracle_rows(w, inp)
    res = G.compare(w, out.float().cpu().numpy().astype(np.float64),
                    lse.cpu().numpy().astype(np.float64), o_ref, lse_ref)
    assert res["ok"], G.summary(res)


def test_fwd_splitkv_empty_rows_and_auto(lib):
    """Rows with no allowed key stay O = 0, LSE = -inf through the merge; the
    automatic split count gives the same result as the oracle."""
    w = tiny("bf16", 64, "sliding_sink", "none", B=1, Hq=2, Hkv=1, Q_LEN=400, KV_LEN=150,
             window=60, sinks=0)
    inp = W.generate(w)
    bm = G.build_gpu_mask(lib, w, inp)
    q, k, v = (G.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    for splits in (4, None):
        out, lse = lib.flex_attention(q, k, v, bm, scale=w.scale, num_splits=splits)
        torch.cuda.synchronize()
        o_ref, lse_ref = G.oracle_rows(w, inp)
        res = G.compare(w, out.float().cpu().numpy().astype(np.float64),
                        lse.cpu().numpy().astype(np.float64), o_ref, lse_ref)
        assert res["ok"] and res["dead_rows"] > 0 and res["dead_ok"], G.summary(res)


def test_fwd_decode_workload_sampled(lib):
    """The decode workload at full size (B=8, Hq=32, Hkv=8, 16 queries, 32768
    keys) with the automatic split count, sampled heads against the oracle."""
    w = W.DECODE_GQA
    inp = W.generate(w)
    bm = G.build_gpu_mask(lib, w, inp)
    q, k, v = (G.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    out, lse = lib.flex_attention(q, k, v, bm, scale=w.scale, num_splits=None)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    l_ = lse.cpu().numpy().astype(np.float64)
    for b, h in ((0, 0), (3, 17), (7, 31)):
        o_ref, lse_ref = G.oracle_rows(w, inp, batches=[b], heads=[h])
        res = G.compare(w, o, l_, o_ref, lse_ref)
        assert res["ok"] and res["n_rows"] == w.Q_LEN, G.summary(res)


@pytest.mark.parametrize("q_len", [1, 16, 33, 64])
@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 2), (8, 1), (3, 3), (14, 2), (6, 2), (5, 1)])
@pytest.mark.parametrize("mask,score", [("noop", "alibi"), ("sliding_sink", "softcap_alibi"),
                                        ("prefix_lm", "alibi"), ("causal", "none")])
@pytest.mark.parametrize("splits", [1, None])
def test_fwd_short_query_heads_packed(lib, q_len, Hq, Hkv, mask, score, splits):
    """Short query tiles (Q_LEN <= 64) put several query heads of one KV group
    in a workgroup, one or two waves each; ALiBi's per-head slope checks that
    every wave takes its own head. Group sizes 4, 2, 8 and 1 (no packing);
    7, 3 and 5 pack four (or two) heads with a partial last pack per KV
    group, whose spare waves store nothing."""
    w = tiny("bf16", 128, mask, score, B=2, Hq=Hq, Hkv=Hkv, Q_LEN=q_len, KV_LEN=700,
             window=200, prefix=40, value_scale=2.0 if "softcap" in score else 1.0)
    inp = W.generate(w)
    bm = G.build_gpu_mask(lib, w, inp)
    q, k, v = (G.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    out, lse = lib.flex_attention(q, k, v, bm, score=w.score, softcap=w.softcap, scale=w.scale,
                                  num_splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = G.oracle_rows(w, inp)
    res = G.compare(w, out.float().cpu().numpy().astype(np.float64),
                    lse.cpu().numpy().astype(np.float64), o_ref, lse_ref)
    assert res["ok"], G.summary(res)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("Hq,Hkv", [(6, 2), (14, 2), (5, 1)])
@pytest.mark.parametrize("mask", ["document_causal", "composite"])
@pytest.mark.parametrize("q_len", [16, 40])
@pytest.mark.parametrize("splits", [1, None])
def test_fwd_ragged_packs_dtypes(lib, dtype, D, Hq, Hkv, mask, q_len, splits):
    """Partial head packs (group sizes 3, 7 and 5) for both 16-bit types and
    head dims 64 and 128, on the masks that read document ids (document
    causal; a composite of same-document-causal OR sinks): 16 queries take
    the 16-row step with packs of four heads, 40 queries two waves a head
    with packs of two. Head dim 256 runs the same shapes one head a
    workgroup."""
    terms = (("causal", "document"), ("sink",)) if mask == "composite" else None
    w = tiny(dtype, D, mask, "alibi", B=2, Hq=Hq, Hkv=Hkv, Q_LEN=q_len, KV_LEN=700,
             doc_len_range=(40, 300), terms=terms)
    check_splits(lib, w, splits)


def test_fwd_short_query_per_head_mask_not_packed(lib):
    """A BlockMask built per head (H_mask = Hq) keeps one head per workgroup:
    same results as the broadcast mask."""
    w = tiny("bf16", 64, "sliding_sink", "alibi", B=1, Hq=8, Hkv=2, Q_LEN=16, KV_LEN=900,
             window=300)
    inp = W.generate(w)
    q, k, v = (G.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    o_ref, lse_ref = G.oracle_rows(w, inp)
    for H_mask in (1, 8):
        bm = G.build_gpu_mask(lib, w, inp, 1, H_mask)
        out, lse = lib.flex_attention(q, k, v, bm, score=w.score, scale=w.scale)
        torch.cuda.synchronize()
        res = G.compare(w, out.float().cpu().numpy().astype(np.float64),
                        lse.cpu().numpy().astype(np.float64), o_ref, lse_ref)
        assert res["ok"], (H_mask, G.summary(res))


@pytest.mark.parametrize("splits", [3, None])
@pytest.mark.parametrize("mask,score", [("noop", "alibi"), ("sliding_sink", "softcap_alibi"),
                                        ("document_causal", "none")])
def test_fwd_f16_splitkv(lib, splits, mask, score):
    """fp16 through the split-KV path and the combine kernel (decode-like
    lengths, packed heads)."""
    w = tiny("f16", 128, mask, score, B=2, Hq=8, Hkv=2, Q_LEN=16, KV_LEN=1500, window=300,
             value_scale=2.0 if "softcap" in score else 1.0)
    check_splits(lib, w, splits)


def check_splits(lib, w, splits):
    inp = W.generate(w)
    bm = G.build_gpu_mask(lib, w, inp)
    q, k, v = (G.to_device(x, w.dtype) for x in (inp.q, inp.k, inp.v))
    out, lse = lib.flex_attention(q, k, v, bm, score=w.score, softcap=w.softcap, scale=w.scale,
                                  num_splits=splits)
    torch.cuda.synchronize()
    o_ref, lse_ref = G.oracle_rows(w, inp)
    res = G.compare(w, out.float().cpu().numpy().astype(np.float64),
                    lse.cpu().numpy().astype(np.float64), o_ref, lse_ref)
    assert res["ok"], G.summary(res)


def test_fwd_f16_dense_causal_sampled(lib):
    """The dense causal GQA workload's shapes in fp16 (B=4, Hq=16, Hkv=4,
    4096 x 4096, D=128), sampled query rows of three heads against the
    oracle."""
    w = W.DENSE_CAUSAL_GQA.with_(name="dense_causal_gqa_f16", dtype="f16")
    inp = W.generate(w)
    bm = G.build_gpu_mask(lib, w, inp)
    o, lse, _ = G.run_gpu(lib, w, inp, bm)
    rows = np.r_[0:3, 1000:1003, 4093:4096]
    for b, h in ((0, 0), (2, 9), (3, 15)):
        o_ref, lse_ref = G.oracle_rows(w, inp, batches=[b], heads=[h], rows=rows)
        res = G.compare(w, o, lse, o_ref, lse_ref)
        assert res["ok"] and res["n_rows"] == len(rows), G.summary(res)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("mask", ["noop", "causal", "sliding_sink", "document_causal",
                                  "prefix_lm"])
@pytest.mark.parametrize("score", ["none", "alibi", "softcap", "softcap_alibi"])
def test_fwd_head_dim_256(lib, dtype, mask, score):
    """Head dim 256 (16-bit kernel, 32-key steps, one workgroup per CU):
    every mask and score kind, GQA, 3 query tiles with a ragged tail."""
    w = tiny(dtype, 256, mask, score, value_scale=2.0 if "softcap" in score else 1.0)
    check_full(lib, w)


@pytest.mark.parametrize("splits", [1, 5])
def test_fwd_head_dim_256_short_query_and_split(lib, splits):
    w = tiny("bf16", 256, "sliding_sink", "softcap_alibi", B=2, Hq=8, Hkv=2, Q_LEN=16,
             KV_LEN=1200, window=500, value_scale=2.0)
    check_splits(lib, w, splits)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 128), ("bf16", 64)])
@pytest.mark.parametrize("case", ["sink_tile", "prefix_tile", "kv_tail"])
@pytest.mark.parametrize("splits", [1, None])
def test_fwd_last_tile_half_step(lib, dtype, D, case, splits):
    """The walk's last tile (a row's lowest partial tile) with a second
    64-key step that no row of the workgroup attends is cut to its first
    step: a sliding window's sink tile for rows past the window, a PrefixLM
    prefix tile for rows past the diagonal band, and a key tail of fewer
    than 64 keys. Head dim 64 has one step per tile (nothing to cut)."""
    if case == "sink_tile":
        w = tiny(dtype, D, "sliding_sink", "none", B=2, Hq=4, Hkv=2, Q_LEN=1100, KV_LEN=1100,
                 window=128, sinks=4)
    elif case == "prefix_tile":
        w = tiny(dtype, D, "prefix_lm", "none", B=1, Hq=4, Hkv=1, Q_LEN=900, KV_LEN=900,
                 prefix=40)
    else:
        w = tiny(dtype, D, "noop", "softcap", B=2, Hq=4, Hkv=2, Q_LEN=200, KV_LEN=950)
    check_splits(lib, w, splits)
