"""GPU backward vs the fp64 oracle, element by element, through the C ABI.

Tolerance (bf16 inputs, bf16 gradients), per element of a gradient row g
(a query row of dQ, a key row of dK / dV):
    |g_gpu - g_ref| <= BWD_ROW_RMS * rms(row of g_ref) + BWD_RTOL * |g_ref|
                       + BWD_FLOOR * rms(g_ref) + BWD_ABS.
The kernels round dS and P to bf16 (relative error up to 2^-8) before their
matrix products and round each gradient to bf16 (up to 2^-8); Delta and
dP - Delta are formed in fp32. The product errors are sums over the row's
terms, so they scale with that row's magnitude, not the tensor's: rows that
attend to few keys (early causal rows) have gradients many times the
tensor's RMS. A CPU simulation of these roundings on the tiny grid stays
under 1.5% of the row RMS; the bound allows 4% of the row RMS, 2% of the
element for the output rounding, 0.1% of the tensor RMS for rows whose
reference is nearly zero, and 1e-5 for gradients that are exactly zero in
the reference (a row with a single allowed key).

The training pair (Delta = dO . O from the forward's fp32 O) adds one
term. That O was formed with P rounded to bf16 for its P.V product, so
Delta_i is off by at most 2^-9 sum_j P_ij |dP_ij| (bound used: 2^-8 times
it, a_i), which reaches dQ_i through -scale * dmod * P_ij * k_j and dK_j
through -scale * dmod * P_ij * q_i:
    dQ_id += 2^-8 scale a_i sum_j P_ij |dmod_ij| |k_jd|
    dK_jd += 2^-8 scale sum_i a_i P_ij |dmod_ij| |q_id|   (over the GQA group)
(dV does not use Delta.) This error does not shrink with the row's
gradient, which is why the training pair is opt-in.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_helpers as G

pytestmark = pytest.mark.gpu

BWD_ROW_RMS = 0.04
BWD_RTOL = 0.02
BWD_FLOOR = 1e-3
BWD_ABS = 1e-5


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_masked_amd as m
    m.load_library()
    return m


def tiny(D, mask, score, B=2, Hq=4, Hkv=2, Q_LEN=300, KV_LEN=300, seed=0, dtype="bf16", **kw):
    return W.Workload(f"bwd_{D}_{mask}_{score}", B=B, Hq=Hq, Hkv=Hkv, Q_LEN=Q_LEN,
                      KV_LEN=KV_LEN, D=D, dtype=dtype, seed=seed, mask=mask,
                      window=kw.get("window", 100), sinks=kw.get("sinks", 3),
                      doc_seed=kw.get("doc_seed", 77),
                      doc_len_range=kw.get("doc_len_range", (20, 150)), score=score,
                      softcap=kw.get("softcap", 20.0), value_scale=kw.get("value_scale", 1.0),
                      prefix=kw.get("prefix", 170), terms=kw.get("terms"))


def mask_of(lib, w, inp, B_mask=1, H_mask=1, separate_full_blocks=True):
    return G.build_gpu_mask(lib, w, inp, B_mask, H_mask, separate_full_blocks,
                            backward_lists=True)


def run_bwd(lib, w, inp, d_out, bm):
    q = G.to_device(inp.q, w.dtype)
    k = G.to_device(inp.k, w.dtype)
    v = G.to_device(inp.v, w.dtype)
    g = G.to_device(d_out, w.dtype)
    out, lse = lib.flex_attention(q, k, v, bm, score=w.score, softcap=w.softcap, scale=w.scale)
    dq, dk, dv = lib.flex_attention_backward(q, k, v, lse, g, bm, score=w.score,
                                             softcap=w.softcap, scale=w.scale)
    torch.cuda.synchronize()
    assert dq.dtype == dk.dtype == dv.dtype == q.dtype
    return [t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]


def oracle_bwd(w, inp, d_out, **sel):
    mask, score = oracle.for_workload(w, inp)
    grad = oracle.score_grad_for(w.score, w.softcap)
    return oracle.attention_backward(inp.q, inp.k, inp.v, d_out, mask, score, grad, w.scale, **sel)


def check(got, ref, name, extra=None):
    """Apply the bound above (plus `extra`, elementwise) to the rows the
    reference computed; returns the largest error over its bound."""
    rows = ~np.isnan(ref).any(axis=-1)
    g, r = got[rows], ref[rows]
    ex = 0.0 if extra is None else extra[rows]
    assert np.all(np.isfinite(g)), f"{name}: non-finite values"
    if not r.size:
        return 0.0
    rms_all = float(np.sqrt(np.mean(r * r)))
    rms_row = np.sqrt(np.mean(r * r, axis=-1, keepdims=True))
    err = np.abs(g - r)
    bound = BWD_ROW_RMS * rms_row + BWD_RTOL * np.abs(r) + BWD_FLOOR * rms_all + BWD_ABS + ex
    ratio = err / bound
    worst = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    assert np.all(err <= bound), (f"{name}: err/bound {ratio[worst]:.3g} at {worst}: err "
                                  f"{err[worst]:.4g}, ref {r[worst]:.4g}, row rms "
                                  f"{float(rms_row[worst[:-1]][0]):.4g}, tensor rms {rms_all:.4g}")
    return float(ratio.max())


def delta_rounding_terms(w, inp, d_out):
    """The training pair's extra bound terms for dQ and dK (fp64, from the
    oracle's probabilities; see the module docstring)."""
    mask_mod, score_mod = oracle.for_workload(w, inp)
    grad = oracle.score_grad_for(w.score, w.softcap)
    _, lse = oracle.attention(inp.q, inp.k, inp.v, mask_mod, score_mod, w.scale)
    q, k, v = (np.asarray(x, np.float64) for x in (inp.q, inp.k, inp.v))
    g = np.asarray(d_out, np.float64)
    ex_q = np.zeros(q.shape)
    ex_k = np.zeros(k.shape)
    qi = np.arange(w.Q_LEN)[:, None]
    kj = np.arange(w.KV_LEN)[None, :]
    for b in range(w.B):
        for h in range(w.Hq):
            hk = h // (w.Hq // w.Hkv)
            s = w.scale * (q[b, h] @ k[b, hk].T)
            sm = score_mod(s, b, h, qi, kj) if score_mod is not None else s
            allowed = np.broadcast_to(mask_mod(b, h, qi, kj), s.shape)
            lse_bh = np.where(np.isfinite(lse[b, h]), lse[b, h], np.inf)[:, None]
            p = np.where(allowed, np.exp(np.where(allowed, sm, -np.inf) - lse_bh), 0.0)
            dmod = np.abs(grad(s, b, h, qi, kj)) if grad is not None else 1.0
            a = (p * np.abs(g[b, h] @ v[b, hk].T)).sum(axis=1)
            c = 2.0 ** -8 * w.scale
            ex_q[b, h] = c * a[:, None] * ((p * dmod) @ np.abs(k[b, hk]))
            ex_k[b, hk] += c * ((p * dmod).T * a[None, :]) @ np.abs(q[b, h])
    return ex_q, ex_k


def full_check(lib, w, B_mask=1, H_mask=1, separate_full_blocks=True):
    inp = W.generate(w)
    d_out = W.generate_upstream(w)
    bm = mask_of(lib, w, inp, B_mask, H_mask, separate_full_blocks)
    got = run_bwd(lib, w, inp, d_out, bm)
    ref = oracle_bwd(w, inp, d_out)
    return [check(g, r, n) for g, r, n in zip(got, ref, ("dq", "dk", "dv"))]


# ------------------------------------------------------------ backward lists

@pytest.mark.parametrize("q_len,kv_len", [(1, 1), (129, 129), (300, 255), (255, 300), (512, 512),
                                          (700, 1), (1, 700)])
@pytest.mark.parametrize("kind,window,sinks", [
    ("noop", 0, 0), ("causal", 0, 0), ("sliding_sink", 200, 130), ("document_causal", 0, 0)])
def test_backward_lists_bit_exact(lib, q_len, kv_len, kind, window, sinks):
    """q_num_blocks / q_indices / full_q_* equal the oracle's transpose."""
    rng = np.random.default_rng(q_len * 31 + kv_len)
    L = max(q_len, kv_len)
    doc = None
    if kind == "document_causal":
        lens = []
        while sum(lens) < L:
            lens.append(int(rng.integers(1, 150)))
        doc = W.document_ids(lens)[:L]
    ref = oracle.create_block_mask(oracle.mask_mod_for(kind, window, sinks, doc), 1, 1, q_len,
                                   kv_len, 128)
    exp = oracle.transpose_block_mask(ref)
    bm = lib.create_block_mask(kind, 1, 1, q_len, kv_len, 128, window=window, num_sinks=sinks,
                               doc_ids=None if doc is None else torch.from_numpy(doc),
                               backward_lists=True)
    torch.cuda.synchronize()
    got = [bm.q_num_blocks, bm.q_indices, bm.full_q_num_blocks, bm.full_q_indices]
    for name, g, e in zip(("q_num", "q_idx", "full_q_num", "full_q_idx"), got, exp):
        assert np.array_equal(g.cpu().numpy(), e), name


@pytest.mark.parametrize("kind", ["noop", "causal"])
def test_backward_lists_large_grid(lib, kind):
    """13 x 4096 tiles: more than the LDS class grid holds, so the builder
    takes its per-KV-tile search path."""
    ref = oracle.create_block_mask(oracle.mask_mod_for(kind), 1, 1, 1664, 524288, 128)
    exp = oracle.transpose_block_mask(ref)
    bm = lib.create_block_mask(kind, 1, 1, 1664, 524288, 128, backward_lists=True)
    torch.cuda.synchronize()
    for g, e in zip((bm.q_num_blocks, bm.q_indices, bm.full_q_num_blocks, bm.full_q_indices), exp):
        assert np.array_equal(g.cpu().numpy(), e)


def test_backward_lists_full_workload(lib):
    """The dense causal workload's lists (32 x 32 tiles)."""
    ref = oracle.create_block_mask(oracle.causal_mask, 1, 1, 4096, 4096, 128)
    exp = oracle.transpose_block_mask(ref)
    bm = lib.create_block_mask("causal", 1, 1, 4096, 4096, 128, backward_lists=True)
    torch.cuda.synchronize()
    for g, e in zip((bm.q_num_blocks, bm.q_indices, bm.full_q_num_blocks, bm.full_q_indices), exp):
        assert np.array_equal(g.cpu().numpy(), e)


# ------------------------------------------------------------------ gradients

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", ["noop", "causal", "sliding_sink", "document_causal",
                                  "prefix_lm"])
@pytest.mark.parametrize("score", ["none", "alibi", "softcap", "softcap_alibi"])
def test_bwd_tiny_grid(lib, D, mask, score):
    """Every head dim x mask x score kind, GQA (2 query heads per KV head),
    3 query and KV tiles with a ragged tail (300 = 2*128 + 44)."""
    w = tiny(D, mask, score, value_scale=2.0 if "softcap" in score else 1.0)
    full_check(lib, w)


@pytest.mark.parametrize("q_len,kv_len", [(1, 1), (1, 200), (200, 1), (129, 257), (257, 129),
                                          (128, 128), (513, 200)])
def test_bwd_ragged_lengths(lib, q_len, kv_len):
    """Lengths that are not multiples of the tile, Q_LEN != KV_LEN (rows with
    no key under causal when Q_LEN > KV_LEN... and tail tiles on both axes)."""
    w = tiny(128, "causal", "none", B=1, Hq=2, Hkv=1, Q_LEN=q_len, KV_LEN=kv_len)
    full_check(lib, w)


def test_bwd_empty_rows(lib):
    """Sliding window without sinks and Q_LEN > KV_LEN + window: query rows
    with no allowed key (LSE = -inf) get dQ = 0 and add nothing."""
    w = tiny(128, "sliding_sink", "none", B=1, Hq=2, Hkv=1, Q_LEN=400, KV_LEN=150, window=60,
             sinks=0)
    full_check(lib, w)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 1), (8, 2)])
def test_bwd_head_groupings(lib, Hq, Hkv):
    """MHA, MQA and GQA with 4 heads per group: dK / dV sum the group."""
    w = tiny(64, "causal", "alibi", B=1, Hq=Hq, Hkv=Hkv, Q_LEN=260, KV_LEN=260)
    full_check(lib, w)


def test_bwd_per_head_mask_rows(lib):
    """A BlockMask built per (b, h) (B and H not broadcast) gives the same
    gradients."""
    w = tiny(128, "sliding_sink", "softcap", B=2, Hq=4, Hkv=2, Q_LEN=384, KV_LEN=384,
             value_scale=2.0)
    full_check(lib, w, B_mask=2, H_mask=4)


def test_bwd_unseparated_mask(lib):
    """separate_full_blocks=False: every tile listed as partial, mask on all."""
    w = tiny(128, "causal", "softcap_alibi", Q_LEN=384, KV_LEN=384, value_scale=2.0)
    full_check(lib, w, separate_full_blocks=False)


def test_bwd_dense_causal_full_size_sampled(lib):
    """The dense causal workload at full size (B=4, Hq=16, Hkv=4, L=4096,
    D=128): dQ rows checked against the oracle on a sample of (b, h, rows)
    (dQ of a row needs only that row), dK / dV of one KV head checked in full
    against the oracle over its four query heads restricted to b = 0."""
    w = W.DENSE_CAUSAL_GQA
    inp = W.generate(w)
    d_out = W.generate_upstream(w)
    bm = mask_of(lib, w, inp)
    dq, dk, dv = run_bwd(lib, w, inp, d_out, bm)
    rows = np.array([0, 1, 127, 128, 2047, 3000, 4095])
    for b, h in ((0, 0), (1, 5), (3, 15)):
        ref_dq, _, _ = oracle_bwd(w, inp, d_out, batches=[b], heads=[h], rows=rows)
        check(dq[b, h, rows], ref_dq[b, h, rows], f"dq[{b},{h}]")
    _, ref_dk, ref_dv = oracle_bwd(w, inp, d_out, batches=[0], heads=[4, 5, 6, 7])
    check(dk[0, 1], ref_dk[0, 1], "dk[0,1]")
    check(dv[0, 1], ref_dv[0, 1], "dv[0,1]")


def test_bwd_deterministic(lib):
    """Two backward calls give bit-identical gradients (no atomics)."""
    w = tiny(128, "document_causal", "alibi", Q_LEN=520, KV_LEN=520)
    inp = W.generate(w)
    d_out = W.generate_upstream(w)
    bm = mask_of(lib, w, inp)
    a = run_bwd(lib, w, inp, d_out, bm)
    b = run_bwd(lib, w, inp, d_out, bm)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_explicit_slopes_and_strided_tensors(lib):
    """Caller-given ALiBi slopes; q, d_out and dq as views of [B, L, H, D]
    memory (strided), k as a strided view too."""
    w = tiny(128, "causal", "alibi", B=2, Hq=4, Hkv=2, Q_LEN=256, KV_LEN=256)
    inp = W.generate(w)
    g = W.generate_upstream(w)
    slopes = np.array([0.3, 0.05, 0.0, 1.5], dtype=np.float32)
    st = lambda x: G.to_device(x.transpose(0, 2, 1, 3), "bf16").transpose(1, 2)  # noqa: E731
    q, k, gd = st(inp.q), st(inp.k), st(g)
    assert not q.is_contiguous() and not k.is_contiguous()
    v = G.to_device(inp.v, "bf16")
    sl = torch.from_numpy(slopes)
    bm = mask_of(lib, w, inp)
    out, lse = lib.flex_attention(q, k, v, bm, score="alibi", alibi_slopes=sl)
    dq_buf = torch.empty((2, 256, 4, 128), dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    dq, dk, dv = lib.flex_attention_backward(q, k, v, lse, gd, bm, score="alibi", alibi_slopes=sl,
                                             dq=dq_buf)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(inp.q, inp.k, inp.v, g, oracle.causal_mask,
                                    oracle.alibi_score(slopes.astype(np.float64)), None, w.scale)
    for t, r, n in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
        check(t.float().cpu().numpy().astype(np.float64), r, n)


@pytest.mark.parametrize("score", ["none", "softcap"])
def test_bwd_negative_scale(lib, score):
    """scale < 0 is a plain multiplier on q.k, as in the forward."""
    w = tiny(128, "sliding_sink", score, B=1, Hq=2, Hkv=1, Q_LEN=300, KV_LEN=300,
             softcap=5.0).with_(extra={"scale": -0.1})
    full_check(lib, w)


def test_bwd_per_batch_documents(lib):
    """Per-batch document ids with a BlockMask built per batch."""
    w = tiny(64, "document_causal", "none", B=2, Hq=2, Hkv=1, Q_LEN=400, KV_LEN=400)
    inp = W.generate(w)
    rng = np.random.default_rng(21)
    docs = []
    for _ in range(2):
        lens = []
        while sum(lens) < 400:
            lens.append(int(rng.integers(10, 120)))
        docs.append(W.document_ids(lens)[:400])
    both = np.stack(docs).astype(np.int32)
    g = W.generate_upstream(w)
    bm = lib.create_block_mask("document_causal", 2, 1, 400, 400, 128,
                               doc_ids=torch.from_numpy(both), backward_lists=True)
    q, k, v = (G.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    out, lse = lib.flex_attention(q, k, v, bm)
    dq, dk, dv = lib.flex_attention_backward(q, k, v, lse, G.to_device(g, "bf16"), bm)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(inp.q, inp.k, inp.v, g, oracle.document_causal_mask(both),
                                    None, None, w.scale)
    for t, r, n in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
        check(t.float().cpu().numpy().astype(np.float64), r, n)


@pytest.mark.parametrize("q_len,kv_len", [(300, 700), (700, 300)])
def test_bwd_sliding_sinks_unequal_lengths(lib, q_len, kv_len):
    """Sliding window + sinks with Q_LEN != KV_LEN (tail tiles on both axes,
    rows beyond the keys, keys beyond the queries)."""
    w = tiny(128, "sliding_sink", "softcap_alibi", B=1, Hq=4, Hkv=1, Q_LEN=q_len, KV_LEN=kv_len,
             window=150, sinks=5, value_scale=2.0)
    full_check(lib, w)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", ["noop", "causal", "sliding_sink", "document_causal", "prefix_lm"])
@pytest.mark.parametrize("score", ["none", "alibi", "softcap", "softcap_alibi"])
def test_training_pair_fp32_out_delta(lib, D, mask, score):
    """flex_attention_train writes the same bf16 O and LSE as flex_attention
    plus an fp32 O; flex_attention_backward(out_f32=...) takes Delta from it
    and meets the same gradient bound against the oracle."""
    w = tiny(D, mask, score, value_scale=2.0 if "softcap" in score else 1.0)
    inp = W.generate(w)
    d_out = W.generate_upstream(w)
    bm = mask_of(lib, w, inp)
    q, k, v = (G.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    g = G.to_device(d_out, "bf16")
    o1, l1 = lib.flex_attention(q, k, v, bm, score=w.score, softcap=w.softcap, scale=w.scale)
    o2, l2, o32 = lib.flex_attention_train(q, k, v, bm, score=w.score, softcap=w.softcap,
                                           scale=w.scale)
    dq, dk, dv = lib.flex_attention_backward(q, k, v, l2, g, bm, score=w.score,
                                             softcap=w.softcap, scale=w.scale, out_f32=o32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o32.to(torch.bfloat16), o2)  # the bf16 O is the fp32 O rounded
    ref = oracle_bwd(w, inp, d_out)
    ex_q, ex_k = delta_rounding_terms(w, inp, d_out)
    for t, r, n, ex in zip((dq, dk, dv), ref, ("dq", "dk", "dv"), (ex_q, ex_k, None)):
        check(t.float().cpu().numpy().astype(np.float64), r, n, ex)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask,score", [("causal", "softcap_alibi"), ("sliding_sink", "alibi"),
                                        ("document_causal", "none")])
@pytest.mark.parametrize("q_len", [5, 16])
def test_training_pair_short_queries(lib, D, mask, score, q_len):
    """At most 16 query rows with four query heads per KV head: the forward
    runs the 16-row step, whose fp32 O feeds Delta; the gradients meet the
    same bound against the oracle."""
    w = tiny(D, mask, score, Hq=8, Hkv=2, Q_LEN=q_len, KV_LEN=700, window=200,
             value_scale=2.0 if "softcap" in score else 1.0)
    inp = W.generate(w)
    d_out = W.generate_upstream(w)
    bm = mask_of(lib, w, inp)
    q, k, v = (G.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    g = G.to_device(d_out, "bf16")
    o1, l1 = lib.flex_attention(q, k, v, bm, score=w.score, softcap=w.softcap, scale=w.scale)
    o2, l2, o32 = lib.flex_attention_train(q, k, v, bm, score=w.score, softcap=w.softcap,
                                           scale=w.scale)
    dq, dk, dv = lib.flex_attention_backward(q, k, v, l2, g, bm, score=w.score,
                                             softcap=w.softcap, scale=w.scale, out_f32=o32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o32.to(torch.bfloat16), o2)
    ref = oracle_bwd(w, inp, d_out)
    ex_q, ex_k = delta_rounding_terms(w, inp, d_out)
    for t, r, n, ex in zip((dq, dk, dv), ref, ("dq", "dk", "dv"), (ex_q, ex_k, None)):
        check(t.float().cpu().numpy().astype(np.float64), r, n, ex)


def test_training_pair_dense_causal_sampled(lib):
    """The dense causal workload's shapes through the training pair: dQ rows
    of two heads against the oracle."""
    w = W.DENSE_CAUSAL_GQA
    inp = W.generate(w)
    d_out = W.generate_upstream(w)
    bm = mask_of(lib, w, inp)
    q, k, v = (G.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    g = G.to_device(d_out, "bf16")
    _, lse, o32 = lib.flex_attention_train(q, k, v, bm, scale=w.scale)
    dq, _, _ = lib.flex_attention_backward(q, k, v, lse, g, bm, scale=w.scale, out_f32=o32)
    torch.cuda.synchronize()
    rows = np.r_[0:2, 2047:2050, 4094:4096]
    got = dq.float().cpu().numpy().astype(np.float64)
    for b, h in ((0, 3), (3, 14)):
        ref = oracle_bwd(w, inp, d_out, batches=[b], heads=[h], rows=rows)[0]
        assert (~np.isnan(ref).any(axis=-1)).sum() == len(rows)
        check(got, ref, "dq")


# ------------------------------------------------------------- fp16 inputs
# The same kernels with fp16 elements: P and dS are rounded to fp16 (2^-11
# relative) instead of bf16 (2^-8) and the gradients are stored in fp16, so
# the bf16-derived bound above holds with room to spare.

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", ["noop", "causal", "sliding_sink", "document_causal",
                                  "prefix_lm"])
@pytest.mark.parametrize("score", ["none", "softcap_alibi"])
def test_bwd_f16_grid(lib, D, mask, score):
    """fp16 q, k, v and dO: every head dim x mask kind, with and without
    score mods, GQA, ragged tail tiles; gradients come back in fp16."""
    w = tiny(D, mask, score, dtype="f16", value_scale=2.0 if "softcap" in score else 1.0)
    full_check(lib, w)


@pytest.mark.parametrize("q_len,kv_len", [(1, 200), (257, 129), (513, 200)])
def test_bwd_f16_ragged_lengths(lib, q_len, kv_len):
    """fp16 with lengths off the tile grid and Q_LEN != KV_LEN."""
    w = tiny(128, "causal", "alibi", B=1, Hq=4, Hkv=1, Q_LEN=q_len, KV_LEN=kv_len, dtype="f16")
    full_check(lib, w)


def test_bwd_f16_matches_bf16_structure(lib):
    """The fp16 and bf16 backward of inputs exact in both types (small
    integers over 8) agree to the rounding of their stored gradients."""
    w = tiny(128, "sliding_sink", "alibi", B=1, Hq=4, Hkv=2, Q_LEN=384, KV_LEN=384)
    inp = W.generate(w)
    rng = np.random.default_rng(5)
    q, k, v, g = (rng.integers(-8, 9, size=x.shape).astype(np.float32) / 8
                  for x in (inp.q, inp.k, inp.v, inp.q))
    bm = mask_of(lib, w, inp)
    res = {}
    for dt in ("bf16", "f16"):
        tq, tk, tv, tg = (G.to_device(x, dt) for x in (q, k, v, g))
        out, lse = lib.flex_attention(tq, tk, tv, bm, score="alibi", scale=w.scale)
        grads = lib.flex_attention_backward(tq, tk, tv, lse, tg, bm, score="alibi",
                                            scale=w.scale)
        torch.cuda.synchronize()
        res[dt] = [t.float().cpu().numpy().astype(np.float64) for t in grads]
    ref = oracle.attention_backward(q, k, v, g, *oracle.for_workload(w, inp),
                                    oracle.score_grad_for("alibi", 0.0), w.scale)
    for n, a, b, r in zip(("dq", "dk", "dv"), res["bf16"], res["f16"], ref):
        # fp16 keeps 3 more mantissa bits at every rounding: its error is the smaller
        ea, eb = np.abs(a - r).max(), np.abs(b - r).max()
        assert eb <= ea, (n, ea, eb)
        check(b, r, n)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask,score", [("causal", "softcap_alibi"), ("document_causal", "none")])
def test_training_pair_f16(lib, D, mask, score):
    """The fp16 training pair: flex_attention_train's fp32 O rounds to its
    fp16 O, and the backward that takes Delta from it meets the bound."""
    w = tiny(D, mask, score, dtype="f16", value_scale=2.0 if "softcap" in score else 1.0)
    inp = W.generate(w)
    d_out = W.generate_upstream(w)
    bm = mask_of(lib, w, inp)
    q, k, v = (G.to_device(x, "f16") for x in (inp.q, inp.k, inp.v))
    g = G.to_device(d_out, "f16")
    o1, l1 = lib.flex_attention(q, k, v, bm, score=w.score, softcap=w.softcap, scale=w.scale)
    o2, l2, o32 = lib.flex_attention_train(q, k, v, bm, score=w.score, softcap=w.softcap,
                                           scale=w.scale)
    dq, dk, dv = lib.flex_attention_backward(q, k, v, l2, g, bm, score=w.score,
                                             softcap=w.softcap, scale=w.scale, out_f32=o32)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o32.to(torch.float16), o2)
    ref = oracle_bwd(w, inp, d_out)
    ex_q, ex_k = delta_rounding_terms(w, inp, d_out)
    for t, r, n, ex in zip((dq, dk, dv), ref, ("dq", "dk", "dv"), (ex_q, ex_k, None)):
        assert t.dtype == torch.float16
        check(t.float().cpu().numpy().astype(np.float64), r, n, ex)


def test_bwd_f16_dense_causal_full_size_sampled(lib):
    """The dense causal workload's shapes (B=4, Hq=16, Hkv=4, L=4096, D=128)
    in fp16: sampled dQ rows of two heads and dK / dV of one KV head of
    b = 0 against the oracle."""
    w = W.DENSE_CAUSAL_GQA.with_(dtype="f16", name="dense_causal_gqa_f16")
    inp = W.generate(w)
    d_out = W.generate_upstream(w)
    bm = mask_of(lib, w, inp)
    dq, dk, dv = run_bwd(lib, w, inp, d_out, bm)
    rows = np.array([0, 1, 128, 2047, 4095])
    for b, h in ((0, 0), (2, 9)):
        ref_dq, _, _ = oracle_bwd(w, inp, d_out, batches=[b], heads=[h], rows=rows)
        check(dq[b, h, rows], ref_dq[b, h, rows], f"dq[{b},{h}]")
    _, ref_dk, ref_dv = oracle_bwd(w, inp, d_out, batches=[0], heads=[8, 9, 10, 11])
    check(dk[0, 2], ref_dk[0, 2], "dk[0,2]")
    check(dv[0, 2], ref_dv[0, 2], "dv[0,2]")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("which", ["k", "v", "q_dout"])
def test_rows_broadcast_with_zero_stride(lib, D, which):
    """A tensor broadcast along the sequence (row stride 0, as torch's expand
    gives) reads its one row for every position: the forward and the backward
    match the same call on a contiguous copy, bit for bit."""
    w = tiny(D, "causal", "none", B=1, Hq=4, Hkv=2, Q_LEN=300, KV_LEN=300)
    inp = W.generate(w)
    g = W.generate_upstream(w)
    dev = lambda x: G.to_device(x, "bf16")  # noqa: E731
    q, k, v, gd = dev(inp.q), dev(inp.k), dev(inp.v), dev(g)
    bcast = lambda t: t[:, :, :1].expand(-1, -1, t.shape[2], -1)  # noqa: E731
    if which == "k":
        k = bcast(k)
    elif which == "v":
        v = bcast(v)
    else:
        q, gd = bcast(q), bcast(gd)
    bm = mask_of(lib, w, inp)
    got = [lib.flex_attention(q, k, v, bm)]
    got.append(lib.flex_attention_backward(q, k, v, got[0][1], gd, bm))
    qc, kc, vc, gc = (t.contiguous() for t in (q, k, v, gd))
    ref = [lib.flex_attention(qc, kc, vc, bm)]
    ref.append(lib.flex_attention_backward(qc, kc, vc, ref[0][1], gc, bm))
    torch.cuda.synchronize()
    for a, b, n in zip(got[0] + got[1], ref[0] + ref[1], ("out", "lse", "dq", "dk", "dv")):
        assert torch.equal(a, b), n
