"""Forward over a paged KV cache on the GPU: against the fp64 oracle on the
keys gathered through the page table, bit-identical to the contiguous
forward on the same keys, with and without split-KV. Unused cache rows are
NaN, so a read outside a sequence would show in the output."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_helpers as G
from tests.test_fwd_gpu import tiny

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_masked_amd as m
    m.load_library()
    return m


def paged_inputs(w, page, seed=11):
    inp = W.generate(w)
    kc, vc, table = W.paged_cache(inp.k, inp.v, page, seed=seed)
    dev = lambda x: G.to_device(x, "bf16")  # noqa: E731
    return inp, dev(inp.q), dev(kc), dev(vc), torch.from_numpy(table).cuda(), (kc, vc, table)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("mask,score", [("noop", "none"), ("causal", "alibi"),
                                        ("sliding_sink", "softcap"),
                                        ("document_causal", "softcap_alibi"),
                                        ("prefix_lm", "none")])
@pytest.mark.parametrize("q_len,kv_len,page", [(300, 300, 128), (16, 1000, 256),
                                               (130, 900, 384)])
@pytest.mark.parametrize("splits", [1, 3])
def test_paged_against_oracle(lib, D, mask, score, q_len, kv_len, page, splits):
    w = tiny("bf16", D, mask, score, B=2, Hq=4, Hkv=2, Q_LEN=q_len, KV_LEN=kv_len,
             window=150, prefix=60, value_scale=2.0 if "softcap" in score else 1.0)
    inp, q, kc, vc, table, host = paged_inputs(w, page)
    # the oracle reads the keys through the page table
    kc_h, vc_h, table_h = host
    assert np.array_equal(oracle.gather_paged(kc_h, table_h, kv_len), inp.k)
    bm = G.build_gpu_mask(lib, w, inp)
    out, lse = lib.flex_attention(q, kc, vc, bm, score=w.score, softcap=w.softcap, scale=w.scale,
                                  num_splits=splits, page_table=table)
    torch.cuda.synchronize()
    mask_mod, score_mod = oracle.for_workload(w, inp)
    o_ref, lse_ref = oracle.attention(inp.q, oracle.gather_paged(kc_h, table_h, kv_len),
                                      oracle.gather_paged(vc_h, table_h, kv_len), mask_mod,
                                      score_mod, w.scale)
    res = G.compare(w, out.float().cpu().numpy().astype(np.float64),
                    lse.cpu().numpy().astype(np.float64), o_ref, lse_ref)
    assert res["ok"], G.summary(res)


@pytest.mark.parametrize("splits", [1, 4])
def test_paged_matches_contiguous_bitwise(lib, splits):
    """Same keys, same tiles, same arithmetic: the paged forward's O and LSE
    equal the contiguous forward's bit for bit."""
    w = tiny("bf16", 128, "sliding_sink", "alibi", B=3, Hq=8, Hkv=2, Q_LEN=200, KV_LEN=1500,
             window=400)
    inp, q, kc, vc, table, _ = paged_inputs(w, 256, seed=3)
    k, v = G.to_device(inp.k, "bf16"), G.to_device(inp.v, "bf16")
    bm = G.build_gpu_mask(lib, w, inp)
    o1, l1 = lib.flex_attention(q, k, v, bm, score="alibi", scale=w.scale, num_splits=splits)
    o2, l2 = lib.flex_attention(q, kc, vc, bm, score="alibi", scale=w.scale, num_splits=splits,
                                page_table=table)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_rejections(lib):
    w = tiny("bf16", 64, "noop", "none", B=1, Hq=2, Hkv=1, Q_LEN=128, KV_LEN=300)
    inp, q, kc, vc, table, _ = paged_inputs(w, 128)
    bm = G.build_gpu_mask(lib, w, inp)
    with pytest.raises(ValueError, match="do not cover"):
        lib.flex_attention(q, kc, vc, bm, page_table=table[:, :2].contiguous())
    k64 = torch.zeros((kc.shape[0] * 2, kc.shape[1], 64, kc.shape[3]), dtype=kc.dtype,
                      device=kc.device)
    with pytest.raises(NotImplementedError, match="multiple of 128"):
        lib.flex_attention(q, k64, k64, bm, page_table=table)
    with pytest.raises(NotImplementedError, match="bf16"):
        lib.flex_attention(q.float(), kc.float(), vc.float(), bm, page_table=table)


def test_paged_decode_workload_sampled(lib):
    """The decode workload at full size (B=8, Hq=32, Hkv=8, 16 queries, 32768
    keys) read through a paged cache (pages of 256 keys at a seeded random
    placement) with the automatic split count: sampled heads against the
    oracle on the contiguous keys the pages hold."""
    w = W.DECODE_GQA
    inp = W.generate(w)
    kc, vc, table = W.paged_cache(inp.k, inp.v, 256, seed=w.seed)
    for b, j in ((0, 0), (5, 77), (7, 127)):  # a few pages hold the sequence's keys
        assert np.array_equal(kc[table[b, j], :, :], inp.k[b, :, 256 * j:256 * j + 256])
    q = G.to_device(inp.q, "bf16")
    kd, vd = G.to_device(kc, "bf16"), G.to_device(vc, "bf16")
    del kc, vc
    bm = G.build_gpu_mask(lib, w, inp)
    out, lse = lib.flex_attention(q, kd, vd, bm, scale=w.scale, num_splits=None,
                                  page_table=torch.from_numpy(table).cuda())
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    l_ = lse.cpu().numpy().astype(np.float64)
    for b, h in ((0, 0), (4, 9), (7, 31)):
        o_ref, lse_ref = G.oracle_rows(w, inp, batches=[b], heads=[h])
        res = G.compare(w, o, l_, o_ref, lse_ref)
        assert res["ok"] and res["n_rows"] == w.Q_LEN, G.summary(res)


@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("mask,score", [("causal", "alibi"), ("sliding_sink", "softcap")])
@pytest.mark.parametrize("splits", [1, 3])
def test_paged_fp16_against_oracle(lib, D, mask, score, splits):
    """fp16 inputs through the paged cache: against the oracle on the
    gathered keys, and bit-identical to the contiguous fp16 forward."""
    w = tiny("f16", D, mask, score, B=2, Hq=4, Hkv=2, Q_LEN=300, KV_LEN=900, window=150,
             value_scale=2.0 if "softcap" in score else 1.0)
    inp = W.generate(w)
    kc_h, vc_h, table_h = W.paged_cache(inp.k, inp.v, 256, seed=5)
    q = G.to_device(inp.q, "f16")
    kc, vc = G.to_device(kc_h, "f16"), G.to_device(vc_h, "f16")
    table = torch.from_numpy(table_h).cuda()
    bm = G.build_gpu_mask(lib, w, inp)
    out, lse = lib.flex_attention(q, kc, vc, bm, score=w.score, softcap=w.softcap, scale=w.scale,
                                  num_splits=splits, page_table=table)
    k, v = G.to_device(inp.k, "f16"), G.to_device(inp.v, "f16")
    o2, l2 = lib.flex_attention(q, k, v, bm, score=w.score, softcap=w.softcap, scale=w.scale,
                                num_splits=splits)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2)
    mask_mod, score_mod = oracle.for_workload(w, inp)
    o_ref, lse_ref = oracle.attention(inp.q, oracle.gather_paged(kc_h, table_h, w.KV_LEN),
                                      oracle.gather_paged(vc_h, table_h, w.KV_LEN), mask_mod,
                                      score_mod, w.scale)
    res = G.compare(w, out.float().cpu().numpy().astype(np.float64),
                    lse.cpu().numpy().astype(np.float64), o_ref, lse_ref)
    assert res["ok"], G.summary(res)
