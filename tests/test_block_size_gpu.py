"""BLOCK_SIZE 256, 384 and 512 (square tiles that are multiples of the
kernels' 128): the builder's tensors bit-exact against the oracle's builder
at that block size, and the forwards (fp32, bf16, fp16; split-KV and paged)
against the fp64 oracle, and the backward. from_kv_blocks takes 128 only."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_helpers as G
from tests.test_block_mask_gpu import expected_schedule
from tests.test_fwd_gpu import tiny

pytestmark = pytest.mark.gpu

KINDS = ["noop", "causal", "sliding_sink", "document_causal", "prefix_lm", "composite"]
TERMS = (("causal", "window"), ("prefix",), ("causal", "document"))


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_masked_amd as m
    m.load_library()
    return m


def build(lib, w, inp, block, **kw):
    doc = torch.from_numpy(inp.doc_ids.astype(np.int32)) if inp.doc_ids is not None else None
    return lib.create_block_mask(w.mask, 1, 1, w.Q_LEN, w.KV_LEN, block, window=w.window,
                                 num_sinks=w.sinks, doc_ids=doc, prefix_len=w.prefix,
                                 terms=w.terms, **kw)


@pytest.mark.parametrize("block", [256, 384, 512])
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("q_len,kv_len", [(300, 300), (1000, 700), (129, 1500), (1500, 1024)])
def test_block_size_builder_bit_exact(lib, block, kind, q_len, kv_len):
    w = tiny("bf16", 64, kind, "none", Q_LEN=q_len, KV_LEN=kv_len, window=300, sinks=3,
             prefix=200, doc_seed=q_len, doc_len_range=(50, 400),
             terms=TERMS if kind == "composite" else None)
    inp = W.generate(w)
    mask_mod, _ = oracle.for_workload(w, inp)
    ref = oracle.create_block_mask(mask_mod, 1, 1, q_len, kv_len, block)
    bm = build(lib, w, inp, block, backward_lists=True)
    torch.cuda.synchronize()
    for got, want in ((bm.kv_num_blocks, ref.kv_num_blocks), (bm.kv_indices, ref.kv_indices),
                      (bm.full_kv_num_blocks, ref.full_kv_num_blocks),
                      (bm.full_kv_indices, ref.full_kv_indices)):
        assert np.array_equal(got.cpu().numpy(), want)
    assert np.array_equal(bm.schedule.cpu().numpy(),
                          expected_schedule(ref.kv_num_blocks, ref.full_kv_num_blocks))
    for got, want in zip((bm.q_num_blocks, bm.q_indices, bm.full_q_num_blocks, bm.full_q_indices),
                         oracle.transpose_block_mask(ref)):
        assert np.array_equal(got.cpu().numpy(), want)


@pytest.mark.parametrize("block", [256, 512])
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 64), ("f32", 64), ("bf16", 256)])
@pytest.mark.parametrize("kind", ["causal", "sliding_sink", "document_causal", "composite"])
def test_block_size_forward(lib, block, dtype, D, kind):
    w = tiny(dtype, D, kind, "softcap_alibi" if dtype != "f32" else "alibi", Q_LEN=700,
             KV_LEN=900, window=300, sinks=3, prefix=200, doc_seed=5, doc_len_range=(50, 400),
             terms=TERMS if kind == "composite" else None,
             value_scale=2.0 if dtype != "f32" else 1.0)
    inp = W.generate(w)
    bm = build(lib, w, inp, block)
    o, lse, _ = G.run_gpu(lib, w, inp, bm)
    o_ref, lse_ref = G.oracle_rows(w, inp)
    res = G.compare(w, o, lse, o_ref, lse_ref)
    assert res["ok"], G.summary(res)


@pytest.mark.parametrize("block", [256, 384])
@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("q_len", [40, 12])
def test_block_size_split_and_paged(lib, block, splits, q_len):
    """Q_LEN = 12 runs the 16-row step; the other 128-row pieces of the
    query tile lie past Q_LEN and exit at once."""
    w = tiny("bf16", 128, "sliding_sink", "alibi", B=2, Hq=8, Hkv=2, Q_LEN=q_len, KV_LEN=1700,
             window=600, sinks=3)
    inp = W.generate(w)
    bm = build(lib, w, inp, block)
    q, k, v = (G.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    kc, vc, table = W.paged_cache(inp.k, inp.v, 256, seed=block)
    o_ref, lse_ref = G.oracle_rows(w, inp)
    for kk, vv, pt in ((k, v, None), (G.to_device(kc, "bf16"), G.to_device(vc, "bf16"),
                                      torch.from_numpy(table).cuda())):
        out, lse = lib.flex_attention(q, kk, vv, bm, score="alibi", scale=w.scale,
                                      num_splits=splits, page_table=pt)
        torch.cuda.synchronize()
        res = G.compare(w, out.float().cpu().numpy().astype(np.float64),
                        lse.cpu().numpy().astype(np.float64), o_ref, lse_ref)
        assert res["ok"], G.summary(res)


def test_block_size_rejections(lib):
    with pytest.raises(NotImplementedError, match="block"):
        lib.create_block_mask("causal", 1, 1, 512, 512, 192)


@pytest.mark.parametrize("block", [256, 512])
@pytest.mark.parametrize("kind,score", [("causal", "softcap"), ("document_causal", "alibi"),
                                        ("sliding_sink", "none"), ("composite", "softcap_alibi")])
def test_block_size_backward(lib, block, kind, score):
    """The backward walks the 128 x 128 pieces of the larger tiles (dQ over
    each row's key pieces, dK/dV over each column's query pieces)."""
    from tests.test_bwd_gpu import tiny as btiny, check, oracle_bwd, run_bwd
    w = btiny(128 if block == 256 else 64, kind, score, Q_LEN=650, KV_LEN=700, window=250,
              sinks=3, prefix=100, doc_seed=3, doc_len_range=(60, 300),
              terms=TERMS if kind == "composite" else None,
              value_scale=2.0 if "softcap" in score else 1.0)
    inp = W.generate(w)
    d_out = W.generate_upstream(w)
    bm = build(lib, w, inp, block, backward_lists=True)
    got = run_bwd(lib, w, inp, d_out, bm)
    ref = oracle_bwd(w, inp, d_out)
    for g, r, n in zip(got, ref, ("dq", "dk", "dv")):
        check(g, r, n)


@pytest.mark.parametrize("blocks", [(256, 128), (128, 256), (512, 256), (128, 384)])
@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("q_len,kv_len", [(300, 300), (1000, 700), (129, 1500)])
def test_non_square_builder_bit_exact(lib, blocks, kind, q_len, kv_len):
    """BLOCK_SIZE as the page's tuple (KV_BLOCK_SIZE, Q_BLOCK_SIZE)."""
    w = tiny("bf16", 64, kind, "none", Q_LEN=q_len, KV_LEN=kv_len, window=300, sinks=3,
             prefix=200, doc_seed=q_len, doc_len_range=(50, 400),
             terms=TERMS if kind == "composite" else None)
    inp = W.generate(w)
    mask_mod, _ = oracle.for_workload(w, inp)
    ref = oracle.create_block_mask(mask_mod, 1, 1, q_len, kv_len, blocks)
    bm = build(lib, w, inp, blocks, backward_lists=True)
    torch.cuda.synchronize()
    assert bm.BLOCK_SIZE == blocks[0] and bm.q_block == blocks[1]
    for got, want in ((bm.kv_num_blocks, ref.kv_num_blocks), (bm.kv_indices, ref.kv_indices),
                      (bm.full_kv_num_blocks, ref.full_kv_num_blocks),
                      (bm.full_kv_indices, ref.full_kv_indices)):
        assert np.array_equal(got.cpu().numpy(), want)
    for got, want in zip((bm.q_num_blocks, bm.q_indices, bm.full_q_num_blocks, bm.full_q_indices),
                         oracle.transpose_block_mask(ref)):
        assert np.array_equal(got.cpu().numpy(), want)


@pytest.mark.parametrize("blocks", [(256, 128), (128, 384)])
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64), ("f16", 256)])
@pytest.mark.parametrize("kind", ["causal", "document_causal", "composite"])
def test_non_square_forward(lib, blocks, dtype, D, kind):
    w = tiny(dtype, D, kind, "alibi", Q_LEN=700, KV_LEN=900, window=300, sinks=3, prefix=200,
             doc_seed=5, doc_len_range=(50, 400), terms=TERMS if kind == "composite" else None)
    inp = W.generate(w)
    bm = build(lib, w, inp, blocks)
    o, lse, _ = G.run_gpu(lib, w, inp, bm)
    o_ref, lse_ref = G.oracle_rows(w, inp)
    res = G.compare(w, o, lse, o_ref, lse_ref)
    assert res["ok"], G.summary(res)


@pytest.mark.parametrize("blocks", [(256, 128), (128, 256)])
def test_non_square_backward(lib, blocks):
    from tests.test_bwd_gpu import tiny as btiny, check, oracle_bwd, run_bwd
    w = btiny(64, "sliding_sink", "softcap", Q_LEN=650, KV_LEN=700, window=250, sinks=3,
              value_scale=2.0)
    inp = W.generate(w)
    d_out = W.generate_upstream(w)
    bm = build(lib, w, inp, blocks, backward_lists=True)
    got = run_bwd(lib, w, inp, d_out, bm)
    ref = oracle_bwd(w, inp, d_out)
    for g, r, n in zip(got, ref, ("dq", "dk", "dv")):
        check(g, r, n)
