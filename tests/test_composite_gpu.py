"""Runtime mask composition (or_masks of and_masks of primitives) on the
GPU: BlockMask tensors bit-exact against the oracle's builder on the
composite element mask (sorted and unsorted document ids), compositions that
spell the fixed kinds give bit-identical BlockMasks and outputs, and the
forward (fp32, bf16, fp16) and backward match the fp64 oracle."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_helpers as G
from tests.test_block_mask_gpu import expected_schedule
from tests.test_bwd_gpu import check as check_grad
from tests.test_fwd_gpu import check_full, tiny

pytestmark = pytest.mark.gpu

COMPOSITIONS = {
    "sliding": [("causal", "window"), ("causal", "sink")],
    "doc_window": [("causal", "document", "window")],
    "prefix_local": [("prefix",), ("causal", "window")],
    "doc_bidir": [("document",)],
    "sink_and_window": [("window", "sink")],
    "four_terms": [("causal", "window"), ("sink",), ("prefix", "document"),
                   ("causal", "document")],
}


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_masked_amd as m
    m.load_library()
    return m


def doc_row(L_, seed, sorted_ids=True):
    rng = np.random.default_rng(seed)
    lens = []
    while sum(lens) < L_:
        lens.append(int(rng.integers(20, 200)))
    ids = np.repeat(np.arange(len(lens)), lens)[:L_].astype(np.int32)
    if not sorted_ids:
        ids = ids[rng.permutation(L_)]
    return ids


@pytest.mark.parametrize("name", sorted(COMPOSITIONS))
@pytest.mark.parametrize("q_len,kv_len", [(300, 300), (129, 700), (700, 129), (1000, 1000)])
@pytest.mark.parametrize("sorted_ids", [True, False])
def test_composite_block_mask_bit_exact(lib, name, q_len, kv_len, sorted_ids):
    terms = COMPOSITIONS[name]
    L_ = max(q_len, kv_len)
    doc = doc_row(L_, q_len + kv_len, sorted_ids)
    mod = oracle.composite_mask(terms, 150, 3, 60, doc)
    ref = oracle.create_block_mask(mod, 1, 1, q_len, kv_len, 128)
    bm = lib.create_block_mask("composite", 1, 1, q_len, kv_len, 128, window=150, num_sinks=3,
                               prefix_len=60, doc_ids=torch.from_numpy(doc), terms=terms,
                               backward_lists=True)
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


@pytest.mark.parametrize("kind,terms,kw", [
    ("sliding_sink", [("causal", "window"), ("causal", "sink")], {}),
    ("prefix_lm", [("causal",), ("prefix",)], {}),
    ("document_causal", [("causal", "document")], {}),
    ("noop", [()], {}),
    ("causal", [("causal",)], {}),
])
def test_composite_spelling_a_fixed_kind_is_identical(lib, kind, terms, kw):
    L_ = 900
    doc = torch.from_numpy(doc_row(L_, 5))
    common = dict(window=200, num_sinks=4, prefix_len=130, doc_ids=doc)
    a = lib.create_block_mask(kind, 1, 1, L_, L_, 128, **common)
    b = lib.create_block_mask("composite", 1, 1, L_, L_, 128, terms=terms, **common)
    torch.cuda.synchronize()
    for x, y in ((a.kv_num_blocks, b.kv_num_blocks), (a.kv_indices, b.kv_indices),
                 (a.full_kv_num_blocks, b.full_kv_num_blocks),
                 (a.full_kv_indices, b.full_kv_indices), (a.schedule, b.schedule)):
        assert torch.equal(x, y)
    rng = np.random.default_rng(1)
    q, k, v = (torch.from_numpy(rng.standard_normal((1, 2, L_, 128), dtype=np.float32))
               .to(torch.bfloat16).cuda() for _ in range(3))
    oa, la = lib.flex_attention(q, k, v, a, score="alibi")
    ob, lb = lib.flex_attention(q, k, v, b, score="alibi")
    torch.cuda.synchronize()
    # the same tiles and the same masked elements: the same arithmetic
    assert torch.equal(oa, ob) and torch.equal(la, lb)


@pytest.mark.parametrize("name", sorted(COMPOSITIONS))
@pytest.mark.parametrize("dtype,D,score", [("bf16", 128, "softcap_alibi"), ("bf16", 64, "none"),
                                           ("f16", 128, "alibi"), ("f32", 64, "alibi"),
                                           ("bf16", 256, "none")])
def test_composite_forward(lib, name, dtype, D, score):
    w = tiny(dtype, D, "composite", score, Q_LEN=520, KV_LEN=520, window=150, sinks=3, prefix=60,
             doc_seed=9, doc_len_range=(40, 200), terms=tuple(COMPOSITIONS[name]),
             value_scale=2.0 if "softcap" in score else 1.0,
             softcap=2.0 if dtype == "f32" else 20.0)
    check_full(lib, w)


@pytest.mark.parametrize("name", sorted(COMPOSITIONS))
def test_composite_forward_split_and_short(lib, name):
    w = tiny("bf16", 128, "composite", "alibi", B=2, Hq=8, Hkv=2, Q_LEN=40, KV_LEN=1500,
             window=300, sinks=3, prefix=60, doc_seed=9, doc_len_range=(40, 400),
             terms=tuple(COMPOSITIONS[name]))
    inp = W.generate(w)
    bm = G.build_gpu_mask(lib, w, inp)
    q, k, v = (G.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    out, lse = lib.flex_attention(q, k, v, bm, score=w.score, scale=w.scale, num_splits=None)
    torch.cuda.synchronize()
    o_ref, lse_ref = G.oracle_rows(w, inp)
    res = G.compare(w, out.float().cpu().numpy().astype(np.float64),
                    lse.cpu().numpy().astype(np.float64), o_ref, lse_ref)
    assert res["ok"], G.summary(res)


@pytest.mark.parametrize("name", ["doc_window", "prefix_local", "doc_bidir", "four_terms"])
@pytest.mark.parametrize("D,score", [(128, "softcap"), (64, "alibi")])
def test_composite_backward(lib, name, D, score):
    from tests.test_bwd_gpu import tiny as btiny, full_check
    w = btiny(D, "composite", score, Q_LEN=400, KV_LEN=400, window=150, sinks=3, prefix=60,
              doc_seed=9, doc_len_range=(40, 200), terms=tuple(COMPOSITIONS[name]),
              value_scale=2.0 if "softcap" in score else 1.0)
    full_check(lib, w)


def test_composite_rejections(lib):
    with pytest.raises(ValueError, match="1 to 4 terms"):
        lib.create_block_mask("composite", 1, 1, 256, 256, terms=[("causal",)] * 5)
    with pytest.raises(ValueError, match="unknown mask primitive"):
        lib.create_block_mask("composite", 1, 1, 256, 256, terms=[("dilated",)])
    with pytest.raises(ValueError, match="needs doc_ids"):
        lib.create_block_mask("composite", 1, 1, 256, 256, terms=[("document",)])
    with pytest.raises(ValueError, match="window"):
        lib.create_block_mask("composite", 1, 1, 256, 256, terms=[("window",)], window=0)
