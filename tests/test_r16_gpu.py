"""The 16-row forward step (query tiles of at most 16 rows with the mask
broadcast over heads and four query heads per KV head or more) on the GPU:
against the fp64 oracle for every mask and score kind, paged and split-KV,
bf16 and fp16, head dims 64 and 128; and against the 32-row step on the same
inputs (a BlockMask built per query head selects that one)."""
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


def _run(lib, w, inp, splits, paged=None, f16=False, H_mask=1):
    dt = "f16" if f16 else "bf16"
    bm = G.build_gpu_mask(lib, w, inp, 1, H_mask)
    q = G.to_device(inp.q, dt)
    if paged is None:
        k, v = G.to_device(inp.k, dt), G.to_device(inp.v, dt)
        table = None
    else:
        kc, vc, tab = paged
        k, v, table = G.to_device(kc, dt), G.to_device(vc, dt), torch.from_numpy(tab).cuda()
    out, lse = lib.flex_attention(q, k, v, bm, score=w.score, softcap=w.softcap, scale=w.scale,
                                  num_splits=splits, page_table=table)
    torch.cuda.synchronize()
    return out, lse


def _check(w, inp, out, lse):
    o_ref, lse_ref = G.oracle_rows(w, inp)
    res = G.compare(w, out.float().cpu().numpy().astype(np.float64),
                    lse.cpu().numpy().astype(np.float64), o_ref, lse_ref)
    assert res["ok"], G.summary(res)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask,score", [("noop", "none"), ("causal", "alibi"),
                                        ("sliding_sink", "softcap_alibi"),
                                        ("document_causal", "softcap"),
                                        ("prefix_lm", "alibi")])
@pytest.mark.parametrize("q_len", [1, 7, 16])
@pytest.mark.parametrize("splits", [1, 5])
def test_r16_against_oracle(lib, D, mask, score, q_len, splits):
    """KV_LEN = 1000 ends inside a 64-key step; Q_LEN = 7 leaves 9 idle rows."""
    w = tiny("bf16", D, mask, score, B=2, Hq=8, Hkv=2, Q_LEN=q_len, KV_LEN=1000, window=300,
             prefix=40, value_scale=2.0 if "softcap" in score else 1.0)
    inp = W.generate(w)
    out, lse = _run(lib, w, inp, splits)
    _check(w, inp, out, lse)


@pytest.mark.parametrize("mask,score", [("sliding_sink", "alibi"), ("document_causal", "none")])
@pytest.mark.parametrize("splits", [1, 3])
def test_r16_paged(lib, mask, score, splits):
    w = tiny("bf16", 128, mask, score, B=2, Hq=8, Hkv=2, Q_LEN=16, KV_LEN=1100, window=300)
    inp = W.generate(w)
    kc, vc, table = W.paged_cache(inp.k, inp.v, 256, seed=4)
    assert np.array_equal(oracle.gather_paged(kc, table, w.KV_LEN), inp.k)
    out, lse = _run(lib, w, inp, splits, paged=(kc, vc, table))
    _check(w, inp, out, lse)


@pytest.mark.parametrize("splits", [1, 4])
def test_r16_fp16(lib, splits):
    w = tiny("f16", 128, "causal", "softcap_alibi", B=2, Hq=8, Hkv=2, Q_LEN=16, KV_LEN=1500,
             value_scale=2.0)
    inp = W.generate(w)
    out, lse = _run(lib, w, inp, splits, f16=True)
    _check(w, inp, out, lse)


@pytest.mark.parametrize("splits", [1, None])
def test_r16_composite(lib, splits):
    """(causal AND window) OR prefix OR (causal AND document): the composite
    mask on the 16-row step."""
    w = tiny("bf16", 128, "composite", "alibi", B=2, Hq=8, Hkv=2, Q_LEN=16, KV_LEN=1300,
             window=300, sinks=3, prefix=60, doc_seed=9, doc_len_range=(40, 400),
             terms=(("causal", "window"), ("prefix",), ("causal", "document")))
    inp = W.generate(w)
    out, lse = _run(lib, w, inp, splits)
    _check(w, inp, out, lse)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("splits", [1, 6])
def test_r16_matches_32_row_step(lib, D, splits):
    """The two steps reorder the same fp32 sums: outputs agree to a few bf16
    ulps and LSE to 1e-5 relative. A BlockMask built per query head keeps
    one head per workgroup and the 32-row step; the broadcast mask packs four
    heads per workgroup on the 16-row step."""
    w = tiny("bf16", D, "sliding_sink", "softcap_alibi", B=3, Hq=16, Hkv=4, Q_LEN=16,
             KV_LEN=2500, window=900, value_scale=2.0)
    inp = W.generate(w)
    o16, l16 = _run(lib, w, inp, splits)
    o32, l32 = _run(lib, w, inp, splits, H_mask=w.Hq)
    d = (o16.float() - o32.float()).abs()
    tol = 2.0 ** -7 * o32.float().abs() + 1e-3
    assert bool((d <= tol).all()), float(d.max())
    assert torch.equal(torch.isinf(l16), torch.isinf(l32))
    fin = torch.isfinite(l32)
    assert float(((l16 - l32)[fin].abs() / l32[fin].abs().clamp_min(1.0)).max()) < 1e-5


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("q_len", [16, 40, 64])
def test_ragged_head_packs_paged(lib, D, splits, q_len):
    """Seven query heads per KV head through a paged cache, with and without
    slices: packs of 4 + 3 on the 16-row step (16 queries), packs of 2 with
    two waves a head (40 and 64 queries)."""
    w = tiny("bf16", D, "sliding_sink", "softcap_alibi", B=2, Hq=14, Hkv=2, Q_LEN=q_len,
             KV_LEN=1100, window=300, value_scale=2.0)
    inp = W.generate(w)
    kc, vc, table = W.paged_cache(inp.k, inp.v, 256, seed=8)
    out, lse = _run(lib, w, inp, splits, paged=(kc, vc, table))
    _check(w, inp, out, lse)
