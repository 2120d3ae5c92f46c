"""The allocation-free split-KV forward (flexattn_fwd_splitkv_noalloc,
partials in the library's per-GPU scratch) through the C ABI, against the
workspace entry point flexattn_fwd_splitkv on the same inputs: two calls in
a row, the second smaller, each bit-identical to the workspace call (the
same kernels) and within the bf16 bounds of the oracle."""
import numpy as np
import pytest
import torch

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


CASES = [
    # B, Hq, Hkv, Q_LEN, KV_LEN, D, mask, score, splits: the second is smaller
    (4, 16, 4, 16, 9000, 128, "sliding_sink", "softcap_alibi", 8),
    (1, 4, 2, 5, 1500, 64, "causal", "alibi", 3),
]


def test_noalloc_matches_workspace_entry(lib):
    for B, Hq, Hkv, M, N, D, mask, score, splits in CASES:
        print(f"noalloc case B={B} Hq={Hq} Hkv={Hkv} M={M} N={N} D={D} {mask} {score} "
              f"splits={splits}", flush=True)
        w = W.Workload(f"noalloc_{M}_{N}", B=B, Hq=Hq, Hkv=Hkv, Q_LEN=M, KV_LEN=N, D=D,
                       dtype="bf16", seed=31 + M, mask=mask, window=700, sinks=4, score=score,
                       softcap=30.0, value_scale=2.0 if "softcap" in score else 1.0)
        inp = W.generate(w)
        q, k, v = (G.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
        bm = G.build_gpu_mask(lib, w, inp)
        ref_out, ref_lse = lib.flex_attention(q, k, v, bm, score=w.score, softcap=w.softcap,
                                              scale=w.scale, num_splits=splits)
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
        lib.flex_attention_noalloc(q, k, v, bm, out, lse, splits, score=w.score,
                                   softcap=w.softcap, scale=w.scale)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
        o_ref, lse_ref = G.oracle_rows(w, inp)
        res = G.compare(w, out.float().cpu().numpy().astype(np.float64),
                        lse.cpu().numpy().astype(np.float64), o_ref, lse_ref)
        assert res["ok"], G.summary(res)


def test_noalloc_rejects_oversized_partials(lib):
    w = W.Workload("noalloc_big", B=8, Hq=32, Hkv=8, Q_LEN=64, KV_LEN=4096, D=128,
                   dtype="bf16", seed=3, mask="noop")
    q = torch.zeros((w.B, w.Hq, w.Q_LEN, w.D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((w.B, w.Hkv, w.KV_LEN, w.D), dtype=torch.bfloat16, device="cuda")
    bm = lib.create_block_mask("noop", 1, 1, w.Q_LEN, w.KV_LEN)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    with pytest.raises(ValueError, match="scratch"):
        lib.flex_attention_noalloc(q, k, k, bm, out, lse, 32)
