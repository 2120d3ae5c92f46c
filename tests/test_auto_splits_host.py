"""Host logic of the launch plan (no GPU): flexattn_fwd_make_plan, the rule
the forward's launcher applies, called through the C ABI. The head packs per
workgroup are exact packs of 4 or 2 heads of one KV group, else partial packs
at head dims up to 128; the split count targets 512 workgroups, at most 64
slices and at most the KV tiles of a row."""
import math

import pytest
import torch

import block_sparse_masked_amd as fa


def _bm(M, N, H=1, block=128):
    """A BlockMask whose extents are set and whose device buffers are not
    (the plan reads only the extents)."""
    nq, nk = math.ceil(M / block), math.ceil(N / block)
    z = torch.zeros(1, H, nq, dtype=torch.int32)
    zi = torch.zeros(1, H, nq, nk, dtype=torch.int32)
    c = fa._BlockMask()
    c.B, c.H, c.Q_LEN, c.KV_LEN, c.BLOCK_SIZE = 1, H, M, N, block
    c.num_q_blocks, c.num_kv_blocks, c.Q_BLOCK_SIZE = nq, nk, block
    return fa.BlockMask("noop", 1, H, M, N, block, z, zi, z, zi,
                        torch.zeros(nq * H, dtype=torch.int32), None, c)


def _splits(B, Hq, Hkv, M, N, D=128, H=1):
    q = torch.empty(B, Hq, M, D, dtype=torch.bfloat16)
    k = torch.empty(B, Hkv, 1, D, dtype=torch.bfloat16)
    return fa.auto_splits(q, k, _bm(M, N, H))


@pytest.mark.parametrize("B,Hq,Hkv,M,N,D,H,want", [
    (8, 32, 8, 16, 32768, 128, 1, 8),     # G = 4: 4 heads a workgroup, 64 items
    (8, 28, 4, 16, 32768, 128, 1, 8),     # G = 7: packs of 4 + 3, 64 items
    (8, 28, 4, 16, 32768, 256, 1, 2),     # G = 7 at D = 256: one head a workgroup
    (8, 16, 8, 16, 32768, 128, 1, 8),     # G = 2: 2 heads of 2 waves, 64 items
    (8, 32, 32, 1, 8192, 128, 1, 1),      # G = 1: 256 items already fill the chip
    (1, 32, 8, 1, 131072, 128, 1, 64),    # 8 items: capped at 64 slices
    (1, 32, 8, 16, 300, 128, 1, 3),       # capped at the row's 3 KV tiles
    (8, 32, 8, 16, 32768, 128, 32, 1),    # per-head mask: no packing, 256 items: no split
    (4, 32, 8, 16, 32768, 128, 32, 4),    # per-head mask, 128 items
    (2, 16, 4, 4096, 4096, 128, 1, 1),    # many query tiles: no split
])
def test_auto_splits(B, Hq, Hkv, M, N, D, H, want):
    assert _splits(B, Hq, Hkv, M, N, D, H) == want


def test_auto_splits_is_one_for_fp32():
    q = torch.empty(1, 4, 16, 64)
    k = torch.empty(1, 4, 1, 64)
    assert fa.auto_splits(q, k, _bm(16, 4096)) == 1


@pytest.mark.parametrize("B,Hq,Hkv,M,D,H,wph,hpw,row16,items", [
    (8, 32, 8, 16, 128, 1, 1, 4, 1, 64),      # decode, G = 4: 16-row step
    (8, 32, 8, 40, 128, 1, 2, 2, 0, 128),     # 40 queries: two waves a head
    (8, 28, 4, 16, 128, 1, 1, 4, 1, 64),      # G = 7: packs of 4 + 3
    (8, 28, 4, 16, 256, 1, 4, 1, 0, 224),     # head dim 256: no partial packs
    (4, 16, 4, 4096, 128, 1, 4, 1, 0, 2048),  # dense causal workload
    (8, 32, 8, 16, 128, 32, 4, 1, 0, 256),    # per-head mask: no packing
])
def test_plan_fields(B, Hq, Hkv, M, D, H, wph, hpw, row16, items):
    q = torch.empty(B, Hq, M, D, dtype=torch.bfloat16)
    k = torch.empty(B, Hkv, 1, D, dtype=torch.bfloat16)
    p = fa.fwd_plan(q, k, _bm(M, 4096, H))
    assert (p["waves_per_head"], p["heads_per_workgroup"], p["row16"], p["work_items"]) == (
        wph, hpw, row16, items)


def test_plan_rejects_mismatched_mask():
    q = torch.empty(1, 4, 16, 64, dtype=torch.bfloat16)
    k = torch.empty(1, 4, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fwd_plan(q, k, _bm(32, 4096))


def test_plan_fp32_workgroups():
    """The fp32 forward runs one workgroup per 8 query rows of each (b, h)
    and does not split."""
    q = torch.empty(2, 3, 300, 64)
    k = torch.empty(2, 3, 1, 64)
    p = fa.fwd_plan(q, k, _bm(300, 4096))
    assert (p["waves_per_head"], p["num_splits"], p["work_items"]) == (0, 1, 2 * 3 * 3 * 128 // 8)
