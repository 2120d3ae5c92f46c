"""Host logic of the automatic split count (no GPU): the head packs per
workgroup follow the launcher's rule (exact packs of 4 or 2 heads of one KV
group, else partial packs at head dims up to 128), and the count targets 512
workgroups, at most 64 slices and at most the KV tiles of a row."""
import math

import pytest
import torch

import block_sparse_masked_amd as fa


def _bm(M, N, H=1, block=128):
    nq, nk = math.ceil(M / block), math.ceil(N / block)
    z = torch.zeros(1, H, nq, dtype=torch.int32)
    zi = torch.zeros(1, H, nq, nk, dtype=torch.int32)
    return fa.BlockMask("noop", 1, H, M, N, block, z, zi, z, zi,
                        torch.zeros(nq * H, dtype=torch.int32), None, None)


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
