"""BlockMask inspection helpers (to_dense, sparsity, to_string) on lists
held in host tensors: they only read the lists, so the oracle's lists stand
in for the builder's."""
import numpy as np
import torch

import block_sparse_masked_amd as lib
import oracle


def host_mask(mod, B, H, Q_LEN, KV_LEN, kind="test"):
    ref = oracle.create_block_mask(mod, B, H, Q_LEN, KV_LEN, 128)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))  # noqa: E731
    bm = lib.BlockMask(kind, B, H, Q_LEN, KV_LEN, 128, t(ref.kv_num_blocks), t(ref.kv_indices),
                       t(ref.full_kv_num_blocks), t(ref.full_kv_indices),
                       torch.zeros(1, dtype=torch.int32), None, lib._BlockMask())
    return bm, ref


def test_to_dense_and_sparsity_match_the_oracle():
    bm, ref = host_mask(oracle.sliding_sink_mask(300, 4), 1, 2, 1000, 1000)
    dense = bm.to_dense()
    part = oracle.to_dense(ref.kv_num_blocks, ref.kv_indices, 8)
    full = oracle.to_dense(ref.full_kv_num_blocks, ref.full_kv_indices, 8)
    assert np.array_equal(dense, part + 2 * full)
    assert abs(bm.sparsity() - ref.sparsity()) < 1e-12


def test_to_string_causal_picture():
    """Causal 512 x 512 (4 x 4 tiles): full below the diagonal, partial on
    it, empty above; uncompressed and compressed to 2 x 2 cells."""
    bm, _ = host_mask(oracle.causal_mask, 1, 1, 512, 512, kind="causal")
    lines = bm.to_string(grid_size=-1).splitlines()
    assert lines[2:] == ["+...", "#+..", "##+.", "###+"]
    assert "sparsity=37.50%" in lines[0]
    small = bm.to_string(grid_size=(2, 2)).splitlines()
    assert small[2:] == ["+.", "#+"]


def test_to_string_limit():
    bm, _ = host_mask(oracle.causal_mask, 2, 3, 256, 256)
    text = bm.to_string(limit=2)
    assert text.count("(b=") == 2 and "4 more" in text
