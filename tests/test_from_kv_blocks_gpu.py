"""BlockMask from caller-given tile lists (from_kv_blocks) on the GPU: the
schedule and backward lists bit-exact, forward and backward against the fp64
oracle with the element mask the lists stand for, round trip with
create_block_mask, and the list checks."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests import gpu_helpers as G
from tests.test_block_mask_gpu import expected_schedule
from tests.test_bwd_gpu import check as check_grad

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_masked_amd as m
    m.load_library()
    return m


def random_lists(B, H, nqb, nkb, seed, p_tile=0.4, p_full=0.5, q_tail=True, kv_tail=True):
    """Random ascending, disjoint partial / full lists; tiles on a ragged
    tail (the last row / column when q_tail / kv_tail) are only partial."""
    rng = np.random.default_rng(seed)
    kv_num = np.zeros((B, H, nqb), np.int32)
    kv_idx = np.zeros((B, H, nqb, nkb), np.int32)
    fn = np.zeros((B, H, nqb), np.int32)
    fi = np.zeros((B, H, nqb, nkb), np.int32)
    for pos in np.ndindex(B, H, nqb):
        tiles = np.nonzero(rng.random(nkb) < p_tile)[0]
        full = tiles[rng.random(len(tiles)) < p_full]
        if q_tail and pos[2] == nqb - 1:
            full = full[:0]
        if kv_tail:
            full = full[full != nkb - 1]
        part = np.setdiff1d(tiles, full)
        kv_num[pos], fn[pos] = len(part), len(full)
        kv_idx[pos + (slice(0, len(part)),)] = part
        fi[pos + (slice(0, len(full)),)] = full
    return kv_num, kv_idx, fn, fi


@pytest.mark.parametrize("kind", ["noop", "causal"])
@pytest.mark.parametrize("B_mask,H_mask", [(1, 1), (2, 4)])
def test_from_kv_blocks_forward_backward(lib, kind, B_mask, H_mask):
    """Random lists (tail tiles on both axes, 3 x 3 tiles) in every derived
    tensor and in the attention they select, forward and backward."""
    Q_LEN, KV_LEN = 300, 300
    w = W.Workload("fkb", B=2, Hq=4, Hkv=2, Q_LEN=Q_LEN, KV_LEN=KV_LEN, D=128, dtype="bf16",
                   seed=3, mask="noop", score="alibi")
    inp = W.generate(w)
    lists = random_lists(B_mask, H_mask, 3, 3, seed=B_mask * 10 + H_mask + (kind == "causal"))
    bm = lib.block_mask_from_kv_blocks(*(torch.from_numpy(x).cuda() for x in lists),
                                       Q_LEN=Q_LEN, KV_LEN=KV_LEN, kind=kind, backward_lists=True)
    torch.cuda.synchronize()
    assert int(bm.status.item()) == 0
    assert np.array_equal(bm.schedule.cpu().numpy(), expected_schedule(lists[0], lists[2]))
    ref_bm = oracle.BlockMask(Q_LEN, KV_LEN, 128, *lists, tile_counts=None)
    for g, e in zip((bm.q_num_blocks, bm.q_indices, bm.full_q_num_blocks, bm.full_q_indices),
                    oracle.transpose_block_mask(ref_bm)):
        assert np.array_equal(g.cpu().numpy(), e)
    mm = oracle.from_kv_blocks_mask(*lists, 128, oracle.mask_mod_for(kind))
    score = oracle.score_mod_for("alibi", w.Hq)
    q, k, v = (G.to_device(x, "bf16") for x in (inp.q, inp.k, inp.v))
    out, lse = lib.flex_attention(q, k, v, bm, score="alibi", scale=w.scale)
    g = W.generate_upstream(w)
    dq, dk, dv = lib.flex_attention_backward(q, k, v, lse, G.to_device(g, "bf16"), bm,
                                             score="alibi", scale=w.scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(inp.q, inp.k, inp.v, mm, score, w.scale)
    res = G.compare(w, out.float().cpu().numpy().astype(np.float64),
                    lse.cpu().numpy().astype(np.float64), o_ref, lse_ref)
    assert res["ok"], G.summary(res)
    ref = oracle.attention_backward(inp.q, inp.k, inp.v, g, mm, score, None, w.scale)
    for t, r, n in zip((dq, dk, dv), ref, ("dq", "dk", "dv")):
        check_grad(t.float().cpu().numpy().astype(np.float64), r, n)


def test_from_kv_blocks_round_trip(lib):
    """Lists made by create_block_mask, handed back with the same mask kind,
    give the same schedule, backward lists and (bit-identical) forward."""
    L = 1000
    a = lib.create_block_mask("sliding_sink", 1, 1, L, L, 128, window=300, num_sinks=4,
                              backward_lists=True)
    b = lib.block_mask_from_kv_blocks(a.kv_num_blocks, a.kv_indices, a.full_kv_num_blocks,
                                      a.full_kv_indices, Q_LEN=L, KV_LEN=L, kind="sliding_sink",
                                      window=300, num_sinks=4, backward_lists=True)
    torch.cuda.synchronize()
    for x, y in ((a.schedule, b.schedule), (a.q_num_blocks, b.q_num_blocks),
                 (a.q_indices, b.q_indices), (a.full_q_num_blocks, b.full_q_num_blocks),
                 (a.full_q_indices, b.full_q_indices)):
        assert torch.equal(x, y)
    rng = np.random.default_rng(0)
    q, k, v = (torch.from_numpy(rng.standard_normal((1, 2, L, 64), dtype=np.float32))
               .to(torch.bfloat16).cuda() for _ in range(3))
    oa, la = lib.flex_attention(q, k, v, a)
    ob, lb = lib.flex_attention(q, k, v, b)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob) and torch.equal(la, lb)


@pytest.mark.parametrize("case,flag", [("count", 1), ("index", 2), ("order", 4), ("overlap", 8),
                                       ("full_tail", 16)])
def test_from_kv_blocks_checks(lib, case, flag):
    """Each kind of bad list sets its flag (and raises with validate=True)."""
    kv_num, kv_idx, fn, fi = random_lists(1, 1, 3, 3, seed=5, p_tile=1.0, p_full=0.0)
    if case == "count":
        kv_num[0, 0, 1] = 4
    elif case == "index":
        kv_idx[0, 0, 0, 1] = 7
    elif case == "order":
        kv_idx[0, 0, 2, :2] = [2, 1]
    elif case == "full_tail":
        kv_num[0, 0, 0] = 2                     # tiles 0, 1 partial; tile 2 full
        fn[0, 0, 0] = 1
        fi[0, 0, 0, 0] = 2
    else:
        fn[0, 0, 0] = 1
        fi[0, 0, 0, 0] = kv_idx[0, 0, 0, 0]
    args = [torch.from_numpy(x).cuda() for x in (kv_num, kv_idx, fn, fi)]
    kw = {"KV_LEN": 300} if case == "full_tail" else {}
    bm = lib.block_mask_from_kv_blocks(*args, validate=False, backward_lists=True, **kw)
    torch.cuda.synchronize()
    assert int(bm.status.item()) & flag
    with pytest.raises(RuntimeError, match="invalid kv block lists"):
        lib.block_mask_from_kv_blocks(*args, **kw)


def test_from_kv_blocks_shape_errors(lib):
    with pytest.raises(RuntimeError):
        lib.block_mask_from_kv_blocks(torch.zeros((1, 1, 3), dtype=torch.int32, device="cuda"),
                                      torch.zeros((1, 1, 2, 3), dtype=torch.int32, device="cuda"))
