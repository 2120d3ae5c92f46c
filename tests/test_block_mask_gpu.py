"""GPU BlockMask builder vs the oracle: bit-exact on every index tensor."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_masked_amd as m
    m.load_library()  # raises if the HIP library is missing
    return m


def expected_schedule(kv_num, full_num):
    key = (kv_num + full_num).reshape(-1)
    return np.array(sorted(range(key.size), key=lambda i: (-int(key[i]), i)), dtype=np.int32)


def check(gpu_bm, ref):
    torch.cuda.synchronize()
    for name in ("kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices"):
        got = getattr(gpu_bm, name).cpu().numpy()
        exp = getattr(ref, name)
        assert got.shape == exp.shape, name
        assert np.array_equal(got, exp), (name, np.argwhere(got != exp)[:5])
    sched = gpu_bm.schedule.cpu().numpy()
    assert np.array_equal(sched, expected_schedule(ref.kv_num_blocks, ref.full_kv_num_blocks))


def doc_for(L, seed):
    rng = np.random.default_rng(seed)
    lens = []
    while sum(lens) < L:
        lens.append(int(rng.integers(1, 150)))
    return W.document_ids(lens)[:L]


SHAPES = [(1, 1), (127, 127), (128, 128), (129, 129), (255, 300), (300, 255), (383, 383),
          (512, 512), (1, 700), (700, 1)]


@pytest.mark.parametrize("q_len,kv_len", SHAPES)
@pytest.mark.parametrize("kind,window,sinks", [
    ("noop", 0, 0), ("causal", 0, 0), ("sliding_sink", 1, 0), ("sliding_sink", 128, 4),
    ("sliding_sink", 200, 0), ("sliding_sink", 200, 130), ("document_causal", 0, 0)])
def test_builder_tiny_grid(lib, q_len, kv_len, kind, window, sinks):
    doc = doc_for(max(q_len, kv_len), seed=q_len * 7 + kv_len) if kind == "document_causal" else None
    ref = oracle.create_block_mask(oracle.mask_mod_for(kind, window, sinks, doc), 1, 1,
                                   q_len, kv_len, 128)
    bm = lib.create_block_mask(kind, 1, 1, q_len, kv_len, 128, window=window, num_sinks=sinks,
                               doc_ids=None if doc is None else torch.from_numpy(doc))
    check(bm, ref)


@pytest.mark.parametrize("q_len,kv_len", [(1, 1), (129, 129), (300, 255), (512, 512), (700, 1)])
@pytest.mark.parametrize("kind,window,sinks", [
    ("noop", 0, 0), ("causal", 0, 0), ("sliding_sink", 200, 130), ("document_causal", 0, 0)])
def test_builder_unseparated(lib, q_len, kv_len, kind, window, sinks):
    """separate_full_blocks=False: every non-empty tile in the partial lists,
    bit-exact against the oracle built the same way."""
    doc = doc_for(max(q_len, kv_len), seed=q_len * 5 + kv_len) if kind == "document_causal" else None
    ref = oracle.create_block_mask(oracle.mask_mod_for(kind, window, sinks, doc), 1, 1,
                                   q_len, kv_len, 128, separate_full_blocks=False)
    bm = lib.create_block_mask(kind, 1, 1, q_len, kv_len, 128, window=window, num_sinks=sinks,
                               doc_ids=None if doc is None else torch.from_numpy(doc),
                               separate_full_blocks=False)
    check(bm, ref)


def test_builder_unseparated_full_workload(lib):
    """The dense causal workload's mask (32 x 32 tiles) without full tiles."""
    ref = oracle.create_block_mask(oracle.causal_mask, 1, 1, 4096, 4096, 128,
                                   separate_full_blocks=False)
    bm = lib.create_block_mask("causal", 1, 1, 4096, 4096, 128, separate_full_blocks=False)
    check(bm, ref)


def test_builder_batched_heads_broadcast(lib):
    """B=2, H=3 build of a (b, h)-independent mask equals the oracle's full build."""
    ref = oracle.create_block_mask(oracle.sliding_sink_mask(150, 3), 2, 3, 600, 600, 128)
    bm = lib.create_block_mask("sliding_sink", 2, 3, 600, 600, 128, window=150, num_sinks=3)
    check(bm, ref)


def test_builder_document_not_sorted(lib):
    """Document ids that are not contiguous runs take the per-element path."""
    rng = np.random.default_rng(5)
    doc = rng.integers(0, 3, size=520).astype(np.int32)
    ref = oracle.create_block_mask(oracle.document_causal_mask(doc), 1, 1, 520, 520, 128)
    bm = lib.create_block_mask("document_causal", 1, 1, 520, 520, 128,
                               doc_ids=torch.from_numpy(doc))
    check(bm, ref)


def test_builder_document_per_batch(lib):
    """Per-batch document ids: each batch row of the BlockMask uses its own ids."""
    d0 = doc_for(700, 1)
    d1 = doc_for(700, 2)
    both = np.stack([d0, d1])
    ref = oracle.create_block_mask(oracle.document_causal_mask(both), 2, 1, 700, 700, 128)
    bm = lib.create_block_mask("document_causal", 2, 1, 700, 700, 128,
                               doc_ids=torch.from_numpy(both))
    check(bm, ref)


def test_builder_document_long_runs(lib):
    """Runs much longer than a tile and a run starting before the search grid."""
    doc = W.document_ids([5000, 3, 2000, 129, 40])
    ref = oracle.create_block_mask(oracle.document_causal_mask(doc), 1, 1, len(doc), len(doc), 128)
    bm = lib.create_block_mask("document_causal", 1, 1, len(doc), len(doc), 128,
                               doc_ids=torch.from_numpy(doc))
    check(bm, ref)


@pytest.mark.parametrize("w", W.WORKLOADS, ids=[w.name for w in W.WORKLOADS])
def test_builder_full_workloads(lib, w):
    """The BlockMask of every measured workload, at full size, bit-exact."""
    inp_doc = None
    if w.mask == "document_causal":
        inp_doc = W.document_ids(W.document_lengths(w.Q_LEN, *w.doc_len_range, w.doc_seed))
    ref = oracle.create_block_mask(oracle.mask_mod_for(w.mask, w.window, w.sinks, inp_doc),
                                   1, 1, w.Q_LEN, w.KV_LEN, 128)
    bm = lib.create_block_mask(w.mask, 1, 1, w.Q_LEN, w.KV_LEN, 128, window=w.window,
                               num_sinks=w.sinks,
                               doc_ids=None if inp_doc is None else torch.from_numpy(inp_doc))
    check(bm, ref)


def test_builder_deterministic(lib):
    a = lib.create_block_mask("causal", 1, 1, 4096, 4096)
    b = lib.create_block_mask("causal", 1, 1, 4096, 4096)
    torch.cuda.synchronize()
    for name in ("kv_num_blocks", "kv_indices", "full_kv_num_blocks", "full_kv_indices", "schedule"):
        assert torch.equal(getattr(a, name), getattr(b, name))


@pytest.mark.parametrize("q_len,kv_len", SHAPES)
@pytest.mark.parametrize("prefix", [0, 1, 100, 128, 200, 700])
def test_builder_prefix_lm(lib, q_len, kv_len, prefix):
    """PrefixLM lists (prefix shorter than, equal to and beyond a tile, and
    beyond the keys), bit-exact against the oracle."""
    ref = oracle.create_block_mask(oracle.prefix_lm_mask(prefix), 1, 1, q_len, kv_len, 128)
    bm = lib.create_block_mask("prefix_lm", 1, 1, q_len, kv_len, 128, prefix_len=prefix)
    check(bm, ref)
