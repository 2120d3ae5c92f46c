"""fp64 CPU oracle for the FlexAttention-style block-sparse forward.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
bench's CPU-baseline leg, never by the GPU product path. See
``oracle/reference.py`` for what each function follows on the pages.
"""
from .reference import (  # noqa: F401
    BlockMask,
    alibi_score,
    alibi_slopes,
    and_masks,
    attention,
    causal_mask,
    classify_tiles,
    create_block_mask,
    create_mask,
    document_causal_mask,
    from_kv_blocks_mask,
    composite_mask,
    prefix_mask,
    document_mask,
    gather_paged,
    noop_mask,
    or_masks,
    prefix_lm_mask,
    sink_mask,
    sliding_sink_mask,
    softcap_alibi_score,
    softcap_score,
    to_dense,
    unmasked_pairs,
    window_mask,
)
from .backward import (  # noqa: F401
    attention_backward,
    score_grad_for,
    softcap_grad,
    transpose_block_mask,
)


def mask_mod_for(kind: str, window: int = 0, sinks: int = 0, doc_ids=None, prefix: int = 0,
                 terms=None):
    """The oracle mask_mod for a mask kind name."""
    if kind == "noop":
        return noop_mask
    if kind == "causal":
        return causal_mask
    if kind == "sliding_sink":
        return sliding_sink_mask(window, sinks)
    if kind == "document_causal":
        if doc_ids is None:
            raise ValueError("document_causal needs doc_ids")
        return document_causal_mask(doc_ids)
    if kind == "prefix_lm":
        return prefix_lm_mask(prefix)
    if kind == "composite":
        return composite_mask(terms, window, sinks, prefix, doc_ids)
    raise ValueError(f"unknown mask kind {kind!r}")


def score_mod_for(kind: str, num_heads: int, softcap: float = 0.0, slopes=None):
    """The oracle score_mod for a score kind name (None for 'none')."""
    if kind == "none":
        return None
    if slopes is None:
        slopes = alibi_slopes(num_heads)
    if kind == "alibi":
        return alibi_score(slopes)
    if kind == "softcap":
        return softcap_score(softcap)
    if kind == "softcap_alibi":
        return softcap_alibi_score(softcap, slopes)
    raise ValueError(f"unknown score kind {kind!r}")


def for_workload(w, inputs):
    """(mask_mod, score_mod) of a ``workloads.Workload`` and its inputs."""
    mask = mask_mod_for(w.mask, w.window, w.sinks, inputs.doc_ids, w.prefix, w.terms)
    score = score_mod_for(w.score, w.Hq, w.softcap)
    return mask, score
