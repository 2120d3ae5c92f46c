"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
the fp64 oracle on the same seeded inputs, and compare them."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads as W

BF16_O_ATOL = 2e-2      # max |O_gpu - O_ref| for bf16 inputs
BF16_LSE_RTOL = 1e-3    # |dLSE| / max(|LSE_ref|, 1) for bf16 inputs
F32_ATOL = 1e-5         # max |O_gpu - O_ref| and |LSE_gpu - LSE_ref| for fp32 inputs


def to_device(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = {"bf16": t.to(torch.bfloat16), "f16": t.to(torch.float16)}.get(dtype, t)
    return t.to(device)


def build_gpu_mask(lib, w: W.Workload, inputs: W.Inputs, B_mask=1, H_mask=1,
                   separate_full_blocks=True, backward_lists=False):
    doc = None
    if inputs.doc_ids is not None:
        doc = torch.from_numpy(inputs.doc_ids.astype(np.int32))
    return lib.create_block_mask(w.mask, B_mask, H_mask, w.Q_LEN, w.KV_LEN, 128,
                                 window=w.window, num_sinks=w.sinks, doc_ids=doc,
                                 separate_full_blocks=separate_full_blocks, prefix_len=w.prefix,
                                 terms=w.terms, backward_lists=backward_lists)


def run_gpu(lib, w: W.Workload, inputs: W.Inputs, bm=None):
    q = to_device(inputs.q, w.dtype)
    k = to_device(inputs.k, w.dtype)
    v = to_device(inputs.v, w.dtype)
    if bm is None:
        bm = build_gpu_mask(lib, w, inputs)
    out, lse = lib.flex_attention(q, k, v, bm, score=w.score, softcap=w.softcap, scale=w.scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), bm


def oracle_rows(w: W.Workload, inputs: W.Inputs, batches=None, heads=None, rows=None):
    mask, score = oracle.for_workload(w, inputs)
    return oracle.attention(inputs.q, inputs.k, inputs.v, mask, score, w.scale,
                            batches=batches, heads=heads, rows=rows)


def bf16_ulp(x: np.ndarray, bits: int = 8) -> np.ndarray:
    """Spacing of bfloat16 numbers at |x| (8 significant bits; 11 for fp16)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(ax)) - (bits - 1))


def compare(w: W.Workload, o_gpu, lse_gpu, o_ref, lse_ref, where=None):
    """Errors on the selected entries (NaN in the reference = not computed).

    Returns a dict; `ok` applies the tolerances for the workload's dtype.
    For bf16 the strict O bound is reported, and `o_ulp_ok` checks
    |dO| <= atol + half a bf16 ulp of the reference (the output itself is
    rounded to bf16)."""
    sel = ~np.isnan(lse_ref) if where is None else where
    og, orf = o_gpu[sel], o_ref[sel]
    lg, lr = lse_gpu[sel], lse_ref[sel]
    res = {"n_rows": int(sel.sum())}
    dead = np.isneginf(lr)
    res["dead_rows"] = int(dead.sum())
    res["dead_ok"] = bool(np.all(np.isneginf(lg[dead])) and np.all(og[dead] == 0.0))
    live = ~dead
    do = np.abs(og[live] - orf[live])
    dl = np.abs(lg[live] - lr[live])
    res["o_max_abs"] = float(do.max()) if do.size else 0.0
    res["lse_max_abs"] = float(dl.max()) if dl.size else 0.0
    res["lse_max_rel_guarded"] = float((dl / np.maximum(np.abs(lr[live]), 1.0)).max()) if dl.size else 0.0
    res["lse_max_rel_strict"] = float((dl / np.abs(lr[live])).max()) if dl.size else 0.0
    res["finite"] = bool(np.all(np.isfinite(og)) and np.all(np.isfinite(lg[live])))
    if w.dtype == "f32":
        res["ok"] = (res["finite"] and res["dead_ok"] and res["o_max_abs"] <= F32_ATOL
                     and res["lse_max_abs"] <= F32_ATOL)
    else:
        # bf16 and fp16 share the bound; the output rounding is the dtype's
        slack = BF16_O_ATOL + 0.5 * bf16_ulp(orf[live], 11 if w.dtype == "f16" else 8)
        res["o_ulp_ok"] = bool(np.all(do <= slack))
        res["o_strict_ok"] = res["o_max_abs"] <= BF16_O_ATOL
        res["ok"] = (res["finite"] and res["dead_ok"] and res["o_ulp_ok"]
                     and res["lse_max_rel_guarded"] <= BF16_LSE_RTOL)
    return res


def summary(res) -> str:
    keys = ("ok", "n_rows", "o_max_abs", "lse_max_abs", "lse_max_rel_guarded", "o_ulp_ok",
            "o_strict_ok", "dead_rows", "dead_ok", "finite")
    return ", ".join(f"{k}={res[k]:.3g}" if isinstance(res.get(k), float) else f"{k}={res.get(k)}"
                     for k in keys if k in res)


def full_size_report(w: W.Workload, o16, o32, lse_gpu, o_ref, lse_ref):
    """The stated bounds at full size, on the rows the reference computed
    (NaN elsewhere). The kernel's fp32 O (the value before the output is
    rounded to the input dtype) must meet the strict max-abs bound; the
    16-bit O is reported strictly and ulp-aware, and each of its elements
    over the strict bound is counted (they can only come from rounding the
    fp32 O, which the caller checks bitwise)."""
    sel = ~np.isnan(lse_ref)
    live = sel & ~np.isneginf(lse_ref)
    rep = {"workload": w.name, "rows": int(sel.sum()), "live_rows": int(live.sum())}
    d32 = np.abs(o32[live] - o_ref[live])
    d16 = np.abs(o16[live] - o_ref[live])
    bits = 11 if w.dtype == "f16" else 8
    slack = BF16_O_ATOL + 0.5 * bf16_ulp(o_ref[live], bits)
    dl = np.abs(lse_gpu[live] - lse_ref[live])
    rep.update({
        "o_f32_max_abs": float(d32.max()),
        "o_max_abs": float(d16.max()),
        "o_over_strict": int((d16 > BF16_O_ATOL).sum()),
        "o_ulp_aware_ok": bool(np.all(d16 <= slack)),
        "lse_max_abs": float(dl.max()),
        "lse_max_rel_guarded": float((dl / np.maximum(np.abs(lse_ref[live]), 1.0)).max()),
        "lse_max_rel_strict": float((dl / np.abs(lse_ref[live])).max()),
        "dead_rows_ok": bool(np.all(np.isneginf(lse_gpu[sel & np.isneginf(lse_ref)]))),
    })
    rep["ok"] = (rep["o_f32_max_abs"] <= BF16_O_ATOL and rep["o_ulp_aware_ok"]
                 and rep["lse_max_rel_guarded"] <= BF16_LSE_RTOL and rep["dead_rows_ok"])
    return rep
