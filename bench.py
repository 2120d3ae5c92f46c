"""Benchmark of the block-sparse attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
the BlockMask build (classify, compact, schedule) followed by the forward.
Inputs are generated once and stay resident in HBM. Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1] [--settle-ms T]

Before the W warmup steps, untimed steps run for T ms of wall time so the
GPU clock has settled (it climbs over the first tens of ms of load).

FLOP accounting: 4 * D flops per allowed (q, kv) pair and (b, h) (2D for
q.k, 2D for p.v); softmax and score_mod arithmetic are not counted. The
allowed-pair count comes from the mask's per-row intervals (closed form).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

import workloads as W

BF16_PEAK_TFLOPS = 2516.6   # MI355X dense bf16 (and fp16) MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
F32_PEAK_TFLOPS = 157.3     # MI355X fp32 (vector / matrix)
HBM_PEAK_GBS = 8000.0


def allowed_pairs_per_head(w: W.Workload, doc_lengths=None) -> int:
    """Allowed (q, kv) pairs of one (b, h), from the per-row allowed intervals."""
    q = np.arange(w.Q_LEN, dtype=np.int64)
    kv_max = w.KV_LEN - 1
    if w.mask == "noop":
        return w.Q_LEN * w.KV_LEN
    if w.mask == "causal":
        return int(np.clip(np.minimum(q, kv_max) + 1, 0, None).sum())
    if w.mask == "sliding_sink":
        hi = np.minimum(q, kv_max)
        lo1 = np.maximum(0, q - w.window + 1)
        n1 = np.clip(hi - lo1 + 1, 0, None)
        hi2 = np.minimum(np.minimum(w.sinks - 1, q), kv_max)
        n2 = np.clip(hi2 + 1, 0, None)
        ov = np.clip(np.minimum(hi, hi2) - lo1 + 1, 0, None)
        return int((n1 + n2 - ov).sum())
    if w.mask == "document_causal":
        lens = np.asarray(doc_lengths, dtype=np.int64)
        return int((lens * (lens + 1) // 2).sum())
    raise ValueError(w.mask)


def algorithmic_bytes(w: W.Workload, nqb: int, nkb: int) -> int:
    """Bytes a forward must move at least once: q, k, v, out, lse and the
    BlockMask it reads."""
    es = 4 if w.dtype == "f32" else 2
    q = w.B * w.Hq * w.Q_LEN * w.D * es
    kv = 2 * w.B * w.Hkv * w.KV_LEN * w.D * es
    out = q
    lse = w.B * w.Hq * w.Q_LEN * 4
    bm = 4 * (2 * nqb + 2 * nqb * nkb + nqb)
    return q + kv + out + lse + bm


HERE = os.path.dirname(os.path.abspath(__file__))


def note(msg: str) -> None:
    """A progress line on stderr as each leg ends (stdout keeps the one JSON line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)
KERNEL_SOURCES = ("fwd_bf16.hip", "fwd_bf16_inst.hip", "fwd_bf16_kernel.hpp", "fwd_plan.hpp",
                  "common.hpp", "fwd_common.hpp")


def measured_traffic(workload: str, field: str = "traffic_bytes_per_launch"):
    """HBM bytes per forward launch (or another field: mfma_util_pct) from
    the committed counter summary of this workload, or None when there is
    none or the kernel sources changed since it was taken."""
    import hashlib
    path = os.path.join(HERE, "profiles", f"fwd_bf16_kernel.{workload}.counters.md")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    for name in KERNEL_SOURCES:
        src = os.path.join(HERE, "block_sparse_masked_amd", "csrc", name)
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if fields.get(f"source_sha256_{name}") != digest:
            return None
    try:
        return float(fields[field]) if "." in fields[field] else int(fields[field])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w: W.Workload, inp: W.Inputs, budget_s: float = 20.0):
    """Time the fp64 oracle (as it stands) on a bounded sample of the same
    workload: whole (b, h) heads, as many as fit the time budget. Returns
    the record and the oracle's O / LSE (NaN outside the heads done)."""
    import oracle  # noqa: E402  (CPU-baseline leg only)
    cores = len(os.sched_getaffinity(0))
    mask, score = oracle.for_workload(w, inp)
    pairs = allowed_pairs_per_head(w, inp.doc_lengths)
    done, t0 = 0, time.perf_counter()
    o_ref = np.full((w.B, w.Hq, w.Q_LEN, w.D), np.nan)
    lse_ref = np.full((w.B, w.Hq, w.Q_LEN), np.nan)
    for b in range(w.B):
        for h in range(w.Hq):
            o, l = oracle.attention(inp.q, inp.k, inp.v, mask, score, w.scale, batches=[b],
                                    heads=[h])
            o_ref[b, h], lse_ref[b, h] = o[b, h], l[b, h]
            done += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 4.0 * w.D * pairs * done
    rec = {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
           "sample": f"{done} of {w.B * w.Hq} (b, h) heads, all {w.Q_LEN} query rows each, "
                     f"fp64 NumPy, {dt:.1f} s",
           "cpu_model": cpu_model(), "blas": blas_vendor()}
    return rec, o_ref, lse_ref


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def blas_vendor() -> str:
    try:
        cfg = np.show_config(mode="dicts")
        blas = cfg.get("Build Dependencies", {}).get("blas", {})
        return f"{blas.get('name', '?')} {blas.get('version', '')}".strip()
    except Exception:  # noqa: BLE001  (older NumPy: no dict mode)
        return "unknown"


def device_facts(torch):
    """CU count and peak engine clock from rocminfo (the spec peak is
    re-derived from them), plus the rate of a large library bf16 GEMM on
    this device as a practical matrix-core reference."""
    import subprocess
    facts = {}
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
        gpu = out[out.index("gfx950"):] if "gfx950" in out else out
        for line in gpu.splitlines():
            line = line.strip()
            if line.startswith("Compute Unit:") and "compute_units" not in facts:
                facts["compute_units"] = int(line.split(":")[1])
            if line.startswith("Max Clock Freq. (MHz):") and "max_clock_mhz" not in facts:
                facts["max_clock_mhz"] = int(line.split(":")[1])
    except Exception as e:  # noqa: BLE001
        facts["rocminfo_error"] = str(e)[:200]
    if "compute_units" in facts and "max_clock_mhz" in facts:
        facts["bf16_peak_tflops_from_clock"] = round(
            facts["compute_units"] * 4096 * facts["max_clock_mhz"] * 1e6 / 1e12, 1)
    n = 8192
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(5):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    reps = 20
    for _ in range(reps):
        torch.matmul(a, b)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    facts["library_gemm_bf16_tflops"] = round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)
    facts["library_gemm_shape"] = f"{n}x{n}x{n} torch.matmul"
    del a, b
    facts.update(mfma_probe(torch, facts.get("compute_units", 256)))
    return facts


def mfma_probe(torch, cus: int):
    """Sustained dense bf16 MFMA rate on this device: libfaprobe.so's kernel
    (every wave issuing 32x32x16 MFMAs back to back, two workgroups of four
    waves per CU) timed with HIP events on the current stream; the clock it
    implies is that rate over 4096 flop/clk per CU."""
    import ctypes
    path = os.path.join(HERE, "block_sparse_masked_amd", "libfaprobe.so")
    if not os.path.exists(path):
        return {"mfma_probe_error": "libfaprobe.so not built"}
    probe = ctypes.CDLL(path)
    probe.faprobe_mfma_bf16.restype = ctypes.c_int
    probe.faprobe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p]
    blocks, iters = 2 * cus, 20000
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def call():
        rc = probe.faprobe_mfma_bf16(iters, blocks, out.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"faprobe_mfma_bf16 failed: HIP error {rc}")
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    ts = []
    for _ in range(5):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        call()
        b.record(stream)
        ts.append((a, b))
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ts]))
    flops = blocks * 4 * 4 * iters * 32768.0
    tflops = flops / (ms * 1e-3) / 1e12
    return {"mfma_probe_bf16_tflops": round(tflops, 1),
            "mfma_probe_implied_clock_mhz": round(tflops * 1e12 / (cus * 4096) / 1e6),
            "mfma_probe": f"{blocks} workgroups x 4 waves x {4 * iters} v_mfma_f32_32x32x16_bf16"}


def errors_vs_oracle(w: W.Workload, out, lse, o32, o_ref, lse_ref):
    """Errors on the rows the oracle computed (NaN elsewhere): strict and
    ulp-aware max-abs of the output, max-abs of the fp32 O the same kernel
    writes before rounding, and relative LSE error (guarded by
    max(|LSE|, 1), and strict)."""
    sel = ~np.isnan(lse_ref)
    live = sel & ~np.isneginf(lse_ref)
    o = out.float().cpu().numpy().astype(np.float64)
    l_ = lse.cpu().numpy().astype(np.float64)
    do = np.abs(o[live] - o_ref[live])
    dl = np.abs(l_[live] - lse_ref[live])
    rec = {"heads_compared": int(sel.any(axis=-1).sum()), "rows_compared": int(sel.sum()),
           "o_max_abs": float(do.max()),
           "lse_max_rel_guarded": float((dl / np.maximum(np.abs(lse_ref[live]), 1.0)).max()),
           "lse_max_rel_strict": float((dl / np.abs(lse_ref[live])).max()),
           "lse_max_abs": float(dl.max())}
    if w.dtype != "f32":
        ax = np.maximum(np.abs(o_ref[live]), np.finfo(np.float32).tiny)
        half_ulp = 0.5 * np.exp2(np.floor(np.log2(ax)) - (10 if w.dtype == "f16" else 7))
        rec["o_over_2e-2"] = int((do > 2e-2).sum())
        rec["o_ulp_aware_ok"] = bool(np.all(do <= 2e-2 + half_ulp))
        if o32 is not None:
            rec["o_f32_max_abs"] = float(np.abs(o32.cpu().numpy()[live] - o_ref[live]).max())
    return rec


def settle(torch, fn, ms: float):
    """Untimed calls of fn for at least ms of wall time: a leg that follows
    host-side input generation starts on an idle GPU, whose clock climbs over
    the first tens of milliseconds of load."""
    t0 = time.perf_counter()
    while True:
        for _ in range(5):
            fn()
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= ms:
            return


def decode_leg(fa, torch, dev, stream, steps: int, settle_ms: float):
    """Split-KV forward on the decode workload (few queries, long KV): HBM
    bound, so reported as bytes moved per second against the HBM peak. Its
    inputs are freed before returning."""
    w = W.DECODE_GQA
    inp = W.generate(w)
    q, k, v = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (inp.q, inp.k, inp.v))
    del inp
    bm = fa.create_block_mask(w.mask, 1, 1, w.Q_LEN, w.KV_LEN, 128, device=dev, stream=stream)
    splits = fa.auto_splits(q, k, bm)
    lib = fa.load_library()
    need = lib.flexattn_fwd_splitkv_workspace_bytes(w.B, w.Hq, w.Q_LEN, w.D, splits)
    ws = torch.empty((need + 3) // 4, dtype=torch.float32, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

    def call():
        fa.flex_attention(q, k, v, bm, scale=w.scale, out=out, lse=lse, stream=stream,
                          num_splits=splits, workspace=ws)
    settle(torch, call, settle_ms)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        call()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = float(np.median([a.elapsed_time(b) for a, b in ev]))
    alg = algorithmic_bytes(w, bm.num_q_blocks, bm.num_kv_blocks)
    rec = {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Q_LEN": w.Q_LEN,
           "KV_LEN": w.KV_LEN, "D": w.D, "mask": w.mask, "num_splits": splits,
           "ms_median": round(ms, 4), "calls": steps,
           "algorithmic_bytes": alg,
           "achieved_gbs": round(alg / (ms * 1e-3) / 1e9, 1),
           "peak_gbs": HBM_PEAK_GBS,
           "frac": round(alg / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "workspace_bytes": need,
           "bound": "hbm"}
    # the same call over a paged copy of the cache (pages of 256 keys at a
    # seeded random placement, page table int32 [B, 129])
    kc, vc, table = W.paged_cache(k.float().cpu().numpy(), v.float().cpu().numpy(), 256,
                                  seed=w.seed)
    del k, v
    kc, vc = (torch.from_numpy(x).to(torch.bfloat16).to(dev) for x in (kc, vc))
    table = torch.from_numpy(table).to(dev)

    def call_paged():
        fa.flex_attention(q, kc, vc, bm, scale=w.scale, out=out, lse=lse, stream=stream,
                          num_splits=splits, workspace=ws, page_table=table)
    settle(torch, call_paged, settle_ms)
    for i in range(steps):
        ev[i][0].record(stream)
        call_paged()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms_p = float(np.median([a.elapsed_time(b) for a, b in ev]))
    rec["paged"] = {"page_size": 256, "ms_median": round(ms_p, 4),
                    "achieved_gbs": round(alg / (ms_p * 1e-3) / 1e9, 1),
                    "frac": round(alg / (ms_p * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    del q, kc, vc, ws, out, lse, table
    torch.cuda.empty_cache()
    return rec


def config_leg(fa, torch, w: W.Workload, steps: int, settle_ms: float, dev, stream):
    """A workload other than the headline one, timed on its own after the
    headline's legs (not part of `value`): the forward alone on resident
    inputs with a BlockMask built once, its effective and dense-equivalent
    rates, its roofline fraction, and its errors against the oracle on whole
    heads (all of them for the fp32 workload, the first and the last (b, h)
    for the others). Inputs are freed before returning."""
    import oracle  # noqa: E402  (error check only)
    inp = W.generate(w)
    tdtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x).to(tdtype).to(dev) for x in (inp.q, inp.k, inp.v))
    doc = torch.from_numpy(inp.doc_ids).to(dev) if inp.doc_ids is not None else None
    bm = fa.create_block_mask(w.mask, 1, 1, w.Q_LEN, w.KV_LEN, 128, window=w.window,
                              num_sinks=w.sinks, doc_ids=doc, device=dev, stream=stream)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)

    def call():
        fa.flex_attention(q, k, v, bm, score=w.score, softcap=w.softcap, scale=w.scale, out=out,
                          lse=lse, stream=stream)
    settle(torch, call, settle_ms)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(stream)
        call()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    times = [a.elapsed_time(b) for a, b in ev]
    ms = float(np.median(times))
    pairs = allowed_pairs_per_head(w, inp.doc_lengths)
    eff = 4.0 * w.D * pairs * w.B * w.Hq
    dense = 4.0 * w.D * w.Q_LEN * w.KV_LEN * w.B * w.Hq
    peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else F32_PEAK_TFLOPS
    alg = algorithmic_bytes(w, bm.num_q_blocks, bm.num_kv_blocks)
    traffic = measured_traffic(w.name) if w.dtype == "bf16" else None
    t = ms * 1e-3
    rec = {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Q_LEN": w.Q_LEN,
           "KV_LEN": w.KV_LEN, "D": w.D, "dtype": w.dtype, "mask": w.mask, "score": w.score,
           "seed": w.seed, "calls": steps,
           "fwd_ms_median": round(ms, 4), "fwd_ms_min": round(float(np.min(times)), 4),
           "effective_tflops": round(eff / t / 1e12, 2),
           "dense_equivalent_tflops": round(dense / t / 1e12, 2),
           "unmasked_fraction": round(pairs / (w.Q_LEN * w.KV_LEN), 4),
           "peak": peak, "frac": round(eff / t / 1e12 / peak, 4),
           "algorithmic_bytes": alg, "algorithmic_gbs": round(alg / t / 1e9, 1),
           "traffic": traffic,
           "traffic_gbs": round(traffic / t / 1e9, 1) if traffic else None,
           "mfma_util_pct": measured_traffic(w.name, "mfma_util_pct") if w.dtype == "bf16"
           else None}
    if inp.doc_lengths is not None:
        rec["doc_lengths"] = [int(x) for x in inp.doc_lengths]
    o32 = None
    if w.dtype != "f32":
        o32 = fa.flex_attention_train(q, k, v, bm, score=w.score, softcap=w.softcap,
                                      scale=w.scale, stream=stream)[2]
    torch.cuda.synchronize()
    pairs_bh = ([(b, h) for b in range(w.B) for h in range(w.Hq)] if w.dtype == "f32"
                else [(0, 0), (w.B - 1, w.Hq - 1)])
    mask, score = oracle.for_workload(w, inp)
    o_ref = np.full(tuple(out.shape), np.nan)
    lse_ref = np.full(tuple(lse.shape), np.nan)
    for b, h in pairs_bh:
        ob, lb = oracle.attention(inp.q, inp.k, inp.v, mask, score, w.scale, batches=[b],
                                  heads=[h])
        o_ref[b, h], lse_ref[b, h] = ob[b, h], lb[b, h]
    rec["errors"] = errors_vs_oracle(w, out, lse, o32, o_ref, lse_ref)
    del q, k, v, out, lse, o32, bm
    torch.cuda.empty_cache()
    return rec


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=W.DENSE_CAUSAL_GQA.name, choices=sorted(W.BY_NAME))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed steps for this long before the warmup steps (clock settling)")
    ap.add_argument("--ablation-steps", type=int, default=20,
                    help="after the timed steps, time this many forwards on a BlockMask built "
                         "with separate_full_blocks=False (0 = skip)")
    ap.add_argument("--backward-steps", type=int, default=10,
                    help="after the forward, time this many backward calls (bf16 workloads; "
                         "0 = skip)")
    ap.add_argument("--decode-steps", type=int, default=20,
                    help="after the forward, time this many split-KV forwards on the decode "
                         "workload (%s; 0 = skip)" % W.DECODE_GQA.name)
    ap.add_argument("--f16-steps", type=int, default=20,
                    help="after the forward, time this many forwards of the same workload with "
                         "fp16 inputs (bf16 workloads; 0 = skip)")
    ap.add_argument("--config-steps", type=int, default=20,
                    help="after the headline legs, time this many forwards of each of the other "
                         "workloads and check their errors against the oracle (0 = skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run 5 plain device copies of MIB MiB "
                         "(reference for the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the forward shards by "
              "(batch, KV head) with no exchange, so no multi-GPU figure is measured here.",
              file=sys.stderr)
        return 2

    import torch
    import block_sparse_masked_amd as fa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20)
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "copies": 5}), flush=True)
        return 0
    fa.load_library()
    w = W.BY_NAME[args.workload]
    inp = W.generate(w)
    dev = torch.device("cuda:0")
    tdtype = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q = torch.from_numpy(inp.q).to(tdtype).to(dev)
    k = torch.from_numpy(inp.k).to(tdtype).to(dev)
    v = torch.from_numpy(inp.v).to(tdtype).to(dev)
    doc = torch.from_numpy(inp.doc_ids).to(dev) if inp.doc_ids is not None else None
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        bm = fa.create_block_mask(w.mask, 1, 1, w.Q_LEN, w.KV_LEN, 128, window=w.window,
                                  num_sinks=w.sinks, doc_ids=doc, device=dev, stream=stream)
        fa.flex_attention(q, k, v, bm, score=w.score, softcap=w.softcap, scale=w.scale,
                          out=out, lse=lse, stream=stream)
        return bm

    # Clock settling (untimed): the GPU raises its clock over the first tens
    # of milliseconds of sustained load, so run steps for at least
    # --settle-ms of wall time before the warmup steps.
    settle_steps = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(10):
            step()
        settle_steps += 10
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        bm = step()
    torch.cuda.synchronize()

    # timed region: K steps; events around the build and the forward of each
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(args.steps):
        ev[i][0].record(stream)
        bm = fa.create_block_mask(w.mask, 1, 1, w.Q_LEN, w.KV_LEN, 128, window=w.window,
                                  num_sinks=w.sinks, doc_ids=doc, device=dev, stream=stream)
        ev[i][1].record(stream)
        fa.flex_attention(q, k, v, bm, score=w.score, softcap=w.softcap, scale=w.scale,
                          out=out, lse=lse, stream=stream)
        ev[i][2].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    build_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(args.steps)]
    fwd_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in range(args.steps)]
    note(f"{args.steps} timed steps of {w.name}: {ms_step:.4f} ms per step")

    # the headline's fp32 O (same kernel, written before rounding) for the
    # error report
    o32_main = None
    if w.dtype != "f32":
        o32_main = fa.flex_attention_train(q, k, v, bm, score=w.score, softcap=w.softcap,
                                           scale=w.scale, stream=stream)[2].cpu()
    out_main, lse_main = out.clone(), lse.clone()

    # Full-tile ablation (after the timed region, not part of `value`): the
    # same forward on a BlockMask built with separate_full_blocks=False, so
    # mask_mod runs on every tile (page "tensorplay.nn.attention API",
    # BlockMask "Details": skipping the mask on full tiles is the speed-up).
    ablation = None
    if args.ablation_steps > 0:
        bm_all = fa.create_block_mask(w.mask, 1, 1, w.Q_LEN, w.KV_LEN, 128, window=w.window,
                                      num_sinks=w.sinks, doc_ids=doc, device=dev, stream=stream,
                                      separate_full_blocks=False)
        settle(torch, lambda: fa.flex_attention(q, k, v, bm_all, score=w.score,
                                                softcap=w.softcap, scale=w.scale, out=out,
                                                lse=lse, stream=stream), args.settle_ms)
        ev_a = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                for _ in range(args.ablation_steps)]
        for i in range(args.ablation_steps):
            ev_a[i][0].record(stream)
            fa.flex_attention(q, k, v, bm_all, score=w.score, softcap=w.softcap, scale=w.scale,
                              out=out, lse=lse, stream=stream)
            ev_a[i][1].record(stream)
        torch.cuda.synchronize()
        all_partial_ms = float(np.median([a.elapsed_time(b) for a, b in ev_a]))
        ablation = {"fwd_ms_median_all_partial": round(all_partial_ms, 4),
                    "fwd_ms_median": round(float(np.median(fwd_ms)), 4),
                    "speedup_from_full_tiles": round(all_partial_ms / float(np.median(fwd_ms)), 4),
                    "calls": args.ablation_steps}
        note("full-tile ablation done")

    # Backward (after the forward's timed region, not part of `value`): one
    # flexattn_bwd call per step on the same inputs with a seeded upstream
    # gradient; the mask carries the backward lists.
    backward = None
    if args.backward_steps > 0 and w.dtype == "bf16":
        bm_b = fa.create_block_mask(w.mask, 1, 1, w.Q_LEN, w.KV_LEN, 128, window=w.window,
                                    num_sinks=w.sinks, doc_ids=doc, device=dev, stream=stream,
                                    backward_lists=True)
        g = torch.from_numpy(W.generate_upstream(w)).to(tdtype).to(dev)
        fa.flex_attention(q, k, v, bm_b, score=w.score, softcap=w.softcap, scale=w.scale,
                          out=out, lse=lse, stream=stream)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
        settle(torch, lambda: fa.flex_attention_backward(
            q, k, v, lse, g, bm_b, score=w.score, softcap=w.softcap, scale=w.scale, dq=dq, dk=dk,
            dv=dv, workspace=ws, stream=stream), args.settle_ms)
        ev_b = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                for _ in range(args.backward_steps)]
        for i in range(args.backward_steps):
            ev_b[i][0].record(stream)
            fa.flex_attention_backward(q, k, v, lse, g, bm_b, score=w.score, softcap=w.softcap,
                                       scale=w.scale, dq=dq, dk=dk, dv=dv, workspace=ws,
                                       stream=stream)
            ev_b[i][1].record(stream)
        torch.cuda.synchronize()
        bwd_ms = float(np.median([a.elapsed_time(b) for a, b in ev_b]))
        backward = {"ms_median": round(bwd_ms, 4), "calls": args.backward_steps}
        # the training pair: the forward also writes fp32 O, and the backward
        # takes Delta = dO . O from it instead of recomputing P and dP
        o32 = torch.empty(q.shape, dtype=torch.float32, device=dev)
        fa.flex_attention_train(q, k, v, bm_b, score=w.score, softcap=w.softcap, scale=w.scale,
                                out=out, lse=lse, out_f32=o32, stream=stream)
        for _ in range(2):
            fa.flex_attention_backward(q, k, v, lse, g, bm_b, score=w.score, softcap=w.softcap,
                                       scale=w.scale, dq=dq, dk=dk, dv=dv, workspace=ws,
                                       stream=stream, out_f32=o32)
        for i in range(args.backward_steps):
            ev_b[i][0].record(stream)
            fa.flex_attention_backward(q, k, v, lse, g, bm_b, score=w.score, softcap=w.softcap,
                                       scale=w.scale, dq=dq, dk=dk, dv=dv, workspace=ws,
                                       stream=stream, out_f32=o32)
            ev_b[i][1].record(stream)
        torch.cuda.synchronize()
        backward["ms_median_from_out"] = round(
            float(np.median([a.elapsed_time(b) for a, b in ev_b])), 4)
        del o32
        note("backward done")

    # fp16 (after the timed region, not part of `value`): the same workload
    # drawn and rounded as fp16, forward only
    f16 = None
    if args.f16_steps > 0 and w.dtype == "bf16":
        w16 = w.with_(name=w.name.replace("bf16", "f16"), dtype="f16")
        inp16 = W.generate(w16)
        q16, k16, v16 = (torch.from_numpy(x).to(torch.float16).to(dev)
                         for x in (inp16.q, inp16.k, inp16.v))
        del inp16
        out16 = torch.empty_like(q16)
        bm16 = fa.create_block_mask(w.mask, 1, 1, w.Q_LEN, w.KV_LEN, 128, window=w.window,
                                    num_sinks=w.sinks, doc_ids=doc, device=dev, stream=stream)
        settle(torch, lambda: fa.flex_attention(q16, k16, v16, bm16, score=w.score,
                                                softcap=w.softcap, scale=w.scale, out=out16,
                                                lse=lse, stream=stream), args.settle_ms)
        ev_h = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                for _ in range(args.f16_steps)]
        for i in range(args.f16_steps):
            ev_h[i][0].record(stream)
            fa.flex_attention(q16, k16, v16, bm16, score=w.score, softcap=w.softcap,
                              scale=w.scale, out=out16, lse=lse, stream=stream)
            ev_h[i][1].record(stream)
        torch.cuda.synchronize()
        f16 = {"ms_median": round(float(np.median([a.elapsed_time(b) for a, b in ev_h])), 4),
               "calls": args.f16_steps}
        del q16, k16, v16, out16
        note("fp16 leg done")

    decode = None
    if args.decode_steps > 0:
        decode = decode_leg(fa, torch, dev, stream, args.decode_steps, args.settle_ms)
        note("decode leg done")

    configs = {}
    if args.config_steps > 0:
        for other in W.WORKLOADS:
            if other.name != w.name:
                configs[other.name] = config_leg(fa, torch, other, args.config_steps,
                                                 args.settle_ms, dev, stream)
                note(f"{other.name} leg done")
    facts = device_facts(torch)

    pairs = allowed_pairs_per_head(w, inp.doc_lengths)
    eff_flops = 4.0 * w.D * pairs * w.B * w.Hq
    dense_flops = 4.0 * w.D * w.Q_LEN * w.KV_LEN * w.B * w.Hq
    nonempty = int(bm.kv_num_blocks.sum().item() + bm.full_kv_num_blocks.sum().item())
    visited_flops = 4.0 * w.D * 128 * 128 * nonempty * w.B * w.Hq
    peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else F32_PEAK_TFLOPS
    fwd_avg = float(np.mean(fwd_ms))
    value = eff_flops / (ms_step * 1e-3) / 1e12
    fwd_tflops = eff_flops / (fwd_avg * 1e-3) / 1e12
    nqb, nkb = bm.num_q_blocks, bm.num_kv_blocks

    rec = {
        "metric": "effective TFLOP/s (unmasked FLOPs) flex-attn fwd bf16; % of MFMA peak",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Q_LEN": w.Q_LEN,
                   "KV_LEN": w.KV_LEN, "D": w.D, "mask": w.mask, "score": w.score,
                   "seed": w.seed, "block": 128, "parallelism": "single-gpu"},
        "pct_of_peak": round(100.0 * value / peak, 2),
        "settle": {"ms": args.settle_ms, "steps": settle_steps},
        "fwd_ms_avg": round(fwd_avg, 4),
        "fwd_ms_min": round(float(np.min(fwd_ms)), 4),
        "fwd_ms_median": round(float(np.median(fwd_ms)), 4),
        "build_ms_avg": round(float(np.mean(build_ms)), 4),
        "fwd_effective_tflops": round(fwd_tflops, 2),
        "dense_equivalent_tflops": round(dense_flops / (fwd_avg * 1e-3) / 1e12, 2),
        "visited_tile_tflops": round(visited_flops / (fwd_avg * 1e-3) / 1e12, 2),
        "unmasked_fraction": round(pairs / (w.Q_LEN * w.KV_LEN), 4),
        "tile_sparsity_pct": round(100.0 * (1 - nonempty / (nqb * nkb)), 2),
        "roofline": {
            "bound": "mfma",
            "kernel": "fwd_bf16_kernel" if w.dtype == "bf16" else "fwd_f32_kernel",
            "achieved": round(fwd_tflops, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(fwd_tflops / peak, 4),
            "traffic": measured_traffic(w.name) if w.dtype == "bf16" else None,
            "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_bytes": algorithmic_bytes(w, nqb, nkb),
            "mfma_util_pct": (measured_traffic(w.name, "mfma_util_pct")
                              if w.dtype == "bf16" else None),
        },
        "device": facts,
    }
    tr = rec["roofline"]["traffic"]
    rec["roofline"]["hbm_gbs"] = round(tr / (fwd_avg * 1e-3) / 1e9, 1) if tr else None
    probe = facts.get("mfma_probe_bf16_tflops")
    if probe and w.dtype == "bf16":
        # beside the published peak: the fraction of the rate the matrix
        # cores sustain on this device at the clock a full matrix load runs at
        rec["roofline"]["frac_of_measured_mfma"] = round(fwd_tflops / probe, 4)
    if configs:
        rec["configs"] = configs
    if ablation is not None:
        rec["full_tile_ablation"] = ablation
    if backward is not None:
        # algorithmic work: five products of 2*D flops per allowed pair (S,
        # dP, dV, dK, dQ); the kernels execute nine (S and dP three times:
        # Delta pass, dQ walk, dK/dV walk)
        alg = 10.0 * w.D * pairs * w.B * w.Hq
        done = 18.0 * w.D * pairs * w.B * w.Hq
        t = backward["ms_median"] * 1e-3
        t2 = backward["ms_median_from_out"] * 1e-3
        backward.update({
            "effective_tflops_from_out": round(alg / t2 / 1e12, 2),
            "effective_tflops": round(alg / t / 1e12, 2),
            "executed_tflops": round(done / t / 1e12, 2),
            "frac_of_peak": round(alg / t / 1e12 / BF16_PEAK_TFLOPS, 4),
            "flop_convention": "10*D per allowed (q, kv) pair and (b, h); executed 18*D"})
        rec["backward"] = backward
    if f16 is not None:
        t = f16["ms_median"] * 1e-3
        f16.update({"effective_tflops": round(eff_flops / t / 1e12, 2),
                    "frac_of_peak": round(eff_flops / t / 1e12 / BF16_PEAK_TFLOPS, 4),
                    "peak": BF16_PEAK_TFLOPS})
        rec["fwd_f16"] = f16
    if decode is not None:
        rec["decode_splitkv"] = decode
    if inp.doc_lengths is not None:
        rec["config"]["doc_lengths"] = [int(x) for x in inp.doc_lengths]
    if not args.no_cpu_baseline:
        rec["cpu_baseline"], o_ref, lse_ref = cpu_baseline(w, inp, args.cpu_budget)
        rec["errors"] = errors_vs_oracle(w, out_main, lse_main, o32_main, o_ref, lse_ref)
        note("cpu baseline done")
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
