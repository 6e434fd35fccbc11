#!/usr/bin/env python3
"""Benchmark of the 1.5-entmax attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A timed step is one full forward (threshold + block mask + sparse output) of
the long-context workload: B=1, H=12, L=8192, d=64, bf16, 64 clustered
centroids, no mask.  The metric is its effective (dense-equivalent)
throughput, 4*d*pairs / time.  The same run also times, each with HIP events
on the stream the library launches on:
  * the threshold kernel alone (the dominant kernel: one dense MFMA score
    sweep, 2*d*pairs FLOP) -> the `roofline` object;
  * the row-wise tau kernel on the 8192 x 8192 fp32 score matrix (HBM-bound;
    3 rotating buffer sets so the 256 MB Infinity Cache cannot serve it);
  * the other forward workloads and the backward;
  * the block-sparsity sweep (clustered L = 8192 with 64 ... 1 cluster runs)
    with a linear fit of forward time against the non-null tile fraction;
  * the clustered forward and the row kernel at alpha = 1.25 and 2;
  * one decode step over a bf16 KV cache (long causal, and window 32 + sink);
  * dense rows wider than 8192 with and without the histogram bracket;
and the fp64 CPU oracle on a bounded sample of the same workload
(`cpu_baseline`).  Rank 0 prints exactly one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
METRIC = "1.5-entmax attn fwd ms + effective TFLOP/s at L=8192; tau-row kernel GB/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


STATS_SOURCES = ["adaptive_sparse_attention_row_amd/csrc/attn_fwd.hip",
                 "adaptive_sparse_attention_row_amd/csrc/attn_common.hpp",
                 "adaptive_sparse_attention_row_amd/csrc/tile_dma.hpp",
                 "adaptive_sparse_attention_row_amd/csrc/device_common.hpp"]
TAUROWS_SOURCES = ["adaptive_sparse_attention_row_amd/csrc/tau_rows.hip",
                   "adaptive_sparse_attention_row_amd/csrc/row_solve.hpp",
                   "adaptive_sparse_attention_row_amd/csrc/device_common.hpp"]


def counter_traffic(name, sources):
    """HBM bytes per launch from a committed rocprofv3 counter summary, valid
    only while the kernel sources are unchanged."""
    path = os.path.join(ROOT, "profiles", f"{name}.counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest(sources):
        return None
    return rec.get("hbm_bytes_per_launch")


class Timer:
    """HIP-event timing of a callable over K launches on torch's current stream
    (the stream the library is handed)."""

    def __init__(self, torch):
        self.torch = torch

    def __call__(self, fn, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for _ in range(steps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps  # ms per call


def pairs_of(cfg):
    L = cfg.L
    if cfg.mask == 0:
        per = L * L
    elif cfg.mask == 1:
        per = L * (L + 1) // 2
    else:
        W = cfg.window
        per = sum(min(i + 1, W + 1) + (1 if i > W else 0) for i in range(L))
    return cfg.B * cfg.H * per


def popcount_mask(bm):
    import numpy as np
    x = bm.view(np.uint32).reshape(-1)
    return int(np.unpackbits(x.view(np.uint8)).sum())


def structural_tiles(cfg):
    from adaptive_sparse_attention_row_amd.workloads import MASK_NONE
    T = -(-cfg.L // 64)
    n = 0
    for I in range(T):
        i0, i1 = I * 64, min(I * 64 + 63, cfg.L - 1)
        for J in range(T):
            c0, c1 = J * 64, min(J * 64 + 63, cfg.L - 1)
            if cfg.mask == MASK_NONE:
                n += 1
            elif c0 > i1:
                continue
            elif cfg.mask == 1:
                n += 1
            elif J == 0 or i0 - c1 <= cfg.window:
                n += 1
    return n * cfg.B * cfg.H


def bench_attn(api, torch, timer, cfg, steps, warmup, with_bwd=False, alpha=1.5):
    """Forward (and backward) timing of one attention workload."""
    from adaptive_sparse_attention_row_amd.workloads import gen_config
    inp = gen_config(cfg)
    q, k, v = (inp[n].cuda() for n in ("q", "k", "v"))
    B, H, L, d = q.shape
    dt = api._dtype_code(q)
    O = torch.empty(B, H, L, d, device="cuda", dtype=torch.float32)
    tau = torch.empty(B, H, L, device="cuda", dtype=torch.float32)
    bm = torch.empty(api.mask_shape(B, H, L, d, dt), device="cuda", dtype=torch.int32)
    lib = api.lib()
    sc, st = float(cfg.scale), api._stream(q.device)
    wsb = lib.entmax_attn_fwd_workspace(B, H, L, d, dt, cfg.mask, cfg.window)
    ws = torch.empty(wsb, device="cuda", dtype=torch.uint8)

    def fwd():
        r = lib.entmax_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), O.data_ptr(), tau.data_ptr(),
                                bm.data_ptr(), B, H, L, d, sc, alpha, dt, cfg.mask, cfg.window, ws.data_ptr(),
                                wsb, st)
        assert r == 0, api.status_str(r)

    def thr():
        r = lib.entmax_attn_threshold(q.data_ptr(), k.data_ptr(), tau.data_ptr(), bm.data_ptr(), B, H, L, d,
                                      sc, alpha, dt, cfg.mask, cfg.window, ws.data_ptr(), wsb, st)
        assert r == 0, api.status_str(r)

    def stats():
        r = lib.entmax_attn_score_stats(q.data_ptr(), k.data_ptr(), B, H, L, d, sc, alpha, dt, cfg.mask,
                                        cfg.window, ws.data_ptr(), wsb, st)
        assert r == 0, api.status_str(r)

    def out():
        r = lib.entmax_attn_output(q.data_ptr(), k.data_ptr(), v.data_ptr(), tau.data_ptr(), bm.data_ptr(),
                                   O.data_ptr(), B, H, L, d, sc, alpha, dt, cfg.mask, cfg.window, st)
        assert r == 0, api.status_str(r)

    t_fwd = timer(fwd, steps, warmup)
    t_thr = timer(thr, steps, warmup)
    t_stats = timer(stats, steps, warmup)
    t_out = timer(out, steps, warmup)
    torch.cuda.synchronize()
    nnz = popcount_mask(bm.cpu().numpy())
    struct = structural_tiles(cfg)
    pairs = pairs_of(cfg)
    res = {
        "fwd_ms": round(t_fwd, 5),
        "threshold_ms": round(t_thr, 5),
        "score_stats_ms": round(t_stats, 5),
        "solve_ms": round(t_thr - t_stats, 5),
        "output_ms": round(t_out, 5),
        "dense_equiv_tflops": round(4 * d * pairs / (t_fwd * 1e-3) / 1e12, 3),
        "score_stats_mfma_tflops": round(2 * d * pairs / (t_stats * 1e-3) / 1e12, 3),
        "nonnull_tiles_64": nnz,
        "structural_tiles_64": struct,
        "block_sparsity_64": round(1.0 - nnz / struct, 5),
        "pairs": pairs,
    }
    if with_bwd:
        do = inp["do"].cuda()
        dq = torch.empty_like(O); dk = torch.empty_like(O); dv = torch.empty_like(O)
        bwsb = lib.entmax_attn_bwd_workspace(B, H, L, d, dt, cfg.mask, cfg.window)
        bws = torch.empty(max(bwsb, 1), device="cuda", dtype=torch.uint8)
        fwd()

        def bwd():
            r = lib.entmax_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(), tau.data_ptr(),
                                    bm.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, L, d,
                                    sc, alpha, dt, cfg.mask, cfg.window, bws.data_ptr(), bwsb, st)
            if r != 0:
                raise RuntimeError(api.status_str(r))

        try:
            t_bwd = timer(bwd, max(1, steps // 2), 1)
            res["bwd_ms"] = round(t_bwd, 5)
            res["bwd_dense_equiv_tflops"] = round(10 * d * pairs / (t_bwd * 1e-3) / 1e12, 3)
        except RuntimeError as e:
            res["bwd"] = f"not available: {e}"
    del q, k, v, O
    torch.cuda.empty_cache()
    return res, (t_fwd, t_stats, t_out)


def bench_sweep(api, torch, timer, steps, warmup):
    """Block-sparsity sweep: the clustered L = 8192 generator with 64 ... 1
    cluster runs per head.  Fits t = t0 + t1 * (non-null tile fraction): t0 is
    the part every configuration pays (the dense score sweep), t1 the part
    that scales with the non-null tiles ("AdaSplash-2: Faster Differentiable
    Sparse Attention", sec. 4.2: runtime falling with block sparsity)."""
    from adaptive_sparse_attention_row_amd.workloads import sweep_configs
    pts = []
    for cfg in sweep_configs():
        r, _ = bench_attn(api, torch, timer, cfg, steps, warmup)
        frac = r["nonnull_tiles_64"] / r["structural_tiles_64"]
        pts.append({"workload": cfg.name, "clusters": cfg.clusters, "nonnull_fraction": round(frac, 5),
                    "fwd_ms": r["fwd_ms"], "score_stats_ms": r["score_stats_ms"], "solve_ms": r["solve_ms"],
                    "output_ms": r["output_ms"], "dense_equiv_tflops": r["dense_equiv_tflops"]})
        log(f"sweep {cfg.name}: non-null {frac:.4f} fwd {r['fwd_ms']:.4f} ms")
    n = len(pts)
    xs = [p["nonnull_fraction"] for p in pts]
    ys = [p["fwd_ms"] for p in pts]
    mx, my = sum(xs) / n, sum(ys) / n
    sxx = sum((x - mx) ** 2 for x in xs)
    t1 = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sxx if sxx > 0 else 0.0
    t0 = my - t1 * mx
    return {"points": pts, "fit_ms": {"t0": round(t0, 5), "t1_per_unit_fraction": round(t1, 5)}}


DECODE_WORKLOADS = [
    # (name, B, H, L, d, mask, window): a long causal cache, and the GPT-2 style
    # window of 32 recent keys plus the sink
    ("decode_B16H16L16384d128_causal", 16, 16, 16384, 128, 1, 0),
    ("decode_B16H12L4096d64_window32_sink", 16, 12, 4096, 64, 2, 32),
]


def bench_decode(api, torch, timer, steps, warmup):
    """One decode step (the query at position L - 1 over a bf16 KV cache).
    HBM-bound: the algorithmic bytes are the K rows of the active keys, the V
    rows of the support only, the query, o and tau.  The support size comes
    from the step's own score row (workspace) and tau."""
    from adaptive_sparse_attention_row_amd.workloads import gen_attn
    out = {}
    lib = api.lib()
    for name, B, H, L, d, mask, W in DECODE_WORKLOADS:
        g = torch.Generator("cpu").manual_seed(60)
        K = torch.randn(B, H, L, d, generator=g).to(torch.bfloat16).cuda()
        V = torch.randn(B, H, L, d, generator=g).to(torch.bfloat16).cuda()
        q = torch.randn(B, H, d, generator=g).to(torch.bfloat16).cuda()
        o = torch.empty(B, H, d, device="cuda")
        tau = torch.empty(B, H, device="cuda")
        wsb = lib.entmax_attn_decode_workspace(B, H, L, d, 1, mask, W)
        ws = torch.empty(wsb // 4, device="cuda")
        st = api._stream(q.device)
        sc = 1.0 / math.sqrt(d)

        def step():
            r = lib.entmax_attn_decode(q.data_ptr(), K.data_ptr(), V.data_ptr(), o.data_ptr(), tau.data_ptr(),
                                       B, H, L, L, d, sc, 1.5, 1, mask, W, ws.data_ptr(), wsb, st)
            assert r == 0, api.status_str(r)

        t = timer(step, max(steps, 20), warmup)
        nact = wsb // 4 // (B * H)
        sup = int((ws.view(B * H, nact) > tau.view(B * H, 1)).sum().item())
        algo = B * H * nact * d * 2 + sup * d * 2 + B * H * d * (2 + 4) + B * H * 4
        gbs = algo / (t * 1e-3) / 1e9
        out[name] = {"ms": round(t, 5), "active_keys_per_head": nact, "support_mean": round(sup / (B * H), 1),
                     "algorithmic_bytes": algo, "GB_per_s": round(gbs, 1),
                     "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                                  "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)},
                     "dense_decode_bytes": B * H * nact * d * 2 * 2}
        del K, V, q, ws
        torch.cuda.empty_cache()
    return out


def bench_wide_rows(api, torch, timer, steps, warmup):
    """Rows wider than 8192 that are dense (every score within reach of the
    maximum, so the candidates overflow the LDS list and each refinement
    step re-reads the row): the streaming row kernel with and without the
    histogram-initialised bracket (AdaSplash-2 sec. 3.1)."""
    rows, cols = 2048, 32768
    g = torch.Generator("cpu").manual_seed(61)
    S = (0.02 * torch.randn(rows, cols, generator=g)).cuda()
    P = torch.empty_like(S)
    tau = torch.empty(rows, device="cuda")
    lib = api.lib()
    st = api._stream(S.device)

    def run():
        r = lib.entmax_tau_rows(S.data_ptr(), P.data_ptr(), tau.data_ptr(), rows, cols, cols, 1.5, st)
        assert r == 0, api.status_str(r)

    out = {"workload": f"rows{rows}x{cols}_f32_dense (0.02 N(0, 1))"}
    for hist in (1, 0):
        prev = api.set_option(api.OPT_ROW_HISTOGRAM, hist)
        try:
            t = timer(run, max(steps // 2, 5), 2)
        finally:
            api.set_option(api.OPT_ROW_HISTOGRAM, prev)
        out["histogram_ms" if hist else "bracket_only_ms"] = round(t, 5)
    del S, P
    torch.cuda.empty_cache()
    return out


def bench_alpha(api, torch, timer, steps, warmup):
    """The clustered L = 8192 forward and the 8192 x 8192 row kernel at
    alpha = 1.25 and alpha = 2 (sparsemax): the general-alpha paths (Newton
    solves, pow weights) next to the alpha = 1.5 numbers."""
    from adaptive_sparse_attention_row_amd.workloads import C4
    out = {}
    for a in (1.25, 2.0):
        r, _ = bench_attn(api, torch, timer, C4, steps, warmup, alpha=a)
        out[f"c4_alpha{a}"] = {k: r[k] for k in ("fwd_ms", "score_stats_ms", "solve_ms", "output_ms",
                                                  "dense_equiv_tflops", "block_sparsity_64")}
        t = bench_tau_rows(api, torch, timer, steps, warmup, alpha=a)
        out[f"c2_alpha{a}"] = {"ms": t["ms"], "GB_per_s": t["GB_per_s"]}
    return out


def bench_tau_rows(api, torch, timer, steps, warmup, alpha=1.5):
    from adaptive_sparse_attention_row_amd.workloads import C2, gen_rows
    S0 = gen_rows(C2.rows, C2.cols, C2.seed).cuda()
    sets = [S0] + [S0.roll(i + 1, 0).contiguous() for i in range(2)]
    Ps = [torch.empty_like(S0) for _ in range(3)]
    taus = [torch.empty(C2.rows, device="cuda") for _ in range(3)]
    lib = api.lib()
    st = api._stream(S0.device)
    it = [0]

    def run():
        i = it[0] % 3
        it[0] += 1
        r = lib.entmax_tau_rows(sets[i].data_ptr(), Ps[i].data_ptr(), taus[i].data_ptr(), C2.rows, C2.cols,
                                C2.cols, alpha, st)
        assert r == 0, api.status_str(r)

    t = timer(run, max(steps, 30), warmup)
    algo_bytes = 4 * C2.rows * C2.cols * 2 + 4 * C2.rows
    gbs = algo_bytes / (t * 1e-3) / 1e9
    del sets, Ps, taus, S0
    torch.cuda.empty_cache()
    return {
        "workload": C2.name,
        "ms": round(t, 5),
        "algorithmic_bytes": algo_bytes,
        "GB_per_s": round(gbs, 1),
        "roofline": {
            "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4),
            "traffic": counter_traffic("tau_rows_c2", TAUROWS_SOURCES),
        },
    }


COPY_BYTES = 256 << 20  # per direction


def bench_copy(torch, timer, steps, warmup):
    """A plain device-to-device copy of COPY_BYTES (3 rotating buffer pairs):
    the reference for scaling the HBM byte counters of the kernels."""
    n = COPY_BYTES // 4
    xs = [torch.randn(n, device="cuda") for _ in range(3)]
    ys = [torch.empty_like(xs[0]) for _ in range(3)]
    it = [0]

    def run():
        i = it[0] % 3
        it[0] += 1
        ys[i].copy_(xs[i])

    t = timer(run, steps, warmup)
    return {"workload": "device copy", "bytes_each_way": COPY_BYTES, "ms": round(t, 5),
            "GB_per_s": round(2 * COPY_BYTES / (t * 1e-3) / 1e9, 1)}


def read_counter_csv(path, kernel_substr, counter):
    """Mean per-dispatch value of `counter` over the dispatches of kernels
    whose name contains kernel_substr, from a rocprofv3 counter_collection.csv."""
    import csv
    vals = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"{path}: no {counter} rows for kernels matching {kernel_substr!r}")
    return sum(vals) / len(vals), len(vals)


def counters_summary(args):
    """Scale FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of a kernel by what the
    same counters read for the copy of known size, and record the HBM bytes
    per launch with the digest of the kernel's sources."""
    sources = {"stats": STATS_SOURCES, "taurows": TAUROWS_SOURCES}[args.sources]
    kf, nkf = read_counter_csv(args.fetch_csv, args.kernel, "FETCH_SIZE")
    kw, nkw = read_counter_csv(args.write_csv, args.kernel, "WRITE_SIZE")
    cf, _ = read_counter_csv(args.copy_fetch_csv, args.copy_kernel, "FETCH_SIZE")
    cw, _ = read_counter_csv(args.copy_write_csv, args.copy_kernel, "WRITE_SIZE")
    ff = COPY_BYTES / 1024.0 / cf   # true KiB per counted KiB, reads
    fw = COPY_BYTES / 1024.0 / cw   # same, writes
    fetch_b = kf * ff * 1024.0
    write_b = kw * fw * 1024.0
    rec = {
        "kernel": args.kernel,
        "source_digest": source_digest(sources),
        "fetch_kib_per_dispatch": round(kf, 1), "write_kib_per_dispatch": round(kw, 1),
        "dispatches": [nkf, nkw],
        "copy_fetch_kib": round(cf, 1), "copy_write_kib": round(cw, 1),
        "scale_fetch": round(ff, 4), "scale_write": round(fw, 4),
        "hbm_fetch_bytes_per_launch": int(fetch_b), "hbm_write_bytes_per_launch": int(write_b),
        "hbm_bytes_per_launch": int(fetch_b + write_b),
    }
    out = os.path.join(ROOT, "profiles", f"{args.counters_summary}.counters.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    with open(os.path.join(ROOT, "profiles", f"{args.counters_summary}.counters.md"), "w") as f:
        f.write(f"# HBM traffic of `{args.kernel}`\n\n")
        f.write("Commands (from /tmp with TMPDIR=/tmp; R = repository root; one counter per run):\n\n```\n")
        f.write(args.commands.replace(";;", "\n") + "\n```\n\n")
        f.write("| | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch |\n|---|---|---|\n")
        f.write(f"| kernel | {kf:.1f} | {kw:.1f} |\n")
        f.write(f"| copy of {COPY_BYTES >> 20} MiB each way | {cf:.1f} | {cw:.1f} |\n\n")
        f.write(f"Scale (true/counted): fetch {ff:.4f}, write {fw:.4f}.  HBM bytes per launch: "
                f"{int(fetch_b)} read + {int(write_b)} written = {int(fetch_b + write_b)}.\n")
    print(json.dumps(rec))


def cpu_baseline(cfg, target_s=15.0):
    """The fp64 oracle on evenly spaced query rows of the same workload."""
    import numpy as np
    import oracle
    from adaptive_sparse_attention_row_amd.workloads import gen_config
    oracle.build(force=False)
    inp = gen_config(cfg)
    Q, K, V = (inp[n].float().numpy() for n in ("q", "k", "v"))
    total = cfg.B * cfg.H * cfg.L
    probe = np.linspace(0, total - 1, 256).astype(np.int64)
    t0 = time.perf_counter()
    oracle.attn_fwd(Q, K, V, cfg.scale, cfg.mask, cfg.window, rows=probe)
    per_row = (time.perf_counter() - t0) / probe.size
    n = int(min(total, max(256, target_s / max(per_row, 1e-9))))
    rows = np.linspace(0, total - 1, n).astype(np.int64)
    t0 = time.perf_counter()
    oracle.attn_fwd(Q, K, V, cfg.scale, cfg.mask, cfg.window, rows=rows)
    dt = time.perf_counter() - t0
    flops = 4 * cfg.d * n * cfg.L  # dense-equivalent, same accounting as the GPU line
    return {
        "value": round(flops / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{n} of {total} query rows (evenly spaced over all heads) of {cfg.name}, "
                  f"fp64 exact tau + dense A.V, {dt:.1f} s wall",
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="time only the headline workload")
    ap.add_argument("--only", choices=["c2", "c3", "c4", "c5", "sweep", "alpha", "decode", "wide", "copy"],
                    default=None,
                    help="run one workload only (for profiler passes); prints its record")
    ap.add_argument("--counters-summary", metavar="NAME", default=None,
                    help="write profiles/NAME.counters.{json,md} from rocprofv3 counter CSVs (no GPU)")
    ap.add_argument("--kernel", default=None, help="kernel name substring (with --counters-summary)")
    ap.add_argument("--sources", choices=["stats", "taurows"], default="stats")
    ap.add_argument("--fetch-csv")
    ap.add_argument("--write-csv")
    ap.add_argument("--copy-fetch-csv")
    ap.add_argument("--copy-write-csv")
    ap.add_argument("--copy-kernel", default="copyBuffer")
    ap.add_argument("--commands", default="", help="the profiling commands, ';;'-separated")
    args = ap.parse_args()
    if args.counters_summary is not None:
        counters_summary(args)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding across GPUs is described in DESIGN.md, not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch
    from adaptive_sparse_attention_row_amd import api
    from adaptive_sparse_attention_row_amd.workloads import C3A, C3B, C4, C5
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    api.lib()
    timer = Timer(torch)
    log(f"device: {torch.cuda.get_device_name(0)}")
    if args.only is not None:
        if args.only == "copy":
            rec = bench_copy(torch, timer, args.steps, args.warmup)
        elif args.only == "c2":
            rec = bench_tau_rows(api, torch, timer, args.steps, args.warmup)
        elif args.only == "c3":
            rec = {C3A.name: bench_attn(api, torch, timer, C3A, args.steps, args.warmup)[0],
                   C3B.name: bench_attn(api, torch, timer, C3B, args.steps, args.warmup)[0]}
        elif args.only == "c4":
            rec = bench_attn(api, torch, timer, C4, args.steps, args.warmup)[0]
        elif args.only == "sweep":
            rec = bench_sweep(api, torch, timer, args.steps, args.warmup)
        elif args.only == "alpha":
            rec = bench_alpha(api, torch, timer, args.steps, args.warmup)
        elif args.only == "decode":
            rec = bench_decode(api, torch, timer, args.steps, args.warmup)
        elif args.only == "wide":
            rec = bench_wide_rows(api, torch, timer, args.steps, args.warmup)
        else:
            rec = bench_attn(api, torch, timer, C5, args.steps, args.warmup, with_bwd=True)[0]
        print(json.dumps({"only": args.only, "record": rec}), flush=True)
        return

    t_wall0 = time.perf_counter()
    head, (t_fwd, t_stats, t_out) = bench_attn(api, torch, timer, C4, args.steps, args.warmup)
    log(f"c4 fwd {head['fwd_ms']:.4f} ms  stats {t_stats:.4f} ms  solve {head['solve_ms']:.4f} ms  output {t_out:.4f} ms  "
        f"{head['dense_equiv_tflops']} TFLOP/s dense-eq, block sparsity {head['block_sparsity_64']}")

    d, pairs = C4.d, head["pairs"]
    achieved = 2 * d * pairs / (t_stats * 1e-3) / 1e12
    roofline = {
        "kernel": "fwd_stats_kernel (entmax_attn_score_stats: the dense MFMA score sweep)",
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": counter_traffic("fwd_stats_c4", STATS_SOURCES),
        "algorithmic_flop_per_launch": 2 * d * pairs,
    }

    extras = {}
    if not args.no_extras:
        extras["c2_tau_rows"] = bench_tau_rows(api, torch, timer, args.steps, args.warmup)
        log(f"c2 tau_rows {extras['c2_tau_rows']['ms']} ms {extras['c2_tau_rows']['GB_per_s']} GB/s")
        for cfg in (C3A, C3B):
            extras[cfg.name], _ = bench_attn(api, torch, timer, cfg, args.steps, args.warmup)
            log(f"{cfg.name}: {extras[cfg.name]}")
        extras[C5.name], _ = bench_attn(api, torch, timer, C5, max(2, args.steps // 4), 2, with_bwd=True)
        log(f"{C5.name}: {extras[C5.name]}")
        extras["sparsity_sweep"] = bench_sweep(api, torch, timer, args.steps, args.warmup)
        log(f"sparsity sweep fit: {extras['sparsity_sweep']['fit_ms']}")
        extras["general_alpha"] = bench_alpha(api, torch, timer, args.steps, args.warmup)
        log(f"general alpha: {extras['general_alpha']}")
        extras["decode"] = bench_decode(api, torch, timer, args.steps, args.warmup)
        log(f"decode: {extras['decode']}")
        extras["wide_dense_rows"] = bench_wide_rows(api, torch, timer, args.steps, args.warmup)
        log(f"wide dense rows: {extras['wide_dense_rows']}")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(C4)
        log(f"cpu baseline: {cpu}")

    value = head["dense_equiv_tflops"]
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["fwd_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": C4.name, "B": C4.B, "H": C4.H, "L": C4.L, "d": C4.d, "mask": "none",
                   "scale": C4.scale, "clusters": C4.clusters, "parallelism": "single GPU"},
        "block_sparsity_64": head["block_sparsity_64"],
        "c4_fwd": head,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "paths": extras,
        "bench_wall_s": round(time.perf_counter() - t_wall0, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
