#!/usr/bin/env python3
"""Benchmark of the 1.5-entmax attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A timed step is one full forward (threshold + block mask + sparse output) of
the long-context workload: B=1, H=12, L=8192, d=64, bf16, 64 clustered
centroids, no mask.  The metric is its effective (dense-equivalent)
throughput, 4*d*pairs / time.  For bf16 inputs the forward is one kernel
launch (the fused score sweep, threshold solve and output), so its time is
that kernel's -> the `roofline` object, against the algorithmic matrix work
(one dense score sweep, 2*d*pairs, plus score recompute and A.V on the
non-null 64x64 tiles, 4*d*pairs*non-null fraction).  The same run also
times, each with HIP events on the stream the library launches on:
  * the score sweep alone (entmax_attn_score_stats, 2*d*pairs FLOP) ->
    `roofline_score_sweep`;
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
PEAK_F32_TFLOPS = 157.3     # MI355X fp32 matrix / vector, published
METRIC = "1.5-entmax attn fwd ms + effective TFLOP/s at L=8192; tau-row kernel GB/s"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


FWD_SOURCES = ["adaptive_sparse_attention_row_amd/csrc/attn_fwd.hip",
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
    """HIP-event timing of a callable on torch's current stream (the stream the
    library is handed).  First an event before the first call and after every
    call, so each call's duration is the gap between consecutive events (the
    median and minimum come from these).  Then the same number of calls
    back to back between two events only: their mean is the launch duration
    a kernel trace reports (an event between every two calls adds a gap of a
    few microseconds).  Returns the median in ms; `last` keeps the median,
    minimum, per-call-event mean and batched mean."""

    def __init__(self, torch):
        self.torch = torch
        self.last = None

    def __call__(self, fn, steps, warmup):
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        st = torch.cuda.current_stream()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        ev[0].record(st)
        for i in range(steps):
            fn()
            ev[i + 1].record(st)
        torch.cuda.synchronize()
        d = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
        med = d[len(d) // 2] if len(d) % 2 else 0.5 * (d[len(d) // 2 - 1] + d[len(d) // 2])
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        for i in range(steps):
            fn()
        e1.record(st)
        torch.cuda.synchronize()
        self.last = {"median_ms": round(med, 5), "min_ms": round(d[0], 5),
                     "event_mean_ms": round(sum(d) / len(d), 5),
                     "mean_ms": round(e0.elapsed_time(e1) / steps, 5), "calls": steps}
        return med


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


def issued_mfma_flop(cfg, ws, bm, scale):
    """Matrix-core FLOPs the forward issues, counted from what its kernels
    sweep (every 64-row x 64-key product is issued whole, masked or not):
      * the score sweep: every (64-row block, key tile) the mask allows, one
        product of 2*64*64*d;
      * the candidate sweep: per 64-row half of a 128-row block, the tiles
        whose largest score beats the smallest lower bound of the half's rows
        (the workspace's row statistics and tile maxima after the call);
      * the output pass: two products (scores again, then A.V) per non-null
        (64-row block, tile) of the blocks whose O the solve kernel did not
        write from its candidate lists (the workspace's per-block flags).
    Sweeps of rows whose lists overflow are not counted.  ws is the workspace
    as a numpy uint8 array after a full forward, laid out as the forward
    kernels lay it out: row statistics [BH][L] (max, lower bound), the
    tile maxima [BH][Tr64][Tc] at the next 256-byte boundary, the candidate
    lists (1 KiB per row of L rounded up to 128), then one int per 128-row
    block."""
    import numpy as np
    BH, L, d = cfg.B * cfg.H, cfg.L, cfg.d
    T = -(-L // 64)
    nQ = -(-L // 128)
    r256 = lambda x: (x + 255) & ~255
    o_um = r256(BH * L * 8)
    o_cl = o_um + r256(BH * T * T * 4)
    o_os = o_cl + r256(BH * nQ * 128 * 128 * 8)
    rowstat = ws[: BH * L * 8].view(np.float32).reshape(BH, L, 2)
    umax = ws[o_um: o_um + BH * T * T * 4].view(np.float32).reshape(BH, T, T) * np.float32(scale)
    ostate = ws[o_os: o_os + BH * nQ * 4].view(np.int32).reshape(BH, nQ)
    unit = 2 * 64 * 64 * d
    stats = structural_tiles(cfg)
    # the (64-row block, tile) pairs the mask allows
    act = np.zeros((T, T), dtype=bool)
    for I in range(T):
        for J in range(T):
            i0, i1, c0, c1 = 64 * I, min(64 * I + 63, L - 1), 64 * J, min(64 * J + 63, L - 1)
            act[I, J] = cfg.mask == 0 or (c0 <= i1 and (cfg.mask == 1 or J == 0 or i0 - c1 <= cfg.window))
    lo = rowstat[:, :, 1]
    pad = np.full((BH, T * 64 - L), np.inf, dtype=np.float32)
    half_min = np.concatenate([lo, pad], axis=1).reshape(BH, T, 64).min(axis=2)   # [BH][Tr64]
    collect = int(((umax > half_min[:, :, None]) & act[None]).sum())
    bits = np.unpackbits(bm.view(np.uint8).reshape(BH, T, -1), axis=2, bitorder="little")[:, :, :T]
    tile_blocks = np.repeat(ostate == 0, 2, axis=1)[:, :T]
    output = int((bits.astype(bool) & tile_blocks[:, :, None]).sum())
    return {"score_sweep": stats * unit, "candidate_sweep": collect * unit, "output": output * 2 * unit,
            "total": (stats + collect + 2 * output) * unit,
            "blocks_from_lists": int((ostate != 0).sum()), "blocks": BH * nQ}


def bench_attn(api, torch, timer, cfg, steps, warmup, with_bwd=False, alpha=1.5, bwd_steps=10):
    """Forward (and backward) timing of one attention workload: the whole
    forward, its threshold half, the score sweep alone, and the output pass
    alone (entmax_attn_output over every block), each the median of `steps`
    calls; plus the MFMA work the forward issued."""
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

    t_stats = timer(stats, steps, warmup)
    stats_t = timer.last
    t_thr = timer(thr, steps, warmup)
    t_out = timer(out, steps, warmup)
    t_fwd = timer(fwd, steps, warmup)   # last: the workspace then holds this call's state
    fwd_t = timer.last
    torch.cuda.synchronize()
    bmn = bm.cpu().numpy()
    nnz = popcount_mask(bmn)
    struct = structural_tiles(cfg)
    pairs = pairs_of(cfg)
    issued = issued_mfma_flop(cfg, ws.cpu().numpy(), bmn, cfg.scale)
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS
    res = {
        "fwd_ms": round(t_fwd, 5),
        "fwd_min_ms": fwd_t["min_ms"],
        "fwd_mean_ms": fwd_t["mean_ms"],
        "threshold_ms": round(t_thr, 5),
        "score_stats_ms": round(t_stats, 5),
        "score_stats_min_ms": stats_t["min_ms"],
        "score_stats_mean_ms": stats_t["mean_ms"],
        "solve_ms": round(t_thr - t_stats, 5),
        "output_pass_alone_ms": round(t_out, 5),
        "after_threshold_ms": round(t_fwd - t_thr, 5),
        "dense_equiv_tflops": round(4 * d * pairs / (t_fwd * 1e-3) / 1e12, 3),
        "score_stats_mfma_tflops": round(2 * d * pairs / (t_stats * 1e-3) / 1e12, 3),
        "issued_mfma_tflop": round(issued["total"] / 1e12, 4),
        "issued_mfma_tflops": round(issued["total"] / (t_fwd * 1e-3) / 1e12, 2),
        "mfma_util_on_issued_work": round(issued["total"] / (t_fwd * 1e-3) / 1e12 / peak, 4),
        "issued_split_tflop": {k2: round(v2 / 1e12, 4) for k2, v2 in issued.items()
                               if k2 in ("score_sweep", "candidate_sweep", "output")},
        "blocks_with_O_from_lists": f"{issued['blocks_from_lists']} of {issued['blocks']}",
        "nonnull_tiles_64": nnz,
        "structural_tiles_64": struct,
        "block_sparsity_64": round(1.0 - nnz / struct, 5),
        "pairs": pairs,
        "calls_per_timing": steps,
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
            assert r == 0, api.status_str(r)

        t_bwd = timer(bwd, bwd_steps, 2)
        res["bwd_ms"] = round(t_bwd, 5)
        res["bwd_min_ms"] = timer.last["min_ms"]
        res["bwd_calls"] = bwd_steps
        res["bwd_dense_equiv_tflops"] = round(10 * d * pairs / (t_bwd * 1e-3) / 1e12, 3)
        res["bwd_12dp_tflops"] = round(12 * d * pairs / (t_bwd * 1e-3) / 1e12, 3)
        res["bwd_frac_of_peak_12dp"] = round(12 * d * pairs / (t_bwd * 1e-3) / 1e12 / peak, 4)
        if cfg.dtype == "bf16" and L <= 16384:
            # the training pair: the forward also writes G.V and sum g, and the
            # backward takes delta from them instead of a pass over the keys
            gvb = torch.empty_like(O)
            gsb = torch.empty_like(tau)

            def fwd_gv():
                r = lib.entmax_attn_fwd_gv(q.data_ptr(), k.data_ptr(), v.data_ptr(), O.data_ptr(),
                                           tau.data_ptr(), bm.data_ptr(), gvb.data_ptr(), gsb.data_ptr(), B, H, L,
                                           d, sc, alpha, dt, cfg.mask, cfg.window, ws.data_ptr(), wsb, st)
                assert r == 0, api.status_str(r)

            def bwd_gv():
                r = lib.entmax_attn_bwd_gv(q.data_ptr(), k.data_ptr(), v.data_ptr(), do.data_ptr(),
                                           tau.data_ptr(), bm.data_ptr(), gvb.data_ptr(), gsb.data_ptr(),
                                           dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, L, d, sc, alpha,
                                           dt, cfg.mask, cfg.window, bws.data_ptr(), bwsb, st)
                assert r == 0, api.status_str(r)

            t_fg = timer(fwd_gv, bwd_steps, 2)
            res["train_fwd_gv_ms"] = round(t_fg, 5)
            t_bg = timer(bwd_gv, bwd_steps, 2)
            res["train_bwd_gv_ms"] = round(t_bg, 5)
            res["train_bwd_gv_min_ms"] = timer.last["min_ms"]
            res["train_bwd_gv_frac_of_peak_12dp"] = round(12 * d * pairs / (t_bg * 1e-3) / 1e12 / peak, 4)
            res["train_step_ms"] = round(t_fg + t_bg, 5)
    del q, k, v, O
    torch.cuda.empty_cache()
    return res, (t_fwd, t_stats, t_out)


def linear_fit(xs, ys):
    """Least squares y = t0 + t1 x, with the coefficient of determination."""
    n = len(xs)
    mx, my = sum(xs) / n, sum(ys) / n
    sxx = sum((x - mx) ** 2 for x in xs)
    t1 = sum((x - mx) * (y - my) for x, y in zip(xs, ys)) / sxx if sxx > 0 else 0.0
    t0 = my - t1 * mx
    ss_res = sum((y - t0 - t1 * x) ** 2 for x, y in zip(xs, ys))
    ss_tot = sum((y - my) ** 2 for y in ys)
    return {"t0": round(t0, 5), "t1_per_unit_fraction": round(t1, 5),
            "r2": round(1.0 - ss_res / ss_tot, 4) if ss_tot > 0 else None}


def sweep_points(api, torch, timer, cfgs, steps, warmup, key):
    pts = []
    for cfg in cfgs:
        r, _ = bench_attn(api, torch, timer, cfg, steps, warmup)
        frac = r["nonnull_tiles_64"] / r["structural_tiles_64"]
        pts.append({"workload": cfg.name, key: getattr(cfg, key), "nonnull_fraction": round(frac, 5),
                    "fwd_ms": r["fwd_ms"], "score_stats_ms": r["score_stats_ms"], "solve_ms": r["solve_ms"],
                    "after_threshold_ms": r["after_threshold_ms"], "dense_equiv_tflops": r["dense_equiv_tflops"],
                    "mfma_util_on_issued_work": r["mfma_util_on_issued_work"],
                    "blocks_with_O_from_lists": r["blocks_with_O_from_lists"]})
        log(f"sweep {cfg.name}: non-null {frac:.4f} fwd {r['fwd_ms']:.4f} ms")
    xs = [p["nonnull_fraction"] for p in pts]
    fits = {ph: linear_fit(xs, [p[ph] for p in pts])
            for ph in ("fwd_ms", "score_stats_ms", "solve_ms", "after_threshold_ms")}
    return {"points": pts, "fit_ms": fits}


def bench_sweep(api, torch, timer, steps, warmup):
    """Block-sparsity sweeps at L = 8192, d = 64, bf16 ("AdaSplash-2: Faster
    Differentiable Sparse Attention", sec. 4.2: runtime falling with block
    sparsity): the clustered generator with 64 ... 1 cluster runs per head,
    and Gaussian Q/K/V with the query standard deviation as the knob (the
    pages' own method; at this length it spans 0 to about 55 % block
    sparsity).  Each fits t = t0 + t1 * (non-null tile fraction) per phase
    (whole forward, score sweep, candidate solve, after the threshold) with
    R^2."""
    from adaptive_sparse_attention_row_amd.workloads import qvar_configs, sweep_configs
    return {"clustered": sweep_points(api, torch, timer, sweep_configs(), steps, warmup, "clusters"),
            "query_variance": sweep_points(api, torch, timer, qvar_configs(), steps, warmup, "q_std")}


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
    maximum, so the candidates overflow any LDS list): 2048 rows of 32768,
    which a workgroup holds in registers (one read, one write per element),
    and 1024 rows of 65536, which are streamed and re-read by every
    refinement step, with and without the histogram-initialised bracket
    (AdaSplash-2 sec. 3.1)."""
    out = {}
    lib = api.lib()
    for rows, cols, hists in ((2048, 32768, (1,)), (1024, 65536, (1, 0))):
        g = torch.Generator("cpu").manual_seed(61)
        S = (0.02 * torch.randn(rows, cols, generator=g)).cuda()
        P = torch.empty_like(S)
        tau = torch.empty(rows, device="cuda")
        st = api._stream(S.device)
        rec = {"workload": f"rows{rows}x{cols}_f32_dense (0.02 N(0, 1))"}
        for hist in hists:
            opts = api._opts(0, row_plain_bracket=not hist)

            def run():
                r = lib.entmax_tau_rows_ex(S.data_ptr(), P.data_ptr(), tau.data_ptr(), rows, cols, cols, 1.5,
                                           opts, st)
                assert r == 0, api.status_str(r)

            t = timer(run, max(steps // 2, 5), 2)
            key = "ms" if len(hists) == 1 else ("histogram_ms" if hist else "bracket_only_ms")
            rec[key] = round(t, 5)
            if len(hists) == 1 or hist:
                rec["GB_per_s"] = round(8 * rows * cols / (timer.last["mean_ms"] * 1e-3) / 1e9, 1)
        out[f"rows{cols}"] = rec
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
        out[f"c4_alpha{a}"] = {k: r[k] for k in ("fwd_ms", "score_stats_ms", "solve_ms", "after_threshold_ms",
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
    tl = timer.last
    algo_bytes = 4 * C2.rows * C2.cols * 2 + 4 * C2.rows
    gbs = algo_bytes / (tl["mean_ms"] * 1e-3) / 1e9
    del sets, Ps, taus, S0
    torch.cuda.empty_cache()
    return {
        "workload": C2.name,
        "ms": round(t, 5),
        "min_ms": tl["min_ms"],
        "mean_launch_ms": tl["mean_ms"],
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
    sources = {"fwd": FWD_SOURCES, "taurows": TAUROWS_SOURCES}[args.sources]
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


def _short_kernel_name(n):
    import re
    import subprocess
    if n.startswith("_Z"):
        # kernel templates over __bf16 (which c++filt does not demangle):
        # <len><name>I<args>E with args DF16b, f, Li<n>E, Lb<0|1>E
        m = re.search(r"_GLOBAL__N_1(\d+)", n)
        if m:
            k = m.end()
            name = n[k:k + int(m.group(1))]
            rest, args = n[k + int(m.group(1)):], []
            if rest.startswith("I"):
                rest = rest[1:]
                while rest and not rest.startswith("E"):
                    a = re.match(r"DF16b|f|Li(\d+)E|Lb([01])E", rest)
                    if not a:
                        break
                    t = a.group(0)
                    args.append("bf16" if t == "DF16b" else "float" if t == "f" else a.group(1) if a.group(1)
                                else ("true" if a.group(2) == "1" else "false"))
                    rest = rest[a.end():]
            n = f"{name}<{', '.join(args)}>" if args else name
        else:
            try:
                n = subprocess.run(["c++filt"], input=n, capture_output=True, text=True,
                                   timeout=10).stdout.strip() or n
            except (OSError, subprocess.SubprocessError):
                pass
    n = re.sub(r"entmax::attn::\(anonymous namespace\)::|entmax::\(anonymous namespace\)::|entmax::", "", n)
    n = re.sub(r"\(FwdParams\)|\(BwdParams\)|\(\w*Params\)", "", n)
    return n.replace("__bf16", "bf16").strip()


def trace_summary(args):
    """profiles/NAME.kernel_trace.md from rocprofv3's kernel_stats.csv."""
    import csv
    rows = list(csv.DictReader(open(args.stats_csv)))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    out = os.path.join(ROOT, "profiles", f"{args.trace_summary}.kernel_trace.md")
    with open(out, "w") as f:
        f.write(f"# Kernel trace: {args.title}\n\n")
        f.write("Command (on the GPU host, from the repository root, TMPDIR=/tmp):\n\n```\n")
        f.write(args.commands.replace(";;", "\n") + "\n```\n\n")
        f.write("From the run's `kernel_stats.csv` (durations in microseconds):\n\n")
        f.write("| kernel | calls | mean | min | max | share |\n|---|---|---|---|---|---|\n")
        for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
            f.write(f"| `{_short_kernel_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                    f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                    f"{100.0 * float(r['TotalDurationNs']) / total:.1f} % |\n")
    print(out)


MFMA_COUNTERS = ["SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_INSTS_VALU_MFMA_MOPS_F16", "SQ_INSTS_MFMA",
                 "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_SALU", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES",
                 "GRBM_GUI_ACTIVE"]


def mfma_summary(args):
    """profiles/NAME.mfma.md: per-dispatch means of the matrix-core and issue
    counters of the named kernels from rocprofv3's counter_collection.csv.
    MOPS counters count matrix operations in units of 512 FLOP."""
    import csv
    recs = {}
    for r in csv.DictReader(open(args.pmc_csv)):
        recs.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], {})[r["Dispatch_Id"]] = \
            float(r["Counter_Value"])
    out = os.path.join(ROOT, "profiles", f"{args.mfma_summary}.mfma.md")
    with open(out, "w") as f:
        f.write(f"# Matrix-core and issue counters: {args.title}\n\n")
        f.write("Command (on the GPU host, from the repository root, TMPDIR=/tmp):\n\n```\n")
        f.write(args.commands.replace(";;", "\n") + "\n```\n\n")
        f.write("Per-dispatch means over the run's dispatches of each kernel.  MFMA FLOP = "
                "(MOPS_BF16 + MOPS_F16) x 512 (for the score sweep this equals 2*d*pairs exactly).  "
                "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs): the busy "
                "counter read as a sum over the SIMDs and GRBM_GUI_ACTIVE as a sum over the XCDs.\n\n")
        f.write("| kernel | dispatches | MFMA GFLOP | MFMA instrs | VALU / MFMA | LDS / MFMA | SALU / MFMA | "
                "MFMA busy |\n|---|---|---|---|---|---|---|---|\n")
        for sub in [k for k in args.kernels.split(";") if k]:
            names = [n for n in recs if sub in n]
            for n in names:
                c = recs[n]
                mean = lambda k: (sum(c[k].values()) / len(c[k])) if k in c and c[k] else float("nan")
                nd = max(len(v) for v in c.values())
                fl = (mean("SQ_INSTS_VALU_MFMA_MOPS_BF16") + mean("SQ_INSTS_VALU_MFMA_MOPS_F16")) * 512
                mf = mean("SQ_INSTS_MFMA")
                f.write(f"| `{_short_kernel_name(n)}` | {nd} | {fl / 1e9:.2f} | {mf:.4g} | "
                        f"{mean('SQ_INSTS_VALU') / mf:.2f} | {mean('SQ_INSTS_LDS') / mf:.2f} | "
                        f"{mean('SQ_INSTS_SALU') / mf:.2f} | "
                        f"{mean('SQ_VALU_MFMA_BUSY_CYCLES') / (1024 * mean('GRBM_GUI_ACTIVE') / 8):.3f} |\n")
        f.write("\nRaw per-dispatch means:\n\n| kernel | " + " | ".join(MFMA_COUNTERS) + " |\n|---|" +
                "---|" * len(MFMA_COUNTERS) + "\n")
        for sub in [k for k in args.kernels.split(";") if k]:
            for n in [n for n in recs if sub in n]:
                c = recs[n]
                vals = [(sum(c[k].values()) / len(c[k])) if k in c and c[k] else float("nan") for k in MFMA_COUNTERS]
                f.write(f"| `{_short_kernel_name(n)}` | " + " | ".join(f"{v:.4g}" for v in vals) + " |\n")
    print(out)


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


def oracle_timings():
    """Wall time of the fp64 oracle on bounded samples of the other workloads,
    on the host cores (the same threads as the CPU baseline): C2 rows, C5
    forward rows, and one whole head of the C5 backward."""
    import numpy as np
    import oracle
    from adaptive_sparse_attention_row_amd.workloads import C2, C5, gen_config, gen_rows
    oracle.build(force=False)
    out = {"cores": oracle.num_threads()}
    S = gen_rows(1024, C2.cols, C2.seed).numpy()
    t0 = time.perf_counter()
    oracle.tau_rows(S)
    dt = time.perf_counter() - t0
    out["c2_rows"] = {"sample": f"1024 of {C2.rows} rows of {C2.name}", "s": round(dt, 3),
                      "rows_per_s": round(1024 / dt, 1), "GB_per_s": round(1024 * C2.cols * 8 / dt / 1e9, 3)}
    inp = gen_config(C5, H=1)
    Q, K, V, dO = (inp[n].float().numpy() for n in ("q", "k", "v", "do"))
    rows = np.linspace(0, C5.L - 1, 2048).astype(np.int64)
    t0 = time.perf_counter()
    oracle.attn_fwd(Q, K, V, C5.scale, C5.mask, C5.window, rows=rows)
    dt = time.perf_counter() - t0
    pairs = int((rows + 1).sum())
    out["c5_fwd_rows"] = {"sample": f"2048 evenly spaced query rows of one head of {C5.name}", "s": round(dt, 3),
                          "dense_equiv_tflops": round(4 * C5.d * pairs / dt / 1e12, 6)}
    t0 = time.perf_counter()
    oracle.attn_bwd_head(Q[0, 0], K[0, 0], V[0, 0], dO[0, 0], C5.scale, C5.mask, C5.window)
    dt = time.perf_counter() - t0
    pairs = C5.L * (C5.L + 1) // 2
    out["c5_bwd_head"] = {"sample": f"the full backward of one head of {C5.name}", "s": round(dt, 3),
                          "dense_equiv_tflops": round(10 * C5.d * pairs / dt / 1e12, 6)}
    return out


def gpu_clock():
    """The GPU's current and peak shader clock as rocm-smi reports them (None
    where the tool or the field is missing)."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True, timeout=20)
        rec = json.loads(r.stdout)
        card = next(iter(rec.values()))
        return {k: v for k, v in card.items() if "sclk" in k.lower() or "fclk" in k.lower() or "mclk" in k.lower()}
    except Exception as e:  # the clock is reported, not required
        return {"error": str(e)[:120]}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="time only the headline workload")
    ap.add_argument("--only", choices=["c1", "c2", "c3", "c4", "c5", "sweep", "alpha", "decode", "wide", "copy"],
                    default=None,
                    help="run one workload only (for profiler passes); prints its record")
    ap.add_argument("--counters-summary", metavar="NAME", default=None,
                    help="write profiles/NAME.counters.{json,md} from rocprofv3 counter CSVs (no GPU)")
    ap.add_argument("--kernel", default=None, help="kernel name substring (with --counters-summary)")
    ap.add_argument("--sources", choices=["fwd", "taurows"], default="fwd")
    ap.add_argument("--fetch-csv")
    ap.add_argument("--write-csv")
    ap.add_argument("--copy-fetch-csv")
    ap.add_argument("--copy-write-csv")
    ap.add_argument("--copy-kernel", default="copyBuffer")
    ap.add_argument("--commands", default="", help="the profiling commands, ';;'-separated")
    ap.add_argument("--trace-summary", metavar="NAME", default=None,
                    help="write profiles/NAME.kernel_trace.md from a rocprofv3 kernel_stats.csv (no GPU)")
    ap.add_argument("--stats-csv")
    ap.add_argument("--mfma-summary", metavar="NAME", default=None,
                    help="write profiles/NAME.mfma.md from a rocprofv3 counter_collection.csv (no GPU)")
    ap.add_argument("--pmc-csv")
    ap.add_argument("--kernels", default="", help="';'-separated kernel name substrings (with --mfma-summary)")
    ap.add_argument("--title", default="")
    args = ap.parse_args()
    if args.counters_summary is not None:
        counters_summary(args)
        return
    if args.trace_summary is not None:
        trace_summary(args)
        return
    if args.mfma_summary is not None:
        mfma_summary(args)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(sharding across GPUs is described in DESIGN.md, not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch
    from adaptive_sparse_attention_row_amd import api
    from adaptive_sparse_attention_row_amd.workloads import C1, C3A, C3B, C4, C5
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    api.lib()
    timer = Timer(torch)
    log(f"device: {torch.cuda.get_device_name(0)}")
    if args.only is not None:
        if args.only == "copy":
            rec = bench_copy(torch, timer, args.steps, args.warmup)
        elif args.only == "c1":
            rec = bench_attn(api, torch, timer, C1, args.steps, args.warmup)[0]
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
            rec = bench_attn(api, torch, timer, C5, args.steps, args.warmup, with_bwd=True, bwd_steps=args.steps)[0]
        print(json.dumps({"only": args.only, "record": rec}), flush=True)
        return

    t_wall0 = time.perf_counter()
    clock_before = gpu_clock()
    head, (t_fwd, t_stats, t_out) = bench_attn(api, torch, timer, C4, args.steps, args.warmup)
    log(f"c4 fwd {head['fwd_ms']:.4f} ms  stats {t_stats:.4f} ms  solve {head['solve_ms']:.4f} ms  output {t_out:.4f} ms  "
        f"{head['dense_equiv_tflops']} TFLOP/s dense-eq, block sparsity {head['block_sparsity_64']}")

    d, pairs = C4.d, head["pairs"]
    # the forward is one launch of the fused kernel; its algorithmic work is
    # the dense score sweep plus recompute and A.V over the non-null tiles
    nonnull_frac = head["nonnull_tiles_64"] / head["structural_tiles_64"]
    alg = int(2 * d * pairs + 4 * d * pairs * nonnull_frac)
    t_fwd_mean = head["fwd_mean_ms"]
    achieved = alg / (t_fwd_mean * 1e-3) / 1e12
    roofline = {
        "kernel": "fwd_fused_kernel<64, 128, false> (entmax_attn_fwd: score sweep, threshold solve and "
                  "sparse output in one launch)",
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
        "traffic": counter_traffic("fwd_fused_c4", FWD_SOURCES),
        "algorithmic_flop_per_launch": alg,
        "flop_accounting": "2*d*pairs (dense score sweep) + 4*d*pairs*non-null 64x64 tile fraction "
                           "(score recompute and A.V on the non-null tiles), over the mean launch time",
        "mean_launch_ms": t_fwd_mean,
    }
    achieved_s = 2 * d * pairs / (head["score_stats_mean_ms"] * 1e-3) / 1e12
    roofline_sweep = {
        "kernel": "fwd_stats_kernel<bf16, 64, 128, false> (entmax_attn_score_stats: the dense score sweep alone)",
        "bound": "mfma",
        "achieved": round(achieved_s, 2),
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": round(achieved_s / PEAK_BF16_TFLOPS, 4),
        "algorithmic_flop_per_launch": 2 * d * pairs,
        "mean_launch_ms": head["score_stats_mean_ms"],
    }

    extras = {}
    if not args.no_extras:
        extras[C1.name], _ = bench_attn(api, torch, timer, C1, args.steps, args.warmup)
        log(f"{C1.name}: fwd {extras[C1.name]['fwd_ms']} ms")
        extras["c2_tau_rows"] = bench_tau_rows(api, torch, timer, args.steps, args.warmup)
        log(f"c2 tau_rows {extras['c2_tau_rows']['ms']} ms {extras['c2_tau_rows']['GB_per_s']} GB/s")
        for cfg in (C3A, C3B):
            extras[cfg.name], _ = bench_attn(api, torch, timer, cfg, args.steps, args.warmup)
            log(f"{cfg.name}: {extras[cfg.name]}")
        extras[C5.name], _ = bench_attn(api, torch, timer, C5, 10, 2, with_bwd=True, bwd_steps=10)
        log(f"{C5.name}: {extras[C5.name]}")
        extras["sparsity_sweep"] = bench_sweep(api, torch, timer, args.steps, args.warmup)
        log(f"sparsity sweep fits: {[(k, v['fit_ms']['fwd_ms']) for k, v in extras['sparsity_sweep'].items()]}")
        extras["general_alpha"] = bench_alpha(api, torch, timer, args.steps, args.warmup)
        log(f"general alpha: {extras['general_alpha']}")
        extras["decode"] = bench_decode(api, torch, timer, args.steps, args.warmup)
        log(f"decode: {extras['decode']}")
        extras["wide_dense_rows"] = bench_wide_rows(api, torch, timer, args.steps, args.warmup)
        log(f"wide dense rows: {extras['wide_dense_rows']}")

    clock_after = gpu_clock()
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(C4)
        log(f"cpu baseline: {cpu}")
        if not args.no_extras:
            extras["oracle_other_workloads"] = oracle_timings()
            log(f"oracle timings: {extras['oracle_other_workloads']}")

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
        "roofline_score_sweep": roofline_sweep,
        "cpu_baseline": cpu,
        "timing": "HIP events around every call on the library's stream; ms values are medians "
                  "(the *_min_ms fields the minima) of `steps` calls after `warmup` calls (C5: 10 of each)",
        "gpu_clock": {"before": clock_before, "after": clock_after},
        "paths": extras,
        "bench_wall_s": round(time.perf_counter() - t_wall0, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
