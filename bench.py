#!/usr/bin/env python3
"""Benchmark: CRISP sparse prefill attention on one MI355X.

One step = the whole path on one synthetic layer already resident in HBM:
crisp_prefill = proxy attention + routing + index selection + block-sparse
attention, every head.  The workload is the Llama-3.1-8B-shaped layer at
512k tokens (32 query / 8 KV heads, d = 128, b = 128, tau 0.3, alpha 1,
gamma 0.95, length-compensated generator).  Printed as one JSON line:

  value          ms per layer (time-like: lower is better)
  speedup        dense causal attention on the same tile engine / value
  stages         select and sparse-attention ms from HIP events
  roofline       the sparse attention kernel: executed-tile MFMA flops per
                 launch / its launch time (HIP events on the launch stream),
                 against the 2.5 PFLOP/s dense bf16 peak
  step_ms        per-step HIP-event times: warm, and after a 512 MiB write
                 that flushes L2 / MALL (median and min)
  selection_roofline  the selection stage against max(HBM, MFMA)
  rules          the decision rules the pages compare, on the same layer:
                 median floor, universal configuration, FlexPrefill's pair
  cpu_baseline   the CPU oracle on a bounded sample of the same layer,
                 extrapolated to ms per layer
  extra          the 128k layers (Llama and Qwen shaped), a 4k-64k
                 length sweep (CRISP vs dense, the length gate) and packed
                 batches of 512k tokens (one varlen call vs one call each)

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-extra] [--no-compare] [--no-sweep]
                       [--no-varlen]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

TILE_FLOPS = 4 * 128 * 128 * 128          # QK^T + PV for one 128 x 128 tile at d = 128
# causal part of a diagonal tile: query row r sees keys 0..r, 129/256 of the tile's pairs
DIAG_USEFUL = 129 / 256
PEAK_BF16_TFLOPS = 2500.0                  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0
# VALU model of the chip (256 CUs at 2.4 GHz, 4 SIMDs of 16 lanes each): a
# full-rate vector op costs one lane-cycle per lane, v_exp_f32 two (measured on
# gfx950: 8 clocks per wave64 instruction against 4 for v_fma_f32, and the two
# do not issue together); 64 lane-cycles per clock per CU.
CU, CLOCK_GHZ, LANE_CYCLES_PER_CLK = 256, 2.4, 64
EXP_LANE_CYCLES = 2


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def profiled_traffic():
    """HBM bytes per launch of the sparse attention kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary, if it was taken on the current
    kernel source (matching sha256 prefix of attn.hip); otherwise None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "attention_llama512k_hbm_counters.txt")
    src = os.path.join(ROOT, "dynamic_sparse_prefill_amd", "csrc", "attn.hip")
    try:
        text = open(path).read()
        want = hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]
    except OSError:
        return None
    if f"attn.hip sha256:{want}" not in text:
        return None
    for line in text.splitlines():
        if line.startswith("sparse attention traffic_bytes_per_launch:"):
            return int(line.split(":")[1].split()[0])
    return None


def timed(fn, steps, warmup, torch):
    """Mean ms per call over `steps` calls after `warmup`, bracketed by device syncs."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        fn()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def event_ms(fn, reps, torch):
    """Mean ms per call from HIP events recorded on the current stream (the launch stream)."""
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / reps


def step_events(fn, reps, torch, flush=None):
    """Per-call ms from HIP events on the launch stream, optionally writing a
    512 MiB buffer (L2 / MALL flush) before each call, outside the events."""
    out = []
    for _ in range(reps):
        if flush is not None:
            flush.fill_(1)
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        e.synchronize()
        out.append(s.elapsed_time(e))
    return out


def head_mix(spec, sel_route, c_struct):
    """Route counts of a layer against how its heads were generated, and the
    C_struct distribution (so a reader sees which heads the router sent where)."""
    conc = np.asarray(spec.concentrated, bool)
    edges = [0.0, 0.01, 0.05, 0.1, 0.2, 0.3, 0.5, 0.75, 1.0001]
    hist, _ = np.histogram(np.asarray(c_struct, np.float64), bins=edges)
    return {"vs": int((sel_route == 1).sum()), "pe": int((sel_route == 0).sum()),
            "dense": int((sel_route == -1).sum()),
            "concentrated": int(conc.sum()), "concentrated_to_vs": int(((sel_route == 1) & conc).sum()),
            "diffuse_to_pe": int(((sel_route == 0) & ~conc).sum()),
            "c_struct_hist": {f"[{a:g},{min(b, 1.0):g})": int(c) for a, b, c in zip(edges[:-1], edges[1:], hist)},
            "c_struct_min_max": [round(float(np.min(c_struct)), 4), round(float(np.max(c_struct)), 4)]}


def selection_stage_bounds(cfg, route, tiles):
    """Lower bounds of the selection's stages from their algorithmic work.
    proxy: K once (HBM), 2*128*n*d flops per query head (bf16 MFMA) and, per
    score, one v_exp_f32 (EXP_LANE_CYCLES lane-cycles) plus three full-rate ops
    (scale and shift, sum, max): the VALU bound is the largest of the three.
    Pooled estimation: Q of the PE heads once (pooling), pooled logits on the
    bf16 matrix unit as six bf16 products per float32 product (the three-part
    split: 6 * 2 * d flops per causal block pair), the pooled matrix written
    once and read by the cut.  Lists: 4 bytes per entry written."""
    nb = cfg.n // 128
    h_pe = int((route == 0).sum())
    tri = nb * (nb + 1) // 2
    scores = cfg.hq * 128 * cfg.n
    proxy = {"hbm_ms": cfg.hkv * cfg.n * 128 * 2 / (PEAK_HBM_GBS * 1e9) * 1e3,
             "mfma_ms": 2 * 128 * cfg.n * 128 * cfg.hq / (PEAK_BF16_TFLOPS * 1e12) * 1e3,
             "valu_ms": scores * (EXP_LANE_CYCLES + 3) / (CU * LANE_CYCLES_PER_CLK * CLOCK_GHZ * 1e9) * 1e3}
    pool = {"hbm_ms": h_pe * cfg.n * 128 * 2 / (PEAK_HBM_GBS * 1e9) * 1e3}
    logits = {"mfma_bf16x6_ms": h_pe * tri * 6 * 2 * 128 / (PEAK_BF16_TFLOPS * 1e12) * 1e3,
              "hbm_ms": h_pe * tri * 4 / (PEAK_HBM_GBS * 1e9) * 1e3}
    cut = {"hbm_ms": 2 * h_pe * tri * 4 / (PEAK_HBM_GBS * 1e9) * 1e3}
    lists = {"hbm_ms": 4 * tiles / (PEAK_HBM_GBS * 1e9) * 1e3}
    out = {}
    for name, b in (("proxy_scores", proxy), ("pool_q", pool), ("pooled_logits", logits), ("pooled_cut", cut),
                    ("lists", lists)):
        bound = max(b, key=b.get)
        out[name] = {k: round(v, 4) for k, v in b.items()}
        out[name]["bound"] = bound.replace("_ms", "")
    out["sum_of_bounds_ms"] = round(sum(max(v for k, v in b.items() if k.endswith("_ms"))
                                        for b in (proxy, pool, logits, cut, lists)), 4)
    return out


def selection_roofline(cfg, route, tiles, sel_ms):
    """Selection as a whole against max(HBM, MFMA): algorithmic bytes = K once,
    Q of the Pooled-Estimation heads once, the pooled matrix of those heads
    written once and read twice (softmax + cut), the lists written once; flops =
    one pass of the proxy scores over K (2 * 128 * n * d * hq)."""
    nb = cfg.n // 128
    h_pe = int((route == 0).sum())
    tri = nb * (nb + 1) // 2
    nbytes = cfg.hkv * cfg.n * 128 * 2 + h_pe * cfg.n * 128 * 2 + 3 * 4 * tri * h_pe + 4 * tiles
    flops = 2 * 128 * cfg.n * 128 * cfg.hq
    t_hbm = nbytes / (PEAK_HBM_GBS * 1e9)
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
    return {"bound": "hbm" if t_hbm >= t_mfma else "mfma", "bytes": int(nbytes), "flops": int(flops),
            "achieved_gbs": round(nbytes / (sel_ms * 1e-3) / 1e9, 1),
            "frac_hbm": round(nbytes / (sel_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "roofline_ms": round(max(t_hbm, t_mfma) * 1e3, 4), "frac": round(max(t_hbm, t_mfma) * 1e3 / sel_ms, 4)}


def compare_rules(cfg, q, k, v, dsp, torch, steps, dense_ms):
    """The decision rules the pages compare on one resident layer: CRISP as
    published, its median-floor variant, the universal configuration (min budget
    8, tau 0.2, alpha 1 / 1.25 / 1.5) and FlexPrefill's pair (JSD router,
    coverage budget at gamma 0.95 / 0.97; JSD threshold 0.1).  For each: ms per
    layer, executed-tile density, Vertical-Slash head count, mean per-direction
    budget of the VS heads, and agreement of the route with C_struct routing."""
    J, M, C = dsp.FLAG_ROUTE_JSD, dsp.FLAG_VS_MEDIAN, dsp.FLAG_VS_COVERAGE
    rules = [("crisp", {}), ("crisp-median-floor", dict(flags=M)),
             ("crisp-universal-a1.0", dict(tau=0.2, alpha=1.0, min_blocks=8)),
             ("crisp-universal-a1.25", dict(tau=0.2, alpha=1.25, min_blocks=8)),
             ("crisp-universal-a1.5", dict(tau=0.2, alpha=1.5, min_blocks=8)),
             ("flexprefill-g0.95", dict(tau=0.1, gamma=0.95, flags=J | C)),
             ("flexprefill-g0.97", dict(tau=0.1, gamma=0.97, flags=J | C)),
             ("jsd-router+noise-floor", dict(tau=0.1, flags=J)),
             ("cstruct-router+coverage-g0.95", dict(flags=C))]
    nb = cfg.n // 128
    dense_tiles = cfg.hq * nb * (nb + 1) // 2
    base_route = None
    out = {}
    for name, over in rules:
        p = dsp.CrispParams(tau=cfg.tau, alpha=cfg.alpha, gamma=cfg.gamma)
        for a, b in over.items():
            setattr(p, a, b)
        o = torch.empty_like(q)
        sel = dsp.new_selection(q, k, diagnostics=True)
        ws = torch.empty(dsp.workspace_bytes(dsp.make_shape(q, k, v, o), p), dtype=torch.uint8, device="cuda")
        ms = timed(lambda: dsp.crisp_prefill(q, k, v, p, sel=sel, o=o, ws=ws), steps, 1, torch)
        route = sel.route.cpu().numpy()
        nv, ns = sel.nv.cpu().numpy(), sel.ns.cpu().numpy()
        vs = route == 1
        tiles = int(sel.row_ptr[-1].item())
        if base_route is None:
            base_route = route
        out[name] = {"ms": round(ms, 3), "speedup_vs_dense": round(dense_ms / ms, 3) if dense_ms else None,
                     "density": round(tiles / dense_tiles, 4), "vs_heads": int(vs.sum()),
                     "vs_budget_blocks": round(float((nv[vs] + ns[vs]).mean()) / 2, 2) if vs.any() else None,
                     "route_agrees_with_cstruct": round(float((route == base_route).mean()), 4)}
        log(f"[bench] rule {name}: {out[name]}")
        del o, sel, ws
    return out


LENGTH_GATE = 8192   # dense_below_n at the crossover the length sweep measures on this GPU


def length_sweep(dsp, torch, synth, ns=(4096, 8192, 16384, 32768, 65536), steps=3):
    """CRISP vs dense ms per layer on Llama-shaped layers of growing length (4k-64k):
    where sparse prefill starts to pay (the length gate).  CRISP is timed as
    enqueued call by call, as one HIP graph replay of the same prefill, and with
    the length gate at LENGTH_GATE tokens (shorter layers take the dense path).
    Also the mean per-direction block budget of the Vertical-Slash heads under
    the noise floor and under a gamma = 0.95 coverage budget (same routing)."""
    res = {}
    for n in ns:
        cfg = synth.custom_config(f"llama-shape-{n // 1024}k", n, 32, 8, seed=7, conc_frac=0.6)
        spec = synth.make_spec(cfg)
        Q, K, V = synth.generate(spec, threads=16)
        to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        q, k, v = to_dev(Q), to_dev(K), to_dev(V)
        p = dsp.CrispParams(tau=cfg.tau, alpha=cfg.alpha, gamma=cfg.gamma)
        o = torch.empty_like(q)
        sel = dsp.new_selection(q, k, diagnostics=False)
        ws = torch.empty(dsp.workspace_bytes(dsp.make_shape(q, k, v, o), p), dtype=torch.uint8, device="cuda")
        reps = max(steps, 20) if n <= 16384 else steps          # short layers: enough calls to time
        ms = timed(lambda: dsp.crisp_prefill(q, k, v, p, sel=sel, o=o, ws=ws), reps, 2, torch)
        # the same prefill captured once in a HIP graph and replayed (no per-kernel launch cost)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            dsp.crisp_prefill(q, k, v, p, sel=sel, o=o, ws=ws)
        gms = timed(graph.replay, reps, 2, torch)
        aws = ws[dsp.select_workspace_bytes(dsp.make_shape(q, k, v, o), p):]
        dms = timed(lambda: dsp.crisp_dense_attn(q, k, v, o=o, ws=aws), reps, 2, torch)
        nb = n // 128
        density = int(sel.row_ptr[-1].item()) / (32 * nb * (nb + 1) // 2)
        # with the length gate at the measured crossover: below it the prefill takes the dense path
        pg = dsp.CrispParams(tau=cfg.tau, alpha=cfg.alpha, gamma=cfg.gamma, dense_below_n=LENGTH_GATE)
        gated = timed(lambda: dsp.crisp_prefill(q, k, v, pg, sel=sel, o=o, ws=ws), reps, 2, torch) if n < LENGTH_GATE else ms
        # per-direction budget of the Vertical-Slash heads under CRISP's noise
        # floor and under a gamma-coverage budget on the same routing: the flat
        # budget against one that grows with n
        budgets = {}
        for rule, over in (("crisp", {}), ("coverage-g0.95", dict(flags=dsp.FLAG_VS_COVERAGE))):
            pb = dsp.CrispParams(tau=cfg.tau, alpha=cfg.alpha, gamma=cfg.gamma)
            for a, b in over.items():
                setattr(pb, a, b)
            sb = dsp.crisp_select(q, k, pb)
            vs = sb.route.cpu().numpy() == 1
            nvs = (sb.nv.cpu().numpy() + sb.ns.cpu().numpy())[vs]
            budgets[rule] = round(float(nvs.mean()) / 2, 2) if vs.any() else None
            del sb
        res[n] = {"crisp_ms": round(ms, 3), "crisp_graph_ms": round(gms, 3), "dense_ms": round(dms, 3),
                  "speedup": round(dms / ms, 3), "speedup_graph": round(dms / gms, 3),
                  "crisp_gated_ms": round(gated, 3), "speedup_gated": round(dms / gated, 3),
                  "density": round(density, 4), "vs_budget_blocks": budgets}
        log(f"[bench] length {n}: {res[n]}")
        del graph, q, k, v, o, sel, ws, aws
        torch.cuda.empty_cache()
    return res


def varlen_batches(dsp, torch, synth, steps=3):
    """Packed batches of Llama-shaped sequences (512k tokens in total): one
    crisp_prefill_varlen call against the same sequences one call each."""
    res = {}
    for name, lens in (("8x64k", [65536] * 8), ("64x8k", [8192] * 64),
                       ("mixed-128k..16k", [131072] + [65536] * 2 + [32768] * 4 + [16384] * 8)):
        parts = []
        for i, n in enumerate(lens):
            cfg = synth.custom_config(f"batch-{i}", n, 32, 8, seed=100 + i, conc_frac=0.6)
            parts.append(synth.generate(synth.make_spec(cfg), threads=16))
        to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        q = to_dev(np.concatenate([p[0] for p in parts], axis=1))
        k = to_dev(np.concatenate([p[1] for p in parts], axis=1))
        v = to_dev(np.concatenate([p[2] for p in parts], axis=1))
        del parts
        cu = [0] + np.cumsum(lens).tolist()
        p = dsp.CrispParams()
        o = torch.empty_like(q)
        sel = dsp.new_varlen_selection(q, k, cu, diagnostics=False)
        ws = torch.empty(dsp.varlen_workspace_bytes(dsp.make_shape(q, k, v, o), cu, p), dtype=torch.uint8,
                         device="cuda")
        ms = timed(lambda: dsp.crisp_prefill_varlen(q, k, v, cu, p, sel=sel, o=o, ws=ws), steps, 1, torch)
        singles = []
        for a, b in zip(cu[:-1], cu[1:]):
            qi, ki, vi = q[:, a:b], k[:, a:b], v[:, a:b]
            si = dsp.new_selection(qi, ki, diagnostics=False)
            wi = torch.empty(dsp.workspace_bytes(dsp.make_shape(qi, ki, vi, o[:, a:b]), p), dtype=torch.uint8,
                             device="cuda")
            singles.append((qi, ki, vi, si, wi, o[:, a:b]))

        def one_by_one():
            for qi, ki, vi, si, wi, oi in singles:
                dsp.crisp_prefill(qi, ki, vi, p, sel=si, o=oi, ws=wi)

        ms1 = timed(one_by_one, steps, 1, torch)
        tok = cu[-1]
        res[name] = {"sequences": len(lens), "tokens": tok, "batch_ms": round(ms, 3), "one_call_each_ms": round(ms1, 3),
                     "batch_tokens_per_s": round(tok / (ms * 1e-3)), "speedup_over_calls": round(ms1 / ms, 3)}
        log(f"[bench] varlen {name}: {res[name]}")
        del q, k, v, o, sel, ws, singles
        torch.cuda.empty_cache()
    return res


def calibrate_copy(mib, torch):
    """One plain device copy of `mib` MiB (read mib, write mib): the reference that
    scales the HBM byte counters of the attention kernel."""
    a = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    log(f"[bench] calibration copy: {mib} MiB read + {mib} MiB written")


def measured_peaks(torch):
    """Attainable peaks on this GPU, reported beside the published ones: the bf16
    MFMA loop of libcrisp_probe.so (8 waves per CU, two per SIMD, as the attention
    kernel) over ~0.4 s launches so that clocks settle as they do under a long
    layer, and a plain 2 GiB device copy (bytes read + written per second)."""
    from dynamic_sparse_prefill_amd import api
    L = api.probe_lib()
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(ncu * 512, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    iters = 3_000_000
    flops = ncu * 8 * iters * 4 * 32768
    def loop(fn, name):
        rates = []
        for _ in range(2):                  # the first launch brings the clocks to their loaded state
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            st = fn(out.data_ptr(), ncu, iters, stream)
            e1.record()
            e1.synchronize()
            if st != 0:
                raise RuntimeError(f"{name} failed: {st}")
            rates.append(flops / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        return rates[-1]
    const_rate = loop(L.crisp_probe_mfma_bf16, "crisp_probe_mfma_bf16")
    data_rate = loop(L.crisp_probe_mfma_bf16_data, "crisp_probe_mfma_bf16_data")
    a = torch.empty(2 << 30, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    e1.synchronize()
    gbs = 5 * 2 * a.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    return {"mfma_bf16_tflops": round(const_rate, 1), "mfma_bf16_random_operands_tflops": round(data_rate, 1),
            "copy_gbs": round(gbs, 1),
            "how": "bf16 MFMA loop, 4 independent 32x32x16 accumulators per wave, 2 waves/SIMD, "
                   "second of two ~0.4 s launches, operands constant (mfma_bf16_tflops) or cycling over "
                   "8 pseudo-random fragment pairs (..._random_operands_tflops); "
                   "HBM: 2 GiB device copy, read + write bytes"}


def run_layer(layer, steps, warmup, torch, dsp, synth, with_dense=True, compare=False, compensate=True):
    spec = synth.make_spec(layer, compensate=compensate)
    cfg = spec.cfg
    t = time.time()
    Q, K, V = synth.generate(spec, threads=16)
    to_dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    del Q, K, V
    log(f"[bench] {cfg.name}: generated and uploaded in {time.time() - t:.1f}s")
    p = dsp.CrispParams(tau=cfg.tau, alpha=cfg.alpha, gamma=cfg.gamma)
    o = torch.empty_like(q)
    sel = dsp.new_selection(q, k, diagnostics=False)
    shape = dsp.make_shape(q, k, v, o)
    ws = torch.empty(dsp.workspace_bytes(shape, p), dtype=torch.uint8, device="cuda")
    sel_ws = ws[: dsp.select_workspace_bytes(shape, p)]
    attn_ws = ws[dsp.select_workspace_bytes(shape, p):]

    step = lambda: dsp.crisp_prefill(q, k, v, p, sel=sel, o=o, ws=ws)
    ms = timed(step, steps, warmup, torch)
    warm = step_events(step, max(1, steps), torch)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold = step_events(step, max(1, steps), torch, flush=flush)
    del flush
    route = sel.route.cpu().numpy()
    cstruct = sel.c_struct.cpu().numpy()
    tiles = int(sel.row_ptr[-1].item())
    nb = cfg.nb
    dense_tiles = cfg.hq * nb * (nb + 1) // 2
    # stage times on the launch stream
    sel_ms = event_ms(lambda: dsp.crisp_select(q, k, p, sel=sel, ws=sel_ws), max(1, steps), torch)
    attn_ms = event_ms(lambda: dsp.crisp_sparse_attn(q, k, v, sel, o=o, ws=attn_ws), max(1, steps), torch)
    out = dict(workload=cfg.name, n=cfg.n, hq=cfg.hq, hkv=cfg.hkv, ms=ms, select_ms=sel_ms, sparse_attn_ms=attn_ms,
               vs_heads=int((route == 1).sum()), pe_heads=int((route == 0).sum()), tiles=tiles,
               dense_tiles=dense_tiles, density=tiles / dense_tiles,
               step_ms={"warm_median": float(np.median(warm)), "warm_min": float(np.min(warm)),
                        "l2_flushed_median": float(np.median(cold)), "l2_flushed_min": float(np.min(cold))})
    out["selection_roofline"] = selection_roofline(cfg, route, tiles, sel_ms)
    out["selection_roofline"]["stage_bounds"] = selection_stage_bounds(cfg, route, tiles)
    out["heads"] = head_mix(spec, route, cstruct)
    # every list holds its diagonal block: hq * nb diagonal tiles, each 129/256 useful
    diag = cfg.hq * nb
    out["useful_flops"] = ((tiles - diag) + diag * DIAG_USEFUL) * TILE_FLOPS
    if with_dense:
        od = torch.empty_like(q)
        dws = attn_ws
        dense = lambda: dsp.crisp_dense_attn(q, k, v, o=od, ws=dws)
        out["dense_ms"] = timed(dense, max(1, steps // 2), 1, torch)
        out["dense_kernel_ms"] = event_ms(dense, 1, torch)
        out["speedup"] = out["dense_ms"] / ms
        out["dense_tflops"] = dense_tiles * TILE_FLOPS / (out["dense_kernel_ms"] * 1e-3) / 1e12
    out["sparse_tflops"] = tiles * TILE_FLOPS / (attn_ms * 1e-3) / 1e12
    out["useful_tflops"] = out["useful_flops"] / (attn_ms * 1e-3) / 1e12
    if compare:
        del sel, o, ws
        torch.cuda.empty_cache()
        out["rules"] = compare_rules(cfg, q, k, v, dsp, torch, 2, out.get("dense_ms"))
        del q, k, v
        torch.cuda.empty_cache()
        return out, spec, route
    del q, k, v, o, ws
    torch.cuda.empty_cache()
    return out, spec, route


def cpu_baseline(spec, route, tiles_total, budget_s=20.0):
    """The oracle as it stands, on a bounded sample of the layer, scaled to ms per layer."""
    from oracle import crisp_oracle as O
    from workloads import synth
    cfg = spec.cfg
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    G = cfg.hq // cfg.hkv
    t_start = time.time()
    res = {}
    for kind in (1, 0):
        hs = np.flatnonzero(route == kind)
        if hs.size == 0:
            continue
        h = int(hs[0])
        q = synth.as_f64(spec, synth.rows(spec, "q", h, 0, cfg.n))
        k = synth.as_f64(spec, synth.rows(spec, "k", h // G, 0, cfg.n))
        t = time.time()
        r = O.select_head(q, k, 128, 128, 128, cfg.tau, cfg.alpha, cfg.gamma)
        res[kind] = (time.time() - t, h, r)
    sel_s = sum(res[kd][0] * int((route == kd).sum()) for kd in res)
    # attention: time rows of the PE head (the long lists) until the budget is used
    kind = 0 if 0 in res else 1
    _, h, r = res[kind]
    q = synth.as_f64(spec, synth.rows(spec, "q", h, 0, cfg.n))
    k = synth.as_f64(spec, synth.rows(spec, "k", h // G, 0, cfg.n))
    v = synth.as_f64(spec, synth.rows(spec, "v", h // G, 0, cfg.n))
    done_tiles, t_att = 0, 0.0
    blocks = []
    # seeded query blocks (the last one first) until about budget_s of host time is spent
    for qb in [cfg.nb - 1] + [b for b in synth.sample_blocks(cfg.nb, 64, 17) if b != cfg.nb - 1]:
        if time.time() - t_start > budget_s:
            break
        t = time.time()
        O.attention_block_rows(q, k, v, qb, r["lists"][qb], 128)
        t_att += time.time() - t
        done_tiles += len(r["lists"][qb])
        blocks.append(qb)
    att_s = t_att / max(done_tiles, 1) * tiles_total
    ms = (sel_s + att_s) * 1e3
    return dict(value=ms, unit="ms/layer", cores=threads, kind="oracle",
                sample=(f"oracle selection of one VS head and one PE head (scaled by the layer's head counts) and "
                        f"attention of {len(blocks)} query blocks ({done_tiles} tiles) of head {h}, scaled by the "
                        f"layer's {tiles_total} executed tiles; {time.time() - t_start:.1f}s of host time"),
                select_ms=sel_s * 1e3, attention_ms=att_s * 1e3)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the attainable-peak probes (MFMA loop, copy)")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--workload", default="llama3.1-8b-512k",
                    choices=["llama3.1-8b-32k", "llama3.1-8b-128k", "qwen2.5-7b-128k", "llama3.1-8b-512k"],
                    help="the layer timed")
    ap.add_argument("--no-dense", action="store_true", help="skip the dense baseline (counter-collection runs)")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip the decision-rule comparison (median floor, universal config, FlexPrefill)")
    ap.add_argument("--no-sweep", action="store_true", help="skip the 4k-64k length sweep (length gate)")
    ap.add_argument("--no-varlen", action="store_true", help="skip the packed-batch (varlen) measurement")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run one plain copy of MIB MiB (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "the path runs on one GPU; sharding by KV group over several GPUs is not implemented",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import dynamic_sparse_prefill_amd as dsp
    from workloads import synth
    dsp.lib()
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, torch)
    main_res, spec, route = run_layer(synth.WORKLOADS[args.workload], args.steps, args.warmup, torch, dsp, synth,
                                      with_dense=not args.no_dense, compare=not args.no_compare)
    log("[bench]", json.dumps(main_res))
    extra = {}
    if not args.no_sweep:
        extra["length_sweep"] = length_sweep(dsp, torch, synth)
    if not args.no_varlen:
        extra["varlen"] = varlen_batches(dsp, torch, synth)
    if not args.no_extra:
        for name in ("llama3.1-8b-128k", "qwen2.5-7b-128k"):
            if name == args.workload:
                continue
            r, _, _ = run_layer(synth.WORKLOADS[name], max(2, args.steps), 1, torch, dsp, synth)
            extra[r["workload"]] = {k: r[k] for k in ("ms", "dense_ms", "speedup", "select_ms", "sparse_attn_ms",
                                                      "density", "heads", "sparse_tflops", "useful_tflops",
                                                      "dense_tflops", "selection_roofline")}
            log("[bench]", json.dumps(r))
        # the 32k Llama layer with the literal generator constants (no length
        # compensation): the anchor share of concentrated heads falls with n,
        # so more of them route to Pooled Estimation
        r, _, _ = run_layer(synth.LLAMA_32K, max(3, args.steps), 1, torch, dsp, synth, compensate=False)
        extra["llama3.1-8b-32k-literal-constants"] = {k: r[k] for k in ("ms", "dense_ms", "speedup", "select_ms",
                                                                        "sparse_attn_ms", "density", "heads")}
        log("[bench]", json.dumps(r))
    peaks = None if args.no_peaks else measured_peaks(torch)
    if peaks:
        log("[bench] measured peaks", json.dumps(peaks))
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(spec, route, main_res["tiles"])
        log("[bench] cpu", json.dumps(cpu))

    ach = main_res["sparse_tflops"]
    line = {
        "metric": "sparse prefill attn ms/layer + speedup vs dense @128k/512k; MFMA % of peak",
        "value": round(main_res["ms"], 3),
        "unit": "ms/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["ms"], 3),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": main_res["workload"], "n": main_res["n"], "hq": main_res["hq"], "hkv": main_res["hkv"],
                   "d": 128, "block": 128, "tau": 0.3, "alpha": 1.0, "gamma": 0.95,
                   "generator": "seeded sink/recency/needle heads, length-compensated"},
        "speedup_vs_dense": round(main_res["speedup"], 3) if "speedup" in main_res else None,
        "dense_ms": round(main_res["dense_ms"], 3) if "dense_ms" in main_res else None,
        "stages": {"select_ms": round(main_res["select_ms"], 3), "sparse_attn_ms": round(main_res["sparse_attn_ms"], 3)},
        "step_ms": {k: round(v, 3) for k, v in main_res["step_ms"].items()},
        "selection_roofline": dict(main_res["selection_roofline"], **(
            {"frac_of_measured_hbm": round(main_res["selection_roofline"]["achieved_gbs"] / peaks["copy_gbs"], 4)}
            if peaks else {})),
        "rules": main_res.get("rules"),
        "density": round(main_res["density"], 4),
        "heads": main_res["heads"],
        "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                     "useful_achieved": round(main_res["useful_tflops"], 2),
                     "useful_frac": round(main_res["useful_tflops"] / PEAK_BF16_TFLOPS, 4),
                     "useful_flops_per_launch": int(main_res["useful_flops"]),
                     "frac_of_measured": round(ach / peaks["mfma_bf16_tflops"], 4) if peaks else None,
                     "frac_of_measured_random_operands":
                         round(ach / peaks["mfma_bf16_random_operands_tflops"], 4) if peaks else None,
                     "traffic": profiled_traffic() if args.workload == "llama3.1-8b-512k" else None,
                     "kernel": "fa_bf16_kernel<false> (sparse attention; event time includes the V re-layout)",
                     "flops_per_launch": main_res["tiles"] * TILE_FLOPS},
        "dense_roofline": ({"achieved": round(main_res["dense_tflops"], 2),
                            "frac": round(main_res["dense_tflops"] / PEAK_BF16_TFLOPS, 4)}
                           if "dense_tflops" in main_res else None),
        "measured_peaks": peaks,
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
