"""Helpers shared by the GPU parity tests and the bench's parity-free paths.

Decision parity (bit-exact): the oracle's decision functions are fed the
GPU's own float32 scores (p^v, p^s, C_struct, pooled P) and must reproduce the
GPU's route, S_v, S_s and every per-block list exactly; entries within 1e-6
relative of a threshold are counted as ties and reported, not failed.

Score fidelity (tolerance): the oracle's float64 scores computed from the
same (bf16-exact) inputs are compared with the GPU's float32 scores.

Attention parity (tolerance): with the GPU's lists, sampled (or all) query
blocks of the GPU output are compared with the oracle's float64 attention:
max-abs <= 2e-2 and mean-abs <= 2e-3 for bf16.
"""
from __future__ import annotations

import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch
from threadpoolctl import threadpool_limits

from oracle import crisp_oracle as O
from workloads import synth

import dynamic_sparse_prefill_amd as dsp

MAX_ABS, MEAN_ABS = 2e-2, 2e-3

# Decision-parity summaries of this session, printed at the end of the pytest
# run (tests/conftest.py) so that tie and exemption counts are visible in the
# run's output even under -q.
REPORTS: list = []


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def to_device(spec, arr):
    if spec.cfg.dtype == "bf16":
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(arr).cuda()


def load_layer(spec, threads=16):
    t = time.time()
    Q, K, V = synth.generate(spec, threads=threads)
    log(f"[gen] {spec.cfg.name}: {time.time() - t:.1f}s")
    return Q, K, V


def params_of(cfg, **over) -> dsp.CrispParams:
    p = dsp.CrispParams(tau=cfg.tau, alpha=cfg.alpha, gamma=cfg.gamma)
    for k, v in over.items():
        setattr(p, k, v)
    return p


def gpu_lists(sel, hq, nb):
    rp = sel.row_ptr.cpu().numpy().astype(np.int64)
    col = sel.col_idx[: int(rp[-1])].cpu().numpy()
    return rp, col


def head_lists(rp, col, h, nb):
    return [col[rp[h * nb + qb]: rp[h * nb + qb + 1]] for qb in range(nb)]


def tri_slice(nb, h):
    t = nb * (nb + 1) // 2
    return slice(h * t, (h + 1) * t)


def tri_to_dense(vals, nb):
    P = np.zeros((nb, nb), np.float32)
    qi, ki = np.tril_indices(nb)
    P[qi, ki] = vals
    return P


def variant_of(p: dsp.CrispParams):
    """(router, budget) names of the oracle for the flags of p."""
    router = "jsd" if p.flags & dsp.FLAG_ROUTE_JSD else "cstruct"
    budget = "median" if p.flags & dsp.FLAG_VS_MEDIAN else ("coverage" if p.flags & dsp.FLAG_VS_COVERAGE else "mean")
    return router, budget


def check_decisions(sel, hq, nb, p: dsp.CrispParams, heads=None, name=None):
    """Bit-exact decision parity from the GPU's own float32 scores.  Returns a
    report dict; with a name, the report is also kept for the session summary."""
    router, budget = variant_of(p)
    abar = sel.abar.cpu().numpy().reshape(hq, nb) if router == "jsd" else None
    jsd_gpu = sel.jsd.cpu().numpy() if router == "jsd" else None
    route = sel.route.cpu().numpy()
    cs = sel.c_struct.cpu().numpy()
    pv = sel.pv.cpu().numpy().reshape(hq, nb) if sel.pv is not None else None
    ps = sel.ps.cpu().numpy().reshape(hq, nb) if sel.ps is not None else None
    nv = sel.nv.cpu().numpy(); ns = sel.ns.cpu().numpy()
    sv = sel.sv.cpu().numpy().reshape(hq, nb); ss = sel.ss.cpu().numpy().reshape(hq, nb)
    rp, col = gpu_lists(sel, hq, nb)
    rep = dict(route_ties=0, vs_ties=0, pe_ties=0, pe_exempt=0, heads_checked=0, vs_heads=0, pe_heads=0,
               dense_heads=0, vs_exempt=0, jsd_err=0.0)
    for h in (range(hq) if heads is None else heads):
        Pd = None
        if route[h] == 0:
            Pd = tri_to_dense(sel.pe_prob[tri_slice(nb, h)].cpu().numpy(), nb)
        if router == "jsd" and route[h] != -1:
            # the divergence is a float64 sum of logarithms: the oracle's value from the
            # GPU's own float32 a_bar and p^v agrees to rounding, and a route that sits
            # within 1e-6 relative of tau is a tie (counted, and the head skipped)
            j = O.jsd(abar[h], pv[h])
            rep["jsd_err"] = max(rep["jsd_err"], abs(j - float(jsd_gpu[h])))
            assert abs(j - float(jsd_gpu[h])) <= 1e-9, f"head {h}: jsd gpu {jsd_gpu[h]} oracle {j}"
            if abs(j - float(np.float32(p.tau))) <= O.TIE_REL * max(float(np.float32(p.tau)), 1e-30):
                rep["route_ties"] += 1
                continue
        r, osv, oss, lists, info = O.decide_from_scores(int(route[h]), cs[h], pv[h] if pv is not None else None,
                                                       ps[h] if ps is not None else None, Pd, nb, p.tau, p.alpha,
                                                       p.gamma, p.min_blocks, router=router, budget=budget,
                                                       abar=abar[h] if abar is not None else None)
        # route and VS thresholds are the same float32 operations on the same float32
        # scores on both sides: they must agree even inside the tie band (ties are
        # only counted).  The PE cut compares sums of the same float32 values taken
        # with different arithmetic: the GPU truncates each entry to a multiple of
        # 2^-46 (error < entries * 2^-46 in both the total and the prefix), the
        # oracle accumulates in extended precision.  A head is exempt only when
        # gamma*T lies within entries * 2^-45 of the prefix at the cut.
        if router == "cstruct":
            rep["route_ties"] += int(route[h] != -1 and O.route_tie(cs[h], p.tau))
        assert r == route[h], f"head {h}: route gpu {route[h]} oracle {r} (C={cs[h]!r})"
        gl = head_lists(rp, col, h, nb)
        if r == 1:
            rep["vs_heads"] += 1
            if budget == "mean":
                rep["vs_ties"] += len(O.vs_ties(pv[h], p.alpha)) + len(O.vs_ties(ps[h], p.alpha))
            elif budget == "median":
                rep["vs_ties"] += len(O.median_ties(pv[h], p.alpha)) + len(O.median_ties(ps[h], p.alpha))
            else:
                # same exemption as the PE cut: the GPU sums 2^-46 fixed-point masses
                rep["vs_ties"] += sum(int(O.pe_tie(i)) for i in info)
                if any(O.pe_tie(i, 0.0, i["entries"] * 2.0 ** -45) for i in info):
                    rep["vs_exempt"] += 1
                    continue
            assert np.array_equal(sv[h, :nv[h]], osv), f"head {h}: S_v differs"
            assert np.array_equal(ss[h, :ns[h]], oss), f"head {h}: S_s differs"
        elif r == 0:
            rep["pe_heads"] += 1
            rep["pe_ties"] += int(O.pe_tie(info))
            if O.pe_tie(info, 0.0, info["entries"] * 2.0 ** -45):
                rep["pe_exempt"] += 1
                continue
        else:
            rep["dense_heads"] += 1
        for qb in range(nb):
            assert np.array_equal(gl[qb], lists[qb]), f"head {h} block {qb}: gpu {gl[qb][:20]} oracle {lists[qb][:20]}"
        rep["heads_checked"] += 1
    if name is not None:
        REPORTS.append((name, dict(rep, tau=float(p.tau), alpha=float(p.alpha), gamma=float(p.gamma),
                                   min_blocks=int(p.min_blocks), flags=int(p.flags))))
    return rep


def oracle_scores(spec, Q, K, h, blk=128, sink=128, local=128):
    """Oracle float64 proxy scores for query head h from the storage-form arrays."""
    cfg = spec.cfg
    n = cfg.n
    g = h // (cfg.hq // cfg.hkv)
    q = synth.as_f64(spec, Q[h, n - blk:])
    k = synth.as_f64(spec, K[g])
    A = O.proxy_attention(q, k)
    return O.vertical_scores(A, blk), O.slash_scores(A, blk), O.c_struct(A, sink, local)


def check_score_fidelity(spec, Q, K, sel, heads, tol=1e-4, sink=128, local=128):
    """GPU float32 p^v, p^s and C_struct against the oracle's float64 values
    computed from the same inputs (anchor windows sink / local)."""
    cfg = spec.cfg
    nb = cfg.nb
    pv = sel.pv.cpu().numpy().reshape(cfg.hq, nb)
    ps = sel.ps.cpu().numpy().reshape(cfg.hq, nb)
    cs = sel.c_struct.cpu().numpy()
    heads = list(heads)

    def one(h):
        with threadpool_limits(2):
            return oracle_scores(spec, Q, K, h, sink=sink, local=local)

    with ThreadPoolExecutor(min(8, max(len(heads), 1))) as ex:
        ref = list(ex.map(one, heads))
    worst = 0.0
    for h, (opv, ops, ocs) in zip(heads, ref):
        e = max(np.abs(pv[h] - opv).max(), np.abs(ps[h] - ops).max(), abs(cs[h] - ocs))
        worst = max(worst, float(e))
        assert e <= tol, f"head {h}: score error {e} (C_struct gpu {cs[h]!r} oracle {ocs!r})"
    return worst


def check_jsd_fidelity(spec, Q, K, sel, heads, tol=1e-5):
    """Oracle float64 pooled estimate and JSD from Q, K against the GPU's."""
    cfg = spec.cfg
    nb, n = cfg.nb, cfg.n
    abar = sel.abar.cpu().numpy().reshape(cfg.hq, nb)
    jg = sel.jsd.cpu().numpy()
    worst = 0.0
    for h in heads:
        g = h // (cfg.hq // cfg.hkv)
        q = synth.as_f64(spec, Q[h, n - 128:])
        k = synth.as_f64(spec, K[g])
        a = O.pooled_estimate(q, k, 128)
        pv = O.vertical_scores(O.proxy_attention(q, k), 128)
        e = max(float(np.abs(a - abar[h]).max()), abs(O.jsd(a, pv) - float(jg[h])))
        worst = max(worst, e)
        assert e <= tol, f"head {h}: a_bar / JSD error {e}"
    return worst


def check_pe_fidelity(spec, Q, K, sel, heads, tol=1e-5):
    cfg = spec.cfg
    nb = cfg.nb
    worst = 0.0
    for h in heads:
        g = h // (cfg.hq // cfg.hkv)
        P = O.pe_probabilities(synth.as_f64(spec, Q[h]), synth.as_f64(spec, K[g]), 128)
        Pg = tri_to_dense(sel.pe_prob[tri_slice(nb, h)].cpu().numpy(), nb).astype(np.float64)
        e = float(np.abs(P - Pg).max())
        worst = max(worst, e)
        assert e <= tol, f"head {h}: pooled-probability error {e}"
    return worst


def check_attention_blocks(spec, Q, K, V, o_gpu, lists_of, heads, blocks, max_abs=MAX_ABS, mean_abs=MEAN_ABS,
                           threads=8):
    """Compare GPU output rows of the given (head, query block) pairs with the
    oracle.  The blocks of one head are computed by the oracle in parallel
    threads (rows are independent given the lists)."""
    cfg = spec.cfg
    G = cfg.hq // cfg.hkv
    blocks = list(blocks)
    kv_cache = {}
    worst_max, sum_abs, cnt = 0.0, 0.0, 0
    for h in heads:
        g = h // G
        if g not in kv_cache:
            kv_cache.clear()
            kv_cache[g] = (synth.as_f64(spec, K[g]), synth.as_f64(spec, V[g]))
        k, v = kv_cache[g]
        q = synth.as_f64(spec, Q[h])
        got_all = o_gpu[h].float().cpu().numpy()

        def one(qb):
            with threadpool_limits(2):
                ref = O.attention_block_rows(q, k, v, qb, lists_of(h, qb), 128)
            err = np.abs(got_all[qb * 128:(qb + 1) * 128].astype(np.float64) - ref)
            return float(err.max()), float(err.sum()), err.size

        if len(blocks) > 1 and threads > 1:
            with ThreadPoolExecutor(min(threads, len(blocks))) as ex:
                res = list(ex.map(one, blocks))
        else:
            res = [one(qb) for qb in blocks]
        for mx, sm, c in res:
            worst_max = max(worst_max, mx)
            sum_abs += sm
            cnt += c
    mean = sum_abs / max(cnt, 1)
    assert worst_max <= max_abs, f"max-abs {worst_max}"
    assert mean <= mean_abs, f"mean-abs {mean}"
    return worst_max, mean
