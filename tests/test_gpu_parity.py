"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Sizes: the tiny fp32 layer and small bf16 layers are compared in full; the
Llama / Qwen layers (32k, 128k, 512k) are compared on every routing and
selection decision and on a seeded sample of query blocks, in the same launch
configuration the bench times.
"""
import os

import numpy as np
import pytest
import torch

from oracle import crisp_oracle as O
from workloads import synth

import dynamic_sparse_prefill_amd as dsp
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dsp.lib()
    yield
    torch.cuda.synchronize()


def _run_layer(spec, Q, K, V, params):
    q, k, v = P.to_device(spec, Q), P.to_device(spec, K), P.to_device(spec, V)
    o, sel = dsp.crisp_prefill(q, k, v, params, pe_prob=True)
    torch.cuda.synchronize()
    return q, k, v, o, sel


def _lists_fn(sel, nb):
    rp, col = P.gpu_lists(sel, None, nb)
    return lambda h, qb: col[rp[h * nb + qb]: rp[h * nb + qb + 1]]


# ------------------------------------------------------------------ tiny fp32 layer, everything in full

def test_tiny_fp32_layer_full():
    spec = synth.make_spec(synth.TINY_FP32_4K)
    cfg = spec.cfg
    Q, K, V = synth.generate(spec)
    p = P.params_of(cfg)
    q, k, v, o, sel = _run_layer(spec, Q, K, V, p)
    route = sel.route.cpu().numpy()
    assert route.tolist() == [1, 0], route            # concentrated head -> VS, diffuse -> PE
    rep = P.check_decisions(sel, cfg.hq, cfg.nb, p)
    P.log("[tiny] decisions", rep)
    assert rep["heads_checked"] == 2
    P.log("[tiny] score err", P.check_score_fidelity(spec, Q, K, sel, [0, 1], tol=1e-5))
    P.log("[tiny] PE prob err", P.check_pe_fidelity(spec, Q, K, sel, [1], tol=1e-6))
    # full outputs, fp32 path: tighter than the bf16 tolerance
    lists = _lists_fn(sel, cfg.nb)
    mx, mean = P.check_attention_blocks(spec, Q, K, V, o, lists, [0, 1], range(cfg.nb), max_abs=1e-4, mean_abs=1e-5)
    P.log(f"[tiny] attention max {mx:.2e} mean {mean:.2e}")
    # independent decisions (oracle's own float64 scores) agree as well
    for h in range(2):
        r = O.select_head(Q[h].astype(np.float64), K[h].astype(np.float64), 128, 128, 128, cfg.tau, cfg.alpha,
                          cfg.gamma)
        assert r["route"] == route[h]
        gl = [lists(h, qb) for qb in range(cfg.nb)]
        assert all(np.array_equal(a, b) for a, b in zip(gl, r["lists"]))
    # dense attention of the same engine against the oracle's dense attention
    od = dsp.crisp_dense_attn(q, k, v)
    torch.cuda.synchronize()
    for h in range(2):
        ref = O.dense_causal_attention(Q[h].astype(np.float64), K[h].astype(np.float64), V[h].astype(np.float64))
        assert np.abs(od[h].cpu().numpy() - ref).max() < 1e-4


# ------------------------------------------------------------------ attention alone, on lists the oracle makes

@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_sparse_attention_on_oracle_lists(dtype):
    cfg = synth.custom_config("lists", 1280, 4, 2, dtype=dtype, seed=11)
    spec = synth.make_spec(cfg)
    Q, K, V = synth.generate(spec)
    nb = cfg.nb
    rng = np.random.default_rng(5)
    per_head = []
    for h in range(cfg.hq):
        lists = []
        for qb in range(nb):
            s = sorted({kb for kb in range(qb + 1) if rng.random() < 0.5} | ({qb} if (qb + h) % 4 else set()))
            lists.append(np.array(s, np.int64))
        per_head.append(lists)
    per_head[1][3] = np.zeros(0, np.int64)             # an empty row: zero output
    per_head[2][7] = np.array([7])                     # diagonal only
    rp, col = O.lists_to_csr(per_head)
    q, k, v = P.to_device(spec, Q), P.to_device(spec, K), P.to_device(spec, V)
    sel = dsp.Selection(torch.zeros(cfg.hq, dtype=torch.int32, device="cuda"),
                        torch.zeros(cfg.hq, device="cuda"),
                        torch.from_numpy(rp.astype(np.int32)).cuda(), torch.from_numpy(col.astype(np.int32)).cuda())
    o = dsp.crisp_sparse_attn(q, k, v, sel)
    torch.cuda.synchronize()
    tol = (2e-2, 2e-3) if dtype == "bf16" else (1e-4, 1e-5)
    mx, mean = P.check_attention_blocks(spec, Q, K, V, o, lambda h, qb: per_head[h][qb], range(cfg.hq), range(nb),
                                        *tol)
    assert torch.all(o[1, 3 * 128:4 * 128] == 0)
    P.log(f"[lists {dtype}] max {mx:.2e} mean {mean:.2e}")


@pytest.mark.parametrize("hq,hkv,n", [(7, 1, 2048), (4, 4, 1152)])
def test_dense_attention_bf16_full(hq, hkv, n):
    cfg = synth.custom_config("dense", n, hq, hkv, seed=3)
    spec = synth.make_spec(cfg)
    Q, K, V = synth.generate(spec)
    q, k, v = P.to_device(spec, Q), P.to_device(spec, K), P.to_device(spec, V)
    o = dsp.crisp_dense_attn(q, k, v)
    torch.cuda.synchronize()
    mx, mean = P.check_attention_blocks(spec, Q, K, V, o, lambda h, qb: range(qb + 1), range(hq), range(cfg.nb))
    P.log(f"[dense {hq}/{hkv} n={n}] max {mx:.2e} mean {mean:.2e}")


def test_strided_layout_matches_contiguous():
    """[n, heads, d] storage (token-major) through the stride arguments gives the same result."""
    cfg = synth.custom_config("strided", 2048, 4, 2, seed=9)
    spec = synth.make_spec(cfg)
    Q, K, V = synth.generate(spec)
    q, k, v = P.to_device(spec, Q), P.to_device(spec, K), P.to_device(spec, V)
    p = P.params_of(cfg)
    o1, s1 = dsp.crisp_prefill(q, k, v, p)
    qt = q.permute(1, 0, 2).contiguous().permute(1, 0, 2)
    kt = k.permute(1, 0, 2).contiguous().permute(1, 0, 2)
    vt = v.permute(1, 0, 2).contiguous().permute(1, 0, 2)
    ot = torch.empty(q.shape[1], q.shape[0], 128, dtype=q.dtype, device="cuda").permute(1, 0, 2)
    o2, s2 = dsp.crisp_prefill(qt, kt, vt, p, o=ot)
    torch.cuda.synchronize()
    assert torch.equal(s1.route, s2.route) and torch.equal(s1.row_ptr, s2.row_ptr)
    assert torch.equal(o1, o2)


# ------------------------------------------------------------------ small mixed layers: selection in full

@pytest.mark.parametrize("n,hq,hkv,seed", [(8192, 8, 2, 21), (1664, 7, 1, 22), (384, 2, 1, 23), (2048, 4, 4, 24)])
def test_small_layer_selection_and_output(n, hq, hkv, seed):
    cfg = synth.custom_config("small", n, hq, hkv, seed=seed, conc_frac=0.5)
    spec = synth.make_spec(cfg)
    Q, K, V = synth.generate(spec)
    p = P.params_of(cfg)
    q, k, v, o, sel = _run_layer(spec, Q, K, V, p)
    rep = P.check_decisions(sel, hq, cfg.nb, p)
    P.log(f"[small n={n}] decisions", rep, "routes", sel.route.cpu().tolist())
    assert rep["heads_checked"] + rep["pe_exempt"] == hq
    P.log("[small] score err", P.check_score_fidelity(spec, Q, K, sel, range(hq)))
    pe = [h for h in range(hq) if sel.route[h].item() == 0]
    if pe:
        P.log("[small] PE prob err", P.check_pe_fidelity(spec, Q, K, sel, pe))
    mx, mean = P.check_attention_blocks(spec, Q, K, V, o, _lists_fn(sel, cfg.nb), range(hq), range(cfg.nb))
    P.log(f"[small] attention max {mx:.2e} mean {mean:.2e}")


def test_dense_fallback_paths():
    cfg = synth.custom_config("fallback", 256, 2, 1, seed=4)
    spec = synth.make_spec(cfg)
    Q, K, V = synth.generate(spec)
    q, k, v, o, sel = _run_layer(spec, Q, K, V, P.params_of(cfg))
    assert sel.route.cpu().tolist() == [-1, -1]
    assert sel.row_ptr.cpu().tolist() == [0, 1, 3, 4, 6]
    P.check_attention_blocks(spec, Q, K, V, o, lambda h, qb: range(qb + 1), range(2), range(2))
    cfg2 = synth.custom_config("gate", 2048, 2, 1, seed=4)
    spec2 = synth.make_spec(cfg2)
    Q2, K2, V2 = synth.generate(spec2)
    _, _, _, o2, sel2 = _run_layer(spec2, Q2, K2, V2, P.params_of(cfg2, dense_below_n=4096))
    assert sel2.route.cpu().tolist() == [-1, -1]
    rp = sel2.row_ptr.cpu().numpy()
    assert np.array_equal(np.diff(rp), np.tile(np.arange(1, 17), 2))
    # one block (n = b): no noise floor exists (N_b - 2 < 1), every head takes the dense path
    cfg3 = synth.custom_config("one-block", 128, 4, 2, seed=5)
    spec3 = synth.make_spec(cfg3)
    Q3, K3, V3 = synth.generate(spec3)
    _, _, _, o3, sel3 = _run_layer(spec3, Q3, K3, V3, P.params_of(cfg3))
    assert sel3.route.cpu().tolist() == [-1] * 4
    assert sel3.row_ptr.cpu().tolist() == [0, 1, 2, 3, 4]
    assert sel3.col_idx[:4].cpu().tolist() == [0, 0, 0, 0]
    P.check_attention_blocks(spec3, Q3, K3, V3, o3, lambda h, qb: [0], range(4), [0])


def test_length_gate_whole_batch_dense():
    """Every sequence of a packed batch below the length gate: the selection is
    written by one launch (route -1, full lists) and equals single calls; the
    output equals dense attention on each sequence and the oracle's on sampled
    blocks."""
    lens = [2048, 512, 4096]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    hq, hkv = 4, 2
    parts = []
    for i, n in enumerate(lens):
        cfg = synth.custom_config(f"gated{i}", n, hq, hkv, seed=120 + i, conc_frac=0.5)
        spec = synth.make_spec(cfg)
        parts.append((spec,) + synth.generate(spec))
    spec0 = parts[0][0]
    q = P.to_device(spec0, np.concatenate([p[1] for p in parts], axis=1))
    k = P.to_device(spec0, np.concatenate([p[2] for p in parts], axis=1))
    v = P.to_device(spec0, np.concatenate([p[3] for p in parts], axis=1))
    params = P.params_of(spec0.cfg, dense_below_n=8192, flags=dsp.FLAG_ROUTE_JSD)
    o, sel = dsp.crisp_prefill_varlen(q, k, v, cu, params)
    torch.cuda.synchronize()
    assert sel.route.cpu().tolist() == [-1] * (hq * len(lens))
    assert torch.all(sel.c_struct == 0) and torch.all(sel.nv == 0) and torch.all(sel.jsd == 0)
    rp0, col0 = 0, 0
    for i, n in enumerate(lens):
        a, b = cu[i], cu[i + 1]
        nb = n // 128
        qi, ki, vi = q[:, a:b].contiguous(), k[:, a:b].contiguous(), v[:, a:b].contiguous()
        oi, si = dsp.crisp_prefill(qi, ki, vi, params)
        od = dsp.crisp_dense_attn(qi, ki, vi)
        torch.cuda.synchronize()
        assert torch.equal(o[:, a:b], oi) and torch.equal(oi, od), f"sequence {i}"
        assert torch.equal(sel.row_ptr[rp0:rp0 + hq * nb + 1], si.row_ptr)
        assert np.array_equal(np.diff(si.row_ptr.cpu().numpy()), np.tile(np.arange(1, nb + 1), hq))
        m = int(si.row_ptr[-1])
        assert torch.equal(sel.col_idx[col0:col0 + m], si.col_idx[:m])
        assert si.col_idx[:m].cpu().tolist() == [kb for _ in range(hq) for qb in range(nb) for kb in range(qb + 1)]
        rp0 += hq * nb + 1
        col0 += hq * nb * (nb + 1) // 2
    sp, Q0, K0, V0 = parts[2]
    P.check_attention_blocks(sp, Q0, K0, V0, o[:, cu[2]:cu[3]], lambda h, qb: range(qb + 1), range(hq),
                             synth.sample_blocks(sp.cfg.nb, 6, 9))


@pytest.mark.parametrize("n", [4096, 8192])
def test_length_sweep_layers(n):
    """The Llama-shaped 4k and 8k layers the bench's length sweep times (same
    generator and seed): every decision of every head bit-exact, every head's
    proxy scores against the oracle, every output row of every head; then the
    same layer with the length gate at 8192 tokens (4k: the dense path)."""
    cfg = synth.custom_config(f"llama-shape-{n // 1024}k", n, 32, 8, seed=7, conc_frac=0.6)
    spec = synth.make_spec(cfg)
    Q, K, V = synth.generate(spec)
    p = P.params_of(cfg)
    q, k, v, o, sel = _run_layer(spec, Q, K, V, p)
    rep = P.check_decisions(sel, cfg.hq, cfg.nb, p, name=cfg.name)
    assert rep["heads_checked"] + rep["pe_exempt"] == cfg.hq, rep
    P.log(f"[{cfg.name}] score err", P.check_score_fidelity(spec, Q, K, sel, range(cfg.hq)))
    mx, mean = P.check_attention_blocks(spec, Q, K, V, o, _lists_fn(sel, cfg.nb), range(cfg.hq), range(cfg.nb))
    P.log(f"[{cfg.name}] attention (every row) max {mx:.2e} mean {mean:.2e}")
    pg = P.params_of(cfg, dense_below_n=8192)
    og, selg = dsp.crisp_prefill(q, k, v, pg)
    torch.cuda.synchronize()
    if n < 8192:
        assert selg.route.cpu().tolist() == [-1] * cfg.hq
        assert torch.equal(og, dsp.crisp_dense_attn(q, k, v))
    else:
        assert torch.equal(selg.route, sel.route) and torch.equal(og, o)


def test_parameter_sweep_and_min_blocks():
    cfg = synth.custom_config("sweep", 8192, 8, 2, seed=31, conc_frac=0.5)
    spec = synth.make_spec(cfg)
    Q, K, V = synth.generate(spec)
    q, k = P.to_device(spec, Q), P.to_device(spec, K)
    for tau in (0.2, 0.3, 0.5):
        for alpha in (0.5, 1.0, 2.0):
            for mb in (0, 8):
                p = P.params_of(cfg, tau=tau, alpha=alpha, min_blocks=mb)
                sel = dsp.crisp_select(q, k, p, pe_prob=True)
                torch.cuda.synchronize()
                rep = P.check_decisions(sel, cfg.hq, cfg.nb, p)
                if mb:
                    nv = sel.nv.cpu().numpy()[sel.route.cpu().numpy() == 1]
                    assert np.all(nv >= mb)


@pytest.mark.parametrize("case", ["llama", "zero_q"])
def test_pe_cut_candidates_equal_full_read(case):
    """Three ways to the same gamma cut of the 64-block layer.  By default a
    head of at most 64 blocks takes the whole cut in one work-group (LDS
    histograms).  CRISP_PE_SMALL=0 sends it through the general passes, whose
    last radix pass counts each row's entries above and at the cut value from
    the few entries that share the cut's top 22 bits; with CRISP_PE_CAND_CAP=0
    as well every head reads its rows in full instead.  The selection, the
    pooled probabilities and the cut must be bitwise the same all three ways.
    With Q = 0 every pooled row is uniform (p = 1/(qb+1)), so the cut falls
    inside a run of equal values and only part of it is taken (the flat-order
    tie rule)."""
    cfg = synth.custom_config("candcap", 8192, 8, 2, seed=51, conc_frac=0.5)
    spec = synth.make_spec(cfg)
    Q, K, V = synth.generate(spec)
    if case == "zero_q":
        Q[:] = 0
    q, k = P.to_device(spec, Q), P.to_device(spec, K)
    p = P.params_of(cfg, tau=2.0) if case == "zero_q" else P.params_of(cfg)   # tau 2: every head pooled

    def select_with(env):
        old = {key: os.environ.get(key) for key in env}
        os.environ.update(env)
        try:
            sel = dsp.crisp_select(q, k, p, pe_prob=True)
            torch.cuda.synchronize()
        finally:
            for key, v in old.items():
                if v is None:
                    del os.environ[key]
                else:
                    os.environ[key] = v
        return sel

    a = select_with({})
    route = a.route.cpu().numpy()
    P.log(f"[cand {case}] routes VS={int((route == 1).sum())} PE={int((route == 0).sum())}")
    assert (route == 0).any()
    if case == "zero_q":
        assert (route == 0).all()
    n = int(a.row_ptr[-1])
    pe = np.repeat(route == 0, cfg.nb * (cfg.nb + 1) // 2)
    for env in ({"CRISP_PE_SMALL": "0"}, {"CRISP_PE_SMALL": "0", "CRISP_PE_CAND_CAP": "0"}):
        b = select_with(env)
        for f in ("route", "c_struct", "row_ptr", "nv", "ns"):
            assert torch.equal(getattr(a, f), getattr(b, f)), (env, f)
        assert torch.equal(a.col_idx[:n], b.col_idx[:n]), env
        assert np.array_equal(a.pe_prob.cpu().numpy()[pe], b.pe_prob.cpu().numpy()[pe]), env
    rep = P.check_decisions(a, cfg.hq, cfg.nb, p, name=f"candcap {case}")
    P.log(f"[cand {case}]", rep)
    assert rep["heads_checked"] + rep["pe_exempt"] + rep["vs_exempt"] + rep["route_ties"] == cfg.hq
    if case == "zero_q":
        # uniform rows: entry (qb, kb) is 1/(qb+1); the kept set is every row
        # above some qb*, part of row qb* in flat order, and the two anchors of
        # the rows below it
        rp = a.row_ptr.cpu().numpy()
        cnt = np.diff(rp)
        full = cnt == np.tile(np.arange(1, cfg.nb + 1), cfg.hq)
        for h in range(cfg.hq):
            c = cnt[h * cfg.nb:(h + 1) * cfg.nb]
            f_ = full[h * cfg.nb:(h + 1) * cfg.nb]
            part = np.nonzero(~f_)[0]
            assert part.size and f_[:part[0]].all(), "rows before the cut are whole"
            assert np.all(c[part[1:]] == np.minimum(2, part[1:] + 1)), "rows past the cut keep their anchors"


def test_selection_is_deterministic():
    cfg = synth.custom_config("det", 16384, 8, 2, seed=41, conc_frac=0.5)
    spec = synth.make_spec(cfg)
    Q, K, V = synth.generate(spec)
    q, k = P.to_device(spec, Q), P.to_device(spec, K)
    p = P.params_of(cfg)
    a = dsp.crisp_select(q, k, p, pe_prob=True)
    b = dsp.crisp_select(q, k, p, pe_prob=True)
    torch.cuda.synchronize()
    for f in ("route", "c_struct", "row_ptr", "pv", "ps", "nv", "ns"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f
    # pooled probabilities are written for Pooled-Estimation heads only
    t = cfg.nb * (cfg.nb + 1) // 2
    for h in range(cfg.hq):
        if a.route[h].item() == 0:
            assert torch.equal(a.pe_prob[h * t:(h + 1) * t], b.pe_prob[h * t:(h + 1) * t])
    n = int(a.row_ptr[-1])
    assert torch.equal(a.col_idx[:n], b.col_idx[:n])


def test_attention_is_deterministic():
    """The persistent attention kernel hands items to work-groups in a different
    order on every call (atomic queues, stealing), but each output row is
    computed by one work-group in a fixed key order: outputs are bitwise
    reproducible, sparse and dense."""
    cfg = synth.custom_config("det-attn", 16384, 8, 2, seed=42, conc_frac=0.5)
    spec = synth.make_spec(cfg)
    Q, K, V = synth.generate(spec)
    q, k, v = P.to_device(spec, Q), P.to_device(spec, K), P.to_device(spec, V)
    sel = dsp.crisp_select(q, k, P.params_of(cfg))
    outs = [dsp.crisp_sparse_attn(q, k, v, sel) for _ in range(3)]
    dense = [dsp.crisp_dense_attn(q, k, v) for _ in range(2)]
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    assert torch.equal(dense[0], dense[1])


def test_calls_on_two_streams_overlap_safely():
    """Two layers prefilled at once on two streams (default priority), each with
    its own outputs and workspace, give bitwise the results of calls made one
    after the other (the library keeps no state between calls)."""
    layers = []
    for i, (hq, hkv) in enumerate(((8, 2), (4, 4))):
        cfg = synth.custom_config(f"streams{i}", 8192, hq, hkv, seed=90 + i, conc_frac=0.5)
        spec = synth.make_spec(cfg)
        Q, K, V = synth.generate(spec)
        layers.append((P.to_device(spec, Q), P.to_device(spec, K), P.to_device(spec, V), P.params_of(cfg)))
    ref = [dsp.crisp_prefill(q, k, v, p)[0] for q, k, v, p in layers]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for (q, k, v, p), st in zip(layers, streams):
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            outs.append(dsp.crisp_prefill(q, k, v, p)[0])
    torch.cuda.synchronize()
    for o, r in zip(outs, ref):
        assert torch.equal(o, r)


def test_output_is_causal():
    cfg = synth.custom_config("causal", 4096, 4, 2, seed=51, conc_frac=0.5)
    spec = synth.make_spec(cfg)
    Q, K, V = synth.generate(spec)
    q, k, v = P.to_device(spec, Q), P.to_device(spec, K), P.to_device(spec, V)
    o = dsp.crisp_dense_attn(q, k, v)
    i = 2500
    k2, v2 = k.clone(), v.clone()
    k2[:, i + 1:] += 3
    v2[:, i + 1:] -= 2
    o2 = dsp.crisp_dense_attn(q, k2, v2)
    torch.cuda.synchronize()
    assert torch.equal(o[:, :i + 1], o2[:, :i + 1])
    assert not torch.equal(o[:, i + 1:], o2[:, i + 1:])


# ------------------------------------------------------------------ the Llama / Qwen layers

# Full-size protocol: every decision of every head bit-exact, every head's
# proxy scores against the oracle's float64 ones, and for every head the
# output rows of query blocks 0, N_b - 1 and 14 seeded others.

_LAYERS = {}


def _layer_on_device(layer):
    """Host arrays and device tensors of a named layer, generated once per session
    (the 128k layers serve several tests)."""
    if layer.name not in _LAYERS:
        _LAYERS.clear()
        torch.cuda.empty_cache()
        spec = synth.make_spec(layer)
        Q, K, V = P.load_layer(spec)
        _LAYERS[layer.name] = (spec, Q, K, V, P.to_device(spec, Q), P.to_device(spec, K), P.to_device(spec, V))
    return _LAYERS[layer.name]


def _drop_layers():
    _LAYERS.clear()
    torch.cuda.empty_cache()


def _big_layer(layer, seed_blocks, pe_fid=None):
    spec, Q, K, V, q, k, v = _layer_on_device(layer)
    cfg = spec.cfg
    p = P.params_of(cfg)
    o, sel = dsp.crisp_prefill(q, k, v, p, pe_prob=True)
    torch.cuda.synchronize()
    route = sel.route.cpu().numpy()
    P.log(f"[{cfg.name}] routes VS={int((route == 1).sum())} PE={int((route == 0).sum())}")
    # diffuse heads route to PE; each KV group's lead concentrated head (its keys carry the
    # recency alignment) routes to VS.  Other concentrated heads go either way depending on
    # their sink / recency strength: that is the router's call, checked bit-exactly below.
    assert np.all(route[~spec.concentrated] == 0), route
    assert np.all(route[spec.lead[spec.lead >= 0]] == 1), route
    P.log(f"[{cfg.name}] C_struct", np.round(sel.c_struct.cpu().numpy(), 3).tolist())
    rep = P.check_decisions(sel, cfg.hq, cfg.nb, p, name=cfg.name)
    P.log(f"[{cfg.name}] decisions", rep)
    # no head of a named layer needs the fixed-point exemption: every list is compared
    assert rep["pe_exempt"] == 0 and rep["vs_exempt"] == 0 and rep["heads_checked"] == cfg.hq, rep
    P.log(f"[{cfg.name}] score err (every head)", P.check_score_fidelity(spec, Q, K, sel, range(cfg.hq)))
    pe = [h for h in range(cfg.hq) if route[h] == 0]
    P.log(f"[{cfg.name}] PE prob err", P.check_pe_fidelity(spec, Q, K, sel, pe[:pe_fid]))
    blocks = synth.sample_blocks(cfg.nb, 14, seed_blocks)
    mx, mean = P.check_attention_blocks(spec, Q, K, V, o, _lists_fn(sel, cfg.nb), range(cfg.hq), blocks)
    P.log(f"[{cfg.name}] attention (every head x {len(blocks)} blocks) max {mx:.2e} mean {mean:.2e}")
    return sel


def test_llama_32k_layer():
    _big_layer(synth.LLAMA_32K, 1)


@pytest.mark.timeout(900)
def test_llama_128k_layer():
    _big_layer(synth.LLAMA_128K, 2)


@pytest.mark.timeout(900)
def test_llama_128k_alpha_tau_sweep():
    """The 128k Llama layer under the sweep alpha in {0.5, 1, 2} x tau in
    {0.2, 0.3, 0.5}: every decision of every head bit-exact for the nine pairs;
    for each alpha at tau = 0.3 the output rows of every Vertical-Slash head
    (the heads alpha acts on) on 16 query blocks."""
    spec, Q, K, V, q, k, v = _layer_on_device(synth.LLAMA_128K)
    cfg = spec.cfg
    sizes = {}
    for tau in (0.2, 0.3, 0.5):
        for alpha in (0.5, 1.0, 2.0):
            p = P.params_of(cfg, tau=tau, alpha=alpha)
            sel = dsp.crisp_select(q, k, p, pe_prob=True)
            torch.cuda.synchronize()
            rep = P.check_decisions(sel, cfg.hq, cfg.nb, p, name=f"{cfg.name} sweep")
            assert rep["pe_exempt"] == 0 and rep["heads_checked"] == cfg.hq, rep
            vs = sel.route.cpu().numpy() == 1
            sizes[(tau, alpha)] = (int(vs.sum()), float(sel.nv.cpu().numpy()[vs].mean()) if vs.any() else 0.0)
    P.log(f"[{cfg.name} sweep] (VS heads, mean |S_v|) per (tau, alpha)", sizes)
    for tau in (0.2, 0.3, 0.5):                   # the budget shrinks as alpha grows
        assert sizes[(tau, 0.5)][1] >= sizes[(tau, 1.0)][1] >= sizes[(tau, 2.0)][1]
    for alpha in (0.5, 2.0):                      # alpha = 1 is the layer test above
        p = P.params_of(cfg, alpha=alpha)
        o, sel = dsp.crisp_prefill(q, k, v, p)
        torch.cuda.synchronize()
        route = sel.route.cpu().numpy()
        heads = [h for h in range(cfg.hq) if route[h] == 1]
        blocks = synth.sample_blocks(cfg.nb, 14, 20 + int(alpha * 2))
        mx, mean = P.check_attention_blocks(spec, Q, K, V, o, _lists_fn(sel, cfg.nb), heads, blocks)
        P.log(f"[{cfg.name} alpha={alpha}] attention ({len(heads)} VS heads x {len(blocks)} blocks) "
              f"max {mx:.2e} mean {mean:.2e}")


@pytest.mark.timeout(900)
def test_dense_attention_llama_128k():
    """Dense attention at 128k, where K and V (512 MB) exceed the last-level
    cache and the persistent kernel orders its work two KV groups at a time:
    one query head of every KV group (a different member of each group) on 16
    query blocks against the oracle's causal attention."""
    spec, Q, K, V, q, k, v = _layer_on_device(synth.LLAMA_128K)
    cfg = spec.cfg
    o = dsp.crisp_dense_attn(q, k, v)
    torch.cuda.synchronize()
    G = cfg.hq // cfg.hkv
    heads = [g * G + g % G for g in range(cfg.hkv)]
    blocks = synth.sample_blocks(cfg.nb, 14, 6)
    mx, mean = P.check_attention_blocks(spec, Q, K, V, o, lambda h, qb: range(qb + 1), heads, blocks)
    P.log(f"[{cfg.name} dense] attention ({len(heads)} heads x {len(blocks)} blocks) max {mx:.2e} mean {mean:.2e}")
    _drop_layers()


@pytest.mark.timeout(900)
def test_qwen_128k_layer():
    _big_layer(synth.QWEN_128K, 3)
    _drop_layers()


@pytest.mark.timeout(1200)
def test_llama_512k_layer():
    _big_layer(synth.LLAMA_512K, 4, pe_fid=4)
    _drop_layers()


@pytest.mark.timeout(1200)
def test_maximum_length_layer():
    """The longest sequence the ABI takes: N_b = 32768 blocks (4,194,304
    tokens), one concentrated and one diffuse query head with their own KV
    heads.  The pooled triangle and the worst-case list capacity hold 537M
    entries per head, so the 64-bit offsets of the pooled matrix, the lists and
    the row scan are all exercised.  The Vertical-Slash head: every decision
    bit-exact against the oracle.  The Pooled-Estimation head (the oracle's
    sort of 537M entries is out of reach): the properties every correct cut has,
    checked on the GPU's own float32 P in float64 -- rows that sum to one, the
    selected mass at least gamma of the total (up to the fixed-point bound),
    every unselected entry no larger than the smallest selected non-anchor
    entry, lists ascending with both anchors.  Output rows of both heads on
    sampled query blocks against the oracle."""
    n = 32768 * 128
    cfg = synth.custom_config("max-nb-32768", n, 2, 2, seed=211, conc_frac=0.5)
    spec = synth.make_spec(cfg)
    assert spec.concentrated.tolist() == [True, False]
    Q, K, V = P.load_layer(spec)
    q, k, v = P.to_device(spec, Q), P.to_device(spec, K), P.to_device(spec, V)
    p = P.params_of(cfg)
    o, sel = dsp.crisp_prefill(q, k, v, p, pe_prob=True)
    torch.cuda.synchronize()
    del q, k, v
    nb = cfg.nb
    assert sel.route.cpu().tolist() == [1, 0], sel.route
    rep = P.check_decisions(sel, cfg.hq, nb, p, heads=[0], name=cfg.name)
    assert rep["heads_checked"] == 1, rep
    P.log(f"[{cfg.name}] score err (VS head)", P.check_score_fidelity(spec, Q, K, sel, [0]))
    # the Pooled-Estimation head's cut, on the GPU's own probabilities (float64 on the device)
    T = nb * (nb + 1) // 2
    Pf = sel.pe_prob[T:2 * T].double()
    starts = torch.arange(nb, device="cuda", dtype=torch.int64)
    starts = starts * (starts + 1) // 2
    cs = torch.cumsum(Pf, 0)
    ends = cs[starts + torch.arange(nb, device="cuda")]
    row_sums = ends - torch.cat([torch.zeros(1, device="cuda", dtype=torch.float64), ends[:-1]])
    assert float((row_sums - 1).abs().max()) < 1e-4
    total = float(cs[-1])
    rp = sel.row_ptr.to(torch.int64)
    a, b = int(rp[nb]), int(rp[2 * nb])
    cols = sel.col_idx[a:b].to(torch.int64)
    lens = (rp[nb + 1:2 * nb + 1] - rp[nb:2 * nb])
    rows = torch.repeat_interleave(torch.arange(nb, device="cuda"), lens)
    assert bool((cols <= rows).all()) and bool((cols >= 0).all())
    first = rp[nb:2 * nb] - a
    last = rp[nb + 1:2 * nb + 1] - a - 1
    assert bool((cols[first] == 0).all()) and bool((cols[last] == torch.arange(nb, device="cuda")).all())
    inner = torch.ones_like(cols, dtype=torch.bool)
    inner[first] = False
    assert bool((cols[1:][inner[1:]] > cols[:-1][inner[1:]]).all())          # ascending within each row
    flat = starts[rows] + cols
    chosen = torch.zeros(T, dtype=torch.bool, device="cuda")
    chosen[flat] = True
    mass = float(Pf[chosen].sum())
    gamma = float(np.float32(p.gamma))                  # the cut is taken at the float32 parameter
    assert mass >= gamma * total - T * 2.0 ** -45, (mass, total)
    anchor = torch.zeros(T, dtype=torch.bool, device="cuda")
    anchor[starts] = True
    anchor[starts + torch.arange(nb, device="cuda")] = True
    smallest_kept = float(Pf[chosen & ~anchor].min())
    largest_dropped = float(Pf[~chosen].max())
    assert largest_dropped <= smallest_kept, (largest_dropped, smallest_kept)
    density = (b - a) / T
    P.log(f"[{cfg.name}] PE head: kept mass {mass / total:.6f} of {total:.1f}, density {density:.3f}, "
          f"dropped <= {largest_dropped:.3e} <= kept {smallest_kept:.3e}")
    del Pf, cs, chosen, anchor, flat, rows
    torch.cuda.empty_cache()
    rpn, col = P.gpu_lists(sel, cfg.hq, nb)
    blocks = synth.sample_blocks(nb, 4, 12)
    mx, mean = P.check_attention_blocks(spec, Q, K, V, o, lambda h, qb: col[rpn[h * nb + qb]: rpn[h * nb + qb + 1]],
                                        [0, 1], blocks, threads=3)
    P.log(f"[{cfg.name}] attention (2 heads x {len(blocks)} blocks) max {mx:.2e} mean {mean:.2e}")


@pytest.mark.timeout(900)
def test_odd_kv_count_beyond_cache():
    """Three KV groups at 196,608 tokens: K and V take 302 MB, more than the
    256 MB last-level cache, so the attention work is ordered two groups at a
    time and the third group runs alone.  Sparse and dense outputs of every
    head on sampled blocks, every decision bit-exact."""
    cfg = synth.custom_config("odd-kv-196k", 196608, 6, 3, seed=17, conc_frac=0.5)
    spec = synth.make_spec(cfg)
    Q, K, V = P.load_layer(spec)
    q, k, v = P.to_device(spec, Q), P.to_device(spec, K), P.to_device(spec, V)
    p = P.params_of(cfg)
    o, sel = dsp.crisp_prefill(q, k, v, p, pe_prob=True)
    od = dsp.crisp_dense_attn(q, k, v)
    torch.cuda.synchronize()
    rep = P.check_decisions(sel, cfg.hq, cfg.nb, p, name=cfg.name)
    assert rep["heads_checked"] + rep["pe_exempt"] == cfg.hq, rep
    route = sel.route.cpu().numpy()
    assert (route == 1).any() and (route == 0).any(), route
    blocks = synth.sample_blocks(cfg.nb, 14, 8)
    mx, mean = P.check_attention_blocks(spec, Q, K, V, o, _lists_fn(sel, cfg.nb), range(cfg.hq), blocks)
    P.log(f"[{cfg.name}] sparse attention max {mx:.2e} mean {mean:.2e}")
    mx, mean = P.check_attention_blocks(spec, Q, K, V, od, lambda h, qb: range(qb + 1), range(cfg.hq), blocks[::2])
    P.log(f"[{cfg.name}] dense attention max {mx:.2e} mean {mean:.2e}")


@pytest.mark.parametrize("sink,local", [(0, 0), (64, 200), (200, 64), (1, 1), (127, 129), (300, 1000),
                                        (0, 4096), (4096, 0)])
def test_anchor_windows(sink, local):
    """Sink and recency windows that are not one block [CRISP §3.2: w_sink and
    w_local are parameters]: windows inside a tile, across tile edges, empty,
    and the whole sequence.  C_struct against the oracle's (same windows), every
    decision bit-exact (route at the default tau and at tau = 0), full outputs."""
    cfg = synth.custom_config("anchors", 4096, 4, 2, seed=71, conc_frac=0.5)
    spec = synth.make_spec(cfg)
    Q, K, V = synth.generate(spec)
    q, k, v = P.to_device(spec, Q), P.to_device(spec, K), P.to_device(spec, V)
    for tau in (cfg.tau, 0.0):
        p = P.params_of(cfg, sink=sink, local=local, tau=tau)
        o, sel = dsp.crisp_prefill(q, k, v, p, pe_prob=True)
        torch.cuda.synchronize()
        err = P.check_score_fidelity(spec, Q, K, sel, range(cfg.hq), sink=sink, local=local)
        rep = P.check_decisions(sel, cfg.hq, cfg.nb, p)
        assert rep["heads_checked"] + rep["pe_exempt"] == cfg.hq, rep
        cs = sel.c_struct.cpu().numpy()
        if sink == 0 and local == 0:
            assert np.all(cs == 0)
        if tau == 0.0:
            assert np.all(sel.route.cpu().numpy() == 1)          # C_struct >= 0 always
        P.log(f"[anchors {sink}/{local} tau={tau}] C_struct {np.round(cs, 4).tolist()} score err {err:.1e} "
              f"routes {sel.route.cpu().tolist()}")
        P.check_attention_blocks(spec, Q, K, V, o, _lists_fn(sel, cfg.nb), range(cfg.hq), range(cfg.nb))
    # windows covering everything: C_struct is the whole proxy mass
    if sink >= cfg.n or local >= cfg.n:
        assert np.all(np.abs(cs - 1.0) < 1e-5), cs


# ------------------------------------------------------------------ variants: JSD router, median floor, coverage budget

VARIANTS = [dsp.FLAG_ROUTE_JSD, dsp.FLAG_VS_MEDIAN, dsp.FLAG_VS_COVERAGE,
            dsp.FLAG_ROUTE_JSD | dsp.FLAG_VS_COVERAGE, dsp.FLAG_ROUTE_JSD | dsp.FLAG_VS_MEDIAN]


@pytest.mark.parametrize("n,hq,hkv,seed", [(8192, 8, 2, 21), (1664, 7, 1, 22), (384, 2, 1, 23)])
def test_variant_selection_and_output(n, hq, hkv, seed):
    """Every variant on small mixed layers: decisions bit-exact from the GPU's
    own scores, the pooled estimate and JSD against the oracle's float64 ones,
    and the full output on the variant's lists.  The JSD threshold is taken at
    0 (every head Vertical-Slash), at the median of the heads' divergences
    (both routes) and above ln 2 (every head Pooled-Estimation)."""
    cfg = synth.custom_config("variant", n, hq, hkv, seed=seed, conc_frac=0.5)
    spec = synth.make_spec(cfg)
    Q, K, V = synth.generate(spec)
    q, k, v = P.to_device(spec, Q), P.to_device(spec, K), P.to_device(spec, V)
    for flags in VARIANTS:
        taus = [cfg.tau]
        if flags & dsp.FLAG_ROUTE_JSD:
            sel0 = dsp.crisp_select(q, k, P.params_of(cfg, tau=0.0, flags=flags), pe_prob=True)
            torch.cuda.synchronize()
            P.log(f"[variant {flags} n={n}] jsd err", P.check_jsd_fidelity(spec, Q, K, sel0, range(hq)))
            taus = [0.0, float(np.median(sel0.jsd.cpu().numpy())), 1.0]
        for tau in taus:
            p = P.params_of(cfg, tau=tau, flags=flags)
            o, sel = dsp.crisp_prefill(q, k, v, p, pe_prob=True)
            torch.cuda.synchronize()
            rep = P.check_decisions(sel, hq, cfg.nb, p)
            route = sel.route.cpu().numpy()
            P.log(f"[variant {flags} n={n} tau={tau:.4g}] routes {route.tolist()} decisions", rep)
            assert rep["heads_checked"] + rep["pe_exempt"] + rep["vs_exempt"] + rep["route_ties"] == hq
            if flags & dsp.FLAG_ROUTE_JSD and tau == 0.0:
                assert np.all(route == 1)
            if tau == 1.0:
                assert np.all(route == 0)
            P.check_attention_blocks(spec, Q, K, V, o, _lists_fn(sel, cfg.nb), range(hq), range(cfg.nb))


def test_variant_min_blocks_and_gamma_sweep():
    cfg = synth.custom_config("vsweep", 8192, 8, 2, seed=31, conc_frac=0.5)
    spec = synth.make_spec(cfg)
    Q, K, V = synth.generate(spec)
    q, k = P.to_device(spec, Q), P.to_device(spec, K)
    for flags in (dsp.FLAG_VS_MEDIAN, dsp.FLAG_VS_COVERAGE):
        for alpha, gamma in ((0.5, 0.9), (1.0, 0.95), (2.0, 0.99), (1.0, 1.0)):
            for mb in (0, 8):
                p = P.params_of(cfg, tau=0.2, alpha=alpha, gamma=gamma, min_blocks=mb, flags=flags)
                sel = dsp.crisp_select(q, k, p, pe_prob=True)
                torch.cuda.synchronize()
                rep = P.check_decisions(sel, cfg.hq, cfg.nb, p)
                vs = sel.route.cpu().numpy() == 1
                if mb:
                    assert np.all(sel.nv.cpu().numpy()[vs] >= mb) and np.all(sel.ns.cpu().numpy()[vs] >= mb)
                if flags == dsp.FLAG_VS_COVERAGE and gamma == 1.0:
                    assert np.all(sel.nv.cpu().numpy()[vs] == cfg.nb)


@pytest.mark.timeout(900)
def test_flexprefill_configuration_llama_128k():
    """FlexPrefill's pair of rules (JSD router, coverage budget at gamma 0.95)
    on the Llama 128k layer: decisions in full, sampled outputs."""
    spec, Q, K, V, q, k, v = _layer_on_device(synth.LLAMA_128K)
    cfg = spec.cfg
    flags = dsp.FLAG_ROUTE_JSD | dsp.FLAG_VS_COVERAGE
    sel0 = dsp.crisp_select(q, k, P.params_of(cfg, tau=0.0, flags=flags))
    torch.cuda.synchronize()
    js = sel0.jsd.cpu().numpy()
    P.log("[flex 128k] jsd", np.round(js, 4).tolist())
    P.log("[flex 128k] jsd err", P.check_jsd_fidelity(spec, Q, K, sel0, [0, 1, 31]))
    p = P.params_of(cfg, tau=float(np.median(js)), flags=flags)
    o, sel = dsp.crisp_prefill(q, k, v, p, pe_prob=True)
    torch.cuda.synchronize()
    _drop_layers()
    rep = P.check_decisions(sel, cfg.hq, cfg.nb, p, name=f"{cfg.name} FlexPrefill")
    P.log("[flex 128k] decisions", rep, "routes", sel.route.cpu().tolist())
    assert rep["heads_checked"] + rep["pe_exempt"] + rep["vs_exempt"] + rep["route_ties"] == cfg.hq
    route = sel.route.cpu().numpy()
    heads = [h for h in range(cfg.hq) if route[h] == 1][:2] + [h for h in range(cfg.hq) if route[h] == 0][:1]
    blocks = synth.sample_blocks(cfg.nb, 4, 5)
    mx, mean = P.check_attention_blocks(spec, Q, K, V, o, _lists_fn(sel, cfg.nb), heads, blocks)
    P.log(f"[flex 128k] attention max {mx:.2e} mean {mean:.2e}")


# ------------------------------------------------------------------ packed batches (varlen)

@pytest.mark.parametrize("flags", [0, dsp.FLAG_ROUTE_JSD | dsp.FLAG_VS_COVERAGE])
def test_varlen_batch_equals_single_calls(flags):
    """Three sequences of different lengths (one short enough for the dense
    path) packed into one call: every selection output and every output row is
    bitwise equal to running each sequence alone; one sequence's outputs are
    also checked against the oracle."""
    lens = [8192, 2048, 256, 4096]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    hq, hkv = 8, 2
    parts = []
    for i, n in enumerate(lens):
        cfg = synth.custom_config(f"varlen{i}", n, hq, hkv, seed=60 + i, conc_frac=0.5)
        spec = synth.make_spec(cfg)
        parts.append((spec,) + synth.generate(spec))
    Q = np.concatenate([p[1] for p in parts], axis=1)
    K = np.concatenate([p[2] for p in parts], axis=1)
    V = np.concatenate([p[3] for p in parts], axis=1)
    spec0 = parts[0][0]
    q, k, v = P.to_device(spec0, Q), P.to_device(spec0, K), P.to_device(spec0, V)
    params = P.params_of(spec0.cfg, tau=0.01 if flags else 0.3, flags=flags)
    o, sel = dsp.crisp_prefill_varlen(q, k, v, cu, params, pe_prob=True)
    torch.cuda.synchronize()
    rows0, rp0, col0 = 0, 0, 0
    for i, n in enumerate(lens):
        a, b = cu[i], cu[i + 1]
        nb = n // 128
        qi, ki, vi = q[:, a:b].contiguous(), k[:, a:b].contiguous(), v[:, a:b].contiguous()
        oi, si = dsp.crisp_prefill(qi, ki, vi, params, pe_prob=True)
        torch.cuda.synchronize()
        assert torch.equal(o[:, a:b], oi), f"sequence {i}: output differs"
        assert torch.equal(sel.route[i * hq:(i + 1) * hq], si.route)
        assert torch.equal(sel.c_struct[i * hq:(i + 1) * hq], si.c_struct)
        assert torch.equal(sel.row_ptr[rp0:rp0 + hq * nb + 1], si.row_ptr)
        m = int(si.row_ptr[-1])
        assert torch.equal(sel.col_idx[col0:col0 + m], si.col_idx[:m])
        if si.route[0].item() != -1:
            assert torch.equal(sel.pv[rows0:rows0 + hq * nb], si.pv)
            if flags:
                assert torch.equal(sel.jsd[i * hq:(i + 1) * hq], si.jsd)
        rows0 += hq * nb
        rp0 += hq * nb + 1
        col0 += hq * nb * (nb + 1) // 2
    # the first sequence against the oracle: decisions from its own scores and sampled rows
    n0, nb0 = lens[0], lens[0] // 128
    sub = dsp.Selection(sel.route[:hq], sel.c_struct[:hq], sel.row_ptr[:hq * nb0 + 1], sel.col_idx,
                        sel.pv[:hq * nb0], sel.ps[:hq * nb0], sel.sv[:hq * nb0], sel.nv[:hq], sel.ss[:hq * nb0],
                        sel.ns[:hq], sel.pe_prob, sel.jsd[:hq], sel.abar[:hq * nb0])
    rep = P.check_decisions(sub, hq, nb0, params)
    P.log(f"[varlen flags={flags}] decisions", rep)
    rp, col = P.gpu_lists(sub, hq, nb0)
    lists = lambda h, qb: col[rp[h * nb0 + qb]: rp[h * nb0 + qb + 1]]
    mx, mean = P.check_attention_blocks(parts[0][0], parts[0][1], parts[0][2], parts[0][3], o[:, :n0], lists,
                                        range(hq), synth.sample_blocks(nb0, 6, 7))
    P.log(f"[varlen] attention max {mx:.2e} mean {mean:.2e}")


def test_varlen_fp32_and_gqa7():
    """Packed batch on the fp32 path (per-sequence attention launches) and with
    GQA 7:1: outputs and lists bitwise equal to single calls."""
    for dtype, hq, hkv, lens in (("fp32", 2, 2, [1024, 384, 2048]), ("bf16", 7, 1, [1664, 4096, 128])):
        cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
        parts = []
        for i, n in enumerate(lens):
            cfg = synth.custom_config(f"vl-{dtype}-{i}", n, hq, hkv, dtype=dtype, seed=80 + i, conc_frac=0.5)
            spec = synth.make_spec(cfg)
            parts.append((spec,) + synth.generate(spec))
        spec0 = parts[0][0]
        q = P.to_device(spec0, np.concatenate([p[1] for p in parts], axis=1))
        k = P.to_device(spec0, np.concatenate([p[2] for p in parts], axis=1))
        v = P.to_device(spec0, np.concatenate([p[3] for p in parts], axis=1))
        params = P.params_of(spec0.cfg)
        o, sel = dsp.crisp_prefill_varlen(q, k, v, cu, params)
        torch.cuda.synchronize()
        rp0, col0 = 0, 0
        for i, n in enumerate(lens):
            a, b = cu[i], cu[i + 1]
            nb = n // 128
            oi, si = dsp.crisp_prefill(q[:, a:b].contiguous(), k[:, a:b].contiguous(), v[:, a:b].contiguous(), params)
            torch.cuda.synchronize()
            assert torch.equal(o[:, a:b], oi), f"{dtype} sequence {i}: output differs"
            assert torch.equal(sel.route[i * hq:(i + 1) * hq], si.route)
            assert torch.equal(sel.row_ptr[rp0:rp0 + hq * nb + 1], si.row_ptr)
            m = int(si.row_ptr[-1])
            assert torch.equal(sel.col_idx[col0:col0 + m], si.col_idx[:m])
            rp0 += hq * nb + 1
            col0 += hq * nb * (nb + 1) // 2


def test_pe_cut_small_varlen_equals_general():
    """A packed batch of short sequences (13, 3, 64 and 1 blocks, every one at
    most 64 blocks, so the gamma cut of each Pooled-Estimation head is taken in
    one work-group) against the general radix passes (CRISP_PE_SMALL=0): the
    whole selection, the pooled probabilities and the outputs are bitwise the
    same.  The second sequence has Q = 0, so its pooled rows are uniform and
    the cut splits a run of equal values."""
    lens = [1664, 384, 8192, 128]
    hq, hkv = 4, 1
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    parts = []
    for i, n in enumerate(lens):
        cfg = synth.custom_config(f"pesmall{i}", n, hq, hkv, seed=90 + i, conc_frac=0.25)
        spec = synth.make_spec(cfg)
        Q, K, V = synth.generate(spec)
        if i == 1:
            Q[:] = 0
        parts.append((spec, Q, K, V))
    spec0 = parts[0][0]
    q = P.to_device(spec0, np.concatenate([p[1] for p in parts], axis=1))
    k = P.to_device(spec0, np.concatenate([p[2] for p in parts], axis=1))
    v = P.to_device(spec0, np.concatenate([p[3] for p in parts], axis=1))
    params = P.params_of(spec0.cfg, tau=0.9)   # most heads pooled (uniform Q: C_struct = 256 / 384)
    o, sel = dsp.crisp_prefill_varlen(q, k, v, cu, params, pe_prob=True)
    torch.cuda.synchronize()
    os.environ["CRISP_PE_SMALL"] = "0"
    try:
        o2, sel2 = dsp.crisp_prefill_varlen(q, k, v, cu, params, pe_prob=True)
        torch.cuda.synchronize()
    finally:
        del os.environ["CRISP_PE_SMALL"]
    route = sel.route.cpu().numpy()
    P.log(f"[pe small varlen] routes {route.tolist()}")
    assert (route == 0).sum() >= 4
    for f in ("route", "c_struct", "row_ptr", "nv", "ns"):
        assert torch.equal(getattr(sel, f), getattr(sel2, f)), f
    n = int(sel.row_ptr[-1])
    assert torch.equal(sel.col_idx[:n], sel2.col_idx[:n])
    off = 0   # pooled probabilities of the Pooled-Estimation heads, sequence by sequence
    for i, ln in enumerate(lens):
        nb = ln // 128
        tri = nb * (nb + 1) // 2
        for h in range(hq):
            if route[i * hq + h] == 0:
                a, b = off + h * tri, off + (h + 1) * tri
                assert torch.equal(sel.pe_prob[a:b], sel2.pe_prob[a:b]), (i, h)
        off += hq * tri
    assert torch.equal(o, o2)


def test_varlen_multi_tile_row_scan():
    """A packed batch whose sequences need different numbers of 4096-row tiles
    in the row-pointer scan (hq * N_b = 4608, 160 and 2560 rows) and different
    numbers of pooled-logit row groups: selection outputs, lists and outputs
    bitwise equal to single calls."""
    hq, hkv, lens = 16, 4, [36864, 1280, 20480]
    cu = np.concatenate([[0], np.cumsum(lens)]).tolist()
    parts = []
    for i, n in enumerate(lens):
        cfg = synth.custom_config(f"vl-tiles-{i}", n, hq, hkv, seed=90 + i, conc_frac=0.5)
        spec = synth.make_spec(cfg)
        parts.append((spec,) + synth.generate(spec))
    spec0 = parts[0][0]
    q = P.to_device(spec0, np.concatenate([p[1] for p in parts], axis=1))
    k = P.to_device(spec0, np.concatenate([p[2] for p in parts], axis=1))
    v = P.to_device(spec0, np.concatenate([p[3] for p in parts], axis=1))
    params = P.params_of(spec0.cfg)
    o, sel = dsp.crisp_prefill_varlen(q, k, v, cu, params)
    torch.cuda.synchronize()
    assert int((sel.route == 0).sum()) > 0 and int((sel.route == 1).sum()) > 0   # both paths exercised
    rows0, rp0, col0 = 0, 0, 0
    for i, n in enumerate(lens):
        a, b = cu[i], cu[i + 1]
        nb = n // 128
        oi, si = dsp.crisp_prefill(q[:, a:b].contiguous(), k[:, a:b].contiguous(), v[:, a:b].contiguous(), params)
        torch.cuda.synchronize()
        assert torch.equal(o[:, a:b], oi), f"sequence {i}: output differs"
        assert torch.equal(sel.route[i * hq:(i + 1) * hq], si.route)
        assert torch.equal(sel.row_ptr[rp0:rp0 + hq * nb + 1], si.row_ptr), f"sequence {i}: row pointers differ"
        m = int(si.row_ptr[-1])
        assert torch.equal(sel.col_idx[col0:col0 + m], si.col_idx[:m])
        assert torch.equal(sel.pv[rows0:rows0 + hq * nb], si.pv)
        rows0 += hq * nb
        rp0 += hq * nb + 1
        col0 += hq * nb * (nb + 1) // 2
