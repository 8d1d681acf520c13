"""A whole crisp_prefill captured in a HIP graph: every replay equals the eager call.

The library allocates nothing, never synchronises and clears its work counters
with kernels (no memset nodes), so a caller can capture a prefill into a graph
with buffers allocated beforehand.  The graph is replayed several times with
eager work and synchronisations between the replays (outputs and workspace are
filled with garbage by a fill kernel before each), and every replay is compared
bit for bit with the eager result: route, C_struct, the CSR lists and the
output.
"""
import pytest
import torch

from workloads import synth

import dynamic_sparse_prefill_amd as dsp
from tests import parity as P

pytestmark = pytest.mark.gpu


def _snapshot(o, sel, nb, hq):
    rp = sel.row_ptr[: hq * nb + 1].clone()
    nnz = int(rp[-1].item())
    return {"o": o.clone(), "route": sel.route.clone(), "c_struct": sel.c_struct.clone(), "row_ptr": rp,
            "col_idx": sel.col_idx[:nnz].clone()}


def _equal(a, b):
    for key in a:
        x, y = a[key], b[key]
        if x.shape != y.shape:
            return key
        if x.dtype == torch.bfloat16:
            x, y = x.view(torch.int16), y.view(torch.int16)
        if not torch.equal(x, y):
            return key
    return None


@pytest.mark.parametrize("n,hq,hkv,seed", [(8192, 8, 2, 71), (3072, 7, 1, 72)])
def test_prefill_replays_in_a_hip_graph(n, hq, hkv, seed):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cfg = synth.custom_config(f"graph{seed}", n, hq, hkv, seed=seed, conc_frac=0.5)
    spec = synth.make_spec(cfg)
    Q, K, V = synth.generate(spec)
    q, k, v = P.to_device(spec, Q), P.to_device(spec, K), P.to_device(spec, V)
    p = P.params_of(cfg)
    o = torch.empty_like(q)
    sel = dsp.new_selection(q, k)
    ws = torch.empty(dsp.workspace_bytes(dsp.make_shape(q, k, v, o), p), dtype=torch.uint8, device=q.device)

    dsp.crisp_prefill(q, k, v, p, sel=sel, o=o, ws=ws)            # eager reference (also warms every cache)
    torch.cuda.synchronize()
    ref = _snapshot(o, sel, cfg.nb, hq)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dsp.crisp_prefill(q, k, v, p, sel=sel, o=o, ws=ws)
    torch.cuda.synchronize()

    for rep in range(4):
        # garbage in every output and in the workspace: nothing may depend on what a buffer held
        o.fill_(float("nan"))
        sel.route.fill_(-7)
        sel.c_struct.fill_(float("nan"))
        sel.row_ptr.fill_(-1)
        sel.col_idx.fill_(-1)
        ws.fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        bad = _equal(ref, _snapshot(o, sel, cfg.nb, hq))
        P.log(f"[graph n={n} hq={hq} hkv={hkv}] replay {rep}: {'equal' if bad is None else 'differs in ' + bad}")
        assert bad is None, (rep, bad)
        # eager work between replays: another prefill on fresh buffers, then a check that it
        # agrees with the reference too
        o2, sel2 = dsp.crisp_prefill(q, k, v, p)
        torch.cuda.synchronize()
        assert _equal(ref, _snapshot(o2, sel2, cfg.nb, hq)) is None, rep
    del graph
