"""The allocation-free prefill (crisp_prefill_noalloc) against crisp_prefill:
same kernels, its workspace in the library's fixed scratch array instead of a
caller buffer.  Two calls in a row, the second on a smaller layer (the scratch
keeps the first call's contents), each bitwise equal to crisp_prefill on the
same inputs; the first layer's outputs are also checked against the oracle."""
import numpy as np
import pytest
import torch

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


def _layer(n, hq, hkv, seed):
    cfg = synth.custom_config(f"noalloc-{n}", n, hq, hkv, seed=seed, conc_frac=0.5)
    spec = synth.make_spec(cfg)
    Q, K, V = synth.generate(spec)
    return spec, (Q, K, V), [P.to_device(spec, X) for X in (Q, K, V)]


def _equal_selection(a, b, nb, hq):
    for f in ("route", "c_struct", "row_ptr", "pv", "ps", "nv", "ns"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f
    m = int(b.row_ptr[-1])
    assert int(a.row_ptr[-1]) == m
    assert torch.equal(a.col_idx[:m], b.col_idx[:m])


def test_noalloc_prefill_equals_prefill_twice_shrinking():
    # a layer using about 3/4 of the scratch first, then a smaller one
    for n, hq, hkv, seed in ((65536, 16, 4, 301), (2048, 4, 2, 302)):
        spec, host, (q, k, v) = _layer(n, hq, hkv, seed)
        cfg = spec.cfg
        p = P.params_of(cfg)
        shape = dsp.make_shape(q, k, v, q)
        need = dsp.workspace_bytes(shape, p)
        assert need <= dsp.noalloc_scratch_bytes(), need
        ref_o, ref_sel = dsp.crisp_prefill(q, k, v, p)
        sel = dsp.new_selection(q, k)
        o = torch.full_like(q, float("nan"))
        torch.cuda.synchronize()
        dsp.crisp_prefill_noalloc(q, k, v, p, sel, o)
        torch.cuda.synchronize()
        _equal_selection(sel, ref_sel, cfg.nb, hq)
        assert torch.equal(o, ref_o)
        route = sel.route.cpu().numpy()
        assert (route == 1).any() and (route == 0).any(), route
        # the oracle on the same outputs: decisions from the GPU's scores, sampled rows
        sel_pe = dsp.new_selection(q, k, pe_prob=True)
        dsp.crisp_prefill_noalloc(q, k, v, p, sel_pe, o)
        torch.cuda.synchronize()
        rep = P.check_decisions(sel_pe, hq, cfg.nb, p)
        assert rep["heads_checked"] + rep["pe_exempt"] == hq, rep
        rp, col = P.gpu_lists(sel_pe, hq, cfg.nb)
        Q, K, V = host
        P.check_attention_blocks(spec, Q, K, V, o, lambda h, qb: col[rp[h * cfg.nb + qb]: rp[h * cfg.nb + qb + 1]],
                                 range(hq), synth.sample_blocks(cfg.nb, 6, 3))
        P.log(f"[noalloc n={n}] equal to crisp_prefill; decisions {rep}")
    # beyond the scratch: rejected before anything is launched (inputs need no values)
    n_big, hq, hkv = 131072, 32, 8
    z = lambda h: torch.zeros(h, n_big, 128, dtype=torch.bfloat16, device="cuda")
    q, k, v = z(hq), z(hkv), z(hkv)
    p = dsp.CrispParams()
    assert dsp.workspace_bytes(dsp.make_shape(q, k, v, q), p) > dsp.noalloc_scratch_bytes()
    with pytest.raises(dsp.CrispError) as e:
        dsp.crisp_prefill_noalloc(q, k, v, p, dsp.new_selection(q, k), torch.empty_like(q))
    assert e.value.status == -5
