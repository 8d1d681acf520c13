"""The seeded input generator: determinism, row-range regeneration, rounding."""
import numpy as np
import torch

from workloads import synth


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 7
    x[:5] = [0.0, -0.0, 1.0, 3.0000002, -2.9999998]
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.to_bf16_bits(x), want)
    back = synth.bf16_bits_to_f32(want)
    assert np.array_equal(back, torch.from_numpy(want.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_generation_is_deterministic_and_row_ranges_regenerate():
    cfg = synth.custom_config("t", 16384, 4, 2, seed=5, conc_frac=0.5)
    spec = synth.make_spec(cfg)
    Q1, K1, V1 = synth.generate(spec, threads=4)
    Q2, K2, V2 = synth.generate(synth.make_spec(cfg), threads=2)
    assert np.array_equal(Q1, Q2) and np.array_equal(K1, K2) and np.array_equal(V1, V2)
    for (r0, r1) in [(0, 10), (4000, 4200), (16384 - 300, 16384)]:
        assert np.array_equal(synth.rows(spec, "q", 3, r0, r1), Q1[3, r0:r1])
        assert np.array_equal(synth.rows(spec, "k", 1, r0, r1), K1[1, r0:r1])
        assert np.array_equal(synth.rows(spec, "v", 0, r0, r1), V1[0, r0:r1])


def test_head_mix_and_planting():
    spec = synth.make_spec(synth.LLAMA_32K)
    assert spec.concentrated.sum() == 19
    spec3 = synth.make_spec(synth.QWEN_128K)
    assert spec3.concentrated.sum() == round(0.45 * 28)
    for g in range(8):
        assert 2 <= len(spec.needle_blocks[g]) <= 8
        assert all(1 <= b <= 256 - 2 for b in spec.needle_blocks[g])
    lit = synth.make_spec(synth.LLAMA_32K, compensate=False)
    assert np.all(lit.c < spec.c) and np.all(lit.rho < spec.rho)
    assert np.allclose(spec.c - lit.c, np.log(8) * np.sqrt(128) / 4, atol=1e-5)
