"""The shared input generators: determinism, bf16 encoding and document bounds."""
import numpy as np
import torch

import synth


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 3
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 0.0]  # exact ties between bf16 neighbours
    bits = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    back = synth.bf16_bits_to_f32(bits)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generators_are_deterministic_and_blockwise():
    a = synth.normal_bf16_bits(0, synth.TID_Q, (3000, 2, 8))
    b = synth.normal_bf16_bits(0, synth.TID_Q, (3000, 2, 8))
    assert np.array_equal(a, b)
    c = synth.normal_bf16_bits(1, synth.TID_Q, (3000, 2, 8))
    assert not np.array_equal(a, c)
    x = synth.bf16_bits_to_f64(a)
    assert abs(x.mean()) < 0.05 and abs(x.std() - 1) < 0.05


def test_loguniform_cu_seqlens():
    for seed in range(5):
        cu = synth.loguniform_cu_seqlens(seed, 131072, 512, 32768)
        lens = np.diff(cu)
        assert cu[0] == 0 and cu[-1] == 131072 and np.all(lens > 0)
        assert np.all(lens[:-1] >= 512) and np.all(lens <= 32768)


def test_workload_shapes():
    w = synth.LLAMA7B_ZIGZAG
    assert (w.s_total, w.hq, w.hkv, w.d, w.cp, w.partition) == (32768, 32, 32, 128, 4, "zigzag")
    g = synth.make_global_inputs(synth.TINY_RING)
    assert g.q.shape == (512, 1, 64) and g.q.dtype == np.float32
