"""The seeded input generator: determinism, slicing, moments and the workload table."""
import math

import numpy as np

import synth
from synth import gen


def test_keys_differ_per_tensor_and_are_stable():
    keys = {gen.tensor_key(0, w, l, t, e) for w in range(5) for l in range(2) for t in range(6) for e in range(3)}
    assert len(keys) == 5 * 2 * 6 * 3
    assert gen.tensor_key(0, 1, 0, 3, 5) == gen.tensor_key(0, 1, 0, 3, 5)


def test_slices_and_gathers_agree_with_full_fill():
    key = gen.tensor_key(0, 9, 0, 0, 0)
    full = gen.host_fill(key, 10_000, 1.0, "f32")
    np.testing.assert_array_equal(gen.host_fill(key, 1000, 1.0, "f32", first=4321), full[4321:5321])
    idx = np.array([0, 7, 9999, 1234])
    np.testing.assert_array_equal(gen.host_gather(key, idx, 1.0), full[idx])
    b = gen.host_fill(key, 10_000, 1.0, "bf16")
    import torch
    ref = torch.from_numpy(full.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(b, ref)


def test_moments_match_the_requested_normal():
    key = gen.tensor_key(0, 9, 0, 1, 0)
    v = gen.host_fill(key, 2_000_000, 0.25, "f32").astype(np.float64)
    assert abs(v.mean()) < 0.25 * 3e-3
    assert abs(v.std() / 0.25 - 1) < 2e-3
    assert np.abs(v).max() <= 0.25 * math.sqrt(12.0) * 1.0001       # Irwin-Hall(4) support
    kurt = ((v - v.mean()) ** 4).mean() / v.var() ** 2
    assert abs(kurt - (3 - 1.2 / 4)) < 0.02                           # 2.7 for n = 4


def test_workload_table():
    c = synth.get_config("prefill8k_bf16")
    assert (c.T, c.H, c.I, c.E, c.k, c.shared) == (8192, 7168, 2048, 256, 8, 1)
    assert c.weight_bytes_per_expert() == 88_080_384
    assert c.flops_ffn() == 6_493_990_551_552
    f = synth.get_config("prefill16k_fp8")
    assert f.weight_bytes_per_expert() == 44_050_944
    imb = synth.get_config("imbalanced_bf16")
    lens = synth.seq_lengths(imb)
    assert len(lens) == 4 and imb.T == lens.sum() and lens.min() >= 6554 and lens.max() <= 8192
    z = synth.router_bias(imb)
    assert sorted(np.round(np.exp(-z / 1.1)).astype(int)) == list(range(1, 257))   # a permutation of ranks
