"""The seeded input generator: host and torch backends agree bit for bit; value ranges."""

import numpy as np
import pytest
import torch

import synth
from synth import gen


def test_words_numpy_equals_torch():
    for seed, tid in [(1234, 0), (1234, 17), (5678, 3), (0, 0), (2 ** 31 - 1, 99)]:
        a = gen.words_np(1000, 5000, seed, tid)
        b = gen.words_torch(1000, 5000, seed, tid).numpy().astype(np.uint64)
        assert np.array_equal(a, b)
    # near the top of the 32-bit counter range
    a = gen.words_np(2 ** 32 - 4096, 4096, 7, 1)
    b = gen.words_torch(2 ** 32 - 4096, 4096, 7, 1).numpy().astype(np.uint64)
    assert np.array_equal(a, b)
    assert a.max() < 2 ** 32


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_normal_numpy_equals_torch(dtype):
    a = gen.normal_np((37, 129), 1234, 5, 0.02, dtype)
    t = gen.normal_torch((37, 129), 1234, 5, 0.02, dtype)
    assert np.array_equal(a, t.float().numpy())


def test_normal_table_shape_and_spread():
    t = gen.normal_table(0.02, "f32").astype(np.float64)
    assert t.shape == (65536,)
    assert np.all(np.diff(t) > 0)
    assert np.allclose(t, -t[::-1])            # symmetric quantiles
    assert abs(t.std() - 0.02) < 0.0005         # standard deviation 0.02 (not variance)
    tb = gen.normal_table(0.02, "bf16")
    assert np.array_equal(gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(tb)), tb)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 0.0], dtype=np.float32)
    got = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(x))
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(got, ref)


def test_tokens_range_and_backends():
    a = gen.tokens_np((4, 1000), 5678, 0, 126336)
    b = gen.tokens_torch((4, 1000), 5678, 0, 126336).numpy()
    assert np.array_equal(a, b)
    assert a.min() >= 0 and a.max() < 126336
    small = gen.tokens_np((20000,), 5678, 0, 511)
    assert small.min() == 0 and small.max() == 510


def test_weights_backends_agree_with_random_gains():
    cfg = synth.configs.get("tiny_f32", random_gains=True, n_layers=1)
    wn = synth.weights_np(cfg)
    wt = synth.weights_torch(cfg, device="cpu")
    for k in wn:
        assert np.array_equal(wn[k], wt[k].float().numpy()), k
    cfgb = synth.configs.get("tiny_f32", random_gains=True, n_layers=1, dtype="bf16")
    wn = synth.weights_np(cfgb)
    wt = synth.weights_torch(cfgb, device="cpu")
    for k in wn:
        assert np.array_equal(wn[k], wt[k].float().numpy()), k


def test_block_state():
    cfg = synth.configs.get("tiny_f32")
    x = synth.block_state_np(cfg, 2)
    P, Bs = cfg["prompt_len"], cfg["block_size"]
    assert np.array_equal(x[:, :P], synth.prompt_np(cfg))
    assert (x[:, P:P + 2 * Bs] != cfg["mask_id"]).all()
    assert (x[:, P + 2 * Bs:] == cfg["mask_id"]).all()
