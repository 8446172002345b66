"""The seeded input generator: deterministic, right distributions, bit-exact
round-to-nearest-even bf16 (against torch's own float32 -> bfloat16 cast)."""
import numpy as np
import torch

import attn_inputs as ai


def _torch_bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def test_rne_matches_torch_random():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(200_000) * 10.0 ** rng.uniform(-40, 38, 200_000)).astype(np.float32)
    assert np.array_equal(ai.f32_to_bf16_bits(x), _torch_bf16_bits(x))


def test_rne_ties_specials_subnormals():
    u = np.array([
        0x3F808000,  # tie, lower even -> stays
        0x3F818000,  # tie, lower odd -> rounds up
        0x3F808001,  # just above tie
        0x3F807FFF,  # just below tie
        0x00000001, 0x00008000, 0x00018000, 0x007FFFFF,  # subnormals incl. ties
        0x80000001, 0x7F7FFFFF, 0xFF7FFFFF,  # largest finite rounds to inf
        0x7F800000, 0xFF800000, 0x00000000, 0x80000000,
    ], dtype=np.uint32)
    x = u.view(np.float32)
    assert np.array_equal(ai.f32_to_bf16_bits(x), _torch_bf16_bits(x))


def _torch_f16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float16) \
        .view(torch.int16).numpy().view(np.uint16)


def test_f16_rne_matches_torch():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200_000) * 10.0 ** rng.uniform(-9, 6, 200_000)).astype(np.float32)
    # plus ties at binary16 precision, subnormals and overflow
    extra = np.array([1 + 2 ** -11, 1 + 3 * 2 ** -11, 2 ** -25, 3 * 2 ** -25, 65520.0, 65519.0,
                      -70000.0, 0.0, -0.0], np.float32)
    x = np.concatenate([x, extra])
    assert np.array_equal(ai.f32_to_f16_bits(x), _torch_f16_bits(x))


def test_f16_inputs_same_draws_as_bf16():
    a = ai.make_qkv(1, 2, 33, 64, 7, sigma_qk=3.0, with_do=True)
    b = ai.make_qkv(1, 2, 33, 64, 7, sigma_qk=3.0, with_do=True, dtype="f16")
    for n in ("q", "k", "v", "do"):
        fa = (a[n].astype(np.uint32) << 16).view(np.float32)
        fb = b[n].view(np.float16).astype(np.float32)
        # both are roundings of the same float32 draw: within half an ulp of bf16
        assert np.all(np.abs(fa - fb) <= np.abs(fb) * 2.0 ** -8 + 1e-30)


def test_rne_nan_stays_nan():
    x = np.array([np.nan, -np.nan], np.float32)
    bits = ai.f32_to_bf16_bits(x)
    back = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.isnan(back).all()


def test_deterministic_and_ordered():
    a = ai.make_qkv(1, 2, 33, 64, seed=7, with_do=True)
    b = ai.make_qkv(1, 2, 33, 64, seed=7, with_do=True)
    for key in ("q", "k", "v", "do"):
        assert a[key].dtype == np.uint16 and a[key].shape == (1, 2, 33, 64)
        assert np.array_equal(a[key], b[key])
    # draw order Q, K, V, dO from one stream
    rng = np.random.default_rng(7)
    for key in ("q", "k", "v", "do"):
        ref = ai.f32_to_bf16_bits(rng.standard_normal((1, 2, 33, 64), dtype=np.float32))
        assert np.array_equal(a[key], ref)


def test_distributions():
    w = ai.WORKLOADS["c5"]
    x = ai.make_qkv(1, 4, 4096, 128, seed=5, sigma_qk=w.sigma_qk, sigma_v=w.sigma_v)
    f = {k: (v.astype(np.uint32) << 16).view(np.float32) for k, v in x.items()}
    assert abs(float(f["q"].std()) - 3.0) < 0.02 and abs(float(f["k"].std()) - 3.0) < 0.02
    assert abs(float(f["v"].std()) - 1.0) < 0.01
    assert abs(float(f["q"].mean())) < 0.01


def test_workloads_table():
    assert [w.label for w in ai.WORKLOADS.values()] == [
        "2x8x512x64", "4x32x1024x128", "8x64x2048x128", "8x64x2048x128", "4x64x4096x128"]
    assert ai.WORKLOADS["c2"].scale == float(np.float32(1 / np.sqrt(128)))
