"""The seeded input generator: determinism, independence of streams and
threads, distribution moments, and the mask recipe (runs without a GPU)."""
import math

import numpy as np
import pytest

import fagen


def test_same_seed_same_bytes_any_thread_count():
    a = fagen.normal_bf16(123, 0, (3, 70001), 1.0, n_threads=1)
    b = fagen.normal_bf16(123, 0, (3, 70001), 1.0, n_threads=7)
    np.testing.assert_array_equal(a, b)


def test_streams_and_seeds_differ():
    a = fagen.normal_bf16(123, 0, (4096,))
    b = fagen.normal_bf16(123, 1, (4096,))
    c = fagen.normal_bf16(124, 0, (4096,))
    assert (a != b).mean() > 0.9 and (a != c).mean() > 0.9


def test_prefix_property():
    """Element i depends only on (seed, stream, i): a shorter tensor is a prefix."""
    a = fagen.normal_bf16(5, 2, (1000,))
    b = fagen.normal_bf16(5, 2, (1001,))
    np.testing.assert_array_equal(a, b[:1000])


def test_splitmix64_reference_values():
    """The mixing function is SplitMix64's: from state 0 its published output
    sequence starts 0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F.
    word(seed, stream, i) is that function on the Weyl sequence that starts at
    the stream's base."""
    golden = 0x9E3779B97F4A7C15
    mask64 = 2**64 - 1

    def mix(z):
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & mask64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & mask64
        return z ^ (z >> 31)
    assert mix(golden) == 0xE220A8397B1DCDAF
    assert mix((2 * golden) & mask64) == 0x6E789E6AA1B965F4
    assert mix((3 * golden) & mask64) == 0x06C45D188009454F
    base = mix((123 ^ golden) & mask64)
    for i in range(5):
        assert fagen.word(123, 0, i) == mix((base + (i + 1) * golden) & mask64)


@pytest.mark.parametrize("sigma", [1.0, 0.5])
def test_normal_moments(sigma):
    n = 1 << 20
    x = fagen.bf16_bits_to_f32(fagen.normal_bf16(99, 0, (n,), sigma)).astype(np.float64)
    se = sigma / math.sqrt(n)
    assert abs(x.mean()) < 5 * se
    assert abs(x.std() / sigma - 1) < 5 / math.sqrt(2 * n) + 2e-3  # + bf16 rounding
    # fraction beyond 2 sigma of a normal: 0.0455
    frac = (np.abs(x) > 2 * sigma).mean()
    assert abs(frac - 0.0455) < 5 * math.sqrt(0.0455 * 0.9545 / n) + 1e-3


def test_values_are_bf16_rounded_nearest_even():
    import torch
    bits = fagen.normal_bf16(7, 0, (4096,), 1.0)
    x = fagen.bf16_bits_to_f32(bits)
    again = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy()
    np.testing.assert_array_equal(again.view(np.uint16), bits)


def test_mask_recipe():
    B, H, ql, kl = 2, 4, 64, 256
    m, rows = fagen.mask_f32(fagen.SEED_BASE + 2, B, H, ql, kl, 0.1, 4)
    assert m.dtype == np.float32 and m.shape == (B, H, ql, kl)
    assert set(np.unique(m)) <= {0.0, -np.inf}
    full = np.isneginf(m).all(-1)
    assert (full.sum(-1) == 4).all()
    for b in range(B):
        for h in range(H):
            assert len(set(rows[b, h])) == 4
            assert set(np.nonzero(full[b, h])[0]) == set(rows[b, h])
    part = np.isneginf(m[~full])
    p = part.mean()
    assert abs(p - 0.1) < 4 * math.sqrt(0.1 * 0.9 / part.size)


def test_workloads_match_their_recipes():
    w = fagen.WORKLOADS["d64_mask_b2_h4_q64_k256_causal"]
    inp = fagen.generate(w)
    assert inp["q"].shape == (2, 4, 64, 64) and inp["k"].shape == (2, 4, 256, 64)
    assert inp["mask"].shape == (2, 4, 64, 256)
    w5 = fagen.WORKLOADS["d256_gqa_b2_h16kv4_q8192_k8192_causal"]
    assert (w5.B, w5.H, w5.Hkv, w5.ql, w5.kl, w5.D, w5.causal, w5.sigma) == \
        (2, 16, 4, 8192, 8192, 256, True, 0.5)
    assert w5.metric_flop == 4 * 2 * 16 * 8192 * 8192 * 256 // 2
    w4 = fagen.WORKLOADS["d64_b8_h16_q4096_k4096_causal"]
    assert w4.metric_flop == 274877906944


def _lcg_reference(seed, n):
    """The page's LCG written out with Python integers and numpy f32 steps:
    state <- state * 6364136223846793005 + 1442695040888963407 (mod 2^64),
    value = f32(state >> 33) / f32(2^32 - 1) - 0.5 in f32."""
    state, out = seed, []
    for _ in range(n):
        state = (state * 6364136223846793005 + 1442695040888963407) % 2**64
        top = np.float32(state >> 33)  # 31-bit integer, rounded to nearest f32
        out.append(np.float32(top / np.float32(2**32 - 1)) - np.float32(0.5))
    return np.array(out, dtype=np.float32)


def test_page_lcg_matches_its_definition():
    for seed in (fagen.SEED_BASE, fagen.SEED_BASE + 1, fagen.SEED_BASE + 203, 0, 2**64 - 1):
        got = fagen.lcg_f32(seed, (257,))
        np.testing.assert_array_equal(got, _lcg_reference(seed, 257))


def test_page_lcg_range_is_below_zero():
    """The page's comment says [-0.5, 0.5]; the top 31 bits over 2^32 make it
    [-0.5, 0)."""
    x = fagen.lcg_f32(fagen.SEED_BASE + 7, (200000,))
    assert x.min() >= -0.5 and x.max() < 0.0
    assert abs(float(x.mean()) + 0.25) < 0.005


def test_page_lcg_bf16_is_torch_rounding():
    import torch
    x = fagen.lcg_f32(fagen.SEED_BASE + 11, (4096,))
    b = fagen.lcg_bf16(fagen.SEED_BASE + 11, (4096,))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(b, ref)
