"""The seeded input generator: determinism, slicing, rounding, distribution."""
import numpy as np
import torch

import synth


def test_deterministic_and_sliceable():
    a = synth.normal(7, 2, (1000,), 0.5, synth.F32)
    b = synth.normal(7, 2, (1000,), 0.5, synth.F32)
    np.testing.assert_array_equal(a, b)
    for first in (0, 1, 2, 333, 998):
        part = synth.normal(7, 2, (1000 - first,), 0.5, synth.F32, first=first)
        np.testing.assert_array_equal(part, a[first:])
    other = synth.normal(7, 3, (1000,), 0.5, synth.F32)
    assert not np.array_equal(a, other)


def test_splitmix64_reference_values():
    # SplitMix64 seeded with 0 yields these first outputs (Steele, Lea, Flood 2014;
    # the published test vector of the generator).
    def splitmix64(state, n):
        out = []
        for _ in range(n):
            state = (state + 0x9E3779B97F4A7C15) & 0xFFFFFFFFFFFFFFFF
            z = state
            z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
            z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
            out.append(z ^ (z >> 31))
        return out
    assert splitmix64(0, 3) == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    # the library's stream (seed, tid) is SplitMix64 from state mix64(seed + G (tid + 1))
    G = 0x9E3779B97F4A7C15

    def mix(z):
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & 0xFFFFFFFFFFFFFFFF
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & 0xFFFFFFFFFFFFFFFF
        return z ^ (z >> 31)
    key = mix((11 + G * 4) & 0xFFFFFFFFFFFFFFFF)
    assert [synth.word(11, 3, p) for p in range(4)] == splitmix64(key, 4)


def test_box_muller_pair():
    import math
    w = synth.word(5, 0, 0)
    u1 = ((w >> 32) + 0.5) / 2**32
    u2 = ((w & 0xFFFFFFFF) + 0.5) / 2**32
    rad = math.sqrt(-2 * math.log(u1))
    x = synth.normal(5, 0, (2,), 1.0, synth.F32)
    assert x[0] == np.float32(rad * math.cos(2 * math.pi * u2))
    assert x[1] == np.float32(rad * math.sin(2 * math.pi * u2))


def test_bf16_round_to_nearest_even():
    g = np.random.default_rng(0)
    x = g.standard_normal(20000).astype(np.float32)   # exactly representable doubles
    ours = np.array([synth.bf16_from_double(float(v)) for v in x], dtype=np.uint16)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    # halfway cases in double: ties go to even; just above a tie rounds up
    one = 1.0
    ulp = 2.0 ** -7
    assert synth.bf16_from_double(one + ulp / 2) == 0x3F80           # tie -> even (down)
    assert synth.bf16_from_double(one + 3 * ulp / 2) == 0x3F82       # tie -> even (up)
    assert synth.bf16_from_double(one + ulp / 2 + 2.0 ** -40) == 0x3F81
    assert synth.bf16_from_double(-2.0) == 0xC000
    assert synth.bf16_from_double(0.0) == 0x0000
    assert synth.bf16_from_double(2.0 ** -130) == 0x0008             # subnormal
    assert synth.bf16_from_double(3.5e38) == 0x7F80                  # overflow -> inf


def test_normal_moments_and_bf16_consistency():
    x = synth.normal(1, 2, (200000,), 1.0, synth.F32).astype(np.float64)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    assert abs(np.mean(x ** 4) - 3.0) < 0.1
    b = synth.normal(1, 2, (1000,), 0.25, synth.BF16)
    f = synth.normal(1, 2, (1000,), 0.25, synth.F32)
    # bf16 is the once-rounded value: within half a bf16 ulp of the fp32 one
    bf = synth.bf16_bits_to_f32(b).astype(np.float64)
    assert np.all(np.abs(bf - f) <= np.abs(f) * 2.0 ** -8 + 1e-30)


def test_workload_recipes():
    s3 = synth.decode_spec(3)
    lens = s3.seq_lengths()
    assert lens.shape == (64,) and lens.min() >= 1024 and lens.max() <= 8192
    assert s3.L == lens.max()
    np.testing.assert_array_equal(lens, synth.decode_spec(3).seq_lengths())
    s2 = synth.decode_spec(2)
    assert (s2.B, s2.Hq, s2.Hkv, s2.D, s2.L, s2.dtype) == (1, 16, 8, 128, 32768, synth.BF16)
    s4 = synth.decode_spec(4)
    assert (s4.B, s4.L) == (2048, 2048)
    p = synth.prefill_spec(5)
    assert (p.B, p.Hq, p.Hkv, p.L, p.D) == (8, 16, 8, 4096, 128)
    k = synth.decode_kv_rows(s2, synth.TID_K, 100, 3)
    full = synth.decode_kv_rows(s2, synth.TID_K, 0, 103)
    np.testing.assert_array_equal(k, full[100:])
