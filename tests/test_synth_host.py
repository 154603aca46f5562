"""The host half of the input generator against an independent pure-Python
rendering of its published definition (SplitMix64, Steele, Lea & Flood 2014)."""
import numpy as np
import pytest

pytestmark = pytest.mark.usefixtures("built_synth")

M64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15


def py_sm64(x):
    z = (x + GOLDEN) & M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & M64
    return z ^ (z >> 31)


def py_key(seed, stream, w, p):
    k = py_sm64(seed)
    k = py_sm64(k ^ stream)
    k = py_sm64(k ^ w)
    return py_sm64(k ^ p)


def py_unit(h):
    return np.float32(np.float32(h >> 40) * np.float32(2.0 ** -23)) - np.float32(1.0)


def py_value(key, dist, scale, i):
    if dist == 0:
        return py_unit(py_sm64((key + i * GOLDEN) & M64))
    h1 = py_sm64((key + 2 * i * GOLDEN) & M64)
    h2 = py_sm64((key + (2 * i + 1) * GOLDEN) & M64)
    a = np.float32(py_unit(h1) + py_unit((h1 << 24) & M64))
    b = np.float32(py_unit(h2) + py_unit((h2 << 24) & M64))
    return np.float32(np.float32(a + b) * np.float32(scale))


def test_splitmix_first_output_from_zero_state():
    import synth
    # first SplitMix64 output for seed 0 (widely published test value)
    assert py_sm64(0) == 0xE220A8397B1DCDAF
    assert synth.host_lib().synth_sm64(0) == 0xE220A8397B1DCDAF


@pytest.mark.parametrize("dist", [0, 1])
def test_host_generator_matches_python_definition(dist):
    import synth
    for (seed, stream, w, p) in [(0, 1, 0, 0), (0, 2, 7, 160), (5, 3, 15, 146), (0, 1, 31, 5999)]:
        k = synth.key(seed, stream, w, p)
        assert k == py_key(seed, stream, w, p)
        scale = synth.scale_for(dist, 1e-3)
        first = 12345
        got = synth.host_f32(k, dist, scale, 64, first=first)
        want = np.array([py_value(k, dist, scale, first + j) for j in range(64)], dtype=np.float32)
        np.testing.assert_array_equal(got.view(np.uint32), want.view(np.uint32))
        idx = np.array([0, 3, 99999, 7], dtype=np.int64)
        np.testing.assert_array_equal(synth.host_gather_f32(k, dist, scale, idx),
                                      np.array([py_value(k, dist, scale, int(i)) for i in idx], np.float32))


def test_distributions():
    import synth
    k = synth.key(0, 1, 0, 0)
    u = synth.host_f32(k, 0, 1.0, 200000)
    assert u.min() >= -1.0 and u.max() < 1.0
    assert abs(u.mean()) < 0.01 and abs(u.var() - 1 / 3) < 0.01
    assert np.all((u.astype(np.float64) + 1) * 2 ** 23 == np.round((u.astype(np.float64) + 1) * 2 ** 23))
    s = synth.scale_for(1, 1e-2)
    z = synth.host_f32(k, 1, s, 200000)
    assert abs(z.std() - 1e-2) < 2e-4 and abs(z.mean()) < 1e-4


def test_bf16_is_round_to_nearest_even():
    import torch
    import synth
    k = synth.key(0, 3, 1, 2)
    s = synth.scale_for(1, 1e-3)
    f = synth.host_f32(k, 1, s, 5000)
    b = synth.host_bf16(k, 1, s, 5000)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(b, ref)
