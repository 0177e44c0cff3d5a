"""The seeded input generators (shared by the oracle tests, GPU tests and the bench)."""

import numpy as np

import synth


def test_splitmix64_published_first_output():
    # splitmix64 seeded with 0: first output 0xE220A8397B1DCDAF (Vigna's reference code)
    assert int(synth.splitmix64(0, np.array([0], np.uint64))[0]) == 0xE220A8397B1DCDAF


def test_stream_slices_agree():
    full = synth.normal_f32(17, 0, 10_001, 1.0)
    for a, b in [(0, 1), (1, 2), (3, 4097), (5000, 10_001), (9999, 10_001)]:
        assert np.array_equal(synth.normal_f32(17, a, b - a, 1.0), full[a:b])


def test_threaded_draw_equals_serial():
    n = 5 * (1 << 21) + 7
    assert np.array_equal(synth.normal_f32(3, 11, n, 0.5), synth._normal_f32_serial(3, 11, n, 0.5))


def test_normal_moments():
    z = synth.normal_f32(5, 0, 1 << 20, 1.0).astype(np.float64)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1.0) < 5e-3
    assert abs(np.mean(z ** 4) - 3.0) < 0.05


def test_rows_and_outliers_are_deterministic():
    wl = synth.WORKLOADS["q4k_262144x1536"]
    a = wl.weight_rows([5, 6, 100])
    b = wl.weight_block(5, 7)
    assert np.array_equal(a[:2], b)
    hot = wl.outlier_rows()
    assert hot.size == round(0.01 * wl.rows) and np.all(np.diff(hot) > 0)
    r = int(hot[0])
    base = synth.normal_f32(wl.seed_w, r * wl.cols, wl.cols, wl.sigma_w)
    assert np.array_equal(wl.weight_rows([r])[0], base * np.float32(10.0))
