"""The oracle on the decode workloads (rows sampled where the full matrix is large):
integer GEMV against the float64 brute force, and the quantizers' round-trip bounds."""

import numpy as np
import pytest

import oracle
import oracle_pins as pins
import synth


def _rows(wl, n):
    if wl.rows <= n:
        return np.arange(wl.rows)
    rng = np.random.default_rng(wl.seed_w)
    pick = np.concatenate([np.arange(8), wl.rows - 8 + np.arange(8),
                           rng.choice(wl.rows, n - 16, replace=False)])
    if wl.outlier_frac:
        pick = np.concatenate([pick, wl.outlier_rows()[:16]])
    return np.unique(pick)


@pytest.mark.parametrize("name,n", [("q4k_512x512", 512), ("q4k_8192x2048", 48),
                                    ("q6k_2048x8192", 16), ("q4k_262144x1536", 64),
                                    ("q4k_16384x2048_b8", 24), ("q40_262144x1536", 64),
                                    ("q80_262144x1536", 64), ("q4k_4096x16384", 16)])
def test_workload_gemv_vs_bruteforce(orc, name, n):
    wl = synth.WORKLOADS[name]
    rows = _rows(wl, n)
    w = wl.weight_rows(rows)
    x = wl.activations()
    pins.check_gemv_bruteforce(orc, wl.wtype, w, x)
    {"q4k": lambda: pins.check_q4k_quantizer(orc, w[:8]),
     "q6k": lambda: pins.check_q6k_quantizer(orc, w[:4]),
     "q40": lambda: pins.check_q40_quantizer(orc, w[:8]),
     "q80": lambda: pins.check_q80_quantizer(orc, w[:8])}[wl.wtype]()


def test_outlier_rows_have_larger_super_scales(orc):
    wl = synth.WORKLOADS["q4k_262144x1536"]
    hot = wl.outlier_rows()
    assert hot.size == 2621 and np.unique(hot).size == hot.size
    cold = np.setdiff1d(np.arange(64), hot)[:16]
    wh = oracle.quantize_q4k(wl.weight_rows(hot[:16]))
    wc = oracle.quantize_q4k(wl.weight_rows(cold))
    hdr_h = oracle.planes("q4k", wh, 16, wl.cols)[1].reshape(-1, 16)
    hdr_c = oracle.planes("q4k", wc, len(cold), wl.cols)[1].reshape(-1, 16)
    dh = oracle.f16_to_f32(hdr_h[:, :2].copy().view(np.uint16)[:, 0])
    dc = oracle.f16_to_f32(hdr_c[:, :2].copy().view(np.uint16)[:, 0])
    ratio = np.median(dh) / np.median(dc)
    assert 8.0 < ratio < 12.5
