"""The CPU oracle against facts fixed outside it (see oracle_pins for what pins what)."""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import oracle_pins as pins
import synth


def test_fp16_codec_matches_ieee_binary16(orc):
    pins.check_fp16(orc)


def test_layout_hand_derived_blocks(orc):
    pins.check_layout_goldens(orc)


def test_layout_q40_q80_hand_derived(orc):
    pins.check_q32_layout_goldens(orc)


def test_layout_q4k_q6k_two_block_tensors(orc):
    pins.check_qk_tensor_goldens(orc)


def test_layout_single_field_probes(orc):
    pins.check_layout_probes(orc)


def test_activation_hand_worked_blocks(orc):
    pins.check_act_cases(orc)


def test_activation_rounding_bound_and_invariants(orc):
    pins.check_act_bounds(orc)


def test_activation_overflowing_inverse(orc):
    pins.check_act_overflowing_inverse(orc)


@pytest.mark.parametrize("sigma", [0.02, 0.002, 1.0])
def test_q4k_quantizer_roundtrip(orc, sigma):
    rng = np.random.default_rng(int(sigma * 1000) + 1)
    w = (rng.standard_normal((16, 1024)) * sigma).astype(np.float32)
    w[3] = np.abs(w[3])                     # all-positive rows: no offset
    w[4] = -np.abs(w[4])                    # all-negative rows
    w[5, :256] = 0.0                        # an all-zero super-block
    w[6, 32:64] = np.float32(-0.01)         # a constant sub-block
    pins.check_q4k_quantizer(orc, w)


@pytest.mark.parametrize("negate", [False, True])
@pytest.mark.parametrize("sigma", [0.02, 0.002, 1.0])
def test_q6k_quantizer_roundtrip(orc, sigma, negate):
    rng = np.random.default_rng(int(sigma * 1000) + 7)
    w = (rng.standard_normal((16, 1024)) * sigma).astype(np.float32)
    w[5, :256] = 0.0
    pins.check_q6k_quantizer(orc, w, negate=negate)


def test_q4k_subnormal_super_scale(orc):
    """sigma 0.002 puts d below fp16's smallest normal (6.1e-5)."""
    w = synth.normal_f32(99, 0, 8 * 512, 0.002).reshape(8, 512)
    buf = pins.check_q4k_quantizer(orc, w)
    d16 = oracle.planes("q4k", buf, 8, 512)[1].reshape(-1, 16)[:, 0:2].copy().view(np.uint16)[:, 0]
    assert np.any(d16 < 0x0400)


@pytest.mark.parametrize("sigma", [0.02, 0.002, 1.0, 1e-6])
def test_q40_quantizer(orc, sigma):
    rng = np.random.default_rng(int(sigma * 1e6) % 1000 + 3)
    w = (rng.standard_normal((12, 1024)) * sigma).astype(np.float32)
    w[2, :32] = 0.0                          # an all-zero block
    w[3, 32:64] = np.float32(sigma)          # a constant block (ties for the maximum)
    w[4, 64:96] = -np.abs(w[4, 64:96])       # one-signed blocks
    w[5, 96:128] = np.abs(w[5, 96:128])
    w[6, 0] = np.float32(8 * sigma)          # a block whose opposite side gets clipped
    w[6, 1:32] = np.float32(-7.9 * sigma)
    pins.check_q40_quantizer(orc, w)


@pytest.mark.parametrize("sigma", [0.02, 1.0, 1e6])
def test_q80_quantizer(orc, sigma):
    rng = np.random.default_rng(int(sigma) % 1000 + 5)
    w = (rng.standard_normal((12, 1024)) * sigma).astype(np.float32)
    w[2, :32] = 0.0
    pins.check_q80_quantizer(orc, w)


def test_q80_quantizer_hand_worked_blocks(orc):
    """The activation fixtures (ties, the scale as one division, x * (127 / amax) against
    x / xd) give the same codes and scales when quantized as Q8_0 weights."""
    for x, q, xd in pins.read_act_cases():
        buf = oracle.quantize_q80(x[None, :], lib=orc)
        codes, scales = oracle.q80_codes(buf, 1, x.size), oracle.q80_scales(buf, 1, x.size)
        assert np.array_equal(codes.reshape(-1), q)
        assert scales.reshape(-1)[0].view(np.uint32) == np.float32(xd).view(np.uint32)


@pytest.mark.parametrize("wtype", ["q4k", "q6k", "q40", "q80"])
def test_gemv_equals_bruteforce_on_random(orc, wtype):
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((24, 768)) * 0.02).astype(np.float32)
    x = rng.standard_normal((3, 768)).astype(np.float32)
    pins.check_gemv_bruteforce(orc, wtype, w, x)


@settings(max_examples=40, deadline=None)
@given(rows=st.integers(1, 8), nb=st.integers(1, 4), nvec=st.integers(1, 3),
       seed=st.integers(0, 2**31 - 1), wtype=st.sampled_from(["q4k", "q6k"]),
       wscale=st.sampled_from([0.02, 0.002, 1.0, 30.0]))
def test_gemv_equals_bruteforce_tiny(orc, rows, nb, nvec, seed, wtype, wscale):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((rows, 256 * nb)) * wscale).astype(np.float32)
    x = (rng.standard_normal((nvec, 256 * nb)) * rng.choice([1e-3, 1.0, 50.0])).astype(np.float32)
    x[:, rng.integers(0, 256 * nb, size=40)] = 0.0
    pins.check_gemv_bruteforce(orc, wtype, w, x)


@settings(max_examples=40, deadline=None)
@given(rows=st.integers(1, 8), nblk=st.integers(1, 12), nvec=st.integers(1, 3),
       seed=st.integers(0, 2**31 - 1), wtype=st.sampled_from(["q40", "q80"]),
       wscale=st.sampled_from([0.02, 0.002, 1.0, 30.0]))
def test_gemv_equals_bruteforce_tiny_q32(orc, rows, nblk, nvec, seed, wtype, wscale):
    """The 32-weight formats on widths that are not multiples of 256."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((rows, 32 * nblk)) * wscale).astype(np.float32)
    x = (rng.standard_normal((nvec, 32 * nblk)) * rng.choice([1e-3, 1.0, 50.0])).astype(np.float32)
    x[:, rng.integers(0, 32 * nblk, size=10)] = 0.0
    pins.check_gemv_bruteforce(orc, wtype, w, x)


@pytest.mark.parametrize("wtype", ["q4k", "q6k", "q40", "q80"])
def test_gemv_one_hot_column_extraction(orc, wtype):
    w = synth.normal_f32(42, 0, 5 * 512, 0.02).reshape(5, 512)
    pins.check_gemv_onehot(orc, wtype, w)


def test_gemv_special_cases(orc):
    pins.check_gemv_special(orc)


def test_gemv_int32_extremes(orc):
    pins.check_gemv_extremes(orc)


@pytest.mark.parametrize("wtype", ["q4k", "q6k", "q40", "q80"])
def test_gemv_many_vectors(orc, wtype):
    """More than 8 vectors (the matrix-core path's range): every y equals the brute-force
    product with the dequantized matrix, and each vector's y, P and S are those of that vector
    alone (vectors never mix)."""
    rng = np.random.default_rng(77)
    nvec, rows, cols = 37, 6, 512
    w = (rng.standard_normal((rows, cols)) * 0.05).astype(np.float32)
    x = (rng.standard_normal((nvec, cols)) * rng.choice([0.01, 1.0, 40.0], size=(nvec, 1))
         ).astype(np.float32)
    x[5] = 0.0
    buf, xq, xd, res = pins.check_gemv_bruteforce(orc, wtype, w, x)
    for v in (0, 5, 17, 36):
        one = oracle.gemv(wtype, buf, rows, cols, xq[v:v + 1], xd[v:v + 1], partials=True, lib=orc)
        assert np.array_equal(one["y"][0], res["y"][v])
        assert np.array_equal(one["P"][0], res["P"][v])
        if wtype == "q4k":
            assert np.array_equal(one["S"][0], res["S"][v])
    assert not res["y"][5].any() and not res["P"][5].any()
