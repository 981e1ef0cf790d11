"""Pins of the oracle's attention step against closed forms: one token,
identical keys (uniform weights), a dominant key, the rotary embedding at
angle 0 (identity) and at a quarter turn (exact swap with a sign), a
hand-computed rotation with rounding, the bf16 rounding of the keys, and the
unrounded reconstruction of the values (a hand-decoded record, the fp32
decompression within its rounding, the magnitude form)."""
import numpy as np

import oracle


def _bits(x):
    return oracle.f32_to_bf16_bits_array(np.asarray(x, np.float32))


def test_bf16_rounding_array():
    # ties to even, values in between, overflow to infinity, signs
    x = np.array([1.0, 1.00390625, 1.005859375, 1.0078125 + 2 ** -9, -3.0, 3.4e38, 1e-40],
                 np.float32)
    got = oracle.f32_to_bf16_bits_array(x)
    want = [oracle.f32_to_bf16_bits(float(v)) for v in x]
    assert list(got) == want
    assert got[0] == 0x3F80 and got[1] == 0x3F80 and got[2] == 0x3F81 and got[5] == 0x7F80


def test_single_token_returns_its_value():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((2, 3, 8)).astype(np.float32)
    k = _bits(rng.standard_normal((2, 1, 8)))
    v = _bits(rng.standard_normal((2, 1, 8)))
    out = oracle.attention(q, k, oracle.bf16_bits_to_f32(v), 0.35)
    np.testing.assert_array_equal(out, np.broadcast_to(oracle.bf16_bits_to_f32(v), out.shape))


def test_identical_keys_average_the_values():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((1, 2, 16)).astype(np.float32)
    k = np.broadcast_to(_bits(rng.standard_normal(16)), (1, 40, 16)).copy()
    v = _bits(rng.standard_normal((1, 40, 16)))
    out = oracle.attention(q, k, oracle.bf16_bits_to_f32(v), 0.25)
    mean = oracle.bf16_bits_to_f32(v[0]).astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(out[0], np.broadcast_to(mean, (2, 16)), rtol=0, atol=1e-14)


def test_dominant_key_takes_the_weight():
    # scores 0 and -gap: the weights are 1/(1+e^-gap) and e^-gap/(1+e^-gap)
    d, gap = 4, 30.0
    q = np.zeros((1, 1, d), np.float32)
    q[0, 0, 0] = 1.0
    k = _bits([[[1.0, 0, 0, 0], [0.0, 0, 0, 0]]])
    v = _bits([[[2.0, 0, 0, 0], [0.0, 4.0, 0, 0]]])
    out = oracle.attention(q, k, oracle.bf16_bits_to_f32(v), gap)
    e = np.exp(-gap)
    np.testing.assert_allclose(out[0, 0], [2.0 / (1 + e), 4.0 * e / (1 + e), 0, 0], rtol=1e-14)


def test_rope_identity_and_quarter_turn():
    rng = np.random.default_rng(3)
    kb = _bits(rng.standard_normal((5, 8)) * 3)
    one, zero = np.ones((5, 4), np.float32), np.zeros((5, 4), np.float32)
    assert np.array_equal(oracle.rope_bf16(kb, one, zero), kb)
    rot = oracle.rope_bf16(kb, zero, one)  # (a, b) -> (-b, a), exact
    assert np.array_equal(rot[:, :4], kb[:, 4:] ^ np.uint16(0x8000))
    assert np.array_equal(rot[:, 4:], kb[:, :4])


def test_rope_rounds_products_and_sum_in_fp32_then_bf16():
    # a = 1 + 2^-7, b = 1; c = s = 0.7071067690849304 (fp32 of 1/sqrt 2)
    a, b = 1.0 + 2.0 ** -7, 1.0
    c = s = np.float32(0.7071067690849304)
    kb = _bits([[a, b]])
    out = oracle.rope_bf16(kb, np.array([[c]], np.float32), np.array([[s]], np.float32))
    lo = np.float32(np.float32(np.float32(a) * c) - np.float32(np.float32(b) * s))
    hi = np.float32(np.float32(np.float32(b) * c) + np.float32(np.float32(a) * s))
    assert out[0, 0] == oracle.f32_to_bf16_bits(float(lo))
    assert out[0, 1] == oracle.f32_to_bf16_bits(float(hi))
    # by hand: a*c and b*s are each within 2^-25 of exact and within a factor 2
    # of each other, so the difference is exact (Sterbenz): |lo - 2^-7 c| <= 2^-24
    assert abs(float(lo) - 2.0 ** -7 * 0.7071067690849304) <= 2.0 ** -24


def test_reconstruct_exact_hand_record():
    # one token, d=8, INT2, one group: code bytes 0b11100100, 0b00011011 unpack
    # (2 bits per element, low bits first) to q = 0,1,2,3, 3,2,1,0, i.e.
    # levels -3,-1,1,3, 3,1,-1,-3; scale byte 0x38 is 1.0 and 0x40 is 2.0
    codes = np.array([[[0b11100100, 0b00011011]]], np.uint8)
    c1 = np.arange(8, dtype=np.float32) * 0.25          # stage 1, row 1
    c2 = np.full(8, 2.0 ** -30, np.float32)             # stage 2, row 0
    cent = np.zeros((1, 2, 2, 8), np.float32)
    cent[0, 0, 1] = c1
    cent[0, 1, 0] = c2
    assign = np.array([[[1], [0]]], np.uint8)
    levels = np.array([-3, -1, 1, 3, 3, 1, -1, -3], np.float64)
    for sbyte, sval in ((0x38, 1.0), (0x40, 2.0)):
        got = oracle.reconstruct_exact(codes, np.array([[[sbyte]]], np.uint8), assign, cent, 2, 8)
        want = levels * sval + c1.astype(np.float64) + 2.0 ** -30
        assert np.array_equal(got[0, 0], want)
        mag = oracle.reconstruct_exact(codes, np.array([[[sbyte]]], np.uint8), assign, cent, 2, 8,
                                       magnitude=True)
        assert np.array_equal(mag[0, 0], np.abs(levels) * sval + np.abs(c1) + 2.0 ** -30)
    # the fp32 decompression drops the 2^-30 term where it is below half an ulp
    dq = oracle.decompress(codes, np.array([[[0x38]]], np.uint8), assign, cent, 2, 8)
    assert dq[0, 0, 0] == np.float32(-3.0) and got[0, 0, 0] != -3.0 * 2.0


def test_reconstruct_exact_against_fp32_decompress():
    # random records: the fp32 decompression (fma for the last stage, then T-1
    # fp32 adds) is within (T+1) * 2^-24 of the magnitude of the exact sum;
    # with no stages it is exact (level times scale is representable)
    from means_residual_compression_amd import synth
    for T, bits, G in ((0, 2, 64), (1, 4, 32), (3, 2, 16), (4, 2, 64)):
        codes, scales, assign, cent = synth.random_record(7 + T, 2, 300, 64, T, 32, bits, G,
                                                          Hg=10, Wg=10)
        cb = cent.view(__import__("torch").int16).numpy().view(np.uint16) if T else \
            np.zeros((2, 0, 32, 64), np.float32)
        ex = oracle.reconstruct_exact(codes, scales, assign, cb, bits, G)
        mag = oracle.reconstruct_exact(codes, scales, assign, cb, bits, G, magnitude=True)
        dq = oracle.decompress(codes, scales, assign, cb, bits, G, out_bf16=False)
        err = np.abs(dq.astype(np.float64) - ex)
        if T == 0:
            assert np.array_equal(dq.astype(np.float64), ex)
        else:
            assert np.all(err <= (T + 1) * 2.0 ** -24 * mag)
