"""Pins for the oracle's number formats: FP8 E4M3 scale codec and bf16 rounding.

The pages fix the scale format as FP8 E4M3 (note.zhuruihan.top, Algorithm-System
Co-design).  The oracle encodes by nearest-value search over the finite E4M3
values; here that is checked against PyTorch's independent float8_e4m3fn cast
(a library routine) wherever that cast is finite, and the saturating reading
above 464 is checked on its own.
"""
import numpy as np
import pytest
import torch


def _torch_e4m3(vals):
    t = torch.tensor(np.asarray(vals, np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_all_codes(oracle):
    codes = [c for c in range(256) if (c & 0x7F) != 0x7F]  # 0x7F/0xFF are NaN
    ref = torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    ours = np.array([oracle.e4m3_decode(c) for c in codes], np.float32)
    np.testing.assert_array_equal(ours, ref)


def _probe_values():
    pos = np.array([oracle_value(c) for c in range(127)], np.float64)
    mids = (pos[:-1] + pos[1:]) / 2  # exact ties between neighbours
    vals = [pos, mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
            np.nextafter(mids.astype(np.float32), np.float32(1e9))]
    rng = np.random.default_rng(5)
    vals.append(np.exp(rng.uniform(np.log(1e-6), np.log(460.0), 20000)))
    vals.append(rng.uniform(0, 2 ** -6, 5000))  # subnormal region
    vals.append([0.0, 2 ** -10, 3 * 2 ** -10, 448.0, 460.0, 463.99, 464.0])
    v = np.concatenate([np.asarray(a, np.float64).ravel() for a in vals]).astype(np.float32)
    return v[(v >= 0) & (v <= 464)]


def oracle_value(code):
    e, m = (code >> 3) & 15, code & 7
    return m * 2.0 ** -9 if e == 0 else (8 + m) * 2.0 ** (e - 10)


def test_e4m3_encode_matches_torch_below_464(oracle):
    v = _probe_values()
    ours = np.array([oracle.e4m3_encode(x) for x in v], np.uint8)
    np.testing.assert_array_equal(ours, _torch_e4m3(v))


def test_e4m3_encode_saturates(oracle):
    # Reading: saturate to the largest finite value (448, code 0x7E) instead of NaN.
    for s in [464.001, 479.0, 480.0, 1e4, 3e38]:
        assert oracle.e4m3_encode(s) == 0x7E
    assert oracle.e4m3_decode(0x7E) == 448.0


def test_e4m3_roundtrip_exact_values(oracle):
    for c in range(127):
        assert oracle.e4m3_encode(oracle.e4m3_decode(c)) == c


def test_bf16_rounding_matches_torch(oracle):
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 10.0 ** rng.integers(-20, 20, 20000),
        # exact ties: a bf16 value plus half its last-place unit
        (torch.tensor(rng.standard_normal(2000), dtype=torch.float32)
         .to(torch.bfloat16).float().numpy()).astype(np.float32),
    ]).astype(np.float32)
    bits = x.view(np.uint32)
    ties = ((bits[-2000:] & 0xFFFF0000) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = np.array([oracle.f32_to_bf16_bits(v) for v in x], np.uint16)
    np.testing.assert_array_equal(ours, ref)


def test_bf16_rounding_at_the_top_and_bottom(oracle):
    """IEEE 754 round-to-nearest: values from the midpoint between the largest
    bf16 (0x7F7F) and 2^128 upward overflow to infinity, values below it stay
    finite; fp32 subnormals round like any other value."""
    cases = {0x7F7F7FFF: 0x7F7F, 0x7F7F8000: 0x7F80, 0x7F7FFFFF: 0x7F80, 0xFF7F8000: 0xFF80,
             0xFF7F7FFF: 0xFF7F, 0x7F7F0000: 0x7F7F, 0x00008000: 0x0000, 0x00018000: 0x0002,
             0x80008001: 0x8001, 0x007FFFFF: 0x0080, 0x00000001: 0x0000, 0x80000000: 0x8000}
    for u, want in cases.items():
        v = np.array([u], np.uint32).view(np.float32)[0]
        assert oracle.f32_to_bf16_bits(v) == want, hex(u)
    # and a sweep of the last two bf16 binades and the subnormal range against torch
    rng = np.random.default_rng(3)
    u = np.concatenate([rng.integers(0x7E000000, 0x7F800000, 4000), rng.integers(0, 0x00800000, 4000)])
    u = (u.astype(np.uint32) | (rng.integers(0, 2, u.size).astype(np.uint32) << 31))
    x = u.view(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = np.array([oracle.f32_to_bf16_bits(v) for v in x], np.uint16)
    np.testing.assert_array_equal(ours, ref)
