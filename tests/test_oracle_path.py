"""Pins for the oracle's whole compress/decompress path (PRQ + Q + DQ).

paper.rainbus.top, method paragraph: R(0) = X; stage t runs SAS on R(t-1);
only R(T) is quantized; reconstruction adds C(t)[pi(t)] from stage T down to 1.
note.zhuruihan.top, "Progressive Residual Quantization": reconstruction adds
centroids back from the last stage to the first.

Pinned by special cases with a known exact answer: C = N (every token its own
centroid -> zero residual -> exact reconstruction), T = 0 (plain group
quantization), and a record whose fp32 result depends on the add order.
"""
import numpy as np
import pytest
import torch

from means_residual_compression_amd import synth


def _bf16_bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 2])
def test_C_equals_N_reconstructs_exactly(oracle, dtype, T):
    N, d = 96, 64
    X = synth.video_cache(0, 0, 2, 6, 4, 4, d, 50.0, torch.float32)
    if dtype == "bf16":
        Xs = _bf16_bits(X.to(torch.bfloat16))
    else:
        Xs = X.numpy()
    idx = np.stack([np.stack([np.random.default_rng(h * 10 + t).permutation(N)
                              for t in range(T)]) for h in range(2)]).astype(np.int32)
    rec = oracle.compress(Xs, C=N, T=T, iters=2, bits=2, G=32, init_idx=idx)
    assert np.all(rec["scales"] == 0)
    out = oracle.decompress(rec["codes"], rec["scales"], rec["assign"], rec["cent"], 2, 32)
    np.testing.assert_array_equal(out, Xs)


@pytest.mark.parametrize("bits", [2, 4])
def test_T0_is_plain_group_quantization(oracle, bits):
    X = synth.video_cache(0, 0, 1, 4, 8, 8, 64, 50.0, torch.float32).numpy()
    rec = oracle.compress(X, C=4, T=0, iters=1, bits=bits, G=32)
    codes, scales = oracle.quantize(X[0], bits, 32)
    np.testing.assert_array_equal(rec["codes"][0], codes)
    np.testing.assert_array_equal(rec["scales"][0], scales)


def test_reconstruction_adds_stage_T_first(oracle):
    """s_hat = 0 and one token, fp32 centroids C3 = 1, C2 = 1e8, C1 = -1e8.
    Stage T down to 1: ((0 + 1) + 1e8) - 1e8 = 1e8 - 1e8 = 0 in fp32 (1e8 + 1
    rounds to 1e8).  Stage 1 up to T would give ((0 - 1e8) + 1e8) + 1 = 1."""
    d = 8
    codes = np.full((1, 1, d * 2 // 8), 0xAA, np.uint8)  # middle code 2 everywhere
    scales = np.zeros((1, 1, 1), np.uint8)
    assign = np.zeros((1, 3, 1), np.uint8)
    cent = np.zeros((1, 3, 1, d), np.float32)
    cent[0, 0], cent[0, 1], cent[0, 2] = -1e8, 1e8, 1.0
    out = oracle.decompress(codes, scales, assign, cent, 2, 8)
    assert np.all(out == 0.0)


def test_decompress_inverts_compress_within_quant_bound(oracle):
    X = synth.video_cache(0, 0, 1, 8, 8, 8, 64, 50.0, torch.float32).numpy()
    N = X.shape[1]
    idx = synth.init_indices(1, 1, 2, N, 16)
    rec = oracle.compress(X, C=16, T=2, iters=5, bits=2, G=32, init_idx=idx)
    out = oracle.decompress(rec["codes"], rec["scales"], rec["assign"], rec["cent"], 2, 32)
    # reconstruct the final residual independently from the record
    R = X[0].astype(np.float32).copy()
    for t in range(2):
        R = R - rec["cent"][0, t][rec["assign"][0, t]]
    sh = np.vectorize(oracle.e4m3_decode)(rec["scales"][0]).repeat(32, axis=1)
    a = np.abs(R).reshape(N, 2, 32).max(2).repeat(32, axis=1)
    bound = np.maximum(sh, a - 3 * sh) + 4 * np.finfo(np.float32).eps * (np.abs(X[0]) + 1)
    assert np.all(np.abs(out[0].astype(np.float64) - X[0]) <= bound)


def test_cache_holds_fp32_centroids_and_record_rounds_them(oracle):
    X = synth.video_cache(0, 1, 1, 4, 8, 8, 64, 50.0, torch.float32)
    Xb = _bf16_bits(X.to(torch.bfloat16))
    idx = synth.init_indices(2, 1, 2, X.shape[1], 8)
    rec = oracle.compress(Xb, C=8, T=2, iters=3, bits=2, G=32, init_idx=idx)
    ref = _bf16_bits(torch.from_numpy(rec["cache"]).to(torch.bfloat16))
    np.testing.assert_array_equal(rec["cent"], ref)


def test_warm_start_equals_caller_init(oracle):
    """Streaming centroid caching (note.zhuruihan.top, Algorithm-System
    Co-design): the next chunk starts k-means from the previous chunk's
    centroids; that is a caller-supplied init equal to the cache."""
    c = dict(Hg=8, Wg=8, d=64, outlier_scale=50.0, dtype=torch.float32)
    ch0 = synth.stream_chunk(0, 0, 1, 0, 2, **c).numpy()
    ch1 = synth.stream_chunk(0, 0, 1, 1, 2, **c).numpy()
    idx = synth.init_indices(3, 1, 2, ch0.shape[1], 8)
    r0 = oracle.compress(ch0, C=8, T=2, iters=4, bits=2, G=32, init_idx=idx)
    r1 = oracle.compress(ch1, C=8, T=2, iters=1, bits=2, G=32, init_c=r0["cache"])
    # one warm iteration: stage-1 assignment is the nearest cached centroid
    pi = oracle.assign(ch1[0], r0["cache"][0, 0])
    np.testing.assert_array_equal(r1["assign"][0, 0], pi)


def test_stage_one_beats_naive_quantization(oracle):
    """First-stage MSE reduction over naive quantization (note.zhuruihan.top,
    PRQ section) -- qualitative on synthetic video-shaped data."""
    X = synth.video_cache(0, 0, 1, 8, 8, 8, 64, 50.0, torch.float32).numpy()
    N = X.shape[1]
    mse = []
    for T in (0, 1, 2):
        idx = synth.init_indices(4, 1, T, N, 16)
        rec = oracle.compress(X, C=16, T=T, iters=6, bits=2, G=32,
                              init_idx=idx if T else None)
        out = oracle.decompress(rec["codes"], rec["scales"], rec["assign"], rec["cent"], 2, 32)
        mse.append(float(((out.astype(np.float64) - X) ** 2).mean()))
    assert mse[1] < mse[0] / 2
    assert mse[2] < mse[1]
