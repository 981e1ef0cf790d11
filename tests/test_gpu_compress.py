"""End-to-end GPU parity of qvg_compress / qvg_decompress / qvg_compress_stream
against the CPU oracle on the same seeded inputs (bit-exact records and
reconstructions), including the workload's tiny fp32 configuration in full,
the Self-Forcing-shaped bf16 cache at full size (and at the QVG-Pro operating
point on a sample of its head-tensors), multi-stage and INT4 runs,
ragged token counts, the C = N and T = 0 special cases, caller-supplied and
streamed (warm-started) initialisation, and run-to-run determinism."""
import numpy as np
import pytest
import torch

import oracle
from means_residual_compression_amd import qvg, synth
from gpu_util import DEV, bits16, mismatch_report, rec_equal, say, to_oracle

pytestmark = pytest.mark.gpu


def _run_both(x, p, idx=None, init_c=None, threads=None):
    """GPU compress+decompress and oracle compress+decompress of the same input."""
    xd = x.to(DEV)
    cache = torch.zeros((x.shape[0], p.T, p.C, x.shape[2]), dtype=torch.float32, device=DEV)
    rec = qvg.compress(xd, p, init_idx=idx,
                       init_centroids=None if init_c is None else torch.from_numpy(init_c).to(DEV),
                       cache_out=cache)
    out = qvg.decompress(rec, p)
    torch.cuda.synchronize()
    ref = oracle.compress(to_oracle(x), C=p.C, T=p.T, iters=p.iters, bits=p.bits, G=p.group,
                          init_idx=idx, init_c=init_c, threads=threads)
    ref_out = oracle.decompress(ref["codes"], ref["scales"], ref["assign"], ref["cent"], p.bits,
                                p.group)
    return rec, out, cache, ref, ref_out


def _check(rec, out, cache, ref, ref_out):
    bad = rec_equal(rec, ref)
    assert not bad, f"record fields differ from the oracle: {bad}"
    if ref["cache"].size:
        assert np.array_equal(cache.cpu().numpy(), ref["cache"])
    got = bits16(out) if out.dtype == torch.bfloat16 else out.cpu().numpy()
    assert np.array_equal(got, ref_out), mismatch_report(got, ref_out)


def test_tiny_fp32_config_full():
    """16 frames x 16x16 grid, d=64, fp32, C=16, 10 iterations, T=1, INT2 G=32."""
    c = synth.CONFIGS["tiny"]
    x = synth.config_cache("tiny")
    p = qvg.params(C=c["C"], T=c["T"], iters=c["iters"], bits=c["bits"], group=c["group"])
    idx = synth.init_indices(100, x.shape[0], p.T, x.shape[1], p.C)
    say("tiny fp32 config", tuple(x.shape))
    _check(*_run_both(x, p, idx))


@pytest.mark.parametrize("T,bits,G,C,N", [(2, 2, 64, 64, 1500), (3, 4, 64, 50, 1203),
                                          (4, 2, 16, 256, 2101), (1, 4, 128, 256, 4681)])
def test_multistage_bf16(T, bits, G, C, N):
    x = synth.video_cache(1, 0, 1, 4, 30, 52, 128, 1e2, torch.bfloat16, n_tokens=N)
    x = torch.cat([x, synth.video_cache(1, 1, 1, 4, 30, 52, 128, 1e3, torch.bfloat16,
                                        n_tokens=N)])
    p = qvg.params(C=C, T=T, iters=3, bits=bits, group=G)
    idx = synth.init_indices(200 + T, x.shape[0], T, N, C)
    say("multistage", T, bits, G, C, N)
    _check(*_run_both(x, p, idx))


@pytest.mark.parametrize("N", [1, 7, 31, 33, 65])
@pytest.mark.parametrize("d,dtype", [(64, torch.float32), (128, torch.bfloat16)])
def test_tiny_token_counts(N, d, dtype):
    """A single token, a partial 32-token tile, and just past one tile: every
    tile, chunk and range boundary of the kernels is ragged."""
    rng = np.random.default_rng(N * 7 + d)
    x = synth.round_to(rng.standard_normal((2, N, d)) * np.exp(rng.uniform(-3, 3, (2, N, 1))), dtype)
    C = min(N, 5)
    p = qvg.params(C=C, T=2, iters=3, bits=2, group=32)
    idx = synth.init_indices(700 + N, 2, p.T, N, C)
    say("tiny token counts", N, d, dtype)
    _check(*_run_both(x, p, idx))


def test_T0_plain_quantization():
    x = synth.video_cache(1, 1, 2, 2, 30, 52, 128, 1e3, torch.bfloat16)
    p = qvg.params(C=1, T=0, iters=1, bits=2, group=64)
    say("T=0")
    _check(*_run_both(x, p))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_C_equals_N_is_lossless(dtype):
    N = 200
    x = synth.video_cache(0, 0, 2, 1, 10, 20, 64, 50.0, dtype)
    idx = np.stack([np.stack([np.random.default_rng(h * 7 + t).permutation(N) for t in range(2)])
                    for h in range(2)]).astype(np.int32)
    p = qvg.params(C=N, T=2, iters=2, bits=2, group=32)
    say("C=N", dtype)
    rec, out, cache, ref, ref_out = _run_both(x, p, idx)
    _check(rec, out, cache, ref, ref_out)
    assert torch.equal(out.cpu(), x)
    assert int(rec.scales.max()) == 0


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_exact_ties_at_later_stages(dtype):
    """Stage 1 starts from every token's own row (C = N), so its residual is
    exactly zero; every later stage starts from centroids +a*e and -a*e (an
    exact tie for every token) plus distant rows.  Each token of stages 2..4
    then needs the exact sequential distances of its two tied candidates on a
    residual rebuilt from 1..3 earlier stages, and the tie goes to the smaller
    index."""
    N, T = 200, 4
    x = synth.video_cache(0, 1, 2, 1, 10, 20, 64, 50.0, dtype)
    H, d = x.shape[0], x.shape[2]
    rng = np.random.default_rng(17)
    init_c = np.zeros((H, T, N, d), np.float32)
    init_c[:, 0] = x.float().numpy()
    e = np.zeros(d, np.float32)
    e[3] = 1.5
    for t in range(1, T):
        init_c[:, t] = (rng.standard_normal((H, N, d)) * 40 + 100).astype(np.float32)
        init_c[:, t, 0] = e
        init_c[:, t, 1] = -e
    p = qvg.params(C=N, T=T, iters=2, bits=2, group=32)
    say("exact ties at later stages", dtype)
    rec, out, cache, ref, ref_out = _run_both(x, p, init_c=init_c)
    _check(rec, out, cache, ref, ref_out)
    assert int(rec.assign[:, 1].max()) == 0  # every token took the smaller tied index


def test_duplicate_init_indices_and_caller_init():
    x = synth.video_cache(1, 0, 2, 3, 30, 52, 128, 1e2, torch.bfloat16)
    N = x.shape[1]
    idx = synth.init_indices(300, 2, 2, N, 32)
    idx[:, :, 5] = idx[:, :, 4]  # duplicate rows: one of the two clusters stays empty
    p = qvg.params(C=32, T=2, iters=4, bits=2, group=64)
    say("duplicate init rows")
    _check(*_run_both(x, p, idx))
    init_c = np.random.default_rng(3).standard_normal((2, 2, 32, 128)).astype(np.float32) * 50
    say("caller-supplied init centroids")
    _check(*_run_both(x, p, init_c=init_c))


def test_streaming_warm_start_chain():
    """Chunks of 3 frames: chunk 0 cold, chunks 1-3 warm-started from the
    previous chunk's cached centroids, checked against the oracle run with the
    oracle's own cache as its initialisation."""
    c = dict(Hg=30, Wg=52, d=128, outlier_scale=1e2, dtype=torch.bfloat16)
    p = qvg.params(C=64, T=2, iters=4, bits=2, group=64)
    H = 2
    cache = torch.zeros((H, p.T, p.C, 128), dtype=torch.float32, device=DEV)
    ref_cache = None
    for k in range(4):
        ch = synth.stream_chunk(2, 0, H, k, 3, **c)
        N = ch.shape[1]
        warm = k > 0
        idx = None if warm else synth.init_indices(400, H, p.T, N, p.C)
        say("stream chunk", k, "warm" if warm else "cold")
        rec = qvg.compress_stream(ch.to(DEV), p, 2, cache, warm, init_idx=idx)
        out = qvg.decompress(rec, p)
        torch.cuda.synchronize()
        ref = oracle.compress(to_oracle(ch), C=p.C, T=p.T, iters=2 if warm else p.iters,
                              bits=p.bits, G=p.group, init_idx=idx, init_c=ref_cache)
        ref_cache = ref["cache"]
        ref_out = oracle.decompress(ref["codes"], ref["scales"], ref["assign"], ref["cent"],
                                    p.bits, p.group)
        _check(rec, out, cache, ref, ref_out)


def test_deterministic_rerun():
    x = synth.video_cache(1, 1, 3, 3, 30, 52, 128, 1e3, torch.bfloat16).to(DEV)
    p = qvg.params(C=128, T=2, iters=3, bits=2, group=64)
    idx = synth.init_indices(500, 3, 2, x.shape[1], 128)
    say("determinism")
    a = qvg.compress(x, p, init_idx=idx)
    b = qvg.compress(x, p, init_idx=idx)
    torch.cuda.synchronize()
    for f in ("codes", "scales", "assign", "centroids"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f


def test_self_forcing_cache_full_size():
    """21 frames x 30x52 = 32760 tokens, d=128, bf16, C=256, 8 iterations,
    T=2, INT2 G=64: all 12 K and 12 V head-tensors, record and reconstruction
    bit-exact against the oracle."""
    cfg = synth.CONFIGS["self_forcing"]
    x = synth.config_cache("self_forcing")
    p = qvg.params(C=cfg["C"], T=cfg["T"], iters=cfg["iters"], bits=cfg["bits"],
                   group=cfg["group"])
    idx = synth.init_indices(1, x.shape[0], p.T, x.shape[1], p.C)
    say("self-forcing full size", tuple(x.shape))
    _check(*_run_both(x, p, idx))


def test_pro_preset_self_forcing_full_size():
    """The QVG-Pro operating point (T=4, INT2, G=16, C=256, 8 iterations) on
    3 K and 3 V head-tensors of the self-forcing-shaped cache at full length
    (32760 tokens), one call per tensor kind: records, cache and
    reconstructions bit-exact against the oracle."""
    cfg = synth.CONFIGS["self_forcing"]
    nk = cfg["heads"]
    x = synth.config_cache("self_forcing")
    p = qvg.preset("pro", iters=cfg["iters"])
    for kind, rows in (("K", [0, 5, 11]), ("V", [nk, nk + 6, nk + 11])):
        xk = x[rows].contiguous()
        idx = synth.init_indices(60 + rows[0], len(rows), p.T, xk.shape[1], p.C)
        say("QVG-Pro preset full length", kind, tuple(xk.shape))
        _check(*_run_both(xk, p, idx))


def test_centroid_sums_that_can_round():
    """bf16 data whose channels mix magnitudes ~2^15 with values ~2^-40 (more
    than 45 binades apart): chunked fp64 partial sums could round, so the
    update proves nothing and re-sums those clusters in token order; the
    record must still equal the oracle's (fp64 token-order sums)."""
    rng = np.random.default_rng(9)
    H, N, d, C = 2, 3000, 128, 8
    x = rng.standard_normal((H, N, d))
    x[:, :, :16] *= 2.0 ** 15
    tiny = rng.random((H, N, d)) < 0.3
    x[tiny] = rng.standard_normal(int(tiny.sum())) * 2.0 ** -40
    x = synth.round_to(x, torch.bfloat16)
    p = qvg.params(C=C, T=2, iters=3, bits=2, group=64)
    idx = synth.init_indices(900, H, p.T, N, p.C)
    say("centroid sums that can round", tuple(x.shape))
    _check(*_run_both(x, p, idx))


def test_incremental_and_full_updates_in_one_call():
    """Heads 0 and 2 hold plain bf16 video data (every centroid sum exact, so
    from the second iteration on their sums move only the tokens whose
    assignment changed); head 1 mixes ~2^15 with ~2^-40 values (full update
    every iteration).  Six iterations, two stages, ragged N: the record and
    the cache must equal the oracle's."""
    rng = np.random.default_rng(17)
    H, N, d, C = 3, 2777, 128, 32
    x = synth.video_cache(5, 0, H, 2, 30, 52, 128, 1e2, torch.float64, n_tokens=N).numpy()
    x[1, :, :16] *= 2.0 ** 15
    tiny = rng.random((N, d)) < 0.3
    x[1][tiny] = rng.standard_normal(int(tiny.sum())) * 2.0 ** -40
    x = synth.round_to(x, torch.bfloat16)
    p = qvg.params(C=C, T=2, iters=6, bits=2, group=64)
    idx = synth.init_indices(901, H, p.T, N, p.C)
    say("incremental and full updates", tuple(x.shape))
    _check(*_run_both(x, p, idx))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_incremental_updates_of_deep_stages(dtype):
    """Eight stages of four iterations: stages 5..8 (four or more earlier
    stages) take the incremental update as a launch of its own, stages 2..4
    inside the chunk-sum launch; both must give the oracle's record."""
    H, N, C = 2, 3001, 16
    x = synth.video_cache(6, 1, H, 2, 30, 52, 128, 1e2, dtype, n_tokens=N)
    p = qvg.params(C=C, T=8, iters=4, bits=2, group=64)
    idx = synth.init_indices(902, H, p.T, N, p.C)
    say("incremental updates of deep stages", tuple(x.shape), dtype)
    _check(*_run_both(x, p, idx))


def test_incremental_updates_with_per_cluster_exactness():
    """fp32 values in [1, 2): every channel spans 23 bits, so a sum over all N
    tokens could round (23 + ceil(log2 N) > 29) and the head-wide proof fails;
    the integer sums still fit (23 + 24 + 10 <= 62), and iterations whose
    largest cluster has at most 64 members (23 + 6 <= 29) are updated from the
    moved tokens, the others in full.  The record must equal the oracle's."""
    rng = np.random.default_rng(23)
    H, N, d, C = 2, 1000, 64, 32
    x = torch.from_numpy(rng.uniform(1.0, 2.0, (H, N, d)).astype(np.float32))
    p = qvg.params(C=C, T=2, iters=6, bits=2, group=32)
    idx = synth.init_indices(903, H, p.T, N, p.C)
    say("incremental updates with per-cluster exactness", tuple(x.shape))
    _check(*_run_both(x, p, idx))


@pytest.mark.parametrize("H,N,C,T,seed", [(1, 40, 40, 1, 3), (2, 300, 16, 2, 11),
                                          (3, 4681, 256, 2, 2 ** 63 + 5), (1, 32760, 256, 1, 1)])
def test_seeded_start_matches_oracle(H, N, C, T, seed):
    """Neither init_idx nor init_centroids: both sides draw the stage-start
    rows from p.seed with their own splitmix64 + partial Fisher-Yates."""
    x = synth.video_cache(3, 0, H, -(-N // (30 * 52)), 30, 52, 128, 1e2, torch.bfloat16,
                          n_tokens=N)
    p = qvg.params(C=C, T=T, iters=2, bits=2, group=64, seed=seed)
    say("seeded start", H, N, C, T, seed)
    rec = qvg.compress(x.to(DEV), p)
    out = qvg.decompress(rec, p)
    torch.cuda.synchronize()
    ref = oracle.compress(to_oracle(x), C=C, T=T, iters=2, bits=2, G=64, seed=seed)
    ref_out = oracle.decompress(ref["codes"], ref["scales"], ref["assign"], ref["cent"], 2, 64)
    _check(rec, out, torch.from_numpy(ref["cache"]), ref, ref_out)


def test_device_rows_equal_host_rows():
    """init_idx in device memory is read by the kernels and gives the record
    the host copy of the same rows gives (and the oracle's)."""
    x = synth.video_cache(4, 1, 2, 2, 30, 52, 128, 1e3, torch.bfloat16, n_tokens=3001)
    p = qvg.params(C=64, T=2, iters=3, bits=2, group=64)
    idx = synth.init_indices(41, 2, p.T, x.shape[1], p.C)
    say("device rows")
    a = qvg.compress(x.to(DEV), p, init_idx=idx)
    b = qvg.compress(x.to(DEV), p, init_idx=torch.from_numpy(idx).to(DEV))
    torch.cuda.synchronize()
    for f in ("codes", "scales", "assign", "centroids"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f
    ref = oracle.compress(to_oracle(x), C=p.C, T=p.T, iters=p.iters, bits=2, G=64, init_idx=idx)
    assert not rec_equal(b, ref)


def test_cold_stream_chunk_draws_from_seed():
    """A cold streamed chunk without init_idx starts from the seeded rows and
    fills the centroid cache like the oracle."""
    x = synth.video_cache(5, 0, 2, 3, 30, 52, 128, 1e2, torch.bfloat16)
    p = qvg.params(C=32, T=2, iters=3, bits=2, group=64, seed=99)
    cache = torch.zeros((2, p.T, p.C, 128), dtype=torch.float32, device=DEV)
    say("cold stream chunk, seeded")
    rec = qvg.compress_stream(x.to(DEV), p, 2, cache, False)
    out = qvg.decompress(rec, p)
    torch.cuda.synchronize()
    ref = oracle.compress(to_oracle(x), C=p.C, T=p.T, iters=p.iters, bits=2, G=64, seed=99)
    ref_out = oracle.decompress(ref["codes"], ref["scales"], ref["assign"], ref["cent"], 2, 64)
    _check(rec, out, cache, ref, ref_out)
