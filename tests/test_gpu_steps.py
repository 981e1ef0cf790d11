"""GPU parity of each step of the path against the CPU oracle, through the C ABI.

Every kernel of the path is checked bit-for-bit on the same seeded inputs:
quantize+pack, subtract, fused dequant, k-means assign (exact argmin, ties to
the smallest index) and k-means update (fp64 token-order means).  Sizes span
several tiles and a ragged tail.
"""
import numpy as np
import pytest
import torch

import oracle
from means_residual_compression_amd import qvg, synth
from gpu_util import DEV, as_f32, bits16, mismatch_report, say, to_oracle

pytestmark = pytest.mark.gpu


def _residual_like(seed, H, N, d, dtype):
    """Rows whose magnitudes span many binades, plus all-zero rows, rows that
    saturate the E4M3 scale and rows whose scales are E4M3 subnormals."""
    rng = np.random.default_rng(seed)
    r = rng.standard_normal((H, N, d)) * np.exp(rng.uniform(-9, 6, (H, N, 1)))
    r[:, ::37] = 0.0
    r[:, 5::41, : d // 2] *= 3000.0
    r[:, 7::43] *= 1e-4
    return synth.round_to(r, dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d,bits,G", [(128, 2, 64), (128, 4, 64), (128, 2, 16), (64, 2, 32),
                                      (64, 4, 64), (128, 4, 128)])
def test_group_quant_pack(dtype, d, bits, G):
    H, N = 3, 1037
    r = _residual_like(1, H, N, d, dtype)
    say("group_quant_pack", dtype, d, bits, G)
    codes, scales = qvg.group_quant_pack(r.to(DEV), bits, G)
    torch.cuda.synchronize()
    rf = as_f32(r)
    for h in range(H):
        c_ref, s_ref = oracle.quantize(rf[h], bits, G)
        assert np.array_equal(scales[h].cpu().numpy(), s_ref), mismatch_report(scales[h].cpu(), s_ref)
        assert np.array_equal(codes[h].cpu().numpy(), c_ref), mismatch_report(codes[h].cpu(), c_ref)


def _boundary_rows(dtype, G=64, d=128):
    """Rows whose groups have maximum 3 s_hat for an E4M3 value s_hat (so the
    group's scale is exactly s_hat) and hold every INT2 decision boundary
    r = B s_hat (B = -2, 0, 2), the neighbouring values of the input dtype on
    both sides, signed zeros, the smallest subnormals, and the group maximum
    with both signs; the rest of each group is seeded noise below the maximum."""
    f32 = dtype == torch.float32
    s_codes = [0x01, 0x05, 0x08, 0x0F, 0x20, 0x33, 0x38, 0x3B, 0x44, 0x55, 0x66, 0x7E]
    rng = np.random.default_rng(77)
    rows = []
    for sc in s_codes:
        sh = oracle.e4m3_decode(sc)
        for sign in (1.0, -1.0):
            g = np.empty(G, np.float64)
            vals = [sign * 3 * sh, -sign * 3 * sh, 0.0, -0.0]
            for B in (-2.0, 0.0, 2.0):
                x = torch.tensor([B * sh], dtype=torch.float64).to(dtype)
                up = torch.nextafter(x, torch.tensor([np.inf], dtype=dtype))
                dn = torch.nextafter(x, torch.tensor([-np.inf], dtype=dtype))
                vals += [float(x), float(up), float(dn)]
            tiny = 2.0 ** -149 if f32 else 2.0 ** -133
            vals += [tiny, -tiny]
            g[:len(vals)] = vals
            g[len(vals):] = rng.uniform(-2.9 * sh, 2.9 * sh, G - len(vals))
            rows.append(g)
    r = np.stack(rows).reshape(-1, d)  # two groups per token at d = 128
    return synth.round_to(r[None], dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_group_quant_pack_int2_boundaries(dtype):
    """INT2 codes at and next to every decision boundary (the kernel decides
    them by exact threshold comparisons, the oracle by IEEE division) equal
    the oracle's bit for bit, across the E4M3 scale range."""
    r = _boundary_rows(dtype)
    say("group_quant_pack boundaries", dtype, tuple(r.shape))
    codes, scales = qvg.group_quant_pack(r.to(DEV), 2, 64)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.quantize(as_f32(r)[0], 2, 64)
    assert np.array_equal(scales[0].cpu().numpy(), s_ref), mismatch_report(scales[0].cpu(), s_ref)
    assert np.array_equal(codes[0].cpu().numpy(), c_ref), mismatch_report(codes[0].cpu(), c_ref)


@pytest.mark.parametrize("rdt,cdt", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.float32),
                                     (torch.float32, torch.bfloat16)])
def test_sas_subtract(rdt, cdt):
    H, N, d, C = 2, 999, 128, 37
    rng = np.random.default_rng(2)
    r = _residual_like(2, H, N, d, rdt)
    chat = synth.round_to(rng.standard_normal((H, C, d)) * 10, cdt)
    pi = torch.from_numpy(rng.integers(0, C, (H, N)).astype(np.uint8))
    say("sas_subtract", rdt, cdt)
    out = qvg.sas_subtract(r.to(DEV), pi.to(DEV), chat.to(DEV))
    torch.cuda.synchronize()
    for h in range(H):
        ref = oracle.subtract(as_f32(r[h]), pi[h].numpy().astype(np.int32), as_f32(chat[h]))
        assert np.array_equal(out[h].cpu().numpy(), ref)


@pytest.mark.parametrize("T,C,bits,G,cdt,odt,d", [
    (*c, 128)[:7] for c in [
    (0, 1, 2, 64, torch.bfloat16, torch.bfloat16),
    (1, 256, 2, 64, torch.bfloat16, torch.bfloat16),
    (2, 256, 2, 64, torch.bfloat16, torch.float32),
    (4, 256, 2, 64, torch.bfloat16, torch.bfloat16),
    (3, 40, 4, 32, torch.float32, torch.float32),
    (4, 256, 4, 16, torch.float32, torch.bfloat16),
    (8, 256, 2, 64, torch.bfloat16, torch.float32),
    (8, 256, 4, 32, torch.float32, torch.bfloat16, 64),
    (2, 200, 2, 8, torch.bfloat16, torch.bfloat16, 64),
    (4, 256, 2, 128, torch.bfloat16, torch.bfloat16),  # one scale per row
    (3, 96, 4, 64, torch.float32, torch.float32, 64),
]])
def test_fused_dequant(T, C, bits, G, cdt, odt, d):
    H, N = 3, 2085
    codes, scales, assign, cent = synth.random_record(11 + T, H, N, d, T, C, bits, G, Hg=40, Wg=52)
    cent = cent.to(cdt)
    p = qvg.params(C=C, T=T, iters=1, bits=bits, group=G)
    rec = qvg.Record(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                     torch.from_numpy(assign).to(DEV), cent.to(DEV))
    say("fused_dequant", T, C, bits, G, cdt, odt)
    out = qvg.decompress(rec, p, out_dtype=odt)
    torch.cuda.synchronize()
    ref = oracle.decompress(codes, scales, assign, to_oracle(cent), bits, G,
                            out_bf16=odt == torch.bfloat16)
    got = bits16(out) if odt == torch.bfloat16 else out.cpu().numpy()
    assert np.array_equal(got, ref), mismatch_report(got, ref)


@pytest.mark.parametrize("N", [1, 7, 32, 33, 4096, 4127])
@pytest.mark.parametrize("T", [2, 4])
def test_fused_dequant_step_edges(T, N):
    """Token counts around a wave's step: rows that leave every wave a partial
    step only, exact multiples of the step (no partial step) and a ragged tail
    after many full steps, with and without the prefetching loop (T >= 3)."""
    H, d, C, bits, G = 2, 128, 256, 2, 64
    codes, scales, assign, cent = synth.random_record(31 + N, H, N, d, T, C, bits, G)
    p = qvg.params(C=C, T=T, iters=1, bits=bits, group=G)
    rec = qvg.Record(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                     torch.from_numpy(assign).to(DEV), cent.to(DEV))
    say("fused_dequant step edges", T, N)
    out = qvg.decompress(rec, p, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.decompress(codes, scales, assign, to_oracle(cent), bits, G, out_bf16=True)
    got = bits16(out)
    assert np.array_equal(got, ref), mismatch_report(got, ref)


def _rounding_patterns(rng, n):
    """fp32 bit patterns across every binade: exact bf16 ties (both parities),
    one ulp either side of a tie, fp32 subnormals, zeros of both signs and the
    values just below the fp32 maximum that round to infinity."""
    u = rng.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    exp = (u >> 23) & 0xFF
    u[exp == 0xFF] &= np.uint32(0xBFFFFFFF)  # no inf/NaN inputs
    k = n // 8
    u[0:k] = (u[0:k] & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    u[k:2 * k] = (u[k:2 * k] & np.uint32(0xFFFF0000)) | np.uint32(0x7FFF)
    u[2 * k:3 * k] = (u[2 * k:3 * k] & np.uint32(0xFFFF0000)) | np.uint32(0x8001)
    u[3 * k:4 * k] &= np.uint32(0x807FFFFF)  # subnormal
    u[4 * k:4 * k + 16] = np.array([0, 0x80000000, 0x7F7FFFFF, 0xFF7FFFFF, 0x7F7F8000, 0x7F7F7FFF,
                                    0x00008000, 0x00018000, 0x80008000, 1, 0x807FFFFF, 0x007FFFFF,
                                    0x3F808000, 0x3F818000, 0xBF808000, 0xBF818000], np.uint32)
    return u.view(np.float32)


@pytest.mark.parametrize("bits", [2, 4])
def test_fused_dequant_every_scale_code(bits):
    """Scale bytes over every finite E4M3 code, subnormals included."""
    H, N, d, C, T, G = 2, 1777, 128, 64, 2, 32
    codes, scales, assign, cent = synth.random_record(21, H, N, d, T, C, bits, G, Hg=40, Wg=52)
    rng = np.random.default_rng(4)
    scales = rng.integers(0, 0x7F, scales.shape, dtype=np.uint8)
    scales[:, :, 0] = np.arange(N * H).reshape(H, N) % 0x7F  # every code appears
    p = qvg.params(C=C, T=T, iters=1, bits=bits, group=G)
    rec = qvg.Record(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                     torch.from_numpy(assign).to(DEV), cent.to(DEV))
    say("fused_dequant every scale code", bits)
    out = qvg.decompress(rec, p, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.decompress(codes, scales, assign, to_oracle(cent), bits, G, out_bf16=False)
    got = out.cpu().numpy()
    assert np.array_equal(got, ref), mismatch_report(got, ref)


def test_fused_dequant_bf16_rounding():
    """With zero scales the output is the fp32 centroid rounded to bf16, so
    crafted centroid bit patterns pin the output rounding (RNE) exactly."""
    H, N, d, C = 2, 1500, 128, 50
    rng = np.random.default_rng(5)
    cent = _rounding_patterns(rng, H * C * d).reshape(H, 1, C, d).copy()
    codes = rng.integers(0, 256, (H, N, d // 4), dtype=np.uint8)
    scales = np.zeros((H, N, d // 64), np.uint8)
    assign = rng.integers(0, C, (H, 1, N), dtype=np.uint8)
    p = qvg.params(C=C, T=1, iters=1, bits=2, group=64)
    rec = qvg.Record(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                     torch.from_numpy(assign).to(DEV), torch.from_numpy(cent).to(DEV))
    say("fused_dequant rounding")
    out = qvg.decompress(rec, p, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref = oracle.decompress(codes, scales, assign, cent, 2, 64, out_bf16=True)
    got = bits16(out)
    assert np.array_equal(got, ref), mismatch_report(got, ref)
    assert (got == 0x7F80).any() and (got == 0xFF80).any()  # overflow to infinity occurred


def _video(H, N, d, kind_mix=True, seed_cfg=1):
    c = synth.CONFIGS["self_forcing"]
    heads = []
    for h in range(H):
        kind = h % 2 if kind_mix else 0
        x = synth.video_head(synth._seed(seed_cfg, kind, h), 8, c["Hg"], c["Wg"], d,
                             synth.OUTLIER_SCALE[kind], n_tokens=N)
        heads.append(x)
    return synth.round_to(np.stack(heads), torch.bfloat16)


@pytest.mark.parametrize("C", [256, 100, 33, 3, 2, 1])
def test_kmeans_assign_bf16_video(C):
    H, N, d = 4, 2500, 128
    x = _video(H, N, d)
    xf = as_f32(x)
    # realistic centroids: two Lloyd iterations of the oracle from seeded rows
    idx = synth.init_indices(21, H, 1, N, C)[:, 0]
    cents = np.stack([oracle.kmeans(xf[h], xf[h][idx[h]], 2)[0] for h in range(H)])
    say("kmeans_assign bf16 video C=", C)
    pi = qvg.kmeans_assign(x.to(DEV), torch.from_numpy(cents).to(DEV))
    torch.cuda.synchronize()
    for h in range(H):
        ref = oracle.assign(xf[h], cents[h])
        assert np.array_equal(pi[h].cpu().numpy().astype(np.int32), ref), \
            mismatch_report(pi[h].cpu().numpy(), ref)


@pytest.mark.parametrize("d", [64, 128])
def test_kmeans_assign_fp32_residual_and_ties(d):
    H, N, C = 2, 1500, 64
    rng = np.random.default_rng(5)
    r = (rng.standard_normal((H, N, d)) * np.exp(rng.uniform(-3, 3, (H, N, 1)))).astype(np.float32)
    cents = r[:, rng.choice(N, C, replace=False)].copy()
    cents[:, 10] = cents[:, 3]          # exact duplicate: ties must go to index 3
    cents[:, 20] = 0.0
    cents[:, 21] = 0.0                  # duplicate zero centroids
    r[:, 100] = 0.0                     # a zero token equidistant from both
    say("kmeans_assign fp32 d=", d)
    pi = qvg.kmeans_assign(torch.from_numpy(r).to(DEV), torch.from_numpy(cents).to(DEV))
    torch.cuda.synchronize()
    for h in range(H):
        ref = oracle.assign(r[h], cents[h])
        assert np.array_equal(pi[h].cpu().numpy().astype(np.int32), ref), \
            mismatch_report(pi[h].cpu().numpy(), ref)
        assert 10 not in set(pi[h].cpu().numpy().tolist())
        assert 21 not in set(pi[h].cpu().numpy().tolist())


@pytest.mark.parametrize("dtype,d", [(torch.bfloat16, 128), (torch.float32, 128), (torch.float32, 64)])
def test_kmeans_update(dtype, d):
    H, N, C = 3, 3001, 200
    rng = np.random.default_rng(6)
    r = _residual_like(6, H, N, d, dtype)
    pi = rng.integers(0, C - 5, (H, N)).astype(np.uint8)  # clusters C-5..C-1 stay empty
    pi[:, :700] = 7                                       # one large cluster
    old = rng.standard_normal((H, C, d)).astype(np.float32)
    cent = torch.from_numpy(old.copy()).to(DEV)
    say("kmeans_update", dtype, d)
    qvg.kmeans_update(r.to(DEV), torch.from_numpy(pi).to(DEV), cent)
    torch.cuda.synchronize()
    rf = as_f32(r)
    for h in range(H):
        ref, cnt = oracle.update(rf[h], pi[h].astype(np.int32), old[h])
        assert np.array_equal(cent[h].cpu().numpy(), ref), mismatch_report(cent[h].cpu().numpy(), ref)
        assert np.array_equal(cent[h, C - 5:].cpu().numpy(), old[h, C - 5:])
