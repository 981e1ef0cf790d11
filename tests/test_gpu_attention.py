"""GPU parity of the fused dequant-attention (qvg_attention) with the oracle.

The oracle rebuilds each record's keys (oracle.decompress, bf16) and rotates
them (oracle.rope_bf16), takes the values unrounded (oracle.reconstruct_exact)
and evaluates softmax(scale q K^T) V in fp64 (oracle.attention).  The kernel
uses the same keys, so the two differ only by the kernel's fp32 roundings of
scores, exponentials, sums and values; the test holds every output element to
the bound those roundings imply for the summation order qvg_attention
documents (_bound), on both value paths (weight sums, rebuilt values), and
requires two calls to agree bit for bit.  Queries aimed at
single tokens (the first, the last, tile and run boundaries) check that every
token position takes part: the token they aim at carries most of the weight,
so a dropped or misplaced token moves the output far beyond the bound."""
import numpy as np
import pytest
import torch

import oracle
from means_residual_compression_amd import qvg, synth
from gpu_util import DEV, bits16, say, to_oracle

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def _runs(H, N):
    """Tiles per run and run count, as the kernel's documented order cuts them."""
    ntiles = -(-N // 64)
    tps = -(-ntiles // min(ntiles, -(-2048 // H), 1024))
    return tps, -(-ntiles // tps)


def _gamma(m):
    return m * U / (1 - m * U)


def _bound(q, K, Vabs, scale, H, N, d, vT, vC, sums, mfma=False):
    """Bound on |kernel - exact| per element for one head; q [Nq, d], K [N, d]
    fp64 holding the exact (bf16) keys, Vabs [N, d] the magnitude
    |level*s_hat| + sum_t |C(t)[pi(t)]| of each value (the exact values are
    level*s_hat + sum_t C(t)[pi(t)]).

    Scores: a d-term fp32 multiply-add chain, then one product with scale:
    |s^ - s| <= delta = scale gamma_d sum_k |q_k K_nk| + u |s|.  On the
    matrix-core scores (mfma: two passes, 2 to 16 queries) each query is
    split into two bf16 parts with |q - hi - lo| <= 2^-16 |q|, the 2d
    products with the bf16 keys are exact and their fp32 accumulation is
    taken in an unknown order with each addition off by at most 2^-23
    relative (twice the round-to-nearest bound; a probe of the instruction
    stayed within 4.7 * 2^-24 of the exact sum over 128 products):
    delta = scale (2^-16 + 1.01 gamma'_2d) sum_k |q_k K_nk| + u |s|.  The
    values of those calls also go through the matrix cores: each weight is
    split the same way (a factor within 1 +- 2^-16 on its residual term) and
    the run's 2 * 64 * tps products are summed with the same 2^-23 per
    addition, i.e. a chain of 4 * 64 * tps in units of u.  Each weight
    e^(s - max) then carries a factor e^(+-delta), the exponential's relative
    error (3u times the argument, bounded by the score range, for the
    argument's roundings, plus 2^-22) and gamma_m from the chains that add it
    up (m: the longest chain of the documented order; with weight sums also
    the chain of a weight sum through its run, the merge and the
    contraction).  Factors shared by a numerator and its denominator
    (rescales, merge weights) cancel.  Moving the weights of a weighted mean
    by factors in [a, b] moves it by at most (b/a - 1) max_n |V_n - O| <=
    (b/a - 1) 2 max|V|; the roundings of the numerator's terms and of the
    denominator add 2 gamma_m max Vabs, a value rebuilt in fp32 (without
    weight sums) is within gamma_(T+1) Vabs of exact, the division adds
    u |O|."""
    Nq = q.shape[0]
    S = scale * (q @ K.T)
    absdot = np.abs(q) @ np.abs(K).T
    if mfma:
        g2 = 2 * d * 2.0 ** -23 / (1 - 2 * d * 2.0 ** -23)
        rel = 2.0 ** -16 + 1.01 * g2
    else:
        rel = _gamma(d)
    delta = (scale * rel * absdot.max(axis=1) + U * np.abs(S).max(axis=1)) * (1 + 1e-6)
    span = S.max(axis=1) - S.min(axis=1) + 2 * delta
    tps, nsplit = _runs(H, N)
    P = 256 // d
    m = (64 // P) * tps + tps + P + 2 * nsplit + 8
    if sums:
        m = max(m, 64 * tps + tps + 2 * nsplit + vT * vC * d // 2048 + 2048 // d + 8)
    if mfma:
        m = max(m, 4 * 64 * tps + tps + 2 * nsplit + vT * vC * d // 2048 + 2048 // d + 8)
    eps = 2.0 ** -22 + 3 * U * span + _gamma(m) + (2.0 ** -16 if mfma else 0.0)
    ratio = np.exp(2 * delta) * (1 + eps) / (1 - eps) - 1
    vmax = Vabs.max(axis=0)
    rebuild = 0.0 if sums else _gamma(vT + 1)
    # weight sums kept in units of 2^-40 (each weight rounded to a unit): at
    # most 2^-41 per token and stage on a weight of at most 1, against a
    # denominator of at least 1 (the largest score's weight)
    fixed = vT * N * 2.0 ** -41 if sums else 0.0
    return (2 * ratio[:, None] + 2.1 * _gamma(m) + rebuild + fixed + U) * vmax[None, :]


def _two_pass(H, N, d, Nq, kT, vpar, cdt):
    """Whether the call takes the documented two-pass path."""
    T, C = vpar[0], vpar[1]
    return (cdt == torch.bfloat16 and 1 <= kT <= 4 and min(Nq, 4) * T * max(C, 1) <= 4096
            and N * 2 * d < 2 ** 32 and H <= 256)


def _sums(H, N, d, Nq, kT, vpar, cdt):
    """Whether the values go through weight sums: on the two-pass path for up
    to 16 queries in groups of 4, else for up to 4 queries at once."""
    T, C = vpar[0], vpar[1]
    if _two_pass(H, N, d, Nq, kT, vpar, cdt):
        return True
    return Nq <= 4 and Nq * T * max(C, 1) <= 4096


def _make(seed, H, N, d, kpar, vpar, cdt):
    """Seeded key and value records (host arrays and device Records)."""
    out = []
    for s, (T, C, bits, G) in ((seed, kpar), (seed + 100, vpar)):
        codes, scales, assign, cent = synth.random_record(s, H, N, d, T, C, bits, G, Hg=40, Wg=52)
        cent = cent.to(cdt)
        dev = qvg.Record(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                         torch.from_numpy(assign).to(DEV), cent.to(DEV))
        out.append(((codes, scales, assign, cent), dev, qvg.params(C=C, T=T, iters=1, bits=bits,
                                                                  group=G)))
    return out


def _oracle_keys(host, p, heads):
    codes, scales, assign, cent = host
    return oracle.decompress(codes[heads], scales[heads], assign[heads], to_oracle(cent)[heads],
                             p.bits, p.group, out_bf16=True)


def _oracle_values(host, p, heads, magnitude=False):
    codes, scales, assign, cent = host
    return oracle.reconstruct_exact(codes[heads], scales[heads], assign[heads],
                                    to_oracle(cent)[heads], p.bits, p.group, magnitude=magnitude)


def _aimed_queries(q, K, targets, scale, gap=24.0):
    """Replace queries 1.. with ones aimed at single tokens: q = a K_n for
    the rotated key K_n, with a such that the token's score is gap."""
    for j, n in enumerate(targets, start=1):
        if j >= q.shape[0]:
            break
        kn = K[n]
        q[j] = (gap / (scale * float(kn @ kn))) * kn
    return q


def _check(got, q, kb, vh, vp, scale, rope, H, N, heads, sums, mfma):
    """got [H, Nq, d] from the kernel; kb bf16 keys and vh the value record
    (host) of the checked heads; sums: whether the call used weight sums;
    mfma: whether the scores came from the matrix cores."""
    d = q.shape[2]
    V = _oracle_values(vh, vp, heads)
    Vabs = _oracle_values(vh, vp, heads, magnitude=True)
    worst = 0.0
    for hi, h in enumerate(heads):
        kbh = kb[hi] if rope is None else oracle.rope_bf16(kb[hi], rope[0], rope[1])
        K = oracle.bf16_bits_to_f32(kbh).astype(np.float64)
        ref = oracle.attention(q[h:h + 1], kb[hi:hi + 1], V[hi:hi + 1], scale, rope)[0]
        tol = _bound(q[h].astype(np.float64), K, Vabs[hi], scale, H, N, d, vp.T, vp.C, sums,
                     mfma)
        err = np.abs(got[h].astype(np.float64) - ref)
        bad = np.argwhere(err > tol)
        assert bad.size == 0, (f"head {h}: {len(bad)} elements outside the bound; first "
                               f"{[(tuple(b), err[tuple(b)], tol[tuple(b)]) for b in bad[:4]]}")
        worst = max(worst, float((err / tol).max()))
    return worst


CASES = [
    # H, N, d, Nq, (T, C, bits, G) keys, values, centroid dtype, rope
    (2, 1000, 128, 1, (2, 64, 2, 64), (2, 64, 2, 64), torch.bfloat16, False),
    (2, 333, 64, 3, (1, 40, 4, 32), (3, 64, 2, 16), torch.float32, True),
    (3, 20000, 128, 16, (4, 256, 2, 16), (4, 256, 2, 16), torch.bfloat16, True),
    (1, 1, 128, 5, (0, 1, 4, 128), (0, 1, 2, 64), torch.bfloat16, False),
    (2, 777, 128, 2, (1, 16, 2, 64), (0, 1, 4, 32), torch.bfloat16, True),
    (4, 321, 128, 4, (1, 256, 2, 64), (1, 256, 2, 64), torch.bfloat16, True),
    (2, 2500, 128, 4, (8, 256, 2, 64), (8, 256, 2, 64), torch.bfloat16, True),
    (5, 130000, 64, 2, (2, 128, 2, 16), (1, 32, 4, 64), torch.float32, False),
    # two-pass variants: d=64 one query (INT4 and INT2 with groups of 8), and
    # three queries with INT4 values
    (2, 4099, 64, 1, (3, 128, 4, 16), (2, 64, 4, 32), torch.bfloat16, True),
    (3, 5000, 64, 1, (4, 256, 2, 8), (4, 256, 2, 8), torch.bfloat16, True),
    (2, 3001, 128, 3, (2, 64, 4, 32), (3, 128, 4, 16), torch.bfloat16, True),
    # two-pass with more than 4 queries (values in groups of 4): a ragged 7
    # (groups of 4 and 3) with INT4 values, 16 at d=64, and 5 (a group of 1)
    (3, 4500, 128, 7, (2, 128, 2, 32), (2, 256, 4, 32), torch.bfloat16, True),
    (2, 6000, 64, 16, (1, 64, 4, 16), (4, 64, 2, 8), torch.bfloat16, False),
    (4, 700, 128, 5, (3, 256, 2, 64), (1, 256, 2, 64), torch.bfloat16, True),
    # 16 queries whose weight sums do not fit (T*C = 2048): rebuilt values
    (2, 2500, 128, 16, (2, 64, 2, 64), (8, 256, 2, 64), torch.bfloat16, False),
    # two passes with value records of more than 4 stages (INT2 and INT4)
    (2, 1500, 128, 6, (2, 64, 2, 64), (8, 64, 2, 32), torch.bfloat16, True),
    (1, 2000, 64, 3, (1, 32, 4, 16), (6, 32, 4, 16), torch.bfloat16, False),
    # more than 4 queries in one values launch: d=64, INT4 values of 6 stages
    (2, 1800, 64, 9, (2, 64, 2, 32), (6, 32, 4, 16), torch.bfloat16, True),
]


@pytest.mark.parametrize("H,N,d,Nq,kpar,vpar,cdt,rope", CASES)
def test_attention_matches_oracle(H, N, d, Nq, kpar, vpar, cdt, rope):
    sums = _sums(H, N, d, Nq, kpar[0], vpar, cdt)
    mfma = Nq >= 2 and _two_pass(H, N, d, Nq, kpar[0], vpar, cdt)
    say("attention", H, N, d, Nq, kpar, vpar, cdt, "rope" if rope else "",
        "two passes" if _two_pass(H, N, d, Nq, kpar[0], vpar, cdt) else "one pass",
        "weight sums" if sums else "rebuilt values")
    (kh, kd, kp), (vh, vd, vp) = _make(17 + N % 97, H, N, d, kpar, vpar, cdt)
    heads = list(range(H))
    kb = _oracle_keys(kh, kp, heads)
    tabs = synth.rope_tables(N, d, start=3) if rope else None
    rope_np = (tabs[0].numpy(), tabs[1].numpy()) if rope else None
    scale = float(np.float32(1.0 / np.sqrt(d)))
    q = synth.queries(5 + H, H, Nq, d).numpy()
    tps, _ = _runs(H, N)
    targets = [0, N - 1, min(64, N - 1), min(64 * tps, N - 1), min(64 * tps - 1, N - 1),
               N // 2]
    for h in heads:
        kbh = kb[h] if rope_np is None else oracle.rope_bf16(kb[h], *rope_np)
        K = oracle.bf16_bits_to_f32(kbh).astype(np.float64)
        q[h] = _aimed_queries(q[h], K, targets, scale)
    qd = torch.from_numpy(q).to(DEV)
    rd = (tabs[0].to(DEV), tabs[1].to(DEV)) if rope else None
    out = qvg.attention(qd, kd, kp, vd, vp, scale, rope=rd)
    again = qvg.attention(qd, kd, kp, vd, vp, scale, rope=rd)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.array_equal(got, again.cpu().numpy()), "two calls differ"
    worst = _check(got, q, kb, vh, vp, scale, rope_np, H, N, heads, sums, mfma)
    say("  worst error / bound", worst)


@pytest.fixture(scope="module")
def decode_records():
    """The decode-side records (40 heads x 262144 tokens, d=128, T=4, C=256,
    INT2, groups of 64) for keys and values, with the rotary tables."""
    H, N, d = 40, 262144, 128
    par = (4, 256, 2, 64)
    say("drawing the decode-side records", H, N, d)
    recs = _make(4, H, N, d, par, par, torch.bfloat16)
    return H, N, d, recs, synth.rope_tables(N, d)


@pytest.mark.parametrize("Nq", [1, 16])
def test_attention_decode_record_full_size(decode_records, Nq):
    """Nq queries per head over the decode-side records, in the launch the
    benchmark times; heads 0, 17 and 39 are checked against the oracle."""
    H, N, d, ((kh, kd, kp), (vh, vd, vp)), tabs = decode_records
    say("attention full size", H, N, d, Nq)
    heads = [0, 17, 39]
    kb = _oracle_keys(kh, kp, heads)
    rope_np = (tabs[0].numpy(), tabs[1].numpy())
    scale = float(np.float32(1.0 / np.sqrt(d)))
    q = synth.queries(9, H, Nq, d).numpy()
    tps, _ = _runs(H, N)
    for hi, h in enumerate(heads):
        K = oracle.bf16_bits_to_f32(oracle.rope_bf16(kb[hi], *rope_np)).astype(np.float64)
        q[h] = _aimed_queries(q[h], K, [0, N - 1, 64 * tps, 64 * tps - 1, 123457], scale)
    out = qvg.attention(torch.from_numpy(q).to(DEV), kd, kp, vd, vp, scale,
                        rope=(tabs[0].to(DEV), tabs[1].to(DEV)))
    torch.cuda.synchronize()
    say("  checking heads", heads)
    sums = _sums(H, N, d, Nq, kp.T, (vp.T, vp.C), torch.bfloat16)
    mfma = Nq >= 2 and _two_pass(H, N, d, Nq, kp.T, (vp.T, vp.C), torch.bfloat16)
    worst = _check(out.cpu().numpy(), q, kb, vh, vp, scale, rope_np, H, N, heads, sums, mfma)
    say("  worst error / bound", worst)


def test_attention_workspace_and_rejects():
    """Workspace sizing follows the documented runs and record layout;
    invalid calls fail with the documented status before any launch."""
    vp4 = qvg.params(C=256, T=4, iters=1, bits=2, group=64)
    for H, N, d, Nq in ((40, 262144, 128, 16), (40, 262144, 128, 1), (3, 20000, 128, 1),
                        (1, 1, 64, 2)):
        tps, ns = _runs(H, N)
        extra = 4 * 256 if min(Nq, 4) * 4 * 256 <= 4096 else 0
        contract = H * Nq * 8 * d if extra else 0
        assert qvg.attention_workspace_size(H, Nq, N, d, vp4) >= (
            H * ns * Nq * (d + 2 + extra) + contract) * 4
    assert qvg.attention_workspace_size(2, 17, 100, 128, vp4) == 0
    assert qvg.attention_workspace_size(2, 1, 100, 96, vp4) == 0
    q = torch.zeros((2, 1, 128), device=DEV)
    (kh, kd, kp), (vh, vd, vp) = _make(3, 2, 100, 128, (1, 16, 2, 64), (1, 16, 2, 64),
                                       torch.bfloat16)
    with pytest.raises(qvg.QvgError, match="rope"):
        qvg.attention(q, kd, kp, vd, vp, 0.1, rope=(torch.zeros((100, 64), device=DEV), None))
    with pytest.raises(qvg.QvgError, match="Nq"):
        qvg.attention(torch.zeros((2, 17, 128), device=DEV), kd, kp, vd, vp, 0.1)
    with pytest.raises(qvg.QvgError, match="workspace"):
        qvg.attention(q, kd, kp, vd, vp, 0.1, ws=torch.empty(16, dtype=torch.uint8, device=DEV))
