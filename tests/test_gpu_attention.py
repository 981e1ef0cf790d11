"""GPU parity of the fused dequant-attention (qvg_attention) with the oracle.

The oracle rebuilds each record's keys and values (oracle.decompress, bf16),
rotates the keys (oracle.rope_bf16) and evaluates softmax(scale q K^T) V in
fp64 (oracle.attention).  The kernel works on the same bf16 numbers, so the
two differ only by the kernel's fp32 roundings of scores, exponentials and
sums; the test holds every output element to the bound those roundings imply
for the summation order qvg_attention documents (_bound).  Queries aimed at
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


def _bound(q, K, V, scale, H, N):
    """Bound on |kernel - exact| per element for one head; q [Nq, d], K, V
    [N, d] fp64 holding the exact (bf16 / fp32) values.

    Scores: a d-term fp32 multiply-add chain, then one product with scale:
    |s^ - s| <= delta = scale gamma_d sum_k |q_k K_nk| + u |s|.  Each weight
    e^(s - max) then carries a factor e^(+-delta), the exponential's relative
    error (3u times the argument, bounded by the score range, for the
    argument's roundings, plus 2^-22) and gamma_m from the chain that adds it
    up (m: the longest chain of the documented order).  Factors shared by a
    numerator and its denominator (rescales, merge weights) cancel.  Moving
    the weights of a weighted mean by factors in [a, b] moves it by at most
    (b/a - 1) max_n |V_n - O| <= (b/a - 1) 2 max|V|; numerator and denominator
    chains rounding apart add 2 gamma_m |O|, the division u |O|."""
    d = q.shape[1]
    S = scale * (q @ K.T)
    absdot = np.abs(q) @ np.abs(K).T
    delta = (scale * _gamma(d) * absdot.max(axis=1) + U * np.abs(S).max(axis=1)) * (1 + 1e-6)
    span = S.max(axis=1) - S.min(axis=1) + 2 * delta
    tps, nsplit = _runs(H, N)
    P = 256 // d
    m = (64 // P) * tps + tps + P + 2 * nsplit + 8
    eps = 2.0 ** -22 + 3 * U * span + _gamma(m)
    ratio = np.exp(2 * delta) * (1 + eps) / (1 - eps) - 1
    vmax = np.abs(V).max(axis=0)
    return (2 * ratio[:, None] + 2.1 * _gamma(m) + U) * vmax[None, :]


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


def _oracle_kv(host, p, heads):
    codes, scales, assign, cent = host
    return oracle.decompress(codes[heads], scales[heads], assign[heads], to_oracle(cent)[heads],
                             p.bits, p.group, out_bf16=True)


def _aimed_queries(q, K, rope, targets, scale, gap=24.0):
    """Replace queries 1.. with ones aimed at single tokens: q = a K_n for
    the rotated key K_n, with a such that the token's score is gap."""
    for j, n in enumerate(targets, start=1):
        if j >= q.shape[0]:
            break
        kn = K[n]
        q[j] = (gap / (scale * float(kn @ kn))) * kn
    return q


def _check(got, q, kb, vb, scale, rope, H, N, heads):
    worst = 0.0
    for hi, h in enumerate(heads):
        kbh = kb[hi] if rope is None else oracle.rope_bf16(kb[hi], rope[0], rope[1])
        K = oracle.bf16_bits_to_f32(kbh).astype(np.float64)
        V = oracle.bf16_bits_to_f32(vb[hi]).astype(np.float64)
        ref = oracle.attention(q[h:h + 1], kb[hi:hi + 1], vb[hi:hi + 1], scale, rope)[0]
        tol = _bound(q[h].astype(np.float64), K, V, scale, H, N)
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
    (4, 321, 128, 4, (1, 256, 2, 64), (1, 256, 2, 64), torch.bfloat16, True),
    (5, 130000, 64, 2, (2, 128, 2, 16), (1, 32, 4, 64), torch.float32, False),
]


@pytest.mark.parametrize("H,N,d,Nq,kpar,vpar,cdt,rope", CASES)
def test_attention_matches_oracle(H, N, d, Nq, kpar, vpar, cdt, rope):
    say("attention", H, N, d, Nq, kpar, vpar, cdt, "rope" if rope else "")
    (kh, kd, kp), (vh, vd, vp) = _make(17 + N % 97, H, N, d, kpar, vpar, cdt)
    heads = list(range(H))
    kb, vb = _oracle_kv(kh, kp, heads), _oracle_kv(vh, vp, heads)
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
        q[h] = _aimed_queries(q[h], K, rope_np, targets, scale)
    qd = torch.from_numpy(q).to(DEV)
    rd = (tabs[0].to(DEV), tabs[1].to(DEV)) if rope else None
    out = qvg.attention(qd, kd, kp, vd, vp, scale, rope=rd)
    torch.cuda.synchronize()
    worst = _check(out.cpu().numpy(), q, kb, vb, scale, rope_np, H, N, heads)
    say("  worst error / bound", worst)


def test_attention_decode_record_full_size():
    """The decode-side record (40 heads x 262144 tokens, d=128, T=4, C=256,
    INT2, groups of 64) for keys and values, 16 queries per head with the
    rotary tables, in the launch the benchmark times; heads 0, 17 and 39 are
    checked against the oracle."""
    H, N, d, Nq = 40, 262144, 128, 16
    say("attention full size", H, N, d, Nq)
    par = (4, 256, 2, 64)
    (kh, kd, kp), (vh, vd, vp) = _make(4, H, N, d, par, par, torch.bfloat16)
    heads = [0, 17, 39]
    kb, vb = _oracle_kv(kh, kp, heads), _oracle_kv(vh, vp, heads)
    tabs = synth.rope_tables(N, d)
    rope_np = (tabs[0].numpy(), tabs[1].numpy())
    scale = float(np.float32(1.0 / np.sqrt(d)))
    q = synth.queries(9, H, Nq, d).numpy()
    tps, _ = _runs(H, N)
    for hi, h in enumerate(heads):
        K = oracle.bf16_bits_to_f32(oracle.rope_bf16(kb[hi], *rope_np)).astype(np.float64)
        q[h] = _aimed_queries(q[h], K, rope_np, [0, N - 1, 64 * tps, 64 * tps - 1, 123457], scale)
    out = qvg.attention(torch.from_numpy(q).to(DEV), kd, kp, vd, vp, scale,
                        rope=(tabs[0].to(DEV), tabs[1].to(DEV)))
    torch.cuda.synchronize()
    worst = _check(out.cpu().numpy(), q, kb, vb, scale, rope_np, H, N, heads)
    say("  worst error / bound", worst)


def test_attention_workspace_and_rejects():
    """Workspace sizing follows the documented runs; invalid calls fail with
    the documented status before any launch."""
    L = qvg.lib()
    for H, N, d, Nq in ((40, 262144, 128, 16), (3, 20000, 128, 1), (1, 1, 64, 2)):
        tps, ns = _runs(H, N)
        assert L.qvg_attention_workspace_size(H, Nq, N, d) >= H * ns * Nq * (d + 2) * 4
    assert L.qvg_attention_workspace_size(2, 17, 100, 128) == 0
    assert L.qvg_attention_workspace_size(2, 1, 100, 96) == 0
    q = torch.zeros((2, 1, 128), device=DEV)
    (kh, kd, kp), (vh, vd, vp) = _make(3, 2, 100, 128, (1, 16, 2, 64), (1, 16, 2, 64),
                                       torch.bfloat16)
    with pytest.raises(qvg.QvgError, match="rope"):
        qvg.attention(q, kd, kp, vd, vp, 0.1, rope=(torch.zeros((100, 64), device=DEV), None))
    with pytest.raises(qvg.QvgError, match="Nq"):
        qvg.attention(torch.zeros((2, 17, 128), device=DEV), kd, kp, vd, vp, 0.1)
    with pytest.raises(qvg.QvgError, match="workspace"):
        qvg.attention(q, kd, kp, vd, vp, 0.1, ws=torch.empty(16, dtype=torch.uint8, device=DEV))
