"""GPU parity at the two largest workload shapes, through the C ABI.

* The long-video cache: 131072 tokens (84 frames of a 39x40 grid plus the
  first 32 tokens of frame 84, scenes cut every 21 frames), d=128, bf16,
  C=256, T=4 stages, INT2 and INT4 with G=64.  Whole records (assignments,
  centroids, codes, scales, fp32 centroid cache) and reconstructions are
  compared bit for bit with the oracle on one K and one V head-tensor, at the
  workload's 8 iterations per stage (the oracle splits each head's
  assignment over the host's threads).
* The decode-side record: 40 head-tensors x 262144 tokens, T=4, C=256, INT2
  G=64, bf16 centroids; the fused dequant of every token is compared bit for
  bit with the oracle's reconstruction.  And the decode shape as the
  benchmark measures it: a video-shaped cache of 20 K + 20 V head-tensors x
  262144 tokens compressed on the GPU (T=4, 8 iterations) and decompressed,
  with a K and a V head-tensor's record and reconstruction checked against
  the oracle's compress of the same input.
* The stream: 20 chunks of 4680 tokens of 24 head-tensors, the first cold and
  the rest warm-started from the centroid cache, sampled head-tensors' records
  and caches compared with the oracle's chain after every chunk.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from means_residual_compression_amd import qvg, synth
from gpu_util import DEV, bits16, mismatch_report, rec_equal, say, to_oracle

pytestmark = pytest.mark.gpu


def _threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _large_heads(kinds):
    c = synth.CONFIGS["long_video"]
    parts = [synth.video_cache(3, k, 1, c["F"], c["Hg"], c["Wg"], c["d"], c["outlier"][k],
                               c["dtype"], c["scene_len"], c["n_tokens"], head_ids=[0])
             for k in kinds]
    return torch.cat(parts, 0), c


@pytest.mark.parametrize("bits,kinds", [(2, (synth.K_KIND, synth.V_KIND)), (4, (synth.V_KIND,))])
def test_large_cache_full_size(bits, kinds):
    x, c = _large_heads(kinds)
    H, N, d = x.shape
    p = qvg.params(C=c["C"], T=c["T"], iters=c["iters"], bits=bits, group=c["group"])
    idx = synth.init_indices(3, H, p.T, N, p.C)
    say("large cache", tuple(x.shape), "bits", bits)
    cache = torch.zeros((H, p.T, p.C, d), dtype=torch.float32, device=DEV)
    rec = qvg.compress(x.to(DEV), p, init_idx=idx, cache_out=cache)
    out = qvg.decompress(rec, p)
    torch.cuda.synchronize()
    ref = oracle.compress(to_oracle(x), C=p.C, T=p.T, iters=p.iters, bits=p.bits, G=p.group,
                          init_idx=idx, threads=_threads())
    bad = rec_equal(rec, ref)
    assert not bad, f"record fields differ from the oracle: {bad}"
    assert np.array_equal(cache.cpu().numpy(), ref["cache"])
    ref_out = oracle.decompress(ref["codes"], ref["scales"], ref["assign"], ref["cent"], p.bits,
                                p.group, threads=_threads())
    got = bits16(out)
    assert np.array_equal(got, ref_out), mismatch_report(got, ref_out)


def test_decode_record_full_size():
    H, N, d, T, C, bits, G = 40, 262144, 128, 4, 256, 2, 64
    codes, scales, assign, cent = synth.random_record(4, H, N, d, T, C, bits, G)
    p = qvg.params(C=C, T=T, iters=1, bits=bits, group=G)
    rec = qvg.Record(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                     torch.from_numpy(assign).to(DEV), cent.to(DEV))
    say("decode-side record", (H, N, d), "T", T)
    out = qvg.decompress(rec, p, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    got = bits16(out)
    del out, rec
    ref = oracle.decompress(codes, scales, assign, to_oracle(cent), bits, G, out_bf16=True,
                            threads=_threads())
    assert np.array_equal(got, ref), mismatch_report(got, ref)


def test_stream_full_size():
    """The stream workload as the benchmark runs it: 12 K + 12 V head-tensors,
    20 chunks of 3 frames (4680 tokens each), d=128, bf16, C=256, T=2, INT2
    G=64; chunk 0 cold (10 iterations from seeded rows), chunks 1-19
    warm-started from the previous chunk's fp32 centroid cache (3
    iterations).  After every chunk the records and caches of head-tensors 0
    (K) and 12 (V) equal the oracle's chain bit for bit."""
    c = synth.CONFIGS["stream"]
    heads = [0, c["heads"]]
    p = qvg.params(C=c["C"], T=c["T"], iters=c["iters"], bits=c["bits"], group=c["group"])
    cache, ref_cache = None, None
    for ci in range(c["chunks"]):
        x = torch.cat([synth.stream_chunk(2, k, c["heads"], ci, c["F"], c["Hg"], c["Wg"], c["d"],
                                          c["outlier"][k], c["dtype"]) for k in c["kinds"]], 0)
        H, N, d = x.shape
        if cache is None:
            cache = torch.zeros((H, p.T, p.C, d), dtype=torch.float32, device=DEV)
        warm = ci > 0
        idx = None if warm else synth.init_indices(2000, H, p.T, N, p.C)
        say("stream chunk", ci, "warm" if warm else "cold", (H, N, d))
        rec = qvg.compress_stream(x.to(DEV), p, c["iters_warm"], cache, warm, init_idx=idx)
        torch.cuda.synchronize()
        ref = oracle.compress(to_oracle(x)[heads], C=p.C, T=p.T,
                              iters=c["iters_warm"] if warm else p.iters, bits=p.bits,
                              G=p.group, init_idx=None if warm else idx[heads],
                              init_c=ref_cache, threads=_threads())
        ref_cache = ref["cache"]
        sub = qvg.Record(rec.codes[heads], rec.scales[heads], rec.assign[heads],
                         rec.centroids[heads])
        bad = rec_equal(sub, ref)
        assert not bad, f"chunk {ci}: {bad} differ from the oracle"
        got_cache = cache[heads].cpu().numpy()
        assert np.array_equal(got_cache, ref_cache), f"chunk {ci}: centroid cache differs"


def test_decode_shape_record_from_gpu_compress():
    c = synth.CONFIGS["long_video"]
    N, d, hk = 262144, 128, 20
    x = torch.cat([synth.video_cache_device(4, k, hk, c["Hg"], c["Wg"], d, c["outlier"][k], N,
                                            c["scene_len"], torch.bfloat16, DEV)
                   for k in c["kinds"]])
    p = qvg.params(C=256, T=4, iters=c["iters"], bits=2, group=64, seed=4)
    say("decode shape from GPU compress", tuple(x.shape))
    rec = qvg.compress(x, p)
    out = qvg.decompress(rec, p)
    torch.cuda.synchronize()
    sel = [0, hk]  # one K and one V head-tensor
    xs = x[sel].cpu()
    got = bits16(out[sel])
    sub = qvg.Record(rec.codes[sel], rec.scales[sel], rec.assign[sel], rec.centroids[sel])
    del out, x
    ref = oracle.compress(to_oracle(xs), C=p.C, T=p.T, iters=p.iters, bits=2, G=64, seed=None,
                          init_idx=np.stack([np.stack([oracle.sample_rows(N, p.C, 4, h, t + 1)
                                                       for t in range(p.T)]) for h in sel]),
                          threads=_threads())
    bad = rec_equal(sub, ref)
    assert not bad, f"record fields differ from the oracle: {bad}"
    ref_out = oracle.decompress(ref["codes"], ref["scales"], ref["assign"], ref["cent"], 2, 64,
                                threads=_threads())
    assert np.array_equal(got, ref_out), mismatch_report(got, ref_out)
