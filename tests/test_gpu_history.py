"""GPU parity of the stream-history reconstruction (qvg_decompress_chunks)
and of the compressed-cache container: every element equals the oracle's
decompression of the chunk record it comes from, bit for bit, with ragged
chunk lengths, more chunks than one launch takes, several stage counts, group
sizes and output dtypes, and chunks evicted from the front."""
import numpy as np
import pytest
import torch

import oracle
from means_residual_compression_amd import qvg, synth
from gpu_util import DEV, bits16, mismatch_report, say, to_oracle

pytestmark = pytest.mark.gpu


def _records(seed, H, lens, d, T, C, bits, G, cdt):
    host, dev = [], []
    for c, n in enumerate(lens):
        codes, scales, assign, cent = synth.random_record(seed + c, H, n, d, T, C, bits, G,
                                                          Hg=40, Wg=52)
        cent = cent.to(cdt)
        host.append((codes, scales, assign, cent))
        dev.append(qvg.Record(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV),
                              torch.from_numpy(assign).to(DEV), cent.to(DEV)))
    return host, dev


def _oracle_history(host, bits, G, out_bf16):
    parts = [oracle.decompress(codes, scales, assign, to_oracle(cent), bits, G, out_bf16=out_bf16)
             for codes, scales, assign, cent in host]
    return np.concatenate(parts, axis=1)


@pytest.mark.parametrize("lens,T,C,bits,G,cdt,odt,d", [
    ([1500, 777, 2101], 2, 256, 2, 64, torch.bfloat16, torch.bfloat16, 128),
    ([4680] * 3 + [1], 4, 256, 2, 16, torch.bfloat16, torch.bfloat16, 128),
    ([31, 300, 65, 1029], 1, 40, 4, 32, torch.float32, torch.float32, 64),
    ([37 + 13 * c for c in range(35)], 3, 64, 2, 64, torch.bfloat16, torch.float32, 128),
    ([900, 450], 0, 1, 4, 128, torch.bfloat16, torch.bfloat16, 128),
])
def test_history_matches_per_chunk_oracle(lens, T, C, bits, G, cdt, odt, d):
    H = 3
    host, dev = _records(31 + T, H, lens, d, T, C, bits, G, cdt)
    p = qvg.params(C=C, T=T, iters=1, bits=bits, group=G)
    say("history", len(lens), "chunks", T, C, bits, G, cdt, odt, d)
    out = qvg.decompress_chunks(dev, p, out_dtype=odt)
    torch.cuda.synchronize()
    assert out.shape == (H, sum(lens), d)
    ref = _oracle_history(host, bits, G, odt == torch.bfloat16)
    got = bits16(out) if odt == torch.bfloat16 else out.cpu().numpy()
    assert np.array_equal(got, ref), mismatch_report(got, ref)


def test_container_stream_with_eviction():
    """Five chunks of a video-shaped stream through the container (the first
    cold, the rest warm from the centroid cache) with a byte budget that keeps
    three; the kept history equals the oracle's decompression of the kept
    records, and the records equal a direct compress_stream chain."""
    H, d = 2, 128
    p = qvg.params(C=64, T=2, iters=3, bits=2, group=64)
    chunks = [synth.stream_chunk(2, synth.K_KIND, H, ci, 1, 30, 52, d, 1e2, torch.bfloat16)
              for ci in range(5)]
    idx = synth.init_indices(800, H, p.T, chunks[0].shape[1], p.C)
    per_chunk = qvg.empty_record(H, chunks[0].shape[1], d, p, torch.bfloat16, DEV).nbytes()
    kv = qvg.CompressedKVCache(p, iters_warm=2, max_bytes=3 * per_chunk)
    say("container stream", len(chunks), "chunks")
    for ch in chunks:
        kv.append(ch.to(DEV), init_idx=idx)
    torch.cuda.synchronize()
    assert len(kv) == 3 and kv.first_token == 2 * chunks[0].shape[1]
    assert kv.nbytes() <= 3 * per_chunk
    # the same chain by hand
    cache = torch.zeros((H, p.T, p.C, d), dtype=torch.float32, device=DEV)
    ref_recs = []
    for ci, ch in enumerate(chunks):
        ref_recs.append(qvg.compress_stream(ch.to(DEV), p, 2, cache, ci > 0,
                                            init_idx=idx if ci == 0 else None))
    for a, b in zip(kv.records, ref_recs[2:]):
        for f in ("codes", "scales", "assign", "centroids"):
            assert torch.equal(getattr(a, f), getattr(b, f)), f
    out = kv.reconstruct()
    torch.cuda.synchronize()
    host = [(r.codes.cpu().numpy(), r.scales.cpu().numpy(), r.assign.cpu().numpy(),
             r.centroids.cpu()) for r in kv.records]
    ref = _oracle_history(host, p.bits, p.group, True)
    got = bits16(out)
    assert np.array_equal(got, ref), mismatch_report(got, ref)
