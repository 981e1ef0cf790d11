"""Warm streamed chunks captured in a HIP graph (through torch.cuda.graph)
and replayed: each replay, with eager work and synchronisation between the
replays, gives the record and centroid cache an eager call gives.  Covers
qvg_compress_stream with a caller workspace and qvg_compress_stream_static
(the entry point without one), so the path is capture-safe: no allocation,
no memset node, no host copy."""
import pytest
import torch

from means_residual_compression_amd import qvg, synth
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def _same(a, b):
    for f in ("codes", "scales", "assign", "centroids"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f


@pytest.mark.parametrize("static", [False, True])
def test_warm_chunk_graph_replays(static):
    c = synth.CONFIGS["stream"]
    p = qvg.params(C=c["C"], T=c["T"], iters=c["iters"], bits=2, group=64, seed=11)
    chunks = [torch.cat([synth.stream_chunk(2, k, 4, ci, c["F"], c["Hg"], c["Wg"], 128,
                                            c["outlier"][k], torch.bfloat16) for k in c["kinds"]])
              .to(DEV) for ci in range(3)]
    H, N, d = chunks[0].shape
    ws = qvg.alloc_workspace(qvg.workspace_size(H, N, d, torch.bfloat16, p), DEV)
    cache = torch.zeros((H, p.T, p.C, d), dtype=torch.float32, device=DEV)
    qvg.compress_stream(chunks[0], p, 3, cache, False, ws=ws)       # cold chunk, eager
    start = cache.clone()
    rec = qvg.empty_record(H, N, d, p, torch.bfloat16, DEV)

    def call(x):
        if static:
            qvg.compress_stream_static(x, p, 3, cache, True, out=rec)
        else:
            qvg.compress_stream(x, p, 3, cache, True, ws=ws, out=rec)

    call(chunks[1])  # eager warm-up outside the capture (first-call set-up)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cache.copy_(start)
    with torch.cuda.graph(g):
        call(chunks[1])
    for rep in range(3):
        say("graph replay", rep, "static" if static else "workspace")
        # eager reference of the same warm step from the same cache
        cache.copy_(start)
        call(chunks[1])
        torch.cuda.synchronize()
        want = qvg.Record(*(t.clone() for t in (rec.codes, rec.scales, rec.assign, rec.centroids)))
        want_cache = cache.clone()
        # eager work in between, then the replay from the same cache
        call(chunks[2])
        cache.copy_(start)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(rec, want)
        assert torch.equal(cache, want_cache)
