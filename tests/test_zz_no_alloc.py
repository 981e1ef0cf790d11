"""qvg_compress_stream_static (the entry point that allocates nothing, its
scratch a static device array) against qvg_compress_stream with a caller
workspace: two calls in a row on the same static scratch, the second with a
smaller chunk, each bit-identical to the workspace entry point, plus the
size limit."""
import ctypes as ct

import numpy as np
import pytest
import torch

from means_residual_compression_amd import qvg, synth
from gpu_util import DEV, say

pytestmark = pytest.mark.gpu


def _same(a, b):
    for f in ("codes", "scales", "assign", "centroids"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f


def test_static_scratch_matches_workspace_entry():
    p = qvg.params(C=256, T=2, iters=4, bits=2, group=64, seed=7)
    big = synth.video_cache(2, 0, 24, 3, 30, 52, 128, 1e2, torch.bfloat16).to(DEV)  # 24 x 4680
    small = synth.video_cache(2, 1, 5, 2, 30, 52, 128, 1e3, torch.bfloat16, n_tokens=1999).to(DEV)
    H, N, d = big.shape
    assert qvg.workspace_size(H, N, d, big.dtype, p) <= qvg.STATIC_SCRATCH_BYTES
    # 1) cold chunk, seeded draw, 24 x 4680
    say("static scratch: cold 24 x 4680")
    ca = torch.zeros((H, p.T, p.C, d), dtype=torch.float32, device=DEV)
    cb = torch.zeros_like(ca)
    ra = qvg.compress_stream_static(big, p, 3, ca, False)
    rb = qvg.compress_stream(big, p, 3, cb, False)
    torch.cuda.synchronize()
    _same(ra, rb)
    assert torch.equal(ca, cb)
    # 2) warm chunk, fewer heads and tokens (the array keeps the last call's data)
    say("static scratch: warm 5 x 1999")
    h2 = small.shape[0]
    ca2, cb2 = ca[:h2].clone(), cb[:h2].clone()
    ra2 = qvg.compress_stream_static(small, p, 3, ca2, True)
    rb2 = qvg.compress_stream(small, p, 3, cb2, True)
    torch.cuda.synchronize()
    _same(ra2, rb2)
    assert torch.equal(ca2, cb2)


def test_static_scratch_rejects_oversized():
    p = qvg.params(C=256, T=2, iters=4, bits=2, group=64)
    H, N, d = 24, 32760, 128
    assert qvg.workspace_size(H, N, d, torch.bfloat16, p) > qvg.STATIC_SCRATCH_BYTES
    L = qvg.lib()
    fake = ct.c_void_p(1 << 20)
    r = qvg._Record(fake, fake, fake, fake)
    st = L.qvg_compress_stream_static(fake, qvg.QVG_BF16, H, N, d, ct.byref(p), 3, fake, 1, None,
                                      ct.byref(r), None)
    assert st == 3  # QVG_ERR_WORKSPACE, before anything is enqueued
    assert "static array" in L.qvg_last_error().decode()
