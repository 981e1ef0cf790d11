"""Host-side tests of the C ABI (no GPU needed): the library loads, exports
every symbol include/qvg.h declares, and rejects invalid arguments with the
documented status codes before touching the device."""
import ctypes as ct
import os
import re

import numpy as np
import pytest
import torch

from means_residual_compression_amd import qvg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation first


def _declared():
    src = open(os.path.join(ROOT, "include", "qvg.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qvg_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    L = qvg.lib()
    names = _declared()
    assert len(names) >= 12
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(qvg.EXPORTS)


def test_status_strings():
    L = qvg.lib()
    assert L.qvg_status_string(0) == b"QVG_OK"
    assert L.qvg_status_string(4) == b"QVG_ERR_HIP"
    assert L.qvg_status_string(99) == b"QVG_UNKNOWN_STATUS"


def _ws(H, N, d, dt, **kw):
    p = qvg.params(**{**dict(C=256, T=2, iters=8, bits=2, group=64), **kw})
    return qvg.lib().qvg_workspace_size(H, N, d, dt, ct.byref(p))


def test_workspace_size_query():
    assert _ws(24, 32760, 128, qvg.QVG_BF16) > 24 * 32760 * 128 * 2  # holds the fp16 fragments
    assert _ws(1, 4096, 64, qvg.QVG_F32, C=16, T=1, iters=10, group=32) > 0
    assert _ws(1, 4096, 96, qvg.QVG_F32) == 0       # d unsupported
    assert _ws(1, 100, 128, qvg.QVG_F32, C=101) == 0  # C > N
    assert _ws(1, 4096, 128, qvg.QVG_F32, bits=3) == 0
    assert _ws(1, 4096, 128, qvg.QVG_F32, group=48) == 0
    assert _ws(1, 4096, 128, qvg.QVG_F32, T=9) == 0
    assert _ws(1, 4096, 128, qvg.QVG_F32, C=257) == 0
    assert _ws(1, 4096, 128, qvg.QVG_F32, T=0, C=1000) == 0  # C still bounded for T=0


def _compress(H=2, N=1000, d=128, dt=qvg.QVG_BF16, x=FAKE, idx="ok", init_c=None, ws=FAKE,
              ws_bytes=None, rec=True, **kw):
    L = qvg.lib()
    p = qvg.params(**{**dict(C=16, T=2, iters=3, bits=2, group=64), **kw})
    if ws_bytes is None:
        ws_bytes = 1 << 40
    keep = None
    ip = None
    if isinstance(idx, str):
        keep = np.zeros((H, max(p.T, 1), p.C), np.int32)
        if idx == "bad":
            keep[-1, -1, -1] = N
        ip = keep.ctypes.data_as(ct.c_void_p)
    r = qvg._Record(FAKE, FAKE, FAKE, FAKE) if rec else None
    st = L.qvg_compress(x, dt, H, N, d, ct.byref(p), ip, init_c, None,
                        ct.byref(r) if rec else None, ws, ws_bytes, None)
    return st, L.qvg_last_error().decode()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(x=None), INVALID, "non-NULL"),
    (dict(rec=False), INVALID, "non-NULL"),
    (dict(d=96), UNSUPPORTED, "head dims"),
    (dict(C=300), UNSUPPORTED, "C=300"),
    (dict(bits=3), UNSUPPORTED, "bits=3"),
    (dict(group=48), UNSUPPORTED, "group=48"),
    (dict(T=9), UNSUPPORTED, "T=9"),
    (dict(N=10, C=16), INVALID, "exceeds N"),
    (dict(iters=0), INVALID, "iterations"),
    (dict(H=0), INVALID, "H=0"),
    (dict(dt=7), INVALID, "dtype"),
    (dict(init_c=FAKE), INVALID, "at most one"),
    (dict(ws=None), WORKSPACE, "NULL"),
    (dict(ws_bytes=1024), WORKSPACE, "smaller"),
    (dict(ws=FAKE + 8), WORKSPACE, "aligned"),
    (dict(idx="bad"), INVALID, "outside [0, N"),
])
def test_compress_rejects(kw, status, msg):
    st, err = _compress(**kw)
    assert st == status, err
    assert msg in err


def test_decompress_and_steps_reject():
    L = qvg.lib()
    p = qvg.params(16, 2, 3, 2, 64)
    r = qvg._Record(FAKE, FAKE, FAKE, FAKE)
    assert L.qvg_decompress(None, 1, 2, 100, 128, ct.byref(p), FAKE, 1, None) == INVALID
    assert L.qvg_decompress(ct.byref(r), 1, 2, 100, 128, ct.byref(p), None, 1, None) == INVALID
    assert L.qvg_decompress(ct.byref(r), 1, 2, 100, 128, ct.byref(p), FAKE, 5, None) == INVALID
    bad = qvg.params(16, 2, 3, 4, 12)
    assert L.qvg_decompress(ct.byref(r), 1, 2, 100, 128, ct.byref(bad), FAKE, 1, None) == UNSUPPORTED
    assert L.qvg_kmeans_assign(FAKE, 1, 2, 100, 128, FAKE, 0, FAKE, FAKE, 1 << 30, None) == UNSUPPORTED
    assert L.qvg_kmeans_assign(FAKE, 1, 2, 100, 128, FAKE, 16, FAKE, FAKE, 16, None) == WORKSPACE
    assert L.qvg_kmeans_update(FAKE, 1, 2, 100, 128, None, 16, FAKE, FAKE, 1 << 30, None) == INVALID
    assert L.qvg_sas_subtract(FAKE, 1, 2, 100, 128, FAKE, FAKE, 9, 16, FAKE, None) == INVALID
    assert L.qvg_group_quant_pack(FAKE, 1, 2, 100, 128, 2, 256, FAKE, FAKE, None) == UNSUPPORTED
    assert L.qvg_compress_stream(FAKE, 1, 2, 100, 128, ct.byref(p), 3, None, 1, None,
                                 ct.byref(r), FAKE, 1 << 40, None) == INVALID


def test_decompress_chunks_rejects():
    L = qvg.lib()
    p = qvg.params(16, 2, 3, 2, 64)
    r = qvg._Record(FAKE, FAKE, FAKE, FAKE)
    recs = (qvg._Record * 2)(r, r)
    nt = (ct.c_int64 * 2)(100, 50)
    call = L.qvg_decompress_chunks
    assert call(None, nt, 2, 1, 2, 128, ct.byref(p), FAKE, 1, None) == INVALID
    assert call(recs, nt, 0, 1, 2, 128, ct.byref(p), FAKE, 1, None) == INVALID
    assert call(recs, (ct.c_int64 * 2)(100, 0), 2, 1, 2, 128, ct.byref(p), FAKE, 1, None) == INVALID
    assert call(recs, nt, 2, 1, 2, 128, ct.byref(p), None, 1, None) == INVALID
    assert call(recs, nt, 2, 1, 2, 96, ct.byref(p), FAKE, 1, None) == UNSUPPORTED
    assert call(recs, (ct.c_int64 * 2)(1 << 29, (1 << 29) + 1), 2, 1, 2, 128, ct.byref(p), FAKE,
                1, None) == UNSUPPORTED
    half = (qvg._Record * 2)(r, qvg._Record(FAKE, FAKE, None, FAKE))
    assert call(half, nt, 2, 1, 2, 128, ct.byref(p), FAKE, 1, None) == INVALID
    assert "chunk 1" in qvg.lib().qvg_last_error().decode()


def test_compressed_cache_accounting():
    """Byte and token accounting and oldest-first eviction of the container
    (host logic only: records built from CPU tensors, nothing compressed)."""
    p = qvg.preset("qvg")

    def rec(n):
        return qvg.Record(torch.zeros((2, n, 32), dtype=torch.uint8),
                          torch.zeros((2, n, 2), dtype=torch.uint8),
                          torch.zeros((2, p.T, n), dtype=torch.uint8),
                          torch.zeros((2, p.T, p.C, 128), dtype=torch.bfloat16))
    kv = qvg.CompressedKVCache(p, iters_warm=3)
    kv.records = [rec(100), rec(60), rec(40)]
    per_tok = 32 + 2 + p.T
    tables = p.T * p.C * 128 * 2
    assert kv.n_tokens() == 200 and len(kv) == 3
    assert kv.nbytes() == 2 * (200 * per_tok + 3 * tables)
    kv.evict(2)
    assert kv.n_tokens() == 40 and kv.first_token == 160 and len(kv) == 1
    kv.evict(5)
    assert len(kv) == 0 and kv.first_token == 200 and kv.nbytes() == 0


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(qvg, "_lib", None)
    monkeypatch.setattr(qvg, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        qvg.lib()


def test_operating_point_presets():
    """QVG: one stage, groups of 64; QVG-Pro: four stages, groups of 16; both
    INT2 with 256 centroids (howistudyai.com explainer, "Step-by-step" and
    "Error analysis").  Overrides replace single fields."""
    q, p = qvg.preset("qvg"), qvg.preset("pro", iters=5)
    assert (q.C, q.T, q.bits, q.group) == (256, 1, 2, 64)
    assert (p.C, p.T, p.bits, p.group, p.iters) == (256, 4, 2, 16, 5)
    assert qvg.preset("pro", bits=4).bits == 4


def test_attention_rejects():
    """qvg_attention validates before any launch: NULL pointers, a single
    rope table, Nq outside [1, 16], unsupported d or params, misaligned
    pointers, and a small workspace return the documented status codes."""
    L = qvg.lib()
    p = qvg.params(16, 2, 1, 2, 64)
    r = qvg._Record(FAKE, FAKE, FAKE, FAKE)
    ws_need = L.qvg_attention_workspace_size(2, 1, 1000, 128, ct.byref(p))
    assert ws_need > 0

    def call(q=FAKE, H=2, Nq=1, d=128, kp=p, vp=p, cos=None, sin=None, out=FAKE, ws=FAKE,
             ws_bytes=1 << 40, N=1000):
        return L.qvg_attention(q, H, Nq, d, ct.byref(r), ct.byref(kp), ct.byref(r), ct.byref(vp),
                               qvg.QVG_BF16, N, 0.1, cos, sin, out, ws, ws_bytes, None)

    assert call(q=None) == INVALID
    assert call(out=None) == INVALID
    assert call(cos=FAKE) == INVALID and "rope" in L.qvg_last_error().decode()
    assert call(Nq=0) == INVALID and call(Nq=17) == INVALID
    assert call(d=96) == UNSUPPORTED
    assert call(kp=qvg.params(16, 2, 1, 3, 64)) == UNSUPPORTED
    assert call(vp=qvg.params(300, 2, 1, 2, 64)) == UNSUPPORTED
    assert call(q=FAKE + 4) == INVALID
    assert call(ws_bytes=ws_need - 1) == WORKSPACE
    assert call(ws=FAKE + 16) == WORKSPACE
    assert L.qvg_attention_workspace_size(2, 17, 1000, 128, ct.byref(p)) == 0
    assert L.qvg_attention_workspace_size(2, 1, 1000, 128, None) == 0


def _runs(H, N):
    """Runs of 64-token tiles per head as qvg.h documents them: tps =
    ceil(ntiles / min(ntiles, ceil(2048/H), 1024)), nsplit = ceil(ntiles/tps)."""
    ntiles = -(-N // 64)
    tps = -(-ntiles // min(ntiles, -(-2048 // H), 1024))
    return tps, -(-ntiles // tps)


@pytest.mark.parametrize("H,N,d,Nq,T,C", [(40, 262144, 128, 1, 4, 256), (40, 262144, 128, 16, 4, 256),
                                          (3, 20000, 128, 4, 1, 256), (1, 1, 64, 2, 0, 1),
                                          (5, 130000, 64, 2, 1, 32), (2, 2500, 128, 4, 8, 256),
                                          (65535, 70, 128, 1, 2, 16)])
def test_attention_workspace_follows_documented_layout(H, N, d, Nq, T, C):
    """The scratch qvg_attention asks for is the documented run records (m, l,
    o[d] and, with weight sums, the T*C sums per run and query) plus, with
    weight sums, the eight contraction parts per (head, query) and the
    two-pass scores (one per head, query and token), rounded up to 256
    bytes.  Weight sums: up to 16 queries, taken 4 at a time, while 4 (or
    Nq, if fewer) times T*C sums fit 4096 entries."""
    p = qvg.params(C, T, 1, 2, 64)
    tps, ns = _runs(H, N)
    sums = Nq <= 16 and min(Nq, 4) * T * C <= 4096
    floats = H * ns * Nq * (d + 2 + (T * C if sums else 0)) + (H * Nq * (8 * d + N) if sums else 0)
    want = -(-floats * 4 // 256) * 256
    assert qvg.lib().qvg_attention_workspace_size(H, Nq, N, d, ct.byref(p)) == want


def test_params_layout_matches_the_header():
    """qvg_params in include/qvg.h: five int32 fields, then the uint64 seed at
    its natural 8-byte alignment."""
    assert ct.sizeof(qvg.Params) == 32
    assert qvg.Params.seed.offset == 24
    assert qvg.Params.group.offset == 16
