"""Thin ctypes binding of libqvg.so (C ABI in include/qvg.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
libqvg.so.  PyTorch supplies device memory and the current stream.  There is
no fallback: if the library is missing or a call fails, an exception is
raised.
"""
from __future__ import annotations

import ctypes as ct
import os
from dataclasses import dataclass

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqvg.so")

QVG_F32, QVG_BF16 = 0, 1
_STATUS = {0: "QVG_OK", 1: "QVG_ERR_INVALID_ARG", 2: "QVG_ERR_UNSUPPORTED",
           3: "QVG_ERR_WORKSPACE", 4: "QVG_ERR_HIP"}
EXPORTS = ["qvg_status_string", "qvg_last_error", "qvg_workspace_size", "qvg_compress",
           "qvg_compress_stream", "qvg_compress_stream_static", "qvg_decompress",
           "qvg_decompress_chunks",
           "qvg_assign_workspace_size",
           "qvg_kmeans_assign", "qvg_update_workspace_size", "qvg_kmeans_update",
           "qvg_sas_subtract", "qvg_group_quant_pack", "qvg_timing_enable", "qvg_timing_reset",
           "qvg_timing_read", "qvg_candidate_counts", "qvg_attention",
           "qvg_attention_workspace_size"]


class QvgError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_STATUS.get(status, status)}: {msg}")
        self.status = status


class Params(ct.Structure):
    _fields_ = [("C", ct.c_int32), ("T", ct.c_int32), ("iters", ct.c_int32),
                ("bits", ct.c_int32), ("group", ct.c_int32), ("seed", ct.c_uint64)]


class _Record(ct.Structure):
    _fields_ = [("codes", ct.c_void_p), ("scales", ct.c_void_p), ("assign", ct.c_void_p),
                ("centroids", ct.c_void_p)]


@dataclass
class Record:
    """Compressed record of H head-tensors (device tensors)."""
    codes: torch.Tensor      # uint8 [H, N, d*bits/8]
    scales: torch.Tensor     # uint8 [H, N, d/G] (E4M3 codes)
    assign: torch.Tensor     # uint8 [H, T, N]
    centroids: torch.Tensor  # [H, T, C, d] in the input dtype

    def _c(self) -> _Record:
        return _Record(self.codes.data_ptr(), self.scales.data_ptr(), self.assign.data_ptr(),
                       self.centroids.data_ptr())

    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size()
                   for t in (self.codes, self.scales, self.assign, self.centroids))


_lib = None


def lib() -> ct.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m means_residual_compression_amd.build`")
        L = ct.CDLL(LIB_PATH)
        p, i64, i32, sz = ct.c_void_p, ct.c_int64, ct.c_int32, ct.c_size_t
        P = ct.POINTER(Params)
        R = ct.POINTER(_Record)
        sig = {
            "qvg_status_string": ([ct.c_int], ct.c_char_p),
            "qvg_last_error": ([], ct.c_char_p),
            "qvg_workspace_size": ([i64, i64, i64, ct.c_int, P], sz),
            "qvg_compress": ([p, ct.c_int, i64, i64, i64, P, p, p, p, R, p, sz, p], ct.c_int),
            "qvg_compress_stream": ([p, ct.c_int, i64, i64, i64, P, i32, p, ct.c_int, p, R, p,
                                     sz, p], ct.c_int),
            "qvg_compress_stream_static": ([p, ct.c_int, i64, i64, i64, P, i32, p, ct.c_int, p,
                                            R, p], ct.c_int),
            "qvg_decompress": ([R, ct.c_int, i64, i64, i64, P, p, ct.c_int, p], ct.c_int),
            "qvg_decompress_chunks": ([R, ct.POINTER(i64), i32, ct.c_int, i64, i64, P, p,
                                       ct.c_int, p], ct.c_int),
            "qvg_assign_workspace_size": ([i64, i64, i64, i32], sz),
            "qvg_kmeans_assign": ([p, ct.c_int, i64, i64, i64, p, i32, p, p, sz, p], ct.c_int),
            "qvg_update_workspace_size": ([i64, i64, i64, i32], sz),
            "qvg_kmeans_update": ([p, ct.c_int, i64, i64, i64, p, i32, p, p, sz, p], ct.c_int),
            "qvg_sas_subtract": ([p, ct.c_int, i64, i64, i64, p, p, ct.c_int, i32, p, p],
                                 ct.c_int),
            "qvg_group_quant_pack": ([p, ct.c_int, i64, i64, i64, i32, i32, p, p, p], ct.c_int),
            "qvg_timing_enable": ([ct.c_int], None),
            "qvg_timing_reset": ([], None),
            "qvg_timing_read": ([ct.c_char_p, ct.POINTER(ct.c_double)], i64),
            "qvg_candidate_counts": ([p, i64, i64, i64, ct.c_int, P, p, i32], ct.c_int),
            "qvg_attention": ([p, i64, i64, i64, R, P, R, P, ct.c_int, i64, ct.c_float, p, p,
                               p, p, sz, p], ct.c_int),
            "qvg_attention_workspace_size": ([i64, i64, i64, i64, P], sz),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes, f.restype = args, res
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise QvgError(status, lib().qvg_last_error().decode())


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return QVG_BF16
    if t.dtype == torch.float32:
        return QVG_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _torch_dt(code: int) -> torch.dtype:
    return torch.bfloat16 if code == QVG_BF16 else torch.float32


def _stream():
    return ct.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous device tensor")


def params(C: int, T: int, iters: int, bits: int, group: int, seed: int = 0) -> Params:
    """Method parameters; `seed` drives the cold-start draw when a compress
    call gets neither init_idx nor init_centroids."""
    return Params(C, T, iters, bits, group, seed)


# The two operating points the howistudyai.com explainer names ("Step-by-step",
# progressive stages and low-bit quantization; "Error analysis", block-size
# trade-off): QVG, one stage with groups of 64 channels (highest
# compression), and QVG-Pro, four stages with groups of 16 (highest
# fidelity); both INT2 with C = 256 centroids (uint8 assignments).  A preset
# is chosen per tensor: K and V head-tensors are compressed by separate calls
# and may use different ones.  The iteration count is not fixed by the pages.
PRESETS = {"qvg": dict(C=256, T=1, bits=2, group=64),
           "pro": dict(C=256, T=4, bits=2, group=16)}


def preset(name: str, iters: int = 8, **override) -> Params:
    """Params of a named operating point, with optional field overrides."""
    kw = dict(PRESETS[name], iters=iters)
    kw.update(override)
    return params(**kw)


def workspace_size(H, N, d, dtype: torch.dtype, p: Params) -> int:
    code = QVG_BF16 if dtype == torch.bfloat16 else QVG_F32
    n = lib().qvg_workspace_size(H, N, d, code, ct.byref(p))
    if n == 0:
        raise QvgError(1, "invalid sizes or parameters for the workspace query")
    return n


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    # torch allocations are 512-byte aligned, which satisfies the 256-byte rule
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def empty_record(H, N, d, p: Params, dtype: torch.dtype, device) -> Record:
    return Record(
        codes=torch.empty((H, N, d * p.bits // 8), dtype=torch.uint8, device=device),
        scales=torch.empty((H, N, d // p.group), dtype=torch.uint8, device=device),
        assign=torch.zeros((H, p.T, N), dtype=torch.uint8, device=device),
        centroids=torch.zeros((H, p.T, p.C, d), dtype=dtype, device=device))


def _idx_ptr(init_idx):
    """int32 [H, T, C] start rows: a numpy array or a CPU torch tensor (pinned
    memory keeps the library's host-to-device copy asynchronous), or a device
    tensor (read by the kernels, no copy)."""
    if init_idx is None:
        return None, None
    if isinstance(init_idx, torch.Tensor):
        if init_idx.dtype != torch.int32 or not init_idx.is_contiguous():
            raise ValueError("init_idx must be a contiguous int32 tensor")
        return init_idx, ct.c_void_p(init_idx.data_ptr())
    a = np.ascontiguousarray(init_idx, dtype=np.int32)
    return a, a.ctypes.data_as(ct.c_void_p)


def compress(x: torch.Tensor, p: Params, init_idx=None, init_centroids=None, cache_out=None,
             ws: torch.Tensor | None = None, out: Record | None = None) -> Record:
    """x: [H, N, d] bf16/fp32 device tensor.  Stage starts: init_idx (int32
    [H, T, C], host or device), else init_centroids (fp32 [H, T, C, d]), else
    rows drawn from p.seed."""
    _dev(x, "x")
    H, N, d = x.shape
    out = out or empty_record(H, N, d, p, x.dtype, x.device)
    ws = ws if ws is not None else alloc_workspace(workspace_size(H, N, d, x.dtype, p), x.device)
    keep, idx_p = _idx_ptr(init_idx)
    rec = out._c()
    _check(lib().qvg_compress(
        x.data_ptr(), _dt(x), H, N, d, ct.byref(p), idx_p,
        None if init_centroids is None else init_centroids.data_ptr(),
        None if cache_out is None else cache_out.data_ptr(), ct.byref(rec),
        ws.data_ptr(), ws.numel(), _stream()))
    del keep
    return out


def compress_stream(chunk: torch.Tensor, p: Params, iters_warm: int, cache: torch.Tensor,
                    warm: bool, init_idx=None, ws: torch.Tensor | None = None,
                    out: Record | None = None) -> Record:
    _dev(chunk, "chunk")
    H, N, d = chunk.shape
    out = out or empty_record(H, N, d, p, chunk.dtype, chunk.device)
    ws = ws if ws is not None else alloc_workspace(workspace_size(H, N, d, chunk.dtype, p),
                                                   chunk.device)
    keep, idx_p = _idx_ptr(init_idx)
    rec = out._c()
    _check(lib().qvg_compress_stream(
        chunk.data_ptr(), _dt(chunk), H, N, d, ct.byref(p), iters_warm, cache.data_ptr(),
        1 if warm else 0, idx_p, ct.byref(rec), ws.data_ptr(), ws.numel(), _stream()))
    del keep
    return out


STATIC_SCRATCH_BYTES = 64 << 20  # QVG_STATIC_SCRATCH_BYTES in include/qvg.h


def compress_stream_static(chunk: torch.Tensor, p: Params, iters_warm: int, cache: torch.Tensor,
                           warm: bool, init_idx=None, out: Record | None = None) -> Record:
    """qvg_compress_stream on the library's static device scratch: no
    workspace argument (the record is still caller memory; pass `out` to
    allocate nothing at all)."""
    _dev(chunk, "chunk")
    H, N, d = chunk.shape
    out = out or empty_record(H, N, d, p, chunk.dtype, chunk.device)
    keep, idx_p = _idx_ptr(init_idx)
    rec = out._c()
    _check(lib().qvg_compress_stream_static(
        chunk.data_ptr(), _dt(chunk), H, N, d, ct.byref(p), iters_warm, cache.data_ptr(),
        1 if warm else 0, idx_p, ct.byref(rec), _stream()))
    del keep
    return out


def decompress(rec: Record, p: Params, out_dtype: torch.dtype | None = None,
               out: torch.Tensor | None = None) -> torch.Tensor:
    H, N = rec.codes.shape[:2]
    d = rec.codes.shape[2] * 8 // p.bits
    cdt = rec.centroids.dtype
    odt = out_dtype or cdt
    if out is None:
        out = torch.empty((H, N, d), dtype=odt, device=rec.codes.device)
    r = rec._c()
    _check(lib().qvg_decompress(ct.byref(r), _dt(rec.centroids), H, N, d, ct.byref(p),
                                out.data_ptr(), _dt(out), _stream()))
    return out


def decompress_chunks(recs: list, p: Params, out_dtype: torch.dtype | None = None,
                      out: torch.Tensor | None = None) -> torch.Tensor:
    """Reconstructs a stream's history [H, sum N_c, d] from its chunk records
    (all with params p), head by head in chunk order, in one pass over the
    records (launches of up to 32 chunks)."""
    if not recs:
        raise ValueError("no chunk records")
    H = recs[0].codes.shape[0]
    d = recs[0].codes.shape[2] * 8 // p.bits
    cdt = recs[0].centroids.dtype
    n_tok = [r.codes.shape[1] for r in recs]
    for r in recs:
        if r.codes.shape[0] != H or r.codes.shape[2] * 8 // p.bits != d or r.centroids.dtype != cdt:
            raise ValueError("chunk records differ in H, d or dtype")
    odt = out_dtype or cdt
    if out is None:
        out = torch.empty((H, sum(n_tok), d), dtype=odt, device=recs[0].codes.device)
    arr = (_Record * len(recs))(*[r._c() for r in recs])
    nt = (ct.c_int64 * len(recs))(*n_tok)
    _check(lib().qvg_decompress_chunks(arr, nt, len(recs), _dt(recs[0].centroids), H, d,
                                       ct.byref(p), out.data_ptr(), _dt(out), _stream()))
    return out


def attention_workspace_size(H: int, Nq: int, N: int, d: int, vp: Params) -> int:
    return lib().qvg_attention_workspace_size(H, Nq, N, d, ct.byref(vp))


def attention(q: torch.Tensor, k_rec: Record, kp: Params, v_rec: Record, vp: Params,
              scale: float, rope: tuple | None = None, ws: torch.Tensor | None = None,
              out: torch.Tensor | None = None) -> torch.Tensor:
    """softmax(scale q K^T) V per head for q [H, Nq, d] fp32 (Nq <= 16) over
    the keys and values the two records hold, rebuilt on chip; rope = (cos,
    sin), each [N, d/2] fp32, rotates the rebuilt keys.  Returns [H, Nq, d]
    fp32."""
    _dev(q, "q")
    H, Nq, d = q.shape
    N = k_rec.codes.shape[1]
    if v_rec.codes.shape[1] != N or k_rec.centroids.dtype != v_rec.centroids.dtype:
        raise ValueError("key and value records differ in token count or centroid dtype")
    if q.dtype != torch.float32 or not q.is_contiguous():
        raise ValueError("q must be contiguous fp32")
    if ws is None:
        ws = alloc_workspace(attention_workspace_size(H, Nq, N, d, vp), q.device)
    if out is None:
        out = torch.empty((H, Nq, d), dtype=torch.float32, device=q.device)
    cos, sin = rope if rope is not None else (None, None)
    kr, vr = k_rec._c(), v_rec._c()
    _check(lib().qvg_attention(
        q.data_ptr(), H, Nq, d, ct.byref(kr), ct.byref(kp), ct.byref(vr), ct.byref(vp),
        _dt(k_rec.centroids), N, float(scale), None if cos is None else cos.data_ptr(),
        None if sin is None else sin.data_ptr(), out.data_ptr(), ws.data_ptr(), ws.numel(),
        _stream()))
    return out


class CompressedKVCache:
    """The compressed KV history of one tensor kind across a stream: one
    record per chunk (each chunk compressed on its own, warm-started from the
    previous chunk's centroids), byte accounting, eviction of the oldest
    chunks, and reconstruction of the whole history in one pass.  Device
    memory is held by the records (torch tensors); nothing else is allocated
    beyond one reused workspace."""

    def __init__(self, p: Params, iters_warm: int, max_bytes: int | None = None):
        self.p, self.iters_warm, self.max_bytes = p, iters_warm, max_bytes
        self.records: list[Record] = []
        self.first_token = 0          # stream position of the oldest kept token
        self._cache = None            # fp32 centroid cache [H, T, C, d]
        self._ws = None

    def __len__(self) -> int:
        return len(self.records)

    def n_tokens(self) -> int:
        return sum(r.codes.shape[1] for r in self.records)

    def nbytes(self) -> int:
        return sum(r.nbytes() for r in self.records)

    def append(self, chunk: torch.Tensor, init_idx=None) -> Record:
        """Compresses the next chunk [H, N, d] and appends its record; the
        first chunk starts cold from init_idx (or from rows drawn from
        p.seed when it is None), later ones warm from the cache.
        Evicts the oldest chunks while the records exceed max_bytes."""
        H, N, d = chunk.shape
        need = workspace_size(H, N, d, chunk.dtype, self.p)
        if self._ws is None or self._ws.numel() < need:
            self._ws = alloc_workspace(need, chunk.device)
        if self._cache is None:
            self._cache = torch.zeros((H, self.p.T, self.p.C, d), dtype=torch.float32,
                                      device=chunk.device)
            rec = compress_stream(chunk, self.p, self.iters_warm, self._cache, False,
                                  init_idx=init_idx, ws=self._ws)
        else:
            rec = compress_stream(chunk, self.p, self.iters_warm, self._cache, True, ws=self._ws)
        self.records.append(rec)
        while self.max_bytes is not None and len(self.records) > 1 and \
                self.nbytes() > self.max_bytes:
            self.evict(1)
        return rec

    def evict(self, n: int = 1):
        """Drops the n oldest chunk records."""
        for _ in range(min(n, len(self.records))):
            self.first_token += self.records[0].codes.shape[1]
            self.records.pop(0)

    def reconstruct(self, out_dtype: torch.dtype | None = None,
                    out: torch.Tensor | None = None) -> torch.Tensor:
        """The kept history [H, n_tokens, d] in stream order."""
        return decompress_chunks(self.records, self.p, out_dtype=out_dtype, out=out)


def kmeans_assign(r: torch.Tensor, centroids: torch.Tensor, ws=None) -> torch.Tensor:
    _dev(r, "r")
    H, N, d = r.shape
    C = centroids.shape[1]
    out = torch.empty((H, N), dtype=torch.uint8, device=r.device)
    n = lib().qvg_assign_workspace_size(H, N, d, C)
    ws = ws if ws is not None else alloc_workspace(max(n, 256), r.device)
    _check(lib().qvg_kmeans_assign(r.data_ptr(), _dt(r), H, N, d, centroids.data_ptr(), C,
                                   out.data_ptr(), ws.data_ptr(), ws.numel(), _stream()))
    return out


def kmeans_update(r: torch.Tensor, assign: torch.Tensor, centroids: torch.Tensor, ws=None):
    """Updates `centroids` (fp32 [H, C, d]) in place and returns it."""
    _dev(r, "r")
    H, N, d = r.shape
    C = centroids.shape[1]
    n = lib().qvg_update_workspace_size(H, N, d, C)
    ws = ws if ws is not None else alloc_workspace(max(n, 256), r.device)
    _check(lib().qvg_kmeans_update(r.data_ptr(), _dt(r), H, N, d, assign.data_ptr(), C,
                                   centroids.data_ptr(), ws.data_ptr(), ws.numel(), _stream()))
    return centroids


def sas_subtract(r: torch.Tensor, assign: torch.Tensor, chat: torch.Tensor) -> torch.Tensor:
    _dev(r, "r")
    H, N, d = r.shape
    out = torch.empty((H, N, d), dtype=torch.float32, device=r.device)
    _check(lib().qvg_sas_subtract(r.data_ptr(), _dt(r), H, N, d, assign.data_ptr(),
                                  chat.data_ptr(), _dt(chat), chat.shape[1], out.data_ptr(),
                                  _stream()))
    return out


def group_quant_pack(r: torch.Tensor, bits: int, group: int):
    _dev(r, "r")
    H, N, d = r.shape
    codes = torch.empty((H, N, d * bits // 8), dtype=torch.uint8, device=r.device)
    scales = torch.empty((H, N, d // group), dtype=torch.uint8, device=r.device)
    _check(lib().qvg_group_quant_pack(r.data_ptr(), _dt(r), H, N, d, bits, group,
                                      codes.data_ptr(), scales.data_ptr(), _stream()))
    return codes, scales


# ------------------------------------------------------------ diagnostics
KERNELS = ["kmeans_assign", "kmeans_resolve", "kmeans_sort",
           "kmeans_accumulate", "kmeans_delta", "kmeans_init", "kmeans_prepare", "kmeans_tables", "absmax",
           "sas_subtract", "group_quant_pack", "fused_dequant", "fill"]


def timing_enable(on: bool = True):
    lib().qvg_timing_enable(1 if on else 0)


def timing_reset():
    lib().qvg_timing_reset()


def timing_read(kernel: str):
    """(total_ms, launches) of the recorded launches of `kernel`."""
    ms = ct.c_double(0.0)
    n = lib().qvg_timing_read(kernel.encode(), ct.byref(ms))
    if n < 0:
        raise QvgError(4, "timing read failed")
    return ms.value, int(n)


def candidate_counts(ws: torch.Tensor, x: torch.Tensor, p: Params, n_iters: int) -> np.ndarray:
    """[n_iters, 2] (re-checked, fully scanned) token counts of the last compress
    that used `ws` for input shaped like `x` (synchronises the device)."""
    H, N, d = x.shape
    out = np.zeros(2 * n_iters, np.uint32)
    _check(lib().qvg_candidate_counts(ws.data_ptr(), H, N, d, _dt(x), ct.byref(p),
                                      out.ctypes.data_as(ct.c_void_p), n_iters))
    return out.reshape(n_iters, 2)
