"""QVG CPU oracle (test infrastructure only).

Plain C implementation in ``qvg_oracle.c`` (see its header for the passages of
the Quant VideoGen pages each function follows), loaded with ctypes and wrapped
for numpy arrays.  Only the tests, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` use this package; the product library never does.
"""
from __future__ import annotations

import ctypes as ct
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qvg_oracle.c")
_LIB = os.path.join(_HERE, "libqvg_oracle.so")
GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
             "-pthread"]

DT_F32, DT_BF16 = 0, 1
_lib = None


def build() -> str:
    """Compile the oracle with gcc (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ct.CDLL(_LIB)
        p, i64, i32, f32 = ct.c_void_p, ct.c_int64, ct.c_int, ct.c_float
        L.qvgo_e4m3_encode.argtypes, L.qvgo_e4m3_encode.restype = [f32], ct.c_uint8
        L.qvgo_e4m3_decode.argtypes, L.qvgo_e4m3_decode.restype = [ct.c_uint8], f32
        L.qvgo_f32_to_bf16.argtypes, L.qvgo_f32_to_bf16.restype = [f32], ct.c_uint16
        L.qvgo_dist.argtypes, L.qvgo_dist.restype = [p, p, i32], ct.c_double
        L.qvgo_assign.argtypes = [p, i64, i32, p, i32, p]
        L.qvgo_update.argtypes = [p, i64, i32, p, i32, p, p]
        L.qvgo_kmeans.argtypes = [p, i64, i32, p, i32, i32, p]
        L.qvgo_subtract.argtypes = [p, i64, i32, p, p, p]
        L.qvgo_quantize.argtypes = [p, i64, i32, i32, i32, p, p]
        L.qvgo_compress.argtypes = [p, i32, i64, i64, i32, i32, i32, i32, i32, i32, p, p,
                                    ct.c_uint64, p, p, p, p, p, i32]
        L.qvgo_splitmix64.argtypes, L.qvgo_splitmix64.restype = [p], ct.c_uint64
        L.qvgo_sample_rows.argtypes = [i64, i32, ct.c_uint64, i64, i32, p]
        L.qvgo_sample_rows.restype = None
        L.qvgo_decompress.argtypes = [p, p, p, p, i32, i64, i64, i32, i32, i32, i32, i32,
                                      p, i32, i32]
        for f in ("qvgo_assign", "qvgo_update", "qvgo_kmeans", "qvgo_quantize", "qvgo_subtract",
                  "qvgo_compress", "qvgo_decompress"):
            getattr(L, f).restype = None
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ct.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


# ----------------------------------------------------------------- codecs
def e4m3_encode(s: float) -> int:
    return int(lib().qvgo_e4m3_encode(float(s)))


def e4m3_decode(code: int) -> float:
    return float(lib().qvgo_e4m3_decode(int(code)))


def f32_to_bf16_bits(x: float) -> int:
    return int(lib().qvgo_f32_to_bf16(float(x)))


# ---------------------------------------------------------------- k-means
def dist(r, c) -> float:
    r = _c(r, np.float32)
    c = _c(c, np.float32)
    return float(lib().qvgo_dist(_ptr(r), _ptr(c), r.shape[-1]))


def assign(R, C) -> np.ndarray:
    R = _c(R, np.float32)
    C = _c(C, np.float32)
    pi = np.empty(R.shape[0], np.int32)
    lib().qvgo_assign(_ptr(R), R.shape[0], R.shape[1], _ptr(C), C.shape[0], _ptr(pi))
    return pi


def update(R, pi, C):
    """Returns (new centroids, counts); C is not modified."""
    R = _c(R, np.float32)
    pi = _c(pi, np.int32)
    Cn = np.array(C, dtype=np.float32, copy=True, order="C")
    cnt = np.empty(Cn.shape[0], np.int64)
    lib().qvgo_update(_ptr(R), R.shape[0], R.shape[1], _ptr(pi), Cn.shape[0], _ptr(Cn),
                      _ptr(cnt))
    return Cn, cnt


def kmeans(R, C0, iters):
    R = _c(R, np.float32)
    C = np.array(C0, dtype=np.float32, copy=True, order="C")
    pi = np.zeros(R.shape[0], np.int32)
    lib().qvgo_kmeans(_ptr(R), R.shape[0], R.shape[1], _ptr(C), C.shape[0], iters, _ptr(pi))
    return C, pi


def subtract(R, pi, C):
    """fp32 residual R - C[pi] (C already in fp32 values of the stored centroids)."""
    R = _c(R, np.float32)
    pi = _c(pi, np.int32)
    C = _c(C, np.float32)
    out = np.empty_like(R)
    lib().qvgo_subtract(_ptr(R), R.shape[0], R.shape[1], _ptr(pi), _ptr(C), _ptr(out))
    return out


def quantize(R, bits, G):
    R = _c(R, np.float32)
    N, d = R.shape
    codes = np.empty((N, d * bits // 8), np.uint8)
    scales = np.empty((N, d // G), np.uint8)
    lib().qvgo_quantize(_ptr(R), N, d, bits, G, _ptr(codes), _ptr(scales))
    return codes, scales


# ------------------------------------------------------------ whole path
def _as_store(X):
    """numpy fp32 -> (array, DT_F32); bf16 given as uint16 bit patterns -> DT_BF16."""
    if X.dtype == np.uint16:
        return _c(X, np.uint16), DT_BF16
    return _c(X, np.float32), DT_F32


def splitmix64(state: int, n: int):
    """The first n outputs of splitmix64 started from `state`."""
    st = ct.c_uint64(state)
    return [int(lib().qvgo_splitmix64(ct.byref(st))) for _ in range(n)]


def sample_rows(N: int, C: int, seed: int, h: int, t: int) -> np.ndarray:
    """Cold-start rows of stage t (1-based) of head h: C distinct indices in
    [0, N) from the seeded partial Fisher-Yates shuffle."""
    rows = np.empty(C, np.int32)
    lib().qvgo_sample_rows(N, C, ct.c_uint64(seed), h, t, _ptr(rows))
    return rows


def compress(X, C, T, iters, bits, G, init_idx=None, init_c=None, seed=None, threads=None):
    """X: [H, N, d] fp32, or bf16 bit patterns as uint16.  Stage starts come
    from init_idx rows, else init_c centroids, else rows drawn with
    sample_rows(seed).  Returns dict with codes, scales, assign [H,T,N] uint8,
    cent [H,T,C,d] (same storage as X), cache [H,T,C,d] fp32."""
    X, dt = _as_store(X)
    H, N, d = X.shape
    if T > 0 and init_idx is None and init_c is None and seed is None:
        raise ValueError("cold start needs init_idx, init_c or a seed")
    idx = None if init_idx is None else _c(init_idx, np.int32)
    ic = None if init_c is None else _c(init_c, np.float32)
    out = dict(codes=np.empty((H, N, d * bits // 8), np.uint8),
               scales=np.empty((H, N, d // G), np.uint8),
               assign=np.zeros((H, T, N), np.uint8),
               cent=np.zeros((H, T, C, d), X.dtype),
               cache=np.zeros((H, T, C, d), np.float32))
    lib().qvgo_compress(_ptr(X), dt, H, N, d, C, T, iters, bits, G, _ptr(idx), _ptr(ic),
                        ct.c_uint64(0 if seed is None else seed), _ptr(out["codes"]), _ptr(out["scales"]), _ptr(out["assign"]),
                        _ptr(out["cent"]), _ptr(out["cache"]), threads or default_threads())
    return out


def decompress(codes, scales, assign, cent, bits, G, out_bf16=None, threads=None):
    """cent: [H,T,C,d] fp32 or uint16 (bf16 bits).  Output dtype follows the
    centroid storage unless out_bf16 is given.  Returns fp32 array or uint16
    bf16 bit patterns."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    assign = _c(assign, np.uint8)
    cent, cdt = _as_store(cent)
    H, T, C, d = cent.shape
    N = codes.shape[1]
    if out_bf16 is None:
        out_bf16 = cdt == DT_BF16
    out = np.empty((H, N, d), np.uint16 if out_bf16 else np.float32)
    lib().qvgo_decompress(_ptr(codes), _ptr(scales), _ptr(assign), _ptr(cent), cdt, H, N, d, C,
                          T, bits, G, _ptr(out), DT_BF16 if out_bf16 else DT_F32,
                          threads or default_threads())
    return out


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------ attention
# The step after the path: attention of a block of queries over the
# reconstructed history (note.zhuruihan.top "Algorithm-System Co-design":
# the fused dequantization serves the attention that reads the cache;
# paper.rainbus.top novelty paragraph: keys are cached before the rotary
# position embedding, so it is applied after reconstruction).  Plain fp64,
# except the steps a model takes in lower precision, written out below.

def f32_to_bf16_bits_array(x) -> np.ndarray:
    """fp32 array -> bf16 bit patterns, round to nearest even, overflow to
    infinity (finite inputs)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def rope_bf16(k_bits, cos, sin) -> np.ndarray:
    """Rotary position embedding, rotate-half form, applied to bf16 keys.
    k_bits: [N, d] bf16 bit patterns; cos, sin: [N, d/2] fp32.  For
    k < d/2 with a = x_k, b = x_{k+d/2}, c = cos[:, k], s = sin[:, k]:
        y_k = a*c - b*s,   y_{k+d/2} = b*c + a*s,
    every product and the sum rounded to fp32 (no fused multiply-add), then
    y rounded to bf16 (RNE).  Returns bf16 bit patterns [N, d]."""
    x = bf16_bits_to_f32(k_bits)
    h = x.shape[1] // 2
    a, b = x[:, :h], x[:, h:]
    c = np.asarray(cos, np.float32)
    s = np.asarray(sin, np.float32)
    lo = np.float32(a * c) - np.float32(b * s)
    hi = np.float32(b * c) + np.float32(a * s)
    return f32_to_bf16_bits_array(np.concatenate([lo, hi], axis=1).astype(np.float32))


def reconstruct_exact(codes, scales, assign, cent, bits, G, magnitude=False) -> np.ndarray:
    """The reconstruction of paper.rainbus.top's DQ step without a final
    rounding: level(q) * s_hat + C(T)[pi(T)] + ... + C(1)[pi(1)] per element,
    in fp64 (each term is exact in fp64: an odd level times an E4M3 scale, or
    a bf16/fp32 centroid).  Codes unpack as stored (element k of a row in
    byte k*bits/8 at bit offset bits*(k mod 8/bits)); levels are 2q - (2^bits
    - 1); assignments above C-1 read row C-1.  With magnitude=True returns
    |level * s_hat| + sum_t |C(t)[pi(t)]| instead (the scale of the rounding
    errors any evaluation of the sum makes).  cent: [H,T,C,d] fp32 or bf16
    bit patterns.  Returns [H, N, d] fp64."""
    codes = np.asarray(codes, np.uint8)
    H, N, nb = codes.shape
    d = nb * 8 // bits
    per, L = 8 // bits, (1 << bits) - 1
    q = np.empty((H, N, d), np.int64)
    for k in range(d):
        q[..., k] = (codes[..., k * bits // 8] >> (bits * (k % per))) & L
    table = np.array([e4m3_decode(c) for c in range(256)], np.float64)
    s = np.repeat(table[np.asarray(scales, np.uint8)], G, axis=-1)
    out = (2 * q - L) * s
    if magnitude:
        out = np.abs(out)
    cent = np.asarray(cent)
    c64 = (bf16_bits_to_f32(cent) if cent.dtype == np.uint16 else cent).astype(np.float64)
    T, C = c64.shape[1], c64.shape[2]
    assign = np.minimum(np.asarray(assign, np.int64), C - 1)
    for h in range(H):
        for t in range(T - 1, -1, -1):
            rows = c64[h, t][assign[h, t]]
            out[h] += np.abs(rows) if magnitude else rows
    return out


def attention(q, k_bits, v, scale, rope=None) -> np.ndarray:
    """O = softmax(scale * q k^T) v per head, in fp64.
    q: [H, Nq, d] fp32; k_bits: [H, N, d] bf16 bit patterns of the
    reconstructed keys; v: [H, N, d] values (taken as fp64; the attention
    step uses reconstruct_exact); rope: None or (cos, sin), each [N, d/2]
    fp32, applied to the keys with rope_bf16.  Softmax subtracts the row
    maximum.  Returns [H, Nq, d] fp64."""
    q = np.asarray(q, np.float32).astype(np.float64)
    H, Nq, d = q.shape
    out = np.empty((H, Nq, d), np.float64)
    for h in range(H):
        kb = k_bits[h] if rope is None else rope_bf16(k_bits[h], rope[0], rope[1])
        K = bf16_bits_to_f32(kb).astype(np.float64)
        V = np.asarray(v[h], np.float64)
        S = float(scale) * (q[h] @ K.T)
        S -= S.max(axis=1, keepdims=True)
        P = np.exp(S)
        P /= P.sum(axis=1, keepdims=True)
        out[h] = P @ V
    return out
