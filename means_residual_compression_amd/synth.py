"""Seeded synthetic inputs shaped like the video KV caches the QVG pages evaluate on.

This module only draws random numbers and lays them out; it holds none of the
compression method's arithmetic, so both the CPU oracle and the HIP path can be
fed from it without sharing any of the method.

The pages' real caches (LongCat-Video-13B, HY-WorldPlay-8B, Self-Forcing-Wan-1.3B;
howistudyai.com page, "The test" section) are not available, so these stand in
for them.  Every generator is a pure function of its integer seed.

Token model (one head of K or V), following the pages' spatiotemporal-redundancy
description (note.zhuruihan.top, "Semantic-Aware Smoothing"; paper.rainbus.top,
novelty paragraph: max|K| ~ 1e2, max|V| ~ 1e3):

    token(f, y, x) = base[y, x] + 0.05 * f * drift[y, x] + eps,
    base, drift ~ N(0, 1)^d,   eps ~ N(0, 0.1^2)^d,

with 4 outlier channels per head (drawn from a seeded permutation) whose base
entries are multiplied by `outlier_scale`.  Tokens are ordered
i = f * (Hg * Wg) + y * Wg + x.  Values are drawn in float64 and rounded (RNE)
to the storage dtype.
"""
from __future__ import annotations

import numpy as np
import torch

K_KIND, V_KIND = 0, 1
OUTLIER_SCALE = {K_KIND: 1e2, V_KIND: 1e3}


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(k) for k in key]))


def round_to(x64: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """fp64 numpy array -> CPU tensor of `dtype` (RNE through fp32)."""
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32))
    return t.to(dtype) if dtype != torch.float32 else t


def _head_fields(rng: np.random.Generator, Hg: int, Wg: int, d: int, outlier_scale: float):
    outl = rng.permutation(d)[:4]
    base = rng.standard_normal((Hg, Wg, d))
    drift = rng.standard_normal((Hg, Wg, d))
    base[..., outl] *= outlier_scale
    return base, drift, outl


def video_head(seed: int, F: int, Hg: int, Wg: int, d: int, outlier_scale: float,
               scene_len: int | None = None, n_tokens: int | None = None) -> np.ndarray:
    """One head-tensor [N, d] (fp64).  With `scene_len`, base and drift are
    re-drawn every `scene_len` frames and f restarts at 0 in each scene.
    `n_tokens` truncates the (F x Hg x Wg) grid in token order."""
    rng = _rng(seed)
    P = Hg * Wg
    N = F * P if n_tokens is None else n_tokens
    if N > F * P:
        raise ValueError(f"n_tokens={N} exceeds the {F} x {Hg} x {Wg} frame grid")
    out = np.empty((N, d), dtype=np.float64)
    fields = None
    for f in range(F):
        lo = f * P
        if lo >= N:
            break
        if scene_len is None:
            if fields is None:
                fields = _head_fields(rng, Hg, Wg, d, outlier_scale)
            fl = f
        else:
            if f % scene_len == 0:
                fields = _head_fields(rng, Hg, Wg, d, outlier_scale)
            fl = f % scene_len
        base, drift, _ = fields
        hi = min(N, lo + P)
        frame = base + 0.05 * fl * drift + 0.1 * rng.standard_normal((Hg, Wg, d))
        out[lo:hi] = frame.reshape(P, d)[: hi - lo]
    return out


def _head_rounded(args):
    seed, F, Hg, Wg, d, outlier_scale, scene_len, n_tokens, dtype = args
    return round_to(video_head(seed, F, Hg, Wg, d, outlier_scale, scene_len, n_tokens), dtype)


def video_cache(family: int, kind: int, heads: int, F: int, Hg: int, Wg: int, d: int,
                outlier_scale: float, dtype: torch.dtype, scene_len: int | None = None,
                n_tokens: int | None = None, head_ids=None, workers: int = 1) -> torch.Tensor:
    """[heads, N, d] CPU tensor; head h uses seed (1000 + 100*family + h, kind).
    `workers` > 1 draws the heads in that many processes (same values)."""
    ids = list(range(heads) if head_ids is None else head_ids)
    jobs = [(_seed(family, kind, h), F, Hg, Wg, d, outlier_scale, scene_len, n_tokens, dtype)
            for h in ids]
    if workers > 1 and len(jobs) > 1:
        import concurrent.futures as cf
        import multiprocessing as mp
        with cf.ProcessPoolExecutor(min(workers, len(jobs)),
                                    mp_context=mp.get_context("spawn")) as ex:
            hs = list(ex.map(_head_rounded, jobs))
    else:
        hs = [_head_rounded(j) for j in jobs]
    return torch.stack(hs)


def video_cache_device(family: int, kind: int, heads: int, Hg: int, Wg: int, d: int,
                       outlier_scale: float, n_tokens: int, scene_len: int, dtype: torch.dtype,
                       device) -> torch.Tensor:
    """The video-shaped recipe of video_head (base + 0.05*f*drift + N(0, 0.1^2)
    noise, 4 outlier channels of base scaled, base and drift re-drawn every
    scene_len frames) drawn on the device with torch's seeded generator, for
    caches too large to draw on the host quickly.  Same distribution as
    video_cache, different random streams.  Returns [heads, n_tokens, d]."""
    P = Hg * Wg
    F = -(-n_tokens // P)
    out = torch.empty((heads, F * P, d), dtype=dtype, device=device)
    for h in range(heads):
        g = torch.Generator(device=device)
        g.manual_seed(_seed(family, kind, h))
        for f0 in range(0, F, scene_len):
            base = torch.randn((P, d), generator=g, device=device)
            drift = torch.randn((P, d), generator=g, device=device)
            outl = torch.randperm(d, generator=g, device=device)[:4]
            base[:, outl] *= outlier_scale
            nf = min(scene_len, F - f0)
            fl = torch.arange(nf, device=device, dtype=torch.float32).view(nf, 1, 1)
            noise = torch.randn((nf, P, d), generator=g, device=device)
            frames = base + 0.05 * fl * drift + 0.1 * noise
            out[h, f0 * P:(f0 + nf) * P] = frames.reshape(nf * P, d).to(dtype)
    return out[:, :n_tokens].contiguous()


def _seed(family: int, kind: int, h: int) -> int:
    return (1000 + 100 * family + h) * 2 + kind


# ---------------------------------------------------------------- stream chunks
def stream_chunk(family: int, kind: int, heads: int, chunk: int, frames_per_chunk: int,
                 Hg: int, Wg: int, d: int, outlier_scale: float,
                 dtype: torch.dtype) -> torch.Tensor:
    """Chunk `chunk` of a continuing video: global frames
    [chunk*fpc, (chunk+1)*fpc); base and drift are fixed per head, so each
    chunk continues the previous chunk's drift."""
    P = Hg * Wg
    out = np.empty((heads, frames_per_chunk * P, d), dtype=np.float64)
    for h in range(heads):
        base, drift, _ = _head_fields(_rng(_seed(family, kind, h)), Hg, Wg, d, outlier_scale)
        rng = _rng(_seed(family, kind, h), chunk + 1)
        for j in range(frames_per_chunk):
            f = chunk * frames_per_chunk + j
            frame = base + 0.05 * f * drift + 0.1 * rng.standard_normal((Hg, Wg, d))
            out[h, j * P:(j + 1) * P] = frame.reshape(P, d)
    return round_to(out, dtype)


# ---------------------------------------------------------------- k-means init draws
def init_indices(seed: int, H: int, T: int, N: int, C: int) -> np.ndarray:
    """Seeded cold-start draw: for each (head, stage) C distinct token indices
    in [0, N), as int32 [H, T, C].  This is the random draw the method makes at
    k-means initialisation; it is an input to both implementations."""
    out = np.empty((H, max(T, 1), C), dtype=np.int32)
    for h in range(H):
        for t in range(max(T, 1)):
            out[h, t] = _rng(seed, h, t).choice(N, size=C, replace=False)
    return out[:, :T] if T > 0 else out[:, :0]


# ---------------------------------------------------------------- named workloads
CONFIGS = {
    # name: seed family, F, Hg, Wg, d, heads per kind, dtype, kinds, method
    # parameters (and scene_len, N, chunking where they apply)
    "tiny": dict(seed=0, F=16, Hg=16, Wg=16, d=64, heads=1, dtype=torch.float32, kinds=(K_KIND,),
            outlier={K_KIND: 50.0}, C=16, T=1, iters=10, bits=2, group=32),
    "self_forcing": dict(seed=1, F=21, Hg=30, Wg=52, d=128, heads=12, dtype=torch.bfloat16, kinds=(K_KIND, V_KIND),
            outlier=OUTLIER_SCALE, C=256, T=2, iters=8, bits=2, group=64),
    "stream": dict(seed=2, F=3, Hg=30, Wg=52, d=128, heads=12, dtype=torch.bfloat16, kinds=(K_KIND, V_KIND),
            outlier=OUTLIER_SCALE, C=256, T=2, iters=10, iters_warm=3, bits=2, group=64,
            chunks=20),
    "long_video": dict(seed=3, F=85, Hg=39, Wg=40, d=128, heads=32, dtype=torch.bfloat16, kinds=(K_KIND, V_KIND),
            outlier=OUTLIER_SCALE, C=256, T=4, iters=8, bits=2, group=64, scene_len=21,
            n_tokens=131072),
}


def config_cache(name: str, heads: int | None = None, n_tokens: int | None = None,
                 workers: int = 1) -> torch.Tensor:
    """All head-tensors of a configuration stacked K-then-V: [kinds*heads, N, d].
    `heads`/`n_tokens` give a smaller sample of the same workload."""
    c = CONFIGS[name]
    nh = c["heads"] if heads is None else heads
    N = c.get("n_tokens") if n_tokens is None else n_tokens
    parts = [video_cache(c["seed"], k, nh, c["F"], c["Hg"], c["Wg"], c["d"], c["outlier"][k],
                         c["dtype"], c.get("scene_len"), N, workers=workers)
             for k in c["kinds"]]
    return torch.cat(parts, 0)


# ---------------------------------------------------------------- decode-side record
def random_record(seed: int, H: int, N: int, d: int, T: int, C: int, bits: int, group: int,
                  Hg: int = 512, Wg: int = 512):
    """A pre-compressed record drawn directly from a seed (decode-only workload):
    uniform random code bytes; per-group FP8 scale bytes drawn uniformly from
    the E4M3 codes of small positive values; per-stage assignments that are
    spatially coherent (a hash of the 4x4 patch block and the stage); bf16
    centroids ~ N(0, 4^-t).  Tokens are laid out on an Hg x Wg grid (frames
    follow in token order).  Returns numpy/torch CPU arrays."""
    rng = _rng(seed)
    codes = rng.integers(0, 256, size=(H, N, d * bits // 8), dtype=np.uint8)
    # E4M3 bytes 0x18..0x3F cover roughly 0.02..1.9 (exponent field 3..7).
    scales = rng.integers(0x18, 0x40, size=(H, N, d // group), dtype=np.uint8)
    i = np.arange(N)
    y = (i // Wg) % Hg
    x = i % Wg
    assign = np.empty((H, T, N), dtype=np.uint8)
    for h in range(H):
        for t in range(T):
            salt = _rng(seed, h, t).integers(0, 2**31)
            key = (y // 4) * 1_000_003 + (x // 4) * 7919 + salt
            key = (key * 2654435761) % (2**32)
            assign[h, t] = ((key >> 8) % C).astype(np.uint8)
    cents = np.zeros((H, T, C, d))
    for h in range(H):
        for t in range(T):
            cents[h, t] = rng.standard_normal((C, d)) * (0.5 ** (t + 1))
    return codes, scales, assign, round_to(cents, torch.bfloat16)


# ---------------------------------------------------------------- attention inputs
def queries(seed: int, H: int, Nq: int, d: int) -> torch.Tensor:
    """Decode-step queries [H, Nq, d] fp32 ~ N(0, 1)."""
    return torch.from_numpy(_rng(seed, 7).standard_normal((H, Nq, d)).astype(np.float32))


def rope_tables(N: int, d: int, base: float = 10000.0, start: int = 0):
    """Rotary-embedding tables of token positions start..start+N-1, rotate-half
    convention: angle(i, k) = i * base^(-2k/d) for k < d/2, evaluated in
    float64 and rounded to fp32.  Returns (cos, sin), each [N, d/2] fp32."""
    pos = np.arange(start, start + N, dtype=np.float64)[:, None]
    inv = base ** (-2.0 * np.arange(d // 2, dtype=np.float64) / d)
    ang = pos * inv[None, :]
    return (torch.from_numpy(np.cos(ang).astype(np.float32)),
            torch.from_numpy(np.sin(ang).astype(np.float32)))
