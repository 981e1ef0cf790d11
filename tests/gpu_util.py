"""Shared helpers for the GPU parity tests (HIP path vs CPU oracle)."""
import sys

import numpy as np
import torch

DEV = torch.device("cuda:0")


def say(*a):
    """Print and flush what names the case before each GPU step."""
    print(*a, flush=True)
    sys.stdout.flush()


def bits16(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> uint16 bit patterns (numpy)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def to_oracle(x: torch.Tensor) -> np.ndarray:
    """CPU/GPU tensor -> the oracle's storage (fp32 array or bf16 bit patterns)."""
    if x.dtype == torch.bfloat16:
        return bits16(x)
    return x.detach().cpu().numpy()


def as_f32(x: torch.Tensor) -> np.ndarray:
    return x.detach().float().cpu().numpy()


def rec_equal(rec, ref):
    """Compare a device Record with an oracle record dict; return list of mismatching fields."""
    bad = []
    for k, g in (("codes", rec.codes), ("scales", rec.scales), ("assign", rec.assign)):
        if not np.array_equal(g.cpu().numpy(), ref[k]):
            bad.append(k)
    c = rec.centroids
    gc = bits16(c) if c.dtype == torch.bfloat16 else c.cpu().numpy()
    if not np.array_equal(gc, ref["cent"]):
        bad.append("cent")
    return bad


def mismatch_report(a: np.ndarray, b: np.ndarray) -> str:
    a = np.asarray(a)
    b = np.asarray(b)
    if a.shape != b.shape:
        return f"shape {a.shape} vs {b.shape}"
    diff = np.nonzero(a.reshape(-1) != b.reshape(-1))[0]
    fa, fb = a.reshape(-1), b.reshape(-1)
    pairs = [(int(i), fa[i].item(), fb[i].item()) for i in diff[:8]]
    return f"{len(diff)} / {a.size} differ; (flat index, got, want): {pairs}"
