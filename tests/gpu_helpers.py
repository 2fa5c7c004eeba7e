"""Shared helpers of the GPU parity tests: seeded host inputs (with the edge
values the method has), upload/download, poisoned outputs with guard bands,
and bitwise comparisons.  The expected values always come from the CPU
oracle on the same host inputs."""
from __future__ import annotations

import numpy as np
import torch

GUARD = 64  # elements of canary after every GPU output
POISON_U8 = 0xAA


def dev():
    return torch.device("cuda", 0)


def to_gpu(a: np.ndarray) -> torch.Tensor:
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev())
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class Guarded:
    """A GPU output buffer of n elements followed by GUARD canary elements,
    everything pre-filled with a poison value."""

    def __init__(self, n: int, dtype: torch.dtype):
        self.n = n
        if dtype in (torch.uint8, torch.int8):
            self.buf = torch.full((n + GUARD,), POISON_U8 if dtype == torch.uint8 else -86,
                                  dtype=dtype, device=dev())
        elif dtype == torch.bfloat16:
            self.buf = torch.full((n + GUARD,), float("nan"), dtype=dtype, device=dev())
        else:
            self.buf = torch.full((n + GUARD,), float("nan"), dtype=dtype, device=dev())
        self.canary = to_host(self.buf[n:]).copy()

    @property
    def t(self) -> torch.Tensor:
        return self.buf[: self.n]

    def host(self) -> np.ndarray:
        tail = to_host(self.buf[self.n:])
        assert tail.tobytes() == self.canary.tobytes(), "write past the end of an output buffer"
        return to_host(self.t)


def bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a.view(np.uint32)
    if a.dtype == np.float16:
        return a.view(np.uint16)
    return a


def assert_bits_equal(got: np.ndarray, exp: np.ndarray, what: str):
    g, e = bits(got), bits(exp)
    assert g.shape == e.shape, (what, g.shape, e.shape)
    bad = np.nonzero(g != e)[0]
    if bad.size:
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} of {g.size} differ; first at {i}: "
                             f"got {got[i]!r} ({g[i]:#x}) expected {exp[i]!r} ({e[i]:#x})")


def grad_values(n: int, seed: int, std: float = 1e-3, outlier_p: float = 0.01,
                outlier_mult: float = 50.0, special: bool = False, block: int = 128) -> np.ndarray:
    """fp32 gradient-like values; with `special`, some blocks are replaced by
    edge cases: all zeros, signed zeros, subnormals, exact half-integer ties
    on a power-of-two scale, one huge value, one tiny value among zeros."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(n) * std).astype(np.float32)
    x[rng.random(n) < outlier_p] *= np.float32(outlier_mult)
    if special and n >= 1:
        nb = -(-n // block)
        kinds = rng.integers(0, 7, size=nb)
        for b in range(nb):
            if rng.random() > 0.3:
                continue
            lo, hi = b * block, min(n, (b + 1) * block)
            m = hi - lo
            k = kinds[b]
            if k == 0:
                x[lo:hi] = 0.0
            elif k == 1:
                x[lo:hi] = -0.0
            elif k == 2:
                x[lo:hi] = (rng.integers(-300, 301, size=m) * np.float32(1e-42)).astype(np.float32)
            elif k == 3:
                e = float(2.0 ** int(rng.integers(-20, 4)))
                x[lo:hi] = (rng.integers(-14, 15, size=m) / 2.0 * e).astype(np.float32)
                x[lo + int(rng.integers(0, m))] = np.float32(7 * e)
            elif k == 4:
                x[lo:hi] = (rng.integers(-254, 255, size=m) / 2.0 * 2.0 ** -9).astype(np.float32)
                x[lo] = np.float32(127 * 2.0 ** -9)
            elif k == 5:
                x[lo + int(rng.integers(0, m))] = np.float32(1e30)
            else:
                x[lo:hi] = 0.0
                x[lo + int(rng.integers(0, m))] = np.float32(3e-45)
    return x


def as_bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def as_f16(x: np.ndarray, seed: int = 0) -> np.ndarray:
    """fp16 inputs from fp32 values: clipped to the finite fp16 range (inputs
    are expected finite), rounded to nearest even, with a few fp16-specific
    values planted: subnormals, the largest finite value and signed zeros."""
    h = np.clip(x, -60000.0, 60000.0).astype(np.float16)
    if h.size >= 8:
        rng = np.random.default_rng(seed)
        idx = rng.choice(h.size, size=min(h.size, 16), replace=False)
        sub = np.array([6e-8, -6e-8, 3e-5, -1.2e-7, 65504.0, -0.0, 0.0, 6.1e-5], np.float16)
        h[idx] = sub[np.arange(idx.size) % sub.size]
    return h


def as_dtype(x: np.ndarray, dt: str, seed: int = 0) -> np.ndarray:
    """fp32 values as the host form of dtype dt: float32, bf16 bits or fp16."""
    if dt == "bf16":
        return as_bf16_bits(x)
    if dt == "fp16":
        return as_f16(x, seed)
    return x


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (h.astype(np.uint32) << 16).view(np.float32)
