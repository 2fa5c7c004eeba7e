"""Seeded synthetic inputs shaped like the pages' workloads.

This module holds none of the method's arithmetic: it only draws random
gradients and weights (torch's generators, CPU or GPU) and lays them out in
the canonical tensor order of the models the pages train:

* Llama-2-style models ("Merge LoCo with Zero++", Experimental Results: a
  0.8B and an 8B Llama2-architecture model) -- the ~0.85B shape (14 layers,
  hidden 2048, FFN 5632, vocab 32000) and the ~7.5B shape (36 layers, hidden
  4096, FFN 11008, vocab 32000), untied input embedding and lm_head.
* GPT-2 124M ("Zero 2 #593": llm.c's GPT-2 training) -- 12 layers, width 768,
  vocab 50257, 1024 positions.

No dataset or trained weight is used: real gradients come from training on
RedPajama-V2 (LoCo) or FineWeb-style text (llm.c); seeded normal draws of the
stated scales stand in for them.  Heavy-tailed tensors (embedding, lm_head
and every tensor of the first and last transformer block) are Student-t with
3 degrees of freedom scaled to the same standard deviation.

Seeds: every stream is named by a tuple (config, role, rank, step,
micro-batch); ``seed_for`` hashes it with base seed 0 into a 63-bit seed.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass

import torch

BASE_SEED = 0


def seed_for(config: str, role: str, rank: int = 0, step: int = 0, mb: int = 0) -> int:
    tag = f"{BASE_SEED}|{config}|{role}|{rank}|{step}|{mb}".encode()
    return int.from_bytes(hashlib.sha256(tag).digest()[:8], "little") & ((1 << 63) - 1)


@dataclass(frozen=True)
class Tensor:
    name: str
    numel: int
    heavy: bool  # drawn heavy-tailed in the gradient recipe


def llama_tensors(layers: int, hidden: int, ffn: int, vocab: int) -> list[Tensor]:
    """Canonical flat order: embed, per layer (attn_norm, q, k, v, o,
    ffn_norm, gate, up, down), final_norm, lm_head."""
    h, f, V = hidden, ffn, vocab
    out = [Tensor("embed", V * h, True)]
    for l in range(layers):
        heavy = l == 0 or l == layers - 1
        out += [
            Tensor(f"l{l}.attn_norm", h, heavy),
            Tensor(f"l{l}.q", h * h, heavy),
            Tensor(f"l{l}.k", h * h, heavy),
            Tensor(f"l{l}.v", h * h, heavy),
            Tensor(f"l{l}.o", h * h, heavy),
            Tensor(f"l{l}.ffn_norm", h, heavy),
            Tensor(f"l{l}.gate", f * h, heavy),
            Tensor(f"l{l}.up", f * h, heavy),
            Tensor(f"l{l}.down", h * f, heavy),
        ]
    out += [Tensor("final_norm", h, False), Tensor("lm_head", V * h, True)]
    return out


def llama_0p85b() -> list[Tensor]:
    return llama_tensors(14, 2048, 5632, 32000)


def llama_7p5b() -> list[Tensor]:
    return llama_tensors(36, 4096, 11008, 32000)


def gpt2_124m() -> list[Tensor]:
    C, V, T, L = 768, 50257, 1024, 12
    out = [Tensor("wte", V * C, False), Tensor("wpe", T * C, False)]
    for l in range(L):
        out += [
            Tensor(f"l{l}.ln1w", C, False), Tensor(f"l{l}.ln1b", C, False),
            Tensor(f"l{l}.qkvw", 3 * C * C, False), Tensor(f"l{l}.qkvb", 3 * C, False),
            Tensor(f"l{l}.attprojw", C * C, False), Tensor(f"l{l}.attprojb", C, False),
            Tensor(f"l{l}.ln2w", C, False), Tensor(f"l{l}.ln2b", C, False),
            Tensor(f"l{l}.fcw", 4 * C * C, False), Tensor(f"l{l}.fcb", 4 * C, False),
            Tensor(f"l{l}.fcprojw", 4 * C * C, False), Tensor(f"l{l}.fcprojb", C, False),
        ]
    out += [Tensor("lnfw", C, False), Tensor("lnfb", C, False)]
    return out


def total(tensors: list[Tensor]) -> int:
    return sum(t.numel for t in tensors)


def _gen(device: torch.device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _fill_normal(out: torch.Tensor, std: float, gen: torch.Generator, heavy: bool) -> None:
    """out (fp32, contiguous) <- N(0, std^2), or std * t_3 / sqrt(3) when heavy."""
    if not heavy:
        torch.randn(out.shape, generator=gen, device=out.device, dtype=torch.float32, out=out)
        out.mul_(std)
        return
    torch.randn(out.shape, generator=gen, device=out.device, dtype=torch.float32, out=out)
    chi2 = torch.zeros_like(out)
    tmp = torch.empty_like(out)
    for _ in range(3):
        torch.randn(out.shape, generator=gen, device=out.device, dtype=torch.float32, out=tmp)
        chi2.addcmul_(tmp, tmp)
    del tmp
    out.div_(chi2.div_(3.0).sqrt_())
    out.mul_(std / math.sqrt(3.0))


def fill_model(out: torch.Tensor, tensors: list[Tensor] | None, std: float, seed: int,
               heavy_tails: bool = False, slab: int = 1 << 27) -> None:
    """Fill a flat buffer (fp32, bf16 or fp16) in place with a gradient/weight of
    the given tensor table.  Values are drawn in fp32 slab by slab and cast to
    the buffer's dtype with torch's round-to-nearest-even conversion."""
    n = out.numel()
    if tensors is None:
        tensors = [Tensor("flat", n, False)]
    assert total(tensors) == n, (total(tensors), n)
    gen = _gen(out.device, seed)
    off = 0
    stage = None
    for t in tensors:
        heavy = heavy_tails and t.heavy
        done = 0
        while done < t.numel:
            m = min(slab, t.numel - done)
            dst = out[off + done: off + done + m]
            if out.dtype == torch.float32:
                _fill_normal(dst, std, gen, heavy)
            else:
                if stage is None or stage.numel() < m:
                    stage = torch.empty(min(slab, max(m, 1)), dtype=torch.float32, device=out.device)
                s = stage[:m]
                _fill_normal(s, std, gen, heavy)
                dst.copy_(s)
            done += m
        off += t.numel


def grad_with_outliers(n: int, std: float, p_outlier: float, mult: float, seed: int,
                       dtype: torch.dtype, device="cpu") -> torch.Tensor:
    """N(0, std^2) with Bernoulli(p_outlier) elements multiplied by mult,
    drawn in fp32 and cast (round to nearest even) to dtype."""
    gen = _gen(torch.device(device), seed)
    x = torch.randn(n, generator=gen, device=device, dtype=torch.float32).mul_(std)
    mask = torch.rand(n, generator=gen, device=device, dtype=torch.float32) < p_outlier
    x = torch.where(mask, x * mult, x)
    return x.to(dtype)


def normal(n: int, std: float, seed: int, dtype: torch.dtype, device="cpu") -> torch.Tensor:
    gen = _gen(torch.device(device), seed)
    return torch.randn(n, generator=gen, device=device, dtype=torch.float32).mul_(std).to(dtype)


def bf16_bits(t: torch.Tensor):
    """Host numpy uint16 view of a bf16 tensor's bit patterns."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")


def from_bf16_bits(a, device="cpu") -> torch.Tensor:
    import numpy as np
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
