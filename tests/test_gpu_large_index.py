"""Buffers past 2^32 elements: every index, block number and Philox counter
of the streaming kernels is 64-bit, so the blocks and windows on both sides
of element 2^31 and 2^32 must come out exactly as the oracle computes them,
and every output element must be written.

qwZ int8 quantize and dequantize ("ZeROPlusPlus.md" notes, section 1.2) on
2^32 + 6,221 bf16 weights (a partial last block of 77), and llm.c's SR
accumulate ("Zero 2 #593", review of llmc/cuda_utils.cuh) on 2^32 + 3,405
bf16 elements (a ragged last tile).  About 30 GB of device memory at most."""
import numpy as np
import pytest
import torch

import oracle as O
from tests.gpu_helpers import assert_bits_equal, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_communication_zero_amd  # noqa: F401  (fails loudly if libzq.so is missing)
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def Z():
    from weight_communication_zero_amd import zq
    return zq


CHUNK = 1 << 28


def fill_normal(t: torch.Tensor, std: float, seed: int) -> None:
    """Seeded N(0, std) in fp32, rounded to t's dtype, one chunk at a time."""
    g = torch.Generator(device="cuda").manual_seed(seed)
    for a in range(0, t.numel(), CHUNK):
        b = min(a + CHUNK, t.numel())
        t[a:b] = torch.randn(b - a, device="cuda", generator=g).mul_(std)


def test_int8_past_2_pow_32_elements():
    B = 2048
    n = (1 << 32) + 3 * B + 77
    nb = -(-n // B)
    w = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    fill_normal(w, 0.02, seed=41)
    codes = torch.full((n,), -128, dtype=torch.int8, device="cuda")  # never a code
    scales = torch.full((nb,), float("nan"), device="cuda")
    wd = torch.full((n,), float("nan"), dtype=torch.bfloat16, device="cuda")
    Z().zq_quant_int8(w, B, codes, scales)
    Z().zq_dequant_int8(codes, scales, B, wd)
    torch.cuda.synchronize()
    assert not bool((codes == -128).any()), "int8 codes left unwritten"
    assert not bool(torch.isnan(scales).any()), "int8 scales left unwritten"
    assert not bool(torch.isnan(wd).any()), "dequantized weights left unwritten"

    def edge_blocks(i):
        return [i // B - 1, i // B, i // B + 1]
    rng = np.random.default_rng(42)
    blocks = [0, 1, nb - 2, nb - 1] + edge_blocks(1 << 31) + edge_blocks(1 << 32)
    blocks = sorted(set(blocks) | set(int(x) for x in rng.integers(0, nb, size=120)))
    s_all = to_host(scales)
    for b in blocks:
        a, e = b * B, min((b + 1) * B, n)
        c_o, s_o = O.quant_int8(to_host(w[a:e]), B)
        what = f"int8 block {b} (elements {a}..{e})"
        assert_bits_equal(to_host(codes[a:e]).view(np.uint8), c_o.view(np.uint8), what + " codes")
        assert_bits_equal(s_all[b:b + 1], s_o, what + " scale")
        assert_bits_equal(to_host(wd[a:e]), O.dequant_int8(c_o, s_o, B, out_bf16=True),
                          what + " dequantized")


def test_sr_past_2_pow_32_elements():
    n = (1 << 32) + 3 * 1024 + 333
    src = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    fill_normal(src, 1.0, seed=43)
    dst = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    # dst = 0: every sum is a bf16 value, so every output equals its src
    Z().zq_sr_accumulate(dst, src, seed=5, counter_base=0)
    torch.cuda.synchronize()
    for a in range(0, n, CHUNK):
        b = min(a + CHUNK, n)
        assert torch.equal(dst[a:b].view(torch.int16), src[a:b].view(torch.int16)), \
            f"an element of [{a}, {b}) was missed or misplaced"
    # a second accumulation that rounds: oracle windows at the edges
    W = 1024
    rng = np.random.default_rng(44)
    starts = [0, n - W, (1 << 31) - W, 1 << 31, (1 << 32) - W, 1 << 32]
    starts = sorted(set(starts) | set(int(x) for x in rng.integers(0, n - W, size=24)))
    fill_normal(src, 1e-2, seed=45)
    win_d = {s0: to_host(dst[s0:s0 + W]).copy() for s0 in starts}
    win_s = {s0: to_host(src[s0:s0 + W]).copy() for s0 in starts}
    seed, cbase = (1 << 33) + 3, 11
    Z().zq_sr_accumulate(dst, src, seed=seed, counter_base=cbase, zero_src=True)
    torch.cuda.synchronize()
    for s0 in starts:
        O.sr_accumulate(win_d[s0], win_s[s0], seed=seed, counter_base=cbase + s0)
        assert_bits_equal(to_host(dst[s0:s0 + W]), win_d[s0], f"SR window at {s0}")
    for a in range(0, n, CHUNK):
        b = min(a + CHUNK, n)
        assert int(torch.count_nonzero(src[a:b].view(torch.int16))) == 0, \
            f"zero_src left elements of [{a}, {b})"
