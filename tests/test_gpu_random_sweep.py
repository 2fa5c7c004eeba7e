"""GPU parity on seeded random configurations: sizes drawn around multiples
of every tile length the kernels use (256, 512, 1024, 2048 elements and the
block itself) plus small offsets, random block sizes, dtypes, peer counts,
flags and coefficients.  Each case is checked against the oracle with the
same bit-exact contract as the fixed-grid parity tests."""
import numpy as np
import pytest
import torch

import oracle as O
from tests.gpu_helpers import (Guarded, as_dtype, assert_bits_equal, grad_values,
                               to_gpu, to_host)
from tests.test_gpu_parity import BLOCKS, Z, check_dr, check_efq, sr_inputs

pytestmark = pytest.mark.gpu

TILES = [256, 512, 1024, 2048]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_communication_zero_amd  # noqa: F401  (fails loudly if libzq.so is missing)
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _size(rng, block):
    m = int(rng.choice(TILES + [block]))
    return max(1, int(rng.integers(1, 10)) * m + int(rng.choice([-3, -1, 0, 1, 5])))


DTYPES = ["fp32", "bf16", "fp16"]


@pytest.mark.parametrize("case", range(64))
def test_efq_random_configs(case):
    rng = np.random.default_rng(1000 + case)
    block = int(rng.choice(BLOCKS))
    n = _size(rng, block)
    gdt = DTYPES[int(rng.integers(0, 3))]
    with_ef = bool(rng.integers(0, 2))
    be, br = [(0.9, 1.0), (1.0, 1.0), (0.0, 1.0), (0.75, 0.25)][int(rng.integers(0, 4))]
    x = grad_values(n, seed=2000 + case, std=10.0 ** rng.uniform(-5, -1), special=True,
                    block=block)
    g = as_dtype(x, gdt, seed=case)
    ef = grad_values(n, seed=3000 + case, std=1e-5) if with_ef else None
    check_efq(g, ef, block, be, br,
              f"random efq case={case} n={n} B={block} {gdt} ef={with_ef} beta=({be},{br})")


@pytest.mark.parametrize("case", range(64))
def test_dequant_reduce_random_configs(case):
    rng = np.random.default_rng(4000 + case)
    block = int(rng.choice(BLOCKS))
    P = int(rng.integers(1, 17))
    n = block * int(rng.integers(1, 12)) * int(rng.choice([1, 2, 3]))
    flags = [(True, False, False), (False, True, False), (False, True, True),
             (True, True, False), (True, True, True)][int(rng.integers(0, 5))]
    alpha = float(rng.choice([1.0, 0.5, 1.0 / P, 0.3]))
    raw = bool(rng.integers(0, 2))
    check_dr(P, n, block, alpha, *flags, seed=5000 + case, raw=raw)


@pytest.mark.parametrize("case", range(32))
def test_int8_random_configs(case):
    rng = np.random.default_rng(6000 + case)
    block = int(rng.choice(BLOCKS))
    n = _size(rng, block)
    wdt = DTYPES[int(rng.integers(0, 3))]
    x = grad_values(n, seed=7000 + case, std=10.0 ** rng.uniform(-3, 0), special=True,
                    block=block)
    w = as_dtype(x, wdt, seed=case)
    c_o, s_o = O.quant_int8(w, block)
    codes = Guarded(n, torch.int8)
    scales = Guarded(-(-n // block), torch.float32)
    Z().zq_quant_int8(to_gpu(w), block, codes.t, scales.t)
    torch.cuda.synchronize()
    what = f"random int8 case={case} n={n} B={block} {wdt}"
    assert_bits_equal(codes.host().view(np.uint8), c_o.view(np.uint8), what + " codes")
    assert_bits_equal(scales.host(), s_o, what + " scales")
    odt = DTYPES[int(rng.integers(0, 3))]
    o_o = O.dequant_int8(c_o, s_o, block, out_bf16=odt == "bf16", out_f16=odt == "fp16")
    out = Guarded(n, {"fp32": torch.float32, "bf16": torch.bfloat16, "fp16": torch.float16}[odt])
    Z().zq_dequant_int8(to_gpu(c_o), to_gpu(s_o), block, out.t)
    torch.cuda.synchronize()
    assert_bits_equal(out.host(), o_o, what + f" dequant to {odt}")


@pytest.mark.parametrize("case", range(32))
def test_sr_random_configs(case):
    rng = np.random.default_rng(8000 + case)
    n = _size(rng, 1024)
    zero_src = bool(rng.integers(0, 2))
    seed = int(rng.integers(0, 1 << 63))
    cb = int(rng.integers(0, 1 << 40))
    d, s = sr_inputs(n, seed=9000 + case, special=True)
    d_o, s_o = d.copy(), s.copy()
    O.sr_accumulate(d_o, s_o, seed, cb, zero_src)
    dg, sg = to_gpu(d), to_gpu(s)
    Z().zq_sr_accumulate(dg, sg, seed, cb, zero_src)
    torch.cuda.synchronize()
    what = f"random sr case={case} n={n} cb={cb} zero={zero_src}"
    assert_bits_equal(to_host(dg), d_o, what + " dst")
    assert_bits_equal(to_host(sg), s_o, what + " src")
