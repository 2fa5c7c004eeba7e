"""GPU parity: libzq's HIP kernels (through the C ABI) against the CPU oracle,
element by element on the same seeded inputs, at sizes that span several
wave tiles and a ragged tail, for every block size and input dtype, with the
edge cases of the method (zero / signed-zero / subnormal / tie / huge blocks,
odd n, n = 1, P = 1 and P = 16, every Philox counter phase, NaN / Inf in
stochastic rounding).  Contract: integer codes, scales (as bits), EF buffers,
requant codes and bf16 outputs bit-exact; fp32 reduced sums within 1e-6
relative of the oracle (guarded by the sum of magnitudes) -- and, as the op
order is fixed, expected bit-exact too.
"""
import numpy as np
import pytest
import torch

import oracle as O
from tests.gpu_helpers import (Guarded, as_bf16_bits, as_dtype, assert_bits_equal, bf16_to_f32,
                               grad_values, to_gpu, to_host)

pytestmark = pytest.mark.gpu

BLOCKS = [32, 64, 128, 256, 512, 1024, 2048, 4096]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_communication_zero_amd  # noqa: F401  (fails loudly if libzq.so is missing)
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def Z():
    from weight_communication_zero_amd import zq
    return zq


def sizes_for(block, vec_tile):
    tile = max(vec_tile, block)
    return [1, 3, block - 1, block + 1, tile + 5, 3 * tile + block // 2 + 3, 5 * tile]


# ------------------------------------------------------- EF int4 quantize --

def run_efq_gpu(g_host, ef_host, block, be, br):
    n = g_host.size
    g = to_gpu(g_host)
    ef = to_gpu(ef_host) if ef_host is not None else None
    codes = Guarded((n + 1) // 2, torch.uint8)
    scales = Guarded(-(-n // block), torch.float32)
    Z().zq_quantize_ef_int4(g, ef, block, be, br, codes.t, scales.t)
    torch.cuda.synchronize()
    return codes.host(), scales.host(), (to_host(ef) if ef is not None else None)


def check_efq(g_host, ef_host, block, be, br, what):
    ef_o = ef_host.copy() if ef_host is not None else None
    c_o, s_o = O.quantize_ef_int4(g_host, ef_o, block, be, br)
    c_g, s_g, ef_g = run_efq_gpu(g_host, ef_host.copy() if ef_host is not None else None, block,
                                 be, br)
    assert_bits_equal(c_g, c_o, f"{what} codes")
    assert_bits_equal(s_g, s_o, f"{what} scales")
    if ef_host is not None:
        assert_bits_equal(ef_g, ef_o, f"{what} ef")


@pytest.mark.parametrize("block", BLOCKS)
@pytest.mark.parametrize("gdt", ["fp32", "bf16", "fp16"])
@pytest.mark.parametrize("with_ef", [False, True])
def test_efq_matches_oracle(block, gdt, with_ef):
    for i, n in enumerate(sizes_for(block, 1024)):
        x = grad_values(n, seed=1000 * block + i, special=True, block=block)
        g = as_dtype(x, gdt, seed=i)
        ef = (grad_values(n, seed=7 + i, std=1e-5) if with_ef else None)
        check_efq(g, ef, block, 0.9, 1.0, f"efq n={n} B={block} {gdt} ef={with_ef}")


@pytest.mark.parametrize("betas", [(1.0, 1.0), (0.0, 1.0), (0.9, 0.1), (0.0, 0.9)])
def test_efq_beta_variants_multistep(betas):
    n, block = 3 * 4096 + 77, 128
    ef_o = np.zeros(n, np.float32)
    ef_g = torch.zeros(n, dtype=torch.float32, device="cuda")
    for step in range(3):
        g = grad_values(n, seed=50 + step, special=(step == 1))
        c_o, s_o = O.quantize_ef_int4(g, ef_o, block, *betas)
        codes = Guarded((n + 1) // 2, torch.uint8)
        scales = Guarded(-(-n // block), torch.float32)
        Z().zq_quantize_ef_int4(to_gpu(g), ef_g, block, betas[0], betas[1], codes.t, scales.t)
        torch.cuda.synchronize()
        assert_bits_equal(codes.host(), c_o, f"codes step {step}")
        assert_bits_equal(scales.host(), s_o, f"scales step {step}")
        assert_bits_equal(to_host(ef_g), ef_o, f"ef step {step}")


def test_efq_random_ties_band():
    """Values that sit exactly on, and within an ulp or two of, the rounding
    boundaries k + 1/2 of their block -- the inputs where the kernel's
    reciprocal fast path must hand over to the IEEE quotient."""
    rng = np.random.default_rng(3)
    block, nb = 128, 512
    out = []
    for b in range(nb):
        s = np.float32(2.0 ** rng.integers(-30, 30) * rng.uniform(1, 2))
        ks = rng.integers(-7, 7, size=block) + 0.5
        x = (ks * s).astype(np.float32)
        d = rng.integers(-1, 2, size=block)
        target = np.where(d < 0, -np.inf, np.where(d > 0, np.inf, x)).astype(np.float32)
        x = np.nextafter(x, target)
        x[0] = np.float32(7) * s  # absmax 7s: scale s (or its rounding)
        out.append(x.astype(np.float32))
    g = np.concatenate(out)
    check_efq(g, None, block, 0.0, 1.0, "tie band int4")
    check_efq(g, np.zeros_like(g), block, 0.0, 1.0, "tie band int4 with ef")


def test_efq_n_zero_is_noop():
    zq = Z()
    codes = torch.full((4,), 0xAA, dtype=torch.uint8, device="cuda")
    zq.zq_quantize_ef_int4(torch.zeros(0, device="cuda"), None, 128, 1.0, 1.0, codes,
                           torch.zeros(1, device="cuda"))
    torch.cuda.synchronize()
    assert (codes.cpu() == 0xAA).all()


def test_error_enqueues_nothing():
    zq = Z()
    n = 4096
    codes = torch.full((n // 2,), 0xAA, dtype=torch.uint8, device="cuda")
    scales = torch.full((n // 128,), 7.0, device="cuda")
    g = torch.ones(n, device="cuda")
    st = zq.lib.zq_quantize_ef_int4(g.data_ptr(), 0, None, n, 100, 1.0, 1.0, codes.data_ptr(),
                                    scales.data_ptr(), None)
    assert st == zq.ZQ_ERR_BLOCK
    st = zq.lib.zq_quantize_ef_int4(g.data_ptr(), 0, g.data_ptr(), n, 128, 1.0, 1.0,
                                    codes.data_ptr(), scales.data_ptr(), None)
    assert st == zq.ZQ_ERR_ALIAS
    torch.cuda.synchronize()
    assert (codes.cpu() == 0xAA).all() and (scales.cpu() == 7.0).all()


# ---------------------------------------------------- dequantize + reduce --

def make_chunks(P, n, block, seed, raw=False):
    """P int4 chunks: quantized random gradients (as a sender would make
    them), or raw random nibbles (-8 included) with random scales."""
    rng = np.random.default_rng(seed)
    codes, scales = [], []
    for p in range(P):
        if raw:
            c = rng.integers(0, 256, size=(n + 1) // 2, dtype=np.uint8)
            if n % 2:
                c[-1] &= 0x0F
            s = (rng.standard_normal(-(-n // block)) * 1e-4).astype(np.float32)
            s[rng.random(s.size) < 0.05] = 0.0
            s[rng.random(s.size) < 0.02] = np.float32(1e-41)
        else:
            x = grad_values(n, seed=seed * 31 + p, std=10.0 ** rng.uniform(-5, -2),
                            special=True, block=block)
            c, s = O.quantize_ef_int4(x, None, block, 0.0, 1.0)
        codes.append(c)
        scales.append(s)
    return codes, scales


def check_dr(P, n, block, alpha, want_out, requant, with_rq_ef, seed, raw=False, chunks=None):
    codes, scales = chunks if chunks is not None else make_chunks(P, n, block, seed, raw=raw)
    rq_ef_host = grad_values(n, seed=seed + 99, std=1e-6) if with_rq_ef else None
    rq_ef_o = rq_ef_host.copy() if with_rq_ef else None
    out_o, rqc_o, rqs_o = O.dequant_reduce(codes, scales, n, block, alpha, want_out=want_out,
                                           requant=requant, rq_ef=rq_ef_o, rq_beta_e=0.9,
                                           rq_beta_r=1.0)
    cg = [to_gpu(c) for c in codes]
    sg = [to_gpu(s) for s in scales]
    out = Guarded(n, torch.float32) if want_out else None
    rqc = Guarded((n + 1) // 2, torch.uint8) if requant else None
    rqs = Guarded(-(-n // block), torch.float32) if requant else None
    rq_ef = to_gpu(rq_ef_host) if with_rq_ef else None
    Z().zq_dequant_reduce(cg, sg, n, block, alpha, out=out.t if out else None,
                          rq_codes=rqc.t if rqc else None, rq_scales=rqs.t if rqs else None,
                          rq_ef=rq_ef, rq_beta_e=0.9, rq_beta_r=1.0)
    torch.cuda.synchronize()
    what = f"dr P={P} n={n} B={block} a={alpha} out={want_out} rq={requant} rqef={with_rq_ef}"
    if want_out:
        got = out.host()
        # contract: 1e-6 relative, guarded by the sum of |d_p|
        mag = np.zeros(n, np.float64)
        for c, s in zip(codes, scales):
            k = np.empty(2 * c.size, np.int16)
            k[0::2], k[1::2] = c & 0x0F, c >> 4
            k = np.where(k >= 8, k - 16, k)[:n]
            mag += np.abs(k.astype(np.float64) * np.repeat(s.astype(np.float64), block)[:n])
        tol = 1e-6 * np.maximum(np.abs(out_o.astype(np.float64)), abs(alpha) * mag)
        assert (np.abs(got.astype(np.float64) - out_o) <= tol).all(), what
        assert_bits_equal(got, out_o, what + " out")
    if requant:
        assert_bits_equal(rqc.host(), rqc_o, what + " rq_codes")
        assert_bits_equal(rqs.host(), rqs_o, what + " rq_scales")
    if with_rq_ef:
        assert_bits_equal(to_host(rq_ef), rq_ef_o, what + " rq_ef")


@pytest.mark.parametrize("block", BLOCKS)
@pytest.mark.parametrize("P", [1, 2, 3, 4, 8, 13, 16])
def test_dequant_reduce_out(block, P):
    for i, n in enumerate([block, max(1024, block) * 3 + block // 2 + 1, max(1024, block) * 4]):
        check_dr(P, n, block, 1.0 / 8 if P > 1 else 1.0, True, False, False, seed=block * P + i)


@pytest.mark.parametrize("block", BLOCKS)
@pytest.mark.parametrize("flags", [(True, True, False), (False, True, False), (False, True, True),
                                   (True, True, True)])
def test_dequant_reduce_requant(block, flags):
    want_out, requant, rqef = flags
    for i, (P, n) in enumerate([(8, max(1024, block) * 3 + 17), (4, max(1024, block) * 2),
                                (1, 2 * block - 1)]):
        check_dr(P, n, block, 1.0, want_out, requant, rqef, seed=7 * block + i)


@pytest.mark.parametrize("block", [64, 4096])
@pytest.mark.parametrize("with_rq_ef", [False, True])
@pytest.mark.parametrize("P", range(1, 17))
def test_requant_every_peer_count(block, with_rq_ef, P):
    """The requant flavours for every peer count 1..16: the kernels are
    compiled for at most 2, 4, 8 and 16 peers and skip the unused ones at
    run time, so each count exercises a different number of live peers in
    its instantiation.  Blocks inside one sub-vector (64) and spanning
    several (4096); a ragged last tile; quantized gradients, not raw."""
    n = max(1024, block) * 3 + 17
    check_dr(P, n, block, 1.0 / P, False, True, with_rq_ef, seed=90 * P + block + with_rq_ef)


@pytest.mark.parametrize("alpha", [1.0, 0.25, 1.0 / 3.0, -2.0])
def test_dequant_reduce_alpha_and_raw_codes(alpha):
    check_dr(6, 4096 * 3 + 5, 128, alpha, True, True, True, seed=11, raw=True)
    check_dr(16, 2048 + 1, 64, alpha, True, True, False, seed=12, raw=True)


def extreme_scale_chunks(P, n, block, seed, top):
    """Raw nibbles (-8 included unless the scales reach 2^120) with positive
    scales log-uniform from the smallest subnormal up to 2^top, and blocks
    with the scales +0, -0, a negative value and the smallest subnormal (and
    for top > 120 also 2^125 and the float just below it).  A zero scale
    with a negative code gives -0, which the sums must keep."""
    rng = np.random.default_rng(seed)
    nb = -(-n // block)
    per_tile = 1024 // block if block <= 1024 else 1
    codes, scales = [], []
    for p in range(P):
        c = rng.integers(0, 256, size=(n + 1) // 2, dtype=np.uint8)
        if n % 2:
            c[-1] &= 0x0F
        e = rng.uniform(-149, top, size=nb)
        s = np.exp2(e).astype(np.float32)
        specials = [np.float32(0.0), np.float32(-0.0), np.float32(-3e-5), np.float32(1e-45)]
        if top > 120:
            specials += [np.float32(2.0 ** 125), np.nextafter(np.float32(2.0 ** 125), np.float32(0))]
        for t, v in enumerate(specials):
            b = ((t + 1) * per_tile) % nb
            if p == t % P:
                s[b] = v
        if top > 120:
            # keep k * s finite: no -8 code and |k| <= 7 where s is huge
            lo, hi = c & 0x0F, c >> 4
            lo = np.where(lo == 8, 7, lo)
            hi = np.where(hi == 8, 7, hi)
            c = (lo | (hi << 4)).astype(np.uint8)
        codes.append(c)
        scales.append(s)
    return codes, scales


@pytest.mark.parametrize("block", [32, 128, 1024, 4096])
@pytest.mark.parametrize("flags", [(True, False, False), (False, True, False), (False, True, True),
                                   (True, True, True)])
def test_dequant_reduce_extreme_scales(block, flags):
    want_out, requant, rqef = flags
    n = max(1024, block) * 9 + 3
    # moderate scales: every peer count; huge scales (up to 2^125): one peer,
    # so that sums stay finite
    for P in (2, 8):
        check_dr(P, n, block, 1.0, want_out, requant, rqef, seed=block + P,
                 chunks=extreme_scale_chunks(P, n, block, block + P, top=30))
    check_dr(1, n, block, 1.0, want_out, requant, rqef, seed=block,
             chunks=extreme_scale_chunks(1, n, block, block, top=124.99))


@pytest.mark.parametrize("with_rq_ef", [False, True])
def test_requant_scales_at_the_decode_boundary(with_rq_ef):
    """8 peers of moderate scales, and in chosen tiles one peer whose block
    scale is 2^124 or 1.5 * 2^124 (the requant kernels then redo that tile
    from the integer nibbles) or the float just below 2^124 (still the k / 16
    decode).  Every sum stays finite, as the contract asks."""
    P, B = 8, 128
    n = 1024 * 8 + 130
    codes, scales = make_chunks(P, n, B, seed=77, raw=True)
    for s in scales:
        s[:] = np.abs(s)
    big = np.float32(2.0 ** 124)
    # (block, peer, scale): one huge scale per block, so no sum overflows;
    # blocks 64 and 65 are the ragged tail
    placed = [(11, 3, big), (19, 5, np.nextafter(big, np.float32(0))), (27, 0, big),
              (28, 7, np.float32(2.0 ** 124 * 1.5)), (35, 2, np.nextafter(big, np.float32(0))),
              (51, 4, big), (65, 1, big)]
    for b, peer, v in placed:
        scales[peer][b] = v
    check_dr(P, n, B, 1.0, False, True, with_rq_ef, seed=78, chunks=(codes, scales))
    check_dr(P, n, B, 1.0, True, True, with_rq_ef, seed=79, chunks=(codes, scales))


# ---------------------------------------------------------------- qwZ int8 --

@pytest.mark.parametrize("block", BLOCKS)
@pytest.mark.parametrize("wdt", ["fp32", "bf16", "fp16"])
def test_quant_dequant_int8(block, wdt):
    for i, n in enumerate(sizes_for(block, 1024)):
        x = grad_values(n, seed=300 * block + i, std=0.02, special=True, block=block)
        w = as_dtype(x, wdt, seed=i)
        c_o, s_o = O.quant_int8(w, block)
        codes = Guarded(n, torch.int8)
        scales = Guarded(-(-n // block), torch.float32)
        Z().zq_quant_int8(to_gpu(w), block, codes.t, scales.t)
        torch.cuda.synchronize()
        what = f"q8 n={n} B={block} {wdt}"
        c_g, s_g = codes.host(), scales.host()
        assert_bits_equal(c_g.view(np.uint8), c_o.view(np.uint8), what + " codes")
        assert_bits_equal(s_g, s_o, what + " scales")
        for odt, tdt in (("bf16", torch.bfloat16), ("fp16", torch.float16),
                         ("fp32", torch.float32)):
            o_o = O.dequant_int8(c_o, s_o, block, out_bf16=odt == "bf16", out_f16=odt == "fp16")
            out = Guarded(n, tdt)
            Z().zq_dequant_int8(to_gpu(c_o), to_gpu(s_o), block, out.t)
            torch.cuda.synchronize()
            assert_bits_equal(out.host(), o_o, what + f" dequant to {odt}")


# ------------------------------------------------------ stochastic rounding --

def sr_inputs(n, seed, special=False):
    rng = np.random.default_rng(seed)
    d = as_bf16_bits((rng.standard_normal(n) * 1e-2).astype(np.float32))
    s = as_bf16_bits((rng.standard_normal(n) * 1e-4).astype(np.float32))
    if special and n >= 16:
        idx = rng.choice(n, size=min(n, 16), replace=False)
        d[idx[0]] = 0x7FC0  # NaN
        d[idx[1]] = 0x7F80  # +inf
        d[idx[2]] = 0xFF80  # -inf
        d[idx[3]] = 0x7F7F  # near max: may round up to inf
        s[idx[3]] = 0x7B00
        d[idx[4]] = 0x8000  # -0
        s[idx[4]] = 0x8000
        d[idx[5]] = 0x0001  # subnormal
        s[idx[5]] = 0x0001
        d[idx[6]] = 0x3F80
        s[idx[6]] = 0x3B80
    return d, s


@pytest.mark.parametrize("phase", range(8))
@pytest.mark.parametrize("zero_src", [False, True])
def test_sr_matches_oracle(phase, zero_src):
    for i, n in enumerate([1, 7, 8, 1023, 1024, 1024 * 5 + 9, 1 << 17]):
        d, s = sr_inputs(n, seed=10 * phase + i, special=True)
        seed = 0x1234_5678_9ABC_DEF0 + i
        cb = 8 * (3 + 1000 * i) + phase
        d_o, s_o = d.copy(), s.copy()
        O.sr_accumulate(d_o, s_o, seed, cb, zero_src)
        dg, sg = to_gpu(d), to_gpu(s)
        Z().zq_sr_accumulate(dg, sg, seed, cb, zero_src)
        torch.cuda.synchronize()
        what = f"sr n={n} phase={phase} zero={zero_src}"
        assert_bits_equal(to_host(dg), d_o, what + " dst")
        assert_bits_equal(to_host(sg), s_o, what + " src")


def test_sr_counter_above_2_pow_35():
    """Counters whose Philox counter needs its high word."""
    n = 4096 + 3
    d, s = sr_inputs(n, seed=5)
    cb = (1 << 35) * 8 + 5
    d_o = d.copy()
    O.sr_accumulate(d_o, s.copy(), 42, cb, False)
    dg = to_gpu(d)
    Z().zq_sr_accumulate(dg, to_gpu(s), 42, cb)
    torch.cuda.synchronize()
    assert_bits_equal(to_host(dg), d_o, "sr high counter")


def test_sr_shard_equals_slice_of_full_run_on_gpu():
    n, P, rank = 8 * 40000, 8, 3
    shard = n // P
    off = rank * shard
    full = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    part = torch.zeros(shard, dtype=torch.bfloat16, device="cuda")
    for m in range(8):
        src = torch.randn(n, generator=torch.Generator().manual_seed(m)).mul_(1e-4).to(torch.bfloat16).cuda()
        Z().zq_sr_accumulate(full, src, m, 0)
        Z().zq_sr_accumulate(part, src[off:off + shard].contiguous(), m, off)
    torch.cuda.synchronize()
    assert torch.equal(full[off:off + shard].view(torch.int16), part.view(torch.int16))


# ------------------------------------------------ batched SR accumulation --

@pytest.mark.parametrize("zero_src", [False, True])
def test_sr_batched_matches_oracle(zero_src):
    """70 segments (three launches of at most 32), ragged lengths, zero-length
    segments, every counter phase, slices anywhere in their buffers."""
    rng = np.random.default_rng(21 + zero_src)
    segs_g, segs_o = [], []
    for i in range(70):
        n = int(rng.choice([0, 1, 7, 8, 1000, 1024, 3000, 20000]))
        off = 8 * int(rng.integers(0, 300))
        tail = int(rng.integers(0, 2000))
        L = off + n + tail
        d = sr_inputs(max(n, 1), seed=100 + i)[0][:n].copy()
        s = sr_inputs(max(L, 1), seed=200 + i)[1][:L].copy()
        seed = int(rng.integers(0, 2 ** 63))
        cb = int(rng.integers(0, 2 ** 40))
        segs_o.append((d, s, n, off, seed, cb))
        segs_g.append((to_gpu(d) if n else torch.zeros(8, dtype=torch.bfloat16, device="cuda"),
                       to_gpu(s) if L else torch.zeros(8, dtype=torch.bfloat16, device="cuda"),
                       n, off, seed, cb))
    expect = [(d.copy(), s.copy(), n, off, seed, cb) for d, s, n, off, seed, cb in segs_o]
    O.sr_accumulate_segments(expect, zero_src)
    Z().zq_sr_accumulate_batched(segs_g, zero_src=zero_src)
    torch.cuda.synchronize()
    for i, ((dg, sg, n, off, _, _), (de, se, _, _, _, _)) in enumerate(zip(segs_g, expect)):
        if n:
            assert_bits_equal(to_host(dg)[:n], de, f"segment {i} dst")
        if se.size:
            assert_bits_equal(to_host(sg)[:se.size], se, f"segment {i} src")


def test_sr_batched_equals_per_tensor_calls():
    """The batched call gives exactly what the per-tensor loop of single
    calls plus a zeroing of each buffer gives."""
    rng = np.random.default_rng(5)
    segs_a, segs_b = [], []
    for i in range(40):
        n = 8 * int(rng.integers(1, 3000))
        P = 8
        full = torch.randn(P * n, generator=torch.Generator().manual_seed(i)).mul_(1e-4).to(torch.bfloat16).cuda()
        dst = torch.randn(n, generator=torch.Generator().manual_seed(1000 + i)).mul_(1e-2).to(torch.bfloat16).cuda()
        segs_a.append((dst.clone(), full.clone(), n, 3 * n, 77 + i, 12345 + 3 * n))
        segs_b.append((dst.clone(), full.clone(), n, 3 * n, 77 + i, 12345 + 3 * n))
    Z().zq_sr_accumulate_batched(segs_a, zero_src=True)
    for dst, full, n, off, seed, cb in segs_b:
        Z().zq_sr_accumulate(dst, full[off:off + n], seed, cb)
        full.zero_()
    torch.cuda.synchronize()
    for (da, fa, *_), (db, fb, *_) in zip(segs_a, segs_b):
        assert torch.equal(da.view(torch.int16), db.view(torch.int16))
        assert torch.equal(fa.view(torch.int16), fb.view(torch.int16))


# -------------------------------------- permuted (ZeRO++ hierarchical) order --

@pytest.mark.parametrize("block", [128, 256, 2048])
@pytest.mark.parametrize("gdt", ["fp32", "bf16", "fp16"])
def test_efq_permuted_matches_oracle(block, gdt):
    rng = np.random.default_rng(block + ["fp32", "bf16", "fp16"].index(gdt))
    for n_part, part in [(1, max(1024, block)), (5, max(1152, block * 3 // 2 // block * block or block)),
                         (8, max(2048, block)), (32, max(1024, block) + block)]:
        part = (part // block) * block
        n = n_part * part
        slots = [int(v) for v in rng.permutation(n_part)]
        x = grad_values(n, seed=n + block, special=True, block=block)
        g = as_dtype(x, gdt, seed=n)
        for with_ef in (False, True):
            ef_h = grad_values(n, seed=3, std=1e-5) if with_ef else None
            ef_o = ef_h.copy() if with_ef else None
            c_o, s_o = O.quantize_ef_int4_permuted(g, ef_o, block, 0.9, 1.0, slots)
            ef_g = to_gpu(ef_h) if with_ef else None
            codes = Guarded((n + 1) // 2, torch.uint8)
            scales = Guarded(n // block, torch.float32)
            Z().zq_quantize_ef_int4_permuted(to_gpu(g), ef_g, block, 0.9, 1.0, codes.t, scales.t,
                                             slots)
            torch.cuda.synchronize()
            what = f"permuted n_part={n_part} part={part} B={block} {gdt} ef={with_ef}"
            assert_bits_equal(codes.host(), c_o, what + " codes")
            assert_bits_equal(scales.host(), s_o, what + " scales")
            if with_ef:
                assert_bits_equal(to_host(ef_g), ef_o, what + " ef")


def test_hierarchical_qgz_delivers_each_rank_its_partition():
    """2 nodes x 4 GPUs simulated on one GPU: every rank quantizes its own
    gradient in ZeRO++'s order, the intra-node all-to-all hands local rank l
    chunk l of its node peers (8-way... here 4-way reduce + requant), the
    inter-node all-to-all hands node n sub-chunk n of the same local rank on
    every node (2-way reduce, alpha 1/8).  Rank r = node*4 + local must end
    with the average of partition r of all 8 gradients: bit-exact against
    the oracle running the same exchanges, and bit-exact against the
    natural-order quantizer with the same two-level reduction of partition r
    alone (the meaning of the order, as pinned on the CPU)."""
    from weight_communication_zero_amd import zeropp_slots
    intra, inter, B = 4, 2, 128
    R = intra * inter
    part = 9 * B * 8  # 9216 elements per partition
    M = R * part
    slots = zeropp_slots(intra, inter)
    grads = [grad_values(M, seed=1000 + r, outlier_p=0.0) for r in range(R)]
    # every rank: EF int4 quantize into ZeRO++ order
    cg, sg, co, so = [], [], [], []
    for r in range(R):
        c = torch.empty(M // 2, dtype=torch.uint8, device="cuda")
        s = torch.empty(M // B, dtype=torch.float32, device="cuda")
        Z().zq_quantize_ef_int4_permuted(to_gpu(grads[r]), None, B, 0.0, 1.0, c, s, slots)
        c_o, s_o = O.quantize_ef_int4_permuted(grads[r], None, B, 0.0, 1.0, slots)
        cg.append(c), sg.append(s), co.append(c_o), so.append(s_o)
    nat = [O.quantize_ef_int4(grads[r], None, B, 0.0, 1.0) for r in range(R)]
    chunk = M // intra  # level-1 chunk: slots [l*inter, (l+1)*inter)
    l1_g, l1_o = {}, {}
    for node in range(inter):
        for l in range(intra):
            peers = [node * intra + q for q in range(intra)]
            cc = [cg[p][l * chunk // 2:(l + 1) * chunk // 2] for p in peers]
            ss = [sg[p][l * chunk // B:(l + 1) * chunk // B] for p in peers]
            rqc = torch.empty(chunk // 2, dtype=torch.uint8, device="cuda")
            rqs = torch.empty(chunk // B, dtype=torch.float32, device="cuda")
            Z().zq_dequant_reduce(cc, ss, chunk, B, 1.0, rq_codes=rqc, rq_scales=rqs)
            _, rc_o, rs_o = O.dequant_reduce([co[p][l * chunk // 2:(l + 1) * chunk // 2] for p in peers],
                                             [so[p][l * chunk // B:(l + 1) * chunk // B] for p in peers],
                                             chunk, B, 1.0, want_out=False, requant=True)
            l1_g[(node, l)] = (rqc, rqs)
            l1_o[(node, l)] = (rc_o, rs_o)
    for node in range(inter):
        for l in range(intra):
            r = node * intra + l
            cc = [l1_g[(nd, l)][0][node * part // 2:(node + 1) * part // 2] for nd in range(inter)]
            ss = [l1_g[(nd, l)][1][node * part // B:(node + 1) * part // B] for nd in range(inter)]
            out = torch.empty(part, dtype=torch.float32, device="cuda")
            Z().zq_dequant_reduce(cc, ss, part, B, 1.0 / R, out=out)
            out_o, _, _ = O.dequant_reduce(
                [l1_o[(nd, l)][0][node * part // 2:(node + 1) * part // 2] for nd in range(inter)],
                [l1_o[(nd, l)][1][node * part // B:(node + 1) * part // B] for nd in range(inter)],
                part, B, 1.0 / R)
            torch.cuda.synchronize()
            got = to_host(out)
            assert_bits_equal(got, out_o, f"rank {r} final shard")
            # what partition r must be: the natural-order quantizer and the
            # same two-level reduction over partition r alone
            sub = []
            for nd in range(inter):
                recv = [(nat[nd * intra + q][0][r * part // 2:(r + 1) * part // 2],
                         nat[nd * intra + q][1][r * part // B:(r + 1) * part // B])
                        for q in range(intra)]
                _, rc_n, rs_n = O.dequant_reduce([a for a, _ in recv], [b for _, b in recv], part,
                                                 B, 1.0, want_out=False, requant=True)
                sub.append((rc_n, rs_n))
            want, _, _ = O.dequant_reduce([a for a, _ in sub], [b for _, b in sub], part, B, 1.0 / R)
            assert_bits_equal(got, want, f"rank {r} holds partition {r}")
            exact = np.mean([g[r * part:(r + 1) * part].astype(np.float64) for g in grads], axis=0)
            err = np.abs(got - exact)
            assert np.corrcoef(got, exact)[0, 1] > 0.95, f"rank {r} did not receive partition {r}"
            assert err.mean() < 0.2 * np.abs(exact).mean(), f"rank {r}: mean error {err.mean()}"


# ------------------------------------------------- batched EF quantize --

@pytest.mark.parametrize("block", [128, 256, 2048])
@pytest.mark.parametrize("gdt", ["fp32", "bf16", "fp16"])
@pytest.mark.parametrize("with_ef", [False, True])
def test_efq_batched_matches_oracle(block, gdt, with_ef):
    """170 tensors (three launches of at most 80), ragged lengths from 1
    element to several tiles."""
    rng = np.random.default_rng(block * 7 + ["fp32", "bf16", "fp16"].index(gdt) * 3 + with_ef)
    segs_g, exp = [], []
    for i in range(170):
        n = int(rng.choice([1, 3, block - 1, block, 1024, 4096, 4096 + 17, 3 * max(1024, block) + 5,
                            20000]))
        x = grad_values(n, seed=300 + i, special=True, block=block)
        g = as_dtype(x, gdt, seed=i)
        ef_h = grad_values(n, seed=900 + i, std=1e-5) if with_ef else None
        ef_o = ef_h.copy() if with_ef else None
        c_o, s_o = O.quantize_ef_int4(g, ef_o, block, 0.9, 1.0)
        exp.append((c_o, s_o, ef_o))
        codes = Guarded((n + 1) // 2, torch.uint8)
        scales = Guarded(-(-n // block), torch.float32)
        segs_g.append((to_gpu(g), to_gpu(ef_h) if with_ef else None, codes, scales))
    Z().zq_quantize_ef_int4_batched([(g, e, c.t, s.t) for g, e, c, s in segs_g], block, 0.9, 1.0)
    torch.cuda.synchronize()
    for i, ((g, e, c, s), (c_o, s_o, ef_o)) in enumerate(zip(segs_g, exp)):
        what = f"batched efq segment {i} n={g.numel()} B={block} {gdt} ef={with_ef}"
        assert_bits_equal(c.host(), c_o, what + " codes")
        assert_bits_equal(s.host(), s_o, what + " scales")
        if with_ef:
            assert_bits_equal(to_host(e), ef_o, what + " ef")


def test_int8_random_ties_band():
    """int8 twin of the int4 tie-band test: values on and a few ulps around
    the rounding boundaries (k + 1/2) s of their 2048-element block."""
    rng = np.random.default_rng(31)
    block, nb = 2048, 64
    out = []
    for b in range(nb):
        s = np.float32(2.0 ** rng.integers(-30, 30) * rng.uniform(1, 2))
        ks = rng.integers(-127, 127, size=block) + 0.5
        x = (ks * s).astype(np.float32)
        for _ in range(int(rng.integers(1, 3))):
            d = rng.integers(-1, 2, size=block)
            target = np.where(d < 0, -np.inf, np.where(d > 0, np.inf, x)).astype(np.float32)
            x = np.nextafter(x, target)
        x[0] = np.float32(127) * s
        out.append(x.astype(np.float32))
    w = np.concatenate(out)
    c_o, s_o = O.quant_int8(w, block)
    codes = Guarded(w.size, torch.int8)
    scales = Guarded(nb, torch.float32)
    Z().zq_quant_int8(to_gpu(w), block, codes.t, scales.t)
    torch.cuda.synchronize()
    assert_bits_equal(codes.host().view(np.uint8), c_o.view(np.uint8), "int8 tie band codes")
    assert_bits_equal(scales.host(), s_o, "int8 tie band scales")


@pytest.mark.parametrize("with_rq_ef", [False, True])
def test_requant_exact_ties(with_rq_ef):
    """Reduced sums that sit exactly on half-integers of the requant scale:
    peer 0 has scale 2^-10 with a code 7 in every block (so the requant scale
    is 2^-10 again), peer 1 adds +-1 at scale 2^-11.  Ties appear only in the
    first two 1024-element tiles, so those tiles take the IEEE path and the
    rest the fast path; the codes must round half to even like the oracle."""
    rng = np.random.default_rng(77)
    n, block = 8192, 128
    k0 = rng.integers(-6, 7, size=n)
    k0[::block] = 7
    k1 = np.zeros(n, dtype=np.int64)
    k1[:2048] = rng.choice([-1, 0, 1], size=2048)
    k1[:2048:block] = 0

    def pack(k):
        u = (k & 0xF).astype(np.uint8)
        return (u[0::2] | (u[1::2] << 4)).astype(np.uint8)
    codes = [pack(k0), pack(k1)]
    scales = [np.full(n // block, 2.0 ** -10, np.float32), np.full(n // block, 2.0 ** -11, np.float32)]
    rq_ef_h = grad_values(n, seed=5, std=1e-6) if with_rq_ef else None
    rq_ef_o = rq_ef_h.copy() if with_rq_ef else None
    _, rqc_o, rqs_o = O.dequant_reduce(codes, scales, n, block, 1.0, want_out=False, requant=True,
                                       rq_ef=rq_ef_o, rq_beta_e=0.9, rq_beta_r=1.0)
    rqc = Guarded(n // 2, torch.uint8)
    rqs = Guarded(n // block, torch.float32)
    rq_ef = to_gpu(rq_ef_h) if with_rq_ef else None
    Z().zq_dequant_reduce([to_gpu(c) for c in codes], [to_gpu(s) for s in scales], n, block, 1.0,
                          rq_codes=rqc.t, rq_scales=rqs.t, rq_ef=rq_ef, rq_beta_e=0.9,
                          rq_beta_r=1.0)
    torch.cuda.synchronize()
    what = f"requant ties rq_ef={with_rq_ef}"
    assert_bits_equal(rqc.host(), rqc_o, what + " codes")
    assert_bits_equal(rqs.host(), rqs_o, what + " scales")
    if with_rq_ef:
        assert_bits_equal(to_host(rq_ef), rq_ef_o, what + " rq_ef")


@pytest.mark.parametrize("P,block", [(8, 128), (5, 256)])
def test_requant_several_tiles_per_wave(P, block):
    """The requant without EF runs a fixed grid of 16,384 waves that walk
    the tiles with a stride of the wave count, so only chunks above 16,384
    tiles give a wave more than one: here about 2^25 outputs (two to four
    tiles per wave, depending on the tile length), an odd length with a
    ragged last tile.  Raw nibbles (-8 included) with positive scales keep
    the input cheap to draw; every code and scale is compared."""
    rng = np.random.default_rng(4000 + P)
    n = 2 * 16384 * 1024 + 5 * 512 + 77
    nb = -(-n // block)
    codes = [rng.integers(0, 256, size=(n + 1) // 2, dtype=np.uint8) for _ in range(P)]
    for c in codes:
        c[-1] &= 0x0F
    scales = [(rng.random(nb) * 1e-3 + 1e-7).astype(np.float32) for _ in range(P)]
    _, rqc_o, rqs_o = O.dequant_reduce(codes, scales, n, block, 1.0, want_out=False, requant=True,
                                       rq_ef=None, rq_beta_e=0.0, rq_beta_r=1.0)
    rqc = Guarded((n + 1) // 2, torch.uint8)
    rqs = Guarded(nb, torch.float32)
    Z().zq_dequant_reduce([to_gpu(c) for c in codes], [to_gpu(s) for s in scales], n, block, 1.0,
                          rq_codes=rqc.t, rq_scales=rqs.t)
    torch.cuda.synchronize()
    what = f"requant P={P} B={block} n={n}"
    assert_bits_equal(rqc.host(), rqc_o, what + " codes")
    assert_bits_equal(rqs.host(), rqs_o, what + " scales")


# ----------------------------------------- batched dequantize + reduce --

def _dr_segments(P, block, sizes, seed, raw):
    """Per-tensor receive buffers: P chunks of n elements each, padded
    strides (16-byte multiples for the codes), quantized gradients or raw
    nibbles."""
    rng = np.random.default_rng(seed)
    segs = []
    for i, n in enumerate(sizes):
        cb, nb = (n + 1) // 2, -(-n // block)
        cs = -(-cb // 16) * 16 + 16 * int(rng.integers(0, 3))
        ss = nb + int(rng.integers(0, 3))
        codes = rng.integers(0, 256, size=(P - 1) * cs + cb if n else 16, dtype=np.uint8)
        scales = (rng.random((P - 1) * ss + nb if n else 1) * 1e-3).astype(np.float32)
        if n and not raw:
            chunks, chunk_scales = make_chunks(P, n, block, seed=seed * 100 + i)
            for p in range(P):
                codes[p * cs:p * cs + cb] = chunks[p]
                scales[p * ss:p * ss + nb] = chunk_scales[p]
        segs.append((codes, scales, n, cs, ss))
    return segs


def _run_dr_batched(segs, P, block, alpha, want_out, requant, with_ef, seed):
    rng = np.random.default_rng(seed + 1)
    efs = [(rng.standard_normal(s[2]) * 1e-6).astype(np.float32) for s in segs] if with_ef else None
    efs_o = [e.copy() for e in efs] if with_ef else None  # updated in place by the oracle
    ref = O.dequant_reduce_segments(segs, P, block, alpha, want_out=want_out, requant=requant,
                                    rq_efs=efs_o, rq_beta_e=0.9, rq_beta_r=1.0)
    bufs = []
    table = []
    for i, (codes, scales, n, cs, ss) in enumerate(segs):
        cg, sg = to_gpu(codes), to_gpu(scales)
        out = Guarded(max(n, 1), torch.float32) if want_out else None
        rqc = Guarded(max((n + 1) // 2, 1), torch.uint8) if requant else None
        rqs = Guarded(max(-(-n // block), 1), torch.float32) if requant else None
        ef = to_gpu(efs[i]) if with_ef and n else None
        bufs.append((cg, sg, out, rqc, rqs, ef))
        table.append((cg, sg, n, cs, ss, out.t if out else None, rqc.t if rqc else None,
                      rqs.t if rqs else None, ef))
    Z().zq_dequant_reduce_batched(table, P, block, alpha, rq_beta_e=0.9, rq_beta_r=1.0)
    torch.cuda.synchronize()
    return ref, efs_o, bufs


@pytest.mark.parametrize("block", [32, 128, 1024, 4096])
@pytest.mark.parametrize("flags", [(True, False, False), (False, True, False), (False, True, True),
                                   (True, True, True)])
def test_dequant_reduce_batched_matches_oracle(block, flags):
    """60 tensors (more than one launch takes) of ragged sizes -- empty,
    shorter than a tile, several tiles plus a tail -- with padded strides,
    against the oracle segment by segment, every output poisoned and
    guarded."""
    want_out, requant, with_ef = flags
    tile = max(1024, block)
    rng = np.random.default_rng(block)
    sizes = [0, 1, block - 1, block, tile, tile + 3, 2 * tile + block // 2 + 1]
    sizes += [int(rng.integers(1, 3 * tile)) for _ in range(60 - len(sizes))]
    for P, raw in ((8, False), (3, True), (16, True), (1, False)):
        segs = _dr_segments(P, block, sizes[: 60 if P == 8 else 20], seed=block + P, raw=raw)
        ref, efs_o, bufs = _run_dr_batched(segs, P, block, 0.125 if P > 1 else 1.0, want_out, requant,
                                           with_ef, seed=block * P)
        for i, ((out_o, rqc_o, rqs_o), (cg, sg, out, rqc, rqs, ef), s) in enumerate(zip(ref, bufs, segs)):
            n = s[2]
            what = f"batched dr B={block} P={P} seg {i} n={n} flags={flags}"
            if n == 0:
                continue
            if want_out:
                assert_bits_equal(out.host()[:n], out_o, what + " out")
            if requant:
                assert_bits_equal(rqc.host(), rqc_o, what + " rq_codes")
                assert_bits_equal(rqs.host(), rqs_o, what + " rq_scales")
            if with_ef:
                assert_bits_equal(to_host(ef), efs_o[i], what + " rq_ef")
        for (cg, sg, out, rqc, rqs, ef), s in zip(bufs, segs):
            if s[2] == 0:  # an empty segment writes nothing
                for g in (out, rqc, rqs):
                    if g is not None:
                        v = to_host(g.buf)
                        assert (v == 0xAA).all() if v.dtype == np.uint8 else np.isnan(v).all()


def test_dequant_reduce_batched_equals_single_calls():
    """The batched call against a loop of zq_dequant_reduce over the same
    tensors (GPU against GPU), requant with EF, P = 8, block 128, including
    two tensors that share one receive buffer."""
    P, B = 8, 128
    sizes = [4096, 1024 * 5 + 77, 512, 100000, 64, 1024]
    segs = _dr_segments(P, B, sizes, seed=3, raw=False)
    segs.append(segs[0])  # the same inputs reduced twice, into other outputs
    rng = np.random.default_rng(4)
    efs = [(rng.standard_normal(s[2]) * 1e-6).astype(np.float32) for s in segs]
    outs_b, outs_s = [], []
    table = []
    for (codes, scales, n, cs, ss), e in zip(segs, efs):
        cg, sg = to_gpu(codes), to_gpu(scales)
        for dst, batched in ((outs_b, True), (outs_s, False)):
            o = torch.empty(n, dtype=torch.float32, device="cuda")
            rc = torch.empty((n + 1) // 2, dtype=torch.uint8, device="cuda")
            rs = torch.empty(-(-n // B), dtype=torch.float32, device="cuda")
            ef = to_gpu(e)
            dst.append((o, rc, rs, ef))
            if batched:
                table.append((cg, sg, n, cs, ss, o, rc, rs, ef))
            else:
                Z().zq_dequant_reduce([cg[p * cs:p * cs + (n + 1) // 2] for p in range(P)],
                                      [sg[p * ss:p * ss + -(-n // B)] for p in range(P)], n, B,
                                      0.125, out=o, rq_codes=rc, rq_scales=rs, rq_ef=ef,
                                      rq_beta_e=0.9, rq_beta_r=1.0)
    Z().zq_dequant_reduce_batched(table, P, B, 0.125, rq_beta_e=0.9, rq_beta_r=1.0)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(outs_b, outs_s)):
        for x, y, name in zip(a, b, ("out", "rq_codes", "rq_scales", "rq_ef")):
            assert_bits_equal(to_host(x), to_host(y), f"segment {i} {name}")
