"""Pins of the CPU oracle against facts that do not come from the oracle:
hand-worked examples (tests/golden), exact rational arithmetic, library
routines (torch CPU rounding and bf16 conversion), identities of the method
(error-feedback telescoping, P = 1 and power-of-two reductions, requant
idempotence), exact enumeration and statistics of stochastic rounding,
published Philox known-answer vectors, and the pages' communication-volume
closed form.  No GPU is used here.
"""
import json
import math
import os
from fractions import Fraction as F

import numpy as np
import pytest
import torch

import oracle as O

RNG = np.random.default_rng(12345)


# ----------------------------------------------------------------- helpers --

def fx(x) -> F:
    """Exact rational value of an fp32 number."""
    return F(float(np.float32(x)))


def f32_bits(x) -> int:
    return int(np.array([x], dtype=np.float32).view(np.uint32)[0])


def bits_f32(u: int) -> np.float32:
    return np.array([u], dtype=np.uint32).view(np.float32)[0]


def bf16_value(h: int) -> F:
    return fx(bits_f32(h << 16))


def nearest_f32(q: F) -> np.float32:
    """The fp32 number nearest to the rational q, ties to even mantissa."""
    f0 = np.float32(float(q))
    cands = [np.nextafter(f0, np.float32(-np.inf)), f0, np.nextafter(f0, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(fx(c) - q), f32_bits(c) & 1))


def brute_code(qf: np.float32, qmax: int) -> int:
    """Nearest integer in [-qmax, qmax] to an fp32 value, ties to even."""
    qq = fx(qf)
    return min(range(-qmax, qmax + 1), key=lambda k: (abs(qq - k), k % 2))


def load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def hexbytes(lst):
    return np.array([int(h, 16) for h in lst], dtype=np.uint8)


def pack_expect(codes):
    """Expected packed bytes for a short code list, from the fixture's
    stated layout (two's-complement nibble, element 2j in the low half)."""
    out = []
    for j in range(0, len(codes), 2):
        lo = codes[j] & 0xF
        hi = (codes[j + 1] & 0xF) if j + 1 < len(codes) else 0
        out.append(lo | (hi << 4))
    return np.array(out, dtype=np.uint8)


# -------------------------------------------------- worked examples (golden) --

def test_quant_worked_examples(golden_dir):
    G = load(golden_dir, "quant_worked_examples.json")
    for case in G["int4_blocks"]:
        k, s = O.quant_block(np.array(case["x"], np.float32), 7)
        assert s == np.float32(case["scale"]) and f32_bits(s) == f32_bits(np.float32(case["scale"]))
        assert k.tolist() == case["codes"], case
        codes, scales = O.quantize_ef_int4(np.array(case["x"], np.float32), None, 4, 0.0, 1.0)
        assert scales[0] == np.float32(case["scale"])
        assert O.int4_decode(codes, 4).tolist() == case["codes"]
        if "packed" in case:
            assert codes.tolist() == hexbytes(case["packed"]).tolist()
    for case in G["int8_blocks"]:
        k, s = O.quant_block(np.array(case["x"], np.float32), 127)
        assert s == np.float32(case["scale"])
        assert k.tolist() == case["codes"], case
        codes, scales = O.quant_int8(np.array(case["x"], np.float32), 4)
        assert codes.tolist() == case["codes"] and scales[0] == np.float32(case["scale"])


def test_ef_worked_example(golden_dir):
    G = load(golden_dir, "quant_worked_examples.json")["ef_int4"]
    g = np.array(G["g"], np.float32)
    for beta_e, key in ((0.0, "e_next_beta0"), (0.5, "e_next_beta_half")):
        e = np.array(G["e"], np.float32)
        codes, scales = O.quantize_ef_int4(g, e, G["block"], beta_e, 1.0)
        assert codes.tolist() == hexbytes(G["packed"]).tolist()
        assert O.int4_decode(codes, 4).tolist() == G["codes"]
        assert scales[0] == np.float32(G["scale"])
        assert e.tolist() == G[key]


def test_int4_decode_worked_example(golden_dir):
    G = load(golden_dir, "quant_worked_examples.json")["int4_decode"]
    assert O.int4_decode(hexbytes(G["bytes"]), 8).tolist() == G["values"]


def test_dequant_reduce_worked_example(golden_dir):
    G = load(golden_dir, "quant_worked_examples.json")["dequant_reduce"]
    codes = [pack_expect(c) for c in G["codes"]]
    scales = [np.array([s], np.float32) for s in G["scales"]]
    out, _, _ = O.dequant_reduce(codes, scales, 4, G["block"], G["alpha"])
    assert out.tolist() == G["out"]


# ------------------------------------------------ quantizer: exact pins --

def _grid_blocks(B, count, qmax):
    """Tiny blocks whose values include exact ties, zeros, signed zeros,
    subnormals and random mantissas."""
    blocks = []
    for _ in range(count):
        kind = RNG.integers(0, 5)
        if kind == 0:  # exact ties on a power-of-two scale
            e = int(RNG.integers(-30, 30))
            s0 = 2.0 ** e
            ks = RNG.integers(-2 * qmax, 2 * qmax + 1, size=B) / 2.0
            x = (ks * s0).astype(np.float32)
            x[RNG.integers(0, B)] = np.float32(qmax * s0 * RNG.choice([-1, 1]))
        elif kind == 1:  # random normals of random scale
            x = (RNG.standard_normal(B) * 10.0 ** RNG.uniform(-8, 8)).astype(np.float32)
        elif kind == 2:  # subnormal and tiny
            x = (RNG.integers(-40, 41, size=B) * np.float32(1.4e-45)).astype(np.float32)
        elif kind == 3:  # zeros and signed zeros
            x = np.array(RNG.choice([0.0, -0.0], size=B), np.float32)
        else:  # one outlier
            x = (RNG.standard_normal(B) * 1e-3).astype(np.float32)
            x[RNG.integers(0, B)] *= np.float32(50.0)
        blocks.append(x)
    return blocks


@pytest.mark.parametrize("qmax", [7, 127])
@pytest.mark.parametrize("B", [2, 4, 8])
def test_quant_block_exact_rational(B, qmax):
    """Scale = the fp32 number nearest to absmax/qmax, code = nearest
    integer (ties even, clamped) to the fp32 number nearest to x/scale --
    all decided in exact rational arithmetic, by brute force over codes."""
    for x in _grid_blocks(B, 300, qmax):
        k, s = O.quant_block(x, qmax)
        a = max(abs(fx(v)) for v in x)
        s_ref = nearest_f32(a / qmax)
        assert f32_bits(s) == f32_bits(s_ref), (x, s, s_ref)
        for v, kv in zip(x, k):
            if s_ref == 0:
                assert kv == 0
            else:
                assert kv == brute_code(nearest_f32(fx(v) / fx(s_ref)), qmax), (x, v, s)


@pytest.mark.parametrize("qmax", [7, 127])
def test_quant_matches_torch_rounding(qmax):
    """Library routine: torch CPU division (IEEE) and torch.round (half to
    even), clamped, reproduce the codes; scale as absmax / qmax."""
    B = 64
    x = (RNG.standard_normal(B * 512) * 1e-3).astype(np.float32)
    x[RNG.random(x.size) < 0.01] *= 50
    x[: 4 * B] = np.round(x[: 4 * B] * 1e3) / 1e3
    xt = torch.from_numpy(x).view(-1, B)
    a = xt.abs().amax(dim=1, keepdim=True)
    s = a / qmax
    kt = torch.where(s == 0, torch.zeros_like(xt), torch.round(xt / s)).clamp(-qmax, qmax)
    for b in range(xt.shape[0]):
        k, sb = O.quant_block(x[b * B:(b + 1) * B], qmax)
        assert f32_bits(sb) == f32_bits(s[b, 0].item())
        assert k.tolist() == kt[b].to(torch.int32).tolist()


@pytest.mark.parametrize("qmax", [7, 127])
def test_quant_error_bound_and_invariants(qmax):
    B = 32
    for trial in range(200):
        x = (RNG.standard_normal(B) * 10.0 ** RNG.uniform(-10, 10)).astype(np.float32)
        k, s = O.quant_block(x, qmax)
        # reconstruction error: |x - k s| <= s (1/2 + qmax 2^-24) for a normal scale
        for v, kv in zip(x, k):
            assert abs(fx(v) - kv * fx(s)) <= fx(s) * (F(1, 2) + F(qmax, 2 ** 24))
        # sign symmetry
        kn, sn = O.quant_block(-x, qmax)
        assert sn == s and (kn == -k).all()
        # power-of-two scaling: same codes, scale times 2^j
        j = int(RNG.integers(-20, 21))
        k2, s2 = O.quant_block((x * np.float32(2.0 ** j)).astype(np.float32), qmax)
        assert (k2 == k).all() and fx(s2) == fx(s) * F(2) ** j
        # permutation inside the block permutes the codes
        perm = RNG.permutation(B)
        kp, sp = O.quant_block(x[perm], qmax)
        assert sp == s and (kp == k[perm]).all()


def test_zero_block_gives_zero_codes_and_positive_zero_scale():
    for x in (np.zeros(8, np.float32), -np.zeros(8, np.float32)):
        k, s = O.quant_block(x, 7)
        assert (k == 0).all() and f32_bits(s) == 0


def test_underflowing_scale_gives_zero_codes():
    # absmax = smallest subnormal: absmax/7 rounds to +0 -> all codes 0
    x = np.array([1.4e-45, -1.4e-45, 0.0, 1.4e-45], np.float32)
    k, s = O.quant_block(x, 7)
    assert f32_bits(s) == 0 and (k == 0).all()


# -------------------------------------------------- packing and tail blocks --

def test_tail_block_scale_uses_only_its_elements_and_odd_n_high_nibble_zero():
    g = np.array([1.0, 2.0, 3.0, 7.0, 0.5], np.float32)  # n = 5, block 4
    codes, scales = O.quantize_ef_int4(g, None, 4, 0.0, 1.0)
    assert scales.tolist() == [1.0, np.float32(0.5) / np.float32(7)]
    assert codes.size == 3 and codes[2] >> 4 == 0 and O.int4_decode(codes, 5)[4] == 7
    codes_b, _ = O.quantize_ef_int4(g, None, 4, 0.0, 1.0)
    assert (codes_b == codes).all()


def test_ef_null_equals_plain_quantizer():
    n, B = 1000, 8
    g = (RNG.standard_normal(n) * 1e-3).astype(np.float32)
    codes, scales = O.quantize_ef_int4(g, None, B, 0.9, 1.0)
    dec = O.int4_decode(codes, n)
    for b in range(0, n, B):
        k, s = O.quant_block(g[b:b + B], 7)
        assert scales[b // B] == s and (dec[b:b + B] == k).all()


def test_bf16_input_is_widened_exactly():
    n, B = 512, 32
    gb = torch.randn(n, generator=torch.Generator().manual_seed(3)).mul(1e-3).to(torch.bfloat16)
    g16 = gb.view(torch.int16).numpy().view(np.uint16)
    g32 = gb.float().numpy()
    e1 = (RNG.standard_normal(n) * 1e-4).astype(np.float32)
    e2 = e1.copy()
    c1, s1 = O.quantize_ef_int4(g16, e1, B, 0.9, 1.0)
    c2, s2 = O.quantize_ef_int4(g32, e2, B, 0.9, 1.0)
    assert (c1 == c2).all() and (s1 == s2).all() and (e1.view(np.uint32) == e2.view(np.uint32)).all()


def test_f16_input_is_widened_exactly():
    """fp16 gradients and weights are widened to fp32 exactly before the
    quantizers see them: the same outputs as from the widened fp32 array."""
    n, B = 1000, 64
    g16 = (RNG.standard_normal(n) * 1e-3).astype(np.float16)  # includes fp16 subnormals
    g16[:4] = [np.float16(6e-8), np.float16(-6e-8), np.float16(65504.0), np.float16(-0.0)]
    e1 = (RNG.standard_normal(n) * 1e-4).astype(np.float32)
    e2 = e1.copy()
    c1, s1 = O.quantize_ef_int4(g16, e1, B, 0.9, 1.0)
    c2, s2 = O.quantize_ef_int4(g16.astype(np.float32), e2, B, 0.9, 1.0)
    assert (c1 == c2).all() and (s1.view(np.uint32) == s2.view(np.uint32)).all()
    assert (e1.view(np.uint32) == e2.view(np.uint32)).all()
    k1, t1 = O.quant_int8(g16, 128)
    k2, t2 = O.quant_int8(g16.astype(np.float32), 128)
    assert (k1 == k2).all() and (t1.view(np.uint32) == t2.view(np.uint32)).all()
    slots = [2, 0, 3, 1]
    p1 = O.quantize_ef_int4_permuted(g16[:512], None, 32, 0.9, 1.0, slots)
    p2 = O.quantize_ef_int4_permuted(g16[:512].astype(np.float32), None, 32, 0.9, 1.0, slots)
    assert (p1[0] == p2[0]).all() and (p1[1].view(np.uint32) == p2[1].view(np.uint32)).all()


# ---------------------------------------------------- error feedback (LoCo) --

@pytest.mark.parametrize("gdtype", ["fp32", "bf16"])
def test_ef_telescoping_identity_exact(gdtype):
    """Plain EF (beta_e = 0, beta_r = 1): sum_t d_t + e_T = sum_t g_t +
    sum_t delta_t, where delta_t = fl(g+e) - (g+e) is the rounding of the
    compensation add.  Checked in exact rational arithmetic with the exact
    dequant k*s, which differs from the receiver's fl(k*s) by at most
    2^-24 |k s| per step."""
    n, B, T = 256, 32, 5
    e = np.zeros(n, np.float32)
    sum_d = [F(0)] * n
    sum_abs_d = [F(0)] * n
    sum_g = [F(0)] * n
    sum_delta = [F(0)] * n
    for t in range(T):
        g32 = (RNG.standard_normal(n) * 1e-3).astype(np.float32)
        g32[RNG.random(n) < 0.02] *= 50
        if gdtype == "bf16":
            gb = torch.from_numpy(g32).to(torch.bfloat16)
            g_in = gb.view(torch.int16).numpy().view(np.uint16)
            g_val = gb.float().numpy()
        else:
            g_in, g_val = g32, g32
        e_prev = e.copy()
        codes, scales = O.quantize_ef_int4(g_in, e, B, 0.0, 1.0)
        dec = O.int4_decode(codes, n)
        for i in range(n):
            c = nearest_f32(fx(g_val[i]) + fx(e_prev[i]))
            sum_delta[i] += fx(c) - (fx(g_val[i]) + fx(e_prev[i]))
            d = int(dec[i]) * fx(scales[i // B])
            sum_d[i] += d
            sum_abs_d[i] += abs(d)
            sum_g[i] += fx(g_val[i])
    for i in range(n):
        lhs = sum_d[i] + fx(e[i])
        rhs = sum_g[i] + sum_delta[i]
        assert abs(lhs - rhs) <= F(1, 2 ** 24) * sum_abs_d[i]


def test_ef_telescoping_with_rounded_dequant_is_exact():
    """Same identity with d_t = fl(k s) (what the receiver reconstructs):
    then it holds with no slack at all, because r = c - d is exact."""
    n, B, T = 256, 32, 5
    e = np.zeros(n, np.float32)
    lhs_acc = [F(0)] * n
    rhs_acc = [F(0)] * n
    for t in range(T):
        g = (RNG.standard_normal(n) * 1e-3).astype(np.float32)
        e_prev = e.copy()
        codes, scales = O.quantize_ef_int4(g, e, B, 0.0, 1.0)
        out, _, _ = O.dequant_reduce([codes], [scales], n, B, 1.0)  # d = fl(k s)
        for i in range(n):
            c = nearest_f32(fx(g[i]) + fx(e_prev[i]))
            lhs_acc[i] += fx(out[i])
            rhs_acc[i] += fx(g[i]) + (fx(c) - fx(g[i]) - fx(e_prev[i]))
    for i in range(n):
        assert lhs_acc[i] + fx(e[i]) == rhs_acc[i]


def test_ef_generalized_identity_literal_beta():
    """e' = beta e + (g+e) - D(Q(g+e)) at beta = 0.9: sum d_t + e_T -
    beta sum_{t<T} e_t = sum g_t + sum delta_t, up to the rounding of the
    two-term EF update (<= 2^-24 (|beta e_{t-1}| + |e_t|) per step)."""
    n, B, T, beta = 128, 32, 6, np.float32(0.9)
    e = np.zeros(n, np.float32)
    acc = [F(0)] * n
    slack = [F(0)] * n
    hist = []
    for t in range(T):
        g = (RNG.standard_normal(n) * 1e-3).astype(np.float32)
        e_prev = e.copy()
        codes, scales = O.quantize_ef_int4(g, e, B, float(beta), 1.0)
        out, _, _ = O.dequant_reduce([codes], [scales], n, B, 1.0)
        for i in range(n):
            c = nearest_f32(fx(g[i]) + fx(e_prev[i]))
            delta = fx(c) - fx(g[i]) - fx(e_prev[i])
            acc[i] += fx(out[i]) - fx(g[i]) - delta
            slack[i] += F(1, 2 ** 23) * (abs(fx(beta) * fx(e_prev[i])) + abs(fx(e[i])))
        hist.append(e.copy())
    for i in range(n):
        lhs = acc[i] + fx(e[i]) - fx(beta) * sum(fx(hist[t][i]) for t in range(T - 1))
        assert abs(lhs) <= slack[i] + F(1, 2 ** 140)


def test_ef_save_restore_equals_straight_run():
    n, B = 4096, 128
    gs = [(RNG.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(10)]
    e_a = np.zeros(n, np.float32)
    outs_a = [O.quantize_ef_int4(g, e_a, B, 0.9, 1.0) for g in gs]
    e_b = np.zeros(n, np.float32)
    outs_b = [O.quantize_ef_int4(g, e_b, B, 0.9, 1.0) for g in gs[:5]]
    saved = e_b.copy()
    e_c = saved.copy()  # "restored" buffer
    outs_b += [O.quantize_ef_int4(g, e_c, B, 0.9, 1.0) for g in gs[5:]]
    assert (e_a.view(np.uint32) == e_c.view(np.uint32)).all()
    for (ca, sa), (cb, sb) in zip(outs_a, outs_b):
        assert (ca == cb).all() and (sa.view(np.uint32) == sb.view(np.uint32)).all()


def test_ef_residual_bound():
    n, B = 2048, 128
    g = (RNG.standard_normal(n) * 1e-3).astype(np.float32)
    e = np.zeros(n, np.float32)
    codes, scales = O.quantize_ef_int4(g, e, B, 0.0, 1.0)
    for i in range(n):
        assert abs(fx(e[i])) <= fx(scales[i // B]) * (F(1, 2) + F(7, 2 ** 24)) * (1 + F(1, 2 ** 22))


# ------------------------------------------------ dequantize + reduce --

def _rand_chunks(P, n, B, seed):
    r = np.random.default_rng(seed)
    codes, scales = [], []
    for p in range(P):
        g = (r.standard_normal(n) * 10.0 ** r.uniform(-4, 0)).astype(np.float32)
        c, s = O.quantize_ef_int4(g, None, B, 0.0, 1.0)
        codes.append(c)
        scales.append(s)
    return codes, scales


@pytest.mark.parametrize("P", [2, 4, 8, 16])
def test_dequant_reduce_within_exact_sum_bound(P):
    n, B = 512, 32
    codes, scales = _rand_chunks(P, n, B, P)
    out, _, _ = O.dequant_reduce(codes, scales, n, B, 1.0)
    decs = [O.int4_decode(c, n) for c in codes]
    for i in range(n):
        terms = [int(decs[p][i]) * fx(scales[p][i // B]) for p in range(P)]
        exact = sum(terms)
        mag = sum(abs(t) for t in terms)
        assert abs(fx(out[i]) - exact) <= P * F(1, 2 ** 24) * mag * F(1001, 1000)


def test_dequant_reduce_p1_equals_compensated_minus_residual():
    """P = 1, alpha = 1: the receiver's value is d = c - e' exactly (plain
    EF), linking the quantizer's residual with the reducer's dequant."""
    n, B = 4096, 128
    g = (RNG.standard_normal(n) * 1e-3).astype(np.float32)
    e0 = (RNG.standard_normal(n) * 1e-5).astype(np.float32)
    e = e0.copy()
    codes, scales = O.quantize_ef_int4(g, e, B, 0.0, 1.0)
    out, _, _ = O.dequant_reduce([codes], [scales], n, B, 1.0)
    c = g + e0  # numpy fp32 add: IEEE round to nearest
    for i in range(n):
        assert fx(out[i]) == fx(c[i]) - fx(e[i])


def test_dequant_reduce_power_of_two_alpha_is_exact():
    n, B, P = 1024, 64, 8
    codes, scales = _rand_chunks(P, n, B, 99)
    out1, _, _ = O.dequant_reduce(codes, scales, n, B, 1.0)
    out8, _, _ = O.dequant_reduce(codes, scales, n, B, 0.125)
    assert (out8 == out1 * np.float32(0.125)).all()


def test_requant_idempotent():
    n, B = 128 * 64, 128
    g = (RNG.standard_normal(n) * 1e-3).astype(np.float32)
    codes, scales = O.quantize_ef_int4(g, None, B, 0.0, 1.0)
    out, rq_codes, rq_scales = O.dequant_reduce([codes], [scales], n, B, 1.0, requant=True)
    assert (rq_codes == codes).all()
    ulp = np.abs(np.spacing(scales))
    assert (np.abs(rq_scales - scales) <= ulp).all()


def test_requant_is_quantizer_of_reduced_value():
    n, B, P = 2048, 128, 8
    codes, scales = _rand_chunks(P, n, B, 5)
    ef = (RNG.standard_normal(n) * 1e-6).astype(np.float32)
    ef2 = ef.copy()
    out, rq_codes, rq_scales = O.dequant_reduce(codes, scales, n, B, 0.25, requant=True,
                                                rq_ef=ef, rq_beta_e=0.9, rq_beta_r=1.0)
    c2, s2 = O.quantize_ef_int4(out, ef2, B, 0.9, 1.0)
    assert (c2 == rq_codes).all() and (s2 == rq_scales).all()
    assert (ef.view(np.uint32) == ef2.view(np.uint32)).all()


# ---------------------------------------------------------- qwZ int8 --

def test_int8_dequant_bf16_matches_torch_rne():
    n, B = 2048 * 8, 2048
    w = (RNG.standard_normal(n) * 0.02).astype(np.float32)
    codes, scales = O.quant_int8(w, B)
    out32 = O.dequant_int8(codes, scales, B, out_bf16=False)
    out16 = O.dequant_int8(codes, scales, B, out_bf16=True)
    ref32 = torch.from_numpy(codes).float() * torch.from_numpy(scales).repeat_interleave(B)
    assert (torch.from_numpy(out32) == ref32).all()
    ref16 = ref32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (out16 == ref16).all()


def test_int8_roundtrip_error_bound():
    n, B = 2048 * 4, 2048
    w = (RNG.standard_normal(n) * 0.02).astype(np.float32)
    codes, scales = O.quant_int8(w, B)
    out = O.dequant_int8(codes, scales, B, out_bf16=False)
    s = np.repeat(scales, B)
    assert (np.abs(w.astype(np.float64) - out) <= s * (0.5 + 2e-6)).all()


def test_bf16_rne_matches_torch_and_worked_examples(golden_dir):
    G = load(golden_dir, "sr_worked_examples.json")
    for c in G["bf16_rne"]:
        assert O.bf16_rne(bits_f32(int(c["x"], 16))) == int(c["out"], 16), c
    u = RNG.integers(0, 2 ** 32, size=20000, dtype=np.uint64).astype(np.uint32)
    u[:16] = [0, 0x80000000, 0x7F800000, 0xFF800000, 0x7FC00000, 0x00008000, 0x00018000,
              0x7F7FFFFF, 0xFF7FFFFF, 0x3F808000, 0x3F818000, 0x00007FFF, 0x807FFFFF,
              0x7F7F8000, 0x33800000, 0x7FFFFFFF]
    x = u.view(np.float32)
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([O.bf16_rne(v) for v in x], dtype=np.uint16)
    isn = np.isnan(x)
    assert (got[~isn] == ref[~isn]).all()
    assert (got[isn] == 0x7FC0).all()


# ------------------------------------------------------ stochastic rounding --

def test_f16_worked_examples(golden_dir):
    G = load(golden_dir, "f16_worked_examples.json")
    for c in G["rne"]:
        assert O.f16_rne(bits_f32(int(c["x"], 16))) == int(c["out"], 16), c
    for c in G["widen"]:
        assert f32_bits(O.f16_to_f32(int(c["h"], 16))) == int(c["out"], 16), c


def test_f16_widening_exhaustive_matches_numpy():
    """All 65,536 fp16 patterns against numpy's float16 -> float32."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = h.view(np.float16).astype(np.float32)
    got = np.array([O.f16_to_f32(int(v)) for v in h], dtype=np.float32)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan].view(np.uint32) == ref[~nan].view(np.uint32)).all()
    assert (np.signbit(got[nan]) == np.signbit(ref[nan])).all()


def test_f16_rne_matches_numpy_at_every_boundary():
    """fp32 -> fp16 against numpy's float32 -> float16 (round to nearest even)
    at every finite fp16 value, every midpoint between neighbours (exact in
    fp32, so each is a true tie), one fp32 ulp either side of each midpoint,
    both signs, the specials and 100,000 random fp32 patterns."""
    h = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)
    v = h.view(np.float16).astype(np.float32)
    nxt = np.append(v[1:], np.float32(65536.0))
    mid64 = (v.astype(np.float64) + nxt.astype(np.float64)) / 2
    mid = mid64.astype(np.float32)
    assert (mid.astype(np.float64) == mid64).all()  # the midpoints are exact
    x = np.concatenate([v, mid, np.nextafter(mid, np.float32(0)), np.nextafter(mid, np.float32(np.inf))])
    rnd = RNG.integers(0, 2 ** 32, size=100000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    x = np.concatenate([x, -x, rnd, np.array([np.inf, -np.inf, np.nan, 1e30, -1e30], np.float32)])
    with np.errstate(over="ignore", invalid="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    got = np.array([O.f16_rne(t) for t in x], dtype=np.uint16)
    nan = np.isnan(x)
    assert (got[~nan] == ref[~nan]).all()
    assert ((got[nan] & 0x7C00) == 0x7C00).all() and ((got[nan] & 0x3FF) != 0).all()


def test_int8_dequant_f16_is_rne_of_the_fp32_product():
    n, B = 4096 + 77, 256
    w = (RNG.standard_normal(n) * 3.0).astype(np.float32)
    w[:3] = [70000.0, -70000.0, 1e-9]
    codes, scales = O.quant_int8(w, B)
    out = O.dequant_int8(codes, scales, B, out_f16=True)
    prod = codes.astype(np.float32) * np.repeat(scales, B)[:n]
    with np.errstate(over="ignore"):
        ref = prod.astype(np.float16)
    assert out.dtype == np.float16
    assert (out.view(np.uint16) == ref.view(np.uint16)).all()
    assert np.isinf(out[:2]).all()  # 70000 is past the fp16 range


def test_philox_known_answers(golden_dir):
    G = load(golden_dir, "philox4x32_10_kat.json")
    for c in G["cases"]:
        out = O.philox4x32_10([int(v, 16) for v in c["ctr"]], [int(v, 16) for v in c["key"]])
        assert out == [int(v, 16) for v in c["out"]]


def test_sr_worked_examples(golden_dir):
    G = load(golden_dir, "sr_worked_examples.json")
    for c in G["cases"]:
        assert O.sr_round(bits_f32(int(c["x"], 16)), int(c["r16"], 16)) == int(c["out"], 16), c


def test_sr_r16_layout_follows_counter_definition():
    """r16 of index q is half (q & 1) of word (q & 7) >> 1 of Philox at
    counter q >> 3 (pinned here against the KAT-pinned block function)."""
    seed = 0x0123456789ABCDEF
    for q in [0, 1, 7, 8, 15, 2 ** 32 * 8 + 3, 46664928 + 5]:
        c = q >> 3
        w = O.philox4x32_10([c & 0xFFFFFFFF, c >> 32, 0, 0], [seed & 0xFFFFFFFF, seed >> 32])
        word = w[(q & 7) >> 1]
        assert O.sr_r16(seed, q) == ((word >> 16) if q & 1 else (word & 0xFFFF))


@pytest.mark.parametrize("xbits", [0x3F808000, 0x3F8A5A5A, 0xBF8A5A5A, 0x00012345, 0x3DCCCCCD,
                                   0xC2F6E979, 0x3F800000, 0x7F7E1234])
def test_sr_exact_enumeration_is_unbiased(xbits):
    """Mean over all 2^16 random numbers equals x exactly, whatever the
    generator: this pins the rounding rule itself."""
    x = bits_f32(xbits)
    total = F(0)
    outs = set()
    for r in range(1 << 16):
        h = O.sr_round(x, r)
        outs.add(h)
        total += bf16_value(h)
    assert total / (1 << 16) == fx(x)
    # bracketing: truncation toward zero, or the next bf16 away from zero
    rz = xbits >> 16
    assert outs <= {rz, rz + 1}


def test_sr_representable_unchanged_and_special_values():
    for xb in [0x3F800000, 0xC0490000, 0x00010000, 0x7F800000, 0xFF800000, 0x80000000, 0]:
        for r in (0, 1, 0x7FFF, 0x8000, 0xFFFF):
            assert O.sr_round(bits_f32(xb), r) == xb >> 16


def test_sr_r16_stream_statistics():
    N = 1 << 22
    r = O.sr_r16_fill(0, 0, N).astype(np.int64)
    counts = np.bincount(r, minlength=1 << 16)
    exp = N / (1 << 16)
    chi2 = ((counts - exp) ** 2 / exp).sum()
    dof = (1 << 16) - 1
    assert abs(chi2 - dof) < 6 * math.sqrt(2 * dof), chi2
    x = (r - r.mean()) / r.std()
    for lag in (1, 2, 4, 7, 8):
        rho = (x[:-lag] * x[lag:]).mean()
        assert abs(rho) < 6 / math.sqrt(N), (lag, rho)
    r2 = O.sr_r16_fill(1, 0, 4096).astype(np.int64)
    assert (r2 != r[:4096]).mean() > 0.99


def test_sr_accumulation_unbiased_while_rne_drifts():
    """Adding 2^-10 to 1.0 sixty-four times: round-to-nearest bf16 never
    moves (the small update is below half an ulp), stochastic rounding
    reaches 1.0625 on average."""
    n, steps = 1 << 16, 64
    one = torch.ones(n, dtype=torch.bfloat16)
    inc = torch.full((n,), 2.0 ** -10, dtype=torch.bfloat16)
    dst = one.view(torch.int16).numpy().view(np.uint16).copy()
    rne = one.clone()
    for m in range(steps):
        src = inc.view(torch.int16).numpy().view(np.uint16).copy()
        O.sr_accumulate(dst, src, seed=m, counter_base=0)
        rne = (rne.float() + inc.float()).to(torch.bfloat16)
    vals = torch.from_numpy(dst.view(np.int16)).view(torch.bfloat16).double().numpy()
    target = 1.0 + steps * 2.0 ** -10
    sigma = math.sqrt(steps) * (2.0 ** -7) / 2 / math.sqrt(n)
    assert abs(vals.mean() - target) < 4 * sigma, (vals.mean(), target, sigma)
    assert (rne == 1.0).all()


def test_sr_shard_equals_slice_of_full_run():
    n, P, rank = 8 * 4099, 8, 3
    shard = n // P
    off = rank * shard
    full = np.zeros(n, np.uint16)
    part = np.zeros(shard, np.uint16)
    for m in range(4):
        src = (torch.randn(n, generator=torch.Generator().manual_seed(m)) * 1e-4).to(torch.bfloat16)
        s16 = src.view(torch.int16).numpy().view(np.uint16)
        O.sr_accumulate(full, s16.copy(), seed=m, counter_base=0)
        O.sr_accumulate(part, s16[off:off + shard].copy(), seed=m, counter_base=off)
    assert (full[off:off + shard] == part).all()


def test_sr_zero_src_clears_only_the_slice_read():
    n = 100
    dst = np.zeros(n, np.uint16)
    src = np.full(n + 10, 0x3F80, np.uint16)
    view = src[:n]
    O.sr_accumulate(dst, view, seed=1, counter_base=0, zero_src=True)
    assert (src[:n] == 0).all() and (src[n:] == 0x3F80).all() and (dst == 0x3F80).all()


# ------------------------------------------------ communication volume --

def test_volume_closed_form_against_pages(golden_dir):
    G = load(golden_dir, "volume_pages.json")
    M = 1 << 30
    zero3, zpp = O.volume_bytes(M, 2 ** 31, 2 ** 31)  # scale terms: one block each
    unit = 2 * M  # "M" on the pages counts fp16 elements
    assert zero3 == G["zero3_fp16_units"] * unit
    assert zpp - 8 == G["zeropp_fp16_units"] * unit
    assert (zpp - 8) == (G["zeropp_parts"]["qwz"] + G["zeropp_parts"]["hpz"]
                         + G["zeropp_parts"]["qgz"]) * unit
    assert zero3 / (zpp - 8) == G["reduction"]
    # with the real block sizes (int8 weights B = 2048, int4 grads B = 128)
    M = 850454528
    zero3, zpp = O.volume_bytes(M, 2048, 128)
    units = zpp / (2 * M)
    assert abs(units - (0.75 + 2 / 2048 + 2 / 128)) < 1e-12
    assert 3.9 < zero3 / zpp < 3.92


# ------------------------------------------- ZeRO++ hierarchical order --

def test_zeropp_slots_worked(golden_dir):
    G = load(golden_dir, "zeropp_order_worked.json")["slots"]
    assert O.zeropp_slots(4, 2) == G["intra4_inter2"]
    assert O.zeropp_slots(8, 4) == G["intra8_inter4"]
    assert O.zeropp_slots(1, 3) == G["intra1_inter3"]
    assert O.zeropp_slots(3, 1) == G["intra3_inter1"]


def test_quantize_permuted_worked(golden_dir):
    G = load(golden_dir, "zeropp_order_worked.json")["quantize_permuted"]
    g = np.array(G["g"], np.float32)
    ef = np.zeros(g.size, np.float32)
    codes, scales = O.quantize_ef_int4_permuted(g, ef, G["block"], G["beta_e"], G["beta_r"],
                                                G["slot_of_part"])
    assert codes.tolist() == hexbytes(G["codes"]).tolist()
    assert scales.tolist() == G["scales"]
    assert ef.tolist() == G["ef_after"]


def test_quantize_permuted_identity_order_is_the_plain_quantizer():
    n, B = 4096, 64
    g = (RNG.standard_normal(n) * 1e-3).astype(np.float32)
    e1 = (RNG.standard_normal(n) * 1e-4).astype(np.float32)
    e2 = e1.copy()
    c1, s1 = O.quantize_ef_int4_permuted(g, e1, B, 0.9, 1.0, list(range(8)))
    c2, s2 = O.quantize_ef_int4(g, e2, B, 0.9, 1.0)
    assert (c1 == c2).all() and (s1.view(np.uint32) == s2.view(np.uint32)).all()
    assert (e1.view(np.uint32) == e2.view(np.uint32)).all()
    with pytest.raises(O.OracleArgumentError):  # not a permutation
        O.quantize_ef_int4_permuted(g, None, B, 0.9, 1.0, [0, 1, 2, 3, 4, 5, 6, 6])
    with pytest.raises(O.OracleArgumentError):  # partitions not whole blocks
        O.quantize_ef_int4_permuted(g[:4096 - 8 * 16], None, B, 0.9, 1.0, list(range(8)))


def _chunk(codes, scales, lo, m, B):
    """Codes and scales of elements [lo, lo + m) of a quantized buffer."""
    return codes[lo // 2:(lo + m) // 2], scales[lo // B:(lo + m) // B]


@pytest.mark.parametrize("intra,inter", [(4, 2), (2, 3)])
def test_two_level_exchange_delivers_each_rank_its_partition(intra, inter):
    """Simulate hierarchical qgZ on the CPU with the oracle: every rank
    quantizes its gradient into ZeRO++'s order; the intra-node all-to-all
    sends chunk j of a buffer to local rank j, which reduces the chunks of
    its node and requantizes; the inter-node all-to-all sends sub-chunk i of
    that to node i, which reduces over nodes.  Rank r must end with exactly
    what the natural-order quantizer and the same two-level reduction give
    for partition r -- the meaning of the order, not its formula."""
    R, B, part = intra * inter, 32, 256
    n = R * part
    rng = np.random.default_rng(intra * 10 + inter)
    grads = [(rng.standard_normal(n) * 1e-3).astype(np.float32) for _ in range(R)]
    ef0 = [(rng.standard_normal(n) * 1e-5).astype(np.float32) for _ in range(R)]
    slots = O.zeropp_slots(intra, inter)
    rank = lambda node, local: node * intra + local
    # permuted path, as the exchanges would run it
    ef_p = [e.copy() for e in ef0]
    q = [O.quantize_ef_int4_permuted(grads[r], ef_p[r], B, 0.9, 1.0, slots) for r in range(R)]
    chunk = inter * part  # elements per intra-node chunk
    lvl1 = {}
    for node in range(inter):
        for j in range(intra):
            recv = [_chunk(*q[rank(node, i)], j * chunk, chunk, B) for i in range(intra)]
            _, rc, rs = O.dequant_reduce([c for c, _ in recv], [s for _, s in recv], chunk, B, 1.0,
                                         want_out=False, requant=True)
            lvl1[node, j] = (rc, rs)
    final = {}
    for node in range(inter):
        for j in range(intra):
            recv = [_chunk(*lvl1[other, j], node * part, part, B) for other in range(inter)]
            out, _, _ = O.dequant_reduce([c for c, _ in recv], [s for _, s in recv], part, B,
                                         1.0 / R)
            final[rank(node, j)] = out
    # natural order: partition r reduced over the ranks of each node, then over nodes
    ef_n = [e.copy() for e in ef0]
    nat = [O.quantize_ef_int4(grads[r], ef_n[r], B, 0.9, 1.0) for r in range(R)]
    for node in range(inter):
        for j in range(intra):
            r = rank(node, j)
            sub = []
            for other in range(inter):
                recv = [_chunk(*nat[rank(other, i)], r * part, part, B) for i in range(intra)]
                _, rc, rs = O.dequant_reduce([c for c, _ in recv], [s for _, s in recv], part, B,
                                             1.0, want_out=False, requant=True)
                sub.append((rc, rs))
            out, _, _ = O.dequant_reduce([c for c, _ in sub], [s for _, s in sub], part, B, 1.0 / R)
            assert (final[r].view(np.uint32) == out.view(np.uint32)).all(), (intra, inter, r)
    for r in range(R):  # the error feedback stays in natural order
        assert (ef_p[r].view(np.uint32) == ef_n[r].view(np.uint32)).all()


# -------------------------------------- per-tensor SR loop (llm.c ZeRO-2) --

def _seg_fixture(golden_dir):
    G = load(golden_dir, "sr_segments_worked.json")
    h = lambda lst: np.array([int(x, 16) for x in lst], np.uint16)
    segs = []
    for c in G["segments"]:
        segs.append((h(c["dst"]), h(c["src"]), c["n"], c["src_offset"], c["seed"],
                     c["counter_base"]))
    return G, segs


@pytest.mark.parametrize("zero_src", [False, True])
def test_sr_segments_worked(golden_dir, zero_src):
    G, segs = _seg_fixture(golden_dir)
    src_before = [s[1].copy() for s in segs]
    O.sr_accumulate_segments(segs, zero_src=zero_src)
    thr = int(G["round_up_threshold"], 16)
    for c, (dst, src, n, off, seed, cb), before in zip(G["segments"], segs, src_before):
        want = []
        for i, v in enumerate(c["dst_after"]):
            if v == "r16":  # the one inexact sum: 1 + 2^-9
                up = O.sr_r16(seed, cb + i) >= thr
                want.append(0x3F81 if up else 0x3F80)
            else:
                want.append(int(v, 16))
        assert dst.tolist() == want, c
        if zero_src:
            assert (src == 0).all()
        else:
            assert (src == before).all()


def test_sr_segments_equal_the_per_tensor_loop():
    """Random segments with distinct offsets, seeds and counter bases: the
    segment loop equals, per tensor, the SR add of the slice followed by
    clearing the whole reduced buffer."""
    rng = np.random.default_rng(5)
    segs, ref = [], []
    for i in range(6):
        ln = int(rng.integers(1, 40)) * 8
        off = int(rng.integers(0, ln // 8)) * 8
        n = int(rng.integers(0, ln - off + 1))
        dst = (torch.randn(n + 3, generator=torch.Generator().manual_seed(i)) * 1e-2).to(
            torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
        src = (torch.randn(ln, generator=torch.Generator().manual_seed(100 + i)) * 1e-4).to(
            torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
        seed, cb = int(rng.integers(0, 2 ** 63)), int(rng.integers(0, 2 ** 40))
        segs.append((dst, src, n, off, seed, cb))
        ref.append((dst.copy(), src.copy(), n, off, seed, cb))
    O.sr_accumulate_segments(segs, zero_src=True)
    for (dst, src, n, off, seed, cb), (rd, rs, _, _, _, _) in zip(segs, ref):
        O.sr_accumulate(rd[:n], rs[off:off + n].copy(), seed, cb)
        rs[:] = 0
        assert (dst == rd).all() and (src == rs).all()


def test_oracle_rejects_bad_arguments():
    g = np.zeros(64, np.float32)
    for block in (0, 3, 8192):
        with pytest.raises(ValueError):
            O.quantize_ef_int4(g, None, block, 0.0, 1.0)
    L = O.lib()
    # called directly: NULL outputs and oversized blocks are refused, nothing written
    assert L.orc_quantize_ef_int4(g.ctypes.data, 0, None, 64, 8192, 0.0, 1.0, None, None) != 0
    assert L.orc_quantize_ef_int4(g.ctypes.data, 0, None, 64, 32, 0.0, 1.0, None, None) != 0
    codes = np.full(64, -86, np.int8)
    assert L.orc_quant_int8(g.ctypes.data, 0, 64, 4097, codes.ctypes.data, None) != 0
    assert (codes == np.int8(-86)).all()
    assert L.orc_zeropp_slots(0, 2, None) != 0


# ---------------------------------- per-parameter receive side (segments) --

def test_dequant_reduce_segments_worked(golden_dir):
    G = load(golden_dir, "dequant_reduce_segments_worked.json")
    segs = [(hexbytes(c["codes"]), np.array(c["scales"], np.float32), c["n"], c["codes_stride"],
             c["scales_stride"]) for c in G["segments"]]
    res = O.dequant_reduce_segments(segs, G["P"], G["block"], G["alpha"], want_out=True,
                                    requant=True)
    for c, (out, rqc, rqs) in zip(G["segments"], res):
        assert out.tolist() == c["out"], c
        assert rqc.tolist() == hexbytes(c["rq_codes"]).tolist(), c
        assert rqs.tolist() == c["rq_scales"], c


def test_dequant_reduce_segments_equal_per_tensor_reduces():
    """Random tensors of ragged sizes and padded strides: every segment
    equals the plain reduce of its P chunks; requant EF per segment."""
    rng = np.random.default_rng(9)
    P, B = 3, 32
    segs, chunks, efs = [], [], []
    for i in range(5):
        n = int(rng.integers(1, 300))
        cs = (n + 1) // 2 + int(rng.integers(0, 5))
        ss = -(-n // B) + int(rng.integers(0, 3))
        codes = rng.integers(0, 256, size=(P - 1) * cs + (n + 1) // 2, dtype=np.uint8)
        scales = (rng.random((P - 1) * ss + -(-n // B)) * 1e-3).astype(np.float32)
        segs.append((codes, scales, n, cs, ss))
        chunks.append(([codes[p * cs:p * cs + (n + 1) // 2] for p in range(P)],
                       [scales[p * ss:p * ss + -(-n // B)] for p in range(P)], n))
        efs.append((rng.standard_normal(n) * 1e-5).astype(np.float32))
    efs_ref = [e.copy() for e in efs]
    res = O.dequant_reduce_segments(segs, P, B, 0.25, want_out=True, requant=True, rq_efs=efs,
                                    rq_beta_e=0.9, rq_beta_r=1.0)
    for (cl, sl, n), (out, rqc, rqs), e_ref, e in zip(chunks, res, efs_ref, efs):
        o2, c2, s2 = O.dequant_reduce(cl, sl, n, B, 0.25, want_out=True, requant=True, rq_ef=e_ref,
                                      rq_beta_e=0.9, rq_beta_r=1.0)
        assert (out.view(np.uint32) == o2.view(np.uint32)).all()
        assert (rqc == c2).all() and (rqs.view(np.uint32) == s2.view(np.uint32)).all()
        assert (e.view(np.uint32) == e_ref.view(np.uint32)).all()
