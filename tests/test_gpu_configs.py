"""GPU parity at the full sizes of the five workloads, through the same entry
points and launch configuration the benchmark times.

Every step of the path is block-local, so the oracle can recompute any set of
blocks on its own: for a sampled output block it recomputes every upstream
block it depends on (the 8 peer blocks of a first-level reduce, the 4 x 8
blocks behind a second-level output), starting from the seeded generator's
inputs and carrying its own error-feedback state across steps -- no oracle
input ever comes from a GPU output.  Blocks gathered into one array stay
independent, so each oracle call runs on the concatenation.

Workloads (seeded, synthetic; no dataset):
  4 ranks x bf16[2^20], N(0, 1e-3) with 1 % outliers x50, block 256, EF beta 1,
      3 steps, full all-to-all of 2^18-element chunks with alpha 1/4 -- fully
      compared (small);
  GPT-2 124M bf16 gradient buffer, 8 micro-batches N(0, 1e-4) accumulated with
      stochastic rounding (seed = micro-batch), full buffer and rank-3-of-8 shard;
  ~0.85B Llama-2-style bf16 weights N(0, 0.02), int8 block 2048, quantize + dequantize;
  ~0.85B fp32 gradient N(0, 1e-3), heavy-tailed tensors, EF int4 block 128,
      beta 0.9, 10 steps, 8-way reduce alpha 1/8;
  ~7.5B fp32 gradient, same recipe, 2 steps: EF quantize, 8-way reduce-requant,
      4-way reduce alpha 1/32.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
from tests.gpu_helpers import assert_bits_equal, to_gpu, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import weight_communication_zero_amd  # noqa: F401
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def Z():
    from weight_communication_zero_amd import zq
    return zq


def gather_blocks(t: torch.Tensor, blocks: np.ndarray, width: int) -> np.ndarray:
    """Host copy of the listed blocks (each `width` elements) of a flat tensor."""
    idx = torch.from_numpy(blocks.astype(np.int64)).to(t.device)
    return to_host(t.view(-1, width).index_select(0, idx).reshape(-1))


def int4_block_bytes(codes: torch.Tensor, blocks: np.ndarray, B: int) -> np.ndarray:
    return gather_blocks(codes, blocks, B // 2)


def assert_sr_brackets(out: torch.Tensor, x: torch.Tensor, what: str):
    """Every stochastically rounded bf16 output is x truncated toward zero
    (its top 16 bits) or the next bf16 away from zero (one more), and x
    itself when bf16 holds it exactly -- over the whole buffer."""
    xb = x.view(torch.int32).to(torch.int64) & 0xFFFFFFFF
    ob = out.view(torch.int16).to(torch.int64) & 0xFFFF
    d = ob - (xb >> 16)
    assert bool(((d == 0) | (d == 1)).all()), f"{what}: a result outside [RZ(x), RZ(x) + 1 ulp]"
    assert bool((d[(xb & 0xFFFF) == 0] == 0).all()), f"{what}: a representable sum moved"


# ------------------------------------------------------------------ 4 ranks --

def test_four_ranks_bf16_block256_full_compare():
    P, n, B, steps = 4, 1 << 20, 256, 3
    nc = n // P
    ef_o = [np.zeros(n, np.float32) for _ in range(P)]
    ef_g = [torch.zeros(n, dtype=torch.float32, device="cuda") for _ in range(P)]
    for step in range(steps):
        codes_o, scales_o, codes_g, scales_g = [], [], [], []
        for r in range(P):
            g = synth.grad_with_outliers(n, 1e-3, 0.01, 50.0, synth.seed_for("c1", "grad", r, step),
                                         torch.bfloat16)
            gh = g.view(torch.int16).numpy().view(np.uint16)
            c_o, s_o = O.quantize_ef_int4(gh, ef_o[r], B, 1.0, 1.0)
            c = torch.empty(n // 2, dtype=torch.uint8, device="cuda")
            s = torch.empty(n // B, dtype=torch.float32, device="cuda")
            Z().zq_quantize_ef_int4(g.cuda(), ef_g[r], B, 1.0, 1.0, c, s)
            codes_o.append(c_o), scales_o.append(s_o), codes_g.append(c), scales_g.append(s)
        torch.cuda.synchronize()
        for r in range(P):
            assert_bits_equal(to_host(codes_g[r]), codes_o[r], f"step {step} rank {r} codes")
            assert_bits_equal(to_host(scales_g[r]), scales_o[r], f"step {step} rank {r} scales")
            assert_bits_equal(to_host(ef_g[r]), ef_o[r], f"step {step} rank {r} ef")
        for dst in range(P):  # all-to-all: destination dst receives chunk dst of every rank
            cs_o = [c[dst * nc // 2:(dst + 1) * nc // 2] for c in codes_o]
            ss_o = [s[dst * nc // B:(dst + 1) * nc // B] for s in scales_o]
            out_o, _, _ = O.dequant_reduce(cs_o, ss_o, nc, B, 0.25)
            out = torch.empty(nc, dtype=torch.float32, device="cuda")
            Z().zq_dequant_reduce([c[dst * nc // 2:(dst + 1) * nc // 2] for c in codes_g],
                                  [s[dst * nc // B:(dst + 1) * nc // B] for s in scales_g], nc, B,
                                  0.25, out=out)
            torch.cuda.synchronize()
            assert_bits_equal(to_host(out), out_o, f"step {step} reduce at rank {dst}")


# --------------------------------------------------------------- GPT-2 SR --

def test_gpt2_sr_accumulation_full_buffer_and_rank3_shard():
    tensors = synth.gpt2_124m()
    n = synth.total(tensors)
    P, rank = 8, 3
    shard = n // P
    off = rank * shard
    rng = np.random.default_rng(2)
    W = 1024
    starts = np.unique(np.concatenate([[0, n - W, off, off + shard - W],
                                       rng.integers(0, n - W, size=60)]))
    dst = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    dsh = torch.zeros(shard, dtype=torch.bfloat16, device="cuda")
    src = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    win_o = {int(s0): np.zeros(W, np.uint16) for s0 in starts}
    for m in range(8):
        synth.fill_model(src, tensors, std=1e-4, seed=synth.seed_for("gpt2", "grad", mb=m))
        src_host = {int(s0): to_host(src[s0:s0 + W]).copy() for s0 in starts}
        x = dst.float() + src.float()  # the fp32 sum (round to nearest) the kernel rounds
        Z().zq_sr_accumulate(dst, src, seed=m, counter_base=0)
        assert_sr_brackets(dst, x, f"GPT-2 full buffer, micro-batch {m}")
        del x
        Z().zq_sr_accumulate(dsh, src[off:off + shard], seed=m, counter_base=off)
        for s0 in starts:
            O.sr_accumulate(win_o[int(s0)], src_host[int(s0)], seed=m, counter_base=int(s0))
    torch.cuda.synchronize()
    assert torch.equal(dst[off:off + shard].view(torch.int16), dsh.view(torch.int16)), \
        "rank-3 shard differs from the same slice of the full-buffer accumulation"
    for s0 in starts:
        assert_bits_equal(to_host(dst[s0:s0 + W]), win_o[int(s0)], f"SR window at {s0}")



def test_sr_past_the_xcd_ordered_map_single_and_batched():
    """SR over 3 full blocks of 131,072 one-tile workgroups (where the
    streaming kernels take XCD-contiguous runs), a trailing partial block of
    12,345 workgroups in dispatch order and a ragged last tile of 333
    elements.  First call: dst = 0, so every output must equal its src value
    exactly (a tile skipped or visited twice shows); second call: windows
    against the oracle at the first and last tiles and on both sides of
    every run boundary, and the bracketing property over the whole buffer;
    zero_src must clear all of src.  Then the same through the batched entry
    point, as one large segment plus a small one."""
    tile, run = 1024, 131072
    n = 3 * run * tile + 12345 * tile + 333
    gen = torch.Generator(device="cuda").manual_seed(11)
    src = torch.randn(n, device="cuda", generator=gen).to(torch.bfloat16)
    dst = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    Z().zq_sr_accumulate(dst, src, seed=1, counter_base=0)
    torch.cuda.synchronize()
    assert torch.equal(dst.view(torch.int16), src.view(torch.int16)), "a tile was missed or repeated"
    W = 1024
    edges = [0, n - W, n - 333 - W]
    for b in range(1, 4):
        edges += [b * run * tile - W, b * run * tile]
        edges += [(b - 1) * run * tile + x * 16384 * tile + o for x in range(1, 8) for o in (-W, 0)]
    rng = np.random.default_rng(12)
    edges += list(rng.integers(0, n - W, size=24))
    starts = sorted(set(int(e) for e in edges))
    src2 = (torch.randn(n, device="cuda", generator=gen) * 1e-2).to(torch.bfloat16)
    win_d = {s0: to_host(dst[s0:s0 + W]).copy() for s0 in starts}
    win_s = {s0: to_host(src2[s0:s0 + W]).copy() for s0 in starts}
    x = dst.float() + src2.float()
    Z().zq_sr_accumulate(dst, src2, seed=(1 << 40) + 7, counter_base=3, zero_src=True)
    torch.cuda.synchronize()
    assert_sr_brackets(dst, x, "large SR")
    del x
    assert int(torch.count_nonzero(src2.view(torch.int16))) == 0, "zero_src left src elements"
    for s0 in starts:
        O.sr_accumulate(win_d[s0], win_s[s0], seed=(1 << 40) + 7, counter_base=3 + s0)
        assert_bits_equal(to_host(dst[s0:s0 + W]), win_d[s0], f"large SR window at {s0}")
    # batched: one large segment and one small one, reduced buffers cleared
    small = 5000
    dst_b = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    dst_s = torch.zeros(small, dtype=torch.bfloat16, device="cuda")
    red_s = torch.randn(4 * small, device="cuda", generator=gen).to(torch.bfloat16)
    want_s = red_s[2 * small:3 * small].clone()
    src3 = src.clone()
    Z().zq_sr_accumulate_batched([(dst_b, src3, n, 0, 9, 0), (dst_s, red_s, small, 2 * small, 10, 77)],
                                 zero_src=True)
    torch.cuda.synchronize()
    assert torch.equal(dst_b.view(torch.int16), src.view(torch.int16)), "batched: tile missed or repeated"
    assert torch.equal(dst_s.view(torch.int16), want_s.view(torch.int16))
    assert int(torch.count_nonzero(src3.view(torch.int16))) == 0
    assert int(torch.count_nonzero(red_s.view(torch.int16))) == 0


# ------------------------------------------------------------ qwZ 0.85B --

@pytest.mark.parametrize("wdt", [torch.bfloat16, torch.float16])
def test_int8_weights_0p85b_sampled_blocks(wdt):
    """qwZ on the 0.85B model's weights, bf16 and the pages' fp16: every
    output written, sampled blocks (first, last, 254 random) against the
    oracle, the dequantized weights in the input's dtype."""
    tensors = synth.llama_0p85b()
    n = synth.total(tensors)
    B = 2048
    w = torch.empty(n, dtype=wdt, device="cuda")
    synth.fill_model(w, tensors, std=0.02, seed=synth.seed_for("llama0p85b", "weights"))
    codes = torch.empty(n, dtype=torch.int8, device="cuda")
    scales = torch.empty(n // B, dtype=torch.float32, device="cuda")
    wd = torch.empty(n, dtype=wdt, device="cuda")
    # poison: -128 is never a code (clamp to +-127), NaN never a finite block's scale
    codes.fill_(-128)
    scales.fill_(float("nan"))
    wd.fill_(float("nan"))
    Z().zq_quant_int8(w, B, codes, scales)
    Z().zq_dequant_int8(codes, scales, B, wd)
    torch.cuda.synchronize()
    assert not bool((codes == -128).any()), "int8 codes left unwritten"
    assert not bool(torch.isnan(scales).any()), "int8 scales left unwritten"
    assert not bool(torch.isnan(wd).any()), "dequantized weights left unwritten"
    nb = n // B
    rng = np.random.default_rng(3)
    blocks = np.unique(np.concatenate([[0, nb - 1], rng.integers(0, nb, size=254)]))
    w_h = gather_blocks(w, blocks, B)
    c_o, s_o = O.quant_int8(w_h, B)
    assert_bits_equal(gather_blocks(codes, blocks, B).view(np.uint8), c_o.view(np.uint8), "codes")
    assert_bits_equal(to_host(scales)[blocks], s_o, "scales")
    f16 = wdt == torch.float16
    assert_bits_equal(gather_blocks(wd, blocks, B),
                      O.dequant_int8(c_o, s_o, B, out_bf16=not f16, out_f16=f16),
                      f"dequantized {wdt}")


# ------------------------------------------- qgZ + LoCo: 0.85B and 7.5B --

def run_two_level(tensors, tag, steps, levels, n_sample, seed, beta=(0.9, 1.0), rq_beta=None,
                  reset_every=None, gdt=torch.float32):
    """EF quantize of the whole gradient, then level-1 reduce over P1 chunks
    (with requant when there is a second level), then level-2 reduce over P2
    sub-chunks; sampled blocks checked at every step.  LoCo variants: `beta`
    = (beta_e, beta_r) of the EF update, `rq_beta` turns on an EF buffer at
    the requant (the per-parameter inter-level EF buffer), `reset_every`
    zeroes the EF buffers every that many steps, `gdt` is the gradient's
    dtype."""
    M = synth.total(tensors)
    B = 128
    P1 = 8
    n1 = M // P1
    nb1 = n1 // B
    two = levels == 2
    P2 = 4 if two else 1
    n2 = n1 // P2
    nb2 = n2 // B
    alpha1, alpha2 = (1.0, 1.0 / 32) if two else (1.0 / 8, None)

    rng = np.random.default_rng(seed)
    S = np.unique(np.concatenate([[0, nb2 - 1], rng.integers(0, nb2, size=n_sample)]))
    L1 = (np.arange(P2)[:, None] * nb2 + S[None, :]).reshape(-1) if two else S  # level-1 blocks
    L0 = (np.arange(P1)[:, None] * nb1 + L1[None, :]).reshape(-1)  # EF-quantize blocks

    g = torch.empty(M, dtype=gdt, device="cuda")
    ef = torch.zeros(M, dtype=torch.float32, device="cuda")
    codes = torch.empty(M // 2, dtype=torch.uint8, device="cuda")
    scales = torch.empty(M // B, dtype=torch.float32, device="cuda")
    chunks_c = [codes[j * n1 // 2:(j + 1) * n1 // 2] for j in range(P1)]
    chunks_s = [scales[j * nb1:(j + 1) * nb1] for j in range(P1)]
    if two:
        rqc = torch.empty(n1 // 2, dtype=torch.uint8, device="cuda")
        rqs = torch.empty(nb1, dtype=torch.float32, device="cuda")
        out = torch.empty(n2, dtype=torch.float32, device="cuda")
        sub_c = [rqc[i * n2 // 2:(i + 1) * n2 // 2] for i in range(P2)]
        sub_s = [rqs[i * nb2:(i + 1) * nb2] for i in range(P2)]
    else:
        out = torch.empty(n1, dtype=torch.float32, device="cuda")
    rq_ef = torch.zeros(n1, dtype=torch.float32, device="cuda") if rq_beta else None
    rq_be, rq_br = rq_beta or (0.0, 1.0)

    ef_o = np.zeros(L0.size * B, np.float32)  # oracle EF of the tracked blocks
    rq_ef_o = np.zeros(L1.size * B, np.float32) if rq_beta else None
    for step in range(steps):
        if reset_every and step and step % reset_every == 0:
            ef.zero_()
            ef_o[:] = 0.0
            if rq_beta:
                rq_ef.zero_()
                rq_ef_o[:] = 0.0
        synth.fill_model(g, tensors, std=1e-3, seed=synth.seed_for(tag, "grad", step=step),
                         heavy_tails=True)
        # Poison every output with values the kernels never produce for
        # finite inputs (nibble 8 = -8, NaN), so the whole-buffer checks below
        # see any tile a launch geometry failed to visit.
        codes.fill_(0x88)
        scales.fill_(float("nan"))
        out.fill_(float("nan"))
        if two:
            rqc.fill_(0x88)
            rqs.fill_(float("nan"))
        Z().zq_quantize_ef_int4(g, ef, B, beta[0], beta[1], codes, scales)
        if two:
            Z().zq_dequant_reduce(chunks_c, chunks_s, n1, B, alpha1, rq_codes=rqc, rq_scales=rqs,
                                  rq_ef=rq_ef, rq_beta_e=rq_be, rq_beta_r=rq_br)
            Z().zq_dequant_reduce(sub_c, sub_s, n2, B, alpha2, out=out)
        else:
            Z().zq_dequant_reduce(chunks_c, chunks_s, n1, B, alpha1, out=out)
        torch.cuda.synchronize()
        what = f"{tag} step {step}"
        for name, c in (("codes", codes),) + ((("requant codes", rqc),) if two else ()):
            assert not bool(((c & 0x0F) == 8).any() | ((c >> 4) == 8).any()), \
                what + f": {name} left unwritten (nibble -8 present)"
        for name, t in (("scales", scales), ("reduced sum", out)) + \
                ((("requant scales", rqs),) if two else ()):
            assert not bool(torch.isnan(t).any()), what + f": {name} left unwritten (NaN present)"

        # oracle: EF quantize of the tracked blocks
        g_h = gather_blocks(g, L0, B)
        c0, s0 = O.quantize_ef_int4(g_h, ef_o, B, beta[0], beta[1])
        assert_bits_equal(int4_block_bytes(codes, L0, B), c0, what + " codes")
        assert_bits_equal(to_host(scales)[L0], s0, what + " scales")
        assert_bits_equal(gather_blocks(ef, L0, B), ef_o, what + " ef")
        # level 1: chunk j of the gathered layout = blocks j*nb1 + L1
        m1 = L1.size * B
        cj = [c0[j * m1 // 2:(j + 1) * m1 // 2] for j in range(P1)]
        sj = [s0[j * L1.size:(j + 1) * L1.size] for j in range(P1)]
        if two:
            _, rc_o, rs_o = O.dequant_reduce(cj, sj, m1, B, alpha1, want_out=False, requant=True,
                                             rq_ef=rq_ef_o, rq_beta_e=rq_be, rq_beta_r=rq_br)
            assert_bits_equal(int4_block_bytes(rqc, L1, B), rc_o, what + " requant codes")
            assert_bits_equal(to_host(rqs)[L1], rs_o, what + " requant scales")
            if rq_beta:
                assert_bits_equal(gather_blocks(rq_ef, L1, B), rq_ef_o, what + " requant ef")
            m2 = S.size * B
            ci = [rc_o[i * m2 // 2:(i + 1) * m2 // 2] for i in range(P2)]
            si = [rs_o[i * S.size:(i + 1) * S.size] for i in range(P2)]
            out_o, _, _ = O.dequant_reduce(ci, si, m2, B, alpha2)
        else:
            out_o, _, _ = O.dequant_reduce(cj, sj, m1, B, alpha1)
        got = gather_blocks(out, S, B)
        assert np.allclose(got, out_o, rtol=1e-6, atol=0), what + " reduced sum (1e-6)"
        assert_bits_equal(got, out_o, what + " reduced sum")


def test_qgz_loco_0p85b_ten_steps_sampled():
    run_two_level(synth.llama_0p85b(), "llama0p85b", steps=10, levels=1, n_sample=64, seed=4)


def test_qgz_loco_7p5b_two_level_sampled():
    run_two_level(synth.llama_7p5b(), "llama7p5b", steps=2, levels=2, n_sample=24, seed=5)


def test_loco_requant_ef_7p5b_two_level_sampled():
    """LoCo variant: an EF buffer at the intra-node requant as well (beta 0.9)."""
    run_two_level(synth.llama_7p5b(), "llama7p5b", steps=3, levels=2, n_sample=16, seed=6,
                  rq_beta=(0.9, 1.0))


def test_qgz_loco_0p85b_fp16_gradients_sampled():
    """fp16 gradients (the LoCo kernel's half loads) through the whole step
    at full size, past the XCD-ordered workgroup map."""
    run_two_level(synth.llama_0p85b(), "llama0p85b", steps=3, levels=1, n_sample=48, seed=8,
                  gdt=torch.float16)


def test_loco_moving_average_with_reset_0p85b_sampled():
    """LoCo variant: moving-average EF (beta, 1 - beta) with the EF buffer
    reset every 4 steps (a caller-side zeroing between calls)."""
    run_two_level(synth.llama_0p85b(), "llama0p85b", steps=10, levels=1, n_sample=48, seed=7,
                  beta=(0.9, 0.1), reset_every=4)


# ------------------------------- llm.c per-tensor ZeRO-2 accumulate, batched --

def gpt2_segments(grads, shards, tensors, rank, P, mb):
    """llm.c's per-tensor loop on the flat GPT-2 buffers: tensor i's reduced
    buffer is grads[off_i : off_i + nelem_i]; its shard (nelem_i / P
    elements at rank * n_i) accumulates into shards[soff_i : soff_i + n_i];
    the random numbers are those of the shard's global indices."""
    segs, off, soff = [], 0, 0
    for i, t in enumerate(tensors):
        n = t.numel // P
        segs.append((shards[soff:soff + n], grads[off:off + t.numel], n, rank * n,
                     (mb << 16) + i, off + rank * n))
        off += t.numel
        soff += n
    return segs


def test_gpt2_per_tensor_zero2_batched():
    tensors = synth.gpt2_124m()
    n = synth.total(tensors)
    P, rank = 8, 3
    grads = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    grads_b = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    shards = torch.zeros(n // P, dtype=torch.bfloat16, device="cuda")
    shards_b = torch.zeros(n // P, dtype=torch.bfloat16, device="cuda")
    rng = np.random.default_rng(8)
    pick = sorted(set([0, len(tensors) - 1] + list(rng.integers(0, len(tensors), size=10))))
    exp = {}
    for mb in range(8):
        synth.fill_model(grads, tensors, std=1e-4, seed=synth.seed_for("gpt2", "grad", mb=mb))
        grads_b.copy_(grads)
        segs = gpt2_segments(grads, shards, tensors, rank, P, mb)
        host = {i: (to_host(segs[i][1]).copy()) for i in pick}
        Z().zq_sr_accumulate_batched(segs, zero_src=True)
        for dst, src, m, off, seed, cb in gpt2_segments(grads_b, shards_b, tensors, rank, P, mb):
            Z().zq_sr_accumulate(dst, src[off:off + m], seed, cb)
            src.zero_()
        torch.cuda.synchronize()
        assert int(grads.view(torch.int16).abs().max()) == 0, "reduced buffers not cleared"
        for i in pick:
            _, _, m, off, seed, cb = segs[i]
            if i not in exp:
                exp[i] = np.zeros(m, np.uint16)
            O.sr_accumulate(exp[i], host[i][off:off + m].copy(), seed, cb)
    assert torch.equal(shards.view(torch.int16), shards_b.view(torch.int16)), \
        "batched call differs from the per-tensor loop"
    segs = gpt2_segments(grads, shards, tensors, rank, P, 0)
    for i in pick:
        assert_bits_equal(to_host(segs[i][0]), exp[i], f"tensor {i} ({tensors[i].name}) shard")


def test_per_tensor_batched_quantize_equals_flat_call_0p85b():
    """DeepSpeed-style per-parameter EF quantize of the 129 tensors of the
    ~0.85B model in one batched call equals the flat call over the same
    buffer bit for bit (every tensor is whole 128-element blocks), over 3 steps
    of EF evolution."""
    tensors = synth.llama_0p85b()
    M = synth.total(tensors)
    B = 128
    g = torch.empty(M, dtype=torch.float32, device="cuda")
    ef_a = torch.zeros(M, dtype=torch.float32, device="cuda")
    ef_b = torch.zeros(M, dtype=torch.float32, device="cuda")
    ca = torch.empty(M // 2, dtype=torch.uint8, device="cuda")
    cb = torch.empty(M // 2, dtype=torch.uint8, device="cuda")
    sa = torch.empty(M // B, dtype=torch.float32, device="cuda")
    sb = torch.empty(M // B, dtype=torch.float32, device="cuda")
    segs, off = [], 0
    for t in tensors:
        n = t.numel
        segs.append((g[off:off + n], ef_b[off:off + n], cb[off // 2:(off + n) // 2],
                     sb[off // B:(off + n) // B]))
        off += n
    from weight_communication_zero_amd import EfqSegmentTable
    table = EfqSegmentTable(segs, B)
    for step in range(3):
        synth.fill_model(g, tensors, std=1e-3, seed=synth.seed_for("llama0p85b", "grad", step=step),
                         heavy_tails=True)
        Z().zq_quantize_ef_int4(g, ef_a, B, 0.9, 1.0, ca, sa)
        Z().zq_quantize_ef_int4_batched(table, B, 0.9, 1.0)
        torch.cuda.synchronize()
        assert torch.equal(ca, cb), f"step {step} codes"
        assert torch.equal(sa.view(torch.int32), sb.view(torch.int32)), f"step {step} scales"
        assert torch.equal(ef_a.view(torch.int32), ef_b.view(torch.int32)), f"step {step} ef"


# ------------------------------------- per-parameter receive side, 7.5B --

def test_per_tensor_batched_reduce_requant_7p5b_sampled():
    """The receive side parameter by parameter over the ~7.5B model's 327
    tensors: tensor i's receive buffer holds its 8 peer chunks of n_i / 8
    elements (contiguous, as an all-to-all delivers them), each reduced and
    requantized on its own with its own requant EF buffer, 2 steps, then a
    third step without requant EF -- one zq_dequant_reduce_batched call per
    step.  Whole outputs poisoned and
    checked written; the first and last output block of every tensor and
    random others recomputed by the oracle from the generator's inputs."""
    tensors = synth.llama_7p5b()
    M = synth.total(tensors)
    B, P = 128, 8
    n1 = M // P
    g = torch.empty(M, dtype=torch.float32, device="cuda")
    codes = torch.empty(M // 2, dtype=torch.uint8, device="cuda")
    scales = torch.empty(M // B, dtype=torch.float32, device="cuda")
    rqc = torch.empty(n1 // 2, dtype=torch.uint8, device="cuda")
    rqs = torch.empty(n1 // B, dtype=torch.float32, device="cuda")
    rq_ef = torch.zeros(n1, dtype=torch.float32, device="cuda")
    segs, where, off, roff = [], [], 0, 0
    for t in tensors:
        m = t.numel // P
        segs.append((codes[off // 2:(off + t.numel) // 2], scales[off // B:(off + t.numel) // B], m,
                     m // 2, m // B, None, rqc[roff // 2:(roff + m) // 2], rqs[roff // B:(roff + m) // B],
                     rq_ef[roff:roff + m]))
        where.append((off, roff, m))
        off += t.numel
        roff += m
    table = Z().DrSegmentTable(segs, P, B)
    table_noef = Z().DrSegmentTable([sg[:8] + (None,) for sg in segs], P, B)
    rng = np.random.default_rng(21)
    # tracked output blocks: (segment, block within the segment)
    picks = []
    for i, (_, _, m) in enumerate(where):
        picks += [(i, 0), (i, m // B - 1)]
    for i in rng.integers(0, len(where), size=200):
        picks.append((int(i), int(rng.integers(0, where[i][2] // B))))
    picks = sorted(set(picks))
    out_blocks = np.array([where[i][1] // B + b for i, b in picks])
    in_blocks = np.array([(where[i][0] + j * where[i][2]) // B + b for i, b in picks for j in range(P)])
    rq_ef_o = np.zeros(out_blocks.size * B, np.float32)
    for step in range(3):
        # steps 0 and 1 with the per-tensor requant EF buffers, step 2 without
        # (the benchmark's batched requant row)
        with_ef = step < 2
        synth.fill_model(g, tensors, std=1e-3, seed=synth.seed_for("llama7p5b", "grad", step=step),
                         heavy_tails=True)
        Z().zq_quantize_ef_int4(g, None, B, 0.0, 1.0, codes, scales)
        rqc.fill_(0x88)
        rqs.fill_(float("nan"))
        Z().zq_dequant_reduce_batched(table if with_ef else table_noef, P, B, 1.0,
                                      rq_beta_e=0.9, rq_beta_r=1.0)
        torch.cuda.synchronize()
        what = f"7.5B per-tensor reduce step {step} ({'with' if with_ef else 'no'} requant EF)"
        assert not bool(((rqc & 0x0F) == 8).any() | ((rqc >> 4) == 8).any()), what + ": codes unwritten"
        assert not bool(torch.isnan(rqs).any()), what + ": scales unwritten"
        # oracle: the 8 input blocks of every tracked output block, in order
        c0, s0 = O.quantize_ef_int4(gather_blocks(g, in_blocks, B), None, B, 0.0, 1.0)
        k = out_blocks.size
        cj = [np.concatenate([c0[(q * P + j) * B // 2:(q * P + j + 1) * B // 2] for q in range(k)])
              for j in range(P)]
        sj = [np.array([s0[q * P + j] for q in range(k)], np.float32) for j in range(P)]
        _, rc_o, rs_o = O.dequant_reduce(cj, sj, k * B, B, 1.0, want_out=False, requant=True,
                                         rq_ef=rq_ef_o if with_ef else None, rq_beta_e=0.9,
                                         rq_beta_r=1.0)
        assert_bits_equal(int4_block_bytes(rqc, out_blocks, B), rc_o, what + " requant codes")
        assert_bits_equal(to_host(rqs)[out_blocks], rs_o, what + " requant scales")
        assert_bits_equal(gather_blocks(rq_ef, out_blocks, B), rq_ef_o, what + " requant ef")


# ------------------- the 7.5B send side in ZeRO++ order and per parameter --

def test_send_side_forms_7p5b_equal_the_flat_call():
    """The benchmark's other two EF-quantize forms at their full 7.5B size,
    each against the flat call from the same EF state: the ZeRO++ order for
    4 nodes of 8 GPUs ("ZeROPlusPlus.md" notes, section 1.2) must hold
    partition p's codes and scales in slot sigma(p) and leave the EF buffer
    exactly as the flat call does; the per-parameter call over the 327
    tensors ("Merge LoCo with Zero++", review thread) must equal the flat
    call everywhere.  The first and last block of every partition are also
    checked against the oracle from host copies of g and the EF state."""
    tensors = synth.llama_7p5b()
    M = synth.total(tensors)
    B, intra, inter = 128, 8, 4
    n_part = intra * inter
    part = M // n_part
    g = torch.empty(M, dtype=torch.float32, device="cuda")
    synth.fill_model(g, tensors, std=1e-3, seed=synth.seed_for("llama7p5b", "grad", step=0),
                     heavy_tails=True)
    ef_flat = torch.empty(M, dtype=torch.float32, device="cuda")
    ef_w = torch.empty(M, dtype=torch.float32, device="cuda")
    ef_seed = synth.seed_for("llama7p5b", "ef")
    synth.fill_model(ef_flat, None, std=1e-5, seed=ef_seed)
    blocks = np.array(sorted({p * part // B for p in range(n_part)} |
                             {(p + 1) * part // B - 1 for p in range(n_part)}))
    g_h = gather_blocks(g, blocks, B)
    e_h = gather_blocks(ef_flat, blocks, B)
    c_flat = torch.empty(M // 2, dtype=torch.uint8, device="cuda")
    s_flat = torch.empty(M // B, dtype=torch.float32, device="cuda")
    Z().zq_quantize_ef_int4(g, ef_flat, B, 0.9, 1.0, c_flat, s_flat)

    c_w = torch.full((M // 2,), 0x88, dtype=torch.uint8, device="cuda")
    s_w = torch.full((M // B,), float("nan"), device="cuda")
    synth.fill_model(ef_w, None, std=1e-5, seed=ef_seed)
    slots = Z().zeropp_slots(intra, inter)
    Z().zq_quantize_ef_int4_permuted(g, ef_w, B, 0.9, 1.0, c_w, s_w, slots)
    torch.cuda.synchronize()
    assert torch.equal(ef_w.view(torch.int32), ef_flat.view(torch.int32)), "permuted: EF differs"
    for p in range(n_part):
        q = slots[p]
        assert torch.equal(c_w[q * part // 2:(q + 1) * part // 2],
                           c_flat[p * part // 2:(p + 1) * part // 2]), f"partition {p} codes"
        assert torch.equal(s_w[q * part // B:(q + 1) * part // B].view(torch.int32),
                           s_flat[p * part // B:(p + 1) * part // B].view(torch.int32)), \
            f"partition {p} scales"
    c_o, s_o = O.quantize_ef_int4(g_h, e_h, B, 0.9, 1.0)
    for i, b in enumerate(blocks):
        p, r = divmod(int(b), part // B)
        slot_block = slots[p] * (part // B) + r
        assert_bits_equal(to_host(c_w[slot_block * B // 2:(slot_block + 1) * B // 2]),
                          c_o[i * B // 2:(i + 1) * B // 2], f"permuted block {b} codes")
        assert_bits_equal(to_host(s_w[slot_block:slot_block + 1]), s_o[i:i + 1],
                          f"permuted block {b} scale")
        assert_bits_equal(to_host(ef_w[b * B:(b + 1) * B]), e_h[i * B:(i + 1) * B],
                          f"block {b} EF")

    c_w.fill_(0x88)
    s_w.fill_(float("nan"))
    synth.fill_model(ef_w, None, std=1e-5, seed=ef_seed)
    segs, off = [], 0
    for t in tensors:
        n = t.numel
        segs.append((g[off:off + n], ef_w[off:off + n], c_w[off // 2:(off + n) // 2],
                     s_w[off // B:(off + n) // B]))
        off += n
    Z().zq_quantize_ef_int4_batched(segs, B, 0.9, 1.0)
    torch.cuda.synchronize()
    assert torch.equal(c_w, c_flat), "per-parameter codes differ from the flat call"
    assert torch.equal(s_w.view(torch.int32), s_flat.view(torch.int32)), "per-parameter scales"
    assert torch.equal(ef_w.view(torch.int32), ef_flat.view(torch.int32)), "per-parameter EF"


def test_efq_bf16_gradients_7p5b_sampled():
    """The EF quantizer on the 7.5B gradient in bf16 (half-precision
    gradients, as the LoCo kernel loads them, "Merge LoCo with Zero++",
    review thread) with an fp32 EF buffer, the benchmark's bf16 row: every
    code and scale written, the first and last block and 254 random ones
    (codes, scales, updated EF) against the oracle."""
    tensors = synth.llama_7p5b()
    M = synth.total(tensors)
    B = 128
    g = torch.empty(M, dtype=torch.bfloat16, device="cuda")
    synth.fill_model(g, tensors, std=1e-3, seed=synth.seed_for("llama7p5b", "grad", step=1),
                     heavy_tails=True)
    ef = torch.empty(M, dtype=torch.float32, device="cuda")
    synth.fill_model(ef, None, std=1e-5, seed=synth.seed_for("llama7p5b", "ef"))
    nb = M // B
    rng = np.random.default_rng(31)
    blocks = np.unique(np.concatenate([[0, nb - 1], rng.integers(0, nb, size=254)]))
    g_h = gather_blocks(g, blocks, B)
    e_h = gather_blocks(ef, blocks, B)
    codes = torch.full((M // 2,), 0x88, dtype=torch.uint8, device="cuda")
    scales = torch.full((nb,), float("nan"), device="cuda")
    Z().zq_quantize_ef_int4(g, ef, B, 0.9, 1.0, codes, scales)
    torch.cuda.synchronize()
    assert not bool(((codes & 0x0F) == 8).any() | ((codes >> 4) == 8).any()), "codes unwritten"
    assert not bool(torch.isnan(scales).any()), "scales unwritten"
    c_o, s_o = O.quantize_ef_int4(g_h, e_h, B, 0.9, 1.0)
    assert_bits_equal(int4_block_bytes(codes, blocks, B), c_o, "bf16 7.5B codes")
    assert_bits_equal(to_host(scales)[blocks], s_o, "bf16 7.5B scales")
    assert_bits_equal(gather_blocks(ef, blocks, B), e_h, "bf16 7.5B EF")
