"""CPU oracle for the ZeRO++ / LoCo block quantization and llm.c stochastic
rounding path -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does, and the
two share no code: this wrapper marshals numpy arrays into the plain C oracle
in ``zq_oracle.c`` (one element at a time, fp32 arithmetic exactly as the
definitions state).  Each function below names the passage it follows; the C
source holds the full statement.

Host arrays only: fp32 data as ``np.float32``, bf16 data as ``np.uint16`` bit
patterns, fp16 data as ``np.float16``, int4 codes as ``np.uint8`` (two per
byte, low nibble first), int8 codes as ``np.int8``.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import build as _build

_lib = None
# Output buffers start poisoned so that every byte the oracle returns was
# written by it (an element it forgot shows up as 0xAA / NaN).
_POISON_U8 = 0xAA


def lib():
    global _lib
    if _lib is None:
        path = _build.ensure_built()
        L = C.CDLL(path)
        vp, sz, u32, f32, i32, u64 = C.c_void_p, C.c_size_t, C.c_uint32, C.c_float, C.c_int, C.c_uint64
        L.orc_quant_block.argtypes = [vp, sz, i32, vp, vp]
        L.orc_quant_block.restype = None
        L.orc_int4_decode.argtypes = [vp, sz]
        L.orc_int4_decode.restype = C.c_int32
        L.orc_quantize_ef_int4.argtypes = [vp, i32, vp, sz, u32, f32, f32, vp, vp]
        L.orc_quantize_ef_int4.restype = i32
        L.orc_quantize_ef_int4_permuted.argtypes = [vp, i32, vp, sz, u32, f32, f32, u32, vp, vp, vp]
        L.orc_quantize_ef_int4_permuted.restype = i32
        L.orc_zeropp_slots.argtypes = [u32, u32, vp]
        L.orc_zeropp_slots.restype = i32
        L.orc_dequant_reduce.argtypes = [u32, vp, vp, sz, u32, f32, vp, vp, vp, vp, f32, f32, vp]
        L.orc_dequant_reduce.restype = i32
        L.orc_dequant_reduce_segments.argtypes = [u32, vp, vp, vp, vp, vp, vp, vp, vp, vp, u32, u32,
                                                  f32, f32, f32, vp]
        L.orc_dequant_reduce_segments.restype = i32
        L.orc_quant_int8.argtypes = [vp, i32, sz, u32, vp, vp]
        L.orc_quant_int8.restype = i32
        L.orc_dequant_int8.argtypes = [vp, vp, sz, u32, vp, i32]
        L.orc_dequant_int8.restype = i32
        L.orc_bf16_rne.argtypes = [f32]
        L.orc_bf16_rne.restype = C.c_uint16
        L.orc_f16_rne.argtypes = [f32]
        L.orc_f16_rne.restype = C.c_uint16
        L.orc_f16_to_f32.argtypes = [C.c_uint16]
        L.orc_f16_to_f32.restype = f32
        L.orc_philox4x32_10.argtypes = [vp, vp, vp]
        L.orc_philox4x32_10.restype = None
        L.orc_sr_r16.argtypes = [u64, u64]
        L.orc_sr_r16.restype = u32
        L.orc_sr_round.argtypes = [f32, u32]
        L.orc_sr_round.restype = C.c_uint16
        L.orc_sr_accumulate.argtypes = [vp, vp, sz, u64, u64, i32]
        L.orc_sr_accumulate.restype = i32
        L.orc_sr_accumulate_segments.argtypes = [u32, vp, vp, vp, vp, vp, vp, vp, i32]
        L.orc_sr_accumulate_segments.restype = i32
        L.orc_sr_r16_fill.argtypes = [u64, u64, sz, vp]
        L.orc_sr_r16_fill.restype = None
        L.orc_volume_bytes.argtypes = [u64, u32, u32, vp]
        L.orc_volume_bytes.restype = None
        _lib = L
    return _lib


class OracleArgumentError(ValueError):
    """The C oracle rejected its arguments (and wrote nothing)."""


def _ok(rc: int, fn: str) -> None:
    if rc != 0:
        raise OracleArgumentError(f"{fn}: arguments rejected by the oracle ({rc})")


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be contiguous"
    return a.ctypes.data


# Element-type codes of the C oracle's data streams.
F32, BF16, F16 = 0, 1, 2


def _dtype_code(a: np.ndarray, what: str) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float16:
        return F16
    raise TypeError(f"{what} must be float32, uint16 (bf16 bits) or float16")


def _check_block(block: int):
    if block < 2 or block % 2 or block > 4096:
        raise ValueError("oracle block must be even and in [2, 4096]")


def int4_code_bytes(n: int) -> int:
    return (n + 1) // 2


def num_blocks(n: int, block: int) -> int:
    return (n + block - 1) // block


def quant_block(x: np.ndarray, qmax: int):
    """Symmetric absmax quantizer of one block ([ZeRO++] notes, section 1.2:
    block-based quantization).  Returns (codes int32[m], scale float32)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    k = np.empty(x.size, dtype=np.int32)
    s = np.zeros(1, dtype=np.float32)
    lib().orc_quant_block(_ptr(x), x.size, qmax, _ptr(k), _ptr(s))
    return k, s[0]


def int4_decode(codes: np.ndarray, n: int) -> np.ndarray:
    """Signed int4 values of the first n elements of a packed code array."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    L = lib()
    return np.array([L.orc_int4_decode(_ptr(codes), i) for i in range(n)], dtype=np.int32)


def quantize_ef_int4(g: np.ndarray, ef: np.ndarray | None, block: int, beta_e: float,
                     beta_r: float):
    """LoCo error-feedback int4 quantize ("Merge LoCo with Zero++", Overview
    and review thread).  g: float32, uint16 (bf16 bits) or float16.  ef
    (float32) is updated in place when given.  Returns (codes
    uint8[ceil(n/2)], scales float32[ceil(n/block)])."""
    _check_block(block)
    g = np.ascontiguousarray(g)
    code = _dtype_code(g, "g")
    n = g.size
    if ef is not None:
        assert ef.dtype == np.float32 and ef.size == n and ef.flags["C_CONTIGUOUS"]
    codes = np.full(int4_code_bytes(n), _POISON_U8, dtype=np.uint8)
    scales = np.full(num_blocks(n, block), np.nan, dtype=np.float32)
    _ok(lib().orc_quantize_ef_int4(_ptr(g), code, _ptr(ef), n, block, beta_e, beta_r,
                                   _ptr(codes), _ptr(scales)), "quantize_ef_int4")
    return codes, scales


def dequant_reduce(codes_list, scales_list, n_chunk: int, block: int, alpha: float,
                   want_out: bool = True, requant: bool = False, rq_ef: np.ndarray | None = None,
                   rq_beta_e: float = 0.0, rq_beta_r: float = 1.0):
    """qgZ receive side ([ZeRO++] notes, section 1.2): dequantize P int4
    chunks and reduce in full precision, optionally requantize for the next
    hierarchy level.  Returns (out or None, rq_codes or None, rq_scales or
    None); rq_ef is updated in place when given."""
    _check_block(block)
    P = len(codes_list)
    assert P == len(scales_list) and P >= 1
    cl = [np.ascontiguousarray(c, dtype=np.uint8) for c in codes_list]
    sl = [np.ascontiguousarray(s, dtype=np.float32) for s in scales_list]
    cptr = (C.c_void_p * P)(*[c.ctypes.data for c in cl])
    sptr = (C.c_void_p * P)(*[s.ctypes.data for s in sl])
    out = np.full(n_chunk, np.nan, dtype=np.float32) if want_out else None
    rq_codes = np.full(int4_code_bytes(n_chunk), _POISON_U8, dtype=np.uint8) if requant else None
    rq_scales = np.full(num_blocks(n_chunk, block), np.nan, dtype=np.float32) if requant else None
    work = np.empty(max(n_chunk, 1), dtype=np.float32)
    if rq_ef is not None:
        assert requant and rq_ef.dtype == np.float32 and rq_ef.size == n_chunk
    _ok(lib().orc_dequant_reduce(P, cptr, sptr, n_chunk, block, alpha, _ptr(out), _ptr(rq_codes),
                                 _ptr(rq_scales), _ptr(rq_ef), rq_beta_e, rq_beta_r, _ptr(work)),
        "dequant_reduce")
    return out, rq_codes, rq_scales


def dequant_reduce_segments(segments, P: int, block: int, alpha: float, want_out: bool = True,
                            requant: bool = False, rq_efs=None, rq_beta_e: float = 0.0,
                            rq_beta_r: float = 1.0):
    """The receive side parameter by parameter ("Merge LoCo with Zero++",
    review thread), done by the C oracle.  `segments`: (codes, scales, n,
    codes_stride, scales_stride) with codes a uint8 array holding the P
    chunks (peer p at byte p * codes_stride) and scales a float32 array
    (peer p at element p * scales_stride).  rq_efs: one float32[n] per
    segment (updated in place) or None.  Returns per segment (out or None,
    rq_codes or None, rq_scales or None)."""
    _check_block(block)
    segs = list(segments)
    m = len(segs)
    cl = [np.ascontiguousarray(c, dtype=np.uint8) for c, _, _, _, _ in segs]
    sl = [np.ascontiguousarray(s_, dtype=np.float32) for _, s_, _, _, _ in segs]
    ns = [int(x[2]) for x in segs]
    for c, s_, (_, _, n, cs, ss) in zip(cl, sl, segs):
        if n:
            assert c.size >= (P - 1) * cs + (n + 1) // 2 and s_.size >= (P - 1) * ss + num_blocks(n, block)
    outs = [np.full(n, np.nan, np.float32) for n in ns] if want_out else None
    rqc = [np.full(int4_code_bytes(n), _POISON_U8, np.uint8) for n in ns] if requant else None
    rqs = [np.full(num_blocks(n, block), np.nan, np.float32) for n in ns] if requant else None
    if rq_efs is not None:
        assert requant and all(e.dtype == np.float32 and e.size == n for e, n in zip(rq_efs, ns))
    arr = lambda lst: None if lst is None else (C.c_void_p * max(m, 1))(*[a.ctypes.data for a in lst])
    u64 = lambda vals: np.array(list(vals) or [0], dtype=np.uint64)
    work = np.empty(max(ns + [1]), np.float32)
    # every array handed to C stays referenced until the call returns
    cstride, sstride, n_arr = u64(x[3] for x in segs), u64(x[4] for x in segs), u64(ns)
    tables = [arr(cl), arr(sl), arr(outs), arr(rqc), arr(rqs), arr(rq_efs)]
    _ok(lib().orc_dequant_reduce_segments(
        m, tables[0], tables[1], _ptr(cstride), _ptr(sstride), _ptr(n_arr), tables[2], tables[3],
        tables[4], tables[5], P, block, alpha, rq_beta_e, rq_beta_r, _ptr(work)),
        "dequant_reduce_segments")
    return [((outs[i] if want_out else None), (rqc[i] if requant else None),
             (rqs[i] if requant else None)) for i in range(m)]


def quant_int8(w: np.ndarray, block: int):
    """qwZ int8 block quantization ([ZeRO++] notes, section 1.2).  w float32,
    uint16 (bf16 bits) or float16.  Returns (codes int8[n], scales
    float32[nb])."""
    _check_block(block)
    w = np.ascontiguousarray(w)
    code = _dtype_code(w, "w")
    codes = np.full(w.size, -86, dtype=np.int8)
    scales = np.full(num_blocks(w.size, block), np.nan, dtype=np.float32)
    _ok(lib().orc_quant_int8(_ptr(w), code, w.size, block, _ptr(codes), _ptr(scales)),
        "quant_int8")
    return codes, scales


def dequant_int8(codes: np.ndarray, scales: np.ndarray, block: int, out_bf16: bool = False,
                 out_f16: bool = False):
    """qwZ dequantize after the all-gather.  Returns float32[n], uint16[n]
    (bf16 bits) or float16[n], the 16-bit forms rounded to nearest even."""
    assert not (out_bf16 and out_f16)
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    dt, code = ((np.uint16, BF16) if out_bf16 else (np.float16, F16) if out_f16
                else (np.float32, F32))
    out = np.zeros(codes.size, dtype=dt)
    _ok(lib().orc_dequant_int8(_ptr(codes), _ptr(scales), codes.size, block, _ptr(out), code),
        "dequant_int8")
    return out


def bf16_rne(x: float) -> int:
    return int(lib().orc_bf16_rne(float(x)))


def f16_rne(x: float) -> int:
    """fp32 -> IEEE binary16 bits, round to nearest even."""
    return int(lib().orc_f16_rne(float(x)))


def f16_to_f32(h: int) -> float:
    """IEEE binary16 bits -> fp32 (exact)."""
    return float(lib().orc_f16_to_f32(int(h)))


def philox4x32_10(ctr, key):
    """Philox-4x32-10 (Salmon et al., SC'11).  ctr: 4 words, key: 2 words."""
    c = np.array(ctr, dtype=np.uint32)
    k = np.array(key, dtype=np.uint32)
    o = np.zeros(4, dtype=np.uint32)
    lib().orc_philox4x32_10(_ptr(c), _ptr(k), _ptr(o))
    return [int(v) for v in o]


def sr_r16(seed: int, q: int) -> int:
    return int(lib().orc_sr_r16(seed, q))


def sr_r16_fill(seed: int, q0: int, n: int) -> np.ndarray:
    out = np.zeros(n, dtype=np.uint16)
    lib().orc_sr_r16_fill(seed, q0, n, _ptr(out))
    return out


def sr_round(x: float, r16: int) -> int:
    """Stochastic rounding of one fp32 value to bf16 with a given 16-bit
    random number ("Zero 2 #593", review of vector_add)."""
    return int(lib().orc_sr_round(float(x), r16))


def sr_accumulate(dst: np.ndarray, src: np.ndarray, seed: int, counter_base: int,
                  zero_src: bool = False):
    """bf16 dst += src with stochastic rounding (in place on dst; src cleared
    when zero_src).  Both uint16 bf16 bit arrays of equal size."""
    assert dst.dtype == np.uint16 and src.dtype == np.uint16 and dst.size == src.size
    assert dst.flags["C_CONTIGUOUS"] and src.flags["C_CONTIGUOUS"]
    _ok(lib().orc_sr_accumulate(_ptr(dst), _ptr(src), dst.size, seed, counter_base,
                                1 if zero_src else 0), "sr_accumulate")


def volume_bytes(M: int, block_w: int, block_g: int):
    """Per-step bytes (ZeRO-3, ZeRO++) for M parameters ([ZeRO++] notes,
    abstract and section 1.2)."""
    o = np.zeros(2, dtype=np.uint64)
    lib().orc_volume_bytes(M, block_w, block_g, _ptr(o))
    return int(o[0]), int(o[1])


def sr_accumulate_segments(segments, zero_src: bool):
    """llm.c's per-tensor ZeRO-2 loop ("Zero 2 #593", review of
    llmc/zero.cuh), done by the C oracle: for each segment (dst, src, n,
    src_offset, seed, counter_base), dst[0:n] += src[src_offset:src_offset+n]
    with stochastic rounding, then -- with zero_src -- the whole src buffer
    is cleared (the memset the review suggests folding into the add).  In
    place on the given contiguous uint16 (bf16 bit) arrays."""
    segs = list(segments)
    m = len(segs)
    for dst, src, n, off, _, _ in segs:
        assert dst.dtype == np.uint16 and src.dtype == np.uint16
        assert dst.flags["C_CONTIGUOUS"] and src.flags["C_CONTIGUOUS"] and dst.size >= n
    ptrs = lambda arrs: (C.c_void_p * max(m, 1))(*[a.ctypes.data for a in arrs])
    u64s = lambda vals: np.array(list(vals) or [0], dtype=np.uint64)
    # every array handed to C stays referenced until the call returns
    n = u64s(s[2] for s in segs)
    off = u64s(s[3] for s in segs)
    ln = u64s(s[1].size for s in segs)
    seed = u64s(s[4] for s in segs)
    cb = u64s(s[5] for s in segs)
    dsts, srcs = ptrs([s[0] for s in segs]), ptrs([s[1] for s in segs])
    _ok(lib().orc_sr_accumulate_segments(m, dsts, srcs, _ptr(n), _ptr(off), _ptr(ln), _ptr(seed),
                                         _ptr(cb), 1 if zero_src else 0), "sr_accumulate_segments")


def zeropp_slots(intra: int, inter: int) -> list[int]:
    """ZeRO++'s partition order for `inter` nodes of `intra` GPUs
    ("ZeROPlusPlus.md" notes, section 1.2: reduce inside the node, then
    across nodes): slot_of_part[r] for rank r = node * intra + local."""
    out = np.zeros(max(intra * inter, 1), dtype=np.uint32)
    _ok(lib().orc_zeropp_slots(intra, inter, _ptr(out)), "zeropp_slots")
    return [int(v) for v in out[:intra * inter]]


def quantize_ef_int4_permuted(g, ef, block: int, beta_e: float, beta_r: float, slot_of_part):
    """The EF int4 quantizer with its outputs in permuted partition order
    ("ZeROPlusPlus.md" notes, section 1.2: hierarchical gradient reduction,
    inside the node first, then across nodes), done by the C oracle: the
    codes and scales of partition p are stored where partition
    slot_of_part[p] would be.  Partitions are equal and whole blocks long."""
    _check_block(block)
    g = np.ascontiguousarray(g)
    code = _dtype_code(g, "g")
    n = g.size
    if ef is not None:
        assert ef.dtype == np.float32 and ef.size == n and ef.flags["C_CONTIGUOUS"]
    slots = np.ascontiguousarray(slot_of_part, dtype=np.uint32)
    codes = np.full(int4_code_bytes(n), _POISON_U8, dtype=np.uint8)
    scales = np.full(num_blocks(n, block), np.nan, dtype=np.float32)
    _ok(lib().orc_quantize_ef_int4_permuted(_ptr(g), code, _ptr(ef), n, block, beta_e, beta_r,
                                            slots.size, _ptr(slots), _ptr(codes), _ptr(scales)),
        "quantize_ef_int4_permuted")
    return codes, scales
