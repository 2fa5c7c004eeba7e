"""ctypes binding of libzq (include/zq.h): argument marshalling only.

Every function takes torch tensors (device memory) or raw integer device
pointers, converts them to the C ABI's plain pointers and sizes, passes the
current torch HIP stream unless one is given, and raises ``ZQError`` on a
non-OK status.  All arithmetic happens in libzq's HIP kernels; there is no
fallback path: if ``libzq.so`` is missing or cannot be loaded, importing this
module fails.
"""
from __future__ import annotations

import ctypes as C
import os
import re

import torch  # loaded first: libzq then binds to the HIP runtime torch uses

_HERE = os.path.dirname(os.path.abspath(__file__))
# ZQ_LIB selects another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("ZQ_LIB") or os.path.join(_HERE, "libzq.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "zq.h")

ZQ_FP32, ZQ_BF16, ZQ_FP16 = 0, 1, 2

STATUS = {
    0: "ZQ_OK", 1: "ZQ_ERR_NULL", 2: "ZQ_ERR_SIZE", 3: "ZQ_ERR_BLOCK", 4: "ZQ_ERR_ALIGN",
    5: "ZQ_ERR_ALIAS", 6: "ZQ_ERR_PEERS", 7: "ZQ_ERR_DTYPE", 8: "ZQ_ERR_LAUNCH",
}
ZQ_OK, ZQ_ERR_NULL, ZQ_ERR_SIZE, ZQ_ERR_BLOCK, ZQ_ERR_ALIGN = 0, 1, 2, 3, 4
ZQ_ERR_ALIAS, ZQ_ERR_PEERS, ZQ_ERR_DTYPE, ZQ_ERR_LAUNCH = 5, 6, 7, 8


class SrSegment(C.Structure):
    """zq_sr_segment of include/zq.h."""
    _fields_ = [("dst", C.c_void_p), ("src", C.c_void_p), ("n", C.c_uint64),
                ("src_offset", C.c_uint64), ("src_len", C.c_uint64), ("seed", C.c_uint64),
                ("counter_base", C.c_uint64)]


class EfqSegment(C.Structure):
    """zq_efq_segment of include/zq.h."""
    _fields_ = [("g", C.c_void_p), ("ef", C.c_void_p), ("codes", C.c_void_p),
                ("scales", C.c_void_p), ("n", C.c_uint64)]


class DrSegment(C.Structure):
    """zq_dr_segment of include/zq.h."""
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("codes_stride", C.c_uint64),
                ("scales_stride", C.c_uint64), ("n", C.c_uint64), ("out", C.c_void_p),
                ("rq_codes", C.c_void_p), ("rq_scales", C.c_void_p), ("rq_ef", C.c_void_p)]


class ZQError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {lib.zq_status_str(status).decode()}")
        self.status = status


def _load() -> C.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; build it with `python -c 'import __graft_entry__ as g; g.build()'`"
            " (hipcc, gfx950)")
    L = C.CDLL(LIB_PATH)
    vp, sz, u32, u64, f32, i32 = C.c_void_p, C.c_size_t, C.c_uint32, C.c_uint64, C.c_float, C.c_int
    L.zq_quantize_ef_int4.argtypes = [vp, i32, vp, sz, u32, f32, f32, vp, vp, vp]
    L.zq_dequant_reduce.argtypes = [u32, vp, vp, sz, u32, f32, vp, vp, vp, vp, f32, f32, vp]
    L.zq_quant_int8.argtypes = [vp, i32, sz, u32, vp, vp, vp]
    L.zq_dequant_int8.argtypes = [vp, vp, sz, u32, vp, i32, vp]
    L.zq_sr_accumulate.argtypes = [vp, vp, sz, u64, u64, i32, vp]
    for f in ("zq_quantize_ef_int4", "zq_dequant_reduce", "zq_quant_int8", "zq_dequant_int8",
              "zq_sr_accumulate"):
        getattr(L, f).restype = i32
    L.zq_quantize_ef_int4_permuted.argtypes = [vp, i32, vp, sz, u32, f32, f32, vp, vp, u32, vp,
                                               vp]
    L.zq_quantize_ef_int4_permuted.restype = i32
    L.zq_quantize_ef_int4_batched.argtypes = [vp, u32, i32, u32, f32, f32, vp]
    L.zq_quantize_ef_int4_batched.restype = i32
    L.zq_dequant_reduce_batched.argtypes = [vp, u32, u32, u32, f32, f32, f32, vp]
    L.zq_dequant_reduce_batched.restype = i32
    L.zq_sr_accumulate_batched.argtypes = [vp, u32, i32, vp]
    L.zq_sr_accumulate_batched.restype = i32
    L.zq_zeropp_slots.argtypes = [u32, u32, vp]
    L.zq_zeropp_slots.restype = u32
    L.zq_int4_code_bytes.argtypes = [sz]
    L.zq_int4_code_bytes.restype = sz
    L.zq_num_blocks.argtypes = [sz, u32]
    L.zq_num_blocks.restype = sz
    L.zq_status_str.argtypes = [i32]
    L.zq_status_str.restype = C.c_char_p
    L.zq_abi_version.argtypes = []
    L.zq_abi_version.restype = u32
    return L


lib = _load()


def declared_symbols() -> list[str]:
    """Function names declared in include/zq.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:zq_status|size_t|const char \*|uint32_t)\s*\*?\s*(zq_\w+)\s*\(",
                                 text, re.M)))


def _p(x) -> int | None:
    """Device pointer of a tensor (or an int already a pointer; None -> NULL)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_contiguous():
        raise ValueError("libzq needs contiguous tensors")
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dtype(t) -> int:
    if t.dtype == torch.float32:
        return ZQ_FP32
    if t.dtype == torch.bfloat16:
        return ZQ_BF16
    if t.dtype == torch.float16:
        return ZQ_FP16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _need(name: str, t, numel: int, dtypes) -> None:
    """Host-side guard before any launch: a tensor argument must be a
    contiguous GPU tensor of an accepted dtype holding at least `numel`
    elements, so no kernel can index past a caller's buffer."""
    if t is None or isinstance(t, int):
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name} is on {t.device}, the current device is "
                         f"cuda:{torch.cuda.current_device()}")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")


_F32 = (torch.float32,)
_BF16 = (torch.bfloat16,)
_FLOAT = (torch.float32, torch.bfloat16, torch.float16)
_U8 = (torch.uint8,)
_I8 = (torch.int8,)


def _check(fn: str, st: int) -> None:
    if st != ZQ_OK:
        raise ZQError(fn, st)


def int4_code_bytes(n: int) -> int:
    return lib.zq_int4_code_bytes(n)


def num_blocks(n: int, block: int) -> int:
    return lib.zq_num_blocks(n, block)


def zq_quantize_ef_int4(g, ef, block: int, beta_e: float, beta_r: float, codes, scales,
                        stream=None, n: int | None = None) -> None:
    """EF int4 quantize: g (fp32/bf16/fp16), ef (fp32 or None, updated in place)
    -> codes (uint8, ceil(n/2)), scales (fp32, ceil(n/block))."""
    n = g.numel() if n is None else n
    nb = (n + block - 1) // block if block > 0 else 0
    _need("g", g, n, _FLOAT)
    _need("ef", ef, n, _F32)
    _need("codes", codes, (n + 1) // 2, _U8)
    _need("scales", scales, nb, _F32)
    _check("zq_quantize_ef_int4",
           lib.zq_quantize_ef_int4(_p(g), _dtype(g), _p(ef), n, block, beta_e, beta_r, _p(codes),
                                   _p(scales), _stream(stream)))


def zeropp_slots(intra: int, inter: int) -> list[int]:
    """ZeRO++'s partition order for `inter` nodes of `intra` GPUs, from
    libzq's zq_zeropp_slots (slot_of_part[r] for rank r)."""
    m = intra * inter
    out = (C.c_uint32 * max(m, 1))()
    got = lib.zq_zeropp_slots(intra, inter, out)
    if got != m or m == 0:
        raise ValueError(f"zq_zeropp_slots rejected intra={intra}, inter={inter}")
    return list(out[:m])


def zq_quantize_ef_int4_permuted(g, ef, block: int, beta_e: float, beta_r: float, codes, scales,
                                 slot_of_part, stream=None, n: int | None = None) -> None:
    """EF int4 quantize whose codes / scales of partition p land in slot
    slot_of_part[p] (g and ef stay in natural order)."""
    n = g.numel() if n is None else n
    nb = (n + block - 1) // block if block > 0 else 0
    _need("g", g, n, _FLOAT)
    _need("ef", ef, n, _F32)
    _need("codes", codes, (n + 1) // 2, _U8)
    _need("scales", scales, nb, _F32)
    slots = (C.c_uint32 * max(len(slot_of_part), 1))(*slot_of_part)
    _check("zq_quantize_ef_int4_permuted",
           lib.zq_quantize_ef_int4_permuted(_p(g), _dtype(g), _p(ef), n, block, beta_e, beta_r,
                                            _p(codes), _p(scales), len(slot_of_part),
                                            C.cast(slots, C.c_void_p), _stream(stream)))


def zq_dequant_reduce(codes_list, scales_list, n_chunk: int, block: int, alpha: float, out=None,
                      rq_codes=None, rq_scales=None, rq_ef=None, rq_beta_e: float = 0.0,
                      rq_beta_r: float = 1.0, stream=None) -> None:
    """Dequantize P int4 chunks, reduce in fp32 (times alpha) into out, and /
    or requantize into rq_codes / rq_scales (with optional rq_ef)."""
    P = len(codes_list)
    if P != len(scales_list):
        raise ValueError("codes_list and scales_list differ in length")
    nb = (n_chunk + block - 1) // block if block > 0 else 0
    for c, sc in zip(codes_list, scales_list):
        _need("codes[p]", c, (n_chunk + 1) // 2, _U8)
        _need("scales[p]", sc, nb, _F32)
    _need("out", out, n_chunk, _F32)
    _need("rq_codes", rq_codes, (n_chunk + 1) // 2, _U8)
    _need("rq_scales", rq_scales, nb, _F32)
    _need("rq_ef", rq_ef, n_chunk, _F32)
    cp = (C.c_void_p * max(P, 1))(*[_p(c) for c in codes_list])
    sp = (C.c_void_p * max(P, 1))(*[_p(s) for s in scales_list])
    _check("zq_dequant_reduce",
           lib.zq_dequant_reduce(P, cp, sp, n_chunk, block, alpha, _p(out), _p(rq_codes),
                                 _p(rq_scales), _p(rq_ef), rq_beta_e, rq_beta_r, _stream(stream)))


def zq_quant_int8(w, block: int, codes, scales, stream=None, n: int | None = None) -> None:
    n = w.numel() if n is None else n
    _need("w", w, n, _FLOAT)
    _need("codes", codes, n, _I8)
    _need("scales", scales, (n + block - 1) // block if block > 0 else 0, _F32)
    _check("zq_quant_int8",
           lib.zq_quant_int8(_p(w), _dtype(w), n, block, _p(codes), _p(scales), _stream(stream)))


def zq_dequant_int8(codes, scales, block: int, out, stream=None, n: int | None = None) -> None:
    n = codes.numel() if n is None else n
    _need("codes", codes, n, _I8)
    _need("scales", scales, (n + block - 1) // block if block > 0 else 0, _F32)
    _need("out", out, n, _FLOAT)
    _check("zq_dequant_int8",
           lib.zq_dequant_int8(_p(codes), _p(scales), n, block, _p(out), _dtype(out),
                               _stream(stream)))


def zq_sr_accumulate(dst, src, seed: int, counter_base: int = 0, zero_src: bool = False,
                     stream=None, n: int | None = None) -> None:
    """bf16 dst += src with stochastic rounding (dst, src: torch.bfloat16)."""
    n = dst.numel() if n is None else n
    _need("dst", dst, n, _BF16)
    _need("src", src, n, _BF16)
    _check("zq_sr_accumulate",
           lib.zq_sr_accumulate(_p(dst), _p(src), n, seed, counter_base, 1 if zero_src else 0,
                                _stream(stream)))


class SrSegmentTable:
    """A marshalled segment table for zq_sr_accumulate_batched: build it once
    for a fixed set of buffers and pass it to every call (the tensors are
    kept alive by the table)."""

    def __init__(self, segments):
        self.segments = list(segments)
        self.arr = (SrSegment * max(len(self.segments), 1))()
        for i, (dst, src, n, off, seed, cb) in enumerate(self.segments):
            _need("dst", dst, n, _BF16)
            _need("src", src, off + n, _BF16)
            src_len = src.numel() if not isinstance(src, int) else off + n
            self.arr[i] = SrSegment(_p(dst), _p(src), n, off, src_len, seed, cb)
        self.ptr = C.cast(self.arr, C.c_void_p)


def zq_sr_accumulate_batched(segments, zero_src: bool = False, stream=None) -> None:
    """Batched SR accumulation.  `segments`: an SrSegmentTable, or an iterable
    of (dst, src, n, src_offset, seed, counter_base) with dst / src bf16
    tensors; src is the whole per-tensor buffer (src_len = src.numel()), of
    which elements [src_offset, src_offset + n) are added into dst[0:n]; with
    zero_src every element of every src buffer is cleared in the same pass."""
    table = segments if isinstance(segments, SrSegmentTable) else SrSegmentTable(segments)
    _check("zq_sr_accumulate_batched",
           lib.zq_sr_accumulate_batched(table.ptr, len(table.segments), 1 if zero_src else 0,
                                        _stream(stream)))


class EfqSegmentTable:
    """A marshalled segment table for zq_quantize_ef_int4_batched: tuples
    (g, ef or None, codes, scales) of per-tensor buffers (n = g.numel())."""

    def __init__(self, segments, block: int):
        self.segments = list(segments)
        self.arr = (EfqSegment * max(len(self.segments), 1))()
        self.dtype = None
        for i, (g, ef, codes, scales) in enumerate(self.segments):
            n = g.numel()
            _need("g", g, n, _FLOAT)
            _need("ef", ef, n, _F32)
            _need("codes", codes, (n + 1) // 2, _U8)
            _need("scales", scales, (n + block - 1) // block, _F32)
            dt = _dtype(g)
            if self.dtype is not None and dt != self.dtype:
                raise TypeError("all segments of a batch share one gradient dtype")
            self.dtype = dt
            self.arr[i] = EfqSegment(_p(g), _p(ef), _p(codes), _p(scales), n)
        self.block = block
        self.ptr = C.cast(self.arr, C.c_void_p)


def zq_quantize_ef_int4_batched(segments, block: int, beta_e: float, beta_r: float,
                                stream=None) -> None:
    """Per-tensor EF int4 quantize of many tensors in one call: `segments` is
    an EfqSegmentTable or an iterable of (g, ef or None, codes, scales)."""
    table = segments if isinstance(segments, EfqSegmentTable) else EfqSegmentTable(segments, block)
    if table.block != block:
        raise ValueError(f"the segment table was checked for block {table.block}, not {block}")
    _check("zq_quantize_ef_int4_batched",
           lib.zq_quantize_ef_int4_batched(table.ptr, len(table.segments),
                                           ZQ_FP32 if table.dtype is None else table.dtype, block,
                                           beta_e, beta_r, _stream(stream)))


class DrSegmentTable:
    """A marshalled segment table for zq_dequant_reduce_batched.  Each
    segment is (codes, scales, n, codes_stride, scales_stride, out, rq_codes,
    rq_scales, rq_ef): codes a uint8 tensor holding the P peer chunks (peer q
    at byte q * codes_stride), scales a float32 tensor (peer q at element
    q * scales_stride); outputs as in zq_dequant_reduce (None for absent)."""

    def __init__(self, segments, P: int, block: int):
        self.segments = list(segments)
        self.arr = (DrSegment * max(len(self.segments), 1))()
        nbk = lambda n: (n + block - 1) // block
        for i, (codes, scales, n, cst, sst, out, rqc, rqs, rqe) in enumerate(self.segments):
            _need("codes", codes, (P - 1) * cst + (n + 1) // 2 if n else 0, _U8)
            _need("scales", scales, (P - 1) * sst + nbk(n) if n else 0, _F32)
            _need("out", out, n, _F32)
            _need("rq_codes", rqc, (n + 1) // 2, _U8)
            _need("rq_scales", rqs, nbk(n), _F32)
            _need("rq_ef", rqe, n, _F32)
            self.arr[i] = DrSegment(_p(codes), _p(scales), cst, sst, n, _p(out), _p(rqc), _p(rqs),
                                    _p(rqe))
        self.P, self.block = P, block
        self.ptr = C.cast(self.arr, C.c_void_p)


def zq_dequant_reduce_batched(segments, P: int, block: int, alpha: float, rq_beta_e: float = 0.0,
                              rq_beta_r: float = 1.0, stream=None) -> None:
    """Per-tensor dequantize-reduce(-requant) of many tensors in one call:
    `segments` is a DrSegmentTable or an iterable of its tuples."""
    table = segments if isinstance(segments, DrSegmentTable) else DrSegmentTable(segments, P, block)
    if (table.P, table.block) != (P, block):
        raise ValueError(f"the segment table was checked for P={table.P}, block={table.block}, "
                         f"not P={P}, block={block}")
    _check("zq_dequant_reduce_batched",
           lib.zq_dequant_reduce_batched(table.ptr, len(table.segments), P, block, alpha, rq_beta_e,
                                         rq_beta_r, _stream(stream)))
