"""C-ABI checks that need no GPU: the library loads, exports every symbol
include/zq.h declares, its host helpers agree with the layout rules, and
every validation error returns its status before any device work (all
pointers below are fake and never dereferenced).  The host helpers are also
tied to the pages' communication-volume closed form via the oracle."""
import ctypes as C

import pytest

import oracle as O
from weight_communication_zero_amd import zq

L = zq.lib
FAKE = 0x10000  # 16-byte aligned, never dereferenced: every call below fails validation first


def test_exports_every_declared_symbol():
    names = zq.declared_symbols()
    assert set(names) == {"zq_quantize_ef_int4", "zq_quantize_ef_int4_permuted",
                          "zq_quantize_ef_int4_batched",
                          "zq_dequant_reduce", "zq_dequant_reduce_batched", "zq_quant_int8",
                          "zq_dequant_int8", "zq_sr_accumulate", "zq_sr_accumulate_batched",
                          "zq_int4_code_bytes", "zq_zeropp_slots",
                          "zq_num_blocks", "zq_status_str", "zq_abi_version"}
    for name in names:
        assert hasattr(L, name), name


def test_host_helpers():
    assert L.zq_abi_version() == 2
    for n in [0, 1, 2, 3, 4095, 2 ** 33 + 1]:
        assert L.zq_int4_code_bytes(n) == (n + 1) // 2
        for b in [32, 128, 4096]:
            assert L.zq_num_blocks(n, b) == -(-n // b)
    assert L.zq_num_blocks(10, 0) == 0
    for s in range(9):
        assert L.zq_status_str(s).decode().startswith(zq.STATUS[s])
    assert L.zq_status_str(99).decode() == "unknown zq_status"


def test_volume_from_library_buffer_sizes_matches_pages():
    """Bytes libzq's layout puts on the wire (codes + fp32 scales) for the
    0.85B model at the int8 / int4 block sizes equal the oracle's closed form
    of the pages' 0.5M + 0 + 0.25M count."""
    M = 850454528
    int8_bytes = M + 4 * L.zq_num_blocks(M, 2048)
    int4_bytes = L.zq_int4_code_bytes(M) + 4 * L.zq_num_blocks(M, 128)
    zero3, zpp = O.volume_bytes(M, 2048, 128)
    assert int8_bytes + 0 + int4_bytes == zpp and zero3 == 6 * M


def efq(g=FAKE, dt=0, ef=None, n=1024, block=128, codes=FAKE + 0x100000, scales=FAKE + 0x200000):
    return L.zq_quantize_ef_int4(g, dt, ef, n, block, 1.0, 1.0, codes, scales, None)


def test_quantize_validation():
    assert efq(dt=3) == zq.ZQ_ERR_DTYPE
    # fp16 (2) is a known dtype: validation goes on, with 2-byte elements
    assert efq(dt=zq.ZQ_FP16, g=FAKE + 4) == zq.ZQ_ERR_ALIGN
    assert efq(dt=zq.ZQ_FP16, codes=FAKE + 0x7F0) == zq.ZQ_ERR_ALIAS  # inside g's 2048 bytes
    assert efq(dt=zq.ZQ_FP32, codes=FAKE + 0xFF0) == zq.ZQ_ERR_ALIAS  # inside g's 4096 bytes
    for b in [0, 16, 100, 8192, 129]:
        assert efq(block=b) == zq.ZQ_ERR_BLOCK
    assert efq(n=(1 << 60) + 1) == zq.ZQ_ERR_SIZE
    assert efq(g=None, n=0) == zq.ZQ_OK  # n == 0 touches no pointer
    assert efq(g=None) == zq.ZQ_ERR_NULL
    assert efq(codes=None) == zq.ZQ_ERR_NULL
    assert efq(scales=None) == zq.ZQ_ERR_NULL
    assert efq(g=FAKE + 4) == zq.ZQ_ERR_ALIGN
    assert efq(ef=FAKE + 0x300008) == zq.ZQ_ERR_ALIGN
    assert efq(codes=FAKE + 0x100001) == zq.ZQ_ERR_ALIGN
    assert efq(scales=FAKE + 0x200002) == zq.ZQ_ERR_ALIGN
    assert efq(codes=FAKE + 0x10) == zq.ZQ_ERR_ALIAS  # codes inside g
    assert efq(scales=FAKE + 0x100010) == zq.ZQ_ERR_ALIAS  # scales inside codes
    assert efq(ef=FAKE + 0x10) == zq.ZQ_ERR_ALIAS  # ef overlaps g
    assert efq(ef=FAKE + 0x300000, codes=FAKE + 0x300000) == zq.ZQ_ERR_ALIAS


def dr(P=4, codes=None, scales=None, n=1024, block=128, out=FAKE + 0x400000, rq_codes=None,
       rq_scales=None, rq_ef=None):
    cp = codes or [FAKE + 0x1000 * i for i in range(max(P, 1))]
    sp = scales or [FAKE + 0x100000 + 0x1000 * i for i in range(max(P, 1))]
    ca = (C.c_void_p * len(cp))(*cp)
    sa = (C.c_void_p * len(sp))(*sp)
    return L.zq_dequant_reduce(P, ca, sa, n, block, 0.25, out, rq_codes, rq_scales, rq_ef, 0.0, 1.0,
                               None)


def test_dequant_reduce_validation():
    assert dr(P=0) == zq.ZQ_ERR_PEERS
    assert dr(P=17) == zq.ZQ_ERR_PEERS
    assert dr(block=48) == zq.ZQ_ERR_BLOCK
    assert dr(n=0, out=None) == zq.ZQ_OK
    assert dr(out=None) == zq.ZQ_ERR_NULL  # neither out nor requant
    assert dr(codes=[FAKE, None, FAKE + 0x2000, FAKE + 0x3000]) == zq.ZQ_ERR_NULL
    assert dr(rq_codes=FAKE + 0x500000) == zq.ZQ_ERR_NULL  # rq_scales missing
    assert dr(rq_ef=FAKE + 0x600000) == zq.ZQ_ERR_NULL  # rq_ef without requant
    assert dr(codes=[FAKE + 8, FAKE + 0x1000, FAKE + 0x2000, FAKE + 0x3000]) == zq.ZQ_ERR_ALIGN
    assert dr(out=FAKE + 0x400004) == zq.ZQ_ERR_ALIGN
    assert dr(out=FAKE + 0x1000) == zq.ZQ_ERR_ALIAS  # out over chunk 1's codes
    assert dr(rq_codes=FAKE + 0x400100, rq_scales=FAKE + 0x500000) == zq.ZQ_ERR_ALIAS
    assert dr(out=None, rq_codes=FAKE + 0x500000, rq_scales=FAKE + 0x100000) == zq.ZQ_ERR_ALIAS


def test_int8_and_sr_validation():
    q8 = lambda **k: L.zq_quant_int8(k.get("w", FAKE), k.get("dt", 1), k.get("n", 4096),
                                     k.get("block", 2048), k.get("codes", FAKE + 0x100000),
                                     k.get("scales", FAKE + 0x200000), None)
    assert q8(dt=5) == zq.ZQ_ERR_DTYPE
    assert q8(block=3000) == zq.ZQ_ERR_BLOCK
    assert q8(w=None) == zq.ZQ_ERR_NULL
    assert q8(codes=FAKE + 0x100008) == zq.ZQ_ERR_ALIGN
    assert q8(codes=FAKE + 0x1000) == zq.ZQ_ERR_ALIAS
    assert q8(dt=zq.ZQ_FP16, codes=FAKE + 0x1000) == zq.ZQ_ERR_ALIAS  # w is 8 KB of fp16
    dq = lambda **k: L.zq_dequant_int8(k.get("codes", FAKE), k.get("scales", FAKE + 0x100000),
                                       k.get("n", 4096), 2048, k.get("out", FAKE + 0x200000),
                                       k.get("dt", 1), None)
    assert dq(dt=9) == zq.ZQ_ERR_DTYPE
    assert dq(out=None) == zq.ZQ_ERR_NULL
    assert dq(out=FAKE + 0x200002) == zq.ZQ_ERR_ALIGN
    assert dq(out=FAKE + 0x800) == zq.ZQ_ERR_ALIAS
    assert dq(dt=zq.ZQ_FP16, out=FAKE + 0x200002) == zq.ZQ_ERR_ALIGN
    sr = lambda **k: L.zq_sr_accumulate(k.get("dst", FAKE), k.get("src", FAKE + 0x100000),
                                        k.get("n", 4096), 1, k.get("cb", 0), 0, None)
    assert sr(n=0, dst=None) == zq.ZQ_OK
    assert sr(dst=None) == zq.ZQ_ERR_NULL
    assert sr(src=FAKE + 0x100004) == zq.ZQ_ERR_ALIGN
    assert sr(src=FAKE + 0x1000) == zq.ZQ_ERR_ALIAS
    assert sr(cb=(1 << 64) - 100) == zq.ZQ_ERR_SIZE


def test_binding_guards_reject_short_or_host_buffers():
    import torch
    with pytest.raises(ValueError):
        zq.zq_quantize_ef_int4(torch.zeros(16), None, 32, 1.0, 1.0, torch.zeros(8, dtype=torch.uint8),
                               torch.zeros(1))


def test_binding_refuses_a_segment_table_used_with_other_sizes():
    """A marshalled table's buffers were checked for its own P and block;
    a call with another P or block would let the kernels index past them,
    so the binding refuses it before calling the library.  The fake
    pointers are misaligned as well, so the C ABI would refuse them too."""
    odd = FAKE + 4
    dr = zq.DrSegmentTable([(odd, odd + 0x100000, 4096, 2048, 32, odd + 0x200000, None, None,
                             None)], P=4, block=128)
    with pytest.raises(ValueError, match="P=4, block=128"):
        zq.zq_dequant_reduce_batched(dr, 8, 128, 1.0)
    with pytest.raises(ValueError, match="P=4, block=128"):
        zq.zq_dequant_reduce_batched(dr, 4, 64, 1.0)
    with pytest.raises(zq.ZQError, match="ALIGN"):  # same sizes: the C ABI's own checks run
        zq.zq_dequant_reduce_batched(dr, 4, 128, 1.0, stream=0)
    # an EF-quantize table of 4096 elements at block 256 (raw pointers)
    efq = zq.EfqSegmentTable.__new__(zq.EfqSegmentTable)
    efq.segments = [None]
    efq.arr = (zq.EfqSegment * 1)(zq.EfqSegment(odd, None, odd + 0x100000, odd + 0x200000, 4096))
    efq.dtype, efq.block, efq.ptr = zq.ZQ_FP32, 256, C.cast(efq.arr, C.c_void_p)
    with pytest.raises(ValueError, match="block 256"):
        zq.zq_quantize_ef_int4_batched(efq, 128, 1.0, 1.0)
    with pytest.raises(zq.ZQError, match="ALIGN"):
        zq.zq_quantize_ef_int4_batched(efq, 256, 1.0, 1.0, stream=0)


def test_sr_batched_validation():
    Seg = zq.SrSegment

    def call(segs, zero=0, n_seg=None):
        arr = (Seg * max(len(segs), 1))(*segs)
        return L.zq_sr_accumulate_batched(C.cast(arr, C.c_void_p), len(segs) if n_seg is None else n_seg,
                                          zero, None)

    ok = Seg(FAKE, FAKE + 0x100000, 100, 8, 200, 1, 0)
    assert L.zq_sr_accumulate_batched(None, 0, 0, None) == zq.ZQ_OK
    assert L.zq_sr_accumulate_batched(None, 3, 0, None) == zq.ZQ_ERR_NULL
    assert call([ok], n_seg=70000) == zq.ZQ_ERR_SIZE
    assert call([Seg(FAKE, FAKE + 0x100000, 100, 8, 50, 1, 0)]) == zq.ZQ_ERR_SIZE  # slice past src_len
    assert call([Seg(FAKE, FAKE + 0x100000, 100, 8, 200, 1, (1 << 64) - 50)]) == zq.ZQ_ERR_SIZE
    assert call([Seg(None, FAKE + 0x100000, 100, 8, 200, 1, 0)]) == zq.ZQ_ERR_NULL
    assert call([Seg(FAKE, None, 100, 8, 200, 1, 0)]) == zq.ZQ_ERR_NULL
    assert call([Seg(FAKE + 2, FAKE + 0x100000, 100, 8, 200, 1, 0)]) == zq.ZQ_ERR_ALIGN
    assert call([Seg(FAKE, FAKE + 0x100000, 100, 4, 200, 1, 0)]) == zq.ZQ_ERR_ALIGN  # offset % 8
    # two segments whose dst overlap
    assert call([ok, Seg(FAKE + 0x40, FAKE + 0x200000, 100, 0, 100, 1, 0)]) == zq.ZQ_ERR_ALIAS
    # reading the same slice twice is allowed, clearing it while another reads it is not
    a = Seg(FAKE, FAKE + 0x100000, 100, 8, 200, 1, 0)
    b = Seg(FAKE + 0x10000, FAKE + 0x100000, 100, 8, 200, 2, 0)
    assert call([a, b], zero=1) == zq.ZQ_ERR_ALIAS
    # a dst inside another segment's read slice
    assert call([a, Seg(FAKE + 0x100000 + 0x20, FAKE + 0x300000, 8, 0, 8, 1, 0)]) == zq.ZQ_ERR_ALIAS


def test_permuted_quantize_validation():
    def call(n=8 * 1024, block=128, n_part=8, slots=None, g=FAKE, codes=FAKE + 0x1000000,
             scales=FAKE + 0x2000000):
        slots = list(range(n_part)) if slots is None else slots
        arr = (C.c_uint32 * max(len(slots), 1))(*slots)
        return L.zq_quantize_ef_int4_permuted(g, 0, None, n, block, 1.0, 1.0, codes, scales,
                                              n_part, C.cast(arr, C.c_void_p), None)
    assert call(block=96) == zq.ZQ_ERR_BLOCK
    assert call(n_part=0, slots=[0]) == zq.ZQ_ERR_SIZE
    assert call(n_part=257, slots=list(range(257))) == zq.ZQ_ERR_SIZE
    assert call(n=8 * 1024 + 8) == zq.ZQ_ERR_SIZE            # not n_part equal partitions
    assert call(n=8 * 512) == zq.ZQ_ERR_SIZE                 # partition shorter than 1024
    assert call(n=8 * 1088, block=128) == zq.ZQ_ERR_SIZE    # partition not whole blocks
    assert call(slots=[0, 1, 2, 3, 4, 5, 6, 6]) == zq.ZQ_ERR_SIZE  # not a permutation
    assert call(slots=[0, 1, 2, 3, 4, 5, 6, 8]) == zq.ZQ_ERR_SIZE
    assert call(g=None) == zq.ZQ_ERR_NULL
    assert call(n=0, g=None) == zq.ZQ_OK
    assert call(codes=FAKE + 0x1000002) == zq.ZQ_ERR_ALIGN
    assert call(codes=FAKE + 0x100) == zq.ZQ_ERR_ALIAS


def test_zeropp_slots_through_the_c_abi(golden_dir):
    """zq_zeropp_slots against the hand-worked tables of the pages' two-level
    order, through the raw C ABI, and the binding passing it through."""
    import json
    import os
    with open(os.path.join(golden_dir, "zeropp_order_worked.json")) as f:
        G = json.load(f)["slots"]
    for (intra, inter), key in (((4, 2), "intra4_inter2"), ((8, 4), "intra8_inter4"),
                                ((1, 3), "intra1_inter3"), ((3, 1), "intra3_inter1")):
        out = (C.c_uint32 * (intra * inter))(*([0xDEAD] * (intra * inter)))
        assert L.zq_zeropp_slots(intra, inter, out) == intra * inter
        assert list(out) == G[key]
        assert zq.zeropp_slots(intra, inter) == G[key]
    out = (C.c_uint32 * 4)(7, 7, 7, 7)
    for intra, inter in ((0, 4), (4, 0), (16, 17)):
        assert L.zq_zeropp_slots(intra, inter, out) == 0
    assert L.zq_zeropp_slots(2, 2, None) == 0
    assert list(out) == [7, 7, 7, 7]
    with pytest.raises(ValueError):
        zq.zeropp_slots(0, 2)


def test_efq_batched_validation():
    Seg = zq.EfqSegment

    def call(segs, dt=0, block=128, n_seg=None):
        arr = (Seg * max(len(segs), 1))(*segs)
        return L.zq_quantize_ef_int4_batched(C.cast(arr, C.c_void_p),
                                             len(segs) if n_seg is None else n_seg, dt, block, 1.0,
                                             1.0, None)

    def seg(base, n=4096, ef=True):
        return Seg(base, base + 0x100000 if ef else None, base + 0x200000, base + 0x300000, n)

    a, b = seg(FAKE), seg(FAKE + 0x1000000)
    assert call([a], dt=3) == zq.ZQ_ERR_DTYPE
    assert call([a], block=33) == zq.ZQ_ERR_BLOCK
    assert L.zq_quantize_ef_int4_batched(None, 0, 0, 128, 1.0, 1.0, None) == zq.ZQ_OK
    assert L.zq_quantize_ef_int4_batched(None, 2, 0, 128, 1.0, 1.0, None) == zq.ZQ_ERR_NULL
    assert call([a], n_seg=70000) == zq.ZQ_ERR_SIZE
    assert call([seg(FAKE, n=(1 << 40) + 1)]) == zq.ZQ_ERR_SIZE
    assert call([a, seg(FAKE + 0x1000000, ef=False)]) == zq.ZQ_ERR_NULL  # EF in some, not all
    assert call([Seg(FAKE, None, None, FAKE + 0x300000, 4096)]) == zq.ZQ_ERR_NULL
    assert call([Seg(FAKE + 8, None, FAKE + 0x200000, FAKE + 0x300000, 4096)]) == zq.ZQ_ERR_ALIGN
    assert call([a, seg(FAKE + 0x100)]) == zq.ZQ_ERR_ALIAS  # b's g inside a's g? no: outputs overlap
    assert call([a, Seg(FAKE + 0x10000, FAKE + 0x1100000, FAKE + 0x200100, FAKE + 0x1300000, 64)]) \
        == zq.ZQ_ERR_ALIAS  # codes overlap
    assert call([Seg(FAKE, None, FAKE + 0x200000, FAKE + 0x300000, 0)]) == zq.ZQ_OK  # all empty


def test_dequant_reduce_batched_validation():
    Seg = zq.DrSegment

    def call(segs, P=8, block=128, n_seg=None):
        arr = (Seg * max(len(segs), 1))(*segs)
        return L.zq_dequant_reduce_batched(C.cast(arr, C.c_void_p),
                                           len(segs) if n_seg is None else n_seg, P, block, 1.0,
                                           0.0, 1.0, None)

    def seg(base, n=4096, out=True, rq=False, ef=False, cs=None, ss=None):
        cs = n // 2 if cs is None else cs
        ss = n // 128 if ss is None else ss
        return Seg(base, base + 0x100000, cs, ss, n, base + 0x200000 if out else None,
                   base + 0x300000 if rq else None, base + 0x340000 if rq else None,
                   base + 0x380000 if ef else None)

    a, b = seg(FAKE), seg(FAKE + 0x1000000)
    assert call([a], P=0) == zq.ZQ_ERR_PEERS
    assert call([a], P=17) == zq.ZQ_ERR_PEERS
    assert call([a], block=48) == zq.ZQ_ERR_BLOCK
    assert L.zq_dequant_reduce_batched(None, 0, 8, 128, 1.0, 0.0, 1.0, None) == zq.ZQ_OK
    assert L.zq_dequant_reduce_batched(None, 3, 8, 128, 1.0, 0.0, 1.0, None) == zq.ZQ_ERR_NULL
    assert call([a], n_seg=65537) == zq.ZQ_ERR_SIZE
    assert call([seg(FAKE, n=(1 << 40) + 2)]) == zq.ZQ_ERR_SIZE
    assert call([a, seg(FAKE + 0x1000000, out=False, rq=True)]) == zq.ZQ_ERR_NULL  # mixed outputs
    assert call([seg(FAKE, out=False)]) == zq.ZQ_ERR_NULL                          # no output
    assert call([seg(FAKE, ef=True)]) == zq.ZQ_ERR_NULL                            # EF without requant
    assert call([Seg(None, FAKE, 2048, 32, 4096, FAKE + 0x200000, None, None, None)]) == zq.ZQ_ERR_NULL
    assert call([seg(FAKE, cs=2047)]) == zq.ZQ_ERR_SIZE                            # stride too short
    assert call([seg(FAKE, ss=31)]) == zq.ZQ_ERR_SIZE
    assert call([seg(FAKE, cs=2056)]) == zq.ZQ_ERR_ALIGN                           # stride % 16
    # for P = 1 the stride is not checked: this call gets as far as the alias check
    assert call([Seg(FAKE, FAKE + 0x100000, 7, 0, 4096, FAKE + 0x400, None, None, None)],
                P=1) == zq.ZQ_ERR_ALIAS
    assert call([Seg(FAKE + 4, FAKE + 0x100000, 2048, 32, 4096, FAKE + 0x200000, None, None,
                     None)]) == zq.ZQ_ERR_ALIGN
    # the output of one segment inside the input chunks of another
    assert call([a, Seg(FAKE + 0x1000000, FAKE + 0x1100000, 2048, 32, 4096, FAKE + 0x2000, None,
                        None, None)]) == zq.ZQ_ERR_ALIAS
    # two segments writing the same output
    assert call([a, Seg(FAKE + 0x1000000, FAKE + 0x1100000, 2048, 32, 4096, FAKE + 0x200000, None,
                        None, None)]) == zq.ZQ_ERR_ALIAS


def test_header_is_c99_and_the_library_links_from_c(tmp_path):
    """include/zq.h is plain C: a C99 program (-pedantic -Werror) includes it,
    links libzq.so and calls the host-only entry points (no GPU is touched)."""
    import os
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    src = tmp_path / "use_zq.c"
    src.write_text(r'''
#include <stdio.h>
#include <string.h>
#include "zq.h"
int main(void) {
    uint32_t slot[8];
    if (zq_zeropp_slots(4, 2, slot) != 8) return 1;
    /* rank node*4 + local sits in slot local*2 + node */
    if (slot[1] != 2 || slot[4] != 1 || slot[7] != 7) return 2;
    if (zq_int4_code_bytes(7) != 4 || zq_num_blocks(1000, 128) != 8) return 3;
    if (strcmp(zq_status_str(ZQ_ERR_ALIGN), zq_status_str(ZQ_OK)) == 0) return 4;
    /* a refused call enqueues nothing and needs no device */
    if (zq_quantize_ef_int4(NULL, ZQ_FP16, NULL, 16, 128, 1.0f, 1.0f, NULL, NULL, NULL) !=
        ZQ_ERR_NULL) return 5;
    puts("ok");
    return 0;
}
''')
    exe = tmp_path / "use_zq"
    lib = os.path.join(root, "weight_communication_zero_amd", "libzq.so")
    r = subprocess.run([gcc, "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
                        "-I", os.path.join(root, "include"), str(src), lib,
                        "-Wl,-rpath," + os.path.dirname(lib), "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)
