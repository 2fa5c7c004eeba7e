"""Benchmark of the qgZ + LoCo data-parallel hot path on one MI355X.

Workload (one step = one pass of the whole gradient path over one batch):
one GPU's share of a ~7.5B Llama-2-style fp32 gradient (36 layers, hidden
4096, FFN 11008, vocab 32000: 7,547,949,056 elements, heavy-tailed embedding,
lm_head and first/last block), i.e. the two-level qgZ of "ZeROPlusPlus.md"
(section 1.2) with LoCo error feedback ("Merge LoCo with Zero++", Overview):
  1. EF int4 quantize of the whole gradient, block 128, beta 0.9;
  2. 8-way dequantize-reduce-requantize of the intra-node chunk (M/8 elements);
  3. 4-way dequantize-reduce of the inter-node sub-chunk (M/32), alpha 1/32.
On one GPU the exchanges are identities: this GPU's own 8 chunks (resp. 4
sub-chunks) stand in for the peers' chunks -- same shapes, same bytes.

value = algorithmic bytes of one step / measured step time (inputs resident
in HBM).  The same run also times the other kernels of the path on their own
workloads (int8 weight quantize/dequantize of a ~0.85B model, stochastic-
rounding accumulation of GPT-2 124M gradients, the 0.85B EF-quantize + 8-way
reduce, the 4-rank bf16 case), the step's variants at 7.5B (requant EF, bf16
and fp16 gradients, the ZeRO++ partition order, the per-parameter batched
calls) and the CPU oracle on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
METRIC = "effective HBM GB/s (and % of peak) for EF-int4 quantize + P-way dequant-reduce"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-rows", action="store_true", help="skip the per-row extra workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--main-only", action="store_true",
                    help="only the step's three kernels (no variant or extra rows): for profiling")
    ap.add_argument("--cpu-sample-elems", type=int, default=3 << 30,
                    help="gradient elements the CPU oracle processes (a multiple of 4096)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="after the timed steps, run a 1 GiB fp32 copy (known HBM bytes) so that "
                         "rocprofv3 memory counters can be scaled")
    ap.add_argument("--kernels", action="store_true",
                    help="time every entry point on 2^31-element buffers next to torch copy / add / "
                         "sum / fill ceilings, print one line and exit (with ZQ_LIB=<build> this "
                         "compares library builds)")
    ap.add_argument("--summarize-rocprof", metavar="DIR",
                    help="print a summary of the rocprofv3 CSV output under DIR and exit")
    return ap.parse_args()


# ----------------------------------------------------------- byte counts --

def efq_bytes(n, block, g_bytes, ef=True):
    return n * (g_bytes + (8 if ef else 0) + 0.5) + 4 * math.ceil(n / block)


def dr_bytes(n, block, P, out=True, rq=False, rq_ef=False):
    per_chunk = 0.5 * n + 4 * math.ceil(n / block)
    b = P * per_chunk
    if out:
        b += 4 * n
    if rq:
        b += per_chunk
    if rq_ef:
        b += 8 * n
    return b


class EventTimer:
    """HIP events on torch's current stream (the stream libzq launches on)."""

    def __init__(self, torch):
        self.torch = torch
        self.spans = {}

    def span(self, name):
        ev0 = self.torch.cuda.Event(enable_timing=True)
        ev1 = self.torch.cuda.Event(enable_timing=True)
        ev0.record()
        timer = self

        class _S:
            def __enter__(self_):
                return self_

            def __exit__(self_, *a):
                ev1.record()
                timer.spans.setdefault(name, []).append((ev0, ev1))
        return _S()

    def ms(self, name):
        return [a.elapsed_time(b) for a, b in self.spans.get(name, [])]


def main():
    args = parse()
    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof)
        return
    if args.kernels:
        kernel_table()
        return
    if args.gpus != 1:
        print(f"bench.py: libzq measures one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU exchange (RCCL all-to-all over xGMI) is not implemented.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from weight_communication_zero_amd import zq

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    log = lambda *a: print("[bench]", *a, file=sys.stderr, flush=True)

    # ---------------------------------------------------- main workload --
    tensors = synth.llama_7p5b()
    M = synth.total(tensors)
    B = 128
    P1, P2 = 8, 4
    n1, n2 = M // P1, M // (P1 * P2)
    beta = 0.9
    log(f"allocating {M} fp32 gradient + EF + codes on {torch.cuda.get_device_name(0)}")
    g = torch.empty(M, dtype=torch.float32, device=dev)
    t0 = time.time()
    synth.fill_model(g, tensors, std=1e-3, seed=synth.seed_for("llama7p5b", "grad"),
                     heavy_tails=True)
    ef = torch.zeros(M, dtype=torch.float32, device=dev)
    codes = torch.empty(zq.int4_code_bytes(M), dtype=torch.uint8, device=dev)
    scales = torch.empty(zq.num_blocks(M, B), dtype=torch.float32, device=dev)
    rq_codes = torch.empty(zq.int4_code_bytes(n1), dtype=torch.uint8, device=dev)
    rq_scales = torch.empty(zq.num_blocks(n1, B), dtype=torch.float32, device=dev)
    out2 = torch.empty(n2, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s")

    cb1, sb1 = n1 // 2, n1 // B
    cb2, sb2 = n2 // 2, n2 // B
    chunks_c = [codes[j * cb1:(j + 1) * cb1] for j in range(P1)]
    chunks_s = [scales[j * sb1:(j + 1) * sb1] for j in range(P1)]
    sub_c = [rq_codes[j * cb2:(j + 1) * cb2] for j in range(P2)]
    sub_s = [rq_scales[j * sb2:(j + 1) * sb2] for j in range(P2)]

    def step(timer=None):
        def run(name, fn):
            if timer is None:
                fn()
            else:
                with timer.span(name):
                    fn()
        run("efq", lambda: zq.zq_quantize_ef_int4(g, ef, B, beta, 1.0, codes, scales))
        run("dr_rq", lambda: zq.zq_dequant_reduce(chunks_c, chunks_s, n1, B, 1.0, out=None,
                                                  rq_codes=rq_codes, rq_scales=rq_scales))
        run("dr", lambda: zq.zq_dequant_reduce(sub_c, sub_s, n2, B, 1.0 / 32, out=out2))

    bytes_efq = efq_bytes(M, B, 4)
    bytes_dr_rq = dr_bytes(n1, B, P1, out=False, rq=True)
    bytes_dr = dr_bytes(n2, B, P2, out=True)
    bytes_step = bytes_efq + bytes_dr_rq + bytes_dr

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timer = EventTimer(torch)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        step(timer)
    t_end.record()
    torch.cuda.synchronize()
    step_ms = t_start.elapsed_time(t_end) / max(args.steps, 1)
    k_ms = {k: float(np.mean(timer.ms(k))) for k in ("efq", "dr_rq", "dr")}
    # spread of the per-launch event times over the timed steps
    k_pct = {k: [round(float(v), 4) for v in np.percentile(timer.ms(k), [10, 50, 90])]
             for k in ("efq", "dr_rq", "dr")}
    value = bytes_step / (step_ms * 1e-3) / 1e9
    log(f"step {step_ms:.3f} ms, {value:.1f} GB/s; kernels (ms) {k_ms}")

    if args.calib_copy:
        a = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    efq_gbs = bytes_efq / (k_ms["efq"] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(efq_gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(efq_gbs / PEAK_HBM_GBS, 4),
                "traffic": measured_traffic("efq_fp32_b128", bytes_efq),
                "kernel": "efq_kernel<fp32, ef, B=128>", "bytes_per_launch": bytes_efq,
                "avg_launch_ms": round(k_ms["efq"], 4)}

    rows = {}
    if not args.main_only:
        rows.update(variant_rows(torch, zq, g, ef, codes, scales, chunks_c, chunks_s, rq_codes,
                                 rq_scales, tensors, M, n1, B, P1, P2, beta, bytes_efq, dev))
    rows.update({
        "efq_fp32_b128_7.5B": row(bytes_efq, k_ms["efq"], M),
        "dequant_reduce_requant_p8_b128_7.5B": row(bytes_dr_rq, k_ms["dr_rq"], n1),
        "dequant_reduce_p4_b128_7.5B": row(bytes_dr, k_ms["dr"], n2),
    })
    for name, k in (("efq_fp32_b128_7.5B", "efq"), ("dequant_reduce_requant_p8_b128_7.5B", "dr_rq"),
                    ("dequant_reduce_p4_b128_7.5B", "dr")):
        rows[name]["ms_p10_p50_p90"] = k_pct[k]
    # counter-measured HBM bytes of the reduce-requant, while its profile is current
    tr = measured_traffic("dequant_reduce_requant_p8_b128_7.5B", bytes_dr_rq)
    rows["dequant_reduce_requant_p8_b128_7.5B"]["traffic"] = tr
    rows["dequant_reduce_requant_p8_b128_7.5B"]["traffic_ratio"] = (
        round(tr / bytes_dr_rq, 4) if tr else None)

    # ---------------------------------------------------- CPU baseline --
    cpu = None
    if not args.no_cpu:
        S = args.cpu_sample_elems
        g_host = g[:S].cpu().numpy()
        cpu = cpu_baseline(g_host, B, beta, P1, P2)
        del g_host
        log(f"cpu baseline {cpu}")

    del g, ef, codes, scales, rq_codes, rq_scales, out2, chunks_c, chunks_s, sub_c, sub_s
    torch.cuda.empty_cache()

    extras = not (args.no_rows or args.main_only)
    if extras:
        rows.update(extra_rows(torch, zq, synth, dev, log, cpu=not args.no_cpu))
    ceil = ceilings(torch, dev) if extras else None
    if ceil:
        roofline["ceilings_measured"] = ceil
        roofline["frac_of_mixed_ceiling"] = round(efq_gbs / ceil["torch_add_2r1w"], 4)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded normal gradients, Student-t heavy-tailed tensors; no dataset)",
        "config": {
            "workload": "two-level qgZ + LoCo on one GPU's share of a ~7.5B Llama-2-style fp32 "
                        "gradient: EF int4 quantize (block 128, beta 0.9) -> 8-way "
                        "dequant-reduce-requant -> 4-way dequant-reduce (alpha 1/32)",
            "elements": M, "block": B, "peers_intra": P1, "peers_inter": P2,
            "bytes_per_step": bytes_step, "frac_of_peak": round(value / PEAK_HBM_GBS, 4),
            "gpu": torch.cuda.get_device_name(0),
            "gpu_arch": getattr(torch.cuda.get_device_properties(0), "gcnArchName", None),
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "pages_context": pages_context(zq, M),
        "rows": rows,
    }
    print(json.dumps(line), flush=True)


def pages_context(zq, M):
    """The pages' own system-level figures, for context only: they publish
    no kernel-level number.  ZeRO++ notes, abstract and section 1.2: ZeRO-3
    moves 3M per step (two fp16 weight all-gathers and one fp16 gradient
    reduce-scatter), ZeRO++ 0.75M (int8 weights, no inter-node backward
    gather, int4 gradients), and trains 2.16x faster at 384 GPUs (GPU model
    and workload not stated).  The bytes are counted for this model with the
    library's own buffer-size helpers, fp32 scales included."""
    zero3 = 3 * 2 * M
    zeropp = (M + 4 * zq.num_blocks(M, 2048)) + (zq.int4_code_bytes(M) + 4 * zq.num_blocks(M, 128))
    return {
        "note": "context only, not a target",
        "comm_bytes_per_step_7.5B": {"zero3": zero3, "zeropp_int8_w2048_int4_g128": zeropp,
                                     "ratio": round(zero3 / zeropp, 3),
                                     "pages": "3M -> 0.75M in fp16 units (4x), scales not counted"},
        "zeropp_throughput_vs_zero": "2.16x at 384 GPUs (GPU model and workload not stated)",
    }


def ceilings(torch, dev):
    """Practical HBM ceilings of this GPU for each traffic mix, from torch's
    own streaming kernels on 2^30-element fp32 buffers: read-only (sum),
    write-only (fill), copy (1 read : 1 write) and add (2 reads : 1 write,
    the mix closest to EF quantize's 8 B read : 4.5 B written)."""
    n = 1 << 30
    a = torch.randn(n, device=dev)
    b = torch.randn(n, device=dev)
    c = torch.empty(n, device=dev)
    out = {
        "torch_sum_read": 4 * n / timed(torch, lambda: a.sum(), 10) / 1e6,
        "torch_fill_write": 4 * n / timed(torch, lambda: c.fill_(1.0), 10) / 1e6,
        "torch_copy_1r1w": 8 * n / timed(torch, lambda: c.copy_(a), 10) / 1e6,
        "torch_add_2r1w": 12 * n / timed(torch, lambda: torch.add(a, b, out=c), 10) / 1e6,
    }
    del a, b, c
    torch.cuda.empty_cache()
    return {k: round(v, 1) for k, v in out.items()}


def variant_rows(torch, zq, g, ef, codes, scales, chunks_c, chunks_s, rq_codes, rq_scales,
                 tensors, M, n1, B, P1, P2, beta, bytes_efq, dev):
    """The LoCo, ZeRO++-order and per-tensor variants of the step's kernels,
    timed on the same 7.5B buffers."""
    # LoCo variant: an EF buffer at the intra-node requant as well
    rq_ef = torch.zeros(n1, dtype=torch.float32, device=dev)
    ms_rqef = timed(torch, lambda: zq.zq_dequant_reduce(chunks_c, chunks_s, n1, B, 1.0,
                                                        rq_codes=rq_codes, rq_scales=rq_scales,
                                                        rq_ef=rq_ef, rq_beta_e=beta,
                                                        rq_beta_r=1.0), 10)
    del rq_ef
    # half-precision gradients (the LoCo kernel loads half values), same EF buffer
    half_ms = {}
    for name, dt in (("bf16", torch.bfloat16), ("fp16", torch.float16)):
        gh = g.to(dt)
        half_ms[name] = timed(torch, lambda: zq.zq_quantize_ef_int4(gh, ef, B, beta, 1.0, codes,
                                                                    scales), 10)
        del gh
    # ZeRO++ hierarchical order (4 nodes x 8 GPUs): EF quantize into permuted partitions
    slots = zq.zeropp_slots(P1, P2)
    ms_perm = timed(torch, lambda: zq.zq_quantize_ef_int4_permuted(g, ef, B, beta, 1.0, codes,
                                                                   scales, slots), 10)
    # DeepSpeed-style per-parameter quantize: the 327 tensors, one batched call
    segs, off = [], 0
    for t in tensors:
        segs.append((g[off:off + t.numel], ef[off:off + t.numel],
                     codes[off // 2:(off + t.numel) // 2], scales[off // B:(off + t.numel) // B]))
        off += t.numel
    table = zq.EfqSegmentTable(segs, B)
    efqb = lambda: zq.zq_quantize_ef_int4_batched(table, B, beta, 1.0)
    ms_batched = timed_burst(torch, efqb, 10)
    host_efqb = host_enqueue_ms(torch, efqb)
    del segs, table
    # the receive side per parameter (LoCo's per-parameter reduce): tensor i's
    # receive buffer holds its 8 peer chunks of n_i / 8 elements; each is
    # reduced and requantized on its own, without and with a requant EF buffer
    # per parameter
    dsegs, dsegs_ef, off, roff = [], [], 0, 0
    rq_ef = torch.zeros(n1, dtype=torch.float32, device=dev)
    for t in tensors:
        m = t.numel // P1
        base = (codes[off // 2:(off + t.numel) // 2], scales[off // B:(off + t.numel) // B], m,
                m // 2, m // B, None, rq_codes[roff // 2:(roff + m) // 2],
                rq_scales[roff // B:(roff + m) // B])
        dsegs.append(base + (None,))
        dsegs_ef.append(base + (rq_ef[roff:roff + m],))
        off += t.numel
        roff += m
    dtable = zq.DrSegmentTable(dsegs, P1, B)
    dtable_ef = zq.DrSegmentTable(dsegs_ef, P1, B)
    drb = lambda: zq.zq_dequant_reduce_batched(dtable, P1, B, 1.0)
    drb_ef = lambda: zq.zq_dequant_reduce_batched(dtable_ef, P1, B, 1.0, beta, 1.0)
    # back-to-back calls: the host's validation of the 327-segment table
    # (reported separately) overlaps the GPU, as in a training loop
    ms_drb = timed_burst(torch, drb, 10)
    ms_drb_ef = timed_burst(torch, drb_ef, 10)
    host_drb = host_enqueue_ms(torch, drb)
    del dsegs, dsegs_ef, dtable, dtable_ef, rq_ef
    return {
        "dequant_reduce_requant_batched_327_tensors_p8_b128_7.5B": dict(
            row(dr_bytes(n1, B, P1, out=False, rq=True), ms_drb, n1),
            host_enqueue_ms=round(host_drb, 4)),
        "dequant_reduce_requant_ef_batched_327_tensors_p8_b128_7.5B": row(
            dr_bytes(n1, B, P1, out=False, rq=True, rq_ef=True), ms_drb_ef, n1),
        "efq_batched_327_tensors_fp32_b128_7.5B": dict(row(bytes_efq, ms_batched, M),
                                                       host_enqueue_ms=round(host_efqb, 4)),
        "efq_permuted_zeropp_4x8_fp32_b128_7.5B": row(bytes_efq, ms_perm, M),
        "efq_bf16_b128_7.5B": row(efq_bytes(M, B, 2), half_ms["bf16"], M),
        "efq_fp16_b128_7.5B": row(efq_bytes(M, B, 2), half_ms["fp16"], M),
        "dequant_reduce_requant_ef_p8_b128_7.5B": row(
            dr_bytes(n1, B, P1, out=False, rq=True, rq_ef=True), ms_rqef, n1),
    }


def row(nbytes, ms, elems):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "GB/s": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4),
            "Gelem/s": round(elems / (ms * 1e-3) / 1e9, 3), "bytes": nbytes}


# The sources that define each profiled kernel: its counter summary stays
# valid while these files are unchanged.
KERNEL_SOURCES = {
    "efq_fp32_b128": ("zq_device.h", "zq_launch.h", "zq_efq.hip"),
    "dequant_reduce_requant_p8_b128_7.5B": ("zq_device.h", "zq_launch.h", "zq_dr_launch.h",
                                            "zq_dr_kernels.h", "zq_dr_b128_256.hip"),
}


def kernel_source_hash(kernel_tag):
    import hashlib
    src = os.path.join(ROOT, "weight_communication_zero_amd", "csrc")
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel_tag]:
        with open(os.path.join(src, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel_tag, algorithmic_bytes):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this kernel, if its recorded source hash matches the current kernel
    source; else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel_tag}_counters.md")
    src = os.path.join(ROOT, "weight_communication_zero_amd", "csrc")
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel_tag]:
        with open(os.path.join(src, f), "rb") as fh:
            h.update(fh.read())
    text = open(path).read()
    m_hash = re.search(r"source_sha256[^:\n]*:\s*([0-9a-f]{64})", text)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_hash or not m_bytes or m_hash.group(1) != h.hexdigest():
        return None
    return float(m_bytes.group(1))


def cpu_baseline(g_host, B, beta, P1, P2):
    """The CPU oracle (single-threaded C, as written: never tuned) on a
    self-contained sample of the same path: EF quantize of the first S
    gradient elements, 8-way reduce-requant of its 8 chunks, 4-way reduce of
    the 4 sub-chunks."""
    import numpy as np

    import oracle as O
    S = g_host.size
    ef = np.zeros(S, np.float32)
    t0 = time.perf_counter()
    c, s = O.quantize_ef_int4(g_host, ef, B, beta, 1.0)
    t1 = time.perf_counter()
    n1 = S // P1
    _, rc, rs = O.dequant_reduce([c[j * n1 // 2:(j + 1) * n1 // 2] for j in range(P1)],
                                 [s[j * n1 // B:(j + 1) * n1 // B] for j in range(P1)], n1, B,
                                 1.0, want_out=False, requant=True)
    t2 = time.perf_counter()
    n2 = n1 // P2
    O.dequant_reduce([rc[j * n2 // 2:(j + 1) * n2 // 2] for j in range(P2)],
                     [rs[j * n2 // B:(j + 1) * n2 // B] for j in range(P2)], n2, B, 1.0 / 32)
    t3 = time.perf_counter()
    nbytes = efq_bytes(S, B, 4) + dr_bytes(n1, B, P1, out=False, rq=True) + dr_bytes(n2, B, P2)
    return {"value": round(nbytes / (t3 - t0) / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"first {S} elements of the same gradient: EF quantize + 8-way "
                      f"reduce-requant of its {n1}-element chunks + 4-way reduce of {n2}",
            "seconds": round(t3 - t0, 2),
            "split_s": {"efq": round(t1 - t0, 2), "dr_rq": round(t2 - t1, 2),
                        "dr": round(t3 - t2, 2)},
            "host": host_cpu_model() or platform.processor() or platform.machine(),
            "host_nproc": os.cpu_count(), "host_mem_gib": host_mem_gib()}


def to_host_np(t):
    """A device tensor as a host numpy array (bf16 as uint16 bit patterns)."""
    import numpy as np
    import torch
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def cpu_row(fn, nbytes, sample, split_of=None):
    """The oracle (single-threaded, as written) timed once on a bounded
    sample of a row's workload, in the row's own GB/s of algorithmic bytes.
    fn returns the seconds of each of its stages when split_of names them."""
    t0 = time.perf_counter()
    parts = fn()
    dt = time.perf_counter() - t0
    out = {"value": round(nbytes / dt / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": sample, "seconds": round(dt, 2)}
    if split_of:
        out["split_s"] = {k: round(v, 2) for k, v in zip(split_of, parts)}
    return out


def oracle_q8(w):
    import oracle as O
    t0 = time.perf_counter()
    c, s = O.quant_int8(w, 2048)
    t1 = time.perf_counter()
    O.dequant_int8(c, s, 2048, out_bf16=True)
    return t1 - t0, time.perf_counter() - t1


def oracle_c4(g):
    import numpy as np

    import oracle as O
    S = g.size
    t0 = time.perf_counter()
    c, s = O.quantize_ef_int4(g, np.zeros(S, np.float32), 128, 0.9, 1.0)
    t1 = time.perf_counter()
    n = S // 8
    O.dequant_reduce([c[j * n // 2:(j + 1) * n // 2] for j in range(8)],
                     [s[j * n // 128:(j + 1) * n // 128] for j in range(8)], n, 128, 0.125)
    return t1 - t0, time.perf_counter() - t1


def oracle_sr(src):
    import numpy as np

    import oracle as O
    O.sr_accumulate(np.zeros(src.size, np.uint16), src.copy(), 0, 0)


def oracle_c1(g):
    import numpy as np

    import oracle as O
    n = g.size
    t0 = time.perf_counter()
    c, s = O.quantize_ef_int4(g, np.zeros(n, np.float32), 256, 1.0, 1.0)
    t1 = time.perf_counter()
    rank, nc = n // 4, n // 16
    O.dequant_reduce([c[r * rank // 2:r * rank // 2 + nc // 2] for r in range(4)],
                     [s[r * rank // 256:r * rank // 256 + nc // 256] for r in range(4)], nc, 256, 0.25)
    return t1 - t0, time.perf_counter() - t1


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def host_mem_gib():
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal:"):
                    return round(int(line.split()[1]) / (1 << 20), 1)
    except OSError:
        pass
    return None


def summarize_rocprof(d):
    """Summaries of rocprofv3 CSVs: kernel_stats (average duration per
    kernel) and counter_collection (per-kernel mean of each counter)."""
    import csv
    import glob
    from collections import defaultdict
    for path in sorted(glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)):
        print(f"# kernel stats: {os.path.relpath(path, d)}")
        print(f"{'calls':>6} {'avg_ms':>10} {'min_ms':>10} {'max_ms':>10} {'pct':>6}  kernel")
        with open(path) as f:
            for r in csv.DictReader(f):
                print(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e6:10.4f} "
                      f"{float(r['MinNs']) / 1e6:10.4f} {float(r['MaxNs']) / 1e6:10.4f} "
                      f"{float(r['Percentage']):6.2f}  {r['Name'][:140]}")
    for path in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        print(f"# counters: {os.path.relpath(path, d)}  (value per dispatch, mean over dispatches)")
        acc = defaultdict(list)
        with open(path) as f:
            for r in csv.DictReader(f):
                acc[(r["Kernel_Name"][:140], r["Counter_Name"], r.get("Grid_Size", ""))].append(
                    float(r["Counter_Value"]))
        print(f"{'dispatches':>10} {'counter':>12} {'mean':>16} {'grid':>12}  kernel")
        for (k, c, gs), v in sorted(acc.items(), key=lambda kv: -sum(kv[1]) / len(kv[1])):
            print(f"{len(v):10d} {c:>12} {sum(v) / len(v):16.1f} {gs:>12}  {k}")


def kernel_table():
    """GB/s of every entry point on 2^31-element buffers (block 128 int4,
    2048 int8, 8- and 4-way reduce), and of torch's copy / add / sum / fill on
    the same buffers as the practical ceilings of each traffic mix."""
    import torch

    from weight_communication_zero_amd import zq
    dev = torch.device("cuda", 0)
    n, B = 1 << 31, 128
    res = {}
    g = torch.randn(n, device=dev).mul_(1e-3)
    ef = torch.zeros(n, device=dev)
    c = torch.empty(n // 2, dtype=torch.uint8, device=dev)
    s = torch.empty(n // B, device=dev)
    res["efq"] = efq_bytes(n, B, 4) / timed(torch, lambda: zq.zq_quantize_ef_int4(
        g, ef, B, 0.9, 1.0, c, s), 10) / 1e6
    n1 = n // 8
    cc = [c[j * n1 // 2:(j + 1) * n1 // 2] for j in range(8)]
    ss = [s[j * n1 // B:(j + 1) * n1 // B] for j in range(8)]
    rqc = torch.empty(n1 // 2, dtype=torch.uint8, device=dev)
    rqs = torch.empty(n1 // B, device=dev)
    out = torch.empty(n1, device=dev)
    res["dr_rq8"] = dr_bytes(n1, B, 8, out=False, rq=True) / timed(torch, lambda: zq.zq_dequant_reduce(
        cc, ss, n1, B, 1.0, rq_codes=rqc, rq_scales=rqs), 10) / 1e6
    res["dr8"] = dr_bytes(n1, B, 8) / timed(torch, lambda: zq.zq_dequant_reduce(
        cc, ss, n1, B, 0.125, out=out), 10) / 1e6
    n2 = n1 // 4
    c2 = [rqc[j * n2 // 2:(j + 1) * n2 // 2] for j in range(4)]
    s2 = [rqs[j * n2 // B:(j + 1) * n2 // B] for j in range(4)]
    res["dr4"] = dr_bytes(n2, B, 4) / timed(torch, lambda: zq.zq_dequant_reduce(
        c2, s2, n2, B, 1 / 32, out=out), 10) / 1e6
    c3 = torch.empty(n, device=dev)
    res["torch_copy"] = 8 * n / timed(torch, lambda: c3.copy_(g), 10) / 1e6
    res["torch_add"] = 12 * n / timed(torch, lambda: torch.add(g, ef, out=c3), 10) / 1e6
    res["torch_sum"] = 4 * n / timed(torch, lambda: g.sum(), 10) / 1e6
    res["torch_fill"] = 4 * n / timed(torch, lambda: c3.fill_(1.0), 10) / 1e6
    del g, ef, c, s, cc, ss, rqc, rqs, out, c2, s2, c3
    torch.cuda.empty_cache()
    w = torch.randn(n, device=dev).mul_(0.02).to(torch.bfloat16)
    c8 = torch.empty(n, dtype=torch.int8, device=dev)
    s8 = torch.empty(n // 2048, device=dev)
    wd = torch.empty(n, dtype=torch.bfloat16, device=dev)
    res["q8"] = (3 * n + 4 * n / 2048) / timed(torch, lambda: zq.zq_quant_int8(w, 2048, c8, s8), 10) / 1e6
    res["dq8"] = (3 * n + 4 * n / 2048) / timed(torch, lambda: zq.zq_dequant_int8(c8, s8, 2048, wd), 10) / 1e6
    src = torch.randn(n, device=dev).mul_(1e-4).to(torch.bfloat16)
    res["sr"] = 6 * n / timed(torch, lambda: zq.zq_sr_accumulate(wd, src, 1, 0), 10) / 1e6
    res["sr_zero"] = 8 * n / timed(torch, lambda: zq.zq_sr_accumulate(wd, src, 1, 0, zero_src=True), 10) / 1e6
    lib = os.path.basename(os.environ.get("ZQ_LIB", "libzq.so"))
    print(f"{lib}  GB/s: " + "  ".join(f"{k} {v:.0f}" for k, v in res.items()), flush=True)


def warm_up(torch, fn, warm=2, min_ms=40.0):
    """At least `warm` calls and, for calls of 50 us or more, about `min_ms`
    of GPU time of the same call before timing: after other work the GPU's
    clocks take tens of ms to settle, and a short burst of ms-long kernels
    timed at once can read 10-20 % slow.  Launch-bound calls keep the short
    warm-up (their bursts are timed as they come)."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    fn()
    b.record()
    torch.cuda.synchronize()
    est = a.elapsed_time(b)
    if est >= 0.05:
        for _ in range(min(400, int(min_ms / est))):
            fn()
    torch.cuda.synchronize()


def timed_burst(torch, fn, reps, warm=2):
    """Average ms per call over `reps` back-to-back calls between two events
    (host enqueue time hides behind the GPU when the GPU is the slower)."""
    warm_up(torch, fn, warm)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def host_enqueue_ms(torch, fn, reps=5):
    """Host time of one call (argument validation and launches, until the
    call returns), median over `reps` calls each started on an idle GPU."""
    import numpy as np
    ts = []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        fn()
        ts.append((time.perf_counter() - t0) * 1e3)
    torch.cuda.synchronize()
    return float(np.median(ts))


def timed(torch, fn, reps, warm=2):
    warm_up(torch, fn, warm)
    evs = []
    for _ in range(reps):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    import numpy as np
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def timed_cold(torch, fn, reps, flush):
    """Median ms of `fn` when each call follows a write of `flush` (>= 1 GiB),
    which evicts the 4 MB L2s and the 256 MB MALL: the HBM-cold time."""
    evs = []
    for _ in range(reps):
        flush.fill_(1.0)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    import numpy as np
    return float(np.median([a.elapsed_time(b) for a, b in evs]))


def cold_fields(nbytes, ms):
    return {"cold_ms": round(ms, 4), "cold_GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1)}


def extra_rows(torch, zq, synth, dev, log, cpu=True):
    """The other rows of the path, each on its own workload; with cpu, each
    row also carries the oracle timed on a bounded sample of it."""
    import ctypes as C
    rows = {}
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
    # qwZ: bf16 weights of the ~0.85B model, block 2048
    t3 = synth.llama_0p85b()
    n = synth.total(t3)
    w = torch.empty(n, dtype=torch.bfloat16, device=dev)
    synth.fill_model(w, t3, std=0.02, seed=synth.seed_for("llama0p85b", "weights"))
    c8 = torch.empty(n, dtype=torch.int8, device=dev)
    s8 = torch.empty(zq.num_blocks(n, 2048), dtype=torch.float32, device=dev)
    wd = torch.empty(n, dtype=torch.bfloat16, device=dev)
    ms = timed_burst(torch, lambda: zq.zq_quant_int8(w, 2048, c8, s8), 20)
    rows["quant_int8_bf16_b2048_0.85B"] = row(n * 3 + 4 * s8.numel(), ms, n)
    ms = timed_burst(torch, lambda: zq.zq_dequant_int8(c8, s8, 2048, wd), 20)
    rows["dequant_int8_bf16_b2048_0.85B"] = row(n * 3 + 4 * s8.numel(), ms, n)
    log("int8 rows", rows["quant_int8_bf16_b2048_0.85B"], rows["dequant_int8_bf16_b2048_0.85B"])
    # the same with the pages' fp16 weights (qwZ: fp16 -> int8 -> fp16)
    wh = torch.empty(n, dtype=torch.float16, device=dev)
    wh.copy_(w)
    ms = timed_burst(torch, lambda: zq.zq_quant_int8(wh, 2048, c8, s8), 20)
    rows["quant_int8_fp16_b2048_0.85B"] = row(n * 3 + 4 * s8.numel(), ms, n)
    ms = timed_burst(torch, lambda: zq.zq_dequant_int8(c8, s8, 2048, wh), 20)
    rows["dequant_int8_fp16_b2048_0.85B"] = row(n * 3 + 4 * s8.numel(), ms, n)
    del wh
    if cpu:
        S = 1 << 27
        wh = to_host_np(w[:S])
        rows["quant_int8_bf16_b2048_0.85B"]["cpu_baseline"] = cpu_row(
            lambda: oracle_q8(wh), 2 * (3 * S + 4 * S / 2048),
            f"first {S} weights: int8 quantize then dequantize (bytes of both)", split_of=("q8", "dq8"))
    del w, c8, s8, wd

    # qgZ + LoCo on the ~0.85B fp32 gradient: EF quantize B=128 + 8-way reduce
    gq = torch.empty(n, dtype=torch.float32, device=dev)
    synth.fill_model(gq, t3, std=1e-3, seed=synth.seed_for("llama0p85b", "grad"), heavy_tails=True)
    efq_ = torch.zeros(n, dtype=torch.float32, device=dev)
    cq = torch.empty(n // 2, dtype=torch.uint8, device=dev)
    sq = torch.empty(n // 128, dtype=torch.float32, device=dev)
    outq = torch.empty(n // 8, dtype=torch.float32, device=dev)
    ms = timed_burst(torch, lambda: zq.zq_quantize_ef_int4(gq, efq_, 128, 0.9, 1.0, cq, sq), 10)
    rows["efq_fp32_b128_0.85B"] = row(efq_bytes(n, 128, 4), ms, n)
    nc = n // 8
    cc = [cq[j * nc // 2:(j + 1) * nc // 2] for j in range(8)]
    ss = [sq[j * nc // 128:(j + 1) * nc // 128] for j in range(8)]
    ms = timed_burst(torch, lambda: zq.zq_dequant_reduce(cc, ss, nc, 128, 0.125, out=outq), 20)
    rows["dequant_reduce_p8_b128_0.85B"] = row(dr_bytes(nc, 128, 8), ms, nc)
    log("0.85B qgZ rows", rows["efq_fp32_b128_0.85B"], rows["dequant_reduce_p8_b128_0.85B"])
    if cpu:
        S = 1 << 28
        gh = to_host_np(gq[:S])
        rows["efq_fp32_b128_0.85B"]["cpu_baseline"] = cpu_row(
            lambda: oracle_c4(gh), efq_bytes(S, 128, 4) + dr_bytes(S // 8, 128, 8),
            f"first {S} gradient elements: EF quantize + 8-way reduce of its {S // 8}-element "
            "chunks (alpha 1/8)", split_of=("efq", "dr"))
    del gq, efq_, cq, sq, outq, cc, ss

    # llm.c ZeRO-2: SR accumulation of GPT-2 124M bf16 grads, full buffer and rank-3 shard
    t2 = synth.gpt2_124m()
    n = synth.total(t2)
    dst = torch.zeros(n, dtype=torch.bfloat16, device=dev)
    src = torch.empty(n, dtype=torch.bfloat16, device=dev)
    synth.fill_model(src, t2, std=1e-4, seed=synth.seed_for("gpt2", "grad", mb=0))
    ms = timed_burst(torch, lambda: zq.zq_sr_accumulate(dst, src, 0, 0), 20)
    rows["sr_accumulate_bf16_gpt2_124M_full"] = row(6 * n, ms, n)
    shard = n // 8
    off = 3 * shard
    dsh = torch.zeros(shard, dtype=torch.bfloat16, device=dev)
    ssh = src[off:off + shard]
    st = torch.cuda.current_stream().cuda_stream
    dp, sp = dsh.data_ptr(), ssh.data_ptr()
    ms = timed_burst(torch, lambda: zq.lib.zq_sr_accumulate(dp, sp, shard, 0, off, 0, st), 200)
    ms_c = timed_cold(torch, lambda: zq.lib.zq_sr_accumulate(dp, sp, shard, 0, off, 0, st), 20, flush)
    rows["sr_accumulate_bf16_gpt2_rank3_shard"] = dict(
        row(6 * shard, ms, shard), **cold_fields(6 * shard, ms_c),
        note="93 MB: back-to-back calls run cache-resident; cold_* follow a 1 GiB write")
    log("SR rows", rows["sr_accumulate_bf16_gpt2_124M_full"])
    if cpu:
        S = 1 << 25
        sh = to_host_np(src[:S])
        rows["sr_accumulate_bf16_gpt2_124M_full"]["cpu_baseline"] = cpu_row(
            lambda: oracle_sr(sh), 6 * S, f"first {S} elements of one micro-batch")
    del dst, src, dsh, ssh

    # llm.c's per-tensor ZeRO-2 loop for rank 3 of 8 over GPT-2's 148 tensors:
    # SR-add each tensor's shard slice and clear each whole reduced buffer --
    # one batched call against 148 single calls + 148 zero fills.
    grads = torch.empty(n, dtype=torch.bfloat16, device=dev)
    synth.fill_model(grads, t2, std=1e-4, seed=synth.seed_for("gpt2", "grad", mb=0))
    shards = torch.zeros(n // 8, dtype=torch.bfloat16, device=dev)
    segs, off, soff = [], 0, 0
    for i, t in enumerate(t2):
        m = t.numel // 8
        segs.append((shards[soff:soff + m], grads[off:off + t.numel], m, 3 * m, i, off + 3 * m))
        off += t.numel
        soff += m
    nbytes = sum(6 * m + 2 * src.numel() for _, src, m, _, _, _ in segs)
    table = zq.SrSegmentTable(segs)
    ms_b = timed_burst(torch, lambda: zq.zq_sr_accumulate_batched(table, zero_src=True), 50)
    ms_bc = timed_cold(torch, lambda: zq.zq_sr_accumulate_batched(table, zero_src=True), 20, flush)

    def loop():
        for d_, s_, m_, o_, sd_, cb_ in segs:
            zq.zq_sr_accumulate(d_, s_[o_:o_ + m_], sd_, cb_)
            s_.zero_()
    ms_l = timed_burst(torch, loop, 5)
    # the same loop recorded once in a HIP graph and replayed: 296 kernel
    # nodes, no host work per call
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        loop()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        loop()
    ms_g = timed_burst(torch, graph.replay, 20)
    del graph
    rows["sr_accumulate_batched_gpt2_148_tensors_rank3"] = dict(
        row(nbytes, ms_b, n // 8), **cold_fields(nbytes, ms_bc),
        note=f"one call for 148 tensors incl. clearing the reduced buffers (marshalled table, "
             f"back-to-back calls); the same work as a Python loop of 148 single calls + 148 "
             f"torch zero_() takes {ms_l:.3f} ms, host overhead included, and {ms_g:.3f} ms "
             f"replayed from a HIP graph",
        python_loop_ms=round(ms_l, 4), graph_loop_ms=round(ms_g, 4))
    log("batched SR", rows["sr_accumulate_batched_gpt2_148_tensors_rank3"])
    del grads, shards, segs

    # 4 simulated ranks, bf16 2^20 each, block 256 (cache-resident, launch-bound)
    n = 4 << 20
    g4 = synth.grad_with_outliers(n, 1e-3, 0.01, 50.0, synth.seed_for("c1", "grad"),
                                  torch.bfloat16, device=dev)
    e4 = torch.zeros(n, dtype=torch.float32, device=dev)
    c4 = torch.empty(n // 2, dtype=torch.uint8, device=dev)
    s4 = torch.empty(n // 256, dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream().cuda_stream
    a4 = (g4.data_ptr(), e4.data_ptr(), c4.data_ptr(), s4.data_ptr())
    ms = timed_burst(torch, lambda: zq.lib.zq_quantize_ef_int4(a4[0], 1, a4[1], n, 256, 1.0, 1.0,
                                                               a4[2], a4[3], st), 200)
    ms_c = timed_cold(torch, lambda: zq.lib.zq_quantize_ef_int4(a4[0], 1, a4[1], n, 256, 1.0, 1.0,
                                                                 a4[2], a4[3], st), 20, flush)
    rows["efq_bf16_b256_4x2^20"] = dict(
        row(efq_bytes(n, 256, 2), ms, n), **cold_fields(efq_bytes(n, 256, 2), ms_c),
        note="44 MB: back-to-back calls run cache-resident and launch-bound; cold_* follow a "
             "1 GiB write")
    # ... and destination rank 0's 4-way reduce of chunk 0 of every rank (alpha 1/4)
    nc, rank_n = n // 16, n // 4  # 2^18 elements per chunk, 2^20 per rank
    out4 = torch.empty(nc, dtype=torch.float32, device=dev)
    cp4 = (C.c_void_p * 4)(*[c4.data_ptr() + r * rank_n // 2 for r in range(4)])
    sp4 = (C.c_void_p * 4)(*[s4.data_ptr() + 4 * (r * rank_n // 256) for r in range(4)])
    op4 = out4.data_ptr()
    dr4 = lambda: zq.lib.zq_dequant_reduce(4, cp4, sp4, nc, 256, 0.25, op4, None, None, None, 0.0,
                                           1.0, st)
    ms = timed_burst(torch, dr4, 200)
    ms_c = timed_cold(torch, dr4, 20, flush)
    rows["dequant_reduce_p4_b256_4x2^18"] = dict(
        row(dr_bytes(nc, 256, 4), ms, nc), **cold_fields(dr_bytes(nc, 256, 4), ms_c),
        note="2.2 MB: launch-bound; cold_* follow a 1 GiB write")
    log("4-rank rows", rows["efq_bf16_b256_4x2^20"], rows["dequant_reduce_p4_b256_4x2^18"])
    if cpu:
        g4h = to_host_np(g4)
        rows["efq_bf16_b256_4x2^20"]["cpu_baseline"] = cpu_row(
            lambda: oracle_c1(g4h), efq_bytes(n, 256, 2) + dr_bytes(nc, 256, 4),
            "the whole workload: EF quantize of the 4 ranks' 2^20 bf16 elements + the 4-way "
            "reduce of chunk 0", split_of=("efq", "dr"))
    del flush, out4
    torch.cuda.empty_cache()
    return rows


if __name__ == "__main__":
    main()
