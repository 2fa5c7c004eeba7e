"""Host-side logic that needs no GPU: the build entry point, the benchmark's
HBM-traffic lookup (valid only while the kernel source is unchanged since the
counters were taken), the build's refusal of kernels that use scratch memory,
and the pages' context figures in the benchmark line."""
import os
import re
import shutil
import subprocess
import sys

import bench
from weight_communication_zero_amd import zq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _load_build():
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "zq_build_for_test", os.path.join(ROOT, "weight_communication_zero_amd", "_build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_build_scripts_load_without_the_package():
    """build() must work on a fresh checkout, where libzq.so does not exist
    yet: it loads the build scripts by path, never through the package
    (whose import loads libzq.so)."""
    code = ("import sys, os; sys.path.insert(0, os.getcwd()); import __graft_entry__ as g; "
            "m = g._load_by_path('zq_build_check', os.path.join('weight_communication_zero_amd', '_build.py')); "
            "o = g._load_by_path('zq_oracle_build_check', os.path.join('oracle', 'build.py')); "
            "assert 'weight_communication_zero_amd' not in sys.modules; "
            "assert m.LIB.endswith('libzq.so') and o.LIB.endswith('libzq_oracle.so'); "
            "assert any(s.endswith('zq_dr.hip') for s in m.sources())")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_traffic_is_read_only_for_the_profiled_source(tmp_path, monkeypatch):
    tag = "efq_fp32_b128"
    alg = 7547949056 * 12.5 + 7547949056 // 128 * 4
    recorded = bench.measured_traffic(tag, alg)
    assert recorded is not None, "the committed counter summary no longer matches the kernel source"
    assert abs(recorded / alg - 1) < 1e-3  # the profile found no re-reads
    # A copy of the tree whose kernel source differs by one byte: no traffic.
    fake = tmp_path / "repo"
    shutil.copytree(os.path.join(ROOT, "profiles"), fake / "profiles")
    shutil.copytree(os.path.join(ROOT, "weight_communication_zero_amd", "csrc"),
                    fake / "weight_communication_zero_amd" / "csrc")
    src = fake / "weight_communication_zero_amd" / "csrc" / "zq_efq.hip"
    src.write_text(src.read_text() + "\n")
    monkeypatch.setattr(bench, "ROOT", str(fake))
    assert bench.measured_traffic(tag, alg) is None


def test_traffic_summary_records_hash_and_bytes():
    for tag in bench.KERNEL_SOURCES:
        text = open(os.path.join(ROOT, "profiles", f"{tag}_counters.md")).read()
        assert re.search(r"source_sha256[^:\n]*:\s*[0-9a-f]{64}", text), tag
        assert re.search(r"hbm_bytes_per_launch:\s*[0-9]+", text), tag


def test_reduce_traffic_is_current_and_near_algorithmic():
    n1 = 7547949056 // 8
    alg = 8 * (n1 // 2 + 4 * (n1 // 128)) + n1 // 2 + 4 * (n1 // 128)
    got = bench.measured_traffic("dequant_reduce_requant_p8_b128_7.5B", alg)
    assert got is not None, "the reduce's counter summary no longer matches its source"
    assert 1.0 <= got / alg < 1.1


def test_pages_context_counts_bytes_with_the_library_helpers():
    M = 7547949056
    ctx = bench.pages_context(zq, M)
    v = ctx["comm_bytes_per_step_7.5B"]
    assert v["zero3"] == 6 * M
    # int8 weights + fp32 scales per 2048, int4 gradients + fp32 scales per 128
    assert v["zeropp_int8_w2048_int4_g128"] == M + 4 * (M // 2048) + M // 2 + 4 * (M // 128)
    # the pages' 4x is the limit without scales; with them it is a bit less
    assert 3.9 < v["ratio"] < 4.0


def test_build_refuses_kernels_that_use_scratch():
    """The build parses the compiler's resource-usage remarks and names
    every kernel with a nonzero scratch size."""
    b = _load_build()
    remarks = "\n".join([
        "x.h:1:1: remark: Function Name: kern_a [-Rpass-analysis=kernel-resource-usage]",
        "x.h:1:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]",
        "x.h:1:1: remark: Function Name: kern_b [-Rpass-analysis=kernel-resource-usage]",
        "x.h:1:1: remark:     ScratchSize [bytes/lane]: 204 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert b.scratch_users(remarks) == [("kern_b", 204)]
    assert b.scratch_users("") == []


def test_requant_scale_division_is_exact_for_every_float(tmp_path):
    """The reduce's requant computes its block scale fl(absmax / 7) as
    q0 = a fl(1/7), e = fma(-q0, 7, a), q1 = fma(e, fl(1/7), q0): the same
    bits as the IEEE division for every non-negative finite float, checked
    exhaustively (2^31 values, split over the host's cores)."""
    exe = str(tmp_path / "div_by_const")
    r = subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-o", exe,
                        os.path.join(ROOT, "tests", "arith", "div_by_const.c"), "-lm"],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe, "7"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and "0 mismatches" in r.stdout, r.stdout
