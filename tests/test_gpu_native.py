"""A native C program uses libzq the way a C caller would: its own
hipMalloc'd buffers and hipStream, no Python in between
(tests/native/zq_c_step.c).  It runs EF int4 quantize, the 4-way reduce
with requant, qwZ int8 quantize / dequantize and SR accumulate on inputs
written here, and checks that a misaligned call is refused; every output
must equal the oracle's bit for bit."""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import oracle as O
from tests.gpu_helpers import assert_bits_equal, grad_values

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NC, NW, NS, B = 40064, 10277, 5003, 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    # device_count() does not initialise the GPU in this process: the C
    # program, a child process, is the only user of the GPU here
    if torch.cuda.device_count() == 0:
        pytest.skip("no GPU")
    yield


def bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_c_program_matches_the_oracle(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    lib_dir = os.path.join(ROOT, "weight_communication_zero_amd")
    exe = tmp_path / "zq_c_step"
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                        "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "native", "zq_c_step.c"),
                        os.path.join(lib_dir, "libzq.so"), "-L/opt/rocm/lib", "-lamdhip64",
                        "-Wl,-rpath," + lib_dir, "-Wl,-rpath,/opt/rocm/lib", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    rng = np.random.default_rng(8)
    n = 4 * NC
    g = grad_values(n, seed=81, std=1e-3)
    ef = grad_values(n, seed=82, std=1e-5)
    w = bf16_bits(rng.standard_normal(NW) * 0.02)
    dst = bf16_bits(rng.standard_normal(NS) * 1e-2)
    src = bf16_bits(rng.standard_normal(NS) * 1e-4)
    for name, a in (("g", g), ("ef", ef), ("w", w), ("dst", dst), ("src", src)):
        a.tofile(tmp_path / f"{name}.bin")
    print(f"running {exe}", flush=True)
    r = subprocess.run([str(exe), str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    got = lambda name, dt: np.fromfile(tmp_path / f"{name}.out", dtype=dt)

    ef_o = ef.copy()
    c_o, s_o = O.quantize_ef_int4(g, ef_o, B, 0.9, 1.0)
    assert_bits_equal(got("codes", np.uint8), c_o, "C caller: codes")
    assert_bits_equal(got("scales", np.float32), s_o, "C caller: scales")
    assert_bits_equal(got("ef", np.float32), ef_o, "C caller: EF")
    out_o, rqc_o, rqs_o = O.dequant_reduce([c_o[j * NC // 2:(j + 1) * NC // 2] for j in range(4)],
                                           [s_o[j * NC // B:(j + 1) * NC // B] for j in range(4)],
                                           NC, B, 0.25, want_out=True, requant=True)
    assert_bits_equal(got("red", np.float32), out_o, "C caller: reduced sums")
    assert_bits_equal(got("rqc", np.uint8), rqc_o, "C caller: requant codes")
    assert_bits_equal(got("rqs", np.float32), rqs_o, "C caller: requant scales")
    c8_o, s8_o = O.quant_int8(w, 2048)
    assert_bits_equal(got("c8", np.int8).view(np.uint8), c8_o.view(np.uint8), "C caller: int8 codes")
    assert_bits_equal(got("s8", np.float32), s8_o, "C caller: int8 scales")
    assert_bits_equal(got("wd", np.uint16), O.dequant_int8(c8_o, s8_o, 2048, out_bf16=True),
                      "C caller: dequantized weights")
    d_o = dst.copy()
    O.sr_accumulate(d_o, src.copy(), seed=77, counter_base=5)
    assert_bits_equal(got("dst", np.uint16), d_o, "C caller: SR accumulate")
