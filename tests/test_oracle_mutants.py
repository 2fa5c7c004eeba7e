"""Planted mistakes in the oracle: the pins must catch each one.

Every case below turns one line of ``oracle/zq_oracle.c`` into a plausible
slip -- a dropped term, a wrong sign, index, constant or rounding, a swapped
operand -- builds that copy with the oracle's own compiler flags and runs the
pin suite (``tests/test_oracle_pins.py``) against it through
``ZQ_ORACLE_LIB``.  Every copy must fail at least one pin, and the unchanged
source built the same way must pass them all.  CPU only; the copies live in a
temporary directory and nothing here touches the GPU library.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "zq_oracle.c")
sys.path.insert(0, ROOT)
from oracle import build as oracle_build  # noqa: E402

# (name, exact text in zq_oracle.c, replacement)
MUTANTS = [
    ("EF update drops the beta_e term", "ef[i] = t1 + t2;", "ef[i] = t2;"),
    ("EF update swaps the coefficients", "float t1 = beta_e * ef[i];", "float t1 = beta_r * ef[i];"),
    ("residual sign", "float r = c[j] - d;", "float r = d - c[j];"),
    ("EF compensation drops e", "c[j] = ef ? gi + ef[i] : gi;", "c[j] = gi;"),
    ("int4 qmax 8", "orc_quant_block(c, m, 7, k, &s);", "orc_quant_block(c, m, 8, k, &s);"),
    ("int8 qmax 128", "orc_quant_block(x, m, 127, k, &scales[b]);",
     "orc_quant_block(x, m, 128, k, &scales[b]);"),
    ("scale by reciprocal multiply", "float s = a / (float)qmax;", "float s = a * (1.0f / (float)qmax);"),
    ("signed maximum instead of absmax", "float v = fabsf(x[i]);", "float v = x[i];"),
    ("ties away from zero", "float r = rintf(q); /*", "float r = roundf(q); /*"),
    ("upper clamp dropped", "r = fminf(r, (float)qmax);", ""),
    ("lower clamp dropped", "r = fmaxf(r, -(float)qmax);", ""),
    ("nibble order swapped", "if ((i & 1u) == 0)\n        codes[i / 2]", "if ((i & 1u) == 1)\n        codes[i / 2]"),
    ("nibble sign extension off by one", "(int32_t)nib - 16", "(int32_t)nib - 15"),
    ("odd tail's high nibble not cleared", "codes[(lo + m) / 2] &= 0x0Fu;", ";"),
    ("reduce skips the second peer", "for (uint32_t p = 1; p < P; p++)", "for (uint32_t p = 2; p < P; p++)"),
    ("reduce scale index off by one", "size_t b = i / block;", "size_t b = (i + 1) / block;"),
    ("reduce drops alpha", "float R = alpha * S;", "float R = S;"),
    ("int8 dequant scale index off by one", "scales[i / block];", "scales[(i + 1) / block];"),
    ("bf16 rounding ties away", "u += 0x7FFFu + keep_lsb;", "u += 0x8000u;"),
    ("int8 dequant truncates to bf16", "((uint16_t *)out)[i] = orc_bf16_rne(v);",
     "((uint16_t *)out)[i] = (uint16_t)(f32_bits(v) >> 16);"),
    ("fp16 widening exponent bias", "ldexpf((float)(f | 0x400u), (int)e - 25)",
     "ldexpf((float)(f | 0x400u), (int)e - 24)"),
    ("fp16 subnormals widened with the implicit bit", "v = ldexpf((float)f, -24);",
     "v = ldexpf((float)(f | 0x400u), -24);"),
    ("fp16 rounding truncates", "uint32_t q = (uint32_t)rintf(ldexpf(a, 10 - E));",
     "uint32_t q = (uint32_t)truncf(ldexpf(a, 10 - E));"),
    ("fp16 rounding ties away", "uint32_t q = (uint32_t)rintf(ldexpf(a, 10 - E));",
     "uint32_t q = (uint32_t)roundf(ldexpf(a, 10 - E));"),
    ("fp16 overflow at the largest finite", "if (a >= 65520.0f)", "if (a > 65504.0f)"),
    ("fp16 subnormal range one binade short", "if (a < 0x1p-14f)", "if (a < 0x1p-15f)"),
    ("fp16 normal results lose the sign",
     "return (uint16_t)(sign | ((((uint32_t)(E + 15)) << 10) + (q - 1024u)));",
     "return (uint16_t)((((uint32_t)(E + 15)) << 10) + (q - 1024u));"),
    ("int8 dequant fp16 output rounded as bf16", "((uint16_t *)out)[i] = orc_f16_rne(v);",
     "((uint16_t *)out)[i] = orc_bf16_rne(v);"),
    ("fp16 input read as bf16", "return f16_to_f32(((const uint16_t *)p)[i]);",
     "return bf16_to_f32(((const uint16_t *)p)[i]);"),
    ("Philox key schedule", "k1 += PHILOX_W1;", "k1 += PHILOX_W0;"),
    ("Philox multipliers swapped", "uint64_t p0 = (uint64_t)PHILOX_M0 * (uint64_t)x0;",
     "uint64_t p0 = (uint64_t)PHILOX_M1 * (uint64_t)x0;"),
    ("Philox output words swapped", "uint32_t y1 = lo1;", "uint32_t y1 = lo0;"),
    ("counter high word dropped", "uint32_t ctr[4] = {(uint32_t)c, (uint32_t)(c >> 32), 0u, 0u};",
     "uint32_t ctr[4] = {(uint32_t)c, 0u, 0u, 0u};"),
    ("r16 halves swapped", "return (q & 1u) ? (word >> 16) : (word & 0xFFFFu);",
     "return (q & 1u) ? (word & 0xFFFFu) : (word >> 16);"),
    ("r16 word index", "uint32_t word = w[(q & 7u) >> 1];", "uint32_t word = w[q & 3u];"),
    ("SR adds 15 random bits", "u = u + (r16 & 0xFFFFu);", "u = u + (r16 & 0x7FFFu);"),
    ("SR keeps the source", "        if (zero_src)\n            src[i] = 0;", ""),
    ("volume counts int4 as a byte", "uint64_t qgz = (M + 1) / 2 +", "uint64_t qgz = M +"),
    ("volume drops the weight scales", "uint64_t qwz = M + 4u * ((M + block_w - 1) / block_w);",
     "uint64_t qwz = M;"),
    ("ZeRO++ slots: identity order", "slot_of_part[node * intra + local] = local * inter + node;",
     "slot_of_part[node * intra + local] = node * intra + local;"),
    ("ZeRO++ slots: inverse map", "slot_of_part[node * intra + local] = local * inter + node;",
     "slot_of_part[local * inter + node] = node * intra + local;"),
    ("permuted quantize: inverse slot map",
     "size_t from = p * part;\n        size_t to = slot_of_part[p] * part;",
     "size_t from = slot_of_part[p] * part;\n        size_t to = p * part;"),
    ("permuted quantize: EF buffer permuted too", "ef ? ef + from : NULL", "ef ? ef + to : NULL"),
    ("segments: only the slice read is cleared", "memset(src[i], 0, len[i] * sizeof(uint16_t));",
     "memset(src[i] + off[i], 0, n[i] * sizeof(uint16_t));"),
    ("segments: cleared before the add",
     "        if (n[i] > 0)\n            orc_sr_accumulate(dst[i], src[i] + off[i], n[i], seed[i], cbase[i], 0);\n"
     "        if (zero_src && len[i] > 0)\n            memset(src[i], 0, len[i] * sizeof(uint16_t));",
     "        if (zero_src && len[i] > 0)\n            memset(src[i], 0, len[i] * sizeof(uint16_t));\n"
     "        if (n[i] > 0)\n            orc_sr_accumulate(dst[i], src[i] + off[i], n[i], seed[i], cbase[i], 0);"),
    ("segments: counter base taken from the offset", "seed[i], cbase[i], 0);", "seed[i], cbase[i] + off[i], 0);"),
    ("segments: one seed for all", "n[i], seed[i], cbase[i], 0);", "n[i], seed[0], cbase[i], 0);"),
    ("reduce segments: scales stepped by the codes stride", "sp[p] = scales[i] + p * sstride[i];",
     "sp[p] = scales[i] + p * cstride[i];"),
    ("reduce segments: every peer reads peer 0", "cp[p] = codes[i] + p * cstride[i];",
     "cp[p] = codes[i];"),
    ("reduce segments: first segment's length for all", "int rc = orc_dequant_reduce(P, cp, sp, n[i], block,",
     "int rc = orc_dequant_reduce(P, cp, sp, n[0], block,"),
]


def _build_and_run(name: str, text: str, workdir: str) -> tuple[str, int, str]:
    src = os.path.join(workdir, "zq_oracle.c")
    lib = os.path.join(workdir, "libzq_oracle.so")
    with open(src, "w") as f:
        f.write(text)
    subprocess.run(["gcc", *oracle_build.CFLAGS, "-o", lib, src, "-lm"], check=True,
                   capture_output=True)
    env = dict(os.environ, ZQ_ORACLE_LIB=lib, PYTHONDONTWRITEBYTECODE="1", OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-2000:]


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with open(SRC) as f:
        original = f.read()
    jobs = [("unchanged", original)]
    for name, old, new in MUTANTS:
        assert original.count(old) == 1, f"mutation site not unique or missing: {name}"
        jobs.append((name, original.replace(old, new)))
    dirs = []
    for i in range(len(jobs)):
        d = tmp_path / f"m{i}"
        d.mkdir()
        dirs.append(str(d))
    workers = max(1, min(8, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        results = list(ex.map(lambda a: _build_and_run(*a), [(n, t, d) for (n, t), d in zip(jobs, dirs)]))
    control = results[0]
    assert control[1] == 0, f"the unchanged oracle failed its pins:\n{control[2]}"
    survivors = [name for name, rc, _ in results[1:] if rc == 0]
    errors = [(name, out) for name, rc, out in results[1:] if rc not in (0, 1)]
    assert not errors, f"pin runs that did not complete: {errors}"
    assert not survivors, f"planted mistakes no pin caught: {survivors}"


if __name__ == "__main__":
    sys.exit(pytest.main([__file__, "-q"]))
