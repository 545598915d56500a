"""Strength of the oracle's pins: each case plants one plausible mistake in a copy
of oracle/oracle.c (a dropped term, a wrong sign, exponent or index, swapped
operands, a wrong tie rule), builds the copy, and runs the pin tests against it
in a child process; the pins must fail on every one of them.  The unmodified
copy runs first and must pass, which shows the harness itself works.

CPU only: nothing here touches the GPU library."""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c (must occur exactly once), replacement)
MUTATIONS = [
    ("bf16 decode shift", "uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)b << 15;"),
    ("fp16 subnormal exponent", "ldexp((double)mt, -24)", "ldexp((double)mt, -25)"),
    ("fp16 normal exponent", "ex - 25);", "ex - 24);"),
    ("bf16 rounding ties away from even",
     "if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;", "if (rem >= 0.5) fl += 1.0;"),
    ("bf16 rounding truncates", "if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;", ""),
    ("bf16 keeps 9 bits", "ldexp(1.0, ue - 7)", "ldexp(1.0, ue - 8)"),
    ("nibble order swapped",
     "uint8_t byte = codes[c / 2];\n        int q = (c % 2 == 0) ? (byte & 0x0F) : (byte >> 4);",
     "uint8_t byte = codes[c / 2];\n        int q = (c % 2 == 1) ? (byte & 0x0F) : (byte >> 4);"),
    ("scale and min fields swapped",
     "double scale = oracle_fp16_to_double((uint16_t)(rec[0] | (rec[1] << 8)));\n"
     "        double mn = oracle_fp16_to_double((uint16_t)(rec[2] | (rec[3] << 8)));",
     "double scale = oracle_fp16_to_double((uint16_t)(rec[2] | (rec[3] << 8)));\n"
     "        double mn = oracle_fp16_to_double((uint16_t)(rec[0] | (rec[1] << 8)));"),
    ("min subtracted", "out[c] = scale * (double)q + mn;", "out[c] = scale * (double)q - mn;"),
    ("min dropped", "out[c] = scale * (double)q + mn;", "out[c] = scale * (double)q;"),
    ("record per 16 columns", "const uint8_t *rec = params + (c / 32) * 4;", "const uint8_t *rec = params + (c / 16) * 4;"),
    ("W1 and W3 rows swapped", "(which == 1 ? gate_row : 0)", "(which == 0 ? gate_row : 0)"),
    ("W2 base misplaced", "return slab + I * 2 * gate_row + r * down_row;", "return slab + I * gate_row + r * down_row;"),
    ("row padding dropped", "(cols / 2 + (cols / 32) * 4 + 15) / 16 * 16", "(cols / 2 + (cols / 32) * 4)"),
    ("gate and up swapped in SwiGLU", "h[r] = g[r] / (1.0 + exp(-g[r])) * u[r];",
     "h[r] = u[r] / (1.0 + exp(-u[r])) * g[r];"),
    ("sigmoid sign", "h[r] = g[r] / (1.0 + exp(-g[r])) * u[r];", "h[r] = g[r] / (1.0 + exp(g[r])) * u[r];"),
    ("SwiGLU without the gate's factor", "h[r] = g[r] / (1.0 + exp(-g[r])) * u[r];",
     "h[r] = 1.0 / (1.0 + exp(-g[r])) * u[r];"),
    ("down projection reads h transposed",
     "for (int64_t c = 0; c < I; ++c) acc += row[c] * h[c];\n        y[r] = acc;\n    }\n    free(row);\n    if (!g_out)",
     "for (int64_t c = 0; c < I; ++c) acc += row[c] * h[I - 1 - c];\n        y[r] = acc;\n    }\n    free(row);\n"
     "    if (!g_out)"),
    ("router bias dropped", "if (bias) acc += (double)bias[e];", "if (0) acc += (double)bias[e];"),
    ("router logits rounded per term",
     "for (int64_t h = 0; h < H; ++h) acc += oracle_bf16_to_double(x[h]) * (double)Wr[e * H + h];",
     "for (int64_t h = 0; h < H; ++h) acc = (float)(acc + (float)(oracle_bf16_to_double(x[h]) * (double)Wr[e * H + h]));"),
    ("top-k ties go to the higher index", "logits[e] > logits[best]", "logits[e] >= logits[best]"),
    ("softmax not normalised", "for (int i = 0; i < k; ++i) w[i] /= sum;", ""),
    ("softmax at temperature 1/2", "w[i] = exp((double)logits[idx[i]] - top);",
     "w[i] = exp(2.0 * ((double)logits[idx[i]] - top));"),
    ("combine slots reversed", "acc += w[t * k + i] * y[(j * per + i) * H + h];",
     "acc += w[t * k + (k - 1 - i)] * y[(j * per + i) * H + h];"),
    ("shared expert dropped", "if (shared) acc += y[(j * per + k) * H + h];", ""),
    ("shared expert halved", "if (shared) acc += y[(j * per + k) * H + h];",
     "if (shared) acc += 0.5 * y[(j * per + k) * H + h];"),
    ("rows subset reads the wrong token", "xd[h] = oracle_bf16_to_double(x[t * H + h]);",
     "xd[h] = oracle_bf16_to_double(x[j * H + h]);"),
    ("E2M1 exponent bias", "ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.5 * m, e)"),
    ("E2M1 subnormal step", "e == 0 ? 0.5 * m :", "e == 0 ? 1.0 * m :"),
    ("E8M0 bias", "ldexp(1.0, (int)v - 127)", "ldexp(1.0, (int)v - 128)"),
    ("MX scale per 16 columns", "oracle_e8m0_to_double(row[cols / 2 + c / 32])",
     "oracle_e8m0_to_double(row[cols / 2 + c / 16])"),
    ("super-block min added", "- dmin * field6(h + 10, j);", "+ dmin * field6(h + 10, j);"),
    ("super-block 6-bit fields misaligned", "return (unsigned)((v >> (6 * j)) & 63);",
     "return (unsigned)((v >> (6 * j + 1)) & 63);"),
    ("super-block scale and min fields swapped", "out[c] = d * field6(h + 4, j) * q - dmin * field6(h + 10, j);",
     "out[c] = d * field6(h + 10, j) * q - dmin * field6(h + 4, j);"),
    ("super-block sub-block of 16 columns", "const int j = (int)((c / 32) % 8);",
     "const int j = (int)((c / 16) % 8);"),
    ("residual norm over H-1", "sqrt(ss / (double)H + eps)", "sqrt(ss / (double)(H - 1) + eps)"),
    ("residual subtracted", "r[h] = (float)((double)r[h] + oracle_bf16_to_double(add[t * H + h]));",
     "r[h] = (float)((double)r[h] - oracle_bf16_to_double(add[t * H + h]));"),
    ("residual eps dropped", "sqrt(ss / (double)H + eps)", "sqrt(ss / (double)H)"),
]


def _build(src_text: str, out: str):
    c = out[:-3] + ".c"
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
                           "-w", "-o", out, c, "-lm"])


def _run_pins(lib: str):
    env = dict(os.environ, MOE_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    p = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"), "-x",
                        "-q", "-p", "no:cacheprovider", "-m", "not gpu"], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    return p.returncode, (p.stdout + p.stderr)[-2000:]


def _mutant(args):
    i, name, old, new, tmp, text = args
    lib = os.path.join(tmp, f"mutant_{i}.so")
    _build(text.replace(old, new), lib)
    rc, tail = _run_pins(lib)
    return name, rc, tail


def test_every_planted_mistake_fails_a_pin():
    text = open(SRC).read()
    for name, old, new in MUTATIONS:
        assert text.count(old) == 1, f"mutation {name!r}: its text occurs {text.count(old)} times in oracle.c"
    with tempfile.TemporaryDirectory() as tmp:
        clean = os.path.join(tmp, "clean.so")
        _build(text, clean)
        rc, tail = _run_pins(clean)
        assert rc == 0, f"the unmodified oracle fails its pins under the harness:\n{tail}"
        jobs = [(i, name, old, new, tmp, text) for i, (name, old, new) in enumerate(MUTATIONS)]
        with cf.ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(_mutant, jobs))
    survivors = [(name, rc, tail) for name, rc, tail in results if rc != 1]
    assert not survivors, "planted mistakes the pins do not catch (or that crash the pins):\n" + "\n".join(
        f"--- {name} (pytest rc {rc})\n{tail}" for name, rc, tail in survivors)
