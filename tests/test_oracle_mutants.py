"""The pins catch plausible mistakes in the oracle. Each case plants one
mistake in a copy of the oracle's C source (a dropped term, a wrong sign or
index, a swapped operand or nibble, a wrong constant or rounding rule),
builds it, and runs the pin suite against that build in a subprocess: at
least one pin must fail. The unmodified source, built the same way, must
pass them all (so a failure is the planted mistake's doing)."""
import concurrent.futures
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

MUTANTS = [
    ("product drops the block scale", "y += s * inner;", "y += inner;"),
    ("product subtracts", "inner += e * xv;", "inner -= e * xv;"),
    ("product reads activation row 0 for every row", "const uint16_t *xm = j->x ? j->x + m * K : NULL;",
     "const uint16_t *xm = j->x ? j->x : NULL;"),
    ("product decodes the odd k from the low nibble",
     "double e = E2M1_TAB[(k % 2 == 0) ? (byte & 15) : (byte >> 4)];",
     "double e = E2M1_TAB[(k % 2 == 0) ? (byte >> 4) : (byte & 15)];"),
    ("product forgets the tensor scale", "j->y[m * j->N + n] = j->gscale * y;", "j->y[m * j->N + n] = y;"),
    ("tolerance scale drops the tensor scale", "l1 += fabs(e * s * j->gscale * xv);", "l1 += fabs(e * s * xv);"),
    ("packing puts the even k in the high nibble", "(codes[2 * j] | (codes[2 * j + 1] << 4))",
     "(codes[2 * j + 1] | (codes[2 * j] << 4))"),
    ("tensor scale divides by 448 instead of 448 * 6", "amax / 2688.0f", "amax / 448.0f"),
    ("block scale divides by 4 instead of 6", "bamax / 6.0f", "bamax / 4.0f"),
    ("E2M1 ties go up", "if (a == mid) { code = (i % 2 == 0) ? i : i + 1; break; }",
     "if (a == mid) { code = i + 1; break; }"),
    ("E2M1 sign from v < 0 (negative zero loses its sign)", "(uint8_t)(code | (signbit(v) ? 8 : 0))",
     "(uint8_t)(code | (v < 0 ? 8 : 0))"),
    ("E4M3 ties go up", "c = (lo % 2 == 0) ? lo : lo + 1;", "c = lo + 1;"),
    ("E4M3 saturates to the NaN code", "        c = 0x7E;", "        c = 0x7F;"),
    ("greedy choice takes the last of equal maxima", "    return a > b;\n}", "    return a >= b;\n}"),
    ("greedy choice ranks NaN below numbers", "    if (isnan(a)) return 1;", "    if (isnan(a)) return 0;"),
    ("FP8 source divides by its scale", "(float)E4M3_TAB[src->fp8[i]] * src->fp8_scale;",
     "(float)E4M3_TAB[src->fp8[i]] / src->fp8_scale;"),
    ("bf16 bits shifted into the wrong place", "uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;"),
    ("dequantiser decodes the nibbles swapped", "int q = (k % 2 == 0) ? (byte & 15) : (byte >> 4);",
     "int q = (k % 2 == 0) ? (byte >> 4) : (byte & 15);"),
    ("dequantiser forgets the tensor scale",
     "out[n * K + k] = E2M1_TAB[q] * E4M3_TAB[scales[n * (K / 16) + k / 16]] * (double)gscale;",
     "out[n * K + k] = E2M1_TAB[q] * E4M3_TAB[scales[n * (K / 16) + k / 16]];"),
    ("silu uses e^z instead of e^-z", "return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    ("swiglu gates the gate product with silu of up", "h[i] = orc_silu(g[i]) * u[i];",
     "h[i] = orc_silu(u[i]) * g[i];"),
    ("rmsnorm sums instead of averaging", "double r = 1.0 / sqrt(ss / (double)K + eps);",
     "double r = 1.0 / sqrt(ss + eps);"),
    ("rmsnorm drops eps", "double r = 1.0 / sqrt(ss / (double)K + eps);", "double r = 1.0 / sqrt(ss / (double)K);"),
    ("rmsnorm forgets the square root", "double r = 1.0 / sqrt(ss / (double)K + eps);",
     "double r = 1.0 / (ss / (double)K + eps);"),
    ("rmsnorm drops the gain", "* r * (double)bf16_to_f32(gain[k]);", "* r;"),
    ("fp64-activation product reads activation row 0", "const double *xdm = j->xd ? j->xd + m * K : NULL;",
     "const double *xdm = j->xd ? j->xd : NULL;"),
    ("MX shared exponent one too large", "int shared = (e - 1) - 2;", "int shared = (e - 1) - 1;"),
    ("MX shared exponent not clamped below", "if (shared < -127) shared = -127;", "if (shared < -128) shared = -128;"),
    ("E8M0 decoded with bias 128", "return ldexp(1.0, (code & 0xFF) - 127);", "return ldexp(1.0, (code & 0xFF) - 128);"),
    ("MX zero block takes the element encoder", "if (amax == 0.0) {", "if (amax < 0.0) {"),
    ("MX product drops the block scale", "acc += s * inner;", "acc += inner;"),
    ("MX tile swaps the half and row-pair fields", "t[4096 + h * 128 + l * 4 + i]", "t[4096 + i * 64 + l * 2 + h]"),
]


def _run_pins(src_text, workdir, tag):
    c = os.path.join(workdir, "%s.c" % tag)
    so = os.path.join(workdir, "lib%s.so" % tag)
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", *oracle.CFLAGS, c, "-o", so, "-lm"])
    env = dict(os.environ)
    env[oracle._OVERRIDE_ENV] = so
    r = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu"],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-2000:]


@pytest.fixture(scope="module")
def pin_runs(tmp_path_factory):
    """The control and every mutant, built and run against the pins, a few at a time."""
    workdir = str(tmp_path_factory.mktemp("oracle_mutants"))
    src = open(oracle._SRC).read()
    jobs = {"control": src}
    for i, (name, old, new) in enumerate(MUTANTS):
        jobs[name] = src.replace(old, new) if old in src else None
    with concurrent.futures.ThreadPoolExecutor(max_workers=6) as ex:
        futs = {name: ex.submit(_run_pins, text, workdir, "m%d" % i)
                for i, (name, text) in enumerate(jobs.items()) if text is not None}
        return {name: f.result() for name, f in futs.items()}


def test_unmodified_oracle_passes_the_pins(pin_runs):
    code, out = pin_runs["control"]
    assert code == 0, out


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_a_pin_catches_the_planted_mistake(name, old, new, pin_runs):
    assert old in open(oracle._SRC).read(), "mutation point not found: " + name
    code, _ = pin_runs[name]
    assert code != 0, "no pin failed for: " + name
