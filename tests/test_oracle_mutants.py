"""The oracle's pins are sensitive: each plausible mistake planted in a copy
of the oracle's C source makes at least one pin in test_oracle_pins.py or
test_oracle_pins_ext.py fail.

Every mutant is compiled into a temporary library and the pins are run
against it in a child process (PKV_ORACLE_LIB points the oracle loader at
it).  CPU only; the shipped oracle is never modified.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pkv_oracle.c")

# (name, text in the oracle, replacement)
MUTANTS = [
    ("head h reads kv head h % Hkv", "const int h = g * G + j;", "const int h = j * Hkv + g;"),
    ("scale dropped", "s[t] = (double)scale * dot;", "s[t] = dot;"),
    ("offset in block off by one", "const int o = t % BS;", "const int o = (t + 1) % BS;"),
    ("one position past the history", "for (int t = 0; t < L; ++t) {", "for (int t = 0; t < L + (L < 60); ++t) {"),
    ("min instead of max as the shift", "if (s[t] > m) m = s[t];", "if (s[t] < m) m = s[t];"),
    ("weights not normalised", "const double w = s[t] / Z;", "const double w = s[t];"),
    ("fp8 scale ignored",
     "pkvo_e4m3fn_to_f64(((const uint8_t*)cache)[row + (size_t)d]) *\n         (double)scales[scale_idx];",
     "pkvo_e4m3fn_to_f64(((const uint8_t*)cache)[row + (size_t)d]) * 1.0;"),
    ("fp8 scale divisor 240 (FNUZ max)", "sc = amax / 448.0f;", "sc = amax / 240.0f;"),
    ("zero-amax scale 0.5", "if (amax == 0.0f) sc = 1.0f;", "if (amax == 0.0f) sc = 0.5f;"),
    ("opening token does not store its scale", "*scale_slot = sc;", "(void)0;"),
    ("e4m3 ties not to even", "(err == best_err && (c & 1) == 0 && (best & 1) == 1)", "(0)"),
    ("e4m3 subnormal exponent", "mag = ldexp((double)m / 8.0, -6);", "mag = ldexp((double)m / 8.0, -7);"),
    ("no saturation", "if (a >= 448.0) return (uint8_t)(sign | 0x7E);", "if (a >= 464.0) return (uint8_t)(sign | 0x7F);"),
    # generalised attention
    ("causal limit one short", "const int lim = L - ql + i;", "const int lim = L - ql + i - 1;"),
    ("causal mask aligned top-left", "const int lim = L - ql + i;", "const int lim = i;"),
    ("window one token too wide", "v = (t > lim - window) || (t < sinks);", "v = (t >= lim - window) || (t < sinks);"),
    ("sinks ignored", "v = (t > lim - window) || (t < sinks);", "v = (t > lim - window);"),
    # int8
    ("int8 scale divisor 128", "sc = amax / 127.0f;", "sc = amax / 128.0f;"),
    ("int8 rounds halves away from zero", "double r = rint((double)y);", "double r = round((double)y);"),
    ("int8 saturates at 126", "if (r > 127.0) r = 127.0;", "if (r > 126.0) r = 126.0;"),
    ("int8 scale ignored", "return (double)((const int8_t*)cache)[row + (size_t)d] * (double)scales[scale_idx];",
     "return (double)((const int8_t*)cache)[row + (size_t)d];"),
    # RoPE
    ("rotation sign flipped in one component", "const double r0 = x0 * c - x1 * sn;", "const double r0 = x0 * c + x1 * sn;"),
    ("pair members swapped", "const double x1 = pkvo_bf16_to_f64(x[base + 2 * i + 1]);",
     "const double x1 = pkvo_bf16_to_f64(x[base + (2 * i + 2) % D]);"),
    ("frequencies theta^(-i/D)", "pow(theta, -(2.0 * i) / (double)D)", "pow(theta, -(double)i / (double)D)"),
    ("Llama 3 band measured from the high edge",
     "double s = (turns - low_freq_factor) / (high_freq_factor - low_freq_factor);",
     "double s = (turns - high_freq_factor) / (high_freq_factor - low_freq_factor);"),
    ("Llama 3 ramp not clamped above the band", "if (s > 1.0) s = 1.0;", "(void)0;"),
    # two blends that agree with the right one at both band edges and are
    # monotone inside: only the library and hand-derived values catch them
    ("Llama 3 harmonic blend", "f[i] = fi * (s + (1.0 - s) / factor);",
     "f[i] = fi / ((1.0 - s) * factor + s);"),
    ("Llama 3 ramp linear in the wavelength",
     "double s = (turns - low_freq_factor) / (high_freq_factor - low_freq_factor);",
     "double s = (original_max / low_freq_factor - two_pi / fi) /\n"
     "               (original_max / low_freq_factor - original_max / high_freq_factor);"),
    ("bf16 rounding truncates", "if (frac > 0.5 || (frac == 0.5 && fmod(lo, 2.0) != 0.0)) lo += 1.0;", "(void)frac;"),
]


def _run_mutant(mut, tmpdir):
    name, old, new = mut
    src = open(SRC).read()
    assert old in src, f"mutation site for '{name}' not found in the oracle"
    idx = MUTANTS.index(mut)
    csrc = os.path.join(tmpdir, f"m{idx}.c")
    lib = os.path.join(tmpdir, f"m{idx}.so")
    with open(csrc, "w") as f:
        f.write(src.replace(old, new, 1))
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    "-o", lib, csrc, "-lm"], check=True, capture_output=True)
    env = dict(os.environ, PKV_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_pins_ext.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode


def test_every_planted_mistake_fails_a_pin():
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda m: _run_mutant(m, tmp), MUTANTS))
    survivors = [name for name, rc in results if rc == 0]
    assert not survivors, f"mutants not caught by any pin: {survivors}"
    # and the shipped oracle passes them (the pins are not failing for another reason)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_pins_ext.py")],
                       cwd=ROOT, capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-2000:]
