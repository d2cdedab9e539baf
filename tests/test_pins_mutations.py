"""The oracle's pins catch planted mistakes.

Each case plants one plausible mistake in a copy of hashgrid_oracle.c (a sign, a dropped
factor, a swapped index, an off-by-one), builds the copy with gcc into a temporary folder and
runs the oracle's pin suite against it (HASHGRID_ORACLE_LIB points the wrapper at the
copy): at least one pin must fail.  The unmodified source, built the same way, must pass.
Every snippet must occur in the source, so a change to the oracle that moves one makes this
test fail rather than pass silently.
"""
import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "hashgrid_oracle.c")

# (name, text in the source, replacement, which occurrence (0-based))
MUTATIONS = [
    # encoder
    ("level progression without the 1e-6 guard", "pow(b, (double)l) + 1e-6)", "pow(b, (double)l))", 0),
    ("hash combines with + instead of XOR", "h ^= (uint32_t)(v[i] * ORC_PRIMES[i]);",
     "h += (uint32_t)(v[i] * ORC_PRIMES[i]);", 0),
    ("second and third primes swapped", "{1u, 2654435761u, 805459861u, 3674653429u}",
     "{1u, 805459861u, 2654435761u, 3674653429u}", 0),
    ("dense stride N instead of N+1", "stride *= (int64_t)c->N[l] + 1;", "stride *= (int64_t)c->N[l];", 0),
    ("dense rule counts N^d vertices", "return pow((double)c->N[l] + 1.0, (double)c->d);",
     "return pow((double)c->N[l], (double)c->d);", 0),
    ("last cell not capped at N-1", "if (b > c->N[l] - 1) b = c->N[l] - 1;", "if (b > c->N[l]) b = c->N[l];", 0),
    ("d-linear weights swapped", "w *= ((cc >> i) & 1) ? t[i] : 1.0 - t[i];",
     "w *= ((cc >> i) & 1) ? 1.0 - t[i] : t[i];", 0),
    ("near-corner derivative basis sign", "*B = t - 2 * t * t + t * t * t;", "*B = -t + 2 * t * t - t * t * t;", 0),
    ("far-corner value basis second derivative sign", "*d2B = 6 - 12 * t; }", "*d2B = -6 + 12 * t; }", 0),
    ("Delta x^|alpha| with the wrong sign of the exponent", "R_POW(Nl, -(real)popcount_bits(alpha))",
     "R_POW(Nl, (real)popcount_bits(alpha))", 0),
    ("gradient without N_l", "w1[i] = s * Nl * dB[i] * others;", "w1[i] = s * dB[i] * others;", 0),
    ("second derivative with N_l instead of N_l^2", "w2[i] = s * Nl * Nl * d2B[i] * others;",
     "w2[i] = s * Nl * d2B[i] * others;", 0),
    ("slot order reversed", "if (same) return rank;", "if (same) return (int)binom(d, k) - 1 - rank;", 0),
    ("diagonal upstream read from the Laplacian slot",
     "real up = (real)(c->d2_mode == 2 ? g_d2[(p * d + i) * LF + col] : g_d2[p * LF + col]);",
     "real up = (real)(c->d2_mode == 2 ? g_d2[(p * d) * LF + col] : g_d2[p * LF + col]);", 1),
    # fused residual
    ("SIREN Laplacian with omega instead of omega^2", "-om * om * s * sumsq + om * co * zs",
     "-om * s * sumsq + om * co * zs", 0),
    ("SIREN reverse: sin for cos on the Laplacian row", "zbar[1 + d] = lbar * om * co;",
     "zbar[1 + d] = lbar * om * s;", 0),
    ("source with the wrong sign", "real src = -(real)d * PI * PI;", "real src = (real)d * PI * PI;", 0),
    # Gaussian RBF
    ("RBF box starts one vertex early", "v[i] = (int64_t)base[i] - k + 1 + mm % side;",
     "v[i] = (int64_t)base[i] - k + mm % side;", 0),
    ("RBF second derivative with eps^2 instead of eps^4", "(4.0 * e2 * e2 * del * del - 2.0 * e2)",
     "(4.0 * e2 * del * del - 2.0 * e2)", 0),
    ("RBF gradient without N_l", "d1[nv][i] = -2.0 * e2 * del * phi[nv] * N;",
     "d1[nv][i] = -2.0 * e2 * del * phi[nv];", 0),
    ("RBF clipping drops the last vertex", "if (v[i] < 0 || v[i] > (int64_t)c->N[l]) inside = 0;",
     "if (v[i] < 0 || v[i] >= (int64_t)c->N[l]) inside = 0;", 0),
    ("RBF eps instead of eps^2", "const real e2 = (real)(c->eps * c->eps)", "const real e2 = (real)(c->eps)", 0),
    # INGP-FD comparator
    ("FD centre weight 1 instead of 2", "(u[2 * i + 1] - (real)2.0 * u[0] + u[2 * i + 2])",
     "(u[2 * i + 1] - (real)1.0 * u[0] + u[2 * i + 2])", 0),
    ("FD shift signs swapped", "(s % 2 == 1) ? x[p * d + i] + e32 : x[p * d + i] - e32",
     "(s % 2 == 1) ? x[p * d + i] - e32 : x[p * d + i] + e32", 0),
    ("FD seed without the factor 2", "const real seed = (real)(2.0 * (double)r * inv_n);",
     "const real seed = (real)(1.0 * (double)r * inv_n);", 1),
    ("FD reverse: sin for cos", "bar[o] * om * R_COS(om * z_s[k * H + o])", "bar[o] * om * R_SIN(om * z_s[k * H + o])", 0),
    ("FD divides by eps instead of eps^2", "u[2 * i + 2]) / (ep * ep);", "u[2 * i + 2]) / ep;", 0),
    ("FD encoder upstream reversed", "ug[(p * S + s) * LF + j] = bar[j];", "ug[(p * S + s) * LF + j] = bar[LF - 1 - j];", 0),
    # coarse-to-fine activation
    ("forward level guard off by one", "(c->kind != 2 && l < active_levels(c))", "(c->kind != 2 && l <= active_levels(c))", 0),
    ("backward level guard off by one", "if (l >= active_levels(c)) continue;", "if (l > active_levels(c)) continue;", 0),
    ("schedule capped one level short", "return a < (int64_t)L ? (int32_t)a : L;", "return a < (int64_t)L ? (int32_t)a : L - 1;", 0),
]


def pin_files() -> list:
    """The oracle's pin suite: tests/test_oracle_*.py and the page fixtures' test."""
    return sorted(glob.glob(os.path.join(ROOT, "tests", "test_oracle_*.py"))) + \
        [os.path.join(ROOT, "tests", "test_golden.py")]


def _plant(src: str, old: str, new: str, which: int) -> str:
    at = -1
    for _ in range(which + 1):
        at = src.find(old, at + 1)
        assert at >= 0, f"snippet not found (occurrence {which}): {old}"
    return src[:at] + new + src[at + len(old):]


def _pins_pass(lib: str) -> tuple[bool, str]:
    tests = pin_files()
    env = dict(os.environ, HASHGRID_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        *tests], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    return r.returncode == 0, r.stdout[-600:]


def test_pins_catch_planted_mistakes(tmp_path):
    from oracle.oracle import build_oracle
    src = open(SRC).read()
    cases = [("unmodified", src)] + [(name, _plant(src, old, new, which)) for name, old, new, which in MUTATIONS]

    def run(i_case):
        i, (name, text) = i_case
        c_path = tmp_path / f"m{i}.c"
        c_path.write_text(text)
        lib = build_oracle(out=str(tmp_path / f"liboracle_m{i}.so"), extra_flags=["-O1"], src=str(c_path))
        ok, tail = _pins_pass(lib)
        return name, ok, tail

    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as pool:
        results = list(pool.map(run, enumerate(cases)))
    assert results[0][1], "the unmodified oracle must pass its pins:\n" + results[0][2]
    survivors = [name for name, ok, _ in results[1:] if ok]
    assert not survivors, f"planted mistakes no pin caught: {survivors}"
    assert len(results) - 1 == len(MUTATIONS) >= 30
