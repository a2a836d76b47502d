"""Planted mistakes: each variant of the oracle below carries one plausible bug, and the pins in
test_oracle_pins.py (test_oracle_polar.py for the polar baseline) must catch every one of them.  Variants are compiled from a patched copy of the
oracle source in a temporary directory; the oracle itself is never modified."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "qamw_oracle.c")

MUTANTS = [
    # sign mask (section 3.3, reading R1): caught by test_oracle_sign.py
    ("splitmix64 first shift", "z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;", "z = (z ^ (z >> 31)) * 0xBF58476D1CE4E5B9ULL;",
     "test_oracle_sign.py"),
    ("sign from output j instead of j + 1", "oracle_splitmix64(seed, d_in, z);",
     "z[0] = 0; oracle_splitmix64(seed, d_in - 1, z + 1);", "test_oracle_sign.py"),
    ("sign mask dropped", "a[j] = eps_of(sign_bits, j) * (a[j] / r);", "a[j] = (a[j] / r);"),
    ("Hadamard sign from i|k", "(__builtin_popcount(i & k) & 1) ? -scale : scale",
     "(__builtin_popcount(i | k) & 1) ? -scale : scale"),
    ("pair second coordinate", "float py = (float)(y[2 * k + 1] / (double)sigma[k]);",
     "float py = (float)(y[2 * k] / (double)sigma[k]);"),
    ("sigma multiplied", "float px = (float)(y[2 * k] / (double)sigma[k]);",
     "float px = (float)(y[2 * k] * (double)sigma[k]);"),
    ("distance sign", "float dx = px - cb[2 * j];", "float dx = px + cb[2 * j];"),
    ("ties to highest index", "if (d < best_d) {", "if (d <= best_d) {"),
    ("norm without sqrt", "double r = sqrt(r2);", "double r = r2;"),
    ("MSB-first packing", "out[q / 8] |= (uint8_t)(1u << (q % 8));", "out[q / 8] |= (uint8_t)(0x80u >> (q % 8));"),
    ("decode keeps channel scale", "* v[j]) / (double)s[j];", "* v[j]);"),
    ("decode wrong column", "acc += H[(size_t)k * block + jj] * x[(size_t)t * block + k];",
     "acc += H[(size_t)k * block + (jj ^ 1)] * x[(size_t)t * block + k];"),
    ("decode drops sign mask", "((rn * eps_of(sign_bits, j)) * v[j])", "((rn * 1.0) * v[j])"),
    ("decode drops sigma", "x[2 * k] = (double)sigma[k] * (double)cb[2 * idx[k]];",
     "x[2 * k] = (double)cb[2 * idx[k]];"),
    ("Lloyd divides by n+1", "cb[2 * j] = (float)(((double)sx[j] * 0x1p-32) / (double)cnt[j]);",
     "cb[2 * j] = (float)(((double)sx[j] * 0x1p-32) / (double)(cnt[j] + 1));"),
    ("Lloyd resets empty cells", "if (cnt[j] > 0) { /* centroid", "if (1) { if (!cnt[j]) cnt[j] = 1; /* centroid"),
    ("calibration counts zero rows", "sum[k] / (double)n_nz", "sum[k] / (double)n_rows"),
    ("calibration constant", "sqrt(ORACLE_PI / 2.0)", "sqrt(2.0 / ORACLE_PI)"),
    ("f16 truncates", "return rint(x / quantum) * quantum;", "return trunc(x / quantum) * quantum;"),
    ("no row alignment", "return (used + 15) / 16 * 16;", "return used;"),
    ("block cap 512", "while (b < 1024 && d_in % (2 * b) == 0)", "while (b < 512 && d_in % (2 * b) == 0)"),
    ("bpw norm bits", "return bits / 2.0 + 16.0 / d_in;", "return bits / 2.0 + 32.0 / d_in;"),
    ("stored norm not rounded via float", "nh = oracle_f16_from_f32((float)r);", "nh = oracle_f16_from_f32((float)(r * 1.001));"),
    # polar baseline (section 3.5): caught by test_oracle_polar.py
    ("Rayleigh moment without the erf term", "- hi + sqrt(0.5 * ORACLE_PI) * (eb - erf(a / sqrt(2.0)));", "- hi;",
     "test_oracle_polar.py"),
    ("phase index truncated", "floor(th * np_ / (2.0 * ORACLE_PI) + 0.5)", "floor(th * np_ / (2.0 * ORACLE_PI))",
     "test_oracle_polar.py"),
    ("magnitude compared unsquared", "if (r2 > thresholds[i] * thresholds[i]) ia = i + 1;",
     "if (r2 > thresholds[i]) ia = i + 1;", "test_oracle_polar.py"),
    ("polar index layout swapped", "return ia + na * ip;", "return ip + np_ * ia;", "test_oracle_polar.py"),
    ("zero pair phase from atan2 of signed zeros", "    if (r2 > 0.0) {\n        double th", "    if (1) {\n        double th",
     "test_oracle_polar.py"),
    # product after dequantization (section 1): caught by test_oracle_qgemm.py
    ("qgemm output transposed", "y[(size_t)m * n_rows + i0 + i] = acc;", "y[(size_t)(i0 + i) * M + m] = acc;",
     "test_oracle_qgemm.py"),
    ("qgemm on fp32-rounded weights", "acc += (double)x[(size_t)m * ld_x + j] * w[(size_t)i * d_in + j];",
     "acc += (double)x[(size_t)m * ld_x + j] * (double)f32[(size_t)i * d_in + j];", "test_oracle_qgemm.py"),
    ("qgemm drops the last column", "for (int32_t j = 0; j < d_in; ++j) acc +=",
     "for (int32_t j = 0; j < d_in - 1; ++j) acc +=", "test_oracle_qgemm.py"),
    # scalar (d = 1) ablation: caught by test_oracle_scalar.py
    ("scalar cell mean sign", "double v = (normal_pdf(a) - normal_pdf(c)) / (normal_cdf(c) - normal_cdf(a));",
     "double v = (normal_pdf(c) - normal_pdf(a)) / (normal_cdf(c) - normal_cdf(a));", "test_oracle_scalar.py"),
    ("scalar ties to the upper level", "if ((double)p > thresholds[i]) ix = i + 1;",
     "if ((double)p >= thresholds[i]) ix = i + 1;", "test_oracle_scalar.py"),
    ("scalar table transposed", "cb[2 * (ix + L * iy)] = (float)levels[ix];", "cb[2 * (ix + L * iy)] = (float)levels[iy];",
     "test_oracle_scalar.py"),
    # activation-aware channel scale: caught by test_oracle_actscale.py
    ("act scale without the root", "double r = sqrt(acc / (double)T);", "double r = acc / (double)T;",
     "test_oracle_actscale.py"),
    ("act scale over T - 1", "double r = sqrt(acc / (double)T);", "double r = sqrt(acc / (double)(T - 1));",
     "test_oracle_actscale.py"),
    ("dead channel scale 0", "scale[j] = r > 0.0 ? (float)pow(r, alpha) : 1.0f;", "scale[j] = (float)pow(r, alpha);",
     "test_oracle_actscale.py"),
    ("polar table angle off by half a bin", "double th = 2.0 * ORACLE_PI * ip / np_;",
     "double th = 2.0 * ORACLE_PI * (ip + 0.5) / np_;", "test_oracle_polar.py"),
]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, mutant):
    name, old, new = mutant[:3]
    pins = mutant[3] if len(mutant) > 3 else "test_oracle_pins.py"
    import oracle
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation anchor must be unique: %r" % old
    variant = tmp_path / "qamw_oracle_mutant.c"
    variant.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmutant.so")
    oracle.compile_to(str(variant), lib)
    env = dict(os.environ, ORACLE_LIB=lib, OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", pins)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "planted mistake '%s' passed every pin:\n%s" % (name, r.stdout[-2000:])
