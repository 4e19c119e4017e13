"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a TEMPORARY COPY of oracle/oracle.c (a dropped term,
a wrong sign or index, a transposed operand, a wrong mask or epsilon), rebuilds that copy and
runs the pin suite against it: every planted mistake must make at least one pin fail.  The
real oracle is never modified.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTS = [
  ("angle formula", "ORACLE_PI * u / (1.0 + fabs(u))", "ORACLE_PI * u / (1.0 + u * u)"),
  ("root sign", "cos(theta + omega) - sin(theta + omega)", "cos(theta + omega) + sin(theta + omega)"),
  ("root from rotated angle", "const double r = sanatan_root(th, omega[a], gamma);\n      const double th_rot = th + t * sanatan_freq(a, d, lambda_base);",
     "const double th_rot = th + t * sanatan_freq(a, d, lambda_base);\n      const double r = sanatan_root(th_rot, omega[a], gamma);"),
  ("feature rotation sign", "th + t * sanatan_freq", "th - t * sanatan_freq"),
  ("kappa (t-s) sign", "(double)(t - s) * sanatan_freq(a, d, lambda_base)", "(double)(s - t) * sanatan_freq(a, d, lambda_base)"),
  ("direct rotation sign", "+ (double)(t - s) * lam[a]", "- (double)(t - s) * lam[a]"),
  ("direct mask strict", "for (int s = 0; s <= t; s++)", "for (int s = 0; s < t; s++)"),
  ("direct eps scaled", "o[n] = num[n] / (den + eps)", "o[n] = num[n] / (den + c * eps)"),
  ("recurrent eps unscaled", "num / (den + c * eps)", "num / (den + eps)"),
  ("freq index", "-(double)a / (double)d", "-(double)(a + 1) / (double)d"),
  ("power off by one", "for (int e = 0; e < p; e++)", "for (int e = 0; e <= p; e++)"),
  ("channel 4 wrong", "row[4 * d + a] = r * c;", "row[4 * d + a] = r * s;"),
  ("gate dropped", "acc += (1.0 + rq * rk) * (1.0 + cos(dth));", "acc += (1.0 + cos(dth));"),
  ("direct gate dropped", ": (1.0 + gate) * (1.0 + cos(dth));", ": 2.0 * (1.0 + cos(dth));"),
  ("four-channel gate applied to the constant", "four ? 1.0 + gate * (1.0 + cos(dth))", "four ? (1.0 + gate) * (1.0 + cos(dth))"),
  ("recurrent read before write", None, None),
  ("S transposed", "S[(size_t)f * dv + n] += fk[f]", "S[(size_t)n * 6 * d + f] += fk[f]"),
  ("direct weight not normalised by c", "double w = kap / c;", "double w = kap;"),
  ("harmonic multiple dropped in kappa_h", "for (int n = 1; n <= nh; n++) ang += cos((double)n * x);", "for (int n = 1; n <= nh; n++) ang += cos(x);"),
  ("harmonic multiple dropped in features", "const double c = cos((double)n * th_rot), s = sin((double)n * th_rot);", "const double c = cos(th_rot), s = sin(th_rot);"),
  ("harmonic gated channel uses the wrong harmonic", "row[(size_t)(2 * nh + 2 * n + 1) * d + a] = r * s;", "row[(size_t)(2 * nh + 2 * n + 1) * d + a] = r * sin(th_rot);"),
  ("harmonic root channel misplaced", "row[(size_t)(2 * nh + 1) * d + a] = r;", "row[(size_t)(2 * nh) * d + a] = r;"),
  ("grad query sin sign", "dth[a] += G * (-(1.0 + rq[ti] * rk[si]) * sin(x)", "dth[a] += G * ((1.0 + rq[ti] * rk[si]) * sin(x)"),
  ("grad key root slope dropped", "+ rq[ti] * (1.0 + cos(x)) * sk[si]);", ");"),
  ("grad output term dropped", "(v[(size_t)s * dv + n] - o[(size_t)t * dv + n])", "v[(size_t)s * dv + n]"),
  ("grad angle slope not squared", "ORACLE_PI / ((1.0 + fabs(u)) * (1.0 + fabs(u)))", "ORACLE_PI / (1.0 + fabs(u))"),
  ("grad root slope sign", "(-sin(theta + omega) - cos(theta + omega))", "(-sin(theta + omega) + cos(theta + omega))"),
  ("grad power factor dropped", "(double)p * pow(kap, (double)(p - 1))", "pow(kap, (double)(p - 1))"),
  ("grad value weight not normalised", "dvs[n] += w * g[(size_t)t * dv + n] / D[t];", "dvs[n] += w * g[(size_t)t * dv + n];"),
]

READ_BEFORE_WRITE = (
    "    oracle_features(k + (size_t)i * d, 1, d, pos0 + i, omega, gamma, lambda_base, fk);\n"
    "    for (int f = 0; f < D; f++) {\n      z[f] += fk[f];",
    "    oracle_features(k + (size_t)i * d, 1, d, pos0 + i, omega, gamma, lambda_base, fk);\n"
    "    if (i > 0) oracle_features(k + (size_t)(i-1) * d, 1, d, pos0 + i - 1, omega, gamma, lambda_base, fk);\n"
    "    for (int f = 0; f < D; f++) {\n      z[f] += fk[f];",
)


@pytest.mark.parametrize("name,old,new", MUTS, ids=[m[0] for m in MUTS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    if name == "recurrent read before write":
        old, new = READ_BEFORE_WRITE
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert old in src, "mutation anchor not found: " + name
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle",
                    ignore=shutil.ignore_patterns("*.so", "*.tmp*", "__pycache__"))
    (tmp_path / "tests" / "golden").mkdir(parents=True)
    for f in ("conftest.py", "test_oracle_pins.py", "test_oracle_four_channel.py", "test_oracle_grad.py",
              "test_oracle_harmonics.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    shutil.copy(os.path.join(ROOT, "tests", "golden", "pages_values.json"), tmp_path / "tests" / "golden")
    (tmp_path / "oracle" / "oracle.c").write_text(src.replace(old, new))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_oracle_pins.py",
                        "tests/test_oracle_four_channel.py", "tests/test_oracle_grad.py",
                        "tests/test_oracle_harmonics.py"],
                       cwd=tmp_path, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, "planted mistake '%s' passed every pin:\n%s" % (name, r.stdout[-2000:])
