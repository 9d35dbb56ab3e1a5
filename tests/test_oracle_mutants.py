"""The oracle's pins must catch plausible mistakes.

Each mutant below plants one typical slip into a copy of the oracle source
(a flipped sign, a dropped term, a wrong comparison, a wrong index or order),
builds it on the CPU, and runs the pin suite against it in a subprocess.  A
mutant that passes every pin would mean the pins do not constrain that part
of the oracle.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = [
    ("gap sign", "dr = mt[r] - m[r];", "dr = m[r] - mt[r];"),
    ("non-strict test", "if (g < lnlam) {", "if (g <= lnlam) {"),
    ("any-row instead of every-row vote", "if (dr > g)\n                g = dr;",
     "if (g == -INFINITY || (dr < g && dr != -INFINITY))\n                g = dr;"),
    ("first block may skip", "dr = INFINITY;", "dr = 0.0;"),
    ("alpha exponent sign", "exp(m[r] - mp)", "exp(mp - m[r])"),
    ("row sum not rescaled", "l[r] = alpha * l[r] + rowsum;", "l[r] = l[r] + rowsum;"),
    ("accumulator not rescaled", "ar[x] *= alpha;", "ar[x] *= 1.0;"),
    ("skipped block still accumulates", "continue; /* no exp, no V read", "if (0) continue; /* no exp, no V read"),
    ("causal off by one", "key <= qpos[r]", "key < qpos[r]"),
    ("scale dropped", "double s = scale * dot;", "double s = dot;"),
    ("V row index", "const double *vc = v + (c0 + c) * dv;", "const double *vc = v + (c0 + c) * dv + (c > 0 ? dv : 0);"),
    ("GQA head mapping", "int64_t hk = h / G;", "int64_t hk = h % Hkv;"),
    ("split length floor", "int64_t per = (nkb_b - j0 + num_splits - 1) / num_splits;",
     "int64_t per = (nkb_b - j0) / num_splits > 0 ? (nkb_b - j0) / num_splits : 1;"),
    ("window edge off by one", "key > qpos[r] - window", "key >= qpos[r] - window"),
    ("seed on the first split too", "(sink_seed && s > 0) ? seed : NULL", "sink_seed ? seed : NULL"),
    ("seed from the block after the first",
     "key = j0 * block_k; key < (j0 + 1) * block_k && key < len", "key = (j0 + 1) * block_k; key < (j0 + 2) * block_k && key < len"),
    ("seed without the scale", "if (scale * dot > seed[r])\n                            seed[r] = scale * dot;",
     "if (dot > seed[r])\n                            seed[r] = dot;"),
    ("decode splits ignore the window", "int64_t j0 = (window > 0 && len > window) ? (len - window) / block_k : 0;",
     "int64_t j0 = 0;"),
    ("merge weight sign", "double w = exp(ms[s * G + r] - M);", "double w = exp(M - ms[s * G + r]);"),
    ("quantile midpoint", "lnl = 0.5 * (s[kk - 1] + s[kk]);", "lnl = s[kk];"),
    ("fit uses lambda only", "sum += log(lambda_at_L[i] * (double)L[i]);", "sum += log(lambda_at_L[i]);"),
    ("table interpolation linear in a", "lna = (1.0 - w) * log(a[i]) + w * log(a[i + 1]);",
     "lna = log((1.0 - w) * a[i] + w * a[i + 1]);"),
    # the reading of non-finite inputs (R24)
    ("masked keys left out of P.V", "if (!seen[c])\n                    continue; /* no row of the unit sees this key */",
     "if (!seen[c] || S[r * bc + c] == -INFINITY)\n                    continue;"),
    ("keys no row sees still enter", "if (!seen[c])\n                    continue; /* no row of the unit sees this key */",
     "if (c0 + c >= klen)\n                    continue;"),
    ("rows without a key skip the update", "double mp = m[r] > mt[r] ? m[r] : mt[r];\n            double alpha",
     "double mp = m[r] > mt[r] ? m[r] : mt[r];\n            if (mp == -INFINITY) continue;\n            double alpha"),
    ("NaN sum finalised as empty", "ob[r * dv + x] = l[r] != 0.0 ?", "ob[r * dv + x] = l[r] > 0.0 ?"),
    ("merge drops NaN splits", "if (ls[s * G + r] == 0.0)\n                            continue;",
     "if (!(ls[s * G + r] > 0.0))\n                            continue;"),
    ("NaN score raises the block max", "if (s > mt[r]) /* a NaN score never raises the max */",
     "if (!(s <= mt[r]))"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", str(mpath),
                    "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB_OVERRIDE=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant '{name}' passed every pin:\n{r.stdout[-2000:]}"
