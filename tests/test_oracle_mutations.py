"""The oracle's pins catch plausible mistakes.

Each case plants one mistake (a dropped term, a wrong index, offset or sign,
swapped operands, a wrong rounding) in a temporary copy of oracle/oracle.c,
builds it into a separate library, and runs tests/test_oracle_pins.py
against it (ORACLE_LIB).  The pins must fail for every mutant; they pass on
the real oracle (test_oracle_pins itself).  CPU only.
"""
import os
import subprocess
import sys

import pytest

from oracle import build as oracle_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, text in oracle.c, replacement): each text occurs exactly once.
MUTANTS = [
    ("mode 0 reads the source rank's head block",
     "+ (g->head_off[r] + h)) * g->d + e;", "+ (g->head_off[j] + h)) * g->d + e;"),
    ("mode 1 drops the sequence offset", "(g->seq_off[r] + s)) * g->H[j]", "(s)) * g->H[j]"),
    ("mode 1 drops the head offset",
     "+ (h - g->head_off[j])) * g->d + e;", "+ (h)) * g->d + e;"),
    ("sequence owner off by one", "if (g->seq_off[j] <= S && S < g->seq_off[j + 1])",
     "if (g->seq_off[j] <= S && S <= g->seq_off[j + 1])"),
    ("window bytes from S_r in mode 0", "bytes = g.s_global * g.H[r] * d * esz;",
     "bytes = g.S[r] * g.H[r] * d * esz;"),
    ("bf16 ties rounded away", "u += 0x7FFFu + lsb;", "u += 0x8000u + 0 * lsb;"),
    ("rotary frequency theta^(-p/d)", "double w = pow(theta, -2.0 * (double)p / (double)d);",
     "double w = pow(theta, -1.0 * (double)p / (double)d);"),
    ("cos and sin swapped", "cos_out[S * half + p] = (float)cos(angle);",
     "cos_out[S * half + p] = (float)sin(angle);"),
    ("gain dropped", "        y[i] = (xf[i] * inv) * gamma[i];", "        y[i] = (xf[i] * inv);"),
    ("eps dropped", "inv = 1.0f / sqrtf(ms + eps);", "inv = 1.0f / sqrtf(ms + 0.0f * eps);"),
    ("mean over d/2", "ms = ss / (float)d;", "ms = ss / (float)(d / 2);"),
    ("rotation sign flipped", "o[2 * p] = float_to_bf16_rne(a - bb);",
     "o[2 * p] = float_to_bf16_rne(a + bb);"),
    ("rotate-half pairing", "float a = y[2 * p] * c;", "float a = y[p] * c;"),
    ("local instead of global position",
     "norm_rope_row(x, o, d, gamma, eps,\n                                  cos_tab + S * (d / 2), sin_tab + S * (d / 2));",
     "norm_rope_row(x, o, d, gamma, eps,\n                                  cos_tab + (S - g.seq_off[j]) * (d / 2), "
     "sin_tab + (S - g.seq_off[j]) * (d / 2));"),
    ("partial sums skip an element", "for (i = 8 * l; i < 8 * l + 8; ++i)",
     "for (i = 8 * l; i < 8 * l + 7; ++i)"),
    ("one chain over the whole row", "part[l] = fmaf(xf[i], xf[i], part[l]);",
     "part[0] = fmaf(xf[i], xf[i], part[0]);"),
    ("tree pairs the halves first", "part[k] = part[2 * k] + part[2 * k + 1];",
     "part[k] = part[k] + part[k + n / 2];"),
    ("tree drops the odd partial", "part[k] = part[2 * k] + part[2 * k + 1];",
     "part[k] = part[2 * k] + part[2 * k];"),
    ("first cosine product contracted into the subtract",
     "o[2 * p] = float_to_bf16_rne(a - bb);",
     "o[2 * p] = float_to_bf16_rne(fmaf(y[2 * p], c, -bb));"),
    ("first sine product contracted into the subtract",
     "o[2 * p] = float_to_bf16_rne(a - bb);",
     "o[2 * p] = float_to_bf16_rne(fmaf(-y[2 * p + 1], s, a));"),
    ("second sine product contracted into the add",
     "o[2 * p + 1] = float_to_bf16_rne(cc + dd);",
     "o[2 * p + 1] = float_to_bf16_rne(fmaf(y[2 * p], s, dd));"),
    ("second cosine product contracted into the add",
     "o[2 * p + 1] = float_to_bf16_rne(cc + dd);",
     "o[2 * p + 1] = float_to_bf16_rne(fmaf(y[2 * p + 1], c, cc));"),
    ("gain folded into inv first", "        y[i] = (xf[i] * inv) * gamma[i];",
     "        y[i] = xf[i] * (inv * gamma[i]);"),
]


def test_every_mutant_text_is_present():
    src = open(SRC).read()
    for name, old, _new in MUTANTS:
        assert src.count(old) == 1, f"{name}: text not found exactly once"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1
    mutant_c = tmp_path / "oracle_mutant.c"
    mutant_c.write_text(src.replace(old, new))
    lib = oracle_build.build(src=str(mutant_c), out=str(tmp_path / "liboracle_mutant.so"))
    env = dict(os.environ, ORACLE_LIB=lib)
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert res.returncode != 0, f"the pins did not catch: {name}"
