"""Plant plausible mistakes in copies of the oracle source; each must trip a pin.

This shows the pins are strong enough: a dropped term, a wrong sign or index, a
transposed operand or a wrong mask in the oracle would not pass unnoticed.
The mutated copies are compiled into a temporary directory and never replace
the committed oracle.
"""
import pytest

import oracle
from tests import oracle_pins as pins

# (name, original text, replacement, count of occurrences to replace: 0 = all)
MUTANTS = [
    ("scale dropped", "s *= scale;", "s *= 1.0;", 0),
    ("diagonal excluded", "int64_t last = causal ? t : S - 1;",
     "int64_t last = causal ? t - 1 : S - 1;", 1),
    ("block mask off by one", "if (causal && kid[j] > gq) continue;",
     "if (causal && kid[j] >= gq) continue;", 0),
    ("zig-zag late chunk mirrored wrong", ": (2 * (int64_t)R - 1 - r) * c + (j - c);",
     ": (R + r) * c + (j - c);", 1),
    ("ring key ids from the query rank", "for (int64_t j = 0; j < n; ++j) kid[j] = fwd[s * n + j];",
     "for (int64_t j = 0; j < n; ++j) kid[j] = fwd[r * n + j];", 1),
    ("merge weight sign", "l_a[r] * exp(ma - m)", "l_a[r] * exp(m - ma)", 1),
    ("merge drops a weight", "(wa * o_a[r * d + c] + wb * o_b[r * d + c]) / l",
     "(o_a[r * d + c] + wb * o_b[r * d + c]) / l", 1),
    ("striped equals contiguous", "t = j * R + r;", "t = r * n + j;", 1),
    ("grouped head index", "int64_t g = h / group;\n    const float *kb = k + (b * Hkv + g) * S * d;",
     "int64_t g = h % Hkv;\n    const float *kb = k + (b * Hkv + g) * S * d;", 1),
    ("log base", "lse_rows[r] = m + log(l);", "lse_rows[r] = m + log2(l);", 1),
    ("ring skips a hop", "for (int64_t hop = 0; hop < R; ++hop)",
     "for (int64_t hop = 0; hop < R - 1; ++hop)", 1),
    ("keys used as values", "o[c] += p * (double)vb[j * d + c];",
     "o[c] += p * (double)kb[j * d + c];", 1),
    ("max never updated", "      if (s > m) m = s;\n", "", 1),
    ("merge forgets the normaliser", "double l = wa + wb;", "double l = wa + wb + 1.0;", 1),
    ("backward drops D", "double ds = pj * (dp[j] - D);", "double ds = pj * dp[j];", 1),
    ("backward dk unscaled", "dkb[j * d + c] += scale * ds * (double)qi[c];",
     "dkb[j * d + c] += ds * (double)qi[c];", 0),
    ("backward dv from dS", "dvb[j * d + c] += pj * (double)gi[c];",
     "dvb[j * d + c] += ds * (double)gi[c];", 0),
    ("block backward mask off by one", "if (causal && kid[j] > qid[i]) continue;",
     "if (causal && kid[j] >= qid[i]) continue;", 1),
    ("block backward uses row max for lse", "double pj = exp(sj * scale - lse[row]);",
     "double pj = exp(sj * scale - lse[row] + 0.1);", 1),
]


@pytest.mark.parametrize("mut", MUTANTS, ids=lambda m: m[0])
def test_mutant_is_caught(tmp_path, mut):
    name, old, new, count = mut
    src = oracle.source_text()
    assert old in src, "mutation anchor not found: %s" % name
    bad = src.replace(old, new) if count == 0 else src.replace(old, new, count)
    orc = oracle.compile_variant(bad, str(tmp_path / "libmutant.so"))
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check(orc)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(check.__name__)
    assert failed, "mutant '%s' passed every pin" % name

