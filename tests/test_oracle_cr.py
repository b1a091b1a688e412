"""The oracle's correctly rounded tier against its pins (tests/pins_cr.py), and planted
mistakes in copies of the oracle that the pins must catch."""
import subprocess

import pytest

import oracle
from oracle.build import SRC
from tests import pins_cr


@pytest.mark.parametrize("check", pins_cr.ALL, ids=[c.__name__ for c in pins_cr.ALL])
def test_pin(check):
    check(oracle.default())


MUTANTS = {
    "sticky_dropped": ("const bool sticky = mag.any_below(lsb - 1);", "const bool sticky = false;"),
    "ties_away": ("if (round && (sticky || (keep & 1u))) keep += 1;", "if (round) keep += 1;"),
    "negative_sign_lost": ("    sign = -1.0;\n", "    sign = 1.0;\n"),
    "subnormal_clamp_dropped": ("if (lsb < lsb_min) lsb = lsb_min;", "(void)lsb_min;"),
    "bias_dropped": ("if (bias) x.add(decode(bias, col, dt));", "(void)bias;"),
    "limb_carry_dropped": ("      carry = t >> 32;\n", "      carry = 0;\n"),
    "zero_is_negative": ("if (c == 0) return 0.0;", "if (c == 0) return -0.0;"),
    "through_float64": ("  if (x.has_nonfinite) return x.nonfinite;\n  BigMag mag = x.pos;",
                        "  if (x.has_nonfinite) return x.nonfinite;\n  if (dt != DT_F32) { (void)0; }\n  BigMag mag = x.pos;\n  if (true) {\n    double d = 0.0; int e0;\n    for (int i = BIG_LIMBS - 1; i >= 0; --i) d = d * 4294967296.0 + static_cast<double>(x.pos.limb[i]) - static_cast<double>(x.neg.limb[i]);\n    (void)e0;\n    return std::ldexp(d, -BIG_LOW);\n  }"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = tmp_path / f"{name}.cpp"
    src.write_text(text.replace(old, new))
    out = str(tmp_path / f"lib{name}.so")
    subprocess.run(["g++", *oracle.build.FLAGS, str(src), "-o", out], check=True)
    O = oracle.Oracle(out)
    failed = []
    for check in pins_cr.ALL:
        try:
            check(O)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"planted mistake {name} passed every pin"
