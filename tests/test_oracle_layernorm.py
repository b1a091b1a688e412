"""The oracle's LayerNorm against its pins (tests/pins_ln.py), and planted mistakes in
copies of the oracle that the pins must catch."""
import subprocess

import pytest

import oracle
from oracle.build import SRC
from tests import pins_ln


@pytest.mark.parametrize("check", pins_ln.ALL, ids=[c.__name__ for c in pins_ln.ALL])
def test_pin(check):
    check(oracle.default())


MUTANTS = {
    "unbiased_variance": ("const double var = kbn_dot(d.data(), d.data(), h, &S) / static_cast<double>(h);",
                          "const double var = kbn_dot(d.data(), d.data(), h, &S) / static_cast<double>(h - 1);"),
    "eps_dropped": ("*rstd = 1.0 / std::sqrt(var + eps);", "*rstd = 1.0 / std::sqrt(var);"),
    "eps_outside_sqrt": ("*rstd = 1.0 / std::sqrt(var + eps);", "*rstd = 1.0 / (std::sqrt(var) + eps);"),
    "mean_not_subtracted": ("for (int64_t j = 0; j < h; ++j) d[j] = d[j] - mu;", "for (int64_t j = 0; j < h; ++j) d[j] = d[j];"),
    "beta_scaled": ("if (beta) v = v + decode(beta, j, dt);", "if (beta) v = v + 2.0 * decode(beta, j, dt);"),
    "gamma_index": ("if (gamma) v = v * decode(gamma, j, dt);", "if (gamma) v = v * decode(gamma, h - 1 - j, dt);"),
    "dx_sign": ("const double v = rstd[i] * ((g[j] - a) - xhat[j] * b);", "const double v = rstd[i] * ((g[j] - a) + xhat[j] * b);"),
    "dx_no_mean_term": ("const double v = rstd[i] * ((g[j] - a) - xhat[j] * b);", "const double v = rstd[i] * (g[j] - xhat[j] * b);"),
    "dx_gamma_dropped": ("g[j] = gamma ? dyv * decode(gamma, j, dt) : dyv;", "g[j] = dyv;"),
    "dgamma_uses_x": ("colx[j * rows + i] = xhat[j];", "colx[j * rows + i] = decode(x, i * h + j, dt);"),
    "dbeta_one_row_short": ("if (dbeta) store(dbeta, j, kbn_dot(&coly[j * rows], ones.data(), rows, &S), pdt);",
                            "if (dbeta) store(dbeta, j, kbn_dot(&coly[j * rows], ones.data(), rows - 1, &S), pdt);"),
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
    for check in pins_ln.ALL:
        try:
            check(O)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"planted mistake {name} passed every LayerNorm pin"
