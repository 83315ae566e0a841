"""The oracle's pins must reject plausible mistakes.

Each case copies ``oracle/qd_oracle.c``, plants one mistake by a textual
replacement (a dropped term, a wrong sign, index or operand), compiles the
copy with gcc on the CPU, and runs the pin tests against it in a child
process; the pins must fail.  The unmodified source must pass the same run.
"""
import os
import subprocess
import sys

import pytest

from oracle import build as obuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "qd_oracle.c")
PINS = [os.path.join(ROOT, "tests", "test_oracle_pins.py"),
        os.path.join(ROOT, "tests", "test_oracle_model.py")]

MUTANTS = {
    "nibble_order": ("j < 16 ? (blockq[j] & 0x0f) : (blockq[j - 16] >> 4)",
                     "j < 16 ? (blockq[j] >> 4) : (blockq[j - 16] & 0x0f)"),
    "code_offset": ("wb[j] = (double)(q4_code(q, j) - 8) * d;",
                    "wb[j] = (double)(q4_code(q, j) - 7) * d;"),
    "f16_exponent": ("v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)(1024 + f), e - 24);"),
    "f16_round_trunc": ("double m = nearbyint(ldexp(a, 10 - E));", "double m = floor(ldexp(a, 10 - E));"),
    "rms_eps_outside": ("1.0 / sqrt(ss / (double)n + eps)", "1.0 / (sqrt(ss / (double)n) + eps)"),
    "rms_sum_not_mean": ("1.0 / sqrt(ss / (double)n + eps)", "1.0 / sqrt(ss + eps)"),
    "rope_sign": ("v[i + half] = a * s + b * c;", "v[i + half] = -a * s + b * c;"),
    "rope_ignores_partial": ("int32_t half = rot / 2;", "int32_t half = hd / 2;"),
    "attn_head_map": ("g = h / grp;", "g = h % nkv;"),
    "attn_no_scale": ("s[t] = dot * scale;", "s[t] = dot;"),
    "model_window": ("for (int64_t t = 0; t <= pos; t++) {\n                const double* kr",
                     "for (int64_t t = 0; t < pos; t++) {\n                const double* kr"),
    "model_no_residual": ("        for (int64_t i = 0; i < H; i++)\n            m->x[i] += m->o[i];\n\n",
                          "        for (int64_t i = 0; i < H; i++)\n            m->x[i] = m->o[i];\n\n"),
    "silu_sign": ("m->g[i] / (1.0 + exp(-m->g[i]))", "m->g[i] / (1.0 + exp(m->g[i]))"),
    "gate_up_swapped": ("or_gemv_q4_0(&L->wgate, m->h, m->g, nt);\n        or_gemv_q4_0(&L->wup, m->h, m->u, nt);",
                        "or_gemv_q4_0(&L->wup, m->h, m->g, nt);\n        or_gemv_q4_0(&L->wgate, m->h, m->u, nt);"),
    "k_norm_weight": ("or_rmsnorm(m->k + gg * hd, L->k_norm, hd, c->eps, m->tmp);",
                      "or_rmsnorm(m->k + gg * hd, L->q_norm, hd, c->eps, m->tmp);"),
    "model_kv_unrounded": ("return m->cfg.kv_round ? or_f16_to_f64(or_f64_to_f16(val)) : val;",
                           "return val;"),
    "e4m3_bias": ("ldexp(1.0 + mant / 8.0, e - 7)", "ldexp(1.0 + mant / 8.0, e - 8)"),
    "e4m3_round_trunc": ("int mant = (int)nearbyint((2.0 * f - 1.0) * 8.0);",
                         "int mant = (int)floor((2.0 * f - 1.0) * 8.0);"),
    "e4m3_no_saturation": ("    if (a > 448.0)\n        a = 448.0;", "    if (a > 480.0)\n        a = 480.0;"),
    "fp8_scale_ignored": ("return or_e4m3_to_f64(or_f64_to_e4m3(val / sc)) * sc;",
                          "return or_e4m3_to_f64(or_f64_to_e4m3(val));"),
    "out_gate_sign": ("m->att[i] *= 1.0 / (1.0 + exp(-m->o[i]));", "m->att[i] *= 1.0 / (1.0 + exp(m->o[i]));"),
    "out_gate_input": ("or_gemv_q4_0(&L->wag, m->h, m->o, nt);", "or_gemv_q4_0(&L->wag, m->x, m->o, nt);"),
    "lm_head_is_embed": ("or_gemv_q4_0(&m->lm_head, m->h, logits, nt);",
                         "or_gemv_q4_0(&m->embed, m->h, logits, nt);"),
    "model_rope_q_full_width": ("or_rope_neox(m->q + hh * hd, (int32_t)hd, c->rot_dim, c->inv_freq, pos);",
                                "or_rope_neox(m->q + hh * hd, (int32_t)hd, (int32_t)hd, c->inv_freq, pos);"),
    "model_rope_k_half_width": ("or_rope_neox(m->k + gg * hd, (int32_t)hd, c->rot_dim, c->inv_freq, pos);",
                                "or_rope_neox(m->k + gg * hd, (int32_t)hd, c->rot_dim / 2, c->inv_freq, pos);"),
    "model_rope_pos": ("or_rope_neox(m->q + hh * hd, (int32_t)hd, c->rot_dim, c->inv_freq, pos);",
                       "or_rope_neox(m->q + hh * hd, (int32_t)hd, c->rot_dim, c->inv_freq, pos + 1);"),
}


def _run_pins(lib_path):
    env = dict(os.environ, QD_ORACLE_LIB=lib_path)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PINS], env=env, cwd=ROOT, capture_output=True, text=True, timeout=600)
    return r.returncode


@pytest.fixture(scope="module")
def workdir(tmp_path_factory):
    return tmp_path_factory.mktemp("mutants")


def test_unmodified_copy_passes(workdir):
    src = open(SRC).read()
    p = workdir / "orig.c"
    p.write_text(src)
    lib = obuild.compile_source(str(p), str(workdir / "orig.so"))
    assert _run_pins(lib) == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(workdir, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    p = workdir / f"{name}.c"
    p.write_text(src.replace(old, new, 1))
    lib = obuild.compile_source(str(p), str(workdir / f"{name}.so"))
    assert _run_pins(lib) != 0, f"pins did not catch mutant {name}"
