"""Pin strength: each plausible mistake planted in a copy of the oracle (on
the CPU, in a temporary directory) must make at least one pin fail."""
import os
import subprocess

import pytest

import oracle
from pins import PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "moda_oracle.c")

# (name, text in moda_oracle.c, replacement, how many occurrences to replace)
MUTANTS = [
    ("no_scale", "const double s = 1.0 / sqrt((double)d);", "const double s = 1.0;", 1),
    ("scale_1_over_d", "const double s = 1.0 / sqrt((double)d);",
     "const double s = 1.0 / (double)d;", 1),
    ("diag_value_dropped", "for (int64_t j = 0; j <= t; ++j) acc +=",
     "for (int64_t j = 0; j < t; ++j) acc +=", 1),
    ("gqa_modulo", "const int64_t g = h / G;", "const int64_t g = h % Hkv;", 2),
    ("gqa_modulo_weights", "const int64_t g = h / (Hq / Hkv);", "const int64_t g = h % Hkv;", 1),
    ("depth_prev_token", "((b * Hkv + g) * T + t) * L * d,",
     "((b * Hkv + g) * T + (t > 0 ? t - 1 : 0)) * L * d,", 1),
    ("depth_values_dropped", "acc += x[t + 1 + i] * elem(vd,", "acc += 0.0 * elem(vd,", 1),
    ("depth_logit_from_values", "x[t + 1 + i] = s * dot(q, q_off, kd,",
     "x[t + 1 + i] = s * dot(q, q_off, vd,", 1),
    ("depth_entry_index", "x[t + 1 + i] = s * dot(q, q_off, kd, dep_off + i * d,",
     "x[t + 1 + i] = s * dot(q, q_off, kd, dep_off,", 1),
    ("no_normalise", "for (int64_t nn = 0; nn < n; ++nn) x[nn] /= Z;", "", 1),
    ("no_max_shift", "x[nn] = exp(x[nn] - m);", "x[nn] = exp(x[nn]);", 1),
    ("lse_no_max", "if (lse) *lse = m + log(Z);", "if (lse) *lse = log(Z);", 1),
    ("seq_keys_head0", "(b * Hkv + g) * T * d, kd", "(b * Hkv) * T * d, kd", 1),
    ("bf16_shift", "<< 16;", "<< 15;", 1),
    ("depth_sign", "x[t + 1 + i] = s * dot(", "x[t + 1 + i] = -s * dot(", 1),
    ("value_from_key", "acc += x[j] * elem(v,", "acc += x[j] * elem(k,", 1),
    # standalone depth attention
    ("depth_only_no_scale", "const double sd = 1.0 / sqrt((double)d);", "const double sd = 1.0;",
     1),
    ("depth_only_prev_token", "const int64_t own = ((b * Hkv + h / grp) * T + t) * L * d;",
     "const int64_t own = ((b * Hkv + h / grp) * T + (t > 0 ? t - 1 : 0)) * L * d;", 1),
    ("depth_only_head_modulo", "(b * Hkv + h / grp)", "(b * Hkv + h % Hkv)", 1),
    ("depth_only_no_max_shift", "c[i] = exp(c[i] - mx);", "c[i] = exp(c[i]);", 1),
    ("depth_only_values_from_keys", "elem(vd, own + i * d + col, dtype)",
     "elem(kd, own + i * d + col, dtype)", 1),
    ("depth_only_lse_no_max", "if (lse) lse[r] = mx + log(Zd);", "if (lse) lse[r] = log(Zd);",
     1),
    ("depth_only_unnormalised", "acc += (c[i] / Zd) *", "acc += c[i] *", 1),
    # backward
    ("bwd_no_D", "const double ds = x[nn] * (dp - D);", "const double ds = x[nn] * dp;", 1),
    ("bwd_dq_no_scale", "dq[r * d + c] += s * ds *", "dq[r * d + c] += ds *", 1),
    ("bwd_dkey_no_scale", "dkey[c] += s * ds *", "dkey[c] += ds *", 1),
    ("bwd_dval_from_ds", "dval[c] += x[nn] *", "dval[c] += ds *", 1),
    ("bwd_group_head0", "h < (bg % Hkv + 1) * G; ++h)", "h < (bg % Hkv) * G + 1; ++h)", 1),
    ("bwd_depth_prev_token", "const int64_t dep_off = (bg * T + t) * L * d;",
     "const int64_t dep_off = (bg * T + (t > 0 ? t - 1 : 0)) * L * d;", 1),
    ("bwd_D_from_dout_only", "D += elem(dout, r * d + c, dtype) * o[c];",
     "D += elem(dout, r * d + c, dtype);", 1),
]


@pytest.fixture(scope="module")
def src_text():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, src_text, name, old, new, count):
    assert src_text.count(old) >= count, f"mutation site for {name} not found"
    mutated = src_text.replace(old, new, count)
    c_path = tmp_path / f"mut_{name}.c"
    c_path.write_text(mutated)
    so_path = str(tmp_path / f"libmut_{name}.so")
    oracle.build(str(c_path), so_path)
    lib = oracle.load(so_path)
    failed = []
    for pname, pin in PINS:
        try:
            pin(lib)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pname)
    assert failed, f"mutant {name} passed every pin"
