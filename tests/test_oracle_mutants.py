"""Plant plausible mistakes in copies of the CPU oracle and check that the
pins (test_oracle_pins.py, test_oracle_attention_pins.py,
test_oracle_xpos_pins.py) catch every one.

Each mutant is one textual change of rope_oracle.c (which must match exactly
once), compiled with gcc into a temporary library and run under the pin suite
via the ROPE_ORACLE_LIB override. Everything here runs on the CPU.
"""
import concurrent.futures as cf
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "rope_oracle.c")

MUTANTS = {
    "rotation_sign_y1": ("double y1 = x1 * c - x2 * sn;", "double y1 = x1 * c + x2 * sn;"),
    "rotation_sign_y2": ("double y2 = x1 * sn + x2 * c;", "double y2 = -x1 * sn + x2 * c;"),
    "dropped_term": ("double y2 = x1 * sn + x2 * c;", "double y2 = x2 * c;"),
    "transposed_operands": ("double y2 = x1 * sn + x2 * c;", "double y2 = x2 * sn + x1 * c;"),
    "cos_sin_swapped": ("double c = c32, sn = (double)direction * (double)s32;",
                        "double c = s32, sn = (double)direction * (double)c32;"),
    "backward_ignores_direction": ("double c = c32, sn = (double)direction * (double)s32;",
                                   "double c = c32, sn = (double)s32;"),
    "split_pair_offset": ("*j2 = i + R / 2;", "*j2 = R - 1 - i;"),
    "interleaved_pair": ("*j1 = 2 * i;\n    *j2 = 2 * i + 1;", "*j1 = 2 * i + 1;\n    *j2 = 2 * i;"),
    "freq_exponent_index": ("double expo = -(2.0 * (double)i) / (double)rotary_dim;",
                            "double expo = -(2.0 * (double)(i + 1)) / (double)rotary_dim;"),
    "freq_exponent_scale": ("double expo = -(2.0 * (double)i) / (double)rotary_dim;",
                            "double expo = -(1.0 * (double)i) / (double)rotary_dim;"),
    "position_off_by_one": ("int64_t p = pos ? (int64_t)pos[b * pos_batch_stride + s] : s;",
                            "int64_t p = pos ? (int64_t)pos[b * pos_batch_stride + s] : s + 1;"),
    "batch_stride_ignored": ("int64_t p = pos ? (int64_t)pos[b * pos_batch_stride + s] : s;",
                             "int64_t p = pos ? (int64_t)pos[s] : s;"),
    "table_bound_unchecked": ("if (p < 0 || p >= table_rows) return -1;",
                              "if (p < 0) return -1;"),
    "bshd_offset": ("return ((b * S + s) * H + h) * D;                          /* [B,S,H,D] */",
                    "return ((b * H + h) * S + s) * D;"),
    "round_toward_zero": ("return ldexp(nearbyint(ldexp(y, -q)), q);",
                          "return ldexp(trunc(ldexp(y, -q)), q);"),
    "no_gradual_underflow": ("if (lead < emin) lead = emin;", ";"),
    "f16_subnormal_scale": ("return sign | (uint16_t)ldexp(r, 24);",
                            "return sign | (uint16_t)ldexp(r, 23);"),
    "bf16_decode": ("uint32_t w = (uint32_t)h << 16;", "uint32_t w = (uint32_t)h << 15;"),
    "table_unrounded_cos": ("*c32 = (float)cos(angle);", "*c32 = (float)cos(angle * 1.0000001);"),
    "exact_mode_sign": ("y[row + j1] = x1 * c - x2 * sn;", "y[row + j1] = x1 * c + x2 * sn;"),
    "exact_mode_pairs_crossed": ("double x1 = y[row + j1], x2 = y[row + j2];",
                                 "double x1 = y[row + j2], x2 = y[row + j1];"),
    "interp_multiplies": ("return ((double)p / interp) * oracle_freq(theta, rotary_dim, i);",
                          "return ((double)p * interp) * oracle_freq(theta, rotary_dim, i);"),
    "interp_ignored": ("return ((double)p / interp) * oracle_freq(theta, rotary_dim, i);",
                       "return (double)p * oracle_freq(theta, rotary_dim, i);"),
    "attn_no_scale": ("            w[j] = scale * dot;", "            w[j] = dot;"),
    "attn_causal_off_by_one": ("int64_t last = causal ? i + (Sk - Sq) : Sk - 1;",
                               "int64_t last = causal ? i + (Sk - Sq) - 1 : Sk - 1;"),
    "attn_gqa_map": ("int64_t hk = h / (Hq / Hk);", "int64_t hk = h % Hk;"),
    "attn_k_unrotated": ("rc = oracle_rope(k, kr, dtype, ORC_BHSD, pairing, 1,",
                         "rc = oracle_rope(k, kr, dtype, ORC_BHSD, pairing, -1,"),
    "attn_values_from_keys": ("acc += w[j] * load_elem(v, ", "acc += w[j] * load_elem(kr, "),
    "attn_query_offset": ("qp[i] = (int32_t)(i + Sk - Sq);", "qp[i] = (int32_t)i;"),
    "pass_through_dims_rotated": ("for (int64_t i = 0; i < R / 2; ++i) {\n          float c32, s32;",
                                  "for (int64_t i = 0; i < D / 2; ++i) {\n          float c32, s32;"),
    "xpos_key_sign": ("return pow(oracle_xpos_zeta(gamma, rotary_dim, i), is_key ? -e : e);",
                      "return pow(oracle_xpos_zeta(gamma, rotary_dim, i), e);"),
    "xpos_second_unscaled": ("store_elem(y, row + jb, dtype, (a1 * sg + a2 * cs) * f32);",
                             "store_elem(y, row + jb, dtype, (a1 * sg + a2 * cs));"),
    "xpos_zeta_over_r": ("return ((double)i / ((double)rotary_dim / 2.0) + gamma) / (1.0 + gamma);",
                         "return ((double)i / (double)rotary_dim + gamma) / (1.0 + gamma);"),
    "xpos_center_ignored": ("double e = ((double)p - center) / scale_base;",
                            "double e = (double)p / scale_base;"),
    "xpos_exact_unscaled": ("y[row + ja] = (a1 * cs - a2 * sg) * f;",
                            "y[row + ja] = (a1 * cs - a2 * sg);"),
}


def _run_mutant(name, old, new, tmp):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutant {name}: pattern must occur exactly once"
    path = os.path.join(tmp, f"{name}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(tmp, f"lib{name}.so")
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                    "-o", lib, path, "-lm"], check=True)
    env = dict(os.environ, ROPE_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_attention_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_xpos_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return name, r.returncode, r.stdout[-2000:]


def test_every_planted_mistake_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with cf.ThreadPoolExecutor(max_workers=4) as ex:
            futs = [ex.submit(_run_mutant, n, o, w, tmp) for n, (o, w) in MUTANTS.items()]
            results = [f.result() for f in futs]
    survivors = [(n, out) for n, rc, out in results if rc == 0]
    assert not survivors, "mutants not caught by any pin: " + ", ".join(n for n, _ in survivors)


def test_unmutated_oracle_passes_under_override():
    """Control: the override path itself does not make the pins fail."""
    with tempfile.TemporaryDirectory() as tmp:
        name, rc, out = _run_mutant("control", "#include <math.h>", "#include <math.h>", tmp)
    assert rc == 0, out
