"""The oracle's pins have teeth: plausible mistakes planted in copies of the
oracle (on the CPU) must each make the pin suite fail.

Each mutant is one textual change to oracle/rrp_oracle.c, compiled with gcc into
a temporary library that the pin suite loads through RRP_ORACLE_LIB.
"""
import concurrent.futures
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "rrp_oracle.c")

MUTANTS = {
    "rope_sign": ("*ob = b * c + a * s;", "*ob = b * c - a * s;"),
    "rope_pair_index": ("*hi = k + head_dim / 2;", "*hi = head_dim - 1 - k;"),
    "inv_freq_exponent": ("-2.0 * (double)k / (double)head_dim", "-2.0 * (double)k / (double)(head_dim - 2)"),
    "hadamard_unnormalised": ("out[blk + i] = acc * norm;", "out[blk + i] = acc;"),
    "hadamard_sign_pattern": ("parity_bit((unsigned)(i & m))", "parity_bit((unsigned)(i | m))"),
    "round_half_up": ("double r = rint(y[i] / shv);", "double r = floor(y[i] / shv + 0.5);"),
    "qmax_8": ("float s = (float)(m / 7.0);", "float s = (float)(m / 8.0);"),
    "codes_use_fp32_scale": ("double shv = orc_f16_value(sh);", "double shv = (double)s;"),
    "nibble_order": ("bytes[i] = (uint8_t)(((unsigned)q[2 * i] & 0xFu) | (((unsigned)q[2 * i + 1] & 0xFu) << 4));",
                     "bytes[i] = (uint8_t)(((unsigned)q[2 * i + 1] & 0xFu) | (((unsigned)q[2 * i] & 0xFu) << 4));"),
    "angle_sign": ("phi = 0.5 * atan2(a - b, 2.0 * c);", "phi = 0.5 * atan2(b - a, 2.0 * c);"),
    "angle_uncentred": ("a = E[2] - E[0] * E[0];", "a = E[2];"),
    "default_is_balanced": ("if (estimator == ORC_EST_STREAM_BALANCED && use_q && use_k) {", "if (use_q && use_k) {"),
    "pair_rotation_transposed": ("rotate2(x[lo], x[hi], cos(phi), sin(phi), &a, &b);",
                                 "rotate2(x[lo], x[hi], cos(phi), -sin(phi), &a, &b);"),
    "pair_rotation_dropped": ("orc_hadamard_blocks(p, head_dim, b, out);", "orc_hadamard_blocks(r, head_dim, b, out); (void)p;"),
    "f16_round_half_up": ("return rint(a / quantum) * quantum;", "return trunc(a / quantum + 0.5) * quantum;"),
    "stats_range_max_only": ("sum_range += hi - lo;", "sum_range += hi;"),
    "v_half_head_hadamard": ("orc_hadamard_blocks(x, d, d, y);", "orc_hadamard_blocks(x, d, d / 2, y);"),
    "v_scale_at_token_not_slot": ("if (in_cache) v_scales[(slot * hk + h) * ng + j] = sh;",
                                  "if (in_cache) v_scales[(t * hk + h) * ng + j] = sh;"),
    "decode_gqa_interleaved": ("const int kv = (int)((int64_t)h * hk / hq);", "const int kv = h % hk;"),
    "decode_one_scale_per_row": ("orc_f16_value(srow[c / group])", "orc_f16_value(srow[0])"),
    "per_head_query_groups_interleaved": ("return s->n_q_heads > 0 ? (int)((int64_t)h * angle_groups(s) / s->n_q_heads) : 0;",
                                          "return h % angle_groups(s);"),
}


def _run_mutant(name, tmpdir):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert before in src, f"mutant {name}: pattern not found"
    csrc = os.path.join(tmpdir, name + ".c")
    so = os.path.join(tmpdir, name + ".so")
    with open(csrc, "w") as f:
        f.write(src.replace(before, after, 1))
    subprocess.run(["gcc", "-O2", "-std=gnu11", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                    "-I", os.path.join(ROOT, "oracle"), csrc, "-o", so, "-lm"], check=True)
    env = dict(os.environ, RRP_ORACLE_LIB=so, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        "-x", "-q", "-p", "no:warnings", "-p", "no:cacheprovider"],
                       env=env, cwd=ROOT, capture_output=True, text=True)
    return name, r.returncode


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with concurrent.futures.ThreadPoolExecutor(max_workers=max(2, min(8, os.cpu_count() or 2))) as ex:
        results = list(ex.map(lambda n: _run_mutant(n, str(tmp_path)), MUTANTS))
    survivors = [n for n, rc in results if rc == 0]
    assert not survivors, f"mutants not caught by any pin: {survivors}"
    assert all(rc == 1 for _, rc in results), results
