"""The oracle's pins must catch plausible mistakes in the oracle (CPU only).

Each case copies oracle.c, plants one mistake in the copy (a dropped or
misplaced bias, an off-by-one window or chunk edge, a reversed causal mask, a
wrong slot or head in the block-table gather, a wrong query position, a
transposed bias index, a sign error in the softmax, a missing normalisation),
builds it with gcc in a temporary directory and runs tests/test_oracle_pins.py
against that build in a subprocess (PA_ORACLE_LIB points the oracle package at
it). The pins must fail for every mutant. A control build of the unmodified
source must pass, so a broken harness cannot make the mutants fail by itself.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# (name, text in oracle.c, replacement); every occurrence is replaced
MUTANTS = [
    ("bias_after_scale", "s[j] = (dot + a) * scale;", "s[j] = dot * scale + a;"),
    ("bias_dropped", "double a = bias_row ? (double)bias_row[j] : 0.0;", "double a = 0.0;"),
    ("window_edge_inclusive", "if (d >= window) return 0;", "if (d > window) return 0;"),
    ("causal_reversed", "if (causal && j > p) return 0;", "if (causal && j < p) return 0;"),
    ("slot_off_by_one", "int64_t slot = j % block_size;",
     "int64_t slot = (j + 1) % block_size;"),
    ("head_ignored", "return ((phys * num_heads + h) * block_size + slot) * head_dim;",
     "return ((phys * num_heads + 0) * block_size + slot) * head_dim;"),
    ("prefill_query_position", "int32_t p = L - nq + t;", "int32_t p = t;"),
    ("softmax_sign", "double w = exp(s[j] - m);", "double w = exp(m - s[j]);"),
    ("chunk_edge_shifted", "if (chunk > 0 && j / chunk != p / chunk) return 0;",
     "if (chunk > 0 && (j + 1) / chunk != (p + 1) / chunk) return 0;"),
    ("chunk_ignored", "if (chunk > 0 && j / chunk != p / chunk) return 0;", ""),
    ("bias_transposed",
     "attn_bias ? attn_bias + ((int64_t)b * num_heads + h) * max_seq_len : NULL;",
     "attn_bias ? attn_bias + ((int64_t)h * num_seqs + b) * max_seq_len : NULL;"),
    ("not_normalised", "for (int32_t d = 0; d < head_dim; ++d) out_row[d] /= z;", ""),
]


def build_and_run_pins(tmp_path, name, source):
    c = tmp_path / ("%s.c" % name)
    c.write_text(source)
    so = tmp_path / ("lib%s.so" % name)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", str(so),
                    str(c), "-I", os.path.join(ROOT, "oracle"), "-lm"], check=True)
    env = dict(os.environ, PA_ORACLE_LIB=str(so))
    return subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-m", "not gpu",
                           "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True,
                          text=True, timeout=600)


def test_pins_pass_on_an_unmodified_build(tmp_path):
    r = build_and_run_pins(tmp_path, "control", open(SRC).read())
    assert r.returncode == 0, r.stdout[-2000:]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    src = open(SRC).read()
    assert old in src, "mutation anchor not found: %s" % old
    r = build_and_run_pins(tmp_path, name, src.replace(old, new))
    assert r.returncode != 0, "the pins did not notice mutation %s" % name
    assert "failed" in r.stdout or "Error" in r.stdout, r.stdout[-2000:]
