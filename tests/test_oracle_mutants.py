"""Planted mistakes in the oracle must fail its pins.

Each case copies ``oracle/q8_oracle.c``, plants one plausible mistake (a
dropped term, a wrong sign or index, a transposed operand, another tie rule),
builds it on the CPU and runs ``tests/test_oracle_pins.py`` against that
library in a child process.  The pins pass on the real oracle (its own test
run) and must fail on every mutant.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "q8_oracle.c")

MUTANTS = {
    "drop_last_byte_of_block": ("for (int t = 0; t < Q8_BLOCK; ++t) s +=",
                                "for (int t = 0; t < Q8_BLOCK - 1; ++t) s +="),
    "unsigned_bytes": ("s += (int32_t)a[t] * (int32_t)w[t];",
                       "s += (int32_t)(uint8_t)a[t] * (int32_t)w[t];"),
    "reversed_activation_scale_block": ("(double)AS[i * KB + b]",
                                        "(double)AS[i * KB + (KB - 1 - b)]"),
    "weight_scale_from_activation_row": ("(double)WS[j * KB + b]",
                                         "(double)WS[i * KB + b]"),
    "subtract_odd_blocks": ("acc += term;", "acc += (b & 1) ? -term : term;"),
    "signed_abs_terms": ("mag += fabs(term);", "mag += term;"),
    "ties_away_from_zero": ("rintf(xb[t] / scale)", "roundf(xb[t] / scale)"),
    "scale_over_128": ("amax / 127.0f", "amax / 128.0f"),
    "reciprocal_multiply": ("rintf(xb[t] / scale)", "rintf(xb[t] * (1.0f / scale))"),
    "q50_qh_bit_order_reversed": ("(((qh >> e) & 1u) << 4)", "(((qh >> (31 - e)) & 1u) << 4)"),
    "q50_nibbles_swapped": ("e < 16 ? (byte & 0x0Fu) : (byte >> 4)", "e < 16 ? (byte >> 4) : (byte & 0x0Fu)"),
    "q50_no_offset": ("return (int32_t)q - 16;", "return (int32_t)q;"),
    "q50_qh_big_endian": ("const uint32_t qh = (uint32_t)blk[0] | ((uint32_t)blk[1] << 8) |",
                          "const uint32_t qh = (uint32_t)blk[3] | ((uint32_t)blk[2] << 8) | 0u * blk[0] |"),
    "qmma_scale_not_transposed": ("(double)WST[b * N + j]", "(double)WST[j * KB + b]"),
    "q50_sampled_column_misindexed": ("q50_one(A, AS, W5, WS, ws_t, ii[s], jj[s], N, K, out + s, abs_terms + s);",
                                      "q50_one(A, AS, W5, WS, ws_t, ii[s], jj[count - 1 - s], N, K, out + s, abs_terms + s);"),
    "transposed_weight_operand": ("W + j * K + b * Q8_BLOCK);\n        double s",
                                  "W + (j % 1) * K + b * Q8_BLOCK);\n        double s"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert old in src, "mutation anchor not found: %s" % name
    mutated = src.replace(old, new)
    c_path = tmp_path / "mutant.c"
    c_path.write_text(mutated)
    so_path = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-shared",
                    "-fPIC", "-o", str(so_path), str(c_path), "-lm"], check=True)
    env = dict(os.environ, Q8_ORACLE_LIB=str(so_path))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, "pins did not catch mutant %s:\n%s" % (name, r.stdout[-2000:])
