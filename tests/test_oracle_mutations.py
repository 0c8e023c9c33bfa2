"""The oracle's pins catch plausible mistakes in it.

Each case plants one mistake in a copy of the oracle's C source (on the CPU
only), builds that copy apart, and runs the pin suites against it in a child
process: they must fail.  The unaltered oracle passes the same suites (the rest
of the CPU test run), so a case that passes here means a part of the oracle no
pin constrains.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

ATTN_SUM = "x[i] = orc_round(x[i] + orc_round(t[i], dt), dt);"

# (name, original text, planted mistake); each original text occurs once
MUTATIONS = [
    ("causal_row_misses_own_key", "causal_base + r + 1)", "causal_base + r + (r == 0 ? 1 : 0))"),
    ("capture_before_layer",
     "        decoder_layer(m, l, x, n, pos, &ks, &vs, ck + pos0 * NK, cv + pos0 * NK, 1, pos0, tree_vis);\n"
     "        if (capture && hidden_out)\n"
     "            for (int s = 0; s < 5; ++s)\n"
     "                if (capture[s] == l)\n"
     "                    memcpy(hidden_out + (int64_t)s * n * H, x, sizeof(double) * (size_t)n * H);",
     "        if (capture && hidden_out)\n"
     "            for (int s = 0; s < 5; ++s)\n"
     "                if (capture[s] == l)\n"
     "                    memcpy(hidden_out + (int64_t)s * n * H, x, sizeof(double) * (size_t)n * H);\n"
     "        decoder_layer(m, l, x, n, pos, &ks, &vs, ck + pos0 * NK, cv + pos0 * NK, 1, pos0, tree_vis);"),
    ("fusion_output_not_rounded", "i < (int64_t)nrows * H; ++i) y[i] = orc_round(y[i], dt);",
     "i < (int64_t)nrows * H; ++i) y[i] = y[i];"),
    ("rope_sign", "v[i] = a * c - b * s;", "v[i] = a * c + b * s;"),
    ("rope_query_position_off_by_one", "orc_rope(q + r * NQ + (int64_t)h * d, d, pos[r], m->rope_base);",
     "orc_rope(q + r * NQ + (int64_t)h * d, d, pos[r] + 1, m->rope_base);"),
    ("swiglu_operands_swapped", "silu(a[i]) * b[i]", "a[i] * silu(b[i])"),
    ("gqa_interleaved_heads", "const int32_t g = h / group;", "const int32_t g = h % (nq / group);"),
    ("argmax_ties_to_highest_id", "if (f > best) { second = best;", "if (f >= best) { second = best;"),
    ("final_norm_dropped",
     "for (int32_t r = 0; r < R; ++r) orc_rmsnorm(x + (int64_t)r * H, H, m->final_norm, dt, m->eps, z + (int64_t)r * H);",
     "for (int64_t i = 0; i < (int64_t)R * H; ++i) z[i] = x[i];"),
    ("accept_compares_wrong_target", "while (n < B - 1 && d[n + 1] == g[n]) ++n;",
     "while (n < B - 1 && d[n + 1] == g[n + 1]) ++n;"),
    ("softmax_scale_1_over_d", "const double scale = 1.0 / sqrt((double)d);", "const double scale = 1.0 / (double)d;"),
    ("attention_residual_dropped", "matvec_rows(m->wo[l], dt, H, NQ, o, R, t);\n    for (int64_t i = 0; i < (int64_t)R * H; ++i) " + ATTN_SUM,
     "matvec_rows(m->wo[l], dt, H, NQ, o, R, t);\n    for (int64_t i = 0; i < (int64_t)R * H; ++i) x[i] = orc_round(t[i], dt);"),
]


@pytest.mark.parametrize("name,before,after", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, name, before, after):
    src = open(oracle._SRC).read()
    assert src.count(before) == 1, f"{name}: the text to alter is not unique in the oracle source"
    mutant = tmp_path / "dflash_oracle_mutant.c"
    mutant.write_text(src.replace(before, after))
    lib = oracle.build(src=str(mutant), out=str(tmp_path / "liboracle_mutant.so"))
    env = dict(os.environ, DFLASH_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py", "tests/test_oracle_ddtree.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    # exit status 1: tests ran and at least one failed (not a collection or usage error)
    assert r.returncode == 1, f"{name}: no pin failed (exit {r.returncode})\n{r.stdout[-3000:]}\n{r.stderr[-2000:]}"
