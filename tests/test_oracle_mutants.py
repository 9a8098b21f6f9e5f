"""Plant plausible mistakes in a copy of the oracle's C source and check that a pin catches each one.

Every mutant is built with gcc into a temporary directory and run through all pins; the test passes
only if at least one pin fails for it. The real oracle is never modified.
"""
import os
import subprocess

import pytest

import oracle as oracle_pkg
import oracle_pins as pins

# (name, [(original text, planted mistake), ...]) -- each original must occur exactly once in the source
MUTANTS = [
    ("router_drops_bias", [("acc = acc + bias[j];", "acc = acc + 0.0f * bias[j];")]),
    ("router_transposed_weight", [("x[k] * Wr[k * E + j]", "x[k] * Wr[j * dm + k]")]),
    ("router_highest_index_on_ties", [("if (best < 0 || l[j] > l[best]) best = j;",
                                       "if (best < 0 || l[j] >= l[best]) best = j;")]),
    ("softmax_drops_a_term", [("for (int32_t j = 0; j < E; ++j)\n            denom +=",
                               "for (int32_t j = 1; j < E; ++j)\n            denom +=")]),
    ("softmax_renormalised_over_selection",
     [("prob[t * K + s] = (float)(exp((double)l[best] - (double)lmax) / denom);",
       "prob[t * K + s] = (float)(exp((double)l[best] - (double)lmax) / exp((double)l[ids[t * K]] - (double)lmax));")]),
    ("gap_sign", [("gap[t] = next < 0 ? INFINITY : last - l[next];", "gap[t] = next < 0 ? INFINITY : l[next] - last;")]),
    ("sort_inclusive_offsets", [("offsets[e + 1] = offsets[e] + counts[e];",
                                 "offsets[e + 1] = offsets[e] + counts[e] + (e == 0);")]),
    ("sort_perm_inverse_swapped", [("inv_perm[a] = pos;", "inv_perm[pos] = (int32_t)a;")]),
    ("sort_reverse_order_within_expert", [("next[e] = offsets[e];", "next[e] = offsets[e + 1];"),
                                          ("int32_t pos = next[ids[a]]++;", "int32_t pos = --next[ids[a]];")]),
    ("in_proj_transposed_weight", [("const float *wc = Wc + (i * di + c) * dm;", "const float *wc = Wc + i * di * dm + c;"),
                                   ("hx += (double)x[k] * (double)wc[k];", "hx += (double)x[k] * (double)wc[k * di];")]),
    ("in_proj_gate_uses_conv_weight", [("hz += (double)x[k] * (double)wg[k];", "hz += (double)x[k] * (double)wc[k];")]),
    ("in_proj_only_first_expert",
     [("for (int32_t s = 0; s < K; ++s) {\n                const int64_t i = ids[t * K + s];\n                const float *wc",
       "for (int32_t s = 0; s < 1; ++s) {\n                const int64_t i = ids[t * K + s];\n                const float *wc")]),
    ("in_proj_dropped_term", [("for (int64_t k = 0; k < dm; ++k) {\n                    hx +=",
                               "for (int64_t k = 1; k < dm; ++k) {\n                    hx +=")]),
    ("silu_sign", [("a[c] = v / (1.0 + exp(-v)) * (double)h[t * di + c];",
                    "a[c] = v / (1.0 + exp(v)) * (double)h[t * di + c];")]),
    ("silu_missing", [("a[c] = v / (1.0 + exp(-v)) * (double)h[t * di + c];", "a[c] = v * (double)h[t * di + c];")]),
    ("out_proj_unscaled", [("o += (double)prob[t * K + s] * acc;", "o += acc;")]),
    ("out_proj_transposed_weight", [("const float *wo = Wo + (i * dm + m) * di;", "const float *wo = Wo + i * dm * di + m;"),
                                    ("acc += a[c] * (double)wo[c];", "acc += a[c] * (double)wo[c * dm];")]),
    ("weighted_in_proj_unscaled", [("yc += (double)prob[t * K + s] * stream;", "yc += stream;")]),
    ("weighted_in_proj_only_first_expert",
     [("for (int32_t s = 0; s < K; ++s) {\n                const int64_t i = ids[t * K + s];\n                const float *w ",
       "for (int32_t s = 0; s < 1; ++s) {\n                const int64_t i = ids[t * K + s];\n                const float *w ")]),
    ("weighted_in_proj_transposed_weight", [("const float *w = W + (i * dout + c) * dm;", "const float *w = W + i * dout * dm + c;"),
                                            ("stream += (double)x[k] * (double)w[k];",
                                             "stream += (double)x[k] * (double)w[k * dout];")]),
    ("conv1d_anticausal_taps", [("const int64_t s = t - (w - 1) + j;", "const int64_t s = t - j;")]),
    # reads the previous sequence's last tokens instead of zeros
    ("conv1d_crosses_sequences", [("if (s < 0) continue;", "if (b * L + s < 0) continue;")]),
    ("conv1d_drops_bias", [("double u = bias ? (double)bias[c] : 0.0;", "double u = 0.0;")]),
    ("conv1d_silu_sign", [("y[bt * C + c] = act ? u / (1.0 + exp(-u)) : u;", "y[bt * C + c] = act ? u / (1.0 + exp(u)) : u;")]),
    ("conv1d_drops_oldest_tap", [("for (int32_t j = 0; j < w; ++j) {\n                const int64_t s",
                                  "for (int32_t j = 1; j < w; ++j) {\n                const int64_t s")]),
    ("dsilu_drops_second_term", [("(sg * (1.0 + v * (1.0 - sg)))", "(sg)")]),
    ("dh_uses_z_not_silu", [("dh[t * di + c] = da * (v * sg);", "dh[t * di + c] = da * v;")]),
    ("out_dgrad_unscaled", [("da += (double)prob[t * K + s] * col;", "da += col;")]),
    ("out_dgrad_transposed_weight", [("col += (double)Wo[(i * dm + m) * di + c] * (double)g[t * dm + m];",
                                      "col += (double)Wo[(i * di + c) * dm + m] * (double)g[t * dm + m];")]),
    ("out_wgrad_unscaled", [("acc += (double)prob[t * K + s] * (double)g[t * dm + m] * a;",
                             "acc += (double)g[t * dm + m] * a;")]),
    ("in_dgrad_drops_gate", [("acc += (double)Wc[(i * di + c) * dm + k] * (double)dx[t * di + c]\n"
                              "                         + (double)Wg[(i * di + c) * dm + k] * (double)dzg[t * di + c];",
                              "acc += (double)Wc[(i * di + c) * dm + k] * (double)dx[t * di + c];")]),
    ("in_wgrad_gate_uses_dx", [("dWg[q] = in_wgrad_entry(X, dzg,", "dWg[q] = in_wgrad_entry(X, dx,")]),
    ("in_wgrad_transposed", [("acc += (double)dy[t * di + c] * (double)X[t * dm + k];",
                              "acc += (double)dy[t * di + k % di] * (double)X[t * dm + c % dm];")]),
]


def _source():
    with open(oracle_pkg.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, edits):
    src = _source()
    for orig, planted in edits:
        assert src.count(orig) == 1, f"mutation site for {name} not unique/present: {orig!r}"
        src = src.replace(orig, planted)
    path = os.path.join(tmp_path, "rom_oracle_mutant.c")
    with open(path, "w") as f:
        f.write(src)
    lib = oracle_pkg.build(path, os.path.join(tmp_path, "liborom_mutant.so"))
    orc = oracle_pkg.Oracle(lib)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, IndexError) as exc:  # a pin (or the wrapper's checks) rejects it
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, f"no pin catches the planted mistake {name}"
