"""CPU tests: the pins are sensitive.  Each case plants one plausible mistake
in a private copy of the oracle source (a dropped term, a wrong index or
sign, a transposed operand, the wrong log base, an off-by-one mask), builds
it into a temporary library, and checks that the pin battery rejects it.
The real oracle is never modified."""
import os

import pytest

import oracle
from pins import ALL_PINS
from pins_bwd import ALL_BWD_PINS

# the end of fa_oracle_attention's row loop (the masked routine ends its
# rows with the same two statements, then frees a second buffer)
_DENSE_END = "\n        }\n        free(w);\n    }"

MUTATIONS = {
    "drop_scale": ("w[j] = scale * dot;", "w[j] = dot;"),
    "diagonal_hidden": ("return (i + 1 < Nk) ? i + 1 : Nk;", "return (i < Nk) ? i : Nk;"),
    "log2_lse": ("lse[t] = m + log(l);" + _DENSE_END, "lse[t] = m + log2(l);" + _DENSE_END),
    "lse_without_max": ("lse[t] = m + log(l);" + _DENSE_END, "lse[t] = log(l);" + _DENSE_END),
    "no_normalisation": ("oi[d] /= l;\n            lse[t] = m + log(l);" + _DENSE_END,
                         "oi[d] /= 1.0;\n            lse[t] = m + log(l);" + _DENSE_END),
    "transposed_values": ("oi[d] += w[j] * vb[j * D + d];",
                          "oi[d] += w[j] * vb[d * Nk + j];"),
    "transposed_keys": ("dot += qi[d] * kb[j * D + d];\n                w[j]",
                        "dot += qi[d] * kb[d * Nk + j];\n                w[j]"),
    "max_not_subtracted": ("w[j] = exp(w[j] - m);", "w[j] = exp(w[j]);"),
    "min_instead_of_max": ("if (w[j] > m)\n                    m = w[j];",
                           "if (w[j] < m || m == -INFINITY)\n                    m = w[j];"),
    "row_index_uses_nk": ("const int64_t i = r % Nq;", "const int64_t i = r % Nk;"),
    "squared_weights_in_sum": ("l += w[j];", "l += w[j] * w[j];"),
    "online_alpha_not_applied_to_acc": ("ar[d] = alpha * ar[d] + pv;", "ar[d] = ar[d] + pv;"),
    "online_alpha_not_applied_to_l": ("l[r] = alpha * l[r] + psum;", "l[r] = l[r] + psum;"),
    "online_mask_direction": ("if (causal && !(i >= j))", "if (causal && !(i <= j))"),
}


_DS_Q = ("const double ds = p * (dp - rd[r]);\n                const double w = fabs(ds) + "
         "p * re[r];\n                for (int64_t d = 0; d < D; ++d) {\n                    gq")
_DS_K = _DS_Q[:-2] + "gv"

# Planted mistakes in the backward pass (fa_oracle_attention_bwd).
BWD_MUTATIONS = {
    "bwd_row_term_without_p": ("}\n                acc += p * dp;", "}\n                acc += dp;"),
    "bwd_dv_without_p": ("gv[d] += p * gi[d];", "gv[d] += gi[d];"),
    "bwd_dk_uses_do": ("gk[d] += ds * qi[d];", "gk[d] += ds * gi[d];"),
    "bwd_dq_uses_v": ("gq[d] += ds * kb[j * D + d];", "gq[d] += ds * vb[j * D + d];"),
    "bwd_dkdv_mask_off_by_one": ("for (int64_t i = causal ? j : 0; i < Nq; ++i)",
                                 "for (int64_t i = causal ? j + 1 : 0; i < Nq; ++i)"),
    "bwd_dq_without_scale": ("gq[d] *= scale;", "gq[d] *= 1.0;"),
    "bwd_dk_without_scale": ("gk[d] *= scale;", "gk[d] *= 1.0;"),
    "bwd_transposed_v_in_row_term": ("dp += gi[d] * vb[j * D + d];\n                    o[d]",
                                     "dp += gi[d] * vb[d * Nk + j];\n                    o[d]"),
    "bwd_dq_row_term_sign": (_DS_Q, _DS_Q.replace("(dp - rd[r])", "(dp + rd[r])")),
    "bwd_dk_row_term_dropped": (_DS_K, _DS_K.replace("(dp - rd[r])", "dp")),
    "bwd_normaliser_squared": ("sum += exp(s[j] - mx);", "sum += exp(2 * (s[j] - mx));"),
    "bwd_dk_score_uses_v": ("dot += qi[d] * kj[d];", "dot += qi[d] * vj[d];"),
}


def _mutated_lib(tmp_path, name, old, new):
    with open(oracle.SOURCE) as f:
        src = f.read()
    assert src.count(old) == 1, f"mutation {name}: pattern must occur exactly once"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = str(tmp_path / f"lib{name}.so")
    oracle.build(out=so, source=str(path), extra_flags=("-w",))
    return oracle.load(so)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(tmp_path, name):
    old, new = MUTATIONS[name]
    lib = _mutated_lib(tmp_path, name, old, new)
    failures = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, RuntimeError, FloatingPointError) as e:
            failures.append((pin.__name__, str(e)[:80]))
    assert failures, f"no pin caught the planted mistake {name!r}"


@pytest.mark.parametrize("name", sorted(BWD_MUTATIONS))
def test_bwd_mutation_is_caught(tmp_path, name):
    old, new = BWD_MUTATIONS[name]
    lib = _mutated_lib(tmp_path, name, old, new)
    failures = []
    for pin in ALL_BWD_PINS:
        try:
            pin(lib)
        except (AssertionError, RuntimeError, FloatingPointError) as e:
            failures.append((pin.__name__, str(e)[:80]))
    assert failures, f"no backward pin caught the planted mistake {name!r}"


def test_unmutated_source_passes_every_pin(tmp_path):
    lib = _mutated_lib(tmp_path, "identity", "int fa_oracle_threads(void)",
                       "int fa_oracle_threads(void)")
    for pin in ALL_PINS + ALL_BWD_PINS:
        pin(lib)
