"""CPU tests: the oracle's local-window + global-token attention against its
pins, and planted mistakes in its visibility rule and in its backward pass."""
import pytest

import oracle
from pins_masked import ALL_MASKED_PINS


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", ALL_MASKED_PINS, ids=lambda p: p.__name__)
def test_masked_pin(pin, lib):
    pin(lib)


MUTATIONS = {
    "window_inclusive": ("(d >= 0 && d < window)", "(d >= 0 && d <= window)"),
    "global_keys_only": ("global = (j < nglobal || i < nglobal)", "global = (j < nglobal)"),
    "global_ignores_causal": ("&& (!causal || j <= i);", ";"),
    "one_sided_noncausal": ("(d > -window && d < window)", "(d >= 0 && d < window)"),
    # the backward (fa_oracle_attention_bwd_masked)
    "bwd_dv_without_p": ("av[d] += p * gi[d];", "av[d] += gi[d];"),
    "bwd_dk_uses_do": ("ak[d] += ds * qi[d];", "ak[d] += ds * gi[d];"),
    "bwd_dq_ignores_mask": (
        "for (int64_t j = 0; j < Nk && l[r] > 0.0; ++j) {\n"
        "                if (!visible_masked(i, j, causal, window, nglobal))\n"
        "                    continue;",
        "for (int64_t j = 0; j < Nk && l[r] > 0.0; ++j) {"),
    "bwd_bk_without_row_term": (
        "ak[d] += ds * qi[d];\n                    if (magn) {\n"
        "                        mv[d] += p * fabs(gi[d]);\n"
        "                        mk[d] += w * fabs(qi[d]);",
        "ak[d] += ds * qi[d];\n                    if (magn) {\n"
        "                        mv[d] += p * fabs(gi[d]);\n"
        "                        mk[d] += fabs(ds) * fabs(qi[d]);"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_masked_mutation_is_caught(tmp_path, name):
    old, new = MUTATIONS[name]
    with open(oracle.SOURCE) as f:
        src = f.read()
    assert src.count(old) == 1
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    so = str(tmp_path / f"lib{name}.so")
    oracle.build(out=so, source=str(path), extra_flags=("-w",))
    mlib = oracle.load(so)
    failures = 0
    for pin in ALL_MASKED_PINS:
        try:
            pin(mlib)
        except (AssertionError, RuntimeError):
            failures += 1
    assert failures, f"no pin caught {name}"
