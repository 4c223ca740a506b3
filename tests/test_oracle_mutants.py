"""The pins must reject plausible mistakes planted in copies of the oracle source.

Forward mutants face the forward pins; backward mutants (mistakes in the
gradient code only) face the backward pins; triangle-multiplication mutants
face its pins.

Each mutant is a textual edit of oracle/evo_ref.c (a dropped term, a wrong
index, a transposed operand, a wrong constant), compiled with gcc into a
temporary directory and loaded through the same ctypes interface.  The real
oracle is never modified.  A mutant survives if every pin passes on it; the
test fails if any mutant survives.
"""
import os

import pytest

import oracle
import oracle_bwd_pins
import oracle_pins
import oracle_trimul_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "evo_ref.c")

MUTANTS = {
    "drop_mask": [("if (a->mask) sj += load", "if (0) sj += load")],
    "drop_pair": [("if (a->pair) sj += load", "if (0) sj += load")],
    "pair_transposed": [("off_pair(a, b, h, i, j)", "off_pair(a, b, h, j, i)")],
    "pair_ignores_head": [("off_pair(a, b, h, i, j)", "off_pair(a, b, 0, i, j)")],
    "mask_by_query": [("off_mask(a, b, n, j)", "off_mask(a, b, n, i)")],
    "mask_ignores_n": [("off_mask(a, b, n, j)", "off_mask(a, b, 0, j)")],
    "scale_1_over_D": [("1.0 / sqrt((double)D)", "1.0 / (double)D")],
    "no_scale": [("double sj = dot * scale;", "double sj = dot;")],
    "scale_on_bias_too": [("double sj = dot * scale;", "double sj = dot;"), ("s[j] = sj;", "s[j] = sj * scale;")],
    "key_index_slip": [("qrow[d] * kd[j * D + d]", "qrow[d] * kd[i * D + d]")],
    "values_from_keys": [("w * vd[j * D + e]", "w * kd[j * D + e]")],
    "kv_ignore_head": [("int64_t o = off_qkv(a, b, n, j, h, d);", "int64_t o = off_qkv(a, b, n, j, 0, d);")],
    "q_ignores_head": [("off_qkv(a, b, n, i, h, d));", "off_qkv(a, b, n, i, 0, d));")],
    "no_normaliser": [("double w = s[j] / Z;", "double w = s[j];")],
    "lse_without_max": [("return m + log(Z);", "return log(Z);")],
    "lse_log2": [("return m + log(Z);", "return m + log2(Z);")],
    "lse_layout_BNLH": [("lse[((b * N + n) * H + h) * L + i]", "lse[((b * N + n) * L + i) * H + h]")],
    "max_added_not_subtracted": [("s[j] = exp(s[j] - m);", "s[j] = exp(s[j] + m);")],
    "max_starts_at_zero": [("double m = -INFINITY;", "double m = 0.0;")],
    "bf16_shift": [("((uint32_t)bits) << 16", "((uint32_t)bits) << 15")],
    "f16_exponent_bias": [("expo - 25", "expo - 24")],
    "f16_subnormal_scale": [("(double)frac, -24)", "(double)frac, -23)")],
}

BWD_MUTANTS = {
    "bwd_drop_delta": [("P[i * L + j] * (dp - delta);", "P[i * L + j] * dp;")],
    "bwd_delta_sign": [("P[i * L + j] * (dp - delta);", "P[i * L + j] * (dp + delta);")],
    "bwd_delta_from_values": [("delta += dod[i * D + e] * od[i * D + e];", "delta += dod[i * D + e] * vd[i * D + e];")],
    "bwd_dp_from_keys": [("dp += dod[i * D + e] * vd[j * D + e];", "dp += dod[i * D + e] * kd[j * D + e];")],
    "bwd_dv_transposed_weights": [("g += P[i * L + j] * dod[i * D + e];", "g += P[j * L + i] * dod[i * D + e];")],
    "bwd_dq_unscaled": [("dq[off_qkv(a, b, n, i, h, d)] = g * scale;", "dq[off_qkv(a, b, n, i, h, d)] = g;")],
    "bwd_dk_unscaled": [("dk[off_qkv(a, b, n, j, h, d)] = g * scale;", "dk[off_qkv(a, b, n, j, h, d)] = g;")],
    "bwd_scale_1_over_D": [("const double scale = 1.0 / sqrt((double)a->D);", "const double scale = 1.0 / (double)a->D;")],
    "bwd_dq_from_values": [("g += P[i * L + j] * kd[j * D + d];", "g += P[i * L + j] * vd[j * D + d];")],
    "bwd_dk_from_keys": [("load(a->q, a->dtype, off_qkv(a, b, n, r, h, d));", "kd[r * D + d];")],
    "bwd_dk_transposed": [("g += P[r * L + j] * load", "g += P[j * L + r] * load")],
    "bwd_unnormalised_weights": [("for (int64_t j = 0; j < L; ++j) Pi[j] /= Z;", "(void)Z;")],
    "bwd_dmask_by_query": [("for (int64_t i = 0; i < L; ++i) g += P[i * L + j];", "for (int64_t i = 0; i < L; ++i) g += P[j * L + i];")],
    "bwd_dmask_last_head_only": [("dmask_row[j] += g;", "dmask_row[j] = g;")],
    "bwd_dpair_transposed": [("dpair_bh[i * L + j] += P[i * L + j];", "dpair_bh[j * L + i] += P[i * L + j];")],
    "bwd_dpair_last_n_only": [("dpair_bh[i * L + j] += P[i * L + j];", "dpair_bh[i * L + j] = P[i * L + j];")],
    "bwd_dout_ignores_head": [("off_qkv(a, b, n, i, h, e));", "off_qkv(a, b, n, i, 0, e));")],
    "bwd_masked_rows_uniform": [("for (int64_t j = 0; j < L; ++j) Pi[j] = 0.0;",
                                 "for (int64_t j = 0; j < L; ++j) Pi[j] = 1.0 / (double)L;")],
}


def _compile_mutant(name, edits, tmp_path):
    with open(SRC) as f:
        text = f.read()
    for old, new in edits:
        assert text.count(old) == 1, f"mutation anchor {old!r} must occur exactly once"
        text = text.replace(old, new)
    src = tmp_path / f"mut_{name}.c"
    src.write_text(text)
    return oracle.load_library(oracle.compile_source(str(src), str(tmp_path / f"libmut_{name}.so")))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    lib = _compile_mutant(name, MUTANTS[name], tmp_path)

    def ref(q, k, v, mask, pair, dtype):
        return oracle.fwd(q, k, v, mask, pair, dtype=dtype, nthreads=2, lib=lib)

    caught_by = None
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(ref)
        except (AssertionError, RuntimeError):
            caught_by = pin.__name__
            break
    assert caught_by is not None, f"mutant {name} passed every pin"


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_bwd_pins_reject_mutant(name, tmp_path):
    lib = _compile_mutant(name, BWD_MUTANTS[name], tmp_path)

    def gref(q, k, v, mask, pair, dout, dtype):
        # one thread: the per-thread pair partials then hold every n in turn
        return oracle.bwd(q, k, v, mask, pair, dout, dtype=dtype, nthreads=1, lib=lib)

    caught_by = None
    for pin in oracle_bwd_pins.ALL_BWD_PINS:
        try:
            pin(gref)
        except (AssertionError, RuntimeError):
            caught_by = pin.__name__
            break
    assert caught_by is not None, f"mutant {name} passed every backward pin"


TRIMUL_MUTANTS = {
    "tm_a_as_incoming": [("const int64_t ia = direction == 0 ? i * L + k : k * L + i;",
                          "const int64_t ia = k * L + i;")],
    "tm_w_transposed": [("const int64_t iw = direction == 0 ? j * L + k : k * L + j;",
                         "const int64_t iw = direction == 0 ? k * L + j : j * L + k;")],
    "tm_out_transposed": [("x[base + i * L + j] = sum;", "x[base + j * L + i] = sum;")],
    "tm_channel_ignored": [("const int64_t base = bc * LL;", "const int64_t base = (bc / C) * C * LL;")],
    "tm_a_times_a": [("sum += load(a, dtype, base + ia) * load(w, dtype, base + iw);",
                      "sum += load(a, dtype, base + ia) * load(a, dtype, base + iw);")],
    "tm_directions_swapped": [("const int64_t ia = direction == 0 ?", "const int64_t ia = direction == 1 ?"),
                              ("const int64_t iw = direction == 0 ?", "const int64_t iw = direction == 1 ?")],
    "tm_last_k_dropped": [("for (int64_t k = 0; k < L; ++k) {\n                    const int64_t ia",
                           "for (int64_t k = 0; k + 1 < L; ++k) {\n                    const int64_t ia")],
}


@pytest.mark.parametrize("name", sorted(TRIMUL_MUTANTS))
def test_trimul_pins_reject_mutant(name, tmp_path):
    lib = _compile_mutant(name, TRIMUL_MUTANTS[name], tmp_path)

    def tref(a, w, dtype, direction):
        return oracle.trimul(a, w, dtype=dtype, direction=direction, nthreads=1, lib=lib)

    caught_by = None
    for pin in oracle_trimul_pins.ALL_TRIMUL_PINS:
        try:
            pin(tref)
        except (AssertionError, RuntimeError):
            caught_by = pin.__name__
            break
    assert caught_by is not None, f"mutant {name} passed every triangle-multiplication pin"
