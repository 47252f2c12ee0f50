"""Planted mistakes in the oracle must each fail at least one pin.

Each mutant is a copy of oracle.c with one plausible slip (a dropped term, a
wrong sign or index, a swapped operand) compiled on the CPU; the pin suite is
then run against it.  This checks the pins, not the product.
"""
import os

import pytest

import oracle
import oracle_checks as oc

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "dropped_scale": ("s[j] = a->scale * dot;", "s[j] = dot;"),
    "no_max_shift_in_sum": ("l += exp(s[j] - m);", "l += exp(s[j]);"),
    "wrong_sign_in_exp": ("double p = exp(s[j] - m) / l;", "double p = exp(m - s[j]) / l;"),
    "no_divide": ("double p = exp(s[j] - m) / l;", "double p = exp(s[j] - m);"),
    "lse_drops_max": ("a->LSE[out_row] = m + log(l);", "a->LSE[out_row] = log(l);"),
    "causal_off_by_one": ("long lim = i + (a->Nk - a->N) + 1;", "long lim = i + (a->Nk - a->N);"),
    "causal_top_left": ("long lim = i + (a->Nk - a->N) + 1;", "long lim = i + 1;"),
    "key_len_by_head": ("nvis = visible_keys(a, b, i);", "nvis = visible_keys(a, bh % a->B, i);"),
    "k_swapped_for_v": ("* widen(a->K, a->dtype, kvoff + (size_t)j * d + c);",
                        "* widen(a->V, a->dtype, kvoff + (size_t)j * d + c);"),
    "bf16_shift": ("(uint32_t)((const uint16_t *)base)[idx] << 16;",
                   "(uint32_t)((const uint16_t *)base)[idx] << 15;"),
    "softmax_no_shift": ("y[j] = exp(x[j] - m) / l;", "y[j] = exp(x[j]) / l;"),
    "softmax_min_not_max": ("if (x[j] > m)\n            m = x[j];", "if (x[j] > m && m == -INFINITY)\n            m = x[j];"),
    "masked_row_lse_zero": ("a->LSE[out_row] = -INFINITY;\n        return;", "a->LSE[out_row] = 0.0;\n        return;"),
    "rows_lse_drops_max": ("LSE[r] = l > 0.0 ? m + log(l) : -INFINITY;", "LSE[r] = l > 0.0 ? log(l) : -INFINITY;"),
    "rows_wrong_stride": ("x[j] = widen(X, dtype, (size_t)r * cols + j);", "x[j] = widen(X, dtype, (size_t)r + j);"),
    "bwd_dropped_scale": ("s[j] = dot * a->scale;", "s[j] = dot;"),
    "bwd_no_max_shift_in_sum": ("l = l + exp(s[j] - m);", "l = l + exp(s[j]);"),
    "bwd_drops_D": ("ds = p[j] * (dp - D);", "ds = p[j] * dp;"),
    "bwd_sign_flip": ("ds = p[j] * (dp - D);", "ds = p[j] * (D - dp);"),
    "bwd_dk_from_do": ("dK[(size_t)j * d + c] += a->scale * ds * widen(a->Q, a->dtype, qo + c);",
                       "dK[(size_t)j * d + c] += a->scale * ds * widen(a->dO, a->dtype, qo + c);"),
    "bwd_dv_uses_ds": ("dV[(size_t)j * d + c] += p[j] * widen(a->dO, a->dtype, qo + c);",
                       "dV[(size_t)j * d + c] += ds * widen(a->dO, a->dtype, qo + c);"),
    "bwd_dq_no_scale": ("dQ[(size_t)i * d + c] += a->scale * ds * widen(a->K, a->dtype, ko + c);",
                        "dQ[(size_t)i * d + c] += ds * widen(a->K, a->dtype, ko + c);"),
    "bwd_D_drops_output": ("D += widen(a->dO, a->dtype, qo + c) * o[c];", "D += widen(a->dO, a->dtype, qo + c);"),
    "bwd_dp_reads_k": ("dp += widen(a->dO, a->dtype, qo + c) * widen(a->V, a->dtype, ko + c);",
                       "dp += widen(a->dO, a->dtype, qo + c) * widen(a->K, a->dtype, ko + c);"),
    "row_index_swapped": ("long bh = flat / a->N, i = flat % a->N, b = bh / a->H;",
                          "long bh = flat / a->N, i = flat % a->N, b = bh % a->B;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    find, repl = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(find) == 1, f"mutation site for {name} not unique/found"
    mpath = tmp_path / "oracle_mutant.c"
    mpath.write_text(src.replace(find, repl))
    so = str(tmp_path / f"liboracle_{name}.so")
    oracle.build(so, str(mpath))
    lib = oracle.load(so, rebuild_if_missing=False)
    failed = []
    for check in oc.ALL_CHECKS:
        try:
            check(lib)
        except (AssertionError, RuntimeError, ValueError, FloatingPointError):
            failed.append(check.__name__)
    assert failed, f"no pin caught mutant {name}"
