"""The oracle's pins must catch plausible mistakes.

Each case copies ``oracle/`` to a temporary directory, plants one mistake in
the copy of ``oracle.c`` (a dropped term, a wrong index or sign, a swapped
order), builds it with gcc on the CPU and runs the pin tests of the affected
routine against it.  At least one pin must fail.  The real oracle is never
touched.
"""
import importlib.util
import os
import shutil
import sys

import pytest

import test_oracle_conv as T_conv
import test_oracle_gdn as T_gdn
import test_oracle_next as T_next
import test_oracle_scan as T_scan
import test_oracle_tdecay as T_td
import test_oracle_wkv as T_wkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, original text, planted text, pin functions with their parameters)
MUTATIONS = [
    ("conv taps reversed", "acc += w[(size_t)c * K + j] * xv;", "acc += w[(size_t)c * K + (K - 1 - j)] * xv;",
     [(T_conv.test_conv_matches_numpy_correlate, dict(S=75, C=64, K=4)),
      (T_conv.test_conv_one_hot_taps_expose_tap_order, {})]),
    ("conv state off by one", "const int src = S + r;", "const int src = S + r - 1;",
     [(T_conv.test_conv_short_chunk_keeps_old_state_rows, dict(S=1)),
      (T_conv.test_conv_chunk_split_invariance, dict(splits=[64, 11]))]),
    ("scan stores pre-update state", "s = a[i] * s + b[i];\n            h[i] = s;",
     "h[i] = s;\n            s = a[i] * s + b[i];",
     [(T_scan.test_scan_closed_form, dict(S=3)), (T_scan.test_scan_special_cases_reduce_to_library_routines, {})]),
    ("scan drops decay on b", "s = a[i] * s + b[i];", "s = a[i] * (s + b[i]);",
     [(T_scan.test_scan_closed_form, dict(S=3))]),
    ("wkv update misses decay", "const double ed = pp + wc;", "const double ed = pp;",
     [(T_wkv.test_wkv_matches_decimal_definition, {}), (T_wkv.test_wkv_matches_page_row_form, dict(splits=[64, 11]))]),
    ("wkv bonus drops u", "const double eb = uc + kt;", "const double eb = kt;",
     [(T_wkv.test_wkv_matches_decimal_definition, {})]),
    ("wkv wrong max sign", "const double q = ed > kt ? ed : kt;", "const double q = ed < kt ? ed : kt;",
     [(T_wkv.test_wkv_matches_decimal_definition, {}), (T_wkv.test_wkv_finite_at_range_edges, {})]),
    ("tdecay uses the previous row's decay", "const double key = k[i], val = v[i], wt = w[i];",
     "const double key = k[i], val = v[i], wt = w[t > 0 ? i - (size_t)C : i];",
     [(T_td.test_tdecay_matches_brute_force_sums, {})]),
    ("tdecay update misses decay", "const double decayed = pp + wt;", "const double decayed = pp;",
     [(T_td.test_tdecay_matches_brute_force_sums, {}), (T_td.test_tdecay_constant_decay_is_rwkv4, {})]),
    ("tdecay bonus drops u", "const double bonus = uc + key;", "const double bonus = key;",
     [(T_td.test_tdecay_matches_brute_force_sums, {}), (T_td.test_tdecay_zero_decay_is_a_running_mean, {})]),
    ("gdn prediction misses decay", "uvec[j] = bt * (vt[j] - dec * sk);", "uvec[j] = bt * (vt[j] - sk);",
     [(T_gdn.test_gdn_token_loop_equals_page_chunk_form, dict(splits=[7, 4]))]),
    ("gdn wrong key head", "const int kh = h / grp;", "const int kh = h % Hk;",
     [(T_gdn.test_gdn_value_heads_share_consecutive_key_heads, {})]),
    ("gdn drops beta", "uvec[j] = bt * (vt[j] - dec * sk);", "uvec[j] = (vt[j] - dec * sk);",
     [(T_gdn.test_gdn_token_loop_equals_page_chunk_form, dict(splits=[7, 4]))]),
    ("gdn transposed state read", "sk += St[(size_t)i * dv + j] * kt[i];", "sk += St[(size_t)j * dv + i] * kt[i];",
     [(T_gdn.test_gdn_token_loop_equals_page_chunk_form, dict(splits=[7, 4])),
      (T_gdn.test_gdn_exact_recall_with_orthonormal_keys, {})]),
    ("inverse drops a term", "for (int m = j; m < i; ++m)", "for (int m = j + 1; m < i; ++m)",
     [(T_gdn.test_unit_lower_inverse_matches_numpy, dict(n=64, par=(0, 64)))]),
    ("time shift never advances", "            prev = cur;\n", "",
     [(T_next.test_time_shift_one_hot_mixes_are_rows_and_shifted_rows, {})]),
    ("time shift mixes the wrong row", "mu * cur + (1.0 - mu) * prev;", "mu * prev + (1.0 - mu) * cur;",
     [(T_next.test_time_shift_one_hot_mixes_are_rows_and_shifted_rows, {})]),
    ("mixer reads h before the update", "                h[n] = a * h[n] + b;\n                acc += Cm[(size_t)t * N + n] * h[n];",
     "                acc += Cm[(size_t)t * N + n] * h[n];\n                h[n] = a * h[n] + b;",
     [(T_next.test_mixer_brute_force_product_form, {}), (T_next.test_mixer_agrees_with_the_pinned_scan, {})]),
    ("mixer decay misses dt", "const double a = exp(dtv * A[(size_t)d * N + n]);", "const double a = exp(A[(size_t)d * N + n]);",
     [(T_next.test_mixer_constant_decay_geometric_closed_form, {})]),
    ("mixer drops the skip term", "y[(size_t)t * Dm + d] = acc + Dp[d] * xv;", "y[(size_t)t * Dm + d] = acc;",
     [(T_next.test_mixer_zero_input_weight_leaves_skip_and_decayed_state, {})]),
    ("mixer transposed A", "exp(dtv * A[(size_t)d * N + n])", "exp(dtv * A[(size_t)(n % Dm) * N + (d % N)])",
     [(T_next.test_mixer_brute_force_product_form, {}), (T_next.test_mixer_constant_decay_geometric_closed_form, {})]),
]


def _mutant(tmp_path, name, orig, new):
    d = tmp_path / ("oracle_mut_" + "".join(ch if ch.isalnum() else "_" for ch in name))
    shutil.copytree(os.path.join(ROOT, "oracle"), d, ignore=shutil.ignore_patterns("*.so", "__pycache__"))
    src = (d / "oracle.c").read_text()
    assert src.count(orig) == 1, f"mutation anchor not unique: {orig!r}"
    (d / "oracle.c").write_text(src.replace(orig, new))
    modname = d.name
    spec = importlib.util.spec_from_file_location(modname, d / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    sys.modules[modname] = mod
    spec.loader.exec_module(mod)
    mod.build(force=True)
    return mod


@pytest.mark.parametrize("name,orig,new,pins", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, name, orig, new, pins):
    mod = _mutant(tmp_path, name, orig, new)
    caught = []
    for fn, kw in pins:
        try:
            fn(mod, **kw)
        except (AssertionError, FloatingPointError, ValueError, ZeroDivisionError, ArithmeticError):
            caught.append(fn.__name__)
    assert caught, f"no pin caught the planted mistake: {name}"
