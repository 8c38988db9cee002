"""The oracle's pins are strong enough to catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's C source (a dropped
term, a wrong sign, index or operand, an off-by-one in the mask or the split
bounds, a wrong decoder constant), builds it on the CPU, binds it in place of
the real oracle and checks that the pin battery of ``test_oracle`` fails.
Every mutant keeps all memory accesses inside the arrays it is given.
"""
import ctypes
import os
import subprocess

import pytest

from oracle import oracle as OR
import test_oracle as T

SRC = os.path.join(os.path.dirname(OR.__file__), "oracle.c")

MUTANTS = {
    "drop_k_scale": ("(k_scale * elem(k, kv_dtype, kbase + d))", "(elem(k, kv_dtype, kbase + d))"),
    "drop_q_scale": ("(q_scale * elem(q, q_dtype, qoff + d))", "(elem(q, q_dtype, qoff + d))"),
    "drop_v_scale": ("(v_scale * elem(v, kv_dtype, vbase + d))", "(elem(v, kv_dtype, vbase + d))"),
    "drop_sm_scale": ("s[j - j0] = sm_scale * acc;", "s[j - j0] = acc;"),
    "gqa_map_modulo": ("const int g = h / group;", "const int g = h % num_kv_heads;"),
    "causal_off_by_one": ("if (causal && j1 > pos + 1) j1 = pos + 1;",
                          "if (causal && j1 > pos) j1 = pos;"),
    "v_uses_k_slot_stride": ("(j % page_size) * v_stride[1]", "(j % page_size) * k_stride[1]"),
    "q_head_major": ("const int64_t qoff = (t * num_qo_heads + h) * (int64_t)head_dim_qk;",
                     "const int64_t qoff = ((int64_t)h * qo_indptr[batch] + t) * (int64_t)head_dim_qk;"),
    "lse_drops_max": ("lse[(int64_t)c * nrows + ri] = m + log(z);",
                      "lse[(int64_t)c * nrows + ri] = log(z);"),
    "unnormalised_o": ("for (int d = 0; d < head_dim_vo; ++d) orow[d] /= z;", ""),
    "split_bounds_overlap": ("p1 = (int64_t)(c + 1) * n / S;",
                             "p1 = (int64_t)(c + 1) * n / S + ((c + 1) < S);"),
    "merge_weight_sign": ("const double w = exp(lc - m);", "const double w = exp(m - lc);"),
    "merge_lse_drops_max": ("if (so) so[r] = m + log(wsum);", "if (so) so[r] = log(wsum);"),
    "f16_bias": ("else v = ldexp(1.0 + m / 1024.0, e - 15);",
                 "else v = ldexp(1.0 + m / 1024.0, e - 14);"),
    "fp8_subnormal_exp": ("if (e == 0) v = ldexp((double)m / 8.0, -6);",
                          "if (e == 0) v = ldexp((double)m / 8.0, -7);"),
    "fp8_bias": ("else v = ldexp(1.0 + m / 8.0, e - 7);", "else v = ldexp(1.0 + m / 8.0, e - 8);"),
    "bf16_truncates_sign": ("uint32_t u = (uint32_t)b << 16;",
                            "uint32_t u = ((uint32_t)b & 0x7fffu) << 16;"),
}


def battery():
    """Run the oracle pins; return the names of those that failed."""
    failed = []
    cases = [
        ("decoders_fp8", T.test_decode_fp8_all_codes),
        ("decoders_bf16", T.test_decode_bf16_all_codes),
        ("decoders_f16", T.test_decode_f16_all_codes),
        ("merge", T.test_merge_special_cases),
    ]
    for name in T.small_cases():
        cases.append((f"dense_{name}", lambda n=name: T.test_oracle_matches_dense(n)))
    cases.append(("split_partials", lambda: T.test_oracle_split_partials_match_dense("c2_small", 3)))
    cases.append(("split_merge", lambda: T.test_split_then_merge_equals_unsplit("c5_small", 4)))
    for name, fn in cases:
        try:
            fn()
        except AssertionError:
            failed.append(name)
    return failed


@pytest.mark.parametrize("mutant", list(MUTANTS))
def test_pins_catch_mutant(mutant, tmp_path, monkeypatch):
    old, new = MUTANTS[mutant]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not found uniquely: {old}"
    path = tmp_path / "oracle_mut.c"
    path.write_text(src.replace(old, new))
    lib_path = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o",
                    str(lib_path), str(path), "-lm"], check=True)
    monkeypatch.setattr(OR, "_lib", OR.declare(ctypes.CDLL(str(lib_path))))
    failed = battery()
    assert failed, f"no pin caught mutant {mutant}"


def test_unmutated_battery_passes():
    assert battery() == []
