"""Plant plausible mistakes in a copy of the oracle's C source and check that
the pins catch each one.  The copies are built in a temporary directory; the
real oracle is never modified."""
import os

import pytest

import oracle
import pins

# (name, exact text in sdpa_oracle.c, replacement)
MUTANTS = [
    ("scale_by_d_not_sqrt_d", "if (!(tau > 0.0)) tau = sqrt((double)d);\n    if (nthreads <= 0) nthreads = omp_get_max_threads();\n    const int64_t nrows",
     "if (!(tau > 0.0)) tau = (double)d;\n    if (nthreads <= 0) nthreads = omp_get_max_threads();\n    const int64_t nrows"),
    ("no_scale", "work[j] = z / tau;", "work[j] = z;"),
    ("multiply_by_tau", "work[j] = z / tau;", "work[j] = z * tau;"),
    ("no_normalisation", "for (int64_t j = 0; j < n_valid; ++j) work[j] /= Z;", ""),
    ("lse_drops_max", "return m + log(Z);", "return log(Z);"),
    ("lse_log2", "return m + log(Z);", "return m + log2(Z);"),
    ("max_shift_sign", "work[j] = exp(work[j] - m);", "work[j] = exp(work[j] + m);"),
    ("causal_masks_diagonal", "if (causal && i + 1 < hi) hi = i + 1;", "if (causal && i < hi) hi = i;"),
    ("causal_ignored", "if (causal && i + 1 < hi) hi = i + 1;", ""),
    ("key_lens_ignored", "if (len < hi) hi = len;", ""),
    ("key_lens_off_by_one", "if (len < hi) hi = len;", "if (len + 1 < hi) hi = len + 1;"),
    ("k_transposed_index", "load_elem(k, dtype, kv_off + j * d + t)", "load_elem(k, dtype, kv_off + t * d + j)"),
    ("v_wrong_row", "acc += work[j] * load_elem(v, dtype, kv_off + j * d + t);",
     "acc += work[j] * load_elem(v, dtype, kv_off + (n_valid - 1 - j) * d + t);"),
    ("dropped_last_key", "for (int64_t j = 0; j < n_valid; ++j) {\n        double z = 0.0;",
     "for (int64_t j = 0; j + 1 < n_valid; ++j) {\n        double z = 0.0;"),
    ("dropped_last_dim", "for (int64_t t = 0; t < d; ++t)\n            z +=",
     "for (int64_t t = 0; t + 1 < d; ++t)\n            z +="),
    ("empty_row_lse_zero", "*lse = -INFINITY;", "*lse = 0.0;"),
    ("bf16_low_half", "uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;",
     "uint32_t bits = (uint32_t)((const uint16_t*)base)[idx];"),
    ("wrong_head_offset", "bh * Lk * d, d, n_valid, tau,\n                          out + row * d",
     "b * Lk * d, d, n_valid, tau,\n                          out + row * d"),
    # backward
    ("bwd_no_centering", "const double ds = a[j] * (da[j] - c);", "const double ds = a[j] * da[j];"),
    ("bwd_centering_unweighted", "c += a[j] * z;", "c += z;"),
    ("bwd_dq_no_scale", "dq[q_off + t] += ds * load_elem(k, dtype, kv_off + j * d + t) / tau;",
     "dq[q_off + t] += ds * load_elem(k, dtype, kv_off + j * d + t);"),
    ("bwd_dk_from_k", "dk[kv_off + j * d + t] += ds * load_elem(q, dtype, q_off + t) / tau;",
     "dk[kv_off + j * d + t] += ds * load_elem(k, dtype, kv_off + j * d + t) / tau;"),
    ("bwd_dv_from_da", "dv[kv_off + j * d + t] += a[j] * load_elem(dout, dtype, q_off + t);",
     "dv[kv_off + j * d + t] += da[j] * load_elem(dout, dtype, q_off + t);"),
    ("bwd_da_from_k", "z += load_elem(dout, dtype, q_off + t) * load_elem(v, dtype, kv_off + j * d + t);",
     "z += load_elem(dout, dtype, q_off + t) * load_elem(k, dtype, kv_off + j * d + t);"),
    # general form
    ("ex_mask_ignored", "sc[j] = z / tau + (mask ? mask[row * Lk + j] : 0.0);", "sc[j] = z / tau;"),
    ("ex_mask_sign", "sc[j] = z / tau + (mask ? mask[row * Lk + j] : 0.0);",
     "sc[j] = z / tau - (mask ? mask[row * Lk + j] : 0.0);"),
    ("ex_mask_transposed", "sc[j] = z / tau + (mask ? mask[row * Lk + j] : 0.0);",
     "sc[j] = z / tau + (mask ? mask[(bh * Lk + j) * Lq + i] : 0.0);"),
    ("ex_tau_ignored", "sc[j] = z / tau + (mask", "sc[j] = z / sqrt((double)d) + (mask"),
    ("ex_value_width_d", "acc += sc[j] / Z * load_elem(v, dtype, (bh * Lk + j) * dv + t);",
     "acc += sc[j] / Z * load_elem(v, dtype, (bh * Lk + j) * d + t);"),
    ("ex_all_masked_not_empty", "if (n <= 0 || m == -INFINITY) {", "if (n <= 0) {"),
]


@pytest.fixture(scope="module")
def source_text():
    with open(oracle.SOURCE, encoding="utf-8") as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, source_text, tmp_path):
    assert source_text.count(old) >= 1, f"mutation site for {name} not found"
    src = tmp_path / f"{name}.c"
    src.write_text(source_text.replace(old, new), encoding="utf-8")
    orc = oracle.Oracle(oracle.compile_source(str(src), str(tmp_path / f"lib{name}.so")))
    failures = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, RuntimeError, ValueError):
            failures.append(pin.__name__)
    assert failures, f"mutant {name} passed every pin"
