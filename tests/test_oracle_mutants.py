"""The oracle's pins are strong enough to catch plausible mistakes.

Each case plants one mistake in a copy of ``oracle/maxsim_oracle.c`` (a
dropped term, a wrong sign, index or operand, a wrong tie rule), compiles the
copy with gcc, and runs the pin tests against it: at least one must fail.
Everything happens on the CPU; the real oracle is untouched.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "maxsim_oracle.c")
PINS = ["tests/test_oracle_fwd.py", "tests/test_oracle_i8.py", "tests/test_oracle_bwd.py",
        "tests/test_oracle_topk.py", "tests/test_oracle_bwd_varlen.py", "tests/test_oracle_chamfer.py"]

MUTANTS = {
    "tie_takes_last_index": ("            if (s > m) {\n                m = s;\n                arg = j;",
                             "            if (s >= m) {\n                m = s;\n                arg = j;"),
    "sum_sign": ("        score += m;", "        score -= m;"),
    "mask_dropped": ("        len[b] = d_lens ? d_lens[b] : Ld;", "        len[b] = Ld;"),
    "f16_exponent_bias": ("ldexp((double)(1024 + frac), expo - 25)", "ldexp((double)(1024 + frac), expo - 24)"),
    "bf16_fraction_width": ("ldexp((double)(128 + frac), expo - 134)", "ldexp((double)(128 + frac), expo - 133)"),
    "i8_tie_takes_last": ("                    if (s > m) {", "                    if (s >= m) {"),
    "i8_query_scale_dropped": ("float v = m * q_scale[(int64_t)q * Lq + i];", "float v = m;"),
    "i8_doc_scale_of_wrong_token": ("float s = (float)dot * d_scale[first + j];",
                                    "float s = (float)dot * d_scale[first];"),
    "csr_cursor_not_advanced": ("        int64_t dst = b * Ld + argmax[s];\n        col_idx[cursor[dst]] = (int32_t)s;\n        cursor[dst] += 1;\n",
                                "        int64_t dst = b * Ld + argmax[s];\n        col_idx[cursor[dst]] = (int32_t)s;\n"),
    "csr_wrong_doc_stride": ("        cnt[b * Ld + t] += 1;", "        cnt[t * B + b] += 1;"),
    "dD_wrong_operand": ("double* ddr = dD + ((int64_t)b * Ld + t) * d;\n                for (int k = 0; k < d; ++k) {\n"
                         "                    dq[k] += gqb * decode(drow[k], dtype);\n"
                         "                    ddr[k] += gqb * decode(qrow[k], dtype);",
                         "double* ddr = dD + ((int64_t)b * Ld + t) * d;\n                for (int k = 0; k < d; ++k) {\n"
                         "                    dq[k] += gqb * decode(drow[k], dtype);\n"
                         "                    ddr[k] += gqb * decode(drow[k], dtype);"),
    "dQ_transposed_upstream": ("++b) {\n            double gqb = (double)g[(int64_t)q * B + b];",
                               "++b) {\n            double gqb = (double)g[(int64_t)b * Nq + q];"),
    "varlen_dD_wrong_operand": ("double* ddr = dD + row * d;\n                for (int k = 0; k < d; ++k) {\n"
                                "                    dq[k] += gqb * decode(drow[k], dtype);\n"
                                "                    ddr[k] += gqb * decode(qrow[k], dtype);",
                                "double* ddr = dD + row * d;\n                for (int k = 0; k < d; ++k) {\n"
                                "                    dq[k] += gqb * decode(drow[k], dtype);\n"
                                "                    ddr[k] += gqb * decode(drow[k], dtype);"),
    "topk_ties_by_descending_index": ("    return (i > j) - (i < j);", "    return (i < j) - (i > j);"),
    "topk_ascending_scores": ("    if (si > sj) return -1;\n    if (si < sj) return 1;",
                              "    if (si > sj) return 1;\n    if (si < sj) return -1;"),
    "pairs_wrong_document_start": ("        const int64_t first = cu_seqlens[b];", "        const int64_t first = cu_seqlens[q];"),
    "varlen_csr_row_of_next_document": ("        cnt[cu_seqlens[b] + t] += 1;", "        cnt[cu_seqlens[b + 1] - 1 - t] += 1;"),
    "varlen_bwd_empty_doc_not_skipped": ("            if (cu_seqlens[b + 1] == cu_seqlens[b]) continue;\n            const double gqb",
                                         "            const double gqb"),
    "pairs_wrong_query": ("++e) qd[e] = decode(Q[(int64_t)q * Lq * d + e], dtype);",
                          "++e) qd[e] = decode(Q[(int64_t)(Nq - 1 - q) * Lq * d + e], dtype);"),
    "chamfer_tie_takes_last": ("            if (dd < best) {", "            if (dd <= best) {"),
    "chamfer_dropped_z": ("const double dd = dx * dx + dy * dy + dz * dz;", "const double dd = dx * dx + dy * dy;"),
    "chamfer_wrong_batch_stride": ("const float* p = B + (b * Nb + t) * 3;", "const float* p = B + (b * Na + t) * 3;"),
    "chamfer_csr_unstable": ("    for (int64_t s = 0; s < (int64_t)Bt * Na; ++s) {  /* ascending s: a stable fill */",
                             "    for (int64_t s = (int64_t)Bt * Na - 1; s >= 0; --s) {  /* ascending s: a stable fill */"),
    "chamfer_reverse_term_dropped": ("                dQ[qj * 3 + k] += w * diff;\n                dP[pi * 3 + k] -= w * diff;",
                                     "                dQ[qj * 3 + k] += w * diff;"),
    "chamfer_own_term_sign": ("                dP[pi * 3 + k] += w * diff;\n                dQ[qj * 3 + k] -= w * diff;",
                              "                dP[pi * 3 + k] -= w * diff;\n                dQ[qj * 3 + k] -= w * diff;"),
    # one padding token read as valid (off-by-one in the mask)
    "mask_off_by_one": ("        len[b] = d_lens ? d_lens[b] : Ld;",
                        "        len[b] = d_lens ? (d_lens[b] < Ld ? d_lens[b] + 1 : Ld) : Ld;"),
    # the INT8 epilogue contracted into one fused multiply-add (one rounding instead of two)
    "i8_epilogue_fma": ("                score = score + v;", "                score = fmaf(m, q_scale[(int64_t)q * Lq + i], score);"),
    # the padded CSR filled in descending source order (unstable within a row)
    "csr_fill_unstable": ("    for (int64_t s = 0; s < nsrc; ++s) { /* ascending s: a stable fill */\n        int64_t b = (s / Lq) % B;\n        if (argmax[s] < 0) continue;",
                          "    for (int64_t s = nsrc - 1; s >= 0; --s) { /* ascending s: a stable fill */\n        int64_t b = (s / Lq) % B;\n        if (argmax[s] < 0) continue;"),
    # an empty document's -1 clamped to its token 0 instead of selecting nothing
    "padded_empty_doc_clamped": ("                if (t < 0) continue;\n                const uint16_t* qrow",
                                 "                if (t < 0) t = 0;\n                const uint16_t* qrow"),
    "chamfer_factor_two_dropped": ("            const double w = 2.0 * (double)gq[qj];", "            const double w = (double)gq[qj];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site for %s not unique" % name
    mut_c = tmp_path / "mutant.c"
    mut_c.write_text(src.replace(old, new))
    mut_so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                    str(mut_c), "-o", str(mut_so), "-lm"], check=True)
    env = dict(os.environ, MAXSIM_ORACLE_LIB=str(mut_so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] + PINS,
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 1, "mutant %s survived the pins:\n%s" % (name, r.stdout[-2000:])
