"""The pins have teeth: plant plausible slips in copies of the oracle source (on
the CPU, never in the GPU path), build each copy with gcc, and require that at
least one pin fails for every one of them.  A slip whose target text is no
longer in the source fails the test, so the list stays in step with the oracle.
"""
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "cssd_oracle.c")

MUTANTS = {
    "conjugated_C_readout": [
        ("sr += cr[n] * vr - ci[n] * vi;", "sr += cr[n] * vr + ci[n] * vi;"),
        ("si += cr[n] * vi + ci[n] * vr;", "si += cr[n] * vi - ci[n] * vr;"),
    ],
    "skip_term_dropped": [
        ("yr[p] = sr + d * xr[p];", "yr[p] = sr;"),
        ("yi[p] = si + d * xi[p];", "yi[p] = si;"),
    ],
    "softplus_dropped": [("double s = softplus(dt);", "double s = dt;")],
    "conjugated_A": [("*ai = mag * sin(s * aim);", "*ai = -mag * sin(s * aim);")],
    "rotation_not_scaled_by_step": [("*ar = mag * cos(s * aim);", "*ar = mag * cos(aim);"),
                                    ("*ai = mag * sin(s * aim);", "*ai = mag * sin(aim);")],
    "sign_in_complex_decay": [("double ni = ar * oii + ai * orr;", "double ni = ar * oii - ai * orr;")],
    "imag_x_ignored_in_outer_product": [("nr += br[n] * xr[p] - bi[n] * xi[p];", "nr += br[n] * xr[p];")],
    "outer_product_conjugates_B": [("ni += br[n] * xi[p] + bi[n] * xr[p];", "ni += br[n] * xi[p] - bi[n] * xr[p];")],
    "initial_state_ignored": [("if (h0_re && h0_im) {", "if (0) {")],
    "wrong_row_index": [("int64_t row = (b * T + t) * H + h; /* (b, t, h) */",
                         "int64_t row = (h * T + t) * Bsz + b;")],
    "skip_from_head_0": [("double d = dskip ? dskip[h] : 0.0;", "double d = dskip ? dskip[0] : 0.0;")],
    "decay_applied_after_input": [
        ("double orr = hr[n * D + p], oii = hi[n * D + p];",
         "double orr = hr[n * D + p] + (br[n] * xr[p] - bi[n] * xi[p]), "
         "oii = hi[n * D + p] + (br[n] * xi[p] + bi[n] * xr[p]);"),
        ("nr += br[n] * xr[p] - bi[n] * xi[p];", "nr += 0.0;"),
        ("ni += br[n] * xi[p] + bi[n] * xr[p];", "ni += 0.0;"),
    ],
    "readout_before_update": [
        # read out h_{t-1} (decayed nothing, no new input) instead of h_t
        ("double vr = hr[n * D + p], vi = hi[n * D + p];",
         "double vr = hr[n * D + p] - (br[n] * xr[p] - bi[n] * xi[p]), "
         "vi = hi[n * D + p] - (br[n] * xi[p] + bi[n] * xr[p]);"),
    ],
    "step_n_power_off_by_one": [("double complex an = cexp((double)n * z);",
                                 "double complex an = cexp((double)(n - 1) * z);")],
    "step_n_series_dropped": [("double complex hn = an * hv + ratio * bk * xp;",
                               "double complex hn = an * hv + bk * xp;")],
    "step_n_wrong_limit_at_unit_decay": [("(a == 1.0) ? (double complex)(double)n :",
                                          "(a == 1.0) ? (double complex)1.0 :")],
    "step_infinite_conjugated_score": [("score += (c_re[bh * N + k] + c_im[bh * N + k] * I) *",
                                        "score += (c_re[bh * N + k] - c_im[bh * N + k] * I) *")],
    "step_infinite_skip_dropped": [("double complex yv = gain * xp + d * xp;",
                                    "double complex yv = gain * xp;")],
    "step_infinite_gain_inverted": [("double complex gain = score / (1.0 - a);",
                                     "double complex gain = score * (1.0 - a);")],
    "backward_readout_not_conjugated": [("G[n * D + p] += conj(cn) * (dy_re[row * D + p]",
                                         "G[n * D + p] += cn * (dy_re[row * D + p]")],
    "backward_decay_not_conjugated": [("G[k] = conj(a) * G[k];", "G[k] = a * G[k];")],
    "backward_skip_dropped": [("double complex acc = d * dyp;", "double complex acc = 0.0;")],
    "backward_softplus_slope_dropped": [
        ("ddt[row] = creal(dz * conj(A)) / (1.0 + exp(-dt[row]));",
         "ddt[row] = creal(dz * conj(A));")],
    "backward_decay_grad_uses_new_state": [("ga += G[k] * conj(hp[k]);", "ga += G[k] * conj(ht[k]);")],
    "backward_dA_without_step_size": [("dA += s * dz;", "dA += dz;")],
    "backward_dC_uses_previous_state": [
        ("acc += (dy_re[row * D + p] + dy_im[row * D + p] * I) * conj(ht[n * D + p]);",
         "acc += (dy_re[row * D + p] + dy_im[row * D + p] * I) * conj(hp[n * D + p]);")],
    "phase_cayley_conjugated": [("double complex lambda = (1.0 + phi[at] * I) / (1.0 - phi[at] * I);",
                                 "double complex lambda = (1.0 - phi[at] * I) / (1.0 + phi[at] * I);")],
    "phase_gate_inverted": [("double alpha = 1.0 / (1.0 + exp(-u[at]));",
                             "double alpha = 1.0 / (1.0 + exp(u[at]));")],
    "phase_input_before_decay": [("psi = alpha * lambda * psi + (b_re[at] + b_im[at] * I);",
                                  "psi = alpha * lambda * (psi + (b_re[at] + b_im[at] * I));")],
    "phase_initial_state_ignored": [
        ("double complex psi = (psi0_re && psi0_im) ? psi0_re[bk] + psi0_im[bk] * I : 0.0;",
         "double complex psi = 0.0;")],
    "born_overlap_not_conjugated": [
        ("overlap += conj(q_re[qi + d] + q_im[qi + d] * I) * (k_re[kj + d] + k_im[kj + d] * I);",
         "overlap += (q_re[qi + d] + q_im[qi + d] * I) * (k_re[kj + d] + k_im[kj + d] * I);")],
    "born_not_causal": [("for (int64_t j = 0; j <= i; ++j) {\n        const int64_t kj",
                         "for (int64_t j = 0; j < T; ++j) {\n        const int64_t kj")],
    "born_diagonal_excluded": [("for (int64_t j = 0; j <= i; ++j) {\n        const int64_t kj",
                                "for (int64_t j = 0; j < i; ++j) {\n        const int64_t kj")],
    "born_modulus_not_squared": [("const double sij = mod * mod / ((double)D * t);",
                                  "const double sij = mod / ((double)D * t);")],
    "born_real_part_score": [("const double sij = mod * mod / ((double)D * t);",
                              "const double sij = creal(overlap) * creal(overlap) / ((double)D * t);")],
    "born_unnormalised": [("const double complex o = den != 0.0 ? num[d] / den : 0.0;",
                           "const double complex o = num[d];")],
    "born_value_of_query_row": [("num[d] += sij * (v_re[kj + d] + v_im[kj + d] * I);",
                                 "num[d] += sij * (v_re[qi + d] + v_im[qi + d] * I);")],
    "born_value_conjugated": [("num[d] += sij * (v_re[kj + d] + v_im[kj + d] * I);",
                               "num[d] += sij * (v_re[kj + d] - v_im[kj + d] * I);")],
    "born_rows_time_and_head_swapped": [
        ("const int64_t b = rows[3 * m], i = rows[3 * m + 1], h = rows[3 * m + 2];",
         "const int64_t b = rows[3 * m], i = rows[3 * m + 2], h = rows[3 * m + 1];")],
    "born_rows_output_not_strided": [("out_re + m * D,\n                 out_im + m * D);",
                                      "out_re + m,\n                 out_im + m);")],
    "born_temperature_of_key": [("const double sij = mod * mod / ((double)D * t);",
                                 "const double sij = mod * mod / ((double)D * (tau ? tau[(b * T + j) * H + h] : 1.0));")],
}


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mut_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, workdir):
    text = open(SRC).read()
    for old, new in MUTANTS[name]:
        assert old in text, f"mutation target not found in oracle source: {old!r}"
        text = text.replace(old, new)
    src = os.path.join(workdir, f"{name}.c")
    with open(src, "w") as f:
        f.write(text)
    so = os.path.join(workdir, f"lib_{name}.so")
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-w", "-o", so, src,
                    "-lm"], check=True)
    lib = oracle.load(path=so)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"
