"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a private copy of the oracle's C source
(built into a temporary directory, on the CPU), runs the pin suite against
that copy in a child process, and requires at least one pin to fail.
"""
import os
import subprocess
import sys

import pytest

from oracle import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))

MUTANTS = {
    "eta_theta_swapped": ("Sx[p] = eta_n * Sx[p] - th[n] * g[p];", "Sx[p] = th[n] * Sx[p] - eta_n * g[p];"),
    "keep_factor_for_forget": ("W[p] = (1.0 - al[n]) * W[p] + Sx[p];", "W[p] = al[n] * W[p] + Sx[p];"),
    "window_off_by_one": ("int i0 = n - c + 1;", "int i0 = n - c;"),
    "error_sign": ("s * gamma * (f[o] - v[o])", "s * gamma * (v[o] - f[o])"),
    "gelu_prime_dropped": ("d1[j] = back * gelu_prime(z[j]) * (gt", "d1[j] = back * gelu(z[j]) * (gt"),
    "w2_transposed_in_backward": ("back += W2[(long)o * h + j] * d2[o];", "back += W2[(long)j * cfg->d_v + o] * d2[o];"),
    "poly2_diagonal_dropped": ("for (int b = a; b < p; ++b)", "for (int b = a + 1; b < p; ++b)"),
    "residual_dropped": ("y[o] += cfg->residual ? r[o] : 0.0;", "y[o] += 0.0;"),
    "halo_ignored": ("if (lo < -halo_valid) lo = -halo_valid;", "if (lo < 0) lo = 0;"),
    "dot_bias_sign": ("-s * gamma * v[o]", "s * gamma * v[o]"),
    "tanh_gelu": ("return 0.5 * z * (1.0 + erf(z / sqrt(2.0)));", "return 0.5 * z * (1.0 + tanh(z));"),
    "stale_chunk_start_state": ("memcpy(Wc, W, sizeof(double) * P);", "if (t0 == 0) memcpy(Wc, W, sizeof(double) * P);"),
    "lp_exponent_p": ("sign_a(e, alpha) * pow(fabs(e), p - 1.0)", "sign_a(e, alpha) * pow(fabs(e), p)"),
    "lp_sign_dropped": ("sign_a(e, alpha) * pow(fabs(e), p - 1.0)", "pow(fabs(e), p - 1.0)"),
    "smooth_sign_slope": ("alpha > 0.0 ? tanh(alpha * e) : sgn(e)", "alpha > 0.0 ? tanh(e) : sgn(e)"),
    "huber_l1_norm_test": ("n2 += (f[o] - v[o]) * (f[o] - v[o]);", "n2 += fabs(f[o] - v[o]); n2 *= 1.0;"),
    "huber_branches_swapped": ("huber_small ? f[o] - v[o] : delta * sign_a(f[o] - v[o], cfg->sign_alpha)",
                               "huber_small ? delta * sign_a(f[o] - v[o], cfg->sign_alpha) : f[o] - v[o]"),
    "huber_delta_dropped": ("huber_small ? f[o] - v[o] : delta * sign_a(f[o] - v[o], cfg->sign_alpha)",
                            "huber_small ? f[o] - v[o] : sign_a(f[o] - v[o], cfg->sign_alpha)"),
    "huber_halo_threshold_lost": ("nd[j] = huber ? dl[i] : 0.0;", "nd[j] = 0.0;"),
    "huber_squared_norm_test": ("huber_small = sqrt(n2) <= delta;", "huber_small = n2 <= delta;"),
    "ln_mean_term_dropped": ("(d2[o] - mg - nh[o] * mgn) / sd", "(d2[o] - nh[o] * mgn) / sd"),
    "ln_nhat_term_dropped": ("(d2[o] - mg - nh[o] * mgn) / sd", "(d2[o] - mg) / sd"),
    "ln_sd_dropped": ("(d2[o] - mg - nh[o] * mgn) / sd", "(d2[o] - mg - nh[o] * mgn)"),
    "ln_unbiased_variance": ("  var /= n;", "  var /= n - 1;"),
    "ln_eps_outside_sqrt": ("const double sd = sqrt(var + eps);", "const double sd = sqrt(var) + eps;"),
    "gated_z3_dropped_in_d1": ("d1[j] = back * gelu_prime(z[j]) * (gt ? z[h + j] : 1.0);", "d1[j] = back * gelu_prime(z[j]);"),
    "gated_d3_with_gelu_prime": ("if (gt) d1[h + j] = back * gelu(z[j]);", "if (gt) d1[h + j] = back * gelu_prime(z[j]);"),
    "gated_w3_block_misplaced": ("double* gW3 = gW2 + (long)dv * h;", "double* gW3 = g;"),
    "muon_ns_coefficient": ("const double a = 3.4445, b = -4.7750, c = 2.0315;", "const double a = 3.4445, b = -4.7750, c = 2.0;"),
    "muon_frobenius_norm_dropped": ("nrm = sqrt(nrm) + 1e-7;", "nrm = 1.0;"),
    "muon_steps_off_by_one": ("for (int s = 0; s < steps; ++s) {", "for (int s = 0; s <= steps; ++s) {"),
    "muon_theta_inside_momentum": ("Sx[p] = eta_n * Sx[p] + g[p];", "Sx[p] = eta_n * Sx[p] + th[n] * g[p];"),
    "muon_momentum_sign": ("Sx[p] = eta_n * Sx[p] + g[p];", "Sx[p] = eta_n * Sx[p] - g[p];"),
    "muon_decay_on_step": ("W[p] = (1.0 - al[n]) * W[p] - th[n] * O[p];", "W[p] = (1.0 - al[n]) * (W[p] - th[n] * O[p]);"),
    "muon_one_matrix_for_the_mlp": ("const int nm = weight_matrices(cfg, rows, cols);",
                                    "int nm = weight_matrices(cfg, rows, cols); nm = 1; rows[0] = 1; cols[0] = (int)P;"),
    "ln_residual_dropped": ("y[o] += cfg->residual ? r[o] : 0.0;", "y[o] += cfg->residual && !cfg->layernorm ? r[o] : 0.0;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(O.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found"
    mut = tmp_path / "atlas_oracle.c"
    mut.write_text(src.replace(old, new))
    (tmp_path / "atlas_oracle.h").write_text(open(os.path.join(os.path.dirname(O.SRC), "atlas_oracle.h")).read())
    lib = O.build(str(mut), str(tmp_path / "liboracle_mut.so"))
    env = dict(os.environ, ATLAS_ORACLE_LIB=lib)
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle_pins.py")],
                       env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
