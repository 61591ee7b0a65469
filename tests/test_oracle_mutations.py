"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of oracle/dust_oracle.c (a wrong Philox
constant, a dropped key advance, swapped counter words, a wrong Box-Muller radius, a flipped
sign, a missing sigma, a scan that leaks across sequences, an off-by-one chunk, an optimizer
step without bias correction, a softmax re-run against unnormalised weights, ...), builds it,
swaps it in for the oracle's library, and requires that at least one of the pins the other
oracle tests use rejects it. The real oracle passes all of them (tests/test_oracle_*.py).
"""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_attn as attn
import test_oracle_generator as gen
import test_oracle_helpers as helpers
import test_oracle_optim as optim
import test_oracle_perturbed_linear as plin
import test_oracle_steps as steps

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "dust_oracle.c")


@pytest.fixture(scope="module")
def rocrand_exe(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        return None
    exe = str(tmp_path_factory.mktemp("xcheck_mut") / "xcheck")
    subprocess.check_call([hipcc, "-O1", "-o", exe, os.path.join(HERE, "rocrand_philox_xcheck.cpp")])
    return exe


def _pin_rocrand(exe):
    def pin():
        if exe is None:
            return
        g = np.random.default_rng(3)
        cases = [(int(g.integers(0, 2**62)), int(g.integers(0, 2**32)), int(g.integers(0, 2**32)),
                  int(g.integers(0, 2**30)), int(g.integers(0, 2**32))) for _ in range(64)]
        lines = ["%d %d %d" % (s, dr | (tg << 32), 4 * (q | (tk << 32))) for s, tg, dr, tk, q in cases]
        out = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True,
                             check=True).stdout.split()
        ref = np.array([int(v) for v in out], dtype=np.uint64).reshape(-1, 4)
        got = np.array([oracle.noise_words(*c) for c in cases], dtype=np.uint64)
        assert np.array_equal(got, ref)
    return pin


def _pin_normal_moments():
    n = oracle.normals(0xBEEF, 1, 0, 0, 0, 4, 256, 256).ravel()
    N = n.size
    assert np.all(np.isfinite(n))
    assert abs(n.mean()) < 5 / np.sqrt(N) and abs(n.var() - 1) < 5 * np.sqrt(2 / N)


PINS_STEPS = [
    steps.test_inject_sigma_zero_is_identity,
    steps.test_inject_leading_dimension_and_offsets,
    steps.test_loss_delta_loss_is_clean_minus_perturbed,
    steps.test_loss_delta_inner_matches_einsum,
    steps.test_scan_gamma_zero_keeps_own_token,
    steps.test_scan_impulse_response,
    steps.test_scan_constant_input_geometric_series,
    lambda: steps.test_scan_brute_force(0.9),
    steps.test_error_estimate_brute_force_tiny,
    steps.test_error_estimate_chunked_population_equals_one_pass,
    lambda: steps.test_error_estimate_recovers_linear_loss_gradient(0.0),
    lambda: steps.test_error_estimate_recovers_linear_loss_gradient(0.9),
    lambda: steps.test_head_ce_matches_torch_cross_entropy(64, 12, 20),
    lambda: steps.test_head_ce_matches_torch_cross_entropy(97, 88, 9),
    steps.test_head_ce_sigma_zero_and_large_logits,
    gen.test_box_muller_at_special_angles,
    lambda: optim.test_sgd_momentum_matches_torch(0.05, 0.9),
    lambda: optim.test_adam_matches_torch(1e-2, 0.9, 0.999, 1e-8, 0.1),
    optim.test_adam_first_step_and_weight_decay_closed_forms,
    lambda: attn.test_scores_equal_an_explicit_attention_rerun(2, 2, 16, 8, 3, 0, 0, 0),
    lambda: attn.test_scores_equal_an_explicit_attention_rerun(1, 3, 24, 4, 2, 64, 5, 100),
    attn.test_identity_attention_is_the_own_token_inner_product,
    attn.test_linear_in_sigma_and_blind_above_the_diagonal,
    lambda: attn.test_key_scores_equal_an_explicit_attention_rerun(2, 2, 12, 8, 3, 0, 0, 0),
    lambda: attn.test_key_scores_equal_an_explicit_attention_rerun(1, 3, 20, 4, 2, 64, 5, 100),
    attn.test_key_scores_first_order_is_the_softmax_jacobian,
    attn.test_key_scores_invariant_to_row_scale_and_blind_above_the_diagonal,
    attn.test_key_scores_vanish_at_sigma_zero_and_for_self_attention,
    lambda: attn.test_query_scores_equal_an_explicit_attention_rerun(2, 2, 12, 8, 3, 0, 0, 0),
    lambda: attn.test_query_scores_equal_an_explicit_attention_rerun(1, 3, 20, 4, 2, 64, 5, 100),
    attn.test_query_scores_first_order_is_the_softmax_jacobian,
    attn.test_query_scores_row_scale_diagonal_and_zeros,
    lambda: attn.test_row_weights_reproduce_an_explicit_softmax_rerun(2, 2, 12, 8),
    attn.test_row_weights_invariants,
    helpers.test_round_bf16_equals_exhaustive_nearest_even_on_ties_subnormals_and_overflow,
    helpers.test_round_bf16_equals_torch_on_fp32_values,
    lambda: helpers.test_normals_at_equals_slices_of_bulk_normals(3, 7, 2**32 + 8),
    lambda: helpers.test_head_ce_at_equals_torch_cross_entropy_of_perturbed_logits(64, 12, 20),
    lambda: plin.test_activation_equals_torch(*plin.ACTS[2]),
    lambda: plin.test_activation_equals_torch(*plin.ACTS[3]),
    lambda: plin.test_perturbed_linear_equals_torch_linear_of_explicit_inputs(*plin.ACTS[3], 7, 300, 2**32 + 64),
    plin.test_sigma_zero_is_the_clean_product_and_the_output_is_affine_in_sigma,
    plin.test_sampled_rows_equal_the_bulk_operand,
    lambda: attn.test_key_and_query_scores_at_large_shifts("keys", 300.0),
    lambda: attn.test_key_and_query_scores_at_large_shifts("queries", 300.0),
]

# (id, text in dust_oracle.c, replacement)
MUTATIONS = [
    ("philox multiplier", "(uint64_t)0xD2511F53u * (uint64_t)x0", "(uint64_t)0xD2511F57u * (uint64_t)x0"),
    ("philox low/high swap", "uint32_t y1 = (uint32_t)pb;", "uint32_t y1 = (uint32_t)(pb >> 32);"),
    ("philox no key advance", "k0 += 0x9E3779B9u;", "k0 += 0u;"),
    ("philox nine rounds", "round < 10; ++round", "round < 9; ++round"),
    ("counter token/draw swapped", "uint32_t ctr[4] = {q, token, draw, tag};", "uint32_t ctr[4] = {q, draw, token, tag};"),
    ("box-muller radius", "double rho = sqrt(-2.0 * log(dust_or_uniform(wa)));",
     "double rho = sqrt(-log(dust_or_uniform(wa)));"),
    ("angle centred in its bin", "return (double)(w >> 9) * (1.0 / 8388608.0);",
     "return ((double)(w >> 9) + 0.5) * (1.0 / 8388608.0);"),
    ("cos and sin swapped", "return sine ? rho * sin(theta) : rho * cos(theta);",
     "return sine ? rho * cos(theta) : rho * sin(theta);"),
    ("uniform bit width", "return ((double)(w >> 9) + 0.5) * (1.0 / 8388608.0);",
     "return ((double)(w >> 8) + 0.5) * (1.0 / 8388608.0);"),
    ("inject sign", "y[t * ld_y + j] +\n                    sigma", "y[t * ld_y + j] -\n                    sigma"),
    ("inject channel offset dropped",
     "(uint32_t)(draw0 + k), (uint32_t)(tok0 + t),\n                                           (uint64_t)(chan0 + j));",
     "(uint32_t)(draw0 + k), (uint32_t)(tok0 + t),\n                                           (uint64_t)(j));"),
    ("bulk normals ignore token offset", "(uint32_t)(tok0 + t),\n                                                          (uint64_t)(chan0 + j));",
     "(uint32_t)(t),\n                                                          (uint64_t)(chan0 + j));"),
    ("loss change sign", "c[i * T + t] = loss_clean[t] - loss_pert[i * T + t];",
     "c[i * T + t] = loss_pert[i * T + t] - loss_clean[t];"),
    ("inner score sign", "c[i * T + s] = -acc;", "c[i * T + s] = acc;"),
    ("scan off by one", "r[i * T + t] = c[i * T + t] + gamma * r[i * T + t + 1];",
     "r[i * T + t] = gamma * (c[i * T + t] + r[i * T + t + 1]);"),
    ("scan leaks across sequences", "r[i * T + last] = c[i * T + last];",
     "r[i * T + last] = c[i * T + last] + (last + 1 < T ? gamma * c[i * T + last + 1] : 0.0);"),
    ("estimate without sigma", "double scale = -1.0 / ((double)K_total * sigma);\n    #pragma omp parallel for collapse(2)",
     "double scale = -1.0 / ((double)K_total);\n    #pragma omp parallel for collapse(2)"),
    ("estimate sign", "double scale = -1.0 / ((double)K_total * sigma);\n    #pragma omp parallel for collapse(2)",
     "double scale = 1.0 / ((double)K_total * sigma);\n    #pragma omp parallel for collapse(2)"),
    ("estimate ignores draw0", "acc += r[i * T + t] * dust_or_normal(seed, tag, (uint32_t)(draw0 + i),",
     "acc += r[i * T + t] * dust_or_normal(seed, tag, (uint32_t)(i),"),
    ("head target not perturbed", "if (j == y) zy = zj;", "if (j == y) zy = z[j];"),
    ("head chunk off by one", "if (j >= v0 && j < v0 + C)\n                    zj += sigma * dust_or_normal(seed, tag, (uint32_t)(draw0 + i),\n                                                 (uint32_t)(tok0 + t), (uint64_t)j);\n                if (zj > m)",
     "if (j >= v0 && j <= v0 + C)\n                    zj += sigma * dust_or_normal(seed, tag, (uint32_t)(draw0 + i),\n                                                 (uint32_t)(tok0 + t), (uint64_t)j);\n                if (zj > m)"),
    ("head clean loss drops max", "loss_clean[t] = m + log(s) - z[y];", "loss_clean[t] = log(s) - z[y];"),
    ("sgd momentum dampened", "buf[i] = mu * buf[i] + g[i];", "buf[i] = mu * buf[i] + (1.0 - mu) * g[i];"),
    ("adam without bias correction", "w[i] = w[i] - lr * (m[i] / bc1) / (sqrt(v[i] / bc2) + eps);",
     "w[i] = w[i] - lr * m[i] / (sqrt(v[i]) + eps);"),
    ("adam decay coupled to the gradient", "w[i] = w[i] * (1.0 - lr * wd);\n        m[i] = b1 * m[i] + (1.0 - b1) * g[i];",
     "m[i] = b1 * m[i] + (1.0 - b1) * (g[i] + wd * w[i]);"),
    ("adam eps inside the root", "(sqrt(v[i] / bc2) + eps)", "sqrt(v[i] / bc2 + eps)"),
    ("attention scores not causal", "for (int64_t sl = 0; sl <= tl; ++sl) {\n                    const double p = P[((b * H + h) * S + tl) * S + sl];",
     "for (int64_t sl = 0; sl < S; ++sl) {\n                    const double p = P[((b * H + h) * S + tl) * S + sl];"),
    ("attention noise at the query token", "(uint32_t)(tok0 + b * S + sl),\n                                              (uint64_t)(chan0 + h * dh + j))",
     "(uint32_t)(tok0 + t),\n                                              (uint64_t)(chan0 + h * dh + j))"),
    ("attention head offset dropped", "(uint64_t)(chan0 + h * dh + j)) *", "(uint64_t)(chan0 + j)) *"),
    ("key scores against unnormalised weights", "/ den - prow[sl] / Z)", "/ den - prow[sl])"),
    ("key logit shift without the softmax scale", "dl[sl] = sigma * tau * dot;", "dl[sl] = sigma * dot;"),
    ("key score sign", "    return -acc;\n}", "    return acc;\n}"),
    ("key noise at the query token", "dust_or_normal(seed, tag, draw, (uint32_t)(tok0 + b * S + sl),",
     "dust_or_normal(seed, tag, draw, (uint32_t)(tok0 + t),"),
    ("key logit uses the key token's query", "dot += q[t * d + h * dh + j] *",
     "dot += q[(b * S + sl) * d + h * dh + j] *"),
    ("key scores not causal", "for (int64_t sl = 0; sl <= tl; ++sl) {\n            double dot = 0.0;",
     "for (int64_t sl = 0; sl < S; ++sl) {\n            double dot = 0.0;"),
    ("key output change drops the value", "* exp(dl[sl] - mx) / den - prow[sl] / Z) *\n                      v[(b * S + sl) * d + h * dh + j];",
     "* exp(dl[sl] - mx) / den - prow[sl] / Z) *\n                      v[t * d + h * dh + j];"),
    ("query noise at the sequence start", "a[j] = dust_or_normal(seed, tag, draw, (uint32_t)(tok0 + t),",
     "a[j] = dust_or_normal(seed, tag, draw, (uint32_t)(tok0 + b * S),"),
    ("query logit uses the query's own key", "dot += a[j] * k[(b * S + sl) * d + h * dh + j];",
     "dot += a[j] * k[t * d + h * dh + j];"),
    ("query logit shift without the softmax scale",
     "dot += a[j] * k[(b * S + sl) * d + h * dh + j];\n            dl[sl] = sigma * tau * dot;",
     "dot += a[j] * k[(b * S + sl) * d + h * dh + j];\n            dl[sl] = sigma * dot;"),
    ("query score sign", "    return -acc;\n}\n\nvoid dust_or_attn_query_scores(",
     "    return acc;\n}\n\nvoid dust_or_attn_query_scores("),
    ("row weights without the base", "wrow[s] = prow[s] * (z * u - base);",
     "wrow[s] = prow[s] * (z * u);"),
    ("row weights without Z", "wrow[s] = prow[s] * (z * u - base);",
     "wrow[s] = prow[s] * (u - base);"),
    ("row weights' inner product on the query's value",
     "u += v[(b * S + s) * d + h * dh + j] * g[(b * S + t) * d + h * dh + j];\n                    wrow",
     "u += v[(b * S + t) * d + h * dh + j] * g[(b * S + t) * d + h * dh + j];\n                    wrow"),
    ("row sum includes the diagonal's successor", "for (int64_t s = 0; s <= t; ++s) {\n                    double u = 0.0;",
     "for (int64_t s = 0; s <= t + (t + 1 < S); ++s) {\n                    double u = 0.0;"),
    ("bf16 ties away from zero", "(rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0))",
     "(rem >= 0.5)"),
    ("bf16 subnormals at fp32's spacing", "if (qexp < -133) qexp = -133;", "if (qexp < -149) qexp = -149;"),
    ("bf16 overflow saturates", "v = INFINITY;   /* beyond", "v = 3.3895313892515355e38;   /* beyond"),
    ("sampled normals ignore draw0", "out[m] = dust_or_normal(seed, tag, (uint32_t)(draw0 + k[m]),",
     "out[m] = dust_or_normal(seed, tag, (uint32_t)(k[m]),"),
    ("sampled normals drop the channel offset", "(uint64_t)(chan0 + j[m]));", "(uint64_t)(j[m]));"),
    ("sampled head loss: target not perturbed", "if (zj > mx) mx = zj;\n            if (j == y) zy = zj;",
     "if (zj > mx) mx = zj;\n            if (j == y) zy = z[j];"),
    ("sampled head loss: chunk off by one", "if (j >= v0 && j < v0 + C)\n                zj += sigma * dust_or_normal(seed, tag, (uint32_t)(draw0 + k[m]),\n                                             (uint32_t)(tok0 + t[m]), (uint64_t)j);\n            if (zj > mx)",
     "if (j > v0 && j < v0 + C)\n                zj += sigma * dust_or_normal(seed, tag, (uint32_t)(draw0 + k[m]),\n                                             (uint32_t)(tok0 + t[m]), (uint64_t)j);\n            if (zj > mx)"),
    ("activation before the noise", "row[j] = dust_or_activation(\n                    y[t * d + j] + sigma",
     "row[j] = dust_or_activation(y[t * d + j], act) + sigma * dust_or_activation(\n                    sigma"),
    ("next layer's weight transposed", "acc += row[j] * w[n * d + j];", "acc += row[j] * w[(j % n_out) * d + n % d];"),
    ("perturbed product drops the token offset", "(uint32_t)(tok0 + t),\n                                                          (uint64_t)(chan0 + j)),\n                    act);",
     "(uint32_t)(t),\n                                                          (uint64_t)(chan0 + j)),\n                    act);"),
    ("gelu cubic coefficient", "(x + 0.044715 * x * x * x)", "(x + 0.04 * x * x * x)"),
    ("squared relu left linear", "if (act == 2) return x > 0.0 ? x * x : 0.0;", "if (act == 2) return x > 0.0 ? x : 0.0;"),
    ("sampled perturbed rows ignore draw0", "sigma * dust_or_normal(seed, tag, (uint32_t)(draw0 + k[q]),",
     "sigma * dust_or_normal(seed, tag, (uint32_t)(k[q]),"),
    ("query head offset dropped", "(uint64_t)(chan0 + h * dh + j));\n        double Z",
     "(uint64_t)(chan0 + j));\n        double Z"),
    ("key re-run without the row maximum", "            Z += prow[sl];\n            if (dl[sl] > mx) mx = dl[sl];",
     "            Z += prow[sl];\n            if (dl[sl] > mx) mx = 0.0;"),
    ("query re-run without the row maximum",
     "dot += a[j] * k[(b * S + sl) * d + h * dh + j];\n            dl[sl] = sigma * tau * dot;\n            Z += prow[sl];\n            if (dl[sl] > mx) mx = dl[sl];",
     "dot += a[j] * k[(b * S + sl) * d + h * dh + j];\n            dl[sl] = sigma * tau * dot;\n            Z += prow[sl];\n            if (dl[sl] > mx) mx = 0.0;"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_reject_planted_mistake(name, old, new, tmp_path, rocrand_exe):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor not found: %s" % name
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new, 1))
    lib_path = str(tmp_path / "libmutant.so")
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-o", lib_path,
                           str(mutant_src), "-lm"])
    saved = oracle._load()
    oracle._lib = oracle._configure(ctypes.CDLL(lib_path))
    failed = []
    try:
        for pin in [_pin_rocrand(rocrand_exe), _pin_normal_moments] + PINS_STEPS:
            try:
                pin()
            except (AssertionError, ValueError, FloatingPointError):
                failed.append(getattr(pin, "__name__", "pin"))
    finally:
        oracle._lib = saved
    assert failed, "no pin rejected the planted mistake '%s'" % name
