"""The pins catch plausible mistakes: each mutant below is the oracle source
with one planted error (a dropped term, a wrong index, a transposed operand,
a wrong sign ...), built on the CPU; at least one pin must fail on every one.
Every mutant keeps all memory accesses in bounds."""
import os

import pytest

import oracle
from tests import pins

MUTANTS = {
    "mean_over_k_minus_1": ("ss / (double)K + eps", "ss / (double)(K > 1 ? K - 1 : 1) + eps"),
    "eps_outside_sqrt": ("sqrt(ss / (double)K + eps)", "(sqrt(ss / (double)K) + eps)"),
    "eps_dropped": ("sqrt(ss / (double)K + eps)", "sqrt(ss / (double)K)"),
    "sqrt_dropped": ("sqrt(ss / (double)K + eps)", "(ss / (double)K + eps)"),
    "multiply_by_rms": ("(X[m * K + k] / r[m]) * g[k]", "(X[m * K + k] * r[m]) * g[k]"),
    "gain_dropped": ("(X[m * K + k] / r[m]) * g[k]", "(X[m * K + k] / r[m])"),
    "gain_wrong_index": ("(X[m * K + k] / r[m]) * g[k]", "(X[m * K + k] / r[m]) * g[m % K]"),
    "abs_not_square": ("ss += X[m * K + k] * X[m * K + k]", "ss += fabs(X[m * K + k])"),
    "k_loop_short": ("for (int64_t k = 0; k < K; ++k) ss +=",
                     "for (int64_t k = 0; k < K - 1; ++k) ss +="),
    "transposed_weight": ("y[n] += a * b[n];", "y[n] += a * B[(n * K + k) % (K * N)];"),
    "weight_row_off_by_one": ("const double* b = B + k * N;",
                              "const double* b = B + ((k + 1) % K) * N;"),
    "gate_sign": ("z1 / (1.0 + exp(-z1)) * Z3[i]", "z1 / (1.0 + exp(z1)) * Z3[i]"),
    "gate_swapped": ("z1 / (1.0 + exp(-z1)) * Z3[i]", "Z3[i] / (1.0 + exp(-Z3[i])) * z1"),
    "gate_no_silu": ("z1 / (1.0 + exp(-z1)) * Z3[i]", "z1 * Z3[i]"),
    "gate_both_w1": ("matmul(A, W3, M, N, K, Z3);", "matmul(A, W1, M, N, K, Z3);"),
    "lora_a_transposed": ("t += Act[m * K + k] * A[r * K + k];",
                          "t += Act[m * K + k] * A[(k * R + r) % (R * K)];"),
    "lora_term_dropped": ("Y[m * N + n] += t * B[r * N + n];", "Y[m * N + n] += 0.0 * B[r * N + n];"),
    "lora_term_sign": ("Y[m * N + n] += t * B[r * N + n];", "Y[m * N + n] -= t * B[r * N + n];"),
    "lora_b_row_wrong": ("Y[m * N + n] += t * B[r * N + n];",
                         "Y[m * N + n] += t * B[((r + 1) % R) * N + n];"),
    "lora_raw_x": ("lora_products(Nrm, W, A, B, M, N, K, R, Y);",
                   "lora_products(X, W, A, B, M, N, K, R, Y);"),
    "attn_scale_missing": ("sc[s] = dot / sqrt((double)D);", "sc[s] = dot;"),
    "attn_scale_by_d": ("sc[s] = dot / sqrt((double)D);", "sc[s] = dot / (double)D;"),
    "attn_gk_on_query": ("normalise(Q + h * D, gq, &rq, 1, D, qn);",
                         "normalise(Q + h * D, gk, &rq, 1, D, qn);"),
    "attn_key_rms_of_query": ("normalise(k, gk, &rk, 1, D, kn + s * D);",
                              "normalise(k, gk, &rq, 1, D, kn + s * D);"),
    "attn_no_max_shift": ("sc[s] = exp(sc[s] - mx);", "sc[s] = exp(sc[s]);"),
    "attn_values_reversed": ("const double* v = Vh + s * D;",
                             "const double* v = Vh + (S - 1 - s) * D;"),
    "attn_unnormalised_weights": ("const double p = sc[s] / den;", "const double p = sc[s];"),
    "prefill_mask_ignored": ("const int64_t nk = causal ? i + Skv - Sq + 1 : Skv;",
                             "const int64_t nk = causal ? Skv : Skv;"),
    "prefill_head_of_query": ("const int64_t h = qh / G;", "const int64_t h = qh % BH;"),
    "prefill_key_gain_is_query_gain": ("normalise(key, gk, &rkey, 1, D, kn + s * D);",
                                       "normalise(key, gq, &rkey, 1, D, kn + s * D);"),
    "lora_last_rank_skipped": ("for (int64_t r = 0; r < R; ++r) {\n      double t = 0.0;",
                               "for (int64_t r = 0; r < R - 1; ++r) {\n      double t = 0.0;"),
}


def _build(tmp_path, name, src_text):
    src = os.path.join(tmp_path, f"{name}.c")
    with open(src, "w") as f:
        f.write(src_text)
    return oracle.load(oracle.build(force=True, src=src, out=os.path.join(tmp_path, f"lib{name}.so")))


@pytest.fixture(scope="module")
def source():
    with open(oracle._SRC) as f:
        return f.read()


def test_unmutated_copy_passes(tmp_path, source):
    lib = _build(str(tmp_path), "copy", source)
    for pin in pins.ALL_PINS:
        pin(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, source, name):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site for {name} not unique/found"
    lib = _build(str(tmp_path), name, source.replace(old, new))
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches mutant {name}"
