"""Planted mistakes: each mutant is a copy of the oracle source with one
plausible error (a dropped term, a wrong tie rule, a swapped operand, ...),
built on the CPU.  Every mutant must fail at least one pin; a mutant that
passes all of them would mean the pins cannot see that class of mistake.
The real oracle is never modified."""
import os
import subprocess

import pytest

import oracle as O
import oracle_pins as P

SRC = os.path.join(os.path.dirname(O.oracle.__file__), "mita_oracle.c")

MUTANTS = {
    "pool_bin_end_floor": ("*r1 = ceil_div((a + 1) * gh, mh);", "*r1 = floor_div((a + 1) * gh, mh);"),
    "pool_count_off_by_one": ("count = (double)((r1 - r0) * (c1 - c0));",
                              "count = (double)((r1 - r0) * (c1 - c0) + 1);"),
    "bf16_double_rounding": ("ldexp(nearbyint(ldexp(x, -q)), q);",
                             "ldexp(nearbyint(ldexp((double)(float)x, -q)), q);"),
    "bf16_ties_away": ("ldexp(nearbyint(ldexp(x, -q)), q);", "ldexp(round(ldexp(x, -q)), q);"),
    "bf16_seven_bits": ("int q = e - 8;", "int q = e - 7;"),
    "topk_ties_to_high_index": ("return (a->t < b->t) ? -1 : (a->t > b->t);",
                                "return (a->t > b->t) ? -1 : (a->t < b->t);"),
    "topk_smallest_scores": ("if (a->s > b->s) return -1;\n  if (a->s < b->s) return 1;",
                             "if (a->s < b->s) return -1;\n  if (a->s > b->s) return 1;"),
    "topk_skips_best": ("dst[j] = (int32_t)row[j].t;", "dst[j] = (int32_t)row[(j + 1) % N].t;"),
    "landmark_values_unscaled": ("logit[t] = scale * dot(Ql + i * d, K + t * d, d);",
                                 "logit[t] = dot(Ql + i * d, K + t * d, d);"),
    "landmark_values_unnormalised": ("Vl[i * d + j] = acc / z;", "Vl[i * d + j] = acc;"),
    "route_ties_to_last": ("if (v > best_v) { /* strict", "if (v >= best_v) { /* strict"),
    "route_argmin": ("if (v > best_v) { /* strict", "if (v < best_v) { /* strict"),
    "bucket_unstable": ("for (int64_t q = 0; q < N; ++q) perm[fill[route[q]]++] = (int32_t)q;",
                        "for (int64_t q = N - 1; q >= 0; --q) perm[fill[route[q]]++] = (int32_t)q;"),
    "output_drops_compressed_values": (
        "for (int64_t i = 0; i < m; ++i) acc += w[i] * Vl[i * d + c];\n        for (int64_t j = 0;",
        "for (int64_t i = 0; i < m; ++i) acc += 0.0 * Vl[i * d + c];\n        for (int64_t j = 0;"),
    "output_raw_logits_unscaled": ("w[m + j] = scale * dot(Q + q * d,", "w[m + j] = dot(Q + q * d,"),
    "output_wrong_expert": ("const int32_t* ex = idx + (int64_t)route[q] * k;",
                            "const int32_t* ex = idx + (int64_t)((route[q] + 1) % m) * k;"),
    "output_keys_as_values": ("acc += w[m + j] * V[(int64_t)ex[j] * d + c];",
                              "acc += w[m + j] * K[(int64_t)ex[j] * d + c];"),
    "output_compressed_keys_from_k": (
        "w[i] = scale * dot(Q + q * d, Ql + i * d, d);\n        if (w[i] > mx) mx = w[i];\n      }\n      for (int64_t j = 0;",
        "w[i] = scale * dot(Q + q * d, K + i * d, d);\n        if (w[i] > mx) mx = w[i];\n      }\n      for (int64_t j = 0;"),
    "route_s_ties_to_high_index": ("if (best < 0 || R[i] > R[best]) best = i;",
                                   "if (best < 0 || R[i] >= R[best]) best = i;"),
    "route_s_smallest_logits": ("if (best < 0 || R[i] > R[best]) best = i;",
                                "if (best < 0 || R[i] < R[best]) best = i;"),
    "route_s_repeats_best": ("if (taken[i]) continue;", "if (0) continue;"),
    "bucket_s_unstable": ("for (int64_t q = 0; q < N; ++q)\n    for (int64_t j = 0; j < s; ++j) perm[",
                          "for (int64_t q = N - 1; q >= 0; --q)\n    for (int64_t j = 0; j < s; ++j) perm["),
    "output_s_repeats_first_expert": ("key[j * k + t] = idx[(int64_t)routes[q * s + j] * k + t];",
                                      "key[j * k + t] = idx[(int64_t)routes[q * s] * k + t];"),
    "output_s_raw_logits_unscaled": ("w[m + t] = scale * dot(", "w[m + t] = dot("),
    "output_s_drops_compressed_values": (
        "for (int64_t i = 0; i < m; ++i) acc += w[i] * Vl[i * d + c];\n        for (int64_t t = 0;",
        "for (int64_t i = 0; i < m; ++i) acc += 0.0 * Vl[i * d + c];\n        for (int64_t t = 0;"),
    # the near-tie report that the comparison protocol's band is built from
    "abs_dot_inflated": ("s += fabs(a[j] * b[j]);", "s += 100.0 * fabs(a[j] * b[j]);"),
    "abs_dot_signed": ("s += fabs(a[j] * b[j]);", "s += a[j] * b[j];"),
    "gap_bound_of_best_key": ("g[2] = abs_dot(Ql + i * d, K + row[k - 1].t * d, d);",
                              "g[2] = abs_dot(Ql + i * d, K + row[0].t * d, d);"),
    "gap_next_bound_of_kth_key": ("g[3] = abs_dot(Ql + i * d, K + row[k].t * d, d);",
                                  "g[3] = abs_dot(Ql + i * d, K + row[k - 1].t * d, d);"),
    "route_runner_up_bound_zero": (
        "g[3] = second_i >= 0 ? abs_dot(Q + q * d, Ql + second_i * d, d) : 0.0;",
        "g[3] = 0.0;"),
    "route_best_bound_of_landmark0": ("g[2] = abs_dot(Q + q * d, Ql + best * d, d);",
                                      "g[2] = abs_dot(Q + q * d, Ql, d);"),
    "route_runner_up_ties_to_last": ("if (v > second) {", "if (v >= second) {"),
    "dense_unscaled": ("w[t] = scale * dot(Q + q * d, K + t * d, d);",
                       "w[t] = dot(Q + q * d, K + t * d, d);"),
    "dense_unnormalised": ("out[p * d + c] = sum / total;", "out[p * d + c] = sum;"),
    "dense_keys_as_values": ("sum += w[t] * V[t * d + c];", "sum += w[t] * K[t * d + c];"),
    "dense_drops_last_key": ("        total += w[t];\n", "        total += (t + 1 < N) ? w[t] : 0.0;\n"),
    # backward pass with the experts and routes held fixed
    "backward_drops_softmax_correction": (
        "const double g = scale * w[m + j] * (dw[m + j] - c);",
        "const double g = scale * w[m + j] * dw[m + j];"),
    "backward_landmark_logit_unscaled": ("const double g = scale * w[i] * (dw[i] - c);",
                                         "const double g = w[i] * (dw[i] - c);"),
    "backward_pool_not_averaged": ("dQ[t * d + a] += dQl[i * d + a] / cnt;",
                                   "dQ[t * d + a] += dQl[i * d + a];"),
    "backward_drops_landmark_value_path": ("dV[t * d + a] += w[t] * dVl[i * d + a];",
                                           "dV[t * d + a] += 0.0 * dVl[i * d + a];"),
    "backward_cross_attention_keys_get_query": ("dK[t * d + a] += g * Ql[i * d + a];",
                                                "dK[t * d + a] += g * Q[i * d + a];"),
    "backward_dq_uses_values": ("dQ[q * d + a] += g * K[t * d + a];",
                                "dQ[q * d + a] += g * V[t * d + a];"),
    "backward_landmark_grad_not_fed_back": ("dQl[i * d + a] += g * K[t * d + a];",
                                            "dQl[i * d + a] += 0.0 * K[t * d + a];"),
    "backward_compressed_value_grad_unweighted": ("dVl[i * d + a] += w[i] * G[a];",
                                                  "dVl[i * d + a] += G[a];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mut = tmp_path / "mutant.c"
    mut.write_text(src.replace(old, new))
    (tmp_path / "mita_oracle.h").write_text(open(SRC[:-1] + "h").read())
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-std=c11", "-O1", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                    "-w", "-o", str(so), str(mut), "-lm"], check=True)
    caught = []
    with O.use_library(str(so)):
        for check in P.ALL_CHECKS:
            try:
                check()
            except Exception:  # any failure of a pin counts as detection
                caught.append(check.__name__)
    assert caught, f"no pin detects mutant {name}"
