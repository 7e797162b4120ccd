"""Plant one plausible mistake at a time in a copy of the oracle and check that
at least one pin catches it (CPU only; the oracle source itself is untouched)."""
import os

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (name, original text, planted mistake[, number of sites])
MUTANTS = [
    ("router_tie_to_higher", "if (l[e] > l[i0]) i0 = e;", "if (l[e] >= l[i0]) i0 = e;"),
    ("router_second_tie", "if (e != i0 && l[e] > l[i1]) i1 = e;", "if (e != i0 && l[e] >= l[i1]) i1 = e;"),
    ("router_no_renorm", "g[2 * t] = (float)(p0 / (p0 + p1));", "g[2 * t] = (float)p0;"),
    ("router_slots_swapped", "idx[2 * t] = i0;\n        idx[2 * t + 1] = i1;",
     "idx[2 * t] = i1;\n        idx[2 * t + 1] = i0;"),
    ("router_Wr_transposed", "ld(Wr, j * (int64_t)E + e, dt)", "ld(Wr, (int64_t)e * d + j, dt)"),
    ("router_softmax_sign", "double p1 = exp(l[i1] - l[i0]) / den;", "double p1 = exp(l[i0] - l[i1]) / den;"),
    ("switch_sign", "double v = w - Dold + Dnew;", "double v = w + Dold + Dnew;"),
    ("switch_drop_old", "double v = w - Dold + Dnew;", "double v = w + Dnew;"),
    ("switch_no_scale", "D += s * (double)g[k] * acc;", "D += (double)g[k] * acc;"),
    ("switch_no_gate", "D += s * (double)g[k] * acc;", "D += s * acc;"),
    ("switch_B_transposed", "ld(B, ((int64_t)e * d_out + i) * r + rho, dt)",
     "ld(B, ((int64_t)e * r + rho) * d_out + i, dt)"),
    ("switch_one_slot", "double D = 0.0;\n    for (int k = 0; k < 2; ++k) {",
     "double D = 0.0;\n    for (int k = 0; k < 1; ++k) {"),
    ("switch_A_index", "ld(A, ((int64_t)e * r + rho) * d_in + j, dt);\n            acc += b * a;",
     "ld(A, ((int64_t)e * r + rho) * d_in + (d_in - 1 - j), dt);\n            acc += b * a;"),
    ("round_truncate", "double nr = nearbyint(n);", "double nr = trunc(n);"),
    ("round_ties_away", "double nr = nearbyint(n);", "double nr = round(n);"),
    ("round_subnormal", "if (qexp < -133) qexp = -133;", "if (qexp < -126) qexp = -126;"),
    ("sgmm_no_gate", "double c = s * (double)g[2 * t + k];", "double c = s;"),
    ("sgmm_B_wrong_expert", "double b = ld(B, ((int64_t)e * d_out + o) * r + rho, dt);",
     "double b = ld(B, ((int64_t)idx[2 * t] * d_out + o) * r + rho, dt);"),
    ("sgmm_x_row", "double p = ld(x, t * d_in + j, dt) * ld(A,", "double p = ld(x, 0 * d_in + j, dt) * ld(A,"),
    ("sgmm_v_slot", "acc += v[k * r + rho] * b;", "acc += v[rho] * b;"),
    ("gemv_x_reversed", "* ld(x, j, dt);", "* ld(x, d_in - 1 - j, dt);"),
    ("gemv_W_transposed", "double p = ld(W, i * d_in + j, dt)", "double p = ld(W, j * d_out + i, dt)"),
    ("gemv_drop_last", "for (int64_t j = 0; j < d_in; ++j) {\n            double p = ld(W,",
     "for (int64_t j = 0; j + 1 < d_in; ++j) {\n            double p = ld(W,"),
    ("gemv_truncate", "y[i] = (float)acc;  /* C conversion: RNE */", "y[i] = (float)trunc(acc * 1048576.0) / 1048576.0f;"),
    ("centroid_tie_to_higher", "if (de[e] < de[eb]) eb = e;", "if (de[e] <= de[eb]) eb = e;"),
    ("centroid_max_over_centroids", "if (s < best) best = s;", "if (s > best || best == INFINITY) best = s;"),
    ("centroid_wrong_centroid", "ld(C, ((int64_t)e * J + j) * d + k, dt)", "ld(C, ((int64_t)j * E + e) * d + k, dt)"),
    ("centroid_abs_not_square", "s += diff * diff;", "s += fabs(diff);"),
    ("centroid_drop_last_dim", "for (int64_t k = 0; k < d; ++k) {\n                    double diff",
     "for (int64_t k = 0; k + 1 < d; ++k) {\n                    double diff"),
    # the tolerance scale S (absum) and the router's decision bound: every parity
    # floor is (gamma_n + extra) * S, so an inflated or deflated S must be caught
    ("switch_absum_x16", "if (absum) absum[q * d_in + j] = S;", "if (absum) absum[q * d_in + j] = 16.0 * S;"),
    ("switch_absum_no_W", "double S = fabs(w);", "double S = 0.0;"),
    ("switch_absum_signed", "acc_abs += fabs(b * a);", "acc_abs += b * a;"),
    ("switch_absum_no_gate", "*S += fabs(s * (double)g[k]) * acc_abs;", "*S += fabs(s) * acc_abs;"),
    ("sgmm_absum_x16", "if (absum) absum[t * d_out + o] = S;", "if (absum) absum[t * d_out + o] = 16.0 * S;"),
    ("sgmm_absum_no_y", "double S = fabs(yo);", "double S = 0.0;"),
    ("sgmm_absum_signed_x", "acc += p;\n                    acc_abs += fabs(p);",
     "acc += p;\n                    acc_abs += p;"),
    ("sgmm_absum_signed_B", "acc_abs += va[k * r + rho] * fabs(b);", "acc_abs += va[k * r + rho] * b;"),
    ("sgmm_absum_one_slot", "S += fabs(c) * acc_abs;", "S += (k == 0) * fabs(c) * acc_abs;"),
    ("router_bound_half", "bound[t] = gam * mx;", "bound[t] = 0.5 * gam * mx;"),
    ("router_bound_x1000", "bound[t] = gam * mx;", "bound[t] = 1000.0 * gam * mx;"),
    # an empty slot (-1) read as expert 0 everywhere it is tested
    ("empty_slot_as_expert0", "if (e < 0) continue;", "if (e < 0) e = 0;", 3),
]


MUTANTS = [m if len(m) == 4 else m + (1,) for m in MUTANTS]


@pytest.mark.parametrize("name,orig,bad,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, orig, bad, count, tmp_path):
    with open(SRC) as f:
        src = f.read()
    assert src.count(orig) == count, f"mutation site for {name} not found {count} time(s)"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(orig, bad))
    so = oracle.build(str(path), str(tmp_path / f"lib{name}.so"))
    lib = oracle.load(so)
    caught = oracle_pins.failing_pins(lib)
    assert caught, f"planted mistake {name} passed every pin"
