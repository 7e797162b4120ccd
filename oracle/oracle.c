/*
 * oracle.c -- plain, slow, binary64 CPU oracle for token-level pre-gated
 * dynamic LoRA (AdaFuse: "Accelerating Dynamic Adapter Inference via
 * Token-Level Pre-Gating and Fused Kernel Optimization").
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; neither includes the other.
 *
 * Every function reads its inputs as exact values (fp32 or bf16 -> binary64,
 * exact), evaluates the plain definition in binary64, and rounds each output
 * once to the output type with round-to-nearest-even.  OpenMP runs rows in
 * parallel for the timed baseline; each output element is computed by the
 * same sequential expression whatever the thread count.
 *
 * Sources (the pages; no line numbers):
 *   - router: AdaFuse digest (gist.science), section 2-가 "token-level
 *     pre-gating": a lightweight top-2 router at the first layer picks the
 *     token's expert set, and the decision is propagated to every layer;
 *     English abstract: one global routing decision per token for all adapter
 *     layers ("decide once, apply everywhere").
 *   - switch: same digest, section 2-나 "fused adapter switching": in one pass,
 *     remove the previous token's adapters and merge the current token's into
 *     the backbone of every layer, on concatenated adapter matrices, in place.
 *     English abstract: merging the selected LoRA adapters into the backbone.
 *   - nearest-centroid pre-gate: the ARIADNE page (training-free routing by
 *     proximity of the input embedding to each adapter's centroids).
 *   - sgmm: the batched unmerged form y += sum_k g_k (x A_k^T) B_k^T of the
 *     same adapters (the pages only name the SGMM kernel; the formula is the
 *     standard LoRA product with per-row gates).
 *
 * Readings where the pages are silent (all repeated in the design notes):
 *   router logits are x.Wr with no bias/noise/temperature; the two weights are
 *   the softmax over all E renormalised over the kept two; slot 0 holds the
 *   larger logit, ties go to the lower expert index; W is [d_out][d_in],
 *   A_e is [r][d_in], B_e is [d_out][r], delta_e = B_e A_e; the LoRA scale s
 *   multiplies every delta; an expert index of -1 marks an empty slot.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define DT_F32 0
#define DT_BF16 1

/* ---- exact loads --------------------------------------------------------- */

static double ld(const void* p, int64_t i, int dt) {
    if (dt == DT_F32) return (double)((const float*)p)[i];
    uint32_t b = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &b, 4);
    return (double)f;
}

/* ---- one rounding from binary64 to the storage type ---------------------- */

/* bf16: 8 significant bits, fp32's exponent range (min normal 2^-126, smallest
 * subnormal 2^-133, max finite (2 - 2^-7) * 2^127). */
static uint16_t bf16_rne_from_double(double v) {
    if (isnan(v)) return 0x7FC0;
    if (v == 0.0) return signbit(v) ? 0x8000 : 0x0000;
    int e;
    (void)frexp(v, &e);                 /* |v| in [2^(e-1), 2^e) */
    int qexp = e - 8;                   /* quantum of the binade */
    if (qexp < -133) qexp = -133;       /* subnormal quantum */
    double n = ldexp(v, -qexp);         /* exact: scaling by a power of two */
    double nr = nearbyint(n);           /* default mode: nearest, ties to even */
    double rv = ldexp(nr, qexp);
    if (fabs(rv) > 0x1.FEp127) rv = copysign(INFINITY, v);
    float f = (float)rv;                /* exact: rv has <= 8 significant bits */
    uint32_t b;
    memcpy(&b, &f, 4);
    return (uint16_t)(b >> 16);
}

static void st(void* p, int64_t i, int dt, double v) {
    if (dt == DT_F32) ((float*)p)[i] = (float)v;  /* C conversion: RNE */
    else ((uint16_t*)p)[i] = bf16_rne_from_double(v);
}

/* Exposed for the rounding pins in the tests. */
void dlmref_round(const double* v, int64_t n, int32_t dt, void* out) {
    for (int64_t i = 0; i < n; ++i) st(out, i, dt, v[i]);
}

/* ---- router -------------------------------------------------------------- */

/*
 * x [T][d], Wr [d][E] (dtype dt).  Outputs idx [T][2] int32, g [T][2] fp32.
 * Optional: logits [T][E] (binary64), margin [T], bound [T].
 *   margin = min(l[i0]-l[i1], l[i1]-l[3rd]) (l[i0]-l[i1] when E == 2), the
 *            distance of the decision from a tie;
 *   bound  = gamma_d * max_e sum_j |x_j Wr_je| with u = 2^-53: a forward bound
 *            on the error of any binary64 evaluation order of one logit.
 */
int dlmref_pregate(const void* x, const void* Wr, int64_t T, int64_t d, int32_t E, int32_t dt,
                   int32_t* idx, float* g, double* logits, double* margin, double* bound) {
    if (T < 0 || d < 1 || E < 2 || !x || !Wr || !idx || !g) return -1;
    const double u = ldexp(1.0, -53);
    const double gam = (double)d * u / (1.0 - (double)d * u);
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double* l = (double*)malloc(sizeof(double) * (size_t)E);
        double* a = (double*)malloc(sizeof(double) * (size_t)E);
        for (int32_t e = 0; e < E; ++e) {
            double s = 0.0, sa = 0.0;
            for (int64_t j = 0; j < d; ++j) {
                double p = ld(x, t * d + j, dt) * ld(Wr, j * (int64_t)E + e, dt);
                s += p;
                sa += fabs(p);
            }
            l[e] = s;
            a[e] = sa;
        }
        /* top-2 on the logits, strict '>' keeps the lower index on ties */
        int32_t i0 = 0;
        for (int32_t e = 1; e < E; ++e) if (l[e] > l[i0]) i0 = e;
        int32_t i1 = (i0 == 0) ? 1 : 0;
        for (int32_t e = 0; e < E; ++e) if (e != i0 && l[e] > l[i1]) i1 = e;
        /* softmax over all E (shifted by the max for range), keep the top two,
         * renormalise them to sum to one */
        double den = 0.0;
        for (int32_t e = 0; e < E; ++e) den += exp(l[e] - l[i0]);
        double p0 = exp(l[i0] - l[i0]) / den;
        double p1 = exp(l[i1] - l[i0]) / den;
        idx[2 * t] = i0;
        idx[2 * t + 1] = i1;
        g[2 * t] = (float)(p0 / (p0 + p1));
        g[2 * t + 1] = (float)(p1 / (p0 + p1));
        if (logits) for (int32_t e = 0; e < E; ++e) logits[t * E + e] = l[e];
        if (margin) {
            double m = l[i0] - l[i1];
            if (E > 2) {
                int32_t i2 = -1;
                for (int32_t e = 0; e < E; ++e)
                    if (e != i0 && e != i1 && (i2 < 0 || l[e] > l[i2])) i2 = e;
                double m2 = l[i1] - l[i2];
                if (m2 < m) m = m2;
            }
            margin[t] = m;
        }
        if (bound) {
            double mx = 0.0;
            for (int32_t e = 0; e < E; ++e) if (a[e] > mx) mx = a[e];
            bound[t] = gam * mx;
        }
        free(l);
        free(a);
    }
    return 0;
}

/* ---- nearest-centroid pre-gate ------------------------------------------- */

/*
 * Training-free routing (ARIADNE page: each adapter is represented by a set of
 * centroids of its training data's embeddings; at inference the input's
 * embedding is compared with every adapter's centroids and the closest adapter
 * is chosen).  Here: x [T][d], centroids C [E][J][d] (dtype dt); the distance
 * of token t to adapter e is min over its J centroids of the squared Euclidean
 * distance; the nearest adapter (ties -> lower index) goes to slot 0 with
 * weight 1, slot 1 is empty (-1, 0), the set format of the top-2 router.
 * Optional: dist [T][E] (binary64 adapter distances) and margin [T] (second
 * smallest minus smallest adapter distance; +inf when E == 1).
 */
int dlmref_pregate_centroid(const void* x, const void* C, int64_t T, int64_t d, int32_t E, int32_t J,
                            int32_t dt, int32_t* idx, float* g, double* dist, double* margin) {
    if (T < 0 || d < 1 || E < 1 || J < 1 || !x || !C || !idx || !g) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        double* de = (double*)malloc(sizeof(double) * (size_t)E);
        for (int32_t e = 0; e < E; ++e) {
            double best = INFINITY;
            for (int32_t j = 0; j < J; ++j) {
                double s = 0.0;
                for (int64_t k = 0; k < d; ++k) {
                    double diff = ld(x, t * d + k, dt) - ld(C, ((int64_t)e * J + j) * d + k, dt);
                    s += diff * diff;
                }
                if (s < best) best = s;
            }
            de[e] = best;
        }
        int32_t eb = 0;
        for (int32_t e = 1; e < E; ++e) if (de[e] < de[eb]) eb = e;
        idx[2 * t] = eb;
        idx[2 * t + 1] = -1;
        g[2 * t] = 1.0f;
        g[2 * t + 1] = 0.0f;
        if (dist) for (int32_t e = 0; e < E; ++e) dist[t * E + e] = de[e];
        if (margin) {
            double m = INFINITY;
            for (int32_t e = 0; e < E; ++e) if (e != eb && de[e] - de[eb] < m) m = de[e] - de[eb];
            margin[t] = m;
        }
        free(de);
    }
    return 0;
}

/* ---- expert sets --------------------------------------------------------- */

/* A set is two (expert, weight) slots; a NULL idx pointer is the empty set and
 * an expert index of -1 is an empty slot. */
static int set_ok(const int32_t* idx, const float* g, int32_t E) {
    if (!idx) return 1;
    if (!g) return 0;
    for (int k = 0; k < 2; ++k) {
        if (idx[k] < -1 || idx[k] >= E) return 0;
        if (idx[k] >= 0 && !isfinite(g[k])) return 0;
    }
    return 1;
}

/* ---- fused switch -------------------------------------------------------- */

/* Gated delta of one set at element (i, j):
 *   s * sum_{k: idx_k >= 0} g_k * sum_rho B[e_k][i][rho] * A[e_k][rho][j]
 * with A [E][r][d_in], B [E][d_out][r].  Also accumulates |terms| into *S. */
static double set_delta(const int32_t* idx, const float* g, const void* A, const void* B,
                        int64_t d_out, int64_t d_in, int32_t r, double s, int dt,
                        int64_t i, int64_t j, double* S) {
    if (!idx) return 0.0;
    double D = 0.0;
    for (int k = 0; k < 2; ++k) {
        int32_t e = idx[k];
        if (e < 0) continue;
        double acc = 0.0, acc_abs = 0.0;
        for (int32_t rho = 0; rho < r; ++rho) {
            double b = ld(B, ((int64_t)e * d_out + i) * r + rho, dt);
            double a = ld(A, ((int64_t)e * r + rho) * d_in + j, dt);
            acc += b * a;
            acc_abs += fabs(b * a);
        }
        D += s * (double)g[k] * acc;
        *S += fabs(s * (double)g[k]) * acc_abs;
    }
    return D;
}

/*
 * Switch a subset of rows of one adapted weight W [d_out][d_in]:
 *   W[i][j] <- round( W[i][j] - delta_old(i,j) + delta_new(i,j) )
 * Wrows [n_rows][d_in] holds the pre-state of rows `rows` and is updated in
 * place.  Optional exact [n_rows][d_in] gets the unrounded binary64 value and
 * absum [n_rows][d_in] the sum of magnitudes of every term (the scale of the
 * rounding error of any fp evaluation of the same expression).
 */
int dlmref_switch_rows(void* Wrows, const int64_t* rows, int64_t n_rows,
                       const void* A, const void* B, int64_t d_out, int64_t d_in,
                       int32_t E, int32_t r, double s, int32_t dt,
                       const int32_t* old_idx, const float* old_g,
                       const int32_t* new_idx, const float* new_g,
                       double* exact, double* absum) {
    if (!Wrows || !rows || !A || !B || n_rows < 0 || d_out < 1 || d_in < 1 || E < 1 || r < 1)
        return -1;
    if (!set_ok(old_idx, old_g, E) || !set_ok(new_idx, new_g, E)) return -2;
    for (int64_t q = 0; q < n_rows; ++q)
        if (rows[q] < 0 || rows[q] >= d_out) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t q = 0; q < n_rows; ++q) {
        int64_t i = rows[q];
        for (int64_t j = 0; j < d_in; ++j) {
            double w = ld(Wrows, q * d_in + j, dt);
            double S = fabs(w);
            double Dold = set_delta(old_idx, old_g, A, B, d_out, d_in, r, s, dt, i, j, &S);
            double Dnew = set_delta(new_idx, new_g, A, B, d_out, d_in, r, s, dt, i, j, &S);
            double v = w - Dold + Dnew;
            if (exact) exact[q * d_in + j] = v;
            if (absum) absum[q * d_in + j] = S;
            st(Wrows, q * d_in + j, dt, v);
        }
    }
    return 0;
}

/* ---- SGMM (batched, unmerged) -------------------------------------------- */

/*
 * For each of n rows t (x [n][d_in], y [n][d_out] in place, idx/g [n][2]):
 *   v_k[rho] = sum_j x[t][j] * A[e_k][rho][j]                 (shrink)
 *   y[t][o] <- round( y[t][o] + sum_k s*g_k * sum_rho v_k[rho] * B[e_k][o][rho] )
 * Slots with e_k = -1 contribute nothing.  exact/absum as for the switch, with
 * absum = |y| + sum_k |s g_k| sum_rho (sum_j |x A|) |B|.
 */
int dlmref_sgmm_rows(const void* x, const int32_t* idx, const float* g,
                     const void* A, const void* B, void* y,
                     int64_t n, int64_t d_in, int64_t d_out, int32_t E, int32_t r,
                     double s, int32_t dt, double* exact, double* absum) {
    if (!x || !idx || !g || !A || !B || !y || n < 0 || d_in < 1 || d_out < 1 || E < 1 || r < 1)
        return -1;
    for (int64_t t = 0; t < n; ++t)
        if (!set_ok(idx + 2 * t, g + 2 * t, E)) return -2;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t t = 0; t < n; ++t) {
        double* v = (double*)calloc((size_t)(2 * r), sizeof(double));
        double* va = (double*)calloc((size_t)(2 * r), sizeof(double));
        for (int k = 0; k < 2; ++k) {
            int32_t e = idx[2 * t + k];
            if (e < 0) continue;
            for (int32_t rho = 0; rho < r; ++rho) {
                double acc = 0.0, acc_abs = 0.0;
                for (int64_t j = 0; j < d_in; ++j) {
                    double p = ld(x, t * d_in + j, dt) * ld(A, ((int64_t)e * r + rho) * d_in + j, dt);
                    acc += p;
                    acc_abs += fabs(p);
                }
                v[k * r + rho] = acc;
                va[k * r + rho] = acc_abs;
            }
        }
        for (int64_t o = 0; o < d_out; ++o) {
            double yo = ld(y, t * d_out + o, dt);
            double S = fabs(yo);
            double D = 0.0;
            for (int k = 0; k < 2; ++k) {
                int32_t e = idx[2 * t + k];
                if (e < 0) continue;
                double acc = 0.0, acc_abs = 0.0;
                for (int32_t rho = 0; rho < r; ++rho) {
                    double b = ld(B, ((int64_t)e * d_out + o) * r + rho, dt);
                    acc += v[k * r + rho] * b;
                    acc_abs += va[k * r + rho] * fabs(b);
                }
                double c = s * (double)g[2 * t + k];
                D += c * acc;
                S += fabs(c) * acc_abs;
            }
            double val = yo + D;
            if (exact) exact[t * d_out + o] = val;
            if (absum) absum[t * d_out + o] = S;
            st(y, t * d_out + o, dt, val);
        }
        free(v);
        free(va);
    }
    return 0;
}

/* ---- merged-weight matrix-vector product ---------------------------------- */

/*
 * The decode step that follows a switch: with the token's adapters merged into
 * the backbone, each adapted projection is the plain product of the merged
 * weight with the layer input (Chinese digest, "technical framework": the fused
 * kernel merges the selected adapter parameters into the backbone and carries
 * out the computation in a single kernel).
 *   y[i] = round_fp32( sum_j W[i][j] * x[j] ),  W [d_out][d_in], x [d_in] (dt)
 * Optional exact [d_out] gets the unrounded binary64 sum and absum [d_out] the
 * sum of |W[i][j] * x[j]|.
 */
int dlmref_gemv(const void* W, const void* x, int64_t d_out, int64_t d_in, int32_t dt,
                float* y, double* exact, double* absum) {
    if (!W || !x || !y || d_out < 1 || d_in < 1) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < d_out; ++i) {
        double acc = 0.0, acc_abs = 0.0;
        for (int64_t j = 0; j < d_in; ++j) {
            double p = ld(W, i * d_in + j, dt) * ld(x, j, dt);
            acc += p;
            acc_abs += fabs(p);
        }
        if (exact) exact[i] = acc;
        if (absum) absum[i] = acc_abs;
        y[i] = (float)acc;  /* C conversion: RNE */
    }
    return 0;
}

/* Threads OpenMP will use (1 when built without OpenMP). */
#ifdef _OPENMP
#include <omp.h>
int dlmref_threads(void) { return omp_get_max_threads(); }
void dlmref_set_threads(int n) { omp_set_num_threads(n); }
#else
int dlmref_threads(void) { return 1; }
void dlmref_set_threads(int n) { (void)n; }
#endif
