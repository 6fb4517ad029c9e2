/*
 * CPU oracle for P-cast attention, fp64, one row at a time.
 *
 * TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline
 * leg of the benchmark call this.  It shares no code with the HIP path.
 *
 * Each requested row (b, h, i) gets
 *   O1  exact attention, softmax(q K^T / sqrt(d) + bias) V over the keys the
 *       row may see (all keys, or j <= i when causal) -- FlashAttention blog,
 *       "Perché l'attenzione è legata alla memoria";
 *   O2  the P-cast block pipeline: online softmax over key blocks of bc in
 *       forward (0 -> last) or reverse (last -> 0) order, P taken relative to
 *       the running max including the current block, the row sum built from
 *       the un-cast P, P multiplied by S and rounded to E4M3 before P.V, and
 *       the accumulator divided by S*l at the end -- P-cast summary sections
 *       1-2 and the blog's online-softmax and FA2 sections;
 *   counters over non-sink keys (bias_j == 0, or all keys without a bias):
 *       total pairs, pairs whose code is 0, pairs whose code would change
 *       between 0 and non-zero under a relative perturbation of eps of S*p,
 *       and pairs whose code is 0 outside the first key block (j >= bc);
 *   slack, a bound on how far O2 may move (max over the d columns) if every
 *       code whose rounding is decided within a relative eps of S*p took the
 *       other side: sum_j (q(y(1+eps)) - q(y(1-eps))) * exp(M_j - m) *
 *       max_c |vhat_jc| / (S l), where M_j is the running max applied to key j.
 *
 * Modes: 0 kernel (vhat = E4M3(V)), 1 pages (vhat = V), 2 bf16 (c = bf16(p),
 * vhat = V, S := 1), 3 nocast (c = S p, vhat = V).
 *
 * E4M3 here is OCP e4m3fn: step 2^(E-3) in binade [2^E, 2^(E+1)) for
 * E >= -6, step 2^-9 below 2^-6, largest value 448; rounding is to nearest
 * with ties to even and magnitudes above 448 saturate to 448.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { MODE_KERNEL = 0, MODE_PAGES = 1, MODE_BF16 = 2, MODE_NOCAST = 3 };

double oracle_e4m3_rne(double x) {
    if (isnan(x)) return x;
    double a = fabs(x);
    double q;
    if (a >= 448.0) {
        q = 448.0;
    } else {
        int e;
        frexp(a, &e);                         /* a = f 2^e, f in [0.5, 1) */
        double step = (a < 0x1p-6) ? 0x1p-9 : ldexp(1.0, (e - 1) - 3);
        q = rint(a / step) * step;            /* exact quotient, RNE */
        if (q > 448.0) q = 448.0;
    }
    return copysign(q, x);
}

double oracle_bf16_rne(double x) {
    if (isnan(x) || isinf(x)) return x;
    double a = fabs(x);
    int e;
    frexp(a, &e);
    int se = e - 8;
    if (se < -133) se = -133;
    double step = ldexp(1.0, se);
    return copysign(rint(a / step) * step, x);
}

static inline double bf16_bits_to_double(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

static inline double cast_code(double y, int mode) {
    switch (mode) {
    case MODE_KERNEL:
    case MODE_PAGES: return oracle_e4m3_rne(y);
    case MODE_BF16: return oracle_bf16_rne(y);
    default: return y;
    }
}

/*
 * rows: flat row ids ((b*Hq + h)*N + i), or NULL for every row in order.
 * Outputs (any may be NULL): o2, o1 [nrows*d]; slack [nrows];
 * cnt [nrows*4] = {total, zero, zero_ambiguous, zero_beyond_block0}.
 * Returns 0, or -1 on a bad argument / allocation failure.
 */
int oracle_rows(const uint16_t* Q, const uint16_t* K, const uint16_t* V, const float* bias,
                int B, int Hq, int Hkv, int N, int d, int causal, double S, int order, int mode,
                int bc, const int64_t* rows, int64_t nrows, double eps,
                double* o2, double* o1, double* slack, int64_t* cnt, int nthreads) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || N <= 0 || d <= 0 || bc <= 0) return -1;
    if (mode < 0 || mode > 3 || !(S > 0.0)) return -1;
    const int64_t total_rows = (int64_t)B * Hq * N;
    if (!rows) nrows = total_rows;
    const double Seff = (mode == MODE_BF16) ? 1.0 : S;
    const int group = Hq / Hkv;
    const double inv_sqrt_d = 1.0 / sqrt((double)d);
    const int64_t kv_elems = (int64_t)B * Hkv * N * d;

    /* Exact key values and the value operand the mode multiplies by. */
    float* kf = (float*)malloc(sizeof(float) * kv_elems);
    double* vh = (double*)malloc(sizeof(double) * kv_elems);
    double* vx = (double*)malloc(sizeof(double) * kv_elems);
    double* vmax = (double*)malloc(sizeof(double) * (int64_t)B * Hkv * N);
    if (!kf || !vh || !vx || !vmax) { free(kf); free(vh); free(vx); free(vmax); return -1; }
    int err = 0;
    #pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1) if (nthreads != 1)
    for (int64_t r = 0; r < (int64_t)B * Hkv * N; ++r) {
        double mx = 0.0;
        for (int c = 0; c < d; ++c) {
            int64_t x = r * d + c;
            kf[x] = (float)bf16_bits_to_double(K[x]);
            double v = bf16_bits_to_double(V[x]);
            vx[x] = v;
            vh[x] = (mode == MODE_KERNEL) ? oracle_e4m3_rne(v) : v;
            if (fabs(vh[x]) > mx) mx = fabs(vh[x]);
        }
        vmax[r] = mx;
    }

    #pragma omp parallel num_threads(nthreads > 0 ? nthreads : 1) if (nthreads != 1)
    {
        double* s = (double*)malloc(sizeof(double) * N);
        double* mt = (double*)malloc(sizeof(double) * N);
        double* dc = (double*)malloc(sizeof(double) * N);
        double* qd = (double*)malloc(sizeof(double) * d);
        double* A = (double*)malloc(sizeof(double) * d);
        double* E = (double*)malloc(sizeof(double) * d);
        if (!s || !mt || !dc || !qd || !A || !E) {
            #pragma omp atomic write
            err = 1;
        } else {
            #pragma omp for schedule(dynamic, 1)
            for (int64_t rr = 0; rr < nrows; ++rr) {
                const int64_t row = rows ? rows[rr] : rr;
                if (row < 0 || row >= total_rows) {
                    #pragma omp atomic write
                    err = 1;
                    continue;
                }
                const int i = (int)(row % N);
                const int64_t bh = row / N;
                const int h = (int)(bh % Hq), b = (int)(bh / Hq);
                const int g = h / group;
                const int64_t kvbase = ((int64_t)b * Hkv + g) * N;
                const int jmax = causal ? i : N - 1;
                for (int c = 0; c < d; ++c) qd[c] = bf16_bits_to_double(Q[row * d + c]);

                /* logits */
                for (int j = 0; j <= jmax; ++j) {
                    const float* kr = kf + (kvbase + j) * d;
                    double acc = 0.0;
                    for (int c = 0; c < d; ++c) acc += qd[c] * (double)kr[c];
                    s[j] = acc * inv_sqrt_d + (bias ? (double)bias[j] : 0.0);
                }

                /* O1: two-pass softmax */
                double m = -INFINITY;
                for (int j = 0; j <= jmax; ++j) if (s[j] > m) m = s[j];
                if (o1) {
                    double den = 0.0;
                    for (int c = 0; c < d; ++c) E[c] = 0.0;
                    for (int j = 0; j <= jmax; ++j) {
                        double w = exp(s[j] - m);
                        den += w;
                        const double* vr = vx + (kvbase + j) * d;
                        for (int c = 0; c < d; ++c) E[c] += w * vr[c];
                    }
                    for (int c = 0; c < d; ++c) o1[rr * d + c] = E[c] / den;
                }

                /* O2: the block pipeline */
                const int nblk = jmax / bc + 1;
                double run = -INFINITY, l = 0.0;
                int64_t tot = 0, zer = 0, amb = 0, zlate = 0;
                for (int c = 0; c < d; ++c) A[c] = 0.0;
                for (int it = 0; it < nblk; ++it) {
                    const int t = order ? nblk - 1 - it : it;
                    const int j0 = t * bc;
                    const int j1 = (j0 + bc - 1 < jmax) ? j0 + bc - 1 : jmax;
                    double mu = -INFINITY;
                    for (int j = j0; j <= j1; ++j) if (s[j] > mu) mu = s[j];
                    const double mp = run > mu ? run : mu;
                    const double alpha = (run == -INFINITY) ? 0.0 : exp(run - mp);
                    l *= alpha;
                    for (int c = 0; c < d; ++c) A[c] *= alpha;
                    for (int j = j0; j <= j1; ++j) {
                        const double p = exp(s[j] - mp);
                        l += p;
                        const double y = Seff * p;
                        const double code = cast_code(y, mode);
                        const double* vr = vh + (kvbase + j) * d;
                        if (code != 0.0)
                            for (int c = 0; c < d; ++c) A[c] += code * vr[c];
                        mt[j] = mp;
                        double lo = code, hi = code;
                        if (mode != MODE_NOCAST) {
                            lo = cast_code(y * (1.0 - eps), mode);
                            hi = cast_code(y * (1.0 + eps), mode);
                        }
                        dc[j] = hi - lo;
                        if (!bias || bias[j] == 0.0f) {
                            tot += 1;
                            zer += (code == 0.0);
                            zlate += (code == 0.0 && j >= bc);
                            amb += (lo == 0.0 && hi != 0.0);
                        }
                    }
                    run = mp;
                }
                const double denom = Seff * l;
                if (o2) for (int c = 0; c < d; ++c) o2[rr * d + c] = A[c] / denom;
                if (slack) {
                    double sl = 0.0;
                    for (int j = 0; j <= jmax; ++j)
                        if (dc[j] != 0.0) sl += dc[j] * exp(mt[j] - run) * vmax[kvbase + j];
                    slack[rr] = sl / denom;
                }
                if (cnt) {
                    cnt[rr * 4 + 0] = tot; cnt[rr * 4 + 1] = zer;
                    cnt[rr * 4 + 2] = amb; cnt[rr * 4 + 3] = zlate;
                }
            }
        }
        free(s); free(mt); free(dc); free(qd); free(A); free(E);
    }
    free(kf); free(vh); free(vx); free(vmax);
    return err ? -1 : 0;
}

/* Vector forms of the two roundings, for cross-checks against the NumPy twin. */
void oracle_e4m3_rne_n(const double* x, double* y, int64_t n) {
    for (int64_t k = 0; k < n; ++k) y[k] = oracle_e4m3_rne(x[k]);
}

void oracle_bf16_rne_n(const double* x, double* y, int64_t n) {
    for (int64_t k = 0; k < n; ++k) y[k] = oracle_bf16_rne(x[k]);
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
