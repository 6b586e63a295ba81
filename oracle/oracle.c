/*
 * Plain fp64 CPU oracle for exact attention, forward and backward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it.  It shares no code, header or constant with the HIP
 * path.
 *
 * What it computes is the plain definition of attention, not the tiled
 * algorithm that reaches it faster.  Every FlashAttention generation computes
 * the same attention (FlashAttention-4 explainer, section "02", the table of
 * four generations and the comment under it), and the lazy rescale with one
 * final correction is exact ("巧招二"), so the oracle is the definition:
 *
 *   s_ij   = scale * sum_d Q[i,d] K[j,d]              (score, all keys j)
 *   s_ij   = -inf                 if causal and j > i  (diagonal mask)
 *   m_i    = max_j s_ij
 *   P_ij   = exp(s_ij - m_i) / sum_k exp(s_ik - m_i)   (row softmax)
 *   O[i,:] = sum_j P_ij V[j,:]
 *   LSE_i  = m_i + log(sum_j exp(s_ij - m_i))          (natural log)
 *
 * softmax(QK^T)V with tiling over rows/keys: "FlashAttention-4 算法解析",
 * section 4 (tiling and the online-softmax pseudocode).  The scale inside the
 * softmax, the natural-log LSE over the scaled scores and the causal rule
 * j <= i are readings the pages leave open; they are listed with the design
 * notes.
 *
 * Backward, given dO (the five products of the backward pass: hotelren
 * FlashAttention-4 summary, section 4.1/4.2 "五阶段流水线"; P is recomputed from
 * Q, K, never stored: hotdry article, section on kernel fusion):
 *
 *   dV[j,:] = sum_i P_ij dO[i,:]
 *   dP_ij   = dO[i,:] . V[j,:]
 *   Delta_i = sum_j P_ij dP_ij
 *   dS_ij   = P_ij (dP_ij - Delta_i)                    ("dsoftmax")
 *   dQ[i,:] = scale * sum_j dS_ij K[j,:]
 *   dK[j,:] = scale * sum_i dS_ij Q[i,:]
 *
 * With grouped heads (Hq = G * Hkv), query head hq reads K/V head hq / G and
 * dK, dV of a K/V head sum over its G query heads.
 *
 * Inputs are bf16 bit patterns (uint16), widened exactly to fp64.  Layout is
 * [B][H][N][D], D contiguous.  Query length Nq and key length Nk may differ
 * (used to evaluate single rows); causal uses j <= i with both indices from 0.
 * Outputs are fp64.  All arithmetic is fp64 with libm exp/log.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_to_f64(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Widen one [rows][D] bf16 slab to fp64. */
static void widen(const uint16_t* src, double* dst, long n) {
    for (long t = 0; t < n; ++t) dst[t] = bf16_to_f64(src[t]);
}

/* Element source of the forward: bf16 bit patterns or fp64 values. */
typedef struct {
    const void* p;
    int is_f64;
} src_t;

static void load(src_t src, long off, double* dst, long n) {
    if (src.is_f64) {
        const double* d = (const double*)src.p + off;
        for (long t = 0; t < n; ++t) dst[t] = d[t];
    } else {
        widen((const uint16_t*)src.p + off, dst, n);
    }
}

static double dot(const double* a, const double* b, int D) {
    double s = 0.0;
    for (int d = 0; d < D; ++d) s += a[d] * b[d];
    return s;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following calls (timing only; the results do not depend on it). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

static int check_shape(int B, int Hq, int Hkv, int Nq, int Nk, int D) {
    if (B < 0 || Hq < 1 || Hkv < 1 || Nq < 0 || Nk < 0 || D < 1) return -1;
    if (Hq % Hkv != 0) return -1;
    return 0;
}

/* Number of keys row i may attend to. */
static int row_keys(int i, int Nk, int causal) {
    if (!causal) return Nk;
    return (i + 1 < Nk) ? i + 1 : Nk;
}

/*
 * Row statistics of one query row: fills s[0..nk) with the scaled scores and
 * returns m (row max) and l = sum_j exp(s_j - m).  nk == 0 gives m = -inf,
 * l = 0 (a row with every key masked).
 */
static void row_scores(const double* qi, const double* K, int nk, int D, double scale,
                       double* s, double* m_out, double* l_out) {
    double m = -INFINITY;
    for (int j = 0; j < nk; ++j) {
        s[j] = scale * dot(qi, K + (long)j * D, D);
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int j = 0; j < nk; ++j) l += exp(s[j] - m);
    *m_out = m;
    *l_out = l;
}

/*
 * Forward: o [B][Hq][Nq][D], lse [B][Hq][Nq].
 * A row with no unmasked key gets O = 0 and LSE = -inf.
 */
static int fwd_impl(src_t q, src_t k, src_t v, double* o, double* lse,
                    int B, int Hq, int Hkv, int Nq, int Nk, int D, int causal, double scale) {
    if (check_shape(B, Hq, Hkv, Nq, Nk, D)) return -1;
    const int G = Hq / Hkv;
    for (int b = 0; b < B; ++b) {
        for (int hq = 0; hq < Hq; ++hq) {
            const int hk = hq / G;
            double* K = (double*)malloc(sizeof(double) * ((size_t)Nk * D + 1));
            double* V = (double*)malloc(sizeof(double) * ((size_t)Nk * D + 1));
            if (!K || !V) { free(K); free(V); return -2; }
            load(k, ((long)b * Hkv + hk) * Nk * D, K, (long)Nk * D);
            load(v, ((long)b * Hkv + hk) * Nk * D, V, (long)Nk * D);
            const long qoff = ((long)b * Hq + hq) * Nq * D;
            double* Oh = o + ((long)b * Hq + hq) * Nq * D;
            double* Lh = lse + ((long)b * Hq + hq) * Nq;
            int fail = 0;
#pragma omp parallel
            {
                double* s = (double*)malloc(sizeof(double) * ((size_t)Nk + 1));
                double* qi = (double*)malloc(sizeof(double) * (size_t)D);
                if (!s || !qi) {
#pragma omp atomic write
                    fail = 1;
                } else {
#pragma omp for schedule(dynamic, 16)
                    for (int i = 0; i < Nq; ++i) {
                        load(q, qoff + (long)i * D, qi, D);
                        const int nk = row_keys(i, Nk, causal);
                        double m, l;
                        row_scores(qi, K, nk, D, scale, s, &m, &l);
                        double* oi = Oh + (long)i * D;
                        for (int d = 0; d < D; ++d) oi[d] = 0.0;
                        if (nk == 0) { Lh[i] = -INFINITY; continue; }
                        for (int j = 0; j < nk; ++j) {
                            const double p = exp(s[j] - m) / l;
                            const double* vj = V + (long)j * D;
                            for (int d = 0; d < D; ++d) oi[d] += p * vj[d];
                        }
                        Lh[i] = m + log(l);
                    }
                }
                free(s);
                free(qi);
            }
            free(K);
            free(V);
            if (fail) return -2;
        }
    }
    return 0;
}

int oracle_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, double* o, double* lse,
               int B, int Hq, int Hkv, int Nq, int Nk, int D, int causal, double scale) {
    const src_t sq = {q, 0}, sk = {k, 0}, sv = {v, 0};
    return fwd_impl(sq, sk, sv, o, lse, B, Hq, Hkv, Nq, Nk, D, causal, scale);
}

/* The same definition on fp64 inputs (used on dequantized values). */
int oracle_fwd_f64(const double* q, const double* k, const double* v, double* o, double* lse,
                   int B, int Hq, int Hkv, int Nq, int Nk, int D, int causal, double scale) {
    const src_t sq = {q, 1}, sk = {k, 1}, sv = {v, 1};
    return fwd_impl(sq, sk, sv, o, lse, B, Hq, Hkv, Nq, Nk, D, causal, scale);
}

/*
 * Backward: dq [B][Hq][Nq][D], dk/dv [B][Hkv][Nk][D], all fp64.
 * P is recomputed here from q and k; the GPU's O and LSE are never used.
 * Pass 1 (over query rows): row stats m_i, l_i, Delta_i and dQ[i].
 * Pass 2 (over key rows):  dK[j], dV[j] summed over every query row of every
 *                          query head of the group.
 */
int oracle_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
               double* dq, double* dk, double* dv,
               int B, int Hq, int Hkv, int Nq, int Nk, int D, int causal, double scale) {
    if (check_shape(B, Hq, Hkv, Nq, Nk, D)) return -1;
    const int G = Hq / Hkv;
    for (int b = 0; b < B; ++b) {
        for (int hk = 0; hk < Hkv; ++hk) {
            const size_t nkd = (size_t)Nk * D + 1, nqd = (size_t)Nq * D + 1;
            double* K = (double*)malloc(sizeof(double) * nkd);
            double* V = (double*)malloc(sizeof(double) * nkd);
            double* Qg = (double*)malloc(sizeof(double) * nqd * G);
            double* dOg = (double*)malloc(sizeof(double) * nqd * G);
            double* M = (double*)malloc(sizeof(double) * ((size_t)Nq * G + 1));
            double* L = (double*)malloc(sizeof(double) * ((size_t)Nq * G + 1));
            double* Dl = (double*)malloc(sizeof(double) * ((size_t)Nq * G + 1));
            if (!K || !V || !Qg || !dOg || !M || !L || !Dl) {
                free(K); free(V); free(Qg); free(dOg); free(M); free(L); free(Dl);
                return -2;
            }
            widen(k + ((long)b * Hkv + hk) * Nk * D, K, (long)Nk * D);
            widen(v + ((long)b * Hkv + hk) * Nk * D, V, (long)Nk * D);
            for (int g = 0; g < G; ++g) {
                const int hq = hk * G + g;
                widen(q + ((long)b * Hq + hq) * Nq * D, Qg + (size_t)g * nqd, (long)Nq * D);
                widen(dout + ((long)b * Hq + hq) * Nq * D, dOg + (size_t)g * nqd, (long)Nq * D);
            }
            int fail = 0;
            /* Pass 1: per query row. */
#pragma omp parallel
            {
                double* s = (double*)malloc(sizeof(double) * ((size_t)Nk + 1));
                double* dp = (double*)malloc(sizeof(double) * ((size_t)Nk + 1));
                if (!s || !dp) {
#pragma omp atomic write
                    fail = 1;
                } else {
#pragma omp for schedule(dynamic, 16) collapse(2)
                    for (int g = 0; g < G; ++g) {
                        for (int i = 0; i < Nq; ++i) {
                            const int hq = hk * G + g;
                            const double* qi = Qg + (size_t)g * nqd + (size_t)i * D;
                            const double* doi = dOg + (size_t)g * nqd + (size_t)i * D;
                            double* dqi = dq + (((long)b * Hq + hq) * Nq + i) * (long)D;
                            const int nk = row_keys(i, Nk, causal);
                            double m, l;
                            row_scores(qi, K, nk, D, scale, s, &m, &l);
                            double delta = 0.0;
                            for (int j = 0; j < nk; ++j) {
                                s[j] = exp(s[j] - m) / l; /* now P_ij */
                                dp[j] = dot(doi, V + (long)j * D, D);
                                delta += s[j] * dp[j];
                            }
                            for (int d = 0; d < D; ++d) dqi[d] = 0.0;
                            for (int j = 0; j < nk; ++j) {
                                const double ds = s[j] * (dp[j] - delta);
                                const double* kj = K + (long)j * D;
                                for (int d = 0; d < D; ++d) dqi[d] += scale * ds * kj[d];
                            }
                            M[(size_t)g * Nq + i] = m;
                            L[(size_t)g * Nq + i] = l;
                            Dl[(size_t)g * Nq + i] = delta;
                        }
                    }
                }
                free(s);
                free(dp);
            }
            if (!fail) {
                /* Pass 2: per key row. */
#pragma omp parallel for schedule(dynamic, 16)
                for (int j = 0; j < Nk; ++j) {
                    const double* kj = K + (long)j * D;
                    const double* vj = V + (long)j * D;
                    double* dkj = dk + (((long)b * Hkv + hk) * Nk + j) * (long)D;
                    double* dvj = dv + (((long)b * Hkv + hk) * Nk + j) * (long)D;
                    for (int d = 0; d < D; ++d) { dkj[d] = 0.0; dvj[d] = 0.0; }
                    for (int g = 0; g < G; ++g) {
                        for (int i = 0; i < Nq; ++i) {
                            if (causal && j > i) continue;
                            const double* qi = Qg + (size_t)g * nqd + (size_t)i * D;
                            const double* doi = dOg + (size_t)g * nqd + (size_t)i * D;
                            const double m = M[(size_t)g * Nq + i], l = L[(size_t)g * Nq + i];
                            const double p = exp(scale * dot(qi, kj, D) - m) / l;
                            const double dpij = dot(doi, vj, D);
                            const double ds = p * (dpij - Dl[(size_t)g * Nq + i]);
                            for (int d = 0; d < D; ++d) {
                                dvj[d] += p * doi[d];
                                dkj[d] += scale * ds * qi[d];
                            }
                        }
                    }
                }
            }
            free(K); free(V); free(Qg); free(dOg); free(M); free(L); free(Dl);
            if (fail) return -2;
        }
    }
    return 0;
}
