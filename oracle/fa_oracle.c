/*
 * fa_oracle.c -- plain fp64 CPU oracle for scaled dot-product attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference against which the
 * GPU kernels are checked.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it.  It shares no code, header,
 * table or constant with the GPU library, and the GPU library never calls it.
 *
 * What it computes is the plain definition of attention, not the tiled
 * method that reaches the same value faster:
 *
 *   s_ij = scale * sum_d q_id * k_jd                 (masked -> -inf)
 *   m_i  = max_j s_ij
 *   l_i  = sum_j exp(s_ij - m_i)
 *   P_ij = exp(s_ij - m_i) / l_i
 *   O_id = sum_j P_ij * v_jd
 *   lse_i = m_i + ln(l_i)
 *
 * Sources (titles of the pages, with the passage):
 *   - "FlashAttention-2 on Ascend NPU: how ops-transformer reaches 3x"
 *     (2048ai.net), section 1 "Background": Attention(Q,K,V) =
 *     softmax(QK^T / sqrt(d_k)) V, with the full N x N score matrix S and
 *     probability matrix P materialised.
 *   - "ops-transformer FlashAttention operator in practice" (ai6s.net),
 *     section 1: the three-step flow (scores, softmax, multiply by V), and
 *     section 4's naive PyTorch baseline (matmul, softmax over the last
 *     axis, matmul), with the causal flag described as an upper-triangular
 *     mask (future keys hidden).
 *   - "catlass FlashAttention tuning for a 13B service" (gsyq.cn), section
 *     "Causal Mask implementation": each position sees only earlier tokens.
 *     Reading used here: key j is visible to query i iff j <= i + (Sk - Sq)
 *     (bottom-right alignment; for Sq == Sk this is j <= i, the diagonal
 *     included).  The masked/dropout functions also take the diagonal's
 *     offset c explicitly (j visible iff j <= i + c): a block of a sequence
 *     split into chunks, queries from global position qs and keys from ks,
 *     sees key j iff ks + j <= qs + i, i.e. c = qs - ks ("FlashAttention-2
 *     on Ascend NPU" (2048ai.net), section 6.4, sequence parallelism: each
 *     device works on its own chunk of the sequence); c = Sk - Sq is the
 *     rule above.
 *   - The log-sum-exp output is not named by the pages; it is the row
 *     normaliser L that their block pseudo-code divides by (lanjinlin.com.cn,
 *     "math principle"), written in natural-log form: lse_i = m_i + ln l_i.
 *     A row with no visible key gets O = 0 and lse = -inf.
 *
 * Precision: inputs are IEEE binary16 or bfloat16 bit patterns, decoded
 * exactly to double by this file's own decoders.  The scale arrives as a
 * float and is widened exactly, so the oracle and the kernel use the same
 * constant.  Everything after decoding is fp64.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC fa_oracle.c -o libfa_oracle.so -lm
 * (see oracle/build.py).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORA_F16 = 0, ORA_BF16 = 1 };

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction
 * bits.  Subnormals are fraction * 2^-24; exponent 31 is inf / NaN. */
double ora_f16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double mag;
    if (expo == 0) {
        mag = ldexp((double)frac, -24);
    } else if (expo == 31) {
        mag = frac ? NAN : INFINITY;
    } else {
        mag = ldexp((double)(1024 + frac), expo - 25);
    }
    return sign ? -mag : mag;
}

/* bfloat16 is the upper half of an IEEE binary32: 1 sign, 8 exponent
 * (bias 127), 7 fraction bits. */
double ora_bf16_to_f64(uint16_t b) {
    int sign = (b >> 15) & 1;
    int expo = (b >> 7) & 0xff;
    int frac = b & 0x7f;
    double mag;
    if (expo == 0) {
        mag = ldexp((double)frac, -133);
    } else if (expo == 255) {
        mag = frac ? NAN : INFINITY;
    } else {
        mag = ldexp((double)(128 + frac), expo - 134);
    }
    return sign ? -mag : mag;
}

void ora_decode(const uint16_t* src, double* dst, int64_t n, int dtype) {
    for (int64_t i = 0; i < n; ++i)
        dst[i] = dtype == ORA_BF16 ? ora_bf16_to_f64(src[i]) : ora_f16_to_f64(src[i]);
}

/* Causal rule with the diagonal at offset c: key j visible to query i iff
 * j <= i + c (everything visible without the causal flag). */
static int visible(int64_t i, int64_t j, int64_t c, int causal) {
    if (!causal) return 1;
    return j <= i + c;
}

/* Probabilities of one query row against all keys of its head: materialise
 * the score row, then the two-pass softmax.  qrow: D values; K: Sk x D
 * row-major; srow: Sk outputs, P_ij (0 where key j is hidden, all 0 when no
 * key is visible).  Returns lse_i (-inf when no key is visible). */
static double row_probs(const double* qrow, const double* K, int64_t i, int64_t Sq, int64_t Sk,
                        int D, double scale, int causal, double* srow) {
    /* scores */
    for (int64_t j = 0; j < Sk; ++j) {
        if (!visible(i, j, Sk - Sq, causal)) { srow[j] = -INFINITY; continue; }
        const double* kr = K + j * D;
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += qrow[d] * kr[d];
        srow[j] = scale * acc;
    }
    /* pass 1: row maximum */
    double m = -INFINITY;
    for (int64_t j = 0; j < Sk; ++j) if (srow[j] > m) m = srow[j];
    if (m == -INFINITY) {
        for (int64_t j = 0; j < Sk; ++j) srow[j] = 0.0;
        return -INFINITY;
    }
    /* pass 2: exponentials and their sum, then normalisation */
    double l = 0.0;
    for (int64_t j = 0; j < Sk; ++j) {
        double p = exp(srow[j] - m);
        srow[j] = p;
        l += p;
    }
    for (int64_t j = 0; j < Sk; ++j) srow[j] = srow[j] / l;
    return m + log(l);
}

/* One query row of the forward: probabilities, then the weighted sum of V.
 * V: Sk x D row-major; srow: Sk scratch.  Writes D outputs and the lse. */
static void row_attention(const double* qrow, const double* K, const double* V, int64_t i,
                          int64_t Sq, int64_t Sk, int D, double scale, int causal,
                          double* srow, double* orow, double* lse_out) {
    *lse_out = row_probs(qrow, K, i, Sq, Sk, D, scale, causal, srow);
    for (int d = 0; d < D; ++d) orow[d] = 0.0;
    for (int64_t j = 0; j < Sk; ++j) {
        double p = srow[j];
        if (p == 0.0) continue;
        const double* vr = V + j * D;
        for (int d = 0; d < D; ++d) orow[d] += p * vr[d];
    }
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

static int thread_id(void) {
#ifdef _OPENMP
    return omp_get_thread_num();
#else
    return 0;
#endif
}

int ora_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Full forward over contiguous [B,H,Sq,D] queries and [B,H,Sk,D] keys and
 * values (16-bit patterns of `dtype`).  o: [B,H,Sq,D] fp64, lse: [B,H,Sq]
 * fp64 (may be NULL).  The score matrix of one head is materialised
 * (Sq x Sk doubles) before the softmax, as the definition reads.
 * Returns 0 on success, nonzero on bad arguments or allocation failure.
 */
int ora_attention_fwd(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      int B, int H, int Sq, int Sk, int D, float scale, int causal, int dtype,
                      double* o, double* lse, int nthreads) {
    if (!q || !k || !v || !o || B < 0 || H < 0 || Sq < 0 || Sk < 0 || D <= 0) return 1;
    if (dtype != ORA_F16 && dtype != ORA_BF16) return 2;
    set_threads(nthreads);
    const double sc = (double)scale;
    const int64_t qh = (int64_t)Sq * D, kh = (int64_t)Sk * D;
    double* Qd = (double*)malloc(sizeof(double) * (size_t)(qh > 0 ? qh : 1));
    double* Kd = (double*)malloc(sizeof(double) * (size_t)(kh > 0 ? kh : 1));
    double* Vd = (double*)malloc(sizeof(double) * (size_t)(kh > 0 ? kh : 1));
    double* Sm = (double*)malloc(sizeof(double) * (size_t)((int64_t)Sq * Sk > 0 ? (int64_t)Sq * Sk : 1));
    if (!Qd || !Kd || !Vd || !Sm) { free(Qd); free(Kd); free(Vd); free(Sm); return 3; }
    for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
        ora_decode(q + bh * qh, Qd, qh, dtype);
        ora_decode(k + bh * kh, Kd, kh, dtype);
        ora_decode(v + bh * kh, Vd, kh, dtype);
        double* ob = o + bh * qh;
        double* lb = lse ? lse + bh * Sq : NULL;
        #pragma omp parallel for schedule(dynamic, 4)
        for (int64_t i = 0; i < Sq; ++i) {
            double l_i;
            row_attention(Qd + i * D, Kd, Vd, i, Sq, Sk, D, sc, causal, Sm + i * Sk, ob + i * D, &l_i);
            if (lb) lb[i] = l_i;
        }
    }
    free(Qd); free(Kd); free(Vd); free(Sm);
    return 0;
}

/*
 * The same definition evaluated on selected rows only, for checks at sizes
 * where the full forward is too slow.  rows[r] is a flat row id
 * (b*H + h)*Sq + i.  o: nrows x D fp64, lse: nrows fp64.
 */
int ora_attention_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                       int B, int H, int Sq, int Sk, int D, float scale, int causal, int dtype,
                       const int64_t* rows, int64_t nrows, double* o, double* lse, int nthreads) {
    if (!q || !k || !v || !o || !lse || !rows || B < 0 || H < 0 || Sq < 0 || Sk < 0 || D <= 0) return 1;
    if (dtype != ORA_F16 && dtype != ORA_BF16) return 2;
    const int64_t total = (int64_t)B * H * Sq;
    for (int64_t r = 0; r < nrows; ++r) if (rows[r] < 0 || rows[r] >= total) return 4;
    set_threads(nthreads);
    const double sc = (double)scale;
    int err = 0;
    #pragma omp parallel
    {
        double* Qr = (double*)malloc(sizeof(double) * (size_t)D);
        double* Kd = (double*)malloc(sizeof(double) * (size_t)((int64_t)Sk * D > 0 ? (int64_t)Sk * D : 1));
        double* Vd = (double*)malloc(sizeof(double) * (size_t)((int64_t)Sk * D > 0 ? (int64_t)Sk * D : 1));
        double* Sr = (double*)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
        int64_t cur_bh = -1;
        if (!Qr || !Kd || !Vd || !Sr) {
            #pragma omp atomic write
            err = 3;
        } else {
            #pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < nrows; ++r) {
                int64_t bh = rows[r] / Sq, i = rows[r] % Sq;
                if (bh != cur_bh) {
                    ora_decode(k + bh * (int64_t)Sk * D, Kd, (int64_t)Sk * D, dtype);
                    ora_decode(v + bh * (int64_t)Sk * D, Vd, (int64_t)Sk * D, dtype);
                    cur_bh = bh;
                }
                ora_decode(q + rows[r] * D, Qr, D, dtype);
                row_attention(Qr, Kd, Vd, i, Sq, Sk, D, sc, causal, Sr, o + r * D, lse + r);
            }
        }
        free(Qr); free(Kd); free(Vd); free(Sr);
    }
    return err;
}

/*
 * Backward of the same definition: the gradients of L = sum_{i,d} O_id dO_id
 * with respect to q, k and v, evaluated as the chain rule reads, one head at
 * a time with the probability matrix materialised (nothing is tiled or
 * recomputed here):
 *
 *   P_ij  = the forward's probabilities (row_probs)
 *   dV_j  = sum_i P_ij dO_i
 *   dP_ij = dO_i . v_j
 *   dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)     (Jacobian of the row softmax)
 *   dQ_i  = scale sum_j dS_ij k_j
 *   dK_j  = scale sum_i dS_ij q_i
 *
 * The pages say only that the backward pass recomputes the scores instead of
 * storing them ("ops-transformer FlashAttention operator in practice",
 * ai6s.net, section 2, table of core optimisations; "FlashAttention-2 on
 * Ascend NPU" (2048ai.net), section 6.2 on checkpointing) and that it comes in
 * a deterministic and a faster atomic-accumulation mode ("catlass
 * FlashAttention tuning for a 13B service" (gsyq.cn), section on the
 * backward pass).  The formulas above are the derivative of the forward's
 * definition; both modes must reach them.
 *
 * q, k, v, dout: contiguous 16-bit patterns ([B,H,Sq,D] for q and dout,
 * [B,H,Sk,D] for k and v).  dq: [B,H,Sq,D] fp64, dk, dv: [B,H,Sk,D] fp64.
 */
static void head_backward(const double* Qd, const double* Kd, const double* Vd, const double* dOd,
                          int64_t Sq, int64_t Sk, int D, double sc, int causal,
                          double* P, double* dS, double* dq, double* dk, double* dv) {
    #pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < Sq; ++i) {
        double* prow = P + i * Sk;
        double* srow = dS + i * Sk;
        row_probs(Qd + i * D, Kd, i, Sq, Sk, D, sc, causal, prow);
        const double* gi = dOd + i * D;
        double rowdot = 0.0;
        for (int64_t j = 0; j < Sk; ++j) {
            const double* vr = Vd + j * D;
            double dp = 0.0;
            for (int d = 0; d < D; ++d) dp += gi[d] * vr[d];
            srow[j] = dp;
            rowdot += prow[j] * dp;
        }
        for (int64_t j = 0; j < Sk; ++j) srow[j] = prow[j] * (srow[j] - rowdot);
        double* gq = dq + i * D;
        for (int d = 0; d < D; ++d) gq[d] = 0.0;
        for (int64_t j = 0; j < Sk; ++j) {
            const double* kr = Kd + j * D;
            for (int d = 0; d < D; ++d) gq[d] += srow[j] * kr[d];
        }
        for (int d = 0; d < D; ++d) gq[d] *= sc;
    }
    #pragma omp parallel for schedule(dynamic, 4)
    for (int64_t j = 0; j < Sk; ++j) {
        double* gk = dk + j * D;
        double* gv = dv + j * D;
        for (int d = 0; d < D; ++d) { gk[d] = 0.0; gv[d] = 0.0; }
        for (int64_t i = 0; i < Sq; ++i) {
            const double pij = P[i * Sk + j], sij = dS[i * Sk + j];
            const double* qr = Qd + i * D;
            const double* gi = dOd + i * D;
            for (int d = 0; d < D; ++d) {
                gv[d] += pij * gi[d];
                gk[d] += sij * qr[d];
            }
        }
        for (int d = 0; d < D; ++d) gk[d] *= sc;
    }
}

int ora_attention_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* dout,
                      int B, int H, int Sq, int Sk, int D, float scale, int causal, int dtype,
                      double* dq, double* dk, double* dv, int nthreads) {
    if (!q || !k || !v || !dout || !dq || !dk || !dv || B < 0 || H < 0 || Sq < 0 || Sk < 0 || D <= 0)
        return 1;
    if (dtype != ORA_F16 && dtype != ORA_BF16) return 2;
    set_threads(nthreads);
    const double sc = (double)scale;
    const int64_t qh = (int64_t)Sq * D, kh = (int64_t)Sk * D, ph = (int64_t)Sq * Sk;
    double* Qd = (double*)malloc(sizeof(double) * (size_t)(qh > 0 ? qh : 1));
    double* dOd = (double*)malloc(sizeof(double) * (size_t)(qh > 0 ? qh : 1));
    double* Kd = (double*)malloc(sizeof(double) * (size_t)(kh > 0 ? kh : 1));
    double* Vd = (double*)malloc(sizeof(double) * (size_t)(kh > 0 ? kh : 1));
    double* P = (double*)malloc(sizeof(double) * (size_t)(ph > 0 ? ph : 1));
    double* dS = (double*)malloc(sizeof(double) * (size_t)(ph > 0 ? ph : 1));
    int rc = 0;
    if (!Qd || !dOd || !Kd || !Vd || !P || !dS) {
        rc = 3;
    } else {
        for (int64_t bh = 0; bh < (int64_t)B * H; ++bh) {
            ora_decode(q + bh * qh, Qd, qh, dtype);
            ora_decode(dout + bh * qh, dOd, qh, dtype);
            ora_decode(k + bh * kh, Kd, kh, dtype);
            ora_decode(v + bh * kh, Vd, kh, dtype);
            head_backward(Qd, Kd, Vd, dOd, Sq, Sk, D, sc, causal, P, dS,
                          dq + bh * qh, dk + bh * kh, dv + bh * kh);
        }
    }
    free(Qd); free(dOd); free(Kd); free(Vd); free(P); free(dS);
    return rc;
}

/*
 * The same gradients on selected rows only, for checks at sizes where the
 * full backward is too slow.  qrows[r] = (b*H + h)*Sq + i selects a dQ row;
 * krows[r] = (b*H + h)*Sk + j selects a dK and a dV row.  A selected key
 * needs every query row of its head (its column of P and dS), so each head
 * named in krows costs one pass over all its rows; the rows are visited in
 * parallel and each thread accumulates its own partial sums, added up in
 * thread order afterwards.  dq: nq x D, dk and dv: nk x D (fp64).
 */
int ora_attention_bwd_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const uint16_t* dout, int B, int H, int Sq, int Sk, int D, float scale,
                           int causal, int dtype, const int64_t* qrows, int64_t nq,
                           const int64_t* krows, int64_t nk, double* dq, double* dk, double* dv,
                           int nthreads) {
    if (!q || !k || !v || !dout || B < 0 || H < 0 || Sq < 0 || Sk < 0 || D <= 0) return 1;
    if ((nq > 0 && (!qrows || !dq)) || (nk > 0 && (!krows || !dk || !dv))) return 1;
    if (dtype != ORA_F16 && dtype != ORA_BF16) return 2;
    const int64_t BH = (int64_t)B * H;
    for (int64_t r = 0; r < nq; ++r) if (qrows[r] < 0 || qrows[r] >= BH * Sq) return 4;
    for (int64_t r = 0; r < nk; ++r) if (krows[r] < 0 || krows[r] >= BH * Sk) return 4;
    set_threads(nthreads);
    const double sc = (double)scale;
    const int64_t kh = (int64_t)Sk * D;
    const int nthr = ora_max_threads();
    const int64_t accn = 2 * (nk > 0 ? nk : 1) * (int64_t)D;
    const size_t skn = (size_t)(Sk > 0 ? Sk : 1);
    double* Kd = (double*)malloc(sizeof(double) * (size_t)(kh > 0 ? kh : 1));
    double* Vd = (double*)malloc(sizeof(double) * (size_t)(kh > 0 ? kh : 1));
    double* Qb = (double*)malloc(sizeof(double) * (size_t)nthr * D);
    double* Gb = (double*)malloc(sizeof(double) * (size_t)nthr * D);
    double* Pb = (double*)malloc(sizeof(double) * (size_t)nthr * skn);
    double* Sb = (double*)malloc(sizeof(double) * (size_t)nthr * skn);
    double* acc = (double*)malloc(sizeof(double) * (size_t)nthr * (size_t)accn);
    if (!Kd || !Vd || !Qb || !Gb || !Pb || !Sb || !acc) {
        free(Kd); free(Vd); free(Qb); free(Gb); free(Pb); free(Sb); free(acc);
        return 3;
    }
    for (int64_t r = 0; r < nk; ++r)
        for (int d = 0; d < D; ++d) { dk[r * D + d] = 0.0; dv[r * D + d] = 0.0; }
    for (int64_t bh = 0; bh < BH; ++bh) {
        int64_t nq_h = 0, nk_h = 0;
        for (int64_t r = 0; r < nq; ++r) nq_h += qrows[r] / Sq == bh;
        for (int64_t r = 0; r < nk; ++r) nk_h += krows[r] / Sk == bh;
        if (nq_h == 0 && nk_h == 0) continue;
        ora_decode(k + bh * kh, Kd, kh, dtype);
        ora_decode(v + bh * kh, Vd, kh, dtype);
        /* query rows to visit: every row of the head when a key is selected */
        const int64_t nvisit = nk_h > 0 ? Sq : 0;
        for (int t = 0; t < nthr; ++t)
            memset(acc + (size_t)t * accn, 0, sizeof(double) * (size_t)accn);
        #pragma omp parallel num_threads(nthr)
        {
            const int t = thread_id();
            double* Qr = Qb + (size_t)t * D;
            double* Gr = Gb + (size_t)t * D;
            double* Pr = Pb + (size_t)t * Sk;
            double* Sr = Sb + (size_t)t * Sk;
            double* ac = acc + (size_t)t * accn;
            /* selected dQ rows of this head */
            #pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < nq; ++r) {
                if (qrows[r] / Sq != bh) continue;
                const int64_t i = qrows[r] % Sq;
                ora_decode(q + qrows[r] * D, Qr, D, dtype);
                ora_decode(dout + qrows[r] * D, Gr, D, dtype);
                row_probs(Qr, Kd, i, Sq, Sk, D, sc, causal, Pr);
                double rowdot = 0.0;
                for (int64_t j = 0; j < Sk; ++j) {
                    const double* vr = Vd + j * D;
                    double dp = 0.0;
                    for (int d = 0; d < D; ++d) dp += Gr[d] * vr[d];
                    Sr[j] = dp;
                    rowdot += Pr[j] * dp;
                }
                double* gq = dq + r * D;
                for (int d = 0; d < D; ++d) gq[d] = 0.0;
                for (int64_t j = 0; j < Sk; ++j) {
                    const double ds = Pr[j] * (Sr[j] - rowdot);
                    const double* kr = Kd + j * D;
                    for (int d = 0; d < D; ++d) gq[d] += ds * kr[d];
                }
                for (int d = 0; d < D; ++d) gq[d] *= sc;
            }
            /* every query row of the head, for the selected keys */
            #pragma omp for schedule(static)
            for (int64_t i = 0; i < nvisit; ++i) {
                ora_decode(q + (bh * Sq + i) * D, Qr, D, dtype);
                ora_decode(dout + (bh * Sq + i) * D, Gr, D, dtype);
                row_probs(Qr, Kd, i, Sq, Sk, D, sc, causal, Pr);
                double rowdot = 0.0;
                for (int64_t j = 0; j < Sk; ++j) {
                    if (Pr[j] == 0.0) continue;
                    const double* vr = Vd + j * D;
                    double dp = 0.0;
                    for (int d = 0; d < D; ++d) dp += Gr[d] * vr[d];
                    rowdot += Pr[j] * dp;
                }
                for (int64_t r = 0; r < nk; ++r) {
                    if (krows[r] / Sk != bh) continue;
                    const int64_t j = krows[r] % Sk;
                    const double pij = Pr[j];
                    if (pij == 0.0) continue;
                    const double* vr = Vd + j * D;
                    double dp = 0.0;
                    for (int d = 0; d < D; ++d) dp += Gr[d] * vr[d];
                    const double sij = pij * (dp - rowdot);
                    double* av = ac + (r * 2) * D;
                    double* ak = ac + (r * 2 + 1) * D;
                    for (int d = 0; d < D; ++d) {
                        av[d] += pij * Gr[d];
                        ak[d] += sij * Qr[d];
                    }
                }
            }
        }
        /* partial sums added up in thread order */
        for (int t = 0; t < nthr; ++t) {
            const double* ac = acc + (size_t)t * accn;
            for (int64_t r = 0; r < nk; ++r) {
                if (krows[r] / Sk != bh) continue;
                for (int d = 0; d < D; ++d) {
                    dv[r * D + d] += ac[(r * 2) * D + d];
                    dk[r * D + d] += ac[(r * 2 + 1) * D + d];
                }
            }
        }
    }
    for (int64_t r = 0; r < nk; ++r)
        for (int d = 0; d < D; ++d) dk[r * D + d] *= sc;
    free(Kd); free(Vd); free(Qb); free(Gb); free(Pb); free(Sb); free(acc);
    return 0;
}

/*
 * Philox4x32-10, the counter-based generator of Salmon, Moraes, Dror and
 * Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC 2011): ten rounds
 * of two 32x32->64-bit multiplications (multipliers 0xD2511F53 and
 * 0xCD9E8D57) whose high halves are XOR-ed with the other counter words and
 * the key, and a Weyl bump of the key (0x9E3779B9, 0xBB67AE85) between
 * rounds.  Written from that definition; pinned against its published
 * known-answer vectors.
 */
void ora_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        const uint32_t n1 = (uint32_t)p1;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
        const uint32_t n3 = (uint32_t)p0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/*
 * Dropout threshold: keep probability 1 - t/65536 with t = round(p * 65536)
 * (ties to even, p < 1), so that the keep decision is an integer comparison.
 */
int ora_dropout_threshold(float p) {
    if (!(p >= 0.0f) || !(p < 1.0f)) return -1;
    const long t = lrintf(p * 65536.0f);
    return t > 65535 ? -1 : (int)t;
}

/* Keep decision of score (bh, i, j): the 16-bit value of key j among the
 * eight that one Philox4x32-10 call gives for counter (j/8, i, bh, offset)
 * under key (seed low word, seed high word): word (j%8)/2, low half for even
 * j, high half for odd j; kept iff that value >= t. */
static int keep_element(uint64_t seed, uint32_t offset, int64_t bh, int64_t i, int64_t j, int t) {
    const uint32_t ctr[4] = {(uint32_t)(j >> 3), (uint32_t)i, (uint32_t)bh, offset};
    const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    ora_philox4x32_10(ctr, key, out);
    const uint32_t r16 = (out[(j & 7) >> 1] >> (16 * (j & 1))) & 0xffffu;
    return (int)r16 >= t;
}

/*
 * The forward with an explicit boolean mask and dropout
 * ("FlashAttention-2 on Ascend NPU" (2048ai.net), section 3.4, fused mask
 * and dropout, and section 6.3):
 *   visible(i,j) = causal rule with the diagonal at offset c (j <= i + c)
 *                  and mask[b,h,i,j] != 0 (nonzero = keep, as the page's
 *                  kernel treats a true entry);
 *   P_ij         = softmax over the visible keys, lse_i as in the forward;
 *   O_i          = sum_j P_ij * keep_ij / (1 - t/65536) * v_j,
 * i.e. standard keep-and-rescale dropout applied to the probabilities (the
 * page's listing writes -inf into the scores instead, which renormalises and
 * is not dropout; that reading is not followed).  The lse is that of the
 * undropped softmax.  mask: uint8 with element strides (batch, head, row) in
 * mstride, columns contiguous; NULL = no mask.  dropout_p = 0 keeps all.
 */
static void row_attention_ext(const double* qrow, const double* K, const double* V, int64_t bh,
                              int64_t i, int64_t c, int64_t Sk, int D, double scale, int causal,
                              const uint8_t* mrow, int t, uint64_t seed, uint32_t offset,
                              double* srow, double* orow, double* lse_out) {
    for (int64_t j = 0; j < Sk; ++j) {
        const int vis = visible(i, j, c, causal) && (!mrow || mrow[j] != 0);
        if (!vis) { srow[j] = -INFINITY; continue; }
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += qrow[d] * K[j * D + d];
        srow[j] = scale * acc;
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < Sk; ++j) if (srow[j] > m) m = srow[j];
    for (int d = 0; d < D; ++d) orow[d] = 0.0;
    if (m == -INFINITY) { *lse_out = -INFINITY; return; }
    double l = 0.0;
    for (int64_t j = 0; j < Sk; ++j) {
        const double e = exp(srow[j] - m);
        srow[j] = e;
        l += e;
    }
    const double keep_scale = 65536.0 / (65536.0 - (double)t);
    for (int64_t j = 0; j < Sk; ++j) {
        if (srow[j] == 0.0) continue;
        if (t > 0 && !keep_element(seed, offset, bh, i, j, t)) continue;
        const double w = srow[j] / l * keep_scale;
        for (int d = 0; d < D; ++d) orow[d] += w * V[j * D + d];
    }
    *lse_out = m + log(l);
}

int ora_attention_fwd_ext(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int H,
                          int Sq, int Sk, int D, const uint8_t* mask, const int64_t* mstride,
                          float dropout_p, uint64_t seed, uint32_t offset, float scale, int causal,
                          int64_t causal_diag, int dtype, const int64_t* rows, int64_t nrows, double* o,
                          double* lse, int nthreads) {
    if (!q || !k || !v || !o || !lse || B < 0 || H < 0 || Sq < 0 || Sk < 0 || D <= 0) return 1;
    if (dtype != ORA_F16 && dtype != ORA_BF16) return 2;
    if (mask && !mstride) return 1;
    const int t = ora_dropout_threshold(dropout_p);
    if (t < 0) return 5;
    const int64_t total = (int64_t)B * H * Sq;
    const int64_t n = rows ? nrows : total;
    if (rows) for (int64_t r = 0; r < nrows; ++r) if (rows[r] < 0 || rows[r] >= total) return 4;
    set_threads(nthreads);
    const double sc = (double)scale;
    const int64_t kh = (int64_t)Sk * D;
    int err = 0;
    #pragma omp parallel
    {
        double* Qr = (double*)malloc(sizeof(double) * (size_t)D);
        double* Kd = (double*)malloc(sizeof(double) * (size_t)(kh > 0 ? kh : 1));
        double* Vd = (double*)malloc(sizeof(double) * (size_t)(kh > 0 ? kh : 1));
        double* Sr = (double*)malloc(sizeof(double) * (size_t)(Sk > 0 ? Sk : 1));
        int64_t cur_bh = -1;
        if (!Qr || !Kd || !Vd || !Sr) {
            #pragma omp atomic write
            err = 3;
        } else {
            #pragma omp for schedule(dynamic, 4)
            for (int64_t r = 0; r < n; ++r) {
                const int64_t row = rows ? rows[r] : r;
                const int64_t bh = row / Sq, i = row % Sq;
                if (bh != cur_bh) {
                    ora_decode(k + bh * kh, Kd, kh, dtype);
                    ora_decode(v + bh * kh, Vd, kh, dtype);
                    cur_bh = bh;
                }
                ora_decode(q + row * D, Qr, D, dtype);
                const uint8_t* mrow = NULL;
                if (mask) {
                    const int64_t b = bh / H, h = bh % H;
                    mrow = mask + b * mstride[0] + h * mstride[1] + i * mstride[2];
                }
                row_attention_ext(Qr, Kd, Vd, bh, i, causal_diag, Sk, D, sc, causal, mrow, t, seed, offset,
                                  Sr, o + r * D, lse + r);
            }
        }
        free(Qr); free(Kd); free(Vd); free(Sr);
    }
    return err;
}

/*
 * Backward of the forward with an explicit mask and dropout
 * (ora_attention_fwd_ext): with P the masked, undropped probabilities, Z the
 * keep indicators and c = 65536 / (65536 - t) the rescale,
 *   O_i   = sum_j P_ij Z_ij c v_j
 *   dV_j  = sum_i P_ij Z_ij c dO_i
 *   dP_ij = Z_ij c (dO_i . v_j)                  (gradient with respect to P_ij)
 *   dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)      (Jacobian of the row softmax)
 *   dQ_i  = scale sum_j dS_ij k_j,   dK_j = scale sum_i dS_ij q_i.
 * The chain rule through the forward's definition; nothing here is tiled.
 * Evaluated row by row: for each head with a selected row or key, every
 * query row's P, Z and dS are formed once; dQ is written for the selected
 * query rows (qrows, flat (b*H+h)*Sq+i) and dK, dV are accumulated for the
 * selected keys (krows, flat (b*H+h)*Sk+j), with per-thread partial sums
 * added in thread order.  dq: nq x D, dk and dv: nk x D (fp64).
 */
int ora_attention_bwd_ext(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                          const uint16_t* dout, int B, int H, int Sq, int Sk, int D,
                          const uint8_t* mask, const int64_t* mstride, float dropout_p,
                          uint64_t seed, uint32_t offset, float scale, int causal, int64_t causal_diag,
                          int dtype, const int64_t* qrows, int64_t nq, const int64_t* krows, int64_t nk,
                          double* dq, double* dk, double* dv, int nthreads) {
    if (!q || !k || !v || !dout || B < 0 || H < 0 || Sq < 0 || Sk < 0 || D <= 0) return 1;
    if ((nq > 0 && (!qrows || !dq)) || (nk > 0 && (!krows || !dk || !dv))) return 1;
    if (mask && !mstride) return 1;
    if (dtype != ORA_F16 && dtype != ORA_BF16) return 2;
    const int t = ora_dropout_threshold(dropout_p);
    if (t < 0) return 5;
    const int64_t BH = (int64_t)B * H;
    for (int64_t r = 0; r < nq; ++r) if (qrows[r] < 0 || qrows[r] >= BH * Sq) return 4;
    for (int64_t r = 0; r < nk; ++r) if (krows[r] < 0 || krows[r] >= BH * Sk) return 4;
    set_threads(nthreads);
    const double sc = (double)scale;
    const double keep_scale = 65536.0 / (double)(65536 - t);
    const int64_t kh = (int64_t)Sk * D;
    const int nthr = ora_max_threads();
    const int64_t accn = 2 * (nk > 0 ? nk : 1) * (int64_t)D;
    const size_t skn = (size_t)(Sk > 0 ? Sk : 1);
    double* Kd = (double*)malloc(sizeof(double) * (size_t)(kh > 0 ? kh : 1));
    double* Vd = (double*)malloc(sizeof(double) * (size_t)(kh > 0 ? kh : 1));
    double* Qb = (double*)malloc(sizeof(double) * (size_t)nthr * D);
    double* Gb = (double*)malloc(sizeof(double) * (size_t)nthr * D);
    double* Pb = (double*)malloc(sizeof(double) * (size_t)nthr * skn);
    double* Zb = (double*)malloc(sizeof(double) * (size_t)nthr * skn);
    double* Db = (double*)malloc(sizeof(double) * (size_t)nthr * skn);
    double* acc = (double*)malloc(sizeof(double) * (size_t)nthr * (size_t)accn);
    if (!Kd || !Vd || !Qb || !Gb || !Pb || !Zb || !Db || !acc) {
        free(Kd); free(Vd); free(Qb); free(Gb); free(Pb); free(Zb); free(Db); free(acc);
        return 3;
    }
    for (int64_t r = 0; r < nk; ++r)
        for (int d = 0; d < D; ++d) { dk[r * D + d] = 0.0; dv[r * D + d] = 0.0; }
    for (int64_t bh = 0; bh < BH; ++bh) {
        int64_t sel = 0;
        for (int64_t r = 0; r < nq; ++r) sel += qrows[r] / Sq == bh;
        for (int64_t r = 0; r < nk; ++r) sel += krows[r] / Sk == bh;
        if (sel == 0) continue;
        ora_decode(k + bh * kh, Kd, kh, dtype);
        ora_decode(v + bh * kh, Vd, kh, dtype);
        const int64_t b = bh / H, h = bh % H;
        for (int th = 0; th < nthr; ++th)
            memset(acc + (size_t)th * accn, 0, sizeof(double) * (size_t)accn);
        #pragma omp parallel for schedule(static) num_threads(nthr)
        for (int64_t i = 0; i < Sq; ++i) {
            const int th = thread_id();
            double* Qr = Qb + (size_t)th * D;
            double* Gr = Gb + (size_t)th * D;
            double* Pr = Pb + (size_t)th * skn;
            double* Zr = Zb + (size_t)th * skn;
            double* dPr = Db + (size_t)th * skn;
            double* ac = acc + (size_t)th * accn;
            ora_decode(q + (bh * Sq + i) * D, Qr, D, dtype);
            ora_decode(dout + (bh * Sq + i) * D, Gr, D, dtype);
            const uint8_t* mrow = mask ? mask + b * mstride[0] + h * mstride[1] + i * mstride[2] : NULL;
            /* masked, undropped probabilities */
            double m = -INFINITY;
            for (int64_t j = 0; j < Sk; ++j) {
                if (!visible(i, j, causal_diag, causal) || (mrow && mrow[j] == 0)) { Pr[j] = -INFINITY; continue; }
                double a = 0.0;
                for (int d = 0; d < D; ++d) a += Qr[d] * Kd[j * D + d];
                Pr[j] = sc * a;
                if (Pr[j] > m) m = Pr[j];
            }
            double l = 0.0;
            for (int64_t j = 0; j < Sk; ++j) {
                Pr[j] = m == -INFINITY ? 0.0 : exp(Pr[j] - m);
                l += Pr[j];
            }
            for (int64_t j = 0; j < Sk; ++j) Pr[j] = l > 0.0 ? Pr[j] / l : 0.0;
            /* keep factors, dP and the row term */
            double rowdot = 0.0;
            for (int64_t j = 0; j < Sk; ++j) {
                Zr[j] = (t == 0 || keep_element(seed, offset, bh, i, j, t)) ? keep_scale : 0.0;
                double a = 0.0;
                for (int d = 0; d < D; ++d) a += Gr[d] * Vd[j * D + d];
                dPr[j] = Zr[j] * a;
                rowdot += Pr[j] * dPr[j];
            }
            /* dQ of a selected row */
            for (int64_t r = 0; r < nq; ++r) {
                if (qrows[r] != bh * Sq + i) continue;
                double* gq = dq + r * D;
                for (int d = 0; d < D; ++d) gq[d] = 0.0;
                for (int64_t j = 0; j < Sk; ++j) {
                    const double ds = Pr[j] * (dPr[j] - rowdot);
                    for (int d = 0; d < D; ++d) gq[d] += ds * Kd[j * D + d];
                }
                for (int d = 0; d < D; ++d) gq[d] *= sc;
            }
            /* dK, dV of the selected keys */
            for (int64_t r = 0; r < nk; ++r) {
                if (krows[r] / Sk != bh) continue;
                const int64_t j = krows[r] - bh * Sk;
                if (Pr[j] == 0.0) continue;
                const double pz = Pr[j] * Zr[j];
                const double ds = Pr[j] * (dPr[j] - rowdot);
                double* av = ac + (r * 2) * D;
                double* ak = ac + (r * 2 + 1) * D;
                for (int d = 0; d < D; ++d) {
                    av[d] += pz * Gr[d];
                    ak[d] += ds * Qr[d];
                }
            }
        }
        for (int th = 0; th < nthr; ++th) {
            const double* ac = acc + (size_t)th * accn;
            for (int64_t r = 0; r < nk; ++r) {
                if (krows[r] / Sk != bh) continue;
                for (int d = 0; d < D; ++d) {
                    dv[r * D + d] += ac[(r * 2) * D + d];
                    dk[r * D + d] += ac[(r * 2 + 1) * D + d];
                }
            }
        }
    }
    for (int64_t r = 0; r < nk; ++r)
        for (int d = 0; d < D; ++d) dk[r * D + d] = sc * dk[r * D + d];
    free(Kd); free(Vd); free(Qb); free(Gb); free(Pb); free(Zb); free(Db); free(acc);
    return 0;
}
