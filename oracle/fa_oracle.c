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
 *     included).
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

static int visible(int64_t i, int64_t j, int64_t Sq, int64_t Sk, int causal) {
    if (!causal) return 1;
    return j <= i + (Sk - Sq);
}

/* One query row against all keys of its head: materialise the score row,
 * two-pass softmax, then the weighted sum of V.  qrow: D values; K, V:
 * Sk x D row-major; srow: Sk scratch.  Writes D outputs and the lse. */
static void row_attention(const double* qrow, const double* K, const double* V, int64_t i,
                          int64_t Sq, int64_t Sk, int D, double scale, int causal,
                          double* srow, double* orow, double* lse_out) {
    /* scores */
    for (int64_t j = 0; j < Sk; ++j) {
        if (!visible(i, j, Sq, Sk, causal)) { srow[j] = -INFINITY; continue; }
        const double* kr = K + j * D;
        double acc = 0.0;
        for (int d = 0; d < D; ++d) acc += qrow[d] * kr[d];
        srow[j] = scale * acc;
    }
    /* pass 1: row maximum */
    double m = -INFINITY;
    for (int64_t j = 0; j < Sk; ++j) if (srow[j] > m) m = srow[j];
    for (int d = 0; d < D; ++d) orow[d] = 0.0;
    if (m == -INFINITY) { *lse_out = -INFINITY; return; }
    /* pass 2: exponentials and their sum */
    double l = 0.0;
    for (int64_t j = 0; j < Sk; ++j) {
        double p = exp(srow[j] - m);
        srow[j] = p;
        l += p;
    }
    /* normalised probabilities times V */
    for (int64_t j = 0; j < Sk; ++j) {
        double p = srow[j] / l;
        if (p == 0.0) continue;
        const double* vr = V + j * D;
        for (int d = 0; d < D; ++d) orow[d] += p * vr[d];
    }
    *lse_out = m + log(l);
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
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
