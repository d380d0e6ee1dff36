/*
 * CPU oracle (fp64). TEST INFRASTRUCTURE ONLY: see oracle.h for the contract,
 * the format reading and who may use it. Built with gcc -O2, no -ffast-math.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int or_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads used by later parallel loops (n >= 1); scheduling only, no arithmetic. */
void or_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

static uint16_t rd16(const uint8_t* p) { return (uint16_t)(p[0] | (p[1] << 8)); }

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double or_half_to_double(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);              /* subnormal: f * 2^-14 / 1024 */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25);  /* (1 + f/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/*
 * 6-bit fields of the Q4_K scale bytes s[0..11]:
 *   j < 4 : sc[j] = low 6 bits of s[j],   m[j] = low 6 bits of s[j+4]
 *   j >= 4: sc[j] = low nibble of s[j+4]  | (top 2 bits of s[j-4]) << 4
 *           m[j]  = high nibble of s[j+4] | (top 2 bits of s[j])   << 4
 */
void or_q4k_unpack_scales(const uint8_t s[12], int sc[8], int m[8]) {
    for (int j = 0; j < 4; ++j) {
        sc[j] = s[j] & 63;
        m[j] = s[j + 4] & 63;
    }
    for (int j = 4; j < 8; ++j) {
        sc[j] = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        m[j] = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* Quant (0..15) of weight i (0..255) of a Q4_K block's 128 nibble bytes. */
static int q4k_quant(const uint8_t* qs, int i) {
    int g = i / 64;          /* 64-weight group, 32 bytes each */
    int r = i % 64;
    uint8_t byte = qs[32 * g + (r % 32)];
    return (r < 32) ? (byte & 15) : (byte >> 4);
}

void or_q4k_dequant_block(const uint8_t blk[144], double w[256]) {
    double d = or_half_to_double(rd16(blk));
    double dmin = or_half_to_double(rd16(blk + 2));
    int sc[8], m[8];
    or_q4k_unpack_scales(blk + 4, sc, m);
    const uint8_t* qs = blk + 16;
    for (int i = 0; i < 256; ++i) {
        int j = i / 32;
        w[i] = d * sc[j] * q4k_quant(qs, i) - dmin * m[j];
    }
}

void or_q8_0_dequant_block(const uint8_t blk[34], double w[32]) {
    double d = or_half_to_double(rd16(blk));
    for (int i = 0; i < 32; ++i) w[i] = d * (double)(int8_t)blk[2 + i];
}

/* 6-bit quant (0..63) of weight i (0..255) of a Q6_K block. */
static int q6k_quant(const uint8_t* ql, const uint8_t* qh, int i) {
    int h = i / 128;         /* 128-weight half: ql + 64h, qh + 32h */
    int p = (i % 128) / 32;  /* quarter of the half */
    int l = i % 32;
    uint8_t lo_byte = ql[64 * h + l + 32 * (p % 2)];
    int lo = (p < 2) ? (lo_byte & 15) : (lo_byte >> 4);
    int hi = (qh[32 * h + l] >> (2 * p)) & 3;
    return lo | (hi << 4);
}

void or_q6k_dequant_block(const uint8_t blk[210], double w[256]) {
    const uint8_t* ql = blk;
    const uint8_t* qh = blk + 128;
    const int8_t* sc = (const int8_t*)(blk + 192);
    double d = or_half_to_double(rd16(blk + 208));
    for (int i = 0; i < 256; ++i) w[i] = d * sc[i / 16] * (q6k_quant(ql, qh, i) - 32);
}

void or_q4k_dequant_row(const uint8_t* row, int64_t K, double* w) {
    for (int64_t b = 0; b < K / 256; ++b) or_q4k_dequant_block(row + 144 * b, w + 256 * b);
}

void or_q8_0_dequant_row(const uint8_t* row, int64_t K, double* w) {
    for (int64_t b = 0; b < K / 32; ++b) or_q8_0_dequant_block(row + 34 * b, w + 32 * b);
}

void or_q6k_dequant_row(const uint8_t* row, int64_t K, double* w) {
    for (int64_t b = 0; b < K / 256; ++b) or_q6k_dequant_block(row + 210 * b, w + 256 * b);
}

/* Plain dot product, sequential in k, of a dequantized row with x. */
static void dot_row(const double* w, const float* x, int64_t K, double* y, double* a) {
    double s = 0.0, t = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double p = w[k] * (double)x[k];
        s += p;
        t += fabs(p);
    }
    *y = s;
    if (a) *a = t;
}

typedef void (*dequant_row_fn)(const uint8_t*, int64_t, double*);

static void gemv_dense(dequant_row_fn deq, int64_t row_bytes, const uint8_t* W, int64_t K,
                       const float* x, const int64_t* rows, int64_t nrows, double* y, double* a) {
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
        for (int64_t i = 0; i < nrows; ++i) {
            int64_t r = rows ? rows[i] : i;
            deq(W + r * row_bytes, K, w);
            dot_row(w, x, K, &y[i], a ? &a[i] : NULL);
        }
        free(w);
    }
}

void or_gemv_q4k(const uint8_t* W, int64_t M, int64_t K, const float* x,
                 const int64_t* rows, int64_t nrows, double* y, double* a) {
    (void)M;
    gemv_dense(or_q4k_dequant_row, (K / 256) * 144, W, K, x, rows, nrows, y, a);
}

void or_gemv_q8_0(const uint8_t* W, int64_t M, int64_t K, const float* x,
                  const int64_t* rows, int64_t nrows, double* y, double* a) {
    (void)M;
    gemv_dense(or_q8_0_dequant_row, (K / 32) * 34, W, K, x, rows, nrows, y, a);
}

void or_gemv_q6k(const uint8_t* W, int64_t M, int64_t K, const float* x,
                 const int64_t* rows, int64_t nrows, double* y, double* a) {
    (void)M;
    gemv_dense(or_q6k_dequant_row, (K / 256) * 210, W, K, x, rows, nrows, y, a);
}

void or_gemv_q4k_factored(const uint8_t* W, int64_t M, int64_t K, const float* x,
                          const int64_t* rows, int64_t nrows, double* y) {
    (void)M;
    int64_t nb = K / 256;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows ? rows[i] : i;
        const uint8_t* row = W + r * nb * 144;
        double acc = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t* blk = row + 144 * b;
            double d = or_half_to_double(rd16(blk));
            double dmin = or_half_to_double(rd16(blk + 2));
            int sc[8], m[8];
            or_q4k_unpack_scales(blk + 4, sc, m);
            for (int j = 0; j < 8; ++j) {
                double S = 0.0, X = 0.0;
                for (int l = 0; l < 32; ++l) {
                    double xv = (double)x[256 * b + 32 * j + l];
                    S += q4k_quant(blk + 16, 32 * j + l) * xv;
                    X += xv;
                }
                acc += d * sc[j] * S - dmin * m[j] * X;
            }
        }
        y[i] = acc;
    }
}

void or_gemm_q4k(const uint8_t* W, int64_t M, int64_t K, const float* X, int64_t ldx,
                 int64_t N, const int64_t* rows, int64_t nrows, double* Y, double* A) {
    for (int64_t n = 0; n < N; ++n)
        or_gemv_q4k(W, M, K, X + n * ldx, rows, nrows, Y + n * nrows, A ? A + n * nrows : NULL);
}

int64_t or_argmax(const double* y, int64_t n) {
    if (n <= 0) return -1;
    int64_t best = 0;
    for (int64_t i = 1; i < n; ++i)
        if (y[i] > y[best]) best = i;   /* strict: ties keep the lower index */
    return best;
}

/* ------------------------------------------------------------------ int8 activations */

void or_quantize_q8_1(const float* x, int64_t K, float* d, int8_t* q, int16_t* s) {
    for (int64_t b = 0; b < K / 32; ++b) {
        const float* xb = x + 32 * b;
        float amax = 0.0f;
        for (int i = 0; i < 32; ++i)
            if (fabsf(xb[i]) > amax) amax = fabsf(xb[i]);
        const float db = amax / 127.0f;
        d[b] = db;
        int sum = 0;
        for (int i = 0; i < 32; ++i) {
            float v = 0.0f;
            if (db != 0.0f) {
                v = rintf(xb[i] / db);
                if (v > 127.0f) v = 127.0f;
                if (v < -127.0f) v = -127.0f;
            }
            q[32 * b + i] = (int8_t)v;
            sum += (int)v;
        }
        s[b] = (int16_t)sum;
    }
}

void or_gemv_q4k_q8_1(const uint8_t* W, int64_t M, int64_t K, const float* d, const int8_t* q,
                      const int64_t* rows, int64_t nrows, double* y, double* a) {
    (void)M;
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
        for (int64_t i = 0; i < nrows; ++i) {
            const int64_t r = rows ? rows[i] : i;
            or_q4k_dequant_row(W + r * (K / 256) * 144, K, w);
            double sum = 0.0, t = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double p = w[k] * ((double)d[k / 32] * (double)q[k]);
                sum += p;
                t += fabs(p);
            }
            y[i] = sum;
            if (a) a[i] = t;
        }
        free(w);
    }
}

void or_gemv_q8_0_q8_1(const uint8_t* W, int64_t M, int64_t K, const float* d, const int8_t* q,
                      const int64_t* rows, int64_t nrows, double* y, double* a) {
    (void)M;
#pragma omp parallel
    {
        double* w = (double*)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
        for (int64_t i = 0; i < nrows; ++i) {
            const int64_t r = rows ? rows[i] : i;
            or_q8_0_dequant_row(W + r * (K / 32) * 34, K, w);
            double sum = 0.0, t = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double p = w[k] * ((double)d[k / 32] * (double)q[k]);
                sum += p;
                t += fabs(p);
            }
            y[i] = sum;
            if (a) a[i] = t;
        }
        free(w);
    }
}

/* ------------------------------------------------------------------ sampling */

static double finite_or_neg_inf(double v) { return v != v ? -INFINITY : v; }

void or_topk(const double* z, int64_t n, int k, int64_t* out_idx) {
    unsigned char* taken = (unsigned char*)calloc((size_t)n, 1);
    for (int r = 0; r < k; ++r) {
        int64_t best = -1;
        for (int64_t i = 0; i < n; ++i) {
            if (taken[i]) continue;
            /* strict comparison: among equal values the lower index stays */
            if (best < 0 || finite_or_neg_inf(z[i]) > finite_or_neg_inf(z[best])) best = i;
        }
        out_idx[r] = best;
        if (best >= 0) taken[best] = 1;
    }
    free(taken);
}

double or_logsumexp(const double* z, int64_t n) {
    double m = -INFINITY;
    for (int64_t i = 0; i < n; ++i)
        if (finite_or_neg_inf(z[i]) > m) m = z[i];
    if (m == -INFINITY) return -INFINITY;
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) s += exp(finite_or_neg_inf(z[i]) - m);
    return m + log(s);
}

int or_sample_topk(const double* z, int k, double temperature, double top_p, double min_p, double u) {
    if (temperature <= 0.0 || k == 1) return 0;
    double* q = (double*)malloc(sizeof(double) * (size_t)k);
    double total = 0.0;
    for (int i = 0; i < k; ++i) {
        q[i] = exp((finite_or_neg_inf(z[i]) - z[0]) / temperature);
        total += q[i];
    }
    /* top-p: shortest prefix whose weight reaches top_p of the total */
    int n = k;
    if (top_p < 1.0) {
        double c = 0.0;
        for (n = 0; n < k;) {
            c += q[n];
            ++n;
            if (c >= top_p * total) break;
        }
    }
    /* min-p: entries whose weight is at least min_p times the largest (q[0] = 1) */
    int m = 0;
    for (int i = 0; i < n; ++i)
        if (q[i] >= min_p * q[0]) m = i + 1;
    double kept = 0.0;
    for (int i = 0; i < m; ++i) kept += q[i];
    const double target = u * kept;
    double c = 0.0;
    int j = m - 1;
    for (int i = 0; i < m; ++i) {
        c += q[i];
        if (c > target) {
            j = i;
            break;
        }
    }
    free(q);
    return j;
}
