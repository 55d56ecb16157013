/*
 * CPU oracle for the transformer linear layer.  TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The product path never calls it, and it shares no
 * code, header or constant with the HIP library.
 *
 * What it computes (the plain definition, no blocking, no reordering):
 *
 *   ref[m][n] = sum_{k=0}^{K-1} x(m,k) * w(n,k)      accumulated in double,
 *                                                     k ascending
 *   ref[m][n] += b[n]                                 if the bias flag is set
 *   ref[m][n]  = gelu_tanh(ref[m][n])                 if the GELU flag is set
 *
 * "One multiply, one RTX 5090, eight kernels", section "The multiply": X holds
 * one row per input vector, W is stored out×in as PyTorch stores it, and each
 * value of Y is the dot product of one row of X with one row of W.
 * Layout 1 ("KN") is the square row-major product of "Writing a CUDA matmul
 * that catches cuBLAS", section "Kernel 1 → 2", where B is [K][N]:
 * w(n,k) = B[k][n].
 *
 * Every product of two stored inputs is exact in double (at most 24-bit
 * significands), so the only rounding is the K additions in ascending k.
 * Nothing is rounded back to the output format: the result stays double.
 *
 * GELU is the tanh form used by GPT-2:
 *   gelu(y) = 0.5 * y * (1 + tanh(sqrt(2/pi) * (y + 0.044715 * y^3)))
 * evaluated in double with libm tanh.  The pages name a GELU epilogue fused
 * after the bias ("Writing a CUDA matmul that catches cuBLAS", section "The
 * residual and GELU go the same way, and cost three detours") without
 * printing the formula; the tanh form is the reading taken.
 *
 * Element formats: 0 = IEEE binary32, 1 = IEEE binary16, 2 = bfloat16 (the
 * upper 16 bits of a binary32).  All are decoded exactly into double here.
 *
 * The end of the file holds the two operations that complete a GPT-2 layer
 * around the GEMMs, written out the same way: layer normalisation and causal
 * scaled dot-product attention.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };
enum { OR_LAYOUT_NK = 0, OR_LAYOUT_KN = 1 };

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double decode_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24); /* subnormal: f * 2^-14 * 2^-10 */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(f + 1024), e - 25); /* (1 + f/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* bfloat16 is the top half of a binary32 pattern. */
static double decode_bf16(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load(const void* base, int64_t idx, int dtype) {
    switch (dtype) {
    case OR_F32: return (double)((const float*)base)[idx];
    case OR_F16: return decode_f16(((const uint16_t*)base)[idx]);
    default: return decode_bf16(((const uint16_t*)base)[idx]);
    }
}

double oracle_gelu_tanh(double y) {
    const double c = sqrt(2.0 / acos(-1.0)); /* sqrt(2/pi) */
    return 0.5 * y * (1.0 + tanh(c * (y + 0.044715 * y * y * y)));
}

double oracle_decode(const void* base, int64_t idx, int dtype) { return load(base, idx, dtype); }

/* One output element, the definition written out. */
static double element(int64_t m, int64_t n, int64_t N, int64_t K, int dtype, int layout,
                      const void* X, const void* W, const void* bias, int flags) {
    double acc = 0.0;
    for (int64_t k = 0; k < K; ++k) {
        double x = load(X, m * K + k, dtype);
        double w = layout == OR_LAYOUT_NK ? load(W, n * K + k, dtype) : load(W, k * N + n, dtype);
        acc += x * w;
    }
    if (flags & 1) acc += load(bias, n, dtype);
    if (flags & 2) acc = oracle_gelu_tanh(acc);
    return acc;
}

static int check(int64_t M, int64_t N, int64_t K, int dtype, int layout, const void* X,
                 const void* W, const void* bias, int flags, const void* Y) {
    if (M < 0 || N < 0 || K < 0) return -1;
    if (dtype < OR_F32 || dtype > OR_BF16) return -1;
    if (layout != OR_LAYOUT_NK && layout != OR_LAYOUT_KN) return -1;
    if (flags & ~3) return -1;
    if ((flags & 1) && !bias) return -1;
    if (!Y || (M * K > 0 && !X) || (N * K > 0 && !W)) return -1;
    return 0;
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
}

/* Rows [m0, m1) of the full output; Y is [(m1-m0)][N] row-major doubles. */
int oracle_linear_rows(int64_t M, int64_t N, int64_t K, int dtype, int layout, const void* X,
                       const void* W, const void* bias, int flags, int64_t m0, int64_t m1,
                       double* Y, int nthreads) {
    if (check(M, N, K, dtype, layout, X, W, bias, flags, Y)) return -1;
    if (m0 < 0 || m1 > M || m0 > m1) return -1;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = m0; m < m1; ++m)
        for (int64_t n = 0; n < N; ++n)
            Y[(m - m0) * N + n] = element(m, n, N, K, dtype, layout, X, W, bias, flags);
    return 0;
}

int oracle_linear(int64_t M, int64_t N, int64_t K, int dtype, int layout, const void* X,
                  const void* W, const void* bias, int flags, double* Y, int nthreads) {
    return oracle_linear_rows(M, N, K, dtype, layout, X, W, bias, flags, 0, M, Y, nthreads);
}

/* Selected elements (mi[i], ni[i]) for sampled checks at full size. */
int oracle_linear_points(int64_t M, int64_t N, int64_t K, int dtype, int layout, const void* X,
                         const void* W, const void* bias, int flags, int64_t npts,
                         const int64_t* mi, const int64_t* ni, double* out, int nthreads) {
    if (check(M, N, K, dtype, layout, X, W, bias, flags, out)) return -1;
    for (int64_t i = 0; i < npts; ++i)
        if (mi[i] < 0 || mi[i] >= M || ni[i] < 0 || ni[i] >= N) return -1;
    set_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t i = 0; i < npts; ++i)
        out[i] = element(mi[i], ni[i], N, K, dtype, layout, X, W, bias, flags);
    return 0;
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---- the operations around the GEMMs in a GPT-2 layer ----------------------------
 *
 * Layer normalisation of each row of X [rows][C] ("mage-003: What the kernels
 * were short of", the layer-normalisation section): mean and biased variance
 * over the row, in double, k ascending; y = (x - mean) / sqrt(var + eps) *
 * gamma + beta.  Y, mean and rstd = 1/sqrt(var + eps) stay double.
 */
int oracle_layernorm(int64_t rows, int64_t C, int dtype, const void* X, const void* gamma, const void* beta,
                     double eps, double* Y, double* mean, double* rstd, int nthreads) {
    if (rows < 1 || C < 1 || !X || !gamma || !beta || !Y || (dtype != OR_F32 && dtype != OR_F16 && dtype != OR_BF16))
        return -1;
    set_threads(nthreads);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double s = 0.0;
        for (int64_t c = 0; c < C; ++c) s += load(X, r * C + c, dtype);
        const double mu = s / (double)C;
        double v = 0.0;
        for (int64_t c = 0; c < C; ++c) {
            const double d = load(X, r * C + c, dtype) - mu;
            v += d * d;
        }
        const double rs = 1.0 / sqrt(v / (double)C + eps);
        for (int64_t c = 0; c < C; ++c)
            Y[r * C + c] = (load(X, r * C + c, dtype) - mu) * rs * load(gamma, c, dtype) + load(beta, c, dtype);
        if (mean) mean[r] = mu;
        if (rstd) rstd[r] = rs;
    }
    return 0;
}

/*
 * Scaled dot-product attention over the output of the qkv projection
 * ("Writing a CUDA matmul that catches cuBLAS", section "Fusing attention:
 * the score matrix never exists"): qkv is [B][T][3C] with C = NH * HS, the
 * query of head h at columns h*HS .. h*HS+HS-1, its key C further and its
 * value 2C further.  For each (b, h, i):
 *   s_j = scale * sum_d q[i][d] k[j][d]   for j <= i (causal) or every j,
 *   m = max_j s_j,  l = sum_j exp(s_j - m),  lse = m + log(l),
 *   out[b][i][h*HS + d] = sum_j exp(s_j - m) / l * v[j][d],
 * with scale = 1/sqrt(HS) (the pages print no scale; the usual one is the
 * reading taken).  Sums in double, j ascending.  out is [B][T][C], lse [B][NH][T].
 */
int oracle_attention(int64_t B, int64_t T, int64_t NH, int64_t HS, int dtype, const void* qkv, int causal,
                     double* out, double* lse, int nthreads) {
    if (B < 1 || T < 1 || NH < 1 || HS < 1 || !qkv || !out || (dtype != OR_F32 && dtype != OR_F16 && dtype != OR_BF16))
        return -1;
    const int64_t C = NH * HS, C3 = 3 * C;
    const double scale = 1.0 / sqrt((double)HS);
    set_threads(nthreads);
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t h = 0; h < NH; ++h) {
            for (int64_t i = 0; i < T; ++i) {
                const int64_t jend = causal ? i + 1 : T;
                const int64_t qrow = (b * T + i) * C3 + h * HS;
                double m = -INFINITY;
                for (int64_t j = 0; j < jend; ++j) {
                    const int64_t krow = (b * T + j) * C3 + C + h * HS;
                    double d = 0.0;
                    for (int64_t e = 0; e < HS; ++e) d += load(qkv, qrow + e, dtype) * load(qkv, krow + e, dtype);
                    d *= scale;
                    if (d > m) m = d;
                }
                double l = 0.0;
                double* o = out + (b * T + i) * C + h * HS;
                for (int64_t e = 0; e < HS; ++e) o[e] = 0.0;
                for (int64_t j = 0; j < jend; ++j) {
                    const int64_t krow = (b * T + j) * C3 + C + h * HS, vrow = (b * T + j) * C3 + 2 * C + h * HS;
                    double d = 0.0;
                    for (int64_t e = 0; e < HS; ++e) d += load(qkv, qrow + e, dtype) * load(qkv, krow + e, dtype);
                    const double p = exp(d * scale - m);
                    l += p;
                    for (int64_t e = 0; e < HS; ++e) o[e] += p * load(qkv, vrow + e, dtype);
                }
                for (int64_t e = 0; e < HS; ++e) o[e] /= l;
                if (lse) lse[(b * NH + h) * T + i] = m + log(l);
            }
        }
    }
    return 0;
}
