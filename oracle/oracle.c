/*
 * oracle.c — TEST INFRASTRUCTURE ONLY.  A plain, slow, obviously-correct fp64
 * reference for the swizzled-operand GEMM.  Only tests/, the smoke() entry and
 * bench.py's cpu_baseline leg may load this library.  It shares no code, header
 * or constant with the GPU library (mma_swizzled_operand_amd/), and the GPU
 * library never calls it.
 *
 * What it computes (tcgen05.mma page, sections "Operands and repeat axes" and
 * "Example: four K16 issues for a 128x64x64 product"): D = A . B^T with B held
 * as (N,K), accumulated into fp32 cells; `accum` off on the first K issue
 * means the old D is ignored, on means it is added.  Block scaling (same page,
 * "Weight-stationary and block scaling") attaches one scale per row and per
 * block of consecutive K elements to each operand.
 *
 *   a(m,k) = A[m*K + k]   (A K-major, stored [M][K])
 *          = A[k*M + m]   (A MN-major, stored [K][M])
 *   b(n,k) = B[n*K + k]   (B K-major, stored [N][K])
 *          = B[k*N + n]   (B MN-major, stored [K][N])
 *   dense:        D[m][n] = beta*D0[m][n] + sum_k a(m,k) * b(n,k)
 *   block-scaled: D[m][n] = beta*D0[m][n]
 *                 + sum_k (2^(SFA[m][k/V]-127) a(m,k)) * (2^(SFB[n][k/V]-127) b(n,k))
 *
 * Every stored element is first decoded to the exact real number its bit
 * pattern encodes (fp64 holds every fp16, bf16, e4m3, e2m3, e3m2, e2m1 and e8m0
 * value exactly),
 * then the K products are summed in fp64 in increasing k.  The componentwise
 * magnitude S[m][n] = sum_k |a*b| is returned beside D for error bounds.
 *
 * Readings taken where the pages are silent: the 8-bit element format is OCP
 * E4M3 (bias 7, no infinities, S.1111.111 is NaN); the 4-bit one (the pages'
 * FP4, "four-bit values") is OCP E2M1, packed two per byte, low nibble first;
 * the 6-bit ones (the pages' FP6, "six-bit values") are OCP E2M3 and E3M2,
 * stored in the pages' padded form of the decompression copy (tcgen05.cp page,
 * "Native FP4/FP6 decompression": each 16-byte block holds sixteen packed
 * values followed by four bytes of padding), read as value j of a block in
 * bits 6j .. 6j+5 of its first twelve bytes taken little-endian; the padded
 * 4-bit form of the same section (sixteen values followed by eight bytes of
 * padding) holds value j in bits 4j .. 4j+3 of the block's first eight bytes
 * (low nibble first);
 * a scale byte E means 2^(E-127) (OCP E8M0, 255 is NaN); scale blocks start
 * at k = 0, V, 2V, ...; beta is 0 or 1 and beta = 0 never reads D0.
 *
 * Parity status of each function is recorded in the header of oracle/__init__.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Element kinds understood by the oracle (its own numbering).  ORC_E2M1
 * elements are packed two per byte: element 2j in bits 0..3 of byte j,
 * element 2j+1 in bits 4..7.  ORC_E2M3 / ORC_E3M2 elements are packed sixteen
 * per 16-byte block: element 16b + j in bits 6j .. 6j+5 of bytes 16b .. 16b+11
 * read as one little-endian number; bytes 16b+12 .. 16b+15 are padding and
 * never read. */
enum { ORC_F16 = 1, ORC_BF16 = 2, ORC_E4M3 = 3, ORC_F32 = 4, ORC_E2M1 = 5, ORC_E2M3 = 6, ORC_E3M2 = 7,
       ORC_E2M1_P64 = 8 };   /* E2M1 sixteen per 16-byte block: value 16b + j in the low (j even) or
                                high (j odd) nibble of byte 16b + j/2; bytes 16b+8 .. 16b+15 padding */
/* Operand majors (its own numbering). */
enum { ORC_KMAJOR = 0, ORC_MNMAJOR = 1 };
/* Return codes. */
enum { ORC_OK = 0, ORC_BAD_ARG = -1, ORC_NO_MEM = -2 };

/* ---- element decoders: bit fields -> exact real value ------------------- */

/* IEEE-754 binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double orc_decode_f16(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 0x1f, f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-14 * 2^-10 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);     /* (1 + f/2^10) * 2^(e-15) */
    return s ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
double orc_decode_bf16(uint16_t h)
{
    int s = h >> 15, e = (h >> 7) & 0xff, f = h & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);                /* f * 2^-126 * 2^-7 */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134);     /* (1 + f/2^7) * 2^(e-127) */
    return s ? -v : v;
}

/* OCP E4M3: 1 sign, 4 exponent (bias 7), 3 fraction bits; no infinities,
 * exponent 15 with fraction 7 is NaN, so the largest finite value is 448. */
double orc_decode_e4m3(uint8_t b)
{
    int s = b >> 7, e = (b >> 3) & 0xf, f = b & 0x7;
    double v;
    if (e == 15 && f == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)f, -9);                  /* f * 2^-6 * 2^-3 */
    else
        v = ldexp((double)(8 + f), e - 10);        /* (1 + f/8) * 2^(e-7) */
    return s ? -v : v;
}

/* OCP E2M1 (4-bit): 1 sign, 2 exponent (bias 1), 1 fraction bit; no
 * infinities or NaN.  Exponent 0 is subnormal: f * 2^-1; otherwise
 * (1 + f/2) * 2^(e-1), so the magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double orc_decode_e2m1(uint8_t nibble)
{
    int s = (nibble >> 3) & 1, e = (nibble >> 1) & 3, f = nibble & 1;
    double v = e == 0 ? ldexp((double)f, -1) : ldexp((double)(2 + f), e - 2);
    return s ? -v : v;
}

/* OCP E2M3 (6-bit): 1 sign, 2 exponent (bias 1), 3 fraction bits; no
 * infinities or NaN.  Exponent 0 is subnormal: f/8; otherwise
 * (1 + f/8) * 2^(e-1); the largest magnitude is 7.5. */
double orc_decode_e2m3(uint8_t code)
{
    int s = (code >> 5) & 1, e = (code >> 3) & 3, f = code & 7;
    double v = e == 0 ? ldexp((double)f, -3) : ldexp((double)(8 + f), e - 4);
    return s ? -v : v;
}

/* OCP E3M2 (6-bit): 1 sign, 3 exponent (bias 3), 2 fraction bits; no
 * infinities or NaN.  Exponent 0 is subnormal: f/4 * 2^-2; otherwise
 * (1 + f/4) * 2^(e-3); the largest magnitude is 28. */
double orc_decode_e3m2(uint8_t code)
{
    int s = (code >> 5) & 1, e = (code >> 2) & 7, f = code & 3;
    double v = e == 0 ? ldexp((double)f, -4) : ldexp((double)(4 + f), e - 5);
    return s ? -v : v;
}

/* The 6-bit code of element idx of a padded FP6 array (see ORC_E2M3). */
static uint8_t fp6_code(const uint8_t *base, int64_t idx)
{
    const uint8_t *blk = base + (idx / 16) * 16;
    const int bit = 6 * (int)(idx % 16);               /* 0 .. 90 */
    const int byte = bit / 8, sh = bit % 8;            /* byte <= 11 */
    unsigned v = blk[byte];
    if (sh > 2)                                        /* the code spills into the next byte (<= 11) */
        v |= (unsigned)blk[byte + 1] << 8;
    return (uint8_t)((v >> sh) & 0x3f);
}

/* OCP E8M0 scale: 2^(E-127); E = 255 is NaN. */
double orc_decode_e8m0(uint8_t b)
{
    return b == 255 ? NAN : ldexp(1.0, (int)b - 127);
}

static int elem_size(int dt)
{
    switch (dt) {
    case ORC_F16: case ORC_BF16: return 2;
    case ORC_E4M3: return 1;
    case ORC_F32: return 4;
    case ORC_E2M1: return 1;   /* storage byte (two elements) */
    case ORC_E2M3: case ORC_E3M2: case ORC_E2M1_P64: return 1;   /* 16 bytes per 16 elements */
    default: return 0;
    }
}

static double decode_one(int dt, const void *base, int64_t idx)
{
    switch (dt) {
    case ORC_F16: return orc_decode_f16(((const uint16_t *)base)[idx]);
    case ORC_BF16: return orc_decode_bf16(((const uint16_t *)base)[idx]);
    case ORC_E4M3: return orc_decode_e4m3(((const uint8_t *)base)[idx]);
    case ORC_F32: return (double)((const float *)base)[idx];
    case ORC_E2M1: {
        const uint8_t byte = ((const uint8_t *)base)[idx >> 1];
        return orc_decode_e2m1((idx & 1) ? byte >> 4 : byte & 0xf);
    }
    case ORC_E2M3: return orc_decode_e2m3(fp6_code((const uint8_t *)base, idx));
    case ORC_E3M2: return orc_decode_e3m2(fp6_code((const uint8_t *)base, idx));
    case ORC_E2M1_P64: {
        const uint8_t byte = ((const uint8_t *)base)[(idx / 16) * 16 + (idx % 16) / 2];
        return orc_decode_e2m1((idx & 1) ? byte >> 4 : byte & 0xf);
    }
    default: return NAN;
    }
}

/* Decode n stored elements of kind dt into fp64. */
int orc_decode(int dt, const void *src, int64_t n, double *dst)
{
    if (!elem_size(dt) || (n > 0 && (!src || !dst)) || n < 0)
        return ORC_BAD_ARG;
    for (int64_t i = 0; i < n; ++i)
        dst[i] = decode_one(dt, src, i);
    return ORC_OK;
}

/* ---- the GEMM ------------------------------------------------------------ */

static int n_threads = 0; /* 0: OpenMP default */

void orc_set_threads(int n) { n_threads = n; }

int orc_get_threads(void)
{
#ifdef _OPENMP
    return n_threads > 0 ? n_threads : omp_get_max_threads();
#else
    return 1;
#endif
}

/* Operand element (row `r` of the logical [R][K] operand, column k), read
 * through its major: K-major storage is [R][K], MN-major storage is [K][R]. */
static double operand_at(int dt, int major, const void *X, int64_t R, int64_t K,
                         int64_t r, int64_t k)
{
    int64_t idx = (major == ORC_KMAJOR) ? r * K + k : k * R + r;
    return decode_one(dt, X, idx);
}

/*
 * Reference D for the selected rows x selected columns of the product.
 *   rows: n_rows indices into [0,M) or NULL for all M rows (n_rows ignored)
 *   cols: n_cols indices into [0,N) or NULL for all N columns
 *   V:    0 for dense; otherwise the number of consecutive K elements that
 *         share one scale byte (SFA is [M][K/V], SFB is [N][K/V])
 *   Dref, Smag: [n_rows][n_cols] row-major fp64 outputs (Smag may be NULL)
 * Returns ORC_OK, ORC_BAD_ARG or ORC_NO_MEM.
 */
int orc_gemm(int64_t M, int64_t N, int64_t K,
             int a_dt, int a_major, const void *A,
             int b_dt, int b_major, const void *B,
             int32_t V, const uint8_t *SFA, const uint8_t *SFB,
             int beta, const float *D0,
             int64_t n_rows, const int64_t *rows,
             int64_t n_cols, const int64_t *cols,
             double *Dref, double *Smag)
{
    if (M <= 0 || N <= 0 || K <= 0 || !A || !B || !Dref)
        return ORC_BAD_ARG;
    if (a_dt == ORC_F32 || b_dt == ORC_F32 || !elem_size(a_dt) || !elem_size(b_dt))
        return ORC_BAD_ARG;
    if ((a_major != ORC_KMAJOR && a_major != ORC_MNMAJOR) ||
        (b_major != ORC_KMAJOR && b_major != ORC_MNMAJOR))
        return ORC_BAD_ARG;
    if (V < 0 || (V > 0 && (K % V != 0 || !SFA || !SFB)))
        return ORC_BAD_ARG;
    if (beta != 0 && beta != 1)
        return ORC_BAD_ARG;
    if (beta == 1 && !D0)
        return ORC_BAD_ARG;
    if (!rows) n_rows = M;
    if (!cols) n_cols = N;
    if (n_rows < 0 || n_cols < 0)
        return ORC_BAD_ARG;
    for (int64_t i = 0; rows && i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= M) return ORC_BAD_ARG;
    for (int64_t j = 0; cols && j < n_cols; ++j)
        if (cols[j] < 0 || cols[j] >= N) return ORC_BAD_ARG;
    if (n_rows == 0 || n_cols == 0)
        return ORC_OK;

    /* Step 1: decode the selected operand rows into K-contiguous fp64 copies,
     * each element multiplied by its block scale (a power of two, so exact). */
    double *a64 = (double *)malloc((size_t)n_rows * (size_t)K * sizeof(double));
    double *b64 = (double *)malloc((size_t)n_cols * (size_t)K * sizeof(double));
    if (!a64 || !b64) {
        free(a64);
        free(b64);
        return ORC_NO_MEM;
    }
    const int64_t KB = V > 0 ? K / V : 0;
    int nt = orc_get_threads();
    (void)nt;
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t m = rows ? rows[i] : i;
        for (int64_t k = 0; k < K; ++k) {
            double v = operand_at(a_dt, a_major, A, M, K, m, k);
            if (V > 0)
                v *= orc_decode_e8m0(SFA[m * KB + k / V]);
            a64[i * K + k] = v;
        }
    }
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t j = 0; j < n_cols; ++j) {
        int64_t n = cols ? cols[j] : j;
        for (int64_t k = 0; k < K; ++k) {
            double v = operand_at(b_dt, b_major, B, N, K, n, k);
            if (V > 0)
                v *= orc_decode_e8m0(SFB[n * KB + k / V]);
            b64[j * K + k] = v;
        }
    }

    /* Step 2: every output is the fp64 sum of its K products, k increasing;
     * then beta*D0 is added. */
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t m = rows ? rows[i] : i;
        const double *ar = a64 + i * K;
        for (int64_t j = 0; j < n_cols; ++j) {
            int64_t n = cols ? cols[j] : j;
            const double *br = b64 + j * K;
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = ar[k] * br[k];
                acc += p;
                mag += fabs(p);
            }
            if (beta == 1) {
                double d0 = (double)D0[m * N + n];
                acc += d0;
            }
            Dref[i * n_cols + j] = acc;
            if (Smag)
                Smag[i * n_cols + j] = mag;
        }
    }
    free(a64);
    free(b64);
    return ORC_OK;
}

/* ---- error-bound helper for the block-scaled GPU path ----------------------
 *
 * Not part of the reference result: D is always the exact orc_gemm above.
 * This function models how gfx950's scaled MFMA (the 8-, 6- and 4-bit
 * block-scaled instructions) sums products, so that the tests can bound the
 * GPU's deviation from the exact D tightly.  The model was established on the
 * GPU with crafted inputs (one large and one small product per output) and is
 * pinned there by a GPU test; it is:
 *
 *   K is cut into groups of GROUP = 8 consecutive elements, starting at k = 0.
 *   In a group, E_max is the largest e(a_k) + e(b_k) over the k whose a_k and
 *   b_k are both nonzero, where e(x) is the exponent of x's bit field:
 *   floor(log2|x|) for a normal value, the format's smallest normal exponent
 *   for a subnormal one.  Every product a_k * b_k of the group is truncated
 *   toward zero to a multiple of 2^(E_max - WINDOW), WINDOW = 13, before the
 *   group's products are added; the scales multiply afterwards (a group lies
 *   inside one scale block).
 *
 * For the selected outputs it returns L[m][n] = sum_k (t_k - p_k) sA sB, the
 * signed change the truncation makes to the exact sum (t_k the truncated
 * product, p_k the exact one, sA, sB the block scales), and
 * Wabs[m][n] = sum_k |t_k - p_k| sA sB.  Arguments as orc_gemm; V > 0 only.
 */
enum { ORC_GROUP = 8, ORC_WINDOW = 13 };

/* Smallest normal exponent of a block-scaled element format. */
static int min_normal_exp(int dt)
{
    switch (dt) {
    case ORC_E4M3: return -6;     /* bias 7 */
    case ORC_E3M2: return -2;     /* bias 3 */
    case ORC_E2M3: return 0;      /* bias 1 */
    case ORC_E2M1: case ORC_E2M1_P64: return 0;   /* bias 1 */
    default: return INT32_MIN;
    }
}

/* e(x) as above; INT32_MIN for zero. */
static int field_exp(int dt, double x)
{
    if (x == 0.0)
        return INT32_MIN;
    int e2;
    (void)frexp(x, &e2);            /* |x| = f * 2^e2, f in [0.5, 1) */
    const int e = e2 - 1;           /* floor(log2 |x|) */
    const int lo = min_normal_exp(dt);
    return e < lo ? lo : e;
}

int orc_mx_group_trunc(int64_t M, int64_t N, int64_t K,
                       int a_dt, int a_major, const void *A,
                       int b_dt, int b_major, const void *B,
                       int32_t V, const uint8_t *SFA, const uint8_t *SFB,
                       int64_t n_rows, const int64_t *rows,
                       int64_t n_cols, const int64_t *cols,
                       double *L, double *Wabs)
{
    if (M <= 0 || N <= 0 || K <= 0 || !A || !B || !L || !Wabs)
        return ORC_BAD_ARG;
    if (min_normal_exp(a_dt) == INT32_MIN || min_normal_exp(b_dt) == INT32_MIN)
        return ORC_BAD_ARG;
    if (V <= 0 || K % V != 0 || V % ORC_GROUP != 0 || !SFA || !SFB)
        return ORC_BAD_ARG;
    if ((a_major != ORC_KMAJOR && a_major != ORC_MNMAJOR) ||
        (b_major != ORC_KMAJOR && b_major != ORC_MNMAJOR))
        return ORC_BAD_ARG;
    if (!rows) n_rows = M;
    if (!cols) n_cols = N;
    if (n_rows < 0 || n_cols < 0)
        return ORC_BAD_ARG;
    for (int64_t i = 0; rows && i < n_rows; ++i)
        if (rows[i] < 0 || rows[i] >= M) return ORC_BAD_ARG;
    for (int64_t j = 0; cols && j < n_cols; ++j)
        if (cols[j] < 0 || cols[j] >= N) return ORC_BAD_ARG;
    if (n_rows == 0 || n_cols == 0)
        return ORC_OK;

    /* unscaled values and their field exponents, K-contiguous */
    double *a64 = (double *)malloc((size_t)n_rows * (size_t)K * sizeof(double));
    double *b64 = (double *)malloc((size_t)n_cols * (size_t)K * sizeof(double));
    int *ea = (int *)malloc((size_t)n_rows * (size_t)K * sizeof(int));
    int *eb = (int *)malloc((size_t)n_cols * (size_t)K * sizeof(int));
    if (!a64 || !b64 || !ea || !eb) {
        free(a64); free(b64); free(ea); free(eb);
        return ORC_NO_MEM;
    }
    const int64_t KB = K / V;
    int nt = orc_get_threads();
    (void)nt;
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t m = rows ? rows[i] : i;
        for (int64_t k = 0; k < K; ++k) {
            double v = operand_at(a_dt, a_major, A, M, K, m, k);
            a64[i * K + k] = v;
            ea[i * K + k] = field_exp(a_dt, v);
        }
    }
#pragma omp parallel for schedule(static) num_threads(nt)
    for (int64_t j = 0; j < n_cols; ++j) {
        int64_t n = cols ? cols[j] : j;
        for (int64_t k = 0; k < K; ++k) {
            double v = operand_at(b_dt, b_major, B, N, K, n, k);
            b64[j * K + k] = v;
            eb[j * K + k] = field_exp(b_dt, v);
        }
    }
#pragma omp parallel for schedule(dynamic, 1) num_threads(nt)
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t m = rows ? rows[i] : i;
        for (int64_t j = 0; j < n_cols; ++j) {
            int64_t n = cols ? cols[j] : j;
            double lsum = 0.0, wsum = 0.0;
            for (int64_t g = 0; g < K; g += ORC_GROUP) {
                int emax = INT32_MIN;
                for (int64_t k = g; k < g + ORC_GROUP; ++k) {
                    const int ka = ea[i * K + k], kb = eb[j * K + k];
                    if (ka != INT32_MIN && kb != INT32_MIN && ka + kb > emax)
                        emax = ka + kb;
                }
                if (emax == INT32_MIN)
                    continue;      /* every product of the group is zero */
                const double lsb = ldexp(1.0, emax - ORC_WINDOW);
                const double s = orc_decode_e8m0(SFA[m * KB + g / V]) * orc_decode_e8m0(SFB[n * KB + g / V]);
                for (int64_t k = g; k < g + ORC_GROUP; ++k) {
                    const double p = a64[i * K + k] * b64[j * K + k];        /* exact */
                    const double t = trunc(p / lsb) * lsb;                   /* exact: lsb is a power of two */
                    lsum += (t - p) * s;
                    wsum += fabs(t - p) * s;
                }
            }
            L[i * n_cols + j] = lsum;
            Wabs[i * n_cols + j] = wsum;
        }
    }
    free(a64); free(b64); free(ea); free(eb);
    return ORC_OK;
}
