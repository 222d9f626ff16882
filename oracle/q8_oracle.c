/*
 * Q8_0 qdot oracle -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU statement of what the Q8_0 block
 * contraction computes.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load this file's library.  The GPU
 * product never links, loads or calls it, and this file includes no GPU
 * header and shares no code with the GPU path.
 *
 * Sources (Phobos documentation pages):
 *   - "Phobos Language Spec", section "Quantized built-ins", Q8_0 table,
 *     row qdot_t: out[i,j] = sum over 32-wide blocks b of
 *     a_scales[i,b] * w_scales[j,b] * (sum over k in b of a[i,k] * w[j,k]);
 *     scales are [M, K/32] and [N, K/32].
 *   - the same table, row qmma_t: the same sum, with w_scales stored
 *     transposed, [K/32, N] (w_scales[b][j]).
 *   - the same table, rows q50_qdot_t / q50_qmma_t: the weight is Q5_0
 *     blocks without their f16 scale, 20 bytes per 32 values: the qh word,
 *     then 16 bytes, byte e holding element e (low nibble) and element
 *     e + 16 (high nibble); each element is q - 16.
 *   - "Quantized built-ins and formats", section "Q8_0": signed bytes with
 *     one scale per block of 32 values; activations are quantized the same
 *     way; the inner sum is taken in integers (four bytes at a time with
 *     dp4a on the pages' hardware).
 *   - "Phobos Language Spec", section "Types": i8 loads sign-extend.
 *
 * Readings where the pages are silent:
 *   - The quantizer (the pages never say how Q8_0 values are produced):
 *     per 32-block, amax = max |x|, d = f32(amax / 127),
 *     q = clamp(round-half-even(x / d), -127, 127) computed in f32, and
 *     d == 0 gives q == 0.  Ties-to-even matches the spec's round()
 *     ("Phobos Language Spec", section "Elementwise").
 *   - Accumulation across blocks is done here in f64, in block order;
 *     AS*WS is exact in f64 (24 + 24 mantissa bits).
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -shared -fPIC.
 * No -ffast-math and no -march: the f32 quantizer must use IEEE division
 * and round-to-nearest-even exactly as written.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define Q8_BLOCK 32

/* Number of threads the OpenMP loops below use (1 without OpenMP). */
int q8o_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the number of threads for later calls (no effect without OpenMP). */
void q8o_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/*
 * Q8_0 quantization of `rows` f32 rows of length K (K >= 0, a multiple of 32).
 * q: int8 [rows][K]; d: f32 [rows][K/32].  Returns 0, or -1 for a bad K.
 */
int q8o_quantize_rows(const float *x, int64_t rows, int64_t K,
                      int8_t *q, float *d) {
    if (K < 0 || K % Q8_BLOCK != 0 || rows < 0) return -1;
    const int64_t KB = K / Q8_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < KB; ++b) {
            const float *xb = x + r * K + b * Q8_BLOCK;
            int8_t *qb = q + r * K + b * Q8_BLOCK;
            float amax = 0.0f;
            for (int t = 0; t < Q8_BLOCK; ++t) {
                float a = fabsf(xb[t]);
                if (a > amax) amax = a;
            }
            float scale = amax / 127.0f; /* one f32 division, rounded to nearest */
            d[r * KB + b] = scale;
            for (int t = 0; t < Q8_BLOCK; ++t) {
                if (scale == 0.0f) {
                    qb[t] = 0;
                    continue;
                }
                float v = rintf(xb[t] / scale); /* f32 division, then ties-to-even */
                if (v > 127.0f) v = 127.0f;
                if (v < -127.0f) v = -127.0f;
                qb[t] = (int8_t)v;
            }
        }
    }
    return 0;
}

/* One block's integer dot: sum over t < 32 of i32(a[t]) * i32(w[t]). */
static int32_t block_dot(const int8_t *a, const int8_t *w) {
    int32_t s = 0;
    for (int t = 0; t < Q8_BLOCK; ++t) s += (int32_t)a[t] * (int32_t)w[t];
    return s;
}

/*
 * Per-block integer partials P[i][j][b] (int32, row-major [M][N][K/32]).
 * K == 0 (no blocks) is accepted throughout: the sums over b are empty.
 * |P| <= 32 * 128 * 128 = 2^19, so int32 is exact.
 */
int q8o_block_partials(const int8_t *A, const int8_t *W, int32_t *P,
                       int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0 || K % Q8_BLOCK != 0) return -1;
    const int64_t KB = K / Q8_BLOCK;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            for (int64_t b = 0; b < KB; ++b)
                P[(i * N + j) * KB + b] =
                    block_dot(A + i * K + b * Q8_BLOCK, W + j * K + b * Q8_BLOCK);
    return 0;
}

/* One output: the definition in f64, plus the sum of |terms|. */
static void qdot_one(const int8_t *A, const float *AS, const int8_t *W,
                     const float *WS, int64_t i, int64_t j, int64_t K,
                     double *out, double *abs_terms) {
    const int64_t KB = K / Q8_BLOCK;
    double acc = 0.0, mag = 0.0;
    for (int64_t b = 0; b < KB; ++b) {
        int32_t p = block_dot(A + i * K + b * Q8_BLOCK, W + j * K + b * Q8_BLOCK);
        double s = (double)AS[i * KB + b] * (double)WS[j * KB + b]; /* exact */
        double term = s * (double)p;
        acc += term;
        mag += fabs(term);
    }
    *out = acc;
    *abs_terms = mag;
}

/*
 * out[i][j] = sum_b AS[i,b] * WS[j,b] * P[i,j,b] in f64, in block order;
 * abs_terms[i][j] = sum_b |AS[i,b] * WS[j,b] * P[i,j,b]|.
 * A int8 [M][K], AS f32 [M][K/32], W int8 [N][K], WS f32 [N][K/32].
 */
int q8o_qdot_f64(const int8_t *A, const float *AS, const int8_t *W,
                 const float *WS, int64_t M, int64_t N, int64_t K,
                 double *out, double *abs_terms) {
    if (M < 0 || N < 0 || K < 0 || K % Q8_BLOCK != 0) return -1;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            qdot_one(A, AS, W, WS, i, j, K, out + i * N + j, abs_terms + i * N + j);
    return 0;
}

/*
 * The same definition at `count` sampled output positions (ii[s], jj[s]),
 * for checks at sizes where the whole output would be too slow here.
 */
int q8o_qdot_f64_at(const int8_t *A, const float *AS, const int8_t *W,
                    const float *WS, int64_t M, int64_t N, int64_t K,
                    const int64_t *ii, const int64_t *jj, int64_t count,
                    double *out, double *abs_terms) {
    if (M < 0 || N < 0 || K < 0 || K % Q8_BLOCK != 0 || count < 0) return -1;
    for (int64_t s = 0; s < count; ++s)
        if (ii[s] < 0 || ii[s] >= M || jj[s] < 0 || jj[s] >= N) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < count; ++s)
        qdot_one(A, AS, W, WS, ii[s], jj[s], K, out + s, abs_terms + s);
    return 0;
}

/* Partials P[s][b] for sampled (ii[s], jj[s]) positions: int32 [count][K/32]. */
int q8o_block_partials_at(const int8_t *A, const int8_t *W, int64_t M, int64_t N,
                          int64_t K, const int64_t *ii, const int64_t *jj,
                          int64_t count, int32_t *P) {
    if (M < 0 || N < 0 || K < 0 || K % Q8_BLOCK != 0 || count < 0) return -1;
    for (int64_t s = 0; s < count; ++s)
        if (ii[s] < 0 || ii[s] >= M || jj[s] < 0 || jj[s] >= N) return -2;
    const int64_t KB = K / Q8_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < count; ++s)
        for (int64_t b = 0; b < KB; ++b)
            P[s * KB + b] = block_dot(A + ii[s] * K + b * Q8_BLOCK,
                                      W + jj[s] * K + b * Q8_BLOCK);
    return 0;
}

/* One output of the qmma_t form: weight scales WST[b][j], f32 [K/32][N]. */
static void qmma_one(const int8_t *A, const float *AS, const int8_t *W,
                     const float *WST, int64_t i, int64_t j, int64_t N, int64_t K,
                     double *out, double *abs_terms) {
    const int64_t KB = K / Q8_BLOCK;
    double acc = 0.0, mag = 0.0;
    for (int64_t b = 0; b < KB; ++b) {
        int32_t p = block_dot(A + i * K + b * Q8_BLOCK, W + j * K + b * Q8_BLOCK);
        double s = (double)AS[i * KB + b] * (double)WST[b * N + j]; /* exact */
        double term = s * (double)p;
        acc += term;
        mag += fabs(term);
    }
    *out = acc;
    *abs_terms = mag;
}

/*
 * qmma_t in f64: out[i][j] = sum_b AS[i,b] * WST[b,j] * P[i,j,b], in block
 * order, and abs_terms as for q8o_qdot_f64.  WST f32 [K/32][N].
 */
int q8o_qmma_f64(const int8_t *A, const float *AS, const int8_t *W,
                 const float *WST, int64_t M, int64_t N, int64_t K,
                 double *out, double *abs_terms) {
    if (M < 0 || N < 0 || K < 0 || K % Q8_BLOCK != 0) return -1;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            qmma_one(A, AS, W, WST, i, j, N, K, out + i * N + j, abs_terms + i * N + j);
    return 0;
}

/* qmma_t at `count` sampled output positions (ii[s], jj[s]). */
int q8o_qmma_f64_at(const int8_t *A, const float *AS, const int8_t *W,
                    const float *WST, int64_t M, int64_t N, int64_t K,
                    const int64_t *ii, const int64_t *jj, int64_t count,
                    double *out, double *abs_terms) {
    if (M < 0 || N < 0 || K < 0 || K % Q8_BLOCK != 0 || count < 0) return -1;
    for (int64_t s = 0; s < count; ++s)
        if (ii[s] < 0 || ii[s] >= M || jj[s] < 0 || jj[s] >= N) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < count; ++s)
        qmma_one(A, AS, W, WST, ii[s], jj[s], N, K, out + s, abs_terms + s);
    return 0;
}

/*
 * Q5_0 weight blocks (the q50_qdot_t / q50_qmma_t rows of the Q8_0 table).
 * Block b of weight row j is the 20 bytes at W5 + (j * K/32 + b) * 20: the
 * qh word (bytes 0..3, little-endian), then bytes 4..19.  Element e < 16 is
 * the low nibble of byte 4 + e, element e + 16 its high nibble; bit e of qh
 * is bit 4 of element e's 5-bit number q (reading: the pages name "the qh
 * word" without a bit order; this is bit e of the little-endian word).  The
 * element's value is q - 16, in [-16, 15].
 */
static int32_t q50_value(const uint8_t *blk, int e) {
    const uint32_t qh = (uint32_t)blk[0] | ((uint32_t)blk[1] << 8) |
                        ((uint32_t)blk[2] << 16) | ((uint32_t)blk[3] << 24);
    const uint8_t byte = blk[4 + (e % 16)];
    const uint32_t nib = e < 16 ? (byte & 0x0Fu) : (byte >> 4);
    const uint32_t q = nib | (((qh >> e) & 1u) << 4);
    return (int32_t)q - 16;
}

static int32_t q50_block_dot(const int8_t *a, const uint8_t *blk) {
    int32_t s = 0;
    for (int e = 0; e < Q8_BLOCK; ++e) s += (int32_t)a[e] * q50_value(blk, e);
    return s;
}

/* Decoded Q5_0 values: Wd int8 [N][K] (each in [-16, 15]). */
int q8o_q50_decode(const uint8_t *W5, int8_t *Wd, int64_t N, int64_t K) {
    if (N < 0 || K < 0 || K % Q8_BLOCK != 0) return -1;
    const int64_t KB = K / Q8_BLOCK;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < N; ++j)
        for (int64_t b = 0; b < KB; ++b)
            for (int e = 0; e < Q8_BLOCK; ++e)
                Wd[j * K + b * Q8_BLOCK + e] = (int8_t)q50_value(W5 + (j * KB + b) * 20, e);
    return 0;
}

/* Per-block integer partials against Q5_0 weights: int32 [M][N][K/32]. */
int q8o_q50_block_partials(const int8_t *A, const uint8_t *W5, int32_t *P,
                           int64_t M, int64_t N, int64_t K) {
    if (M < 0 || N < 0 || K < 0 || K % Q8_BLOCK != 0) return -1;
    const int64_t KB = K / Q8_BLOCK;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            for (int64_t b = 0; b < KB; ++b)
                P[(i * N + j) * KB + b] =
                    q50_block_dot(A + i * K + b * Q8_BLOCK, W5 + (j * KB + b) * 20);
    return 0;
}

/* One output against Q5_0 weights; ws_t: scales [K/32][N] (q50_qmma_t). */
static void q50_one(const int8_t *A, const float *AS, const uint8_t *W5,
                    const float *WS, int ws_t, int64_t i, int64_t j, int64_t N,
                    int64_t K, double *out, double *abs_terms) {
    const int64_t KB = K / Q8_BLOCK;
    double acc = 0.0, mag = 0.0;
    for (int64_t b = 0; b < KB; ++b) {
        int32_t p = q50_block_dot(A + i * K + b * Q8_BLOCK, W5 + (j * KB + b) * 20);
        double ws = ws_t ? (double)WS[b * N + j] : (double)WS[j * KB + b];
        double term = (double)AS[i * KB + b] * ws * (double)p; /* AS*WS exact */
        acc += term;
        mag += fabs(term);
    }
    *out = acc;
    *abs_terms = mag;
}

/* q50_qdot_t (ws_t == 0, WS [N][K/32]) or q50_qmma_t (ws_t != 0, WS [K/32][N]) in f64. */
int q8o_q50_f64(const int8_t *A, const float *AS, const uint8_t *W5, const float *WS,
                int ws_t, int64_t M, int64_t N, int64_t K, double *out, double *abs_terms) {
    if (M < 0 || N < 0 || K < 0 || K % Q8_BLOCK != 0) return -1;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            q50_one(A, AS, W5, WS, ws_t, i, j, N, K, out + i * N + j, abs_terms + i * N + j);
    return 0;
}

/* The same at `count` sampled output positions (ii[s], jj[s]). */
int q8o_q50_f64_at(const int8_t *A, const float *AS, const uint8_t *W5, const float *WS,
                   int ws_t, int64_t M, int64_t N, int64_t K, const int64_t *ii,
                   const int64_t *jj, int64_t count, double *out, double *abs_terms) {
    if (M < 0 || N < 0 || K < 0 || K % Q8_BLOCK != 0 || count < 0) return -1;
    for (int64_t s = 0; s < count; ++s)
        if (ii[s] < 0 || ii[s] >= M || jj[s] < 0 || jj[s] >= N) return -2;
#pragma omp parallel for schedule(static)
    for (int64_t s = 0; s < count; ++s)
        q50_one(A, AS, W5, WS, ws_t, ii[s], jj[s], N, K, out + s, abs_terms + s);
    return 0;
}
