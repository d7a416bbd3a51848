/*
 * xq_oracle.c — plain, slow, obviously correct CPU oracle for the quantized
 * decode mat-vec.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the bench's
 * cpu_baseline leg load this library. The HIP library neither links nor
 * includes it, and nothing here comes from the HIP library. It is
 * single-threaded, uses no SIMD intrinsics and is built with
 * -O2 -fno-fast-math -ffp-contract=off, so every float operation below is one
 * IEEE operation with one rounding (the arithmetic rule of "The kernel
 * reference interpreter", section Arithmetic).
 *
 * The XQO_FAULT_* macros plant one known mistake each. They exist only so the
 * tests can build a faulted copy of the oracle and show that its pins catch
 * the mistake (the instrument test of "The kernel reference interpreter",
 * section Testing the instrument). The default build defines none of them.
 *
 * What is computed, and where the pages say so:
 *
 *  q8_K activation block, 320 bytes per 256 activations ("25 — Writing XPU
 *  Kernels", section 25.2, the integer-route bullet; section 25.2.1, the
 *  reading of the q8_K offsets): 256 int8 codes at +0, eight int32 sums of
 *  32 codes at +256, one f32 scale at +288. Bytes 292..319 are not defined by
 *  the pages; the oracle writes zeros there and comparisons skip them.
 *  The quantizer is an encoding, so it is written as its steps: amax, the
 *  scale amax/127 (an f32 division, the scale being an f32), each code the
 *  f32 quotient x/d rounded to nearest with ties to even, then the sums.
 *  Parity unpinned by the pages on two points, both read plainly and pinned
 *  by the tests against closed forms: ties-to-even, and division by d rather
 *  than multiplication by a reciprocal.
 *
 *  Q4_K super-block, 144 bytes per 256 weights: f16 d, f16 dmin, twelve bytes
 *  of packed 6-bit scales and mins, 128 bytes of nibbles with group g at
 *  16 + 32*g ("cajeta.xpu — one kernel, any device", section 2.3, the
 *  load-alignment example). Group g holds sub-block 2g in its low nibbles and
 *  sub-block 2g+1 in its high nibbles, byte t giving weight t of each (the
 *  same low/high split as the IQ4_NL payload of section 25.2.1). The 6-bit
 *  packing is not on the pages; it is the public GGUF Q4_K convention.
 *  Weight i of sub-block j is d*sc_j*q_i - dmin*m_j: the nibble is unsigned
 *  (the unsigned-by-signed dot of section 25.1 and section 25.5) and the min
 *  is an offset paid back through the activation sums (section 25.2.1, the
 *  Q4_0 note that an offset rides on the activation sum).
 *
 *  IQ4_NL resident row (section 25.2.1 and its reading): the row's f16 block
 *  scales, padded to a dword, then one 16-byte payload per 32-weight block.
 *  Byte t of a payload gives weight t (low nibble) and weight t+16 (high
 *  nibble); a nibble selects a signed int8 from the 16-entry codebook; the
 *  weight is d_c * kv[nibble].
 *
 *  The mat-vec: the integer route of section 25.2 computes, up to the order of
 *  rounding, the plain dot of the dequantized weights with the dequantized
 *  activation (xs * code). The oracle is that definition: every weight and
 *  every activation dequantized to double, one double sum per row. The
 *  per-block integer partials are likewise written as their plain sums over
 *  the block's elements.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define Q4K_BYTES 144
#define Q8K_BYTES 320
#define QK 256

/* ---- f16 ---------------------------------------------------------------- */

/* Exact IEEE binary16 -> double, including subnormals, zeros, Inf and NaN. */
double xqo_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int m = h & 1023;
    double v;
    if (e == 0) {
        v = ldexp((double)m, -24);
    } else if (e == 31) {
        v = (m == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + m), e - 25);
    }
    return sign ? -v : v;
}

static uint16_t rd_u16(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

static float rd_f32(const uint8_t *p)
{
    uint32_t u = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) |
                 ((uint32_t)p[3] << 24);
    float v;
    memcpy(&v, &u, 4);
    return v;
}

static void wr_i32(uint8_t *p, int32_t v)
{
    uint32_t u;
    memcpy(&u, &v, 4);
    p[0] = (uint8_t)u; p[1] = (uint8_t)(u >> 8); p[2] = (uint8_t)(u >> 16); p[3] = (uint8_t)(u >> 24);
}

static void wr_f32(uint8_t *p, float v)
{
    uint32_t u;
    memcpy(&u, &v, 4);
    p[0] = (uint8_t)u; p[1] = (uint8_t)(u >> 8); p[2] = (uint8_t)(u >> 16); p[3] = (uint8_t)(u >> 24);
}

/* ---- q8_K --------------------------------------------------------------- */

/* Quantize one block of 256 f32 activations into a 320-byte q8_K block. */
static void quantize_block(const float *x, uint8_t *out)
{
    /* Step 1: the largest magnitude of the block. */
    float amax = 0.0f;
    for (int i = 0; i < QK; i++) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    /* Step 2: the block scale, one f32 division. */
    float d = amax / 127.0f;
    /* Step 3: each code is x/d rounded to nearest (ties to even). An all-zero
     * block has d == 0 and all codes 0. |x/d| <= 127*(1+2^-23), so the clamp
     * never acts; it is kept so the code range is explicit. */
    int8_t q[QK];
    for (int i = 0; i < QK; i++) {
        if (d == 0.0f) {
            q[i] = 0;
        } else {
            float t = x[i] / d;
#ifdef XQO_FAULT_TIES_AWAY
            float r = roundf(t);
#else
            float r = rintf(t);
#endif
            if (r > 127.0f) r = 127.0f;
            if (r < -127.0f) r = -127.0f;
            q[i] = (int8_t)r;
        }
    }
    /* Step 4: the eight sums of 32 consecutive codes. */
    int32_t s[8];
    for (int j = 0; j < 8; j++) {
        int32_t acc = 0;
        for (int t = 0; t < 32; t++) acc += q[32 * j + t];
        s[j] = acc;
    }
    /* Step 5: store codes, sums and scale; zero the undefined tail. */
    memset(out, 0, Q8K_BYTES);
    memcpy(out, q, QK);
    for (int j = 0; j < 8; j++) wr_i32(out + 256 + 4 * j, s[j]);
    wr_f32(out + 288, d);
}

/* x: f32 [rows][K]; out: [rows][K/256] q8_K blocks. */
void xqo_quantize_q8k(const float *x, int64_t rows, int64_t K, uint8_t *out)
{
    int64_t nb = K / QK;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++)
            quantize_block(x + r * K + b * QK, out + (r * nb + b) * Q8K_BYTES);
}

/* Dequantized activation: xs_b * code_i, as double [rows][K]. */
void xqo_dequant_q8k(const uint8_t *xq, int64_t rows, int64_t K, double *out)
{
    int64_t nb = K / QK;
    for (int64_t r = 0; r < rows; r++)
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = xq + (r * nb + b) * Q8K_BYTES;
            double xs = (double)rd_f32(blk + 288);
            for (int i = 0; i < QK; i++)
                out[r * K + b * QK + i] = xs * (double)(int8_t)blk[i];
        }
}

/* ---- Q4_K --------------------------------------------------------------- */

/* The 6-bit scale and min of sub-block j (0..7) from header bytes 4..15. */
void xqo_q4k_scale_min(const uint8_t *blk, int j, int *sc, int *m)
{
    const uint8_t *p = blk + 4;
#ifdef XQO_FAULT_SCALE_HIBITS
    if (j < 8) {
        *sc = p[j % 4] & 63;
        *m = p[j % 4 + 4] & 63;
    } else
#endif
    if (j < 4) {
        *sc = p[j] & 63;
        *m = p[j + 4] & 63;
    } else {
        *sc = (p[j + 4] & 15) | ((p[j - 4] >> 6) << 4);
        *m = (p[j + 4] >> 4) | ((p[j] >> 6) << 4);
    }
}

/* Sub-block index and unsigned 4-bit code of weight i (0..255) of a block. */
static void q4k_code(const uint8_t *blk, int i, int *j, int *q)
{
    int g = i / 64;
    int w = i % 64;
#ifdef XQO_FAULT_NIBBLE_SWAP
    w = (w + 32) % 64;
#endif
    if (w < 32) {
        *j = 2 * g;
        *q = blk[16 + 32 * g + w] & 15;
    } else {
        *j = 2 * g + 1;
        *q = blk[16 + 32 * g + (w - 32)] >> 4;
    }
}

int xqo_q4k_code(const uint8_t *blk, int i)
{
    int j, q;
    q4k_code(blk, i, &j, &q);
    return q;
}

/* Dequantized Q4_K weights, double [N][K]. */
void xqo_dequant_q4k(const uint8_t *w, int64_t N, int64_t K, double *out)
{
    int64_t nb = K / QK;
    for (int64_t r = 0; r < N; r++)
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = w + (r * nb + b) * Q4K_BYTES;
            double d = xqo_f16_to_f64(rd_u16(blk));
            double dmin = xqo_f16_to_f64(rd_u16(blk + 2));
            for (int i = 0; i < QK; i++) {
                int j, q, sc, m;
                q4k_code(blk, i, &j, &q);
                xqo_q4k_scale_min(blk, j, &sc, &m);
                out[r * K + b * QK + i] = d * (double)sc * (double)q - dmin * (double)m;
            }
        }
}

/* Exact per-block integer partials of selected rows (all rows if rows is
 * NULL): S = sum_i sc_j(i)*q_i*code_i and M = sum_i m_j(i)*code_i over the
 * 256 elements of block b, against activation row xrow of xq.
 * S, M: int32 [nrows][K/256]. */
void xqo_q4k_partials(const uint8_t *w, const uint8_t *xq, int64_t N, int64_t K,
                      const int64_t *rows, int64_t nrows, int32_t *S, int32_t *M)
{
    int64_t nb = K / QK;
    if (!rows) nrows = N;
    for (int64_t k = 0; k < nrows; k++) {
        int64_t r = rows ? rows[k] : k;
        for (int64_t b = 0; b < nb; b++) {
            const uint8_t *blk = w + (r * nb + b) * Q4K_BYTES;
            const uint8_t *xb = xq + b * Q8K_BYTES;
            int64_t s = 0, mm = 0;
            for (int i = 0; i < QK; i++) {
                int j, q, sc, m;
                q4k_code(blk, i, &j, &q);
                xqo_q4k_scale_min(blk, j, &sc, &m);
                int code = (int8_t)xb[i];
                s += (int64_t)sc * q * code;
                mm += (int64_t)m * code;
            }
            S[k * nb + b] = (int32_t)s;
            M[k * nb + b] = (int32_t)mm;
        }
    }
}

/* One output of the Q4_K mat-vec by the plain definition, against the q8_K
 * activation row xrow (K/256 blocks). Two magnitude sums come with it:
 *  *Tb, the sum over blocks of the magnitudes of the two terms the integer
 *      route adds per block, |d*xs*S| + |dmin*xs*M|, with S and M the block's
 *      exact integer partials (the sum of |terms| of the f32 bar);
 *  *Te, the sum over elements of |d*sc*q*xhat| + |dmin*m*xhat|.
 * Te >= Tb >= |y| by the triangle inequality. Either may be NULL. */
static void q4k_dot(const uint8_t *wrow, const uint8_t *xrow, int64_t nb, double *y, double *Tb,
                    double *Te)
{
    double acc = 0.0, mag_b = 0.0, mag_e = 0.0;
    for (int64_t b = 0; b < nb; b++) {
        const uint8_t *blk = wrow + b * Q4K_BYTES;
        const uint8_t *xb = xrow + b * Q8K_BYTES;
        double d = xqo_f16_to_f64(rd_u16(blk));
        double dmin = xqo_f16_to_f64(rd_u16(blk + 2));
        double xs = (double)rd_f32(xb + 288);
        int64_t S = 0, M = 0;
#ifdef XQO_FAULT_TB_SUBBLOCK
        double sub_mag = 0.0;
        int64_t S_j = 0, M_j = 0;
#endif
        for (int i = 0; i < QK; i++) {
            int j, q, sc, m;
            q4k_code(blk, i, &j, &q);
            xqo_q4k_scale_min(blk, j, &sc, &m);
            int code = (int8_t)xb[i];
            double xhat = xs * (double)code;
            double wsc = d * (double)sc * (double)q;
            double wmin = dmin * (double)m;
#ifdef XQO_FAULT_MIN_SIGN
            wmin = -wmin;
#endif
            acc += (wsc - wmin) * xhat;
            mag_e += fabs(wsc * xhat) + fabs(wmin * xhat);
#ifdef XQO_FAULT_T_DOUBLE
            mag_e += fabs(wsc * xhat);
#endif
            S += (int64_t)sc * q * code;
            M += (int64_t)m * code;
#ifdef XQO_FAULT_TB_SUBBLOCK
            S_j += (int64_t)sc * q * code;
            M_j += (int64_t)m * code;
            if (i % 32 == 31) {
                sub_mag += fabs(d * xs * (double)S_j) + fabs(dmin * xs * (double)M_j);
                S_j = 0;
                M_j = 0;
            }
#endif
        }
#ifdef XQO_FAULT_TB_SUBBLOCK
        mag_b += sub_mag;
#else
        mag_b += fabs(d * xs * (double)S) + fabs(dmin * xs * (double)M);
#endif
    }
    *y = acc;
    if (Tb) *Tb = mag_b;
    if (Te) *Te = mag_e;
}

/* y = W * xhat for selected rows (all if rows is NULL); xq holds one q8_K
 * activation row. y, Tb, Te: double [nrows] (Tb, Te may be NULL). */
void xqo_gemv_q4k(const uint8_t *w, const uint8_t *xq, int64_t N, int64_t K,
                  const int64_t *rows, int64_t nrows, double *y, double *Tb, double *Te)
{
    int64_t nb = K / QK;
    if (!rows) nrows = N;
    for (int64_t k = 0; k < nrows; k++) {
        int64_t r = rows ? rows[k] : k;
        q4k_dot(w + r * nb * Q4K_BYTES, xq, nb, &y[k], Tb ? &Tb[k] : NULL, Te ? &Te[k] : NULL);
    }
}

/* Y[m][n] = sum_i W[n][i] * xhat[m][i] for the listed (m, n) pairs (all
 * M*N pairs in row-major order if ms is NULL). y, Tb, Te: double [count]
 * (Tb, Te may be NULL). */
void xqo_gemm_q4k(const uint8_t *w, const uint8_t *xq, int64_t Mrows, int64_t N, int64_t K,
                  const int64_t *ms, const int64_t *ns, int64_t count, double *y, double *Tb,
                  double *Te)
{
    int64_t nb = K / QK;
    if (!ms) count = Mrows * N;
    for (int64_t k = 0; k < count; k++) {
        int64_t m = ms ? ms[k] : k / N;
        int64_t n = ms ? ns[k] : k % N;
        q4k_dot(w + n * nb * Q4K_BYTES, xq + m * nb * Q8K_BYTES, nb, &y[k], Tb ? &Tb[k] : NULL,
                Te ? &Te[k] : NULL);
    }
}

/* ---- IQ4_NL ------------------------------------------------------------- */

static const int8_t IQ4NL_KV[16] = {-127, -104, -83, -65, -49, -35, -22, -10,
                                    1,    13,   25,  38,  53,  69,  89,  113};

int xqo_iq4nl_codebook(int nibble) { return IQ4NL_KV[nibble & 15]; }

static void iq4nl_geometry(int64_t K, int64_t *bpr, int64_t *prefix, int64_t *row_bytes)
{
    *bpr = K / 32;
    *prefix = ((*bpr * 2 + 3) / 4) * 4;
    *row_bytes = *prefix + 16 * *bpr;
}

/* Nibble of weight t (0..31) of a 16-byte payload. */
static int iq4nl_nibble(const uint8_t *payload, int t)
{
#ifdef XQO_FAULT_IQ4_HALVES
    return (t < 16) ? (payload[t] >> 4) : (payload[t - 16] & 15);
#else
    return (t < 16) ? (payload[t] & 15) : (payload[t - 16] >> 4);
#endif
}

void xqo_dequant_iq4nl(const uint8_t *w, int64_t N, int64_t K, double *out)
{
    int64_t bpr, prefix, row_bytes;
    iq4nl_geometry(K, &bpr, &prefix, &row_bytes);
    for (int64_t r = 0; r < N; r++) {
        const uint8_t *row = w + r * row_bytes;
        for (int64_t c = 0; c < bpr; c++) {
            double d = xqo_f16_to_f64(rd_u16(row + 2 * c));
            const uint8_t *pay = row + prefix + 16 * c;
            for (int t = 0; t < 32; t++)
                out[r * K + 32 * c + t] = d * (double)IQ4NL_KV[iq4nl_nibble(pay, t)];
        }
    }
}

/* D[r][c] = sum_t kv[nibble_t] * code_(32c+t): int32 [nrows][K/32]. */
void xqo_iq4nl_partials(const uint8_t *w, const uint8_t *xq, int64_t N, int64_t K,
                        const int64_t *rows, int64_t nrows, int32_t *D)
{
    int64_t bpr, prefix, row_bytes;
    iq4nl_geometry(K, &bpr, &prefix, &row_bytes);
    if (!rows) nrows = N;
    for (int64_t k = 0; k < nrows; k++) {
        int64_t r = rows ? rows[k] : k;
        const uint8_t *row = w + r * row_bytes;
        for (int64_t c = 0; c < bpr; c++) {
            const uint8_t *pay = row + prefix + 16 * c;
            int64_t acc = 0;
            for (int t = 0; t < 32; t++) {
                int64_t i = 32 * c + t;
                int code = (int8_t)xq[(i / QK) * Q8K_BYTES + (i % QK)];
                acc += (int64_t)IQ4NL_KV[iq4nl_nibble(pay, t)] * code;
            }
            D[k * bpr + c] = (int32_t)acc;
        }
    }
}

/* y = W * xhat for selected rows (all if rows is NULL). Tb is the sum over
 * 32-blocks of |d_c*xs*D_c|, D_c the block's exact integer partial (the sum of
 * |terms| of the f32 bar); Te the sum over elements of |d_c*kv*xhat|. y, Tb,
 * Te: double [nrows] (Tb, Te may be NULL). */
void xqo_gemv_iq4nl(const uint8_t *w, const uint8_t *xq, int64_t N, int64_t K,
                    const int64_t *rows, int64_t nrows, double *y, double *Tb, double *Te)
{
    int64_t bpr, prefix, row_bytes;
    iq4nl_geometry(K, &bpr, &prefix, &row_bytes);
    if (!rows) nrows = N;
    for (int64_t k = 0; k < nrows; k++) {
        int64_t r = rows ? rows[k] : k;
        const uint8_t *row = w + r * row_bytes;
        double acc = 0.0, mag_b = 0.0, mag_e = 0.0;
        for (int64_t c = 0; c < bpr; c++) {
            double d = xqo_f16_to_f64(rd_u16(row + 2 * c));
            const uint8_t *pay = row + prefix + 16 * c;
            const uint8_t *xb = xq + ((32 * c) / QK) * Q8K_BYTES;
            double xs = (double)rd_f32(xb + 288);
            int64_t D = 0;
            for (int t = 0; t < 32; t++) {
                int64_t i = 32 * c + t;
                int code = (int8_t)xb[i % QK];
                int kv = IQ4NL_KV[iq4nl_nibble(pay, t)];
                double term = d * (double)kv * (xs * (double)code);
                acc += term;
                mag_e += fabs(term);
                D += (int64_t)kv * code;
            }
#ifdef XQO_FAULT_TB_IQ4_ELEM
            (void)D;
            mag_b = mag_e;
#else
            mag_b += fabs(d * xs * (double)D);
#endif
        }
        y[k] = acc;
        if (Tb) Tb[k] = mag_b;
        if (Te) Te[k] = mag_e;
    }
}

/* ---- Q4_0 ---------------------------------------------------------------- */
/* Q4_0 shares the IQ4_NL block shape and resident row (f16 scale per 32
 * weights, 16 payload bytes: byte t holds weight t in its low nibble and weight
 * t+16 in its high nibble); the weight is d * (nibble - 8) ("25 — Writing XPU
 * Kernels", section 25.2: the Q4_0 twin of the IQ4_NL kernel, whose -8 rides on
 * the activation's sum). */

static int q4_0_value(int nibble)
{
#ifdef XQO_FAULT_Q40_OFFSET
    return nibble - 7;
#else
    return nibble - 8;
#endif
}

void xqo_dequant_q4_0(const uint8_t *w, int64_t N, int64_t K, double *out)
{
    int64_t bpr, prefix, row_bytes;
    iq4nl_geometry(K, &bpr, &prefix, &row_bytes);
    for (int64_t r = 0; r < N; r++) {
        const uint8_t *row = w + r * row_bytes;
        for (int64_t c = 0; c < bpr; c++) {
            double d = xqo_f16_to_f64(rd_u16(row + 2 * c));
            const uint8_t *pay = row + prefix + 16 * c;
            for (int t = 0; t < 32; t++)
                out[r * K + 32 * c + t] = d * (double)q4_0_value(iq4nl_nibble(pay, t));
        }
    }
}

/* D[r][c] = sum_t (nibble_t - 8) * code_(32c+t): int32 [nrows][K/32]. */
void xqo_q4_0_partials(const uint8_t *w, const uint8_t *xq, int64_t N, int64_t K,
                       const int64_t *rows, int64_t nrows, int32_t *D)
{
    int64_t bpr, prefix, row_bytes;
    iq4nl_geometry(K, &bpr, &prefix, &row_bytes);
    if (!rows) nrows = N;
    for (int64_t k = 0; k < nrows; k++) {
        int64_t r = rows ? rows[k] : k;
        const uint8_t *row = w + r * row_bytes;
        for (int64_t c = 0; c < bpr; c++) {
            const uint8_t *pay = row + prefix + 16 * c;
            int64_t acc = 0;
            for (int t = 0; t < 32; t++) {
                int64_t i = 32 * c + t;
                int code = (int8_t)xq[(i / QK) * Q8K_BYTES + (i % QK)];
                acc += (int64_t)q4_0_value(iq4nl_nibble(pay, t)) * code;
            }
            D[k * bpr + c] = (int32_t)acc;
        }
    }
}

/* As xqo_gemv_iq4nl, with weight d_c*(nibble-8) and D_c = sum (nibble-8)*code. */
void xqo_gemv_q4_0(const uint8_t *w, const uint8_t *xq, int64_t N, int64_t K,
                   const int64_t *rows, int64_t nrows, double *y, double *Tb, double *Te)
{
    int64_t bpr, prefix, row_bytes;
    iq4nl_geometry(K, &bpr, &prefix, &row_bytes);
    if (!rows) nrows = N;
    for (int64_t k = 0; k < nrows; k++) {
        int64_t r = rows ? rows[k] : k;
        const uint8_t *row = w + r * row_bytes;
        double acc = 0.0, mag_b = 0.0, mag_e = 0.0;
        for (int64_t c = 0; c < bpr; c++) {
            double d = xqo_f16_to_f64(rd_u16(row + 2 * c));
            const uint8_t *pay = row + prefix + 16 * c;
            const uint8_t *xb = xq + ((32 * c) / QK) * Q8K_BYTES;
            double xs = (double)rd_f32(xb + 288);
            int64_t D = 0;
            for (int t = 0; t < 32; t++) {
                int64_t i = 32 * c + t;
                int code = (int8_t)xb[i % QK];
                int v = q4_0_value(iq4nl_nibble(pay, t));
                double term = d * (double)v * (xs * (double)code);
                acc += term;
                mag_e += fabs(term);
                D += (int64_t)v * code;
            }
            mag_b += fabs(d * xs * (double)D);
        }
        y[k] = acc;
        if (Tb) Tb[k] = mag_b;
        if (Te) Te[k] = mag_e;
    }
}
