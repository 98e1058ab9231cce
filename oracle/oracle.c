/*
 * oracle.c - TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously correct CPU statement of what the ternary bit-plane GEMV
 * computes. Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library. The GPU library shares no code, header, table or helper
 * with it, and this file includes nothing from the GPU library.
 *
 * Sources (cited by page title and section):
 *   [TP] "Tritium: One Weight Format for Ternary Inference on Commodity CPUs and
 *        Multiplier-Free Hardware" - sections "Background / The model", "The .trit v1
 *        layout" (Equations 2-3 in the introduction), "Invariants", "On popcount",
 *        "The hardware core", "Verification", "Numerics" (the Reference, Folded and IntMlp
 *        modes around the matvec).
 *   [BC] "BITCOS: Intel's Ternary LLM Weight Format Goes Below 1.58 Bits" - "A bitmap and a sign".
 *   [TF] "The .trit format, version 1" - section 1 "Why bit planes", 2.3 "Ternary
 *        payload", 2.4 "Dense payload", 3 "A complete file", 4 "Validation".
 *
 * Readings where the pages leave a step open (each is also listed in the design notes):
 *   - Activation dequantisation: an int8 code q stands for x_scale * q (absmax), and the
 *     weight for w_scale * trit ([TF] 2.3). The fp32 output multiplies the exact integer
 *     sum by each scale in turn, ((float)acc * x_scale) * w_scale, the order [TP]
 *     "Why exactness, concretely" says the reference uses. A float64 value of the same
 *     product is returned beside it.
 *   - When several beats break an invariant, the first in row-major order is reported,
 *     at its lowest offending bit; within one beat P1 is checked before P2.
 *   - The dense head is y = W x over bfloat16 inputs; the oracle accumulates in float64
 *     and also returns sum |w * x| for the tolerance.
 *   - BITCOS row form: the page fixes the two arrays (presence, compacted signs) but not how a
 *     kernel blocks them; here each row's signs start on a 32-bit word, found through a per-row
 *     word index (oracle_bitcos_pack_rows).
 *   - IntMlp: gate and up share the activation (and so its scale); K = S_g^2 S_u is one
 *     float64 number, (S_g * S_g) * S_u with S = (double)x_scale * (double)w_scale.
 *
 * Parity pins live in the test suite (worked example bytes of [TF] section 3, brute force
 * against a dense integer product, closed-form invariants, the -128 extremes case).
 */
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

enum {
    OR_OK = 0,
    OR_E_INVAL = 1, /* bad argument or a weight value outside {-1, 0, +1} */
    OR_E_SIZE = 2,  /* byte length does not match rows * beats_per_row * 16 */
    OR_E_P1 = 3,    /* pos & neg != 0 in some beat */
    OR_E_P2 = 4,    /* a padding bit is set in some row's last beat */
    OR_E_RANGE = 5  /* an accumulator left the int32 range (cannot happen for valid input) */
};

typedef struct {
    int32_t code;
    int64_t row, beat, col;
} or_err;

static int set_err(or_err *e, int code, int64_t row, int64_t beat, int64_t col) {
    if (e) {
        e->code = code;
        e->row = row;
        e->beat = beat;
        e->col = col;
    }
    return code;
}

/* [TF] 2.3: beats_per_row = ceil(cols / 64). */
int64_t oracle_beats_per_row(int64_t cols) { return cols / 64 + (cols % 64 != 0); }

/* [TF] 2.3: byte_len = rows * beats_per_row * 16; -1 for a negative shape or one whose byte count
 * does not fit in int64 (no buffer has that length). */
int64_t oracle_byte_len(int64_t rows, int64_t cols) {
    if (rows < 0 || cols < 0) return -1;
    int64_t bpr = oracle_beats_per_row(cols);
    if (bpr && rows > INT64_MAX / 16 / bpr) return -1;
    return rows * bpr * 16;
}

/* [TF] 2.3 / [TP] "Invariants" (P2): the valid-column mask of a row's last beat, built in 64 bits. */
uint64_t oracle_tail_mask(int64_t cols) {
    int64_t r = cols % 64;
    if (r == 0) return UINT64_MAX;
    return (UINT64_C(1) << r) - UINT64_C(1);
}

/* All integers are little-endian ([TF] section 2): assemble byte by byte, host order independent. */
static uint64_t load_le64(const uint8_t *p) {
    uint64_t v = 0;
    for (int j = 0; j < 8; ++j) v |= (uint64_t)p[j] << (8 * j);
    return v;
}

static void store_le64(uint8_t *p, uint64_t v) {
    for (int j = 0; j < 8; ++j) p[j] = (uint8_t)(v >> (8 * j));
}

static int lowest_bit(uint64_t v) {
    int k = 0;
    while (!((v >> k) & 1)) ++k;
    return k;
}

/*
 * [TF] 2.3 "Ternary payload": beat b of row r is 16 bytes at (r * bpr + b) * 16;
 * bytes 0..8 hold pos (bit k set => W[r][64b + k] = +1), bytes 8..16 hold neg
 * (bit k set => W[r][64b + k] = -1). Neither bit => 0. Bits past cols stay clear.
 */
int oracle_pack(const int8_t *w, int64_t rows, int64_t cols, uint8_t *planes, int64_t len, or_err *e) {
    if (rows < 0 || cols < 0) return set_err(e, OR_E_INVAL, -1, -1, -1);
    int64_t bpr = oracle_beats_per_row(cols);
    if (len != oracle_byte_len(rows, cols)) return set_err(e, OR_E_SIZE, -1, -1, -1);
    /* Rows are independent; each records its first bad column, and the first bad row wins. */
    int64_t first_bad_row = rows, first_bad_col = -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t bad = -1;
        for (int64_t b = 0; b < bpr && bad < 0; ++b) {
            uint64_t pos = 0, neg = 0;
            for (int k = 0; k < 64; ++k) {
                int64_t c = 64 * b + k;
                if (c >= cols) break;
                int8_t v = w[r * cols + c];
                if (v == 1)
                    pos |= UINT64_C(1) << k;
                else if (v == -1)
                    neg |= UINT64_C(1) << k;
                else if (v != 0) {
                    bad = c;
                    break;
                }
            }
            uint8_t *beat = planes + (r * bpr + b) * 16;
            store_le64(beat, pos);
            store_le64(beat + 8, neg);
        }
        if (bad >= 0) {
#pragma omp critical
            if (r < first_bad_row) {
                first_bad_row = r;
                first_bad_col = bad;
            }
        }
    }
    if (first_bad_row < rows) return set_err(e, OR_E_INVAL, first_bad_row, first_bad_col / 64, first_bad_col);
    return set_err(e, OR_OK, -1, -1, -1);
}

/*
 * [TF] section 4, checks 15, 17 and 18; [TP] "Invariants":
 *   length: len == rows * bpr * 16;
 *   P1: pos & neg == 0 in every beat (reported with row, beat and column);
 *   P2: (pos | neg) & ~tail == 0 in every row's last beat (reported with the row).
 */
int oracle_validate(const uint8_t *planes, int64_t len, int64_t rows, int64_t cols, or_err *e) {
    if (rows < 0 || cols < 0) return set_err(e, OR_E_INVAL, -1, -1, -1);
    int64_t bpr = oracle_beats_per_row(cols);
    if (len != oracle_byte_len(rows, cols)) return set_err(e, OR_E_SIZE, -1, -1, -1);
    uint64_t tail = oracle_tail_mask(cols);
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < bpr; ++b) {
            const uint8_t *beat = planes + (r * bpr + b) * 16;
            uint64_t pos = load_le64(beat), neg = load_le64(beat + 8);
            if (pos & neg) return set_err(e, OR_E_P1, r, b, 64 * b + lowest_bit(pos & neg));
            if (b == bpr - 1 && ((pos | neg) & ~tail))
                return set_err(e, OR_E_P2, r, b, 64 * b + lowest_bit((pos | neg) & ~tail));
        }
    }
    return set_err(e, OR_OK, -1, -1, -1);
}

/* The trit of one weight, read from its beat's two planes ([TF] 2.3). */
static int oracle_trit(const uint8_t *planes, int64_t bpr, int64_t r, int64_t c) {
    const uint8_t *beat = planes + (r * bpr + c / 64) * 16;
    int k = (int)(c % 64);
    int p = (int)((load_le64(beat) >> k) & 1);
    int n = (int)((load_le64(beat + 8) >> k) & 1);
    return p - n;
}

/* Expand validated planes to one int8 per weight (the inverse of oracle_pack). */
int oracle_unpack(const uint8_t *planes, int64_t len, int64_t rows, int64_t cols, int8_t *w, or_err *e) {
    int rc = oracle_validate(planes, len, rows, cols, e);
    if (rc) return rc;
    int64_t bpr = oracle_beats_per_row(cols);
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) w[r * cols + c] = (int8_t)oracle_trit(planes, bpr, r, c);
    return OR_OK;
}

/*
 * The exact sum of one row: acc = sum_c W[r][c] * x[c] with W decoded one weight at a
 * time and x sign-extended before it takes part ([TP] introduction, Equations 2-3;
 * "The hardware core": -128 is widened, never negated in eight bits).
 * Returns 0 and stores acc, or OR_E_RANGE if the sum leaves int32 (impossible:
 * |acc| <= 128 * cols).
 */
static int oracle_row_sum(const uint8_t *planes, int64_t bpr, int64_t r, int64_t cols, const int8_t *x,
                          int32_t *acc_out) {
    int64_t acc = 0;
    for (int64_t c = 0; c < cols; ++c) {
        int64_t w = oracle_trit(planes, bpr, r, c);
        int64_t xv = (int64_t)x[c];
        acc += w * xv;
    }
    if (acc < INT32_MIN || acc > INT32_MAX) return OR_E_RANGE;
    *acc_out = (int32_t)acc;
    return OR_OK;
}

/* Dequantised output of one row: each scale applied in turn in fp32, plus the float64 product. */
static void oracle_dequant(int32_t acc, float x_scale, float w_scale, float *y32, double *y64) {
    float a = (float)acc; /* exact: |acc| < 2^24 */
    float t = a * x_scale;
    *y32 = t * w_scale;
    *y64 = (double)acc * (double)x_scale * (double)w_scale;
}

/*
 * Batch-1 ternary GEMV: out_i32[r] = sum_c W[r][c] x[c]; out_f32 / out_f64 the dequantised
 * values (either may be NULL). The planes are validated first; invalid planes are refused.
 * x must hold at least cols codes; only the first cols are read.
 */
int oracle_gemv(const uint8_t *planes, int64_t len, int64_t rows, int64_t cols, const int8_t *x, int64_t x_len,
                float x_scale, float w_scale, int32_t *out_i32, float *out_f32, double *out_f64, int nthreads,
                or_err *e) {
    int rc = oracle_validate(planes, len, rows, cols, e);
    if (rc) return rc;
    if (x_len < cols) return set_err(e, OR_E_INVAL, -1, -1, -1);
    int64_t bpr = oracle_beats_per_row(cols);
    int bad = 0;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1) reduction(| : bad)
    for (int64_t r = 0; r < rows; ++r) {
        int32_t acc = 0;
        if (oracle_row_sum(planes, bpr, r, cols, x, &acc)) {
            bad |= 1;
            continue;
        }
        out_i32[r] = acc;
        float y32;
        double y64;
        oracle_dequant(acc, x_scale, w_scale, &y32, &y64);
        if (out_f32) out_f32[r] = y32;
        if (out_f64) out_f64[r] = y64;
    }
    if (bad) return set_err(e, OR_E_RANGE, -1, -1, -1);
    return set_err(e, OR_OK, -1, -1, -1);
}

/*
 * The second, independent formulation ([TP] "On popcount", "Verification"): split x into
 * its eight two's-complement bit planes X_j (bit k of X_j = bit j of x[64b + k]); then
 *   acc = sum_b sum_j c_j * (popcount(pos & X_j) - popcount(neg & X_j)),
 * c_j = 2^j for j < 7 and c_7 = -128. It never forms a per-weight trit.
 */
static int popcount64(uint64_t v) {
    int n = 0;
    while (v) {
        n += (int)(v & 1);
        v >>= 1;
    }
    return n;
}

int oracle_gemv_bitserial(const uint8_t *planes, int64_t len, int64_t rows, int64_t cols, const int8_t *x,
                          int64_t x_len, int32_t *out_i32, int nthreads, or_err *e) {
    int rc = oracle_validate(planes, len, rows, cols, e);
    if (rc) return rc;
    if (x_len < cols) return set_err(e, OR_E_INVAL, -1, -1, -1);
    int64_t bpr = oracle_beats_per_row(cols);
    int bad = 0;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1) reduction(| : bad)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t acc = 0;
        for (int64_t b = 0; b < bpr; ++b) {
            const uint8_t *beat = planes + (r * bpr + b) * 16;
            uint64_t pos = load_le64(beat), neg = load_le64(beat + 8);
            for (int j = 0; j < 8; ++j) {
                uint64_t xj = 0;
                for (int k = 0; k < 64; ++k) {
                    int64_t c = 64 * b + k;
                    if (c < cols && ((((uint8_t)x[c]) >> j) & 1)) xj |= UINT64_C(1) << k;
                }
                int64_t cj = (j == 7) ? -128 : ((int64_t)1 << j);
                acc += cj * (int64_t)(popcount64(pos & xj) - popcount64(neg & xj));
            }
        }
        if (acc < INT32_MIN || acc > INT32_MAX)
            bad |= 1;
        else
            out_i32[r] = (int32_t)acc;
    }
    if (bad) return set_err(e, OR_E_RANGE, -1, -1, -1);
    return set_err(e, OR_OK, -1, -1, -1);
}

/*
 * Small batch: the batch-1 GEMV applied to each of `batch` activations. X is token-major,
 * row t at X + t * ldx (ldx >= cols); out_*[t * rows + r]; x_scales[t] per token, one
 * w_scale for the matrix.
 */
int oracle_gemm_small_batch(const uint8_t *planes, int64_t len, int64_t rows, int64_t cols, const int8_t *X,
                            int64_t batch, int64_t ldx, const float *x_scales, float w_scale, int32_t *out_i32,
                            float *out_f32, double *out_f64, int nthreads, or_err *e) {
    if (batch < 0 || ldx < cols) return set_err(e, OR_E_INVAL, -1, -1, -1);
    for (int64_t t = 0; t < batch; ++t) {
        int rc = oracle_gemv(planes, len, rows, cols, X + t * ldx, ldx, x_scales[t], w_scale, out_i32 + t * rows,
                             out_f32 ? out_f32 + t * rows : NULL, out_f64 ? out_f64 + t * rows : NULL, nthreads, e);
        if (rc) return rc;
    }
    return set_err(e, OR_OK, -1, -1, -1);
}

/* bfloat16 is the upper half of an IEEE binary32 ([TF] 2.4 stores BF16 little-endian); widening is exact. */
static double bf16_to_double(uint16_t h) {
    uint32_t b = (uint32_t)h << 16;
    float f;
    memcpy(&f, &b, 4);
    return (double)f;
}

/*
 * Dense head ([TP] "Where the bytes are", [TF] 2.4): y[v] = sum_h W[v][h] x[h] over bf16
 * W [rows x cols] row-major and bf16 x [cols], accumulated in float64 in column order;
 * s[v] = sum_h |W[v][h] x[h]| (the scale of the admissible rounding error).
 */
int oracle_dense_head(const uint16_t *w, int64_t rows, int64_t cols, const uint16_t *x, double *y, double *s,
                      int nthreads) {
    if (rows < 0 || cols < 0) return OR_E_INVAL;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1)
    for (int64_t v = 0; v < rows; ++v) {
        double acc = 0.0, mag = 0.0;
        for (int64_t h = 0; h < cols; ++h) {
            double p = bf16_to_double(w[v * cols + h]) * bf16_to_double(x[h]);
            acc += p;
            mag += p < 0 ? -p : p;
        }
        y[v] = acc;
        if (s) s[v] = mag;
    }
    return OR_OK;
}

/*
 * Activation quantisation in front of a matvec ([TP] "Numerics": the Reference and Folded modes).
 * h is the float32 residual stream [n], g the float32 RMS-norm gain [n]; eps the norm's epsilon
 * (the pages give none; callers pass it).
 *
 *   rms = sqrt(sum_i h_i^2 / n + eps), the sum and the root in float64 over i in order.
 *
 * Reference (folded == 0): the norm is materialised, y_i = (h_i / (float)rms) * g_i in float32;
 *   then the absmax code of y: m = max_i |y_i|, q_i = rint((127 * y_i) / m) (float32, ties to even),
 *   scale = m / 127 (float32).
 * Folded (folded == 1): the per-element divide leaves. Absmax codes do not change when every input
 *   is scaled by one positive number, and y = u / rms with u_i = h_i * g_i, so the codes are taken
 *   from u directly and the rms survives only in the per-token scale:
 *   m = max_i |u_i|, q_i = rint((127 * u_i) / m) (float32), scale = (float)((m / 127) / rms) in float64.
 * m == 0 gives all-zero codes and scale 0. In exact arithmetic the two modes give the same codes
 * and scales; in floating point a code may differ by one where the value sits at a rounding tie.
 */
static double oracle_rms(const float *h, int64_t n, float eps) {
    double ss = 0.0;
    for (int64_t i = 0; i < n; ++i) ss += (double)h[i] * (double)h[i];
    return sqrt(ss / (double)n + (double)eps);
}

/* One absmax code. Non-finite input (the pages give no rule; reading adopted on both sides): a code
 * whose float32 value is NaN is 0. That covers u = NaN, and u = +-inf once m is infinite (inf / inf);
 * NaN entries never raise m, since a comparison with NaN is false. Finite values clamp to +-127. */
static int8_t oracle_code(float v, float m) {
    float t = (127.0f * v) / m;
    float r = rintf(t);
    if (r != r) return 0;
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    return (int8_t)r;
}

int oracle_quantize(const float *h, const float *g, int64_t n, float eps, int folded, int8_t *q, float *scale) {
    if (n <= 0 || !h || !g || !q || !scale || !(eps >= 0.0f)) return OR_E_INVAL;
    const double rms = oracle_rms(h, n, eps);
    float *v = (float *)malloc((size_t)n * sizeof(float));
    if (!v) return OR_E_INVAL;
    const float rms32 = (float)rms;
    for (int64_t i = 0; i < n; ++i) v[i] = folded ? h[i] * g[i] : (h[i] / rms32) * g[i];
    float m = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(v[i]);
        if (a > m) m = a;
    }
    if (m == 0.0f) {
        memset(q, 0, (size_t)n);
        *scale = 0.0f;
    } else {
        for (int64_t i = 0; i < n; ++i) q[i] = oracle_code(v[i], m);
        *scale = folded ? (float)(((double)m / 127.0) / rms) : m / 127.0f;
    }
    free(v);
    return OR_OK;
}

/*
 * IntMlp ([TP] "Numerics", the third mode): the squared-ReLU stage of the MLP in exact integers.
 * The gate and up projections of one token share the activation x; their exact row sums are a_g and
 * a_u, and their dequantisation scales S_g = x_scale * w_g and S_u = x_scale * w_u are uniform and
 * positive, so
 *   relu(a_g S_g)^2 (a_u S_u) = t K,   t = relu(a_g)^2 a_u (an integer),   K = S_g^2 S_u.
 * t is formed in 64-bit integers (checked in 128 bits: |a| <= 128 cols, so t fits whenever
 * 128 cols < 2^21, and |t| < 2^55 at 2560 columns as the pages state). K is one float64 number:
 * S_g and S_u are exact float64 products of two floats; K = (S_g * S_g) * S_u, two roundings.
 * a_g and a_u come from oracle_gemv. gate_i32 / up_i32 may be NULL.
 */
int oracle_intmlp(const uint8_t *gate, const uint8_t *up, int64_t len, int64_t rows, int64_t cols,
                  const int8_t *x, int64_t x_len, float x_scale, float w_gate, float w_up, int64_t *t,
                  double *k, int32_t *gate_i32, int32_t *up_i32, int nthreads, or_err *e) {
    if (rows < 0 || !t || !k) return set_err(e, OR_E_INVAL, -1, -1, -1);
    int32_t *ag = (int32_t *)malloc((size_t)(rows > 0 ? rows : 1) * sizeof(int32_t));
    int32_t *au = (int32_t *)malloc((size_t)(rows > 0 ? rows : 1) * sizeof(int32_t));
    if (!ag || !au) {
        free(ag);
        free(au);
        return set_err(e, OR_E_INVAL, -1, -1, -1);
    }
    int rc = oracle_gemv(gate, len, rows, cols, x, x_len, x_scale, w_gate, ag, NULL, NULL, nthreads, e);
    if (!rc) rc = oracle_gemv(up, len, rows, cols, x, x_len, x_scale, w_up, au, NULL, NULL, nthreads, e);
    if (!rc) {
        for (int64_t r = 0; r < rows; ++r) {
            const __int128 g = ag[r] > 0 ? (__int128)ag[r] : 0;
            const __int128 v = g * g * (__int128)au[r];
            if (v > (__int128)INT64_MAX || v < -(__int128)INT64_MAX) {
                rc = set_err(e, OR_E_RANGE, r, -1, -1);
                break;
            }
            t[r] = (int64_t)v;
            if (gate_i32) gate_i32[r] = ag[r];
            if (up_i32) up_i32[r] = au[r];
        }
    }
    if (!rc) {
        const double sg = (double)x_scale * (double)w_gate;
        const double su = (double)x_scale * (double)w_up;
        *k = (sg * sg) * su;
    }
    free(ag);
    free(au);
    return rc;
}

/*
 * BITCOS ("BITCOS: Intel's Ternary LLM Weight Format Goes Below 1.58 Bits", "A bitmap and a sign"):
 * every weight gets a presence bit (set when it is nonzero); every nonzero weight, in the same
 * order, gets a sign bit (set when it is -1). Zeros cost their presence bit only, so n weights with
 * nnz nonzeros take n + nnz bits, 2 - z bits per weight at zero density z.
 *
 * Flat form: bit i of the bitmap is bit (i & 7) of byte i >> 3; the k-th nonzero's sign is bit
 * (k & 7) of byte k >> 3 of the sign vector, set for -1. This is the layout of the packer and
 * unpacker the page prints in "A bitmap and a sign" (pack_bitcos / unpack_bitcos, tested there by a
 * round trip on a flat list); the two functions below are written from that definition, not from the
 * printed code. Sizes: ceil(n / 8) + ceil(nnz / 8) bytes.
 *
 * Row form (the layout the GPU reads; the page leaves the blocking to the kernel): per row,
 * bpr = ceil(cols / 64) presence words (u64, column c at bit c & 63 of word c >> 6, padding clear),
 * then the row's signs in u32 words, the row's k-th nonzero at bit k & 31 of word
 * row_start[r] + (k >> 5), unused bits clear; row_start[rows] is the total word count.
 */
int oracle_bitcos_pack_flat(const int8_t *w, int64_t n, uint8_t *bitmap, uint8_t *signs, int64_t *nnz) {
    if (n < 0 || (n && (!w || !bitmap || !signs)) || !nnz) return OR_E_INVAL;
    int64_t k = 0;
    for (int64_t i = 0; i < n; ++i)
        if (w[i] < -1 || w[i] > 1) return OR_E_INVAL;
    memset(bitmap, 0, (size_t)((n + 7) / 8));
    for (int64_t i = 0; i < n; ++i) {
        if (w[i] == 0) continue;
        bitmap[i >> 3] |= (uint8_t)(1u << (i & 7));
        if ((k & 7) == 0) signs[k >> 3] = 0;
        if (w[i] < 0) signs[k >> 3] |= (uint8_t)(1u << (k & 7));
        ++k;
    }
    *nnz = k;
    return OR_OK;
}

/* The inverse, from the definition of the two arrays: the k-th set presence bit (in weight order)
 * takes sign bit k (the page's unpack_bitcos in "A bitmap and a sign" decodes the same layout; this
 * one is written from the definition) and checks its bounds: bitmap_len must cover n bits, and a bitmap with more set bits than the
 * sign_len bytes hold sign bits is refused (OR_E_SIZE) instead of read past the signs. */
int oracle_bitcos_unpack_flat(const uint8_t *bitmap, int64_t bitmap_len, const uint8_t *signs, int64_t sign_len,
                              int64_t n, int8_t *w) {
    if (n < 0 || bitmap_len < (n + 7) / 8 || sign_len < 0) return OR_E_INVAL;
    if (n && (!bitmap || !w)) return OR_E_INVAL;
    if (sign_len > 0 && !signs) return OR_E_INVAL;
    int64_t next_sign = 0; /* the sign bit the next nonzero weight takes */
    for (int64_t i = 0; i < n; ++i) {
        const int present = (bitmap[i / 8] >> (i % 8)) & 1;
        if (!present) {
            w[i] = 0;
            continue;
        }
        if (next_sign >= 8 * sign_len) return OR_E_SIZE;
        const int negative = (signs[next_sign / 8] >> (next_sign % 8)) & 1;
        w[i] = negative ? (int8_t)-1 : (int8_t)1;
        ++next_sign;
    }
    return OR_OK;
}

/* Row form. sign_words receives row_start[rows] words; pass sign_words = NULL to get the count
 * into row_start only. */
int oracle_bitcos_pack_rows(const int8_t *w, int64_t rows, int64_t cols, uint64_t *presence, uint32_t *sign_words,
                            uint32_t *row_start) {
    if (rows < 0 || cols < 0 || !row_start || (rows * cols && !w)) return OR_E_INVAL;
    const int64_t bpr = oracle_beats_per_row(cols);
    uint64_t total = 0;
    for (int64_t r = 0; r < rows; ++r) {
        row_start[r] = (uint32_t)total;
        int64_t k = 0;
        for (int64_t c = 0; c < cols; ++c) {
            const int8_t v = w[r * cols + c];
            if (v < -1 || v > 1) return OR_E_INVAL;
            if (v != 0) ++k;
        }
        total += (uint64_t)((k + 31) / 32);
        if (total > 0xFFFFFFFFull) return OR_E_RANGE;
    }
    row_start[rows] = (uint32_t)total;
    if (!sign_words) return OR_OK;
    if (rows * bpr && !presence) return OR_E_INVAL;
    memset(sign_words, 0, (size_t)total * 4);
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < bpr; ++b) presence[r * bpr + b] = 0;
        int64_t k = 0;
        for (int64_t c = 0; c < cols; ++c) {
            const int8_t v = w[r * cols + c];
            if (v == 0) continue;
            presence[r * bpr + (c >> 6)] |= UINT64_C(1) << (c & 63);
            if (v < 0) sign_words[row_start[r] + (k >> 5)] |= UINT32_C(1) << (k & 31);
            ++k;
        }
    }
    return OR_OK;
}

/* y = W x from the row form, one weight at a time: weight (r, c) is 0 without its presence bit, else
 * -1 or +1 by the sign bit of the row's nonzero it is. Dequantisation as oracle_gemv. */
int oracle_bitcos_gemv(const uint64_t *presence, const uint32_t *sign_words, const uint32_t *row_start, int64_t rows,
                       int64_t cols, const int8_t *x, float x_scale, float w_scale, int32_t *out_i32, float *out_f32,
                       double *out_f64, int nthreads) {
    if (rows < 0 || cols < 0 || !row_start || !out_i32) return OR_E_INVAL;
    const int64_t bpr = oracle_beats_per_row(cols);
    int bad = 0;
#pragma omp parallel for schedule(static) num_threads(nthreads > 0 ? nthreads : 1) reduction(| : bad)
    for (int64_t r = 0; r < rows; ++r) {
        int64_t acc = 0, k = 0;
        for (int64_t c = 0; c < cols; ++c) {
            if (!((presence[r * bpr + (c >> 6)] >> (c & 63)) & 1)) continue;
            const int neg = (int)((sign_words[row_start[r] + (k >> 5)] >> (k & 31)) & 1);
            acc += neg ? -(int64_t)x[c] : (int64_t)x[c];
            ++k;
        }
        if (acc > INT32_MAX || acc < INT32_MIN) {
            bad |= 1;
            continue;
        }
        out_i32[r] = (int32_t)acc;
        float y32;
        double y64;
        oracle_dequant((int32_t)acc, x_scale, w_scale, &y32, &y64);
        if (out_f32) out_f32[r] = y32;
        if (out_f64) out_f64[r] = y64;
    }
    return bad ? OR_E_RANGE : OR_OK;
}
