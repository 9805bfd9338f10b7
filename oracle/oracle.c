/*
 * oracle.c -- plain, slow, obviously-correct CPU oracle for the BitNet b1.58
 * W2A8 ternary linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call, link or
 * load this file or the library built from it; only the test-suite, the
 * smoke check and the CPU-baseline leg of the benchmark do.  It shares no
 * code, header, table or helper with the HIP library.
 *
 * Source pages (cited by title and section):
 *   [W2A8] "BitNet GPU 推理框架：从零构建 W2A8 的 2-bit 大模型 CUDA GEMV 内核"
 *          (blog.gitcode.com) -- the W2A8 decode GEMV this layer is.
 *
 * What is computed, and where the pages define it:
 *   quant_absmax_i8  per-token absmax int8 activations, s = 127 / max|x|,
 *                    round, clamp to [-128, 127]                   [W2A8] §六 item 3
 *   unpack_tiles       ternary weights stored as 2-bit codes w + 2, four per
 *                    byte, the 16 codes of a 32-bit word interleaved so that
 *                    shift 2i + mask 0x03030303 yields elements 4i..4i+3
 *                                                                  [W2A8] §5.2
 *                    (the 16-row x 256-K tiling is this project's own layout;
 *                    its bit-level definition is restated at unpack_tiles)
 *   gemm_i32         int32 dot products of int8 activations and ternary
 *                    weights, exactly the int32 matmul the page's test uses
 *                                                                  [W2A8] §三 item 2, §5.3
 *   epilogue_bf16    rescale by the weight scale of the output's N-segment
 *                    and by the activation scale, round to bf16     [W2A8] §5.3
 *   absmean_scales,  ternarise a bf16 weight matrix by its mean absolute
 *   ternary_from_scale  value: s = 1/mean, Wt = clamp(round(W*s), -1, 1),
 *                    ws = 1/s, in the page's bf16 arithmetic       [W2A8] §4.2
 *   rmsnorm_bf16,    the glue between a block's projections: the norms,
 *   relu2_glu_bf16,  the MLP activation and the residual adds of the model
 *   add_bf16         the page converts (names only; formulas are readings,
 *                    stated at the functions)                      [W2A8] §4.1
 *
 * Readings where the page is ambiguous (each one is listed with its reason in
 * the design notes):
 *   - the activation scale s = 127/amax multiplies x on the way in, so the
 *     epilogue divides by it: y = acc * ws / s;
 *   - "round" is round-half-to-even (the page's torch round);
 *   - amax is clamped below at 1e-5, as the page's weight quantiser does;
 *   - floating point: the quantiser runs in IEEE fp32 (one correctly rounded
 *     division, one correctly rounded multiply); the epilogue runs in fp64 and
 *     is rounded once to bf16 (round to nearest, ties to even).
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -ffp-contract=off (no fast-math).
 */
#include <stdint.h>
#include <stddef.h>
#include <math.h>
#include <string.h>

#define OR_OK 0
#define OR_ERR_ARG (-1)      /* bad argument */
#define OR_ERR_RANGE (-2)    /* a sum does not fit in int32 */
#define OR_ERR_CODE (-3)     /* a real weight position holds code 0 */
#define OR_ERR_PAD (-4)      /* a padding position holds a non-zero code */

/* ---------------------------------------------------------------------- */
/* bf16 helpers                                                             */
/* ---------------------------------------------------------------------- */

/* bf16 -> fp32 is exact: a bf16 is the top 16 bits of an fp32. */
static float bf16_bits_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * Round a double to the nearest bf16 (ties to even), from the IEEE 754
 * definition of the format: 1 sign bit, 8 exponent bits (bias 127), 7
 * fraction bits; normal numbers are 2^E * (1 + f/128) with E in
 * [-126, 127], subnormals are 2^-126 * f/128.  So the spacing of
 * representable values around |v| is 2^(E-7) for normal |v| (E = exponent
 * of the leading bit) and 2^-133 below 2^-126.  Dividing |v| by that
 * spacing is an exact power-of-two scaling, nearbyint() rounds the
 * quotient to an integer with ties to even (default rounding mode), and
 * scaling back is exact again.  A result of 2^128 or more overflows to
 * infinity.
 */
uint16_t oracle_bf16_rne(double v)
{
    if (isnan(v))
        return (uint16_t)0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0x0000;
    double a = fabs(v);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80);
    int e2;
    (void)frexp(a, &e2);          /* a = m * 2^e2, m in [0.5, 1) */
    int E = e2 - 1;                /* exponent of the leading bit */
    int spacing_exp = (E < -126) ? -133 : E - 7;
    double r = nearbyint(ldexp(a, -spacing_exp));
    double rounded = ldexp(r, spacing_exp);
    if (rounded >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80);
    /* rounded is exactly representable in bf16, hence in fp32: take the
       top half of its fp32 encoding. */
    float f = (float)rounded;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (uint16_t)(u >> 16));
}

void oracle_bf16_rne_array(const double* v, uint16_t* out, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        out[i] = oracle_bf16_rne(v[i]);
}

/* ---------------------------------------------------------------------- */
/* Per-token absmax int8 quantisation  ([W2A8] §六 item 3)                  */
/* ---------------------------------------------------------------------- */

/*
 * For every row m of x (M rows of K values):
 *   amax = max(max_k |x[m][k]|, 1e-5)
 *   s[m] = 127 / amax                      (one fp32 division)
 *   q[m][k] = clamp(round_half_even(x[m][k] * s[m]), -128, 127)
 * x must be finite.
 */
int oracle_quant_absmax_i8_f32(const float* x, int M, int K, int8_t* q, float* s)
{
    if (!x || !q || !s || M < 0 || K < 0)
        return OR_ERR_ARG;
    for (int m = 0; m < M; ++m) {
        const float* row = x + (size_t)m * K;
        float amax = 0.0f;
        for (int k = 0; k < K; ++k) {
            float a = fabsf(row[k]);
            if (a > amax)
                amax = a;
        }
        if (amax < 1e-5f)
            amax = 1e-5f;
        float sm = 127.0f / amax;
        for (int k = 0; k < K; ++k) {
            float prod = row[k] * sm;
            float r = nearbyintf(prod);
            if (r > 127.0f)
                r = 127.0f;
            if (r < -128.0f)
                r = -128.0f;
            q[(size_t)m * K + k] = (int8_t)r;
        }
        s[m] = sm;
    }
    return OR_OK;
}

/* Same, for bf16 input (given as raw 16-bit patterns), widened exactly to fp32. */
int oracle_quant_absmax_i8_bf16(const uint16_t* x, int M, int K, int8_t* q, float* s)
{
    if (!x || !q || !s || M < 0 || K < 0)
        return OR_ERR_ARG;
    for (int m = 0; m < M; ++m) {
        const uint16_t* row = x + (size_t)m * K;
        float amax = 0.0f;
        for (int k = 0; k < K; ++k) {
            float a = fabsf(bf16_bits_to_float(row[k]));
            if (a > amax)
                amax = a;
        }
        if (amax < 1e-5f)
            amax = 1e-5f;
        float sm = 127.0f / amax;
        for (int k = 0; k < K; ++k) {
            float prod = bf16_bits_to_float(row[k]) * sm;
            float r = nearbyintf(prod);
            if (r > 127.0f)
                r = 127.0f;
            if (r < -128.0f)
                r = -128.0f;
            q[(size_t)m * K + k] = (int8_t)r;
        }
        s[m] = sm;
    }
    return OR_OK;
}

/* ---------------------------------------------------------------------- */
/* Unpack of the packed ternary weights                                      */
/* ---------------------------------------------------------------------- */

/*
 * Packed size of an N x K ternary matrix in the tiled layout: ceil(N/16) *
 * ceil(K/256) tiles of 1024 bytes each.
 */
size_t oracle_packed_bytes(int N, int K)
{
    if (N <= 0 || K <= 0)
        return 0;
    size_t bands = ((size_t)N + 15) / 16;
    size_t steps = ((size_t)K + 255) / 256;
    return bands * steps * 1024;
}

/* Byte offset and bit position of element (n, k) in the tiled layout. */
static size_t layout_byte(size_t n, size_t k, size_t steps, int *bit)
{
    size_t t = (n / 16) * steps + k / 256;
    size_t q = 16 * ((n % 16) / 4) + (k % 256) / 16;
    size_t i = n % 4;
    size_t e = k % 16;
    *bit = (int)(2 * (e / 4));
    return t * 1024 + 16 * q + 4 * i + e % 4;
}

/*
 * Layout, stated at the level of single bits.  The weight w[n][k] of an
 * N x K matrix (row n = output n) is stored as the 2-bit code w + 2
 * ({-1,0,1} -> {1,2,3}, as on [W2A8] §5.2); the code lives in
 *   tile      t = (n / 16) * ceil(K/256) + (k / 256)     (1024 bytes each)
 *   slot      q = 16 * ((n % 16) / 4) + (k % 256) / 16   (16 bytes each)
 *   word      i = n % 4                                  (4 bytes each, little endian)
 *   element   e = k % 16
 *   byte      t*1024 + 16*q + 4*i + (e % 4)
 *   bits      2*(e / 4) .. 2*(e / 4) + 1 of that byte
 * so a tile is 16 rows x 256 K, a 16-byte slot holds four rows
 * (4*((n%16)/4) .. +3) of one 16-wide K chunk, and inside each 32-bit word
 * element e sits at bit 8*(e%4) + 2*(e/4): the word holds its 16 elements
 * in the page's interleaved order 0,4,8,12,1,5,9,13,2,6,10,14,3,7,11,15
 * ([W2A8] §5.2).  Positions with n >= N or k >= K (padding of the last
 * tile row/column) hold code 0.  Code 0 at a real position is an error.
 *
 * Returns OR_OK, OR_ERR_CODE (and *bad = flat index n*K+k of the first bad
 * code) or OR_ERR_PAD (and *bad = byte offset of the first bad padding byte).
 */
int oracle_unpack_tiles(const uint8_t* packed, int N, int K, int8_t* w, int64_t* bad)
{
    if (!packed || !w || N <= 0 || K <= 0)
        return OR_ERR_ARG;
    size_t steps = ((size_t)K + 255) / 256;
    size_t bands = ((size_t)N + 15) / 16;
    /* every real position */
    for (int n = 0; n < N; ++n) {
        for (int k = 0; k < K; ++k) {
            int bit;
            size_t byte = layout_byte((size_t)n, (size_t)k, steps, &bit);
            int code = (packed[byte] >> bit) & 3;
            if (code == 0) {
                if (bad)
                    *bad = (int64_t)n * K + k;
                return OR_ERR_CODE;
            }
            w[(size_t)n * K + k] = (int8_t)(code - 2);
        }
    }
    /* every padding position must be code 0 */
    for (size_t n = 0; n < bands * 16; ++n) {
        for (size_t k = 0; k < steps * 256; ++k) {
            if (n < (size_t)N && k < (size_t)K)
                continue;
            int bit;
            size_t byte = layout_byte(n, k, steps, &bit);
            if (((packed[byte] >> bit) & 3) != 0) {
                if (bad)
                    *bad = (int64_t)byte;
                return OR_ERR_PAD;
            }
        }
    }
    return OR_OK;
}

/* ---------------------------------------------------------------------- */
/* int32 GEMM / GEMV  ([W2A8] §三 item 2, §5.3)                              */
/* ---------------------------------------------------------------------- */

/*
 * acc[m][n] = sum_k xq[m][k] * w[n][k]   (xq: M x K int8, w: N x K int8)
 * Summed in int64; OR_ERR_RANGE if a result does not fit in int32.
 */
int oracle_gemm_i32(const int8_t* xq, const int8_t* w, int M, int N, int K, int32_t* acc)
{
    if (!xq || !w || !acc || M < 0 || N < 0 || K < 0)
        return OR_ERR_ARG;
    for (int m = 0; m < M; ++m) {
        const int8_t* xr = xq + (size_t)m * K;
        for (int n = 0; n < N; ++n) {
            const int8_t* wr = w + (size_t)n * K;
            int64_t sum = 0;
            for (int k = 0; k < K; ++k)
                sum += (int64_t)xr[k] * (int64_t)wr[k];
            if (sum > INT32_MAX || sum < INT32_MIN)
                return OR_ERR_RANGE;
            acc[(size_t)m * N + n] = (int32_t)sum;
        }
    }
    return OR_OK;
}

/* ---------------------------------------------------------------------- */
/* Epilogue  ([W2A8] §5.3)                                                   */
/* ---------------------------------------------------------------------- */

/*
 * y[m][n] = bf16_rne( acc[m][n] * ws[n / (N / ws_num)] / s[m] )
 * evaluated in fp64 as ((double)acc * (double)ws) / (double)s.  The product
 * is exact (|acc| < 2^31, ws has 8 significant bits); the quotient is
 * rounded once to fp64 and then once to bf16.
 * ws holds ws_num bf16 scales, one per equal N-segment; N % ws_num == 0.
 */
int oracle_epilogue_bf16(const int32_t* acc, const float* s, const uint16_t* ws, int ws_num,
                         int M, int N, uint16_t* y)
{
    if (!acc || !s || !ws || !y || M < 0 || N <= 0 || ws_num <= 0 || N % ws_num != 0)
        return OR_ERR_ARG;
    int seg = N / ws_num;
    for (int m = 0; m < M; ++m) {
        for (int n = 0; n < N; ++n) {
            double wsv = (double)bf16_bits_to_float(ws[n / seg]);
            double val = ((double)acc[(size_t)m * N + n] * wsv) / (double)s[m];
            y[(size_t)m * N + n] = oracle_bf16_rne(val);
        }
    }
    return OR_OK;
}

/* ---------------------------------------------------------------------- */
/* Whole layer                                                               */
/* ---------------------------------------------------------------------- */

/* int8 activations in: acc = gemm_i32(xq, w); y = epilogue(acc). */
int oracle_bitlinear_i8(const int8_t* xq, const int8_t* w, const float* s, const uint16_t* ws,
                        int ws_num, int M, int N, int K, int32_t* acc, uint16_t* y)
{
    int rc = oracle_gemm_i32(xq, w, M, N, K, acc);
    if (rc != OR_OK)
        return rc;
    return oracle_epilogue_bf16(acc, s, ws, ws_num, M, N, y);
}

/* bf16 activations in: quantise each row, then the int8 layer. */
int oracle_bitlinear_bf16(const uint16_t* x, const int8_t* w, const uint16_t* ws, int ws_num,
                          int M, int N, int K, int8_t* q, float* s, int32_t* acc, uint16_t* y)
{
    int rc = oracle_quant_absmax_i8_bf16(x, M, K, q, s);
    if (rc != OR_OK)
        return rc;
    return oracle_bitlinear_i8(q, w, s, ws, ws_num, M, N, K, acc, y);
}

/* ---------------------------------------------------------------------- */
/* Weight ternarisation by the mean absolute value  ([W2A8] §4.2)           */
/* ---------------------------------------------------------------------- */

/*
 * The page's converter quantises each projection matrix W (bf16) on its own:
 *     s  = 1 / max(mean|W|, 1e-5)
 *     Wt = clamp(round(W * s), -1, 1)          stored as int8, then packed
 *     ws = 1 / s                               the matrix's weight scale
 * written as torch operations on bf16 tensors.  Such an operation computes in
 * fp32 and rounds its result to bf16 (nearest, ties to even); that is the
 * arithmetic followed here, step by step.  Readings:
 *   - mean|W| is the exact mean of the bf16 magnitudes, rounded once to bf16
 *     (torch accumulates in fp32 in an unspecified order; the exact mean is
 *     the order-free value it approximates).  It is passed in as mean_bits,
 *     computed by the Python side (exact integer arithmetic);
 *   - the clamp compares in fp32 with 1e-5f and stores bf16(1e-5f) below it;
 *   - round is round half to even; W must be finite.
 */

/* bf16 of an fp32 value, via the fp64 rounding above (fp32 -> fp64 is exact). */
static uint16_t bf16_of_float(float f)
{
    return oracle_bf16_rne((double)f);
}

/* From the bf16 mean: the multiplier s and the weight scale ws (both bf16). */
int oracle_absmean_scales(uint16_t mean_bits, uint16_t* s_bits, uint16_t* ws_bits)
{
    if (!s_bits || !ws_bits)
        return OR_ERR_ARG;
    float mean = bf16_bits_to_float(mean_bits);
    if (!(mean >= 0.0f) || isinf(mean))
        return OR_ERR_ARG;
    if (mean < 1e-5f)
        mean = bf16_bits_to_float(bf16_of_float(1e-5f));
    uint16_t s = bf16_of_float(1.0f / mean);             /* one fp32 division */
    uint16_t ws = bf16_of_float(1.0f / bf16_bits_to_float(s));
    *s_bits = s;
    *ws_bits = ws;
    return OR_OK;
}

/* Wt[i] = clamp(round(bf16(W[i] * s)), -1, 1) for n bf16 weights. */
int oracle_ternary_from_scale(const uint16_t* w, size_t n, uint16_t s_bits, int8_t* q)
{
    if ((!w || !q) && n)
        return OR_ERR_ARG;
    float s = bf16_bits_to_float(s_bits);
    for (size_t i = 0; i < n; ++i) {
        /* fl32(w * s): exact (8 x 8 significant bits) unless it underflows */
        float prod = bf16_bits_to_float(w[i]) * s;
        float t = bf16_bits_to_float(bf16_of_float(prod));
        float r = nearbyintf(t);                         /* ties to even */
        if (r > 1.0f)
            r = 1.0f;
        if (r < -1.0f)
            r = -1.0f;
        q[i] = (int8_t)r;
    }
    return OR_OK;
}

/* ---------------------------------------------------------------------- */
/* Glue between the layers of a block (decode step chained through the     */
/* model's norms, activation and residuals)                                 */
/* ---------------------------------------------------------------------- */
/*
 * [W2A8] §4.1 names the norms of the model it converts -- attention_norm and
 * ffn_norm before the attention and MLP inputs, and BitNet b1.58's own
 * attn_sub_norm and ffn_sub_norm -- and the fused projections wqkv, wo, w13
 * (gate_proj then up_proj) and w2, but states neither the norm's formula
 * nor the MLP activation.  Readings (each listed with its reason in the
 * design notes): every norm is an RMSNorm with a bf16 weight and
 * eps = fp32(1e-5); the MLP activation is the squared ReLU of the gate half
 * times the up half of w13's output; a residual adds two bf16 vectors.  All
 * of it runs in fp64 and is rounded once to bf16.
 */

/* y[i] = bf16( fl64(x[i] * g[i]) * fl64(1 / sqrt(sum_j x[j]^2 / K + eps)) ):
 * the inverse root mean square of the row (the sum taken in fp64 in index
 * order), applied to the exact product of the element and its weight. */
int oracle_rmsnorm_bf16(const uint16_t* x, const uint16_t* g, int K, float eps, uint16_t* y)
{
    if (!x || !g || !y || K < 1 || !(eps >= 0.0f))
        return OR_ERR_ARG;
    double sum = 0.0;
    for (int i = 0; i < K; ++i) {
        double v = (double)bf16_bits_to_float(x[i]);
        sum += v * v;
    }
    double inv = 1.0 / sqrt(sum / (double)K + (double)eps);
    for (int i = 0; i < K; ++i) {
        double prod = (double)bf16_bits_to_float(x[i]) * (double)bf16_bits_to_float(g[i]);
        y[i] = oracle_bf16_rne(prod * inv);
    }
    return OR_OK;
}

/* m[i] = bf16( max(gate[i], 0)^2 * up[i] ), exact in fp64 before the
 * rounding (a bf16 has 8 significant bits, so the product has at most 24,
 * and its exponent stays inside fp64's range). */
int oracle_relu2_glu_bf16(const uint16_t* gate, const uint16_t* up, int K, uint16_t* m)
{
    if (!gate || !up || !m || K < 1)
        return OR_ERR_ARG;
    for (int i = 0; i < K; ++i) {
        double a = (double)bf16_bits_to_float(gate[i]);
        double r = a > 0.0 ? a : 0.0;
        m[i] = oracle_bf16_rne(r * r * (double)bf16_bits_to_float(up[i]));
    }
    return OR_OK;
}

/* out[i] = bf16( a[i] + b[i] ): the fp64 sum of two bf16 values is exact
 * unless their exponents differ by more than 45, and then the smaller lies
 * far below half a bf16 unit of the larger, so rounding that sum gives the
 * bf16 of the exact sum either way. */
int oracle_add_bf16(const uint16_t* a, const uint16_t* b, int n, uint16_t* out)
{
    if (!a || !b || !out || n < 0)
        return OR_ERR_ARG;
    for (int i = 0; i < n; ++i)
        out[i] = oracle_bf16_rne((double)bf16_bits_to_float(a[i]) + (double)bf16_bits_to_float(b[i]));
    return OR_OK;
}
