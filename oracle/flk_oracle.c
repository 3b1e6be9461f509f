/*
 * flk_oracle.c -- plain, slow, scalar CPU oracle for the FlashLoop packed-KV codec.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  The product path never
 * links it, and this file shares no source with the HIP implementation.
 *
 * What it computes follows two pages:
 *   [RFC] "FlashLoop integration -- token-sparse prefill, sparse decode attention, and KV
 *         residual quantization" (vllm-rlt issue #156), section 3.3 "Quantized base and
 *         cross-loop KV residuals" (and 3.1 for the nested active sets, 7.4 for storage);
 *   [PR]  vllm-rlt pull request #166 (standalone INT4 codec), its "Purpose" list and the
 *         review that follows it (storage arithmetic, nibble order, compact-row K groups).
 *
 * Every floating-point step is written out one IEEE operation at a time.  Build with
 *   gcc -O2 -ffp-contract=off -fno-fast-math -std=c11
 * on x86-64 (SSE arithmetic, FLT_EVAL_METHOD == 0, round-to-nearest-even, no FTZ/DAZ),
 * so every `float` expression below is one correctly rounded binary32 operation.
 *
 * Data conventions (the readings are listed with their reasons in the design notes):
 *   - tensors are [rows, H, D] row-major, channels contiguous; BF16 values are passed
 *     as their 16-bit patterns (uint16_t);
 *   - group size 64.  K ("kind" 0): a group is up to 64 consecutive compact rows of one
 *     (head, channel).  V ("kind" 1): a group is up to 64 consecutive channels of one
 *     (row, head).  The last group along the axis may be shorter;
 *   - K group ownership has two forms.  Compact-row groups (the default): up to 64
 *     consecutive compact rows.  Tile groups ("page-local", asked for by the PR review's
 *     item 3, "Group ownership vs 16-token pages"): the compact rows whose positions lie in
 *     one 64-position tile [64t, 64t+64), 0 to 64 of them.  Dense streams are the same in
 *     both forms;
 *   - params are one uint32 per group: FP16 minimum in the low half, FP16 scale in the
 *     high half.  K params are laid out [ceil(n/64)][H][D] (compact-row groups) or
 *     [ceil(T/64)][H][D] (tile groups; an empty tile's params are 0), V params
 *     [n][H][ceil(D/64)];
 *   - codes are two per byte, [row][H][D/2]; byte j of (row, head) holds the code of
 *     channel 2j in its low nibble and channel 2j+1 in its high nibble.
 *
 * Parity of these layouts with the original Torch module cannot be checked: that module
 * is not available.  The conventions are pinned by the tests instead.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_E_NONFINITE 1   /* a group holds an Inf or NaN input value               */
#define ORC_E_RANGE 2       /* a group's FP16 minimum or scale overflows binary16     */
#define ORC_E_ARG 3         /* bad shape or argument                                  */

#define ORC_GROUP 64

/* ------------------------------------------------------------------------------------ */
/* IEEE-754 conversions, written from the definition of round-to-nearest, ties-to-even.  */
/* ------------------------------------------------------------------------------------ */

/* Round the finite value v (any binary32 value, carried exactly in a double) to the
 * binary format with p significand bits, minimum normal exponent emin and maximum
 * exponent emax.  Rounding is to nearest, ties to the candidate with an even last
 * significand bit; a result above the largest finite value becomes infinity, as IEEE
 * 754 prescribes for an unbounded-exponent rounding that lands beyond it.             */
static double round_to_format(double v, int p, int emin, int emax) {
    if (v == 0.0 || isnan(v) || isinf(v)) return v;
    double a = fabs(v);
    int e;
    (void)frexp(a, &e);          /* a = m * 2^e with m in [0.5, 1): leading bit at e-1 */
    int lead = e - 1;
    if (lead < emin) lead = emin; /* below the normal range the quantum stays fixed     */
    double quantum = ldexp(1.0, lead - (p - 1));
    double q = a / quantum;       /* exact: scaling by a power of two                    */
    double fl = floor(q);
    double rem = q - fl;          /* exact                                                */
    double r;
    if (rem > 0.5) r = fl + 1.0;
    else if (rem < 0.5) r = fl;
    else r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    double res = r * quantum;
    double max_finite = ldexp(2.0 - ldexp(1.0, 1 - p), emax);
    if (res > max_finite) res = INFINITY;
    return copysign(res, v);
}

/* binary32 -> bfloat16 (8 significand bits, exponent range of binary32).  bfloat16 is
 * the upper half of a binary32 pattern, so the rounded value's binary32 bits carry it. */
uint16_t orc_bf16_from_f32(float x) {
    if (isnan(x)) {
        uint32_t u; memcpy(&u, &x, 4);
        return (uint16_t)((u >> 16) | 0x0040u);   /* keep sign, force a quiet NaN */
    }
    float r = (float)round_to_format((double)x, 8, -126, 127);
    uint32_t u; memcpy(&u, &r, 4);
    return (uint16_t)(u >> 16);
}

float orc_f32_from_bf16(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f; memcpy(&f, &u, 4);
    return f;
}

/* binary32 -> binary16 (11 significand bits, emin -14, emax 15), subnormals kept. */
uint16_t orc_f16_from_f32(float x) {
    if (isnan(x)) return (uint16_t)(signbit(x) ? 0xFE00u : 0x7E00u);
    double r = round_to_format((double)x, 11, -14, 15);
    uint16_t sign = signbit(r) ? 0x8000u : 0u;
    double a = fabs(r);
    if (isinf(a)) return (uint16_t)(sign | 0x7C00u);
    if (a == 0.0) return sign;
    if (a < ldexp(1.0, -14)) {                     /* subnormal: a = mant * 2^-24 */
        return (uint16_t)(sign | (uint16_t)(a / ldexp(1.0, -24)));
    }
    int e;
    double m = frexp(a, &e);                        /* a = m * 2^e, m in [0.5, 1) */
    int exp_field = (e - 1) + 15;
    double frac = (m * 2.0 - 1.0) * 1024.0;         /* exact: 10 fraction bits    */
    return (uint16_t)(sign | (uint16_t)(exp_field << 10) | (uint16_t)frac);
}

float orc_f32_from_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int exp_field = (h >> 10) & 0x1F;
    int frac = h & 0x3FF;
    double v;
    if (exp_field == 0) v = ldexp((double)frac, -24);
    else if (exp_field == 31) v = frac ? NAN : INFINITY;
    else v = ldexp(1.0 + frac / 1024.0, exp_field - 15);
    return (float)(sign ? -v : v);
}

/* Array forms, for the conversion pins in the test suite. */
void orc_bf16_from_f32_array(const float* x, uint16_t* out, size_t n) {
    for (size_t i = 0; i < n; ++i) out[i] = orc_bf16_from_f32(x[i]);
}
void orc_f16_from_f32_array(const float* x, uint16_t* out, size_t n) {
    for (size_t i = 0; i < n; ++i) out[i] = orc_f16_from_f32(x[i]);
}
void orc_f32_from_f16_array(const uint16_t* h, float* out, size_t n) {
    for (size_t i = 0; i < n; ++i) out[i] = orc_f32_from_f16(h[i]);
}

/* ------------------------------------------------------------------------------------ */
/* Affine INT4 group quantizer (RFC section 3.3; PR #166 "Purpose").                     */
/* ------------------------------------------------------------------------------------ */

/* Total order on binary32 values in which -0 sorts below +0 (inputs are finite). */
static int total_less(float a, float b) {
    if (a < b) return 1;
    if (a == b && signbit(a) && !signbit(b)) return 1;
    return 0;
}

/* Quantize one group of `len` values.  Steps, in the RFC's order:
 *   min, max of the group;  scale = (max - min) / 15 in binary32;  both rounded to
 *   binary16 (the stored FP16 metadata);  a group whose FP16 scale is zero is the
 *   "constant group" (all codes 0, decoding to the minimum);  otherwise
 *   code = clamp(round_half_even((x - min) / scale), 0, 15).
 * By default the codes use the FP16-rounded minimum and scale, so the stored metadata is
 * the metadata the codes were chosen for.  With f32_params != 0 the codes use the binary32
 * minimum and scale before FP16 rounding instead (the upstream convention the PR review
 * describes); the stored params are FP16 either way.                                    */
static int quantize_group(const float* v, int len, int f32_params,
                          uint16_t* min16_out, uint16_t* scale16_out, uint8_t* codes) {
    for (int i = 0; i < len; ++i)
        if (!isfinite(v[i])) return ORC_E_NONFINITE;
    float mn = v[0], mx = v[0];
    for (int i = 1; i < len; ++i) {
        if (total_less(v[i], mn)) mn = v[i];
        if (total_less(mx, v[i])) mx = v[i];
    }
    float range = mx - mn;
    float scale32 = range / 15.0f;
    uint16_t min16 = orc_f16_from_f32(mn);
    uint16_t scale16 = orc_f16_from_f32(scale32);
    if ((min16 & 0x7FFFu) >= 0x7C00u || (scale16 & 0x7FFFu) >= 0x7C00u) return ORC_E_RANGE;
    *min16_out = min16;
    *scale16_out = scale16;

    float m = f32_params ? mn : orc_f32_from_f16(min16);
    float s = f32_params ? scale32 : orc_f32_from_f16(scale16);
    if (s == 0.0f) {                                  /* constant group */
        for (int i = 0; i < len; ++i) codes[i] = 0;
        return ORC_OK;
    }
    for (int i = 0; i < len; ++i) {
        float y = v[i] - m;
        float q = y / s;
        float k = nearbyintf(q);                       /* ties to even (FE_TONEAREST) */
        if (k < 0.0f) k = 0.0f;
        if (k > 15.0f) k = 15.0f;
        codes[i] = (uint8_t)k;
    }
    return ORC_OK;
}

/* decode = min + scale * code in binary32 (the product is exact: at most 15 significant
 * bits), then rounded to BF16, the compute dtype. */
static uint16_t dequant_one(uint32_t param, int code) {
    float m = orc_f32_from_f16((uint16_t)(param & 0xFFFFu));
    float s = orc_f32_from_f16((uint16_t)(param >> 16));
    float prod = s * (float)code;
    float x = m + prod;
    return orc_bf16_from_f32(x);
}

static size_t ceil_div(size_t a, size_t b) { return (a + b - 1) / b; }

/* Group counts and storage sizes (RFC section 7.4 resource accounting; PR review: 4 code
 * bits plus 32 parameter bits per 64 elements). */
size_t orc_num_groups(int kind, int H, int D, int n) {
    if (kind == 0) return ceil_div((size_t)n, ORC_GROUP) * (size_t)H * (size_t)D;
    return (size_t)n * (size_t)H * ceil_div((size_t)D, ORC_GROUP);
}
size_t orc_codes_bytes(int H, int D, int n) { return (size_t)n * (size_t)H * (size_t)D / 2; }
size_t orc_params_bytes(int kind, int H, int D, int n) { return 4 * orc_num_groups(kind, H, D, n); }
size_t orc_rows_bytes(int n, int sparse) { return sparse ? 4 * (size_t)n : 0; }

static size_t xidx(int H, int D, int row, int h, int c) {
    return ((size_t)row * (size_t)H + (size_t)h) * (size_t)D + (size_t)c;
}

static void put_code(uint8_t* codes, int H, int D, int row, int h, int c, int code) {
    size_t byte = ((size_t)row * (size_t)H + (size_t)h) * (size_t)(D / 2) + (size_t)(c / 2);
    if (c % 2 == 0) codes[byte] = (uint8_t)((codes[byte] & 0xF0u) | (uint8_t)code);
    else codes[byte] = (uint8_t)((codes[byte] & 0x0Fu) | (uint8_t)(code << 4));
}

static int get_code(const uint8_t* codes, int H, int D, int row, int h, int c) {
    size_t byte = ((size_t)row * (size_t)H + (size_t)h) * (size_t)(D / 2) + (size_t)(c / 2);
    return (c % 2 == 0) ? (codes[byte] & 0x0F) : (codes[byte] >> 4);
}

static size_t param_index(int kind, int H, int D, int row, int h, int c) {
    if (kind == 0) return ((size_t)(row / ORC_GROUP) * (size_t)H + (size_t)h) * (size_t)D + (size_t)c;
    size_t gv = ceil_div((size_t)D, ORC_GROUP);
    return ((size_t)row * (size_t)H + (size_t)h) * gv + (size_t)(c / ORC_GROUP);
}

static int check_shape(int kind, int H, int D, int n) {
    if (kind != 0 && kind != 1) return ORC_E_ARG;
    if (H <= 0 || D <= 0 || (D % 2) != 0 || n < 0) return ORC_E_ARG;
    return ORC_OK;
}

/* Quantize a [n, H, D] BF16 tensor with the grouping of `kind`: fills codes and params. */
int orc_quantize(int kind, int H, int D, int n, const uint16_t* x, uint8_t* codes,
                 uint32_t* params, int f32_params) {
    int st = check_shape(kind, H, D, n);
    if (st) return st;
    float vals[ORC_GROUP];
    uint8_t gc[ORC_GROUP];
    memset(codes, 0, orc_codes_bytes(H, D, n));
    if (kind == 0) {
        /* K: groups run down the compact rows of each (head, channel). */
        for (int g = 0; g * ORC_GROUP < n; ++g) {
            int r0 = g * ORC_GROUP;
            int len = (n - r0 < ORC_GROUP) ? n - r0 : ORC_GROUP;
            for (int h = 0; h < H; ++h)
                for (int c = 0; c < D; ++c) {
                    for (int i = 0; i < len; ++i) vals[i] = orc_f32_from_bf16(x[xidx(H, D, r0 + i, h, c)]);
                    uint16_t m16, s16;
                    st = quantize_group(vals, len, f32_params, &m16, &s16, gc);
                    if (st) return st;
                    params[param_index(0, H, D, r0, h, c)] = (uint32_t)m16 | ((uint32_t)s16 << 16);
                    for (int i = 0; i < len; ++i) put_code(codes, H, D, r0 + i, h, c, gc[i]);
                }
        }
    } else {
        /* V: groups run along the channels of each (row, head). */
        for (int row = 0; row < n; ++row)
            for (int h = 0; h < H; ++h)
                for (int c0 = 0; c0 < D; c0 += ORC_GROUP) {
                    int len = (D - c0 < ORC_GROUP) ? D - c0 : ORC_GROUP;
                    for (int i = 0; i < len; ++i) vals[i] = orc_f32_from_bf16(x[xidx(H, D, row, h, c0 + i)]);
                    uint16_t m16, s16;
                    st = quantize_group(vals, len, f32_params, &m16, &s16, gc);
                    if (st) return st;
                    params[param_index(1, H, D, row, h, c0)] = (uint32_t)m16 | ((uint32_t)s16 << 16);
                    for (int i = 0; i < len; ++i) put_code(codes, H, D, row, h, c0 + i, gc[i]);
                }
    }
    return ORC_OK;
}

/* Dequantize a packed [n, H, D] tensor back to BF16. */
int orc_dequantize(int kind, int H, int D, int n, const uint8_t* codes, const uint32_t* params,
                   uint16_t* xhat) {
    int st = check_shape(kind, H, D, n);
    if (st) return st;
    for (int row = 0; row < n; ++row)
        for (int h = 0; h < H; ++h)
            for (int c = 0; c < D; ++c)
                xhat[xidx(H, D, row, h, c)] =
                    dequant_one(params[param_index(kind, H, D, row, h, c)], get_code(codes, H, D, row, h, c));
    return ORC_OK;
}

/* ------------------------------------------------------------------------------------ */
/* Page-local K groups (PR review, item 3 "Group ownership vs 16-token pages": a K group   */
/* that follows compact-row order can mix rows of distant positions, so a page cannot be   */
/* freed, moved or shared alone; the review points to grouping that never merges rows of   */
/* different logical 64-token groups).  Group t of (head, channel) holds exactly the       */
/* compact rows whose logical positions lie in [64t, 64t+64).                              */
/* ------------------------------------------------------------------------------------ */

/* Logical position of compact row j (rows == NULL: the dense identity). */
static int32_t position_of(const int32_t* rows, int j) { return rows ? rows[j] : j; }

static int check_rows(const int32_t* rows, int n, int T) {
    if (n < 0 || n > T || (rows == NULL && n != T)) return ORC_E_ARG;
    for (int j = 0; rows && j < n; ++j)
        if (rows[j] < 0 || rows[j] >= T || (j > 0 && rows[j] <= rows[j - 1])) return ORC_E_ARG;
    return ORC_OK;
}

size_t orc_k_tile_params_bytes(int H, int D, int T) {
    return 4 * ceil_div((size_t)T, ORC_GROUP) * (size_t)H * (size_t)D;
}

/* Quantize K rows x [n, H, D] (compact row j at position rows[j]) with tile groups.
 * params: [ceil(T/64)][H][D]; an empty tile gets params 0 (no group to describe).      */
int orc_quantize_k_tiles(int H, int D, int T, int n, const int32_t* rows, const uint16_t* x,
                         uint8_t* codes, uint32_t* params, int f32_params) {
    int st = check_shape(0, H, D, n);
    if (st) return st;
    if (T < 1) return ORC_E_ARG;
    st = check_rows(rows, n, T);
    if (st) return st;
    int ntiles = (T + ORC_GROUP - 1) / ORC_GROUP;
    int members[ORC_GROUP];
    float vals[ORC_GROUP];
    uint8_t gc[ORC_GROUP];
    memset(codes, 0, orc_codes_bytes(H, D, n));
    for (int t = 0; t < ntiles; ++t) {
        /* the group's members: every compact row whose position falls in tile t */
        int len = 0;
        for (int j = 0; j < n; ++j)
            if (position_of(rows, j) / ORC_GROUP == t) members[len++] = j;
        for (int h = 0; h < H; ++h)
            for (int c = 0; c < D; ++c) {
                size_t pi = ((size_t)t * (size_t)H + (size_t)h) * (size_t)D + (size_t)c;
                if (len == 0) { params[pi] = 0; continue; }
                for (int i = 0; i < len; ++i) vals[i] = orc_f32_from_bf16(x[xidx(H, D, members[i], h, c)]);
                uint16_t m16, s16;
                st = quantize_group(vals, len, f32_params, &m16, &s16, gc);
                if (st) return st;
                params[pi] = (uint32_t)m16 | ((uint32_t)s16 << 16);
                for (int i = 0; i < len; ++i) put_code(codes, H, D, members[i], h, c, gc[i]);
            }
    }
    return ORC_OK;
}

/* Dequantize tile-grouped K: row j reads the params of the tile holding its position. */
int orc_dequantize_k_tiles(int H, int D, int T, int n, const int32_t* rows, const uint8_t* codes,
                           const uint32_t* params, uint16_t* xhat) {
    int st = check_shape(0, H, D, n);
    if (st) return st;
    if (T < 1) return ORC_E_ARG;
    st = check_rows(rows, n, T);
    if (st) return st;
    for (int j = 0; j < n; ++j) {
        size_t t = (size_t)(position_of(rows, j) / ORC_GROUP);
        for (int h = 0; h < H; ++h)
            for (int c = 0; c < D; ++c)
                xhat[xidx(H, D, j, h, c)] =
                    dequant_one(params[(t * (size_t)H + (size_t)h) * (size_t)D + (size_t)c],
                                get_code(codes, H, D, j, h, c));
    }
    return ORC_OK;
}

/* The quantizer and dequantizer of a stream: K with tile groups when k_tiles != 0, else the
 * grouping of `kind` over the compact rows. */
static int quantize_stream(int kind, int k_tiles, int H, int D, int T, int n, const int32_t* rows,
                           const uint16_t* x, uint8_t* codes, uint32_t* params, int f32_params) {
    if (kind == 0 && k_tiles) return orc_quantize_k_tiles(H, D, T, n, rows, x, codes, params, f32_params);
    return orc_quantize(kind, H, D, n, x, codes, params, f32_params);
}

static int dequantize_stream(int kind, int k_tiles, int H, int D, int T, int n, const int32_t* rows,
                             const uint8_t* codes, const uint32_t* params, uint16_t* xhat) {
    if (kind == 0 && k_tiles) return orc_dequantize_k_tiles(H, D, T, n, rows, codes, params, xhat);
    return orc_dequantize(kind, H, D, n, codes, params, xhat);
}

/* ------------------------------------------------------------------------------------ */
/* Base and cross-loop residuals (RFC section 3.3).                                      */
/* ------------------------------------------------------------------------------------ */

/* X_hat[1] = dequantize(quantize(X[1])) over all T positions (loop 1 is always dense,
 * RFC section 3.1).  Writes the packed base and recon = X_hat[1].  k_tiles selects tile
 * groups for K (a dense stream's tile groups are its compact-row groups). */
int orc_encode_base(int kind, int H, int D, int T, const uint16_t* x, uint8_t* codes,
                    uint32_t* params, uint16_t* recon, int f32_params, int k_tiles) {
    if (T < 1) return ORC_E_ARG;
    int st = quantize_stream(kind, k_tiles, H, D, T, T, NULL, x, codes, params, f32_params);
    if (st) return st;
    return dequantize_stream(kind, k_tiles, H, D, T, T, NULL, codes, params, recon);
}

/* Loop r >= 2.  rows == NULL means dense (n == T, compact row j is position j); otherwise
 * rows holds the n active positions in ascending order (the logical-position-to-compact-
 * row map), and x_rows holds X[r] at those positions only.
 *   delta[j]          = bf16(X[r][j] - X_hat[r-1][rows[j]])      (subtract the RECONSTRUCTED
 *                                                                  predecessor)
 *   delta_hat         = dequantize(quantize(delta))               (K groups over compact j,
 *                                                                  or per tile if k_tiles)
 *   X_hat[r][rows[j]] = bf16(X_hat[r-1][rows[j]] + delta_hat[j])
 *   X_hat[r][p]       = X_hat[r-1][p] for every p not in rows      (absent = inherit)
 * recon holds X_hat[r-1] on entry and X_hat[r] on return.  Subtraction and addition are
 * carried out in binary32 and rounded to BF16, the compute dtype (PR #166 "Purpose").  */
int orc_encode_residual(int kind, int H, int D, int T, int n, const int32_t* rows,
                        const uint16_t* x_rows, uint16_t* recon, uint8_t* codes, uint32_t* params,
                        int f32_params, int k_tiles) {
    int st = check_shape(kind, H, D, n);
    if (st) return st;
    st = check_rows(rows, n, T);
    if (st) return st;
    size_t W = (size_t)H * (size_t)D;
    uint16_t* delta = (uint16_t*)malloc(((size_t)n * W + 1) * sizeof(uint16_t));
    uint16_t* dhat = (uint16_t*)malloc(((size_t)n * W + 1) * sizeof(uint16_t));
    if (!delta || !dhat) { free(delta); free(dhat); return ORC_E_ARG; }
    for (int j = 0; j < n; ++j) {
        int p = rows ? rows[j] : j;
        for (size_t e = 0; e < W; ++e) {
            float a = orc_f32_from_bf16(x_rows[(size_t)j * W + e]);
            float b = orc_f32_from_bf16(recon[(size_t)p * W + e]);
            float d = a - b;
            delta[(size_t)j * W + e] = orc_bf16_from_f32(d);
        }
    }
    st = quantize_stream(kind, k_tiles, H, D, T, n, rows, delta, codes, params, f32_params);
    if (!st) st = dequantize_stream(kind, k_tiles, H, D, T, n, rows, codes, params, dhat);
    if (!st) {
        for (int j = 0; j < n; ++j) {
            int p = rows ? rows[j] : j;
            for (size_t e = 0; e < W; ++e) {
                float a = orc_f32_from_bf16(recon[(size_t)p * W + e]);
                float b = orc_f32_from_bf16(dhat[(size_t)j * W + e]);
                float s = a + b;
                recon[(size_t)p * W + e] = orc_bf16_from_f32(s);
            }
        }
    }
    free(delta);
    free(dhat);
    return st;
}

/* Rebuild X_hat[R] from the packed streams alone (never from X): decode the base, then for
 * each later loop in order add its decoded residual at the positions it covers; positions
 * a loop does not cover keep their value (RFC section 3.3: t1 resolves to base + delta2,
 * t2 to base + delta2 + delta3, t4 to base + delta2 + delta3 + delta4).
 * Stream l (0 = base) has n_rows[l] rows, rows_list[l] (NULL = dense), codes and params. */
int orc_reconstruct(int kind, int H, int D, int T, int n_loops, const int32_t* n_rows,
                    const int32_t* const* rows_list, const uint8_t* const* codes_list,
                    const uint32_t* const* params_list, uint16_t* out, int k_tiles) {
    int st = check_shape(kind, H, D, T);
    if (st) return st;
    if (T < 1 || n_loops < 1 || n_rows[0] != T || rows_list[0] != NULL) return ORC_E_ARG;
    size_t W = (size_t)H * (size_t)D;
    st = dequantize_stream(kind, k_tiles, H, D, T, T, NULL, codes_list[0], params_list[0], out);
    if (st) return st;
    for (int l = 1; l < n_loops; ++l) {
        int n = n_rows[l];
        const int32_t* rows = rows_list[l];
        st = check_rows(rows, n, T);
        if (st) return st;
        uint16_t* dhat = (uint16_t*)malloc(((size_t)n * W + 1) * sizeof(uint16_t));
        if (!dhat) return ORC_E_ARG;
        st = dequantize_stream(kind, k_tiles, H, D, T, n, rows, codes_list[l], params_list[l], dhat);
        if (st) { free(dhat); return st; }
        for (int j = 0; j < n; ++j) {
            int p = rows ? rows[j] : j;
            for (size_t e = 0; e < W; ++e) {
                float a = orc_f32_from_bf16(out[(size_t)p * W + e]);
                float b = orc_f32_from_bf16(dhat[(size_t)j * W + e]);
                float s = a + b;
                out[(size_t)p * W + e] = orc_bf16_from_f32(s);
            }
        }
        free(dhat);
    }
    return ORC_OK;
}

/* The inverse position map at 64-position granularity (RFC section 3.3: explicit
 * logical-position-to-compact-row mappings): out[t] = number of rows < 64*t, for
 * t = 0 .. ceil(T/64).  Written as the definition, a count per tile. */
int orc_tile_index(const int32_t* rows, int n, int T, int32_t* out) {
    if (n < 0 || T < 1) return ORC_E_ARG;
    int ntiles = (T + ORC_GROUP - 1) / ORC_GROUP;
    for (int t = 0; t <= ntiles; ++t) {
        int32_t count = 0;
        for (int j = 0; j < n; ++j)
            if (rows[j] < (int64_t)ORC_GROUP * t) ++count;
        out[t] = count;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------------------------ */
/* Decode attention over reconstructed K/V (the consumer the RFC describes in section     */
/* 3.3's last paragraph and section 3.2: historical K/V "at the requested depth,          */
/* reconstructed if compressed").  Textbook single-query softmax attention in binary64.  */
/* ------------------------------------------------------------------------------------ */

/* q: [Hq, D] BF16.  khat, vhat: [T, Hkv, D] BF16.  Query head i reads KV head
 * i / (Hq / Hkv) (grouped-query attention).  out: [Hq, D] binary64.                      */
int orc_decode_attn(int Hq, int Hkv, int D, int T, const uint16_t* q, const uint16_t* khat,
                    const uint16_t* vhat, double softmax_scale, double* out) {
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || T <= 0 || D <= 0) return ORC_E_ARG;
    int group = Hq / Hkv;
    double* s = (double*)malloc((size_t)T * sizeof(double));
    if (!s) return ORC_E_ARG;
    for (int i = 0; i < Hq; ++i) {
        int h = i / group;
        double smax = -INFINITY;
        for (int t = 0; t < T; ++t) {
            double acc = 0.0;
            for (int c = 0; c < D; ++c)
                acc += (double)orc_f32_from_bf16(q[(size_t)i * D + c]) *
                       (double)orc_f32_from_bf16(khat[xidx(Hkv, D, t, h, c)]);
            s[t] = softmax_scale * acc;
            if (s[t] > smax) smax = s[t];
        }
        double denom = 0.0;
        for (int t = 0; t < T; ++t) { s[t] = exp(s[t] - smax); denom += s[t]; }
        for (int c = 0; c < D; ++c) {
            double acc = 0.0;
            for (int t = 0; t < T; ++t) acc += s[t] * (double)orc_f32_from_bf16(vhat[xidx(Hkv, D, t, h, c)]);
            out[(size_t)i * D + c] = acc / denom;
        }
    }
    free(s);
    return ORC_OK;
}

/* ------------------------------------------------------------------------------------ */
/* Sparse decode attention (RFC section 3.2 "Sparse decode attention").  Loop 2 is the    */
/* reference: full attention over the keys at that depth, keeping per query head the     */
/* selected positions S (the k highest reference probabilities), their mass m, the full   */
/* output O_ref and the selected keys' weighted value sum C_ref.  A later loop r attends  */
/* to the keys of S alone at depth r and corrects the reference output:                  */
/*   p_local = softmax(scale * q_r . K_r[S]),  C_new = m * (p_local . V_r[S]),            */
/*   O_r = O_ref - C_ref + C_new.                                                          */
/* Everything here is binary64.  Selection orders keys by reference score (the            */
/* probabilities are a monotone function of it), higher first, equal scores by the lower  */
/* position; S is returned in ascending position order.                                   */
/* ------------------------------------------------------------------------------------ */

static const double* g_sort_scores;   /* qsort has no context argument */

static int by_score_then_position(const void* a, const void* b) {
    int32_t i = *(const int32_t*)a, j = *(const int32_t*)b;
    double si = g_sort_scores[i], sj = g_sort_scores[j];
    if (si > sj) return -1;
    if (si < sj) return 1;
    return (i < j) ? -1 : (i > j);
}

static int by_position(const void* a, const void* b) {
    int32_t i = *(const int32_t*)a, j = *(const int32_t*)b;
    return (i < j) ? -1 : (i > j);
}

/* The reference statistics from probabilities p [T] and values v [T, D] (rows of one head):
 * O_ref = sum_t p_t v_t, and over the selected positions sel [k]: m = sum p_t,
 * C_ref = sum p_t v_t. */
int orc_sparse_stats(int T, int D, const double* p, const double* v, int k, const int32_t* sel, double* m,
                     double* o_ref, double* c_ref) {
    if (T <= 0 || D <= 0 || k < 1 || k > T) return ORC_E_ARG;
    for (int c = 0; c < D; ++c) {
        double acc = 0.0;
        for (int t = 0; t < T; ++t) acc += p[t] * v[(size_t)t * D + c];
        o_ref[c] = acc;
        c_ref[c] = 0.0;
    }
    double mm = 0.0;
    for (int r = 0; r < k; ++r) {
        int t = sel[r];
        if (t < 0 || t >= T) return ORC_E_ARG;
        mm += p[t];
        for (int c = 0; c < D; ++c) c_ref[c] += p[t] * v[(size_t)t * D + c];
    }
    *m = mm;
    return ORC_OK;
}

/* The correction of a later loop from its probabilities over the selected keys p_local [k]
 * and their values v_sel [k, D]: out = O_ref - C_ref + m * sum_r p_local_r v_sel_r. */
int orc_sparse_correct(int k, int D, const double* p_local, const double* v_sel, double m, const double* o_ref,
                       const double* c_ref, double* out) {
    if (k < 1 || D <= 0) return ORC_E_ARG;
    for (int c = 0; c < D; ++c) {
        double acc = 0.0;
        for (int r = 0; r < k; ++r) acc += p_local[r] * v_sel[(size_t)r * D + c];
        out[c] = o_ref[c] - c_ref[c] + m * acc;
    }
    return ORC_OK;
}

/* Scaled scores of one query head against every key of its KV head, and their softmax. */
static void head_softmax(int Hkv, int D, const uint16_t* qi, const uint16_t* khat, int h, double scale,
                         const int32_t* keys, int n, double* sc, double* p) {
    double smax = -INFINITY;
    for (int r = 0; r < n; ++r) {
        int t = keys ? keys[r] : r;
        double acc = 0.0;
        for (int c = 0; c < D; ++c)
            acc += (double)orc_f32_from_bf16(qi[c]) * (double)orc_f32_from_bf16(khat[xidx(Hkv, D, t, h, c)]);
        sc[r] = scale * acc;
        if (sc[r] > smax) smax = sc[r];
    }
    double denom = 0.0;
    for (int r = 0; r < n; ++r) { p[r] = exp(sc[r] - smax); denom += p[r]; }
    for (int r = 0; r < n; ++r) p[r] /= denom;
}

/* Values of the given keys of one KV head as binary64 rows [n, D]. */
static void head_values(int Hkv, int D, const uint16_t* vhat, int h, const int32_t* keys, int n, double* out) {
    for (int r = 0; r < n; ++r) {
        int t = keys ? keys[r] : r;
        for (int c = 0; c < D; ++c) out[(size_t)r * D + c] = (double)orc_f32_from_bf16(vhat[xidx(Hkv, D, t, h, c)]);
    }
}

/* The k keys with the highest scores, equal scores by the lower position, in position order. */
int orc_topk_positions(int T, const double* scores, int k, int32_t* sel) {
    if (T <= 0 || k < 1 || k > T) return ORC_E_ARG;
    int32_t* order = (int32_t*)malloc((size_t)T * sizeof(int32_t));
    if (!order) return ORC_E_ARG;
    for (int t = 0; t < T; ++t) order[t] = t;
    g_sort_scores = scores;
    qsort(order, (size_t)T, sizeof(int32_t), by_score_then_position);
    qsort(order, (size_t)k, sizeof(int32_t), by_position);
    memcpy(sel, order, (size_t)k * sizeof(int32_t));
    free(order);
    return ORC_OK;
}

/* Reference loop.  q: [Hq, D] BF16; khat, vhat: [T, Hkv, D] BF16 at the reference depth; k keys
 * kept per query head (1 <= k <= T).  Outputs: sel [Hq, k] ascending positions, mass [Hq],
 * o_ref [Hq, D], c_ref [Hq, D]. */
int orc_sparse_reference(int Hq, int Hkv, int D, int T, const uint16_t* q, const uint16_t* khat,
                         const uint16_t* vhat, double scale, int k, int32_t* sel, double* mass,
                         double* o_ref, double* c_ref) {
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || T <= 0 || D <= 0 || k < 1 || k > T) return ORC_E_ARG;
    int group = Hq / Hkv, st = ORC_OK;
    double* sc = (double*)malloc((size_t)T * sizeof(double));
    double* p = (double*)malloc((size_t)T * sizeof(double));
    double* v = (double*)malloc((size_t)T * (size_t)D * sizeof(double));
    if (!sc || !p || !v) st = ORC_E_ARG;
    for (int i = 0; i < Hq && st == ORC_OK; ++i) {
        int h = i / group;
        head_softmax(Hkv, D, q + (size_t)i * D, khat, h, scale, NULL, T, sc, p);
        head_values(Hkv, D, vhat, h, NULL, T, v);
        st = orc_topk_positions(T, sc, k, sel + (size_t)i * k);
        if (st == ORC_OK)
            st = orc_sparse_stats(T, D, p, v, k, sel + (size_t)i * k, mass + i, o_ref + (size_t)i * D,
                                  c_ref + (size_t)i * D);
    }
    free(sc);
    free(p);
    free(v);
    return st;
}

/* A later loop: q [Hq, D] BF16 of that loop, khat / vhat [T, Hkv, D] at its depth; sel, mass,
 * o_ref, c_ref from the reference loop.  out [Hq, D] binary64. */
int orc_sparse_loop(int Hq, int Hkv, int D, int T, const uint16_t* q, const uint16_t* khat,
                    const uint16_t* vhat, double scale, int k, const int32_t* sel, const double* mass,
                    const double* o_ref, const double* c_ref, double* out) {
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || T <= 0 || D <= 0 || k < 1 || k > T) return ORC_E_ARG;
    for (size_t r = 0; r < (size_t)Hq * (size_t)k; ++r)
        if (sel[r] < 0 || sel[r] >= T) return ORC_E_ARG;
    int group = Hq / Hkv, st = ORC_OK;
    double* sc = (double*)malloc((size_t)k * sizeof(double));
    double* p = (double*)malloc((size_t)k * sizeof(double));
    double* v = (double*)malloc((size_t)k * (size_t)D * sizeof(double));
    if (!sc || !p || !v) st = ORC_E_ARG;
    for (int i = 0; i < Hq && st == ORC_OK; ++i) {
        int h = i / group;
        const int32_t* keys = sel + (size_t)i * k;
        head_softmax(Hkv, D, q + (size_t)i * D, khat, h, scale, keys, k, sc, p);
        head_values(Hkv, D, vhat, h, keys, k, v);
        st = orc_sparse_correct(k, D, p, v, mass[i], o_ref + (size_t)i * D, c_ref + (size_t)i * D,
                                out + (size_t)i * D);
    }
    free(sc);
    free(p);
    free(v);
    return st;
}

/* Scaled scores of every query head against every key of its KV head: out [Hq, T]. */
int orc_attn_scores(int Hq, int Hkv, int D, int T, const uint16_t* q, const uint16_t* khat, double scale,
                    double* out) {
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || T <= 0 || D <= 0) return ORC_E_ARG;
    int group = Hq / Hkv;
    double* p = (double*)malloc((size_t)T * sizeof(double));
    if (!p) return ORC_E_ARG;
    for (int i = 0; i < Hq; ++i)
        head_softmax(Hkv, D, q + (size_t)i * D, khat, i / group, scale, NULL, T, out + (size_t)i * T, p);
    free(p);
    return ORC_OK;
}

/* The reference statistics for a given selection sel [Hq, k] (parity checks of a selection
 * made elsewhere): mass [Hq], o_ref [Hq, D], c_ref [Hq, D]. */
int orc_sparse_reference_given(int Hq, int Hkv, int D, int T, const uint16_t* q, const uint16_t* khat,
                               const uint16_t* vhat, double scale, int k, const int32_t* sel, double* mass,
                               double* o_ref, double* c_ref) {
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || T <= 0 || D <= 0 || k < 1 || k > T) return ORC_E_ARG;
    int group = Hq / Hkv, st = ORC_OK;
    double* sc = (double*)malloc((size_t)T * sizeof(double));
    double* p = (double*)malloc((size_t)T * sizeof(double));
    double* v = (double*)malloc((size_t)T * (size_t)D * sizeof(double));
    if (!sc || !p || !v) st = ORC_E_ARG;
    for (int i = 0; i < Hq && st == ORC_OK; ++i) {
        int h = i / group;
        head_softmax(Hkv, D, q + (size_t)i * D, khat, h, scale, NULL, T, sc, p);
        head_values(Hkv, D, vhat, h, NULL, T, v);
        st = orc_sparse_stats(T, D, p, v, k, sel + (size_t)i * k, mass + i, o_ref + (size_t)i * D,
                              c_ref + (size_t)i * D);
    }
    free(sc);
    free(p);
    free(v);
    return st;
}
