/*
 * tq_oracle.c -- plain, slow CPU reference for group-wise ternary weight
 * quantization, packing, unpacking and the packed-ternary x bf16 matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library; the two agree only through the data format below.
 *
 * Sources (web pages; cited by title and section):
 *  [P4] precisit "pack-unpack-run" README, the paragraph describing codec.py
 *       (absmean scale rounded to fp16, nearest-even ternary codes, five
 *       base-three digits per byte, per-group byte alignment with zero-trit
 *       padding, byte values 243..255 invalid), the scale-rule paragraph
 *       (no calibration, zero stored scale -> zero group, columns divisible
 *       by the group size) and the payload-rate paragraph.
 *  [P2] tiny-llm "Week 2 Day 3: Quantize the Model", sections
 *       "Mathematical Formulation" and "Computation Flow" (per-group
 *       factoring of the scale out of the inner sum; fp32-or-wider
 *       accumulator per output element); for the W4A16 functions at the
 *       end also "Group-Wise Affine Quantization", "Reconstruct a Stored
 *       Group" and "Packed Storage Layout".
 *
 * Readings where the pages leave a step open (all listed in the design doc):
 *  - digit = code + 1 and the first weight of five is the least significant
 *    base-3 digit:  byte = sum_i (c[5b+i] + 1) * 3^i.
 *  - padding trits (positions >= G in a group's last byte) hold code 0.
 *  - scale = one round-to-nearest-even to fp16 of the EXACT mean of |w|
 *    (exact integer sum of the bf16 magnitudes, then one rounding).
 *  - code = +1 if w > s/2, -1 if w < -s/2, else 0 (|w| == s/2 -> 0).
 *  - non-finite weight in a group: status NONFINITE, scale 0x7E00, codes 0.
 *  - mean that rounds to >= 65520: status SCALE_OVERFLOW, scale 0x7C00,
 *    codes 0.
 *  - unpack: byte >= 243 -> INVALID_BYTE and code 0 for that byte's
 *    positions; a padding trit that is not code 0 -> BAD_PADDING.
 *
 * Everything here is scalar C.  Floating-point matmul is done in fp64:
 * every product x*c*s is exact in fp64 (bf16 x fp16 significands need 19
 * bits), so only the order of the fp64 sum rounds.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stddef.h>
#include <stdlib.h>
#include <string.h>

/* Return codes (same numeric values as the library's host-side codes). */
#define OR_OK          0
#define OR_ERR_NULL   -1
#define OR_ERR_SHAPE  -2

/* Status bits OR-ed into *status (same values as the library's device bits). */
#define OR_NONFINITE       1
#define OR_SCALE_OVERFLOW  2
#define OR_INVALID_BYTE    4
#define OR_BAD_PADDING     8

/* ------------------------------------------------------------------------ */
/* Sizes                                                                      */
/* ------------------------------------------------------------------------ */

/* Bytes per group: ceil(G/5) base-3 bytes ([P4] codec.py description). */
static int64_t bytes_per_group(int64_t G) { return (G + 4) / 5; }

/* Packed bytes of one row of K weights; 0 if the arguments are invalid. */
int64_t oracle_packed_row_bytes(int64_t K, int64_t G)
{
    if (K < 1 || G < 1 || K % G != 0) return 0;
    return (K / G) * bytes_per_group(G);
}

static int check_shape(int64_t N, int64_t K, int64_t G)
{
    if (N < 1 || K < 1 || G < 1) return OR_ERR_SHAPE;
    if (K % G != 0) return OR_ERR_SHAPE;  /* [P4] scale-rule paragraph */
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* A small unsigned big integer: 8 little-endian 64-bit limbs (512 bits).    */
/* The exact sum of G bf16 magnitudes is below G * 2^261, so 512 bits hold   */
/* it for any G below 2^250.                                                  */
/* ------------------------------------------------------------------------ */

#define NLIMB 8
typedef struct { uint64_t w[NLIMB]; } big_t;

static void big_zero(big_t *a) { memset(a, 0, sizeof *a); }

static int big_is_zero(const big_t *a)
{
    for (int i = 0; i < NLIMB; ++i) if (a->w[i]) return 0;
    return 1;
}

/* a += v * 2^sh, with v < 2^64. */
static void big_add_shifted(big_t *a, uint64_t v, int sh)
{
    int limb = sh / 64, off = sh % 64;
    uint64_t lo = v << off;
    uint64_t hi = off ? (v >> (64 - off)) : 0;
    uint64_t carry = 0;
    for (int i = limb; i < NLIMB; ++i) {
        uint64_t add = (i == limb) ? lo : (i == limb + 1) ? hi : 0;
        uint64_t s = a->w[i] + add;
        uint64_t c1 = s < add;
        uint64_t s2 = s + carry;
        uint64_t c2 = s2 < s;
        a->w[i] = s2;
        carry = c1 + c2;
        if (i > limb + 1 && carry == 0) break;
    }
}

/* Bit number i of a. */
static int big_bit(const big_t *a, int i)
{
    if (i < 0 || i >= 64 * NLIMB) return 0;
    return (int)((a->w[i / 64] >> (i % 64)) & 1u);
}

/* 1 if any bit below position n is set. */
static int big_any_below(const big_t *a, int n)
{
    for (int i = 0; i < n && i < 64 * NLIMB; ++i) if (big_bit(a, i)) return 1;
    return 0;
}

/* q = a >> n (floor). */
static void big_shr(const big_t *a, int n, big_t *q)
{
    big_zero(q);
    for (int i = n; i < 64 * NLIMB; ++i)
        if (big_bit(a, i)) q->w[(i - n) / 64] |= (uint64_t)1 << ((i - n) % 64);
}

/* q = floor(a / d), returns a mod d; d >= 1 and d < 2^32. */
static uint64_t big_divmod_small(const big_t *a, uint64_t d, big_t *q)
{
    big_zero(q);
    uint64_t rem = 0;
    for (int i = 64 * NLIMB - 1; i >= 0; --i) {
        rem = (rem << 1) | (uint64_t)big_bit(a, i);
        if (rem >= d) {
            rem -= d;
            q->w[i / 64] |= (uint64_t)1 << (i % 64);
        }
    }
    return rem;
}

/* -1, 0, +1 as a <, ==, > (G * 2^n). */
static int big_cmp_g_pow2(const big_t *a, uint64_t G, int n)
{
    big_t b;
    big_zero(&b);
    big_add_shifted(&b, G, n);
    for (int i = NLIMB - 1; i >= 0; --i) {
        if (a->w[i] > b.w[i]) return 1;
        if (a->w[i] < b.w[i]) return -1;
    }
    return 0;
}

/*
 * Round-half-even of the rational a / (G * 2^n) to an integer, for results
 * that fit in 64 bits.  Written as: a / 2^n = A + f with integer A and
 * fraction f in [0,1); A = G*q + r; the exact quotient is q + (r + f)/G and
 * the decision compares (r + f)/G with 1/2.
 */
static uint64_t big_rne_div(const big_t *a, uint64_t G, int n)
{
    big_t A, Q;
    big_shr(a, n, &A);
    uint64_t r = big_divmod_small(&A, G, &Q);
    uint64_t q = Q.w[0];
    /* f compared with 1/2: sign of (f - 1/2) and whether f > 0. */
    int f_pos = big_any_below(a, n);
    int f_cmp_half;                       /* -1: f < 1/2, 0: f == 1/2, 1: f > 1/2 */
    if (n == 0) f_cmp_half = -1;          /* f == 0 */
    else if (!big_bit(a, n - 1)) f_cmp_half = -1;
    else f_cmp_half = big_any_below(a, n - 1) ? 1 : 0;

    /* 2(r + f) compared with G. */
    int up;
    if (2 * r + 2 <= G) up = 0;                         /* 2r + 2f < G     */
    else if (2 * r > G) up = 1;                         /* 2r >= G + 1     */
    else if (2 * r == G) up = f_pos ? 1 : (int)(q & 1); /* exact tie if f=0 */
    else /* 2r == G - 1 */ up = (f_cmp_half > 0) ? 1 : (f_cmp_half == 0 ? (int)(q & 1) : 0);
    return q + (uint64_t)up;
}

/* ------------------------------------------------------------------------ */
/* group scale                                                                */
/* ------------------------------------------------------------------------ */

/*
 * bf16 magnitude bits u (sign cleared, finite) as sig * 2^(e - 133) with an
 * integer significand sig <= 255 and e >= 0:
 *   normal    (E = u>>7 in 1..254): value = (128 + m) * 2^(E - 134)
 *   subnormal (E = 0):              value = m * 2^-133
 */
static void bf16_mag_parts(uint16_t u, uint64_t *sig, int *e)
{
    int E = (u >> 7) & 0xFF;
    int m = u & 0x7F;
    if (E == 0) { *sig = (uint64_t)m; *e = 0; }
    else        { *sig = (uint64_t)(128 + m); *e = E - 1; }
}

/*
 * Scale of one group ([P4] codec.py description and scale-rule paragraph):
 * the mean of |w| over the G weights, rounded once to fp16 with ties to
 * even.  The sum is exact: sum |w| = A * 2^-133 with A an integer.
 *
 * In units of the fp16 subnormal step 2^-24 the mean is V = A / (G * 2^109).
 *   V < 1024:  subnormal (or the smallest normal if it rounds up to 1024);
 *              fp16 bits = RNE(V).
 *   else:      V in [2^(10+k), 2^(11+k)) for some k >= 0; the fp16 value is
 *              Q * 2^k with Q = RNE(V / 2^k) in [1024, 2048], whose bits are
 *              (k << 10) + Q (a carry to 2048 moves into the exponent).
 * Returns the status bits of the group (0 or OR_SCALE_OVERFLOW).
 */
static int scale_bits_of_sum(const big_t *A, int64_t G, int sh, uint16_t *out_bits)
{
    if (big_is_zero(A)) { *out_bits = 0; return 0; }

    uint64_t bits;
    if (big_cmp_g_pow2(A, (uint64_t)G, sh + 10) < 0) {
        bits = big_rne_div(A, (uint64_t)G, sh);            /* 0 .. 1024 */
    } else {
        int k = 0;
        /* smallest k with V < 2^(11+k); past k = 29 the result overflows */
        while (k < 40 && big_cmp_g_pow2(A, (uint64_t)G, sh + 11 + k) >= 0) ++k;
        if (k >= 30) { *out_bits = 0x7C00; return OR_SCALE_OVERFLOW; }
        uint64_t Q = big_rne_div(A, (uint64_t)G, sh + k);  /* 1024 .. 2048 */
        bits = ((uint64_t)k << 10) + Q;
    }
    if (bits >= 0x7C00) { *out_bits = 0x7C00; return OR_SCALE_OVERFLOW; }
    *out_bits = (uint16_t)bits;
    return 0;
}

static int group_scale_bits(const uint16_t *w, int64_t G, uint16_t *out_bits)
{
    big_t A;
    big_zero(&A);
    for (int64_t j = 0; j < G; ++j) {
        uint64_t sig; int e;
        bf16_mag_parts((uint16_t)(w[j] & 0x7FFF), &sig, &e);
        big_add_shifted(&A, sig, e);
    }
    /* A counts units of 2^-133; V = A / (G * 2^109) in units of 2^-24 */
    return scale_bits_of_sum(&A, G, 109, out_bits);
}

/* ------------------------------------------------------------------------ */
/* Plain conversions to double (exact)                                        */
/* ------------------------------------------------------------------------ */

/* bf16 bits -> double, exact; non-finite inputs are not passed here. */
static double bf16_to_double(uint16_t b)
{
    uint64_t sig; int e;
    bf16_mag_parts((uint16_t)(b & 0x7FFF), &sig, &e);
    double v = ldexp((double)sig, e - 133);
    return (b & 0x8000) ? -v : v;
}

/* fp16 bits -> double, exact; finite inputs only. */
static double f16_to_double(uint16_t h)
{
    int E = (h >> 10) & 0x1F;
    int m = h & 0x3FF;
    double v = (E == 0) ? ldexp((double)m, -24) : ldexp((double)(1024 + m), E - 25);
    return (h & 0x8000) ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* quantize + pack                                                           */
/* ------------------------------------------------------------------------ */

/*
 * Scale and codes of one group of G weights: sets *sbits and code[0, npad)
 * (code[j] = 0 for j >= G), returns the group's status bits.  A group with
 * an Inf/NaN weight gets scale 0x7E00, one whose mean overflows fp16 gets
 * 0x7C00; both keep every code at 0.
 */
static int group_scale_and_codes(const uint16_t *wg, int64_t G, int64_t npad, uint16_t *sbits,
                                 int8_t *code)
{
    int gst = 0;
    *sbits = 0;
    for (int64_t j = 0; j < G; ++j)
        if (((wg[j] >> 7) & 0xFF) == 0xFF) gst |= OR_NONFINITE;
    if (gst) *sbits = 0x7E00;
    else gst |= group_scale_bits(wg, G, sbits);

    /* Codes.  |w| == s/2 is a tie and goes to 0 (round half to even of
     * +-0.5); beyond 1.5 s the code saturates at +-1. */
    for (int64_t t = 0; t < npad; ++t) code[t] = 0;  /* padding = 0 */
    if (!gst) {
        double half = 0.5 * f16_to_double(*sbits);
        for (int64_t j = 0; j < G; ++j) {
            double v = bf16_to_double(wg[j]);
            code[j] = (int8_t)(v > half ? 1 : (v < -half ? -1 : 0));
        }
    }
    return gst;
}

/*
 * w[N,K] bf16 bits, row-major; groups of G along K.
 * packed[N][K/G][ceil(G/5)] bytes, scales[N][K/G] fp16 bits.
 * *status receives the OR of all group status bits (may be NULL).
 */
int oracle_quantize_pack(const uint16_t *w, int64_t N, int64_t K, int64_t G,
                         uint8_t *packed, uint16_t *scales, int32_t *status)
{
    if (!w || !packed || !scales) return OR_ERR_NULL;
    int rc = check_shape(N, K, G);
    if (rc) return rc;
    const int64_t nG = K / G, B = bytes_per_group(G);
    int32_t st = 0;
    int8_t *code = (int8_t *)__builtin_alloca((size_t)(5 * B));

    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < nG; ++g) {
            const uint16_t *wg = w + n * K + g * G;
            uint8_t *pg = packed + (n * nG + g) * B;
            uint16_t sbits;
            int gst = group_scale_and_codes(wg, G, 5 * B, &sbits, code);

            /* Five base-3 digits per byte, first weight lowest digit. */
            for (int64_t b = 0; b < B; ++b) {
                int byte = 0, p3 = 1;
                for (int i = 0; i < 5; ++i) {
                    byte += (code[5 * b + i] + 1) * p3;
                    p3 *= 3;
                }
                pg[b] = (uint8_t)byte;
            }
            scales[n * nG + g] = sbits;
            st |= gst;
        }
    }
    if (status) *status |= st;
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* unpack                                                                     */
/* ------------------------------------------------------------------------ */

/* packed -> codes[N,K] int8 in {-1,0,1}. */
int oracle_unpack(const uint8_t *packed, int64_t N, int64_t K, int64_t G,
                  int8_t *codes, int32_t *status)
{
    if (!packed || !codes) return OR_ERR_NULL;
    int rc = check_shape(N, K, G);
    if (rc) return rc;
    const int64_t nG = K / G, B = bytes_per_group(G);
    int32_t st = 0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < nG; ++g) {
            const uint8_t *pg = packed + (n * nG + g) * B;
            int8_t *cg = codes + n * K + g * G;
            for (int64_t b = 0; b < B; ++b) {
                int v = pg[b];
                int valid = v < 243;
                if (!valid) st |= OR_INVALID_BYTE;
                for (int i = 0; i < 5; ++i) {
                    int d = v % 3;
                    v /= 3;
                    int64_t pos = 5 * b + i;
                    if (pos < G) cg[pos] = (int8_t)(valid ? d - 1 : 0);
                    else if (valid && d != 1) st |= OR_BAD_PADDING;
                }
            }
        }
    }
    if (status) *status |= st;
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* decode to bf16                                                             */
/* ------------------------------------------------------------------------ */

/* Nearest bf16 to a finite double, ties to even (sign kept, zero kept as
 * +-0).  Only reached with |v| in the fp16 range, which lies inside bf16's
 * normal range, so there is no subnormal or overflow case. */
static uint16_t double_to_bf16_rne(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    int e;
    double m = frexp(a, &e);          /* a = m * 2^e, 0.5 <= m < 1 */
    double q = ldexp(m, 8);           /* 128 <= q < 256: 8 significant bits */
    double r = floor(q);
    double frac = q - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    if (r == 256.0) { r = 128.0; e += 1; }
    int E = e - 1 + 127;              /* a = (r / 128) * 2^(e - 1) */
    return (uint16_t)(sign | (uint16_t)(E << 7) | (uint16_t)((int)r - 128));
}

/*
 * out[n,k] = bf16_RNE(c[n,k] * s[n,k/G]) as bf16 bits ([P4] codec.py
 * description: decoding gives back c * s; screen.py description: the decoder
 * hands the selected weights back as bf16).  c comes from the bytes exactly as in
 * oracle_unpack (an invalid byte gives code 0 at its five positions and sets
 * INVALID_BYTE; a padding trit other than code 0 sets BAD_PADDING).  The
 * product is the IEEE one: c = 0 gives a zero with the sign of s, c = -1
 * negates.  A non-finite scale sets NONFINITE; its group's outputs are then
 * not defined here (they are written as 0).
 */
int oracle_dequantize(const uint8_t *packed, const uint16_t *scales, int64_t N, int64_t K,
                      int64_t G, uint16_t *out, int32_t *status)
{
    if (!packed || !scales || !out) return OR_ERR_NULL;
    int rc = check_shape(N, K, G);
    if (rc) return rc;
    const int64_t nG = K / G;
    int8_t *codes = (int8_t *)malloc((size_t)(N * K));
    if (!codes) return OR_ERR_NULL;
    int32_t st = 0;
    rc = oracle_unpack(packed, N, K, G, codes, &st);
    if (rc) { free(codes); return rc; }
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < nG; ++g) {
            uint16_t sb = scales[n * nG + g];
            int finite = ((sb >> 10) & 0x1F) != 0x1F;
            if (!finite) st |= OR_NONFINITE;
            double s = finite ? f16_to_double(sb) : 0.0;
            for (int64_t j = 0; j < G; ++j) {
                int64_t k = g * G + j;
                double v = (double)codes[n * K + k] * s;  /* exact */
                out[n * K + k] = finite ? double_to_bf16_rne(v) : 0;
            }
        }
    }
    free(codes);
    if (status) *status |= st;
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* fake quantization (QAT forward)                                           */
/* ------------------------------------------------------------------------ */

/*
 * w_hat[n,k] = bf16_RNE(c[n,k] * s[n,k/G]) straight from bf16 weights, with
 * s and c the group scale and codes above.  Avenue README, introduction and
 * closing remarks: BitNet-style quantization-aware training keeps latent
 * weights.  Reading taken here: the forward pass uses w_hat, and the
 * backward pass is straight-through (the gradient of w_hat is the gradient
 * of w), so the backward needs no arithmetic.  A
 * flagged group (non-finite weight, scale overflow) gives w_hat = +0 and
 * its status bits; scales[N][K/G] receives the scales as quantize_pack
 * would store them (may be NULL).
 */
int oracle_fake_quantize(const uint16_t *w, int64_t N, int64_t K, int64_t G, uint16_t *w_hat,
                         uint16_t *scales, int32_t *status)
{
    if (!w || !w_hat) return OR_ERR_NULL;
    int rc = check_shape(N, K, G);
    if (rc) return rc;
    const int64_t nG = K / G;
    int32_t st = 0;
    int8_t *code = (int8_t *)malloc((size_t)G);
    if (!code) return OR_ERR_NULL;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < nG; ++g) {
            uint16_t sbits;
            int gst = group_scale_and_codes(w + n * K + g * G, G, G, &sbits, code);
            double s = gst ? 0.0 : f16_to_double(sbits);
            for (int64_t j = 0; j < G; ++j)
                w_hat[n * K + g * G + j] = gst ? 0 : double_to_bf16_rne((double)code[j] * s);
            if (scales) scales[n * nG + g] = sbits;
            st |= gst;
        }
    }
    free(code);
    if (status) *status |= st;
    return OR_OK;
}

/*
 * The same forward from fp32 latent weights (Avenue README, introduction:
 * BitNet-style training keeps latent full-precision weights).  Reading
 * taken here: the scale is the exact mean of the fp32 magnitudes rounded
 * once to fp16, the codes compare the fp32 weights with s/2 exactly (ties
 * to 0), and the output is c * s in fp32, which is exact (no rounding).
 * Flags as above; a flagged group gives w_hat = +0.
 *
 * fp32 magnitude bits u (sign cleared, finite) as sig * 2^(e - 149):
 *   normal    (E = u>>23 in 1..254): value = (2^23 + m) * 2^(E - 150)
 *   subnormal (E = 0):               value = m * 2^-149
 * The exact sum of G magnitudes is below G * 2^277 units, so the 512-bit
 * integer holds it for any G below 2^234.
 */
static void f32_mag_parts(uint32_t u, uint64_t *sig, int *e)
{
    int E = (int)((u >> 23) & 0xFF);
    uint64_t m = u & 0x7FFFFFu;
    if (E == 0) { *sig = m; *e = 0; }
    else        { *sig = (1ull << 23) + m; *e = E - 1; }
}

static double f32_to_double(uint32_t b)
{
    uint64_t sig; int e;
    f32_mag_parts(b & 0x7FFFFFFFu, &sig, &e);
    double v = ldexp((double)sig, e - 149);
    return (b & 0x80000000u) ? -v : v;
}

int oracle_fake_quantize_f32(const uint32_t *w, int64_t N, int64_t K, int64_t G,
                             uint32_t *w_hat, uint16_t *scales, int32_t *status)
{
    if (!w || !w_hat) return OR_ERR_NULL;
    int rc = check_shape(N, K, G);
    if (rc) return rc;
    const int64_t nG = K / G;
    int32_t st = 0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < nG; ++g) {
            const uint32_t *wg = w + n * K + g * G;
            uint16_t sbits = 0;
            int gst = 0;
            for (int64_t j = 0; j < G; ++j)
                if (((wg[j] >> 23) & 0xFF) == 0xFF) gst |= OR_NONFINITE;
            if (gst) {
                sbits = 0x7E00;
            } else {
                big_t A;
                big_zero(&A);
                for (int64_t j = 0; j < G; ++j) {
                    uint64_t sig; int e;
                    f32_mag_parts(wg[j] & 0x7FFFFFFFu, &sig, &e);
                    big_add_shifted(&A, sig, e);
                }
                /* A counts units of 2^-149; V = A / (G * 2^125) in units of 2^-24 */
                gst = scale_bits_of_sum(&A, G, 125, &sbits);
            }
            const double s = gst ? 0.0 : f16_to_double(sbits);
            for (int64_t j = 0; j < G; ++j) {
                float out = 0.0f;
                if (!gst) {
                    double v = f32_to_double(wg[j]);
                    double c = v > 0.5 * s ? 1.0 : (v < -0.5 * s ? -1.0 : 0.0);
                    out = (float)(c * s);  /* exact: s is an fp16 value */
                }
                uint32_t ob;
                memcpy(&ob, &out, sizeof ob);
                w_hat[n * K + g * G + j] = ob;
            }
            if (scales) scales[n * nG + g] = sbits;
            st |= gst;
        }
    }
    if (status) *status |= st;
    return OR_OK;
}

/* ------------------------------------------------------------------------ */
/* matmul in fp64                                                             */
/* ------------------------------------------------------------------------ */

/*
 * y[m,n] = sum_k x[m,k] * c[n,k] * s[n, k/G], summed in fp64 in k order
 * ([P2] "Mathematical Formulation": the group scale multiplies the group's
 * inner sum; here every term is formed exactly instead).
 * bound[m,n] = sum_k |x[m,k] * c[n,k] * s[n, k/G]| (may be NULL).
 * x: [M,K] bf16 bits (finite).  Invalid bytes decode to code 0 and set
 * INVALID_BYTE.  Non-finite scales (never produced by the packer for a
 * valid group) are passed through as IEEE values.
 */
int oracle_unpack2(const uint8_t *packed, int64_t N, int64_t K, int64_t G, int8_t *codes,
                   int32_t *status);

/* y = x * W_hat^T over rows decoded from the base-3 format (two_bit = 0) or
 * the 2-bit format (two_bit = 1), for the weight rows n0 <= n < n1 (every
 * output y[m][n] is computed on its own, so any split of the rows gives the
 * same values). */
static int matmul_rows(const uint16_t *x, const uint8_t *packed, const uint16_t *scales,
                       int64_t M, int64_t N, int64_t K, int64_t G, int two_bit,
                       int64_t n0, int64_t n1, double *y, double *bound, int32_t *status)
{
    if (!x || !packed || !scales || !y) return OR_ERR_NULL;
    if (M < 1) return OR_ERR_SHAPE;
    int rc = check_shape(N, K, G);
    if (rc) return rc;
    if (two_bit && G % 4) return OR_ERR_SHAPE;
    const int64_t nG = K / G;
    int8_t *crow = (int8_t *)malloc((size_t)K);
    double *wrow = (double *)malloc((size_t)K * sizeof(double));
    double *xd = (double *)malloc((size_t)(M * K) * sizeof(double));
    if (!crow || !wrow || !xd) { free(crow); free(wrow); free(xd); return OR_ERR_NULL; }
    for (int64_t i = 0; i < M * K; ++i) xd[i] = bf16_to_double(x[i]);
    int32_t st = 0;

    for (int64_t n = n0; n < n1; ++n) {
        /* decode row n: w_hat = c * s */
        int32_t rst = 0;
        if (two_bit) oracle_unpack2(packed + n * (K / 4), 1, K, G, crow, &rst);
        else oracle_unpack(packed + n * oracle_packed_row_bytes(K, G), 1, K, G, crow, &rst);
        st |= rst & OR_INVALID_BYTE;
        for (int64_t g = 0; g < nG; ++g) {
            uint16_t h = scales[n * nG + g];
            double s;
            if (((h >> 10) & 0x1F) == 0x1F)  /* inf / NaN scale */
                s = (h & 0x3FF) ? NAN : ((h & 0x8000) ? -INFINITY : INFINITY);
            else
                s = f16_to_double(h);
            for (int64_t j = 0; j < G; ++j) wrow[g * G + j] = (double)crow[g * G + j] * s;
        }
        for (int64_t m = 0; m < M; ++m) {
            const double *xm = xd + m * K;
            double acc = 0.0, bacc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double t = xm[k] * wrow[k];
                acc += t;
                bacc += fabs(t);
            }
            y[m * N + n] = acc;
            if (bound) bound[m * N + n] = bacc;
        }
    }
    free(crow); free(wrow); free(xd);
    if (status) *status |= st;
    return OR_OK;
}

int oracle_matmul(const uint16_t *x, const uint8_t *packed, const uint16_t *scales,
                  int64_t M, int64_t N, int64_t K, int64_t G,
                  double *y, double *bound, int32_t *status)
{
    return matmul_rows(x, packed, scales, M, N, K, G, 0, 0, N, y, bound, status);
}

/* ------------------------------------------------------------------------ */
/* 2-bit format: four codes a byte                                           */
/* ------------------------------------------------------------------------ */

/*
 * Ternary codes in two bits each, four a byte (Avenue README, size note:
 * model sizes counted for 2-bit packing; "Autoregressive Language Model on
 * the 6502 Processor": ternary parameters packed four a byte).  Reading
 * taken here: field f = c + 1 in {0, 1, 2}, the first weight in the lowest
 * two bits, G/4 bytes a group, the same fp16 group scales and code rule as
 * the base-3 format; field value 3 is invalid.
 *   packed[N][K/G][G/4] bytes, scales[N][K/G] fp16 bits.
 */
int oracle_quantize_pack2(const uint16_t *w, int64_t N, int64_t K, int64_t G,
                          uint8_t *packed, uint16_t *scales, int32_t *status)
{
    if (!w || !packed || !scales) return OR_ERR_NULL;
    int rc = check_shape(N, K, G);
    if (rc) return rc;
    if (G % 4) return OR_ERR_SHAPE;
    const int64_t nG = K / G;
    int32_t st = 0;
    int8_t *code = (int8_t *)malloc((size_t)G);
    if (!code) return OR_ERR_NULL;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t g = 0; g < nG; ++g) {
            uint16_t sbits;
            int gst = group_scale_and_codes(w + n * K + g * G, G, G, &sbits, code);
            uint8_t *pg = packed + n * (K / 4) + g * (G / 4);
            for (int64_t b = 0; b < G / 4; ++b) {
                int byte = 0;
                for (int i = 0; i < 4; ++i) byte |= (code[4 * b + i] + 1) << (2 * i);
                pg[b] = (uint8_t)byte;
            }
            scales[n * nG + g] = sbits;
            st |= gst;
        }
    }
    free(code);
    if (status) *status |= st;
    return OR_OK;
}

/* 2-bit packed -> codes[N,K] in {-1,0,1}; a field of 3 reads as code 0 and
 * sets INVALID_BYTE. */
int oracle_unpack2(const uint8_t *packed, int64_t N, int64_t K, int64_t G, int8_t *codes,
                   int32_t *status)
{
    if (!packed || !codes) return OR_ERR_NULL;
    int rc = check_shape(N, K, G);
    if (rc) return rc;
    if (G % 4) return OR_ERR_SHAPE;
    int32_t st = 0;
    for (int64_t i = 0; i < N * K; ++i) {
        int f = (packed[i / 4] >> (2 * (i % 4))) & 3;
        if (f == 3) { st |= OR_INVALID_BYTE; f = 1; }
        codes[i] = (int8_t)(f - 1);
    }
    if (status) *status |= st;
    return OR_OK;
}

int oracle_matmul2(const uint16_t *x, const uint8_t *packed, const uint16_t *scales,
                   int64_t M, int64_t N, int64_t K, int64_t G,
                   double *y, double *bound, int32_t *status)
{
    return matmul_rows(x, packed, scales, M, N, K, G, 1, 0, N, y, bound, status);
}


/* ------------------------------------------------------------------------ */
/* W4A16: group-wise affine int4 weights ([P2] "Group-Wise Affine          */
/* Quantization", "Reconstruct a Stored Group", "Packed Storage Layout",   */
/* "Computation Flow").  Layout:                                            */
/*   packed [N][K/8] uint32, weight 8p + i in bits 4i..4i+3 of word p        */
/*   scales, biases [N][K/G] bf16 bits; w_hat = q * s + b, q in [0, 15]      */
/* The page defines no quantizer (the stored codes and parameters are used  */
/* as they are), so there is none here.                                     */
/* ------------------------------------------------------------------------ */

static int check_w4(int64_t N, int64_t K, int64_t G)
{
    if (N < 1 || K < 1 || G < 8 || G % 8 || K % G) return OR_ERR_SHAPE;
    return OR_OK;
}

/* The unsigned 4-bit code of weight k of a row (eight codes a word, the
 * first in the lowest four bits). */
static int w4_code(const uint32_t *row, int64_t k)
{
    return (int)((row[k / 8] >> (4 * (k % 8))) & 0xFu);
}

/* codes[N][K] = the unpacked unsigned codes. */
int oracle_w4_unpack(const uint32_t *packed, int64_t N, int64_t K, uint8_t *codes)
{
    if (!packed || !codes) return OR_ERR_NULL;
    if (N < 1 || K < 1 || K % 8) return OR_ERR_SHAPE;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) codes[n * K + k] = (uint8_t)w4_code(packed + n * (K / 8), k);
    return OR_OK;
}

/* bf16 bits -> double, non-finite values included (exact). */
static double bf16_any_to_double(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* w_hat[N][K] = q * s + b in fp64.  q * s is exact (4 x 8 significant bits);
 * the sum with b is exact unless the exponents of q*s and b lie more than
 * about 40 binades apart. */
int oracle_w4a16_dequantize(const uint32_t *packed, const uint16_t *scales,
                            const uint16_t *biases, int64_t N, int64_t K, int64_t G,
                            double *w_hat)
{
    if (!packed || !scales || !biases || !w_hat) return OR_ERR_NULL;
    int rc = check_w4(N, K, G);
    if (rc) return rc;
    const int64_t nG = K / G;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            const double s = bf16_any_to_double(scales[n * nG + k / G]);
            const double b = bf16_any_to_double(biases[n * nG + k / G]);
            w_hat[n * K + k] = (double)w4_code(packed + n * (K / 8), k) * s + b;
        }
    return OR_OK;
}

/*
 * y[m][n] = sum_k x[m][k] * (q[n][k] * s[n][k/G] + b[n][k/G]), taken in the
 * page's order: group by group, word by word, code by code, one
 * reconstructed weight times one activation added to one accumulator
 * (fp64 here, where the page asks for a float accumulator).
 * bound[m][n] = sum_k |x[m][k]| * (|q s| + |b|): the size of the terms of
 * the factored form s * sum(x q) + b * sum(x) that a kernel may evaluate.
 */
static int w4a16_matmul_rows(const uint16_t *x, const uint32_t *packed, const uint16_t *scales,
                             const uint16_t *biases, int64_t M, int64_t N, int64_t K, int64_t G,
                             int64_t n0, int64_t n1, double *y, double *bound)
{
    if (!x || !packed || !scales || !biases || !y || !bound) return OR_ERR_NULL;
    int rc = check_w4(N, K, G);
    if (rc) return rc;
    if (M < 1) return OR_ERR_SHAPE;
    const int64_t nG = K / G;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = n0; n < n1; ++n) {
            const uint32_t *row = packed + n * (K / 8);
            double acc = 0.0, bacc = 0.0;
            for (int64_t g = 0; g < nG; ++g) {
                const double s = bf16_any_to_double(scales[n * nG + g]);
                const double b = bf16_any_to_double(biases[n * nG + g]);
                for (int64_t p = 0; p < G / 8; ++p) {
                    const uint32_t word = row[g * (G / 8) + p];
                    for (int i = 0; i < 8; ++i) {
                        const double q = (double)((word >> (4 * i)) & 0xFu);
                        const double a = bf16_any_to_double(x[m * K + g * G + 8 * p + i]);
                        acc += a * (q * s + b);
                        bacc += fabs(a) * (fabs(q * s) + fabs(b));
                    }
                }
            }
            y[m * N + n] = acc;
            bound[m * N + n] = bacc;
        }
    return OR_OK;
}

int oracle_w4a16_matmul(const uint16_t *x, const uint32_t *packed, const uint16_t *scales,
                        const uint16_t *biases, int64_t M, int64_t N, int64_t K, int64_t G,
                        double *y, double *bound)
{
    return w4a16_matmul_rows(x, packed, scales, biases, M, N, K, G, 0, N, y, bound);
}

/* ------------------------------------------------------------------------ */
/* Row-partitioned threading (for test and baseline throughput only)        */
/* ------------------------------------------------------------------------ */

/*
 * The _mt entry points split the weight rows into `threads` contiguous
 * ranges and run the single-thread code above on each range in its own
 * POSIX thread.  No output depends on another row, and each output is
 * computed by the same loop in the same order as in the single-thread call,
 * so the results are identical for every thread count.
 */
enum { MT_QUANT, MT_MATMUL, MT_MATMUL2, MT_W4A16 };

typedef struct {
    int kind;
    const uint16_t *x, *w, *scales_in, *biases;
    const void *packed_in;
    uint8_t *packed_out;
    uint16_t *scales_out;
    int64_t M, N, K, G, n0, n1;
    double *y, *bound;
    int32_t status;
    int rc;
} mt_job;

static void *mt_run(void *arg)
{
    mt_job *j = (mt_job *)arg;
    j->status = 0;
    switch (j->kind) {
    case MT_QUANT: {
        const int64_t rb = oracle_packed_row_bytes(j->K, j->G), nG = j->K / j->G;
        j->rc = j->n1 > j->n0
                    ? oracle_quantize_pack(j->w + j->n0 * j->K, j->n1 - j->n0, j->K, j->G,
                                           j->packed_out + j->n0 * rb,
                                           j->scales_out + j->n0 * nG, &j->status)
                    : OR_OK;
        break;
    }
    case MT_MATMUL:
    case MT_MATMUL2:
        j->rc = matmul_rows(j->x, (const uint8_t *)j->packed_in, j->scales_in, j->M, j->N, j->K,
                            j->G, j->kind == MT_MATMUL2, j->n0, j->n1, j->y, j->bound,
                            &j->status);
        break;
    default:
        j->rc = w4a16_matmul_rows(j->x, (const uint32_t *)j->packed_in, j->scales_in, j->biases,
                                  j->M, j->N, j->K, j->G, j->n0, j->n1, j->y, j->bound);
        break;
    }
    return NULL;
}

static int mt_split(mt_job proto, int threads, int32_t *status)
{
    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    if (threads > proto.N) threads = (int)(proto.N > 0 ? proto.N : 1);
    mt_job jobs[256];
    pthread_t tids[256];
    int started[256];
    for (int t = 0; t < threads; ++t) {
        jobs[t] = proto;
        jobs[t].n0 = proto.N * t / threads;
        jobs[t].n1 = proto.N * (t + 1) / threads;
        started[t] = t > 0 && pthread_create(&tids[t], NULL, mt_run, &jobs[t]) == 0;
        if (t > 0 && !started[t]) mt_run(&jobs[t]);  /* no thread: run it here */
    }
    mt_run(&jobs[0]);
    int rc = OR_OK;
    int32_t st = 0;
    for (int t = 0; t < threads; ++t) {
        if (started[t]) pthread_join(tids[t], NULL);
        if (jobs[t].rc && !rc) rc = jobs[t].rc;
        st |= jobs[t].status;
    }
    if (!rc && status) *status |= st;
    return rc;
}

int oracle_quantize_pack_mt(const uint16_t *w, int64_t N, int64_t K, int64_t G,
                            uint8_t *packed, uint16_t *scales, int32_t *status, int threads)
{
    if (!w || !packed || !scales) return OR_ERR_NULL;
    int rc = check_shape(N, K, G);
    if (rc) return rc;
    mt_job p = {0};
    p.kind = MT_QUANT; p.w = w; p.packed_out = packed; p.scales_out = scales;
    p.N = N; p.K = K; p.G = G;
    return mt_split(p, threads, status);
}

int oracle_matmul_mt(const uint16_t *x, const uint8_t *packed, const uint16_t *scales,
                     int64_t M, int64_t N, int64_t K, int64_t G, double *y, double *bound,
                     int32_t *status, int threads)
{
    if (!x || !packed || !scales || !y) return OR_ERR_NULL;
    int rc = check_shape(N, K, G);
    if (rc) return rc;
    if (M < 1) return OR_ERR_SHAPE;
    mt_job p = {0};
    p.kind = MT_MATMUL; p.x = x; p.packed_in = packed; p.scales_in = scales;
    p.M = M; p.N = N; p.K = K; p.G = G; p.y = y; p.bound = bound;
    return mt_split(p, threads, status);
}

int oracle_matmul2_mt(const uint16_t *x, const uint8_t *packed, const uint16_t *scales,
                      int64_t M, int64_t N, int64_t K, int64_t G, double *y, double *bound,
                      int32_t *status, int threads)
{
    if (!x || !packed || !scales || !y) return OR_ERR_NULL;
    int rc = check_shape(N, K, G);
    if (rc) return rc;
    if (M < 1 || G % 4) return OR_ERR_SHAPE;
    mt_job p = {0};
    p.kind = MT_MATMUL2; p.x = x; p.packed_in = packed; p.scales_in = scales;
    p.M = M; p.N = N; p.K = K; p.G = G; p.y = y; p.bound = bound;
    return mt_split(p, threads, status);
}

int oracle_w4a16_matmul_mt(const uint16_t *x, const uint32_t *packed, const uint16_t *scales,
                           const uint16_t *biases, int64_t M, int64_t N, int64_t K, int64_t G,
                           double *y, double *bound, int threads)
{
    if (!x || !packed || !scales || !biases || !y || !bound) return OR_ERR_NULL;
    int rc = check_w4(N, K, G);
    if (rc) return rc;
    if (M < 1) return OR_ERR_SHAPE;
    mt_job p = {0};
    p.kind = MT_W4A16; p.x = x; p.packed_in = packed; p.scales_in = scales; p.biases = biases;
    p.M = M; p.N = N; p.K = K; p.G = G; p.y = y; p.bound = bound;
    return mt_split(p, threads, NULL);
}
