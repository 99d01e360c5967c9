/*
 * qbn oracle: plain, slow CPU definitions of what 4-bit block-quantized
 * weights decode to, of the dot products built on them, and of the int4
 * layout repacks.
 *
 * TEST INFRASTRUCTURE ONLY. The library's product path never links, loads
 * or calls this file. Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it. It shares no source with the HIP
 * kernels: every decoder below is written from the formats' definitions,
 * not from any table or helper used on the GPU.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared, no SIMD intrinsics, no fast-math.
 *
 * Sources (page title, section):
 *  [FB]  "Four Bits, Three Contracts: an interactive guide to MXFP4, NVFP4
 *        and Q4_K" (shivasnotes.com, blog 6006)
 *  [WK]  "Why 4-Bit Quantization Is King: Understanding Q4_K, MXFP4, and
 *        NVFP4" (shivasnotes.com, blog 5996)
 *  [BP]  "Bit Packing Architecture" (aicassindra.com)
 *  [NV]  "Chapter 7 - NVFP4: the native lane" (Muser book,
 *        highperformanceailab.com)
 *
 * Every decoded weight is an IEEE binary32 value; products that the format
 * definition makes exact are formed in binary64 and cast once, and the only
 * inexact steps (NVFP4's multiply by scale2, Q4_K's gain-minus-offset) are
 * rounded exactly once to binary32, as the formats prescribe.
 * Dot products are formed in binary64 with Neumaier-compensated sums.
 *
 * W4A8 ([WK] section 7): activations are quantized to int8 codes with one
 * binary32 scale per 256 elements by the Q8_K rule of [NV] section 7.4.2;
 * the Q4_K x int8 dot then uses each weight's exact value
 * d*s_j*q - dmin*m_j, which is what the integer route (integer dot, code
 * sums, scales applied afterwards) computes.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------ */
/* Scalar decoders                                                     */
/* ------------------------------------------------------------------ */

/* E2M1 element code: 1 sign, 2 exponent, 1 fraction bit, exponent bias 1.
 * Exponent field 0 holds zero and the single subnormal magnitude 0.5.
 * Code 8 is negative zero. [FB] section 1; [NV] section 7.1, Figure 7.1. */
ORACLE_API double oracle_e2m1(unsigned code)
{
    unsigned s = (code >> 3) & 1u;
    unsigned e = (code >> 1) & 3u;
    unsigned m = code & 1u;
    double mag;
    if (e == 0)
        mag = 0.5 * (double)m;
    else
        mag = ldexp(1.0 + (double)m / 2.0, (int)e - 1);
    return s ? -mag : mag;
}

/* E8M0 shared scale: an unsigned biased exponent, value 2^(b-127); the byte
 * 255 is reserved for NaN and there is no zero. [FB] section 3. */
ORACLE_API double oracle_e8m0(unsigned b)
{
    b &= 0xFFu;
    if (b == 255u)
        return NAN;
    return ldexp(1.0, (int)b - 127);
}

/* E4M3FN scale: sign, 4 exponent bits with bias 7, 3 fraction bits, no
 * infinities; NaN only where exponent and fraction are all ones (0x7f, 0xff);
 * exponent field 0 is subnormal with value fraction * 2^-9.
 * [FB] section 4; [NV] sections 7.1, 7.2 and 7.8. */
ORACLE_API double oracle_e4m3fn(unsigned b)
{
    b &= 0xFFu;
    unsigned s = b >> 7;
    unsigned e = (b >> 3) & 15u;
    unsigned m = b & 7u;
    double mag;
    if (e == 15u && m == 7u)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -mag : mag;
}

/* IEEE binary16 from its bit pattern (the fp16 d, dmin, Q4_0 d and group
 * scales are little-endian binary16). */
ORACLE_API double oracle_f16(unsigned h)
{
    h &= 0xFFFFu;
    unsigned s = h >> 15;
    unsigned e = (h >> 10) & 31u;
    unsigned f = h & 1023u;
    double mag;
    if (e == 31u)
        mag = f ? NAN : INFINITY;
    else if (e == 0)
        mag = ldexp((double)f, -24);
    else
        mag = ldexp(1.0 + (double)f / 1024.0, (int)e - 15);
    return s ? -mag : mag;
}

/* bfloat16 bit pattern to its value (the upper half of a binary32). */
ORACLE_API double oracle_bf16_value(unsigned bits)
{
    uint32_t u = (uint32_t)(bits & 0xFFFFu) << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* binary32 to bfloat16 with round-to-nearest-even on the dropped 16 bits.
 * NaN stays NaN (quiet). */
ORACLE_API unsigned oracle_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu))
        return ((u >> 16) | 0x40u) & 0xFFFFu;
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (u >> 16) & 0xFFFFu;
}

static unsigned rd_u16(const uint8_t *p) { return (unsigned)p[0] | ((unsigned)p[1] << 8); }
static uint32_t rd_u32(const uint8_t *p)
{
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

/* Logical element i of a row of two-codes-per-byte E2M1: the low nibble of
 * byte i/2 holds the even element, the high nibble the odd one.
 * [NV] Figure 7.2; the MXFP4 rows use the same order. */
static unsigned nibble_lo_even(const uint8_t *row, int64_t i)
{
    uint8_t byte = row[i / 2];
    return (i & 1) ? (byte >> 4) : (byte & 15u);
}

/* ------------------------------------------------------------------ */
/* Q4_K super-block metadata                                          */
/* ------------------------------------------------------------------ */

/* Unpack the eight 6-bit (scale, min) pairs from the 12 metadata bytes B.
 * Pairs 0..3 keep their six bits whole in B[j] and B[j+4]; pairs 4..7 put
 * their low four bits in B[j+4] (scale low nibble, min high nibble) and their
 * top two bits in the top of B[j-4] (scale) and B[j] (min).
 * [FB] section 6. */
ORACLE_API void oracle_q4k_unpack_scales(const uint8_t *B, unsigned *s, unsigned *m)
{
    for (int j = 0; j < 8; ++j) {
        if (j < 4) {
            s[j] = B[j] & 63u;
            m[j] = B[j + 4] & 63u;
        } else {
            s[j] = (unsigned)(B[j + 4] & 15u) | ((unsigned)(B[j - 4] >> 6) << 4);
            m[j] = (unsigned)(B[j + 4] >> 4) | ((unsigned)(B[j] >> 6) << 4);
        }
    }
}

/* Inverse of the above (encode side, used to build fixtures). */
ORACLE_API void oracle_q4k_pack_scales(const unsigned *s, const unsigned *m, uint8_t *B)
{
    memset(B, 0, 12);
    for (int j = 0; j < 4; ++j) {
        B[j] = (uint8_t)((s[j] & 63u) | ((s[j + 4] >> 4) << 6));
        B[j + 4] = (uint8_t)((m[j] & 63u) | ((m[j + 4] >> 4) << 6));
        B[j + 8] = (uint8_t)((s[j + 4] & 15u) | ((m[j + 4] & 15u) << 4));
    }
}

/* ------------------------------------------------------------------ */
/* Row dequantizers: decode row r of an n x k weight into out[0..k)    */
/* ------------------------------------------------------------------ */

/* MXFP4: codes u8 [n][k/2] (low nibble = even element), E8M0 scales u8
 * [n][k/32] with groups running along k. w = E2M1(code) * 2^(b-127); the
 * product is exact in binary32 or overflows to infinity. [FB] section 3. */
static void mxfp4_row(const uint8_t *codes, const uint8_t *scales, int64_t k, int64_t r, float *out)
{
    const uint8_t *crow = codes + r * (k / 2);
    const uint8_t *srow = scales + r * (k / 32);
    for (int64_t i = 0; i < k; ++i)
        out[i] = (float)(oracle_e2m1(nibble_lo_even(crow, i)) * oracle_e8m0(srow[i / 32]));
}

/* NVFP4: codes u8 [n][k/2], E4M3FN scales u8 [n][k/16], one binary32 scale2
 * per tensor. Pinned order: (E2M1 * E4M3FN) first (exact), then times scale2
 * with one rounding to binary32. [NV] sections 7.1 and 7.2; [FB] section 4. */
static void nvfp4_row(const uint8_t *codes, const uint8_t *scales, float scale2, int64_t k, int64_t r,
                      float *out)
{
    const uint8_t *crow = codes + r * (k / 2);
    const uint8_t *srow = scales + r * (k / 16);
    for (int64_t i = 0; i < k; ++i) {
        float local = (float)(oracle_e2m1(nibble_lo_even(crow, i)) * oracle_e4m3fn(srow[i / 16]));
        out[i] = (float)((double)local * (double)scale2);
    }
}

/* CKE's NVFP4 storage block ([WK] section 5): [n][k/64] blocks of 36 bytes
 * holding 64 consecutive weights of a row. Bytes 0..3 are the E4M3FN
 * subscales of the four 16-weight subblocks, in order; bytes 4..35 are the
 * codes, eight bytes per subblock in subblock order. Inside subblock j, the
 * low nibble of its byte i is weight 16j + i and the high nibble weight
 * 16j + 8 + i (split-half order, not adjacent pairs). The per-tensor scale2
 * is a separate operand. Reconstruction is the NVFP4 rule: (E2M1 * E4M3FN)
 * exactly, then times scale2 with one rounding. */
static void nvfp4_cke_row(const uint8_t *data, float scale2, int64_t k, int64_t r, float *out)
{
    const uint8_t *row = data + r * (k / 64) * 36;
    for (int64_t i = 0; i < k; ++i) {
        const uint8_t *blk = row + (i / 64) * 36;
        const int64_t j = (i % 64) / 16; /* subblock */
        const int64_t l = i % 16;        /* weight inside the subblock */
        const unsigned byte = blk[4 + 8 * j + (l % 8)];
        const unsigned code = l < 8 ? (byte & 15u) : (byte >> 4);
        float local = (float)(oracle_e2m1(code) * oracle_e4m3fn(blk[j]));
        out[i] = (float)((double)local * (double)scale2);
    }
}

/* Q4_K: 144-byte super-blocks of 256 weights, [n][k/256]. Byte layout:
 * fp16 d at 0, fp16 dmin at 2, 12 metadata bytes at 4, 128 code bytes at 16.
 * Code byte 32c+l (c = 0..3, l = 0..31) holds, in its low nibble, output
 * 64c+l (sub-block 2c) and, in its high nibble, output 64c+32+l (sub-block
 * 2c+1). w = (d*s_j)*q - dmin*m_j: the gain and offset are exact binary32
 * products and the difference is rounded once.
 * [FB] sections 5 and 6; [WK] sections 4 and 7b. */
static void q4k_row(const uint8_t *blocks, int64_t k, int64_t r, float *out)
{
    int64_t nb = k / 256;
    for (int64_t b = 0; b < nb; ++b) {
        const uint8_t *blk = blocks + (r * nb + b) * 144;
        double d = oracle_f16(rd_u16(blk + 0));
        double dmin = oracle_f16(rd_u16(blk + 2));
        unsigned s[8], m[8];
        oracle_q4k_unpack_scales(blk + 4, s, m);
        const uint8_t *qs = blk + 16;
        for (int c = 0; c < 4; ++c) {
            for (int l = 0; l < 32; ++l) {
                uint8_t byte = qs[32 * c + l];
                for (int half = 0; half < 2; ++half) {
                    int j = 2 * c + half;
                    unsigned q = half ? (byte >> 4) : (byte & 15u);
                    float gain = (float)(d * (double)s[j]);
                    float offset = (float)(dmin * (double)m[j]);
                    out[b * 256 + 64 * c + 32 * half + l] = fmaf(gain, (float)q, -offset);
                }
            }
        }
    }
}

/* Q4_0: 18-byte blocks of 32 weights, [n][k/32]: fp16 d, then 16 bytes where
 * byte j holds element j (low nibble) and element j+16 (high nibble).
 * w = d * (q - 8), exact in binary32. [BP] "Real layouts compared". */
static void q4_0_row(const uint8_t *blocks, int64_t k, int64_t r, float *out)
{
    int64_t nb = k / 32;
    for (int64_t b = 0; b < nb; ++b) {
        const uint8_t *blk = blocks + (r * nb + b) * 18;
        double d = oracle_f16(rd_u16(blk));
        for (int j = 0; j < 16; ++j) {
            uint8_t byte = blk[2 + j];
            out[b * 32 + j] = (float)(d * ((double)(byte & 15u) - 8.0));
            out[b * 32 + j + 16] = (float)(d * ((double)(byte >> 4) - 8.0));
        }
    }
}

/* ------------------------------------------------------------------ */
/* int4 layouts: GPTQ, AWQ, Q4_0 codes <-> logical u8 matrix q[K][N]   */
/* ------------------------------------------------------------------ */

/* Generic b-bit little-endian word stream ([BP] "The packing arithmetic"):
 * the stream is the concatenation of the words' bits, least significant bit
 * of word 0 first, and element i owns stream bits i*b .. i*b + b - 1, its
 * own least significant bit first. Written bit by bit from that definition,
 * so an element that runs past a word boundary needs no special case.
 * 1 <= bits <= 32. */
static unsigned stream_bit(const uint32_t *words, int64_t s)
{
    return (unsigned)(words[s / 32] >> (s % 32)) & 1u;
}

ORACLE_API void oracle_pack_bits(const uint32_t *vals, int64_t count, int bits, uint32_t *words)
{
    int64_t total = count * bits;
    for (int64_t w = 0; w < (total + 31) / 32; ++w)
        words[w] = 0;
    for (int64_t s = 0; s < total; ++s) {
        unsigned bit = (unsigned)(vals[s / bits] >> (s % bits)) & 1u;
        words[s / 32] |= (uint32_t)bit << (s % 32);
    }
}

ORACLE_API void oracle_unpack_bits(const uint32_t *words, int64_t count, int bits, uint32_t *vals)
{
    for (int64_t i = 0; i < count; ++i) {
        uint32_t v = 0;
        for (int t = 0; t < bits; ++t)
            v |= (uint32_t)stream_bit(words, i * bits + t) << t;
        vals[i] = v;
    }
}

/* AWQ slot order: slot t of a word holds logical column ORDER[t] of its
 * group of eight. [BP] "Real layouts compared". */
static const int AWQ_ORDER[8] = {0, 2, 4, 6, 1, 3, 5, 7};

/* GPTQ qweight: int32 [K/8][N], packed along K; each column is a 4-bit
 * stream along K, so row 8r+j sits at bits 4j of word [r][n]. [BP]. */
ORACLE_API void oracle_gptq_pack(const uint8_t *q, int64_t K, int64_t N, uint32_t *qw)
{
    uint32_t col[8], word;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t r = 0; r < K / 8; ++r) {
            for (int j = 0; j < 8; ++j)
                col[j] = q[(r * 8 + j) * N + n];
            oracle_pack_bits(col, 8, 4, &word);
            qw[r * N + n] = word;
        }
}

ORACLE_API void oracle_gptq_unpack(const uint32_t *qw, int64_t K, int64_t N, uint8_t *q)
{
    uint32_t col[8];
    for (int64_t n = 0; n < N; ++n)
        for (int64_t r = 0; r < K / 8; ++r) {
            oracle_unpack_bits(&qw[r * N + n], 8, 4, col);
            for (int j = 0; j < 8; ++j)
                q[(r * 8 + j) * N + n] = (uint8_t)col[j];
        }
}

/* AWQ qweight: int32 [K][N/8], packed along N; within each group of eight
 * columns the slots hold columns 0,2,4,6,1,3,5,7. [BP]. */
ORACLE_API void oracle_awq_pack(const uint8_t *q, int64_t K, int64_t N, uint32_t *qw)
{
    uint32_t slots[8], word;
    for (int64_t kk = 0; kk < K; ++kk)
        for (int64_t g = 0; g < N / 8; ++g) {
            for (int t = 0; t < 8; ++t)
                slots[t] = q[kk * N + g * 8 + AWQ_ORDER[t]];
            oracle_pack_bits(slots, 8, 4, &word);
            qw[kk * (N / 8) + g] = word;
        }
}

ORACLE_API void oracle_awq_unpack(const uint32_t *qw, int64_t K, int64_t N, uint8_t *q)
{
    uint32_t slots[8];
    for (int64_t kk = 0; kk < K; ++kk)
        for (int64_t g = 0; g < N / 8; ++g) {
            oracle_unpack_bits(&qw[kk * (N / 8) + g], 8, 4, slots);
            for (int t = 0; t < 8; ++t)
                q[kk * N + g * 8 + AWQ_ORDER[t]] = (uint8_t)slots[t];
        }
}

/* GPTQ qzeros: int32 [G][N/8], packed along the output dimension as a
 * 4-bit stream, column 8c + j at bits 4j of word [g][c] ([BP] "Real layouts
 * compared"). version 1 (AutoGPTQ's pack step) stores z - 1, version 2
 * stores z ([BP] ibid. and "Repacking between formats", step 2). Unpacking
 * adds the one back for version 1, so a stored nibble s reads as s + 1
 * (1..16); packing version 1 stores (z - 1) mod 16, so z = 0 reads back as
 * 16. Returns -1 for an unknown version. */
ORACLE_API int oracle_qzeros_unpack(const uint32_t *qz, int64_t G, int64_t N, int version, uint8_t *zeros)
{
    if (version != 1 && version != 2)
        return -1;
    uint32_t vals[8];
    for (int64_t g = 0; g < G; ++g)
        for (int64_t c = 0; c < N / 8; ++c) {
            oracle_unpack_bits(&qz[g * (N / 8) + c], 8, 4, vals);
            for (int j = 0; j < 8; ++j)
                zeros[g * N + 8 * c + j] = (uint8_t)(vals[j] + (version == 1 ? 1u : 0u));
        }
    return 0;
}

ORACLE_API int oracle_qzeros_pack(const uint8_t *zeros, int64_t G, int64_t N, int version, uint32_t *qz)
{
    if (version != 1 && version != 2)
        return -1;
    uint32_t vals[8];
    for (int64_t g = 0; g < G; ++g)
        for (int64_t c = 0; c < N / 8; ++c) {
            for (int j = 0; j < 8; ++j)
                vals[j] = ((uint32_t)zeros[g * N + 8 * c + j] - (version == 1 ? 1u : 0u)) & 15u;
            oracle_pack_bits(vals, 8, 4, &qz[g * (N / 8) + c]);
        }
    return 0;
}

/* GPTQ act-order: g_idx[k] is the group of input row k ([BP] "Real layouts
 * compared"). Resolving it ([BP] "Repacking between formats", step 3) orders
 * the rows by group, keeping the original order inside a group: perm[i] is
 * the source row placed at i, so that rows of group g fill g*group ..
 * g*group + group - 1 and a layout without g_idx applies. Applying the same
 * perm to the activations leaves every dot product's terms unchanged.
 * Returns 0; -1 if a g_idx is outside 0..K/group-1; -2 if a group does not
 * hold exactly `group` rows. */
ORACLE_API int oracle_resolve_g_idx(const int32_t *g_idx, int64_t K, int64_t group, int32_t *perm)
{
    int64_t G = K / group;
    for (int64_t k = 0; k < K; ++k)
        if (g_idx[k] < 0 || g_idx[k] >= G)
            return -1;
    int64_t i = 0;
    for (int64_t g = 0; g < G; ++g) {
        int64_t count = 0;
        for (int64_t k = 0; k < K; ++k)
            if (g_idx[k] == g) {
                perm[i++] = (int32_t)k;
                ++count;
            }
        if (count != group)
            return -2;
    }
    return 0;
}

/* Q4_0 code layout for a K x N logical matrix: blocks run along K within
 * each output column n and are stored [N][K/32] x 18 bytes; block (n, b)
 * holds q[32b .. 32b+31][n], byte j = element j (low) | element j+16 (high).
 * d_bits[(n*(K/32)) + b] is written as the fp16 d of each block. */
/* CKE split-half NVFP4 blocks (layout in nvfp4_cke_row above) from
 * logical E2M1 codes u8 [n][k] (0..15) and E4M3FN subscale bytes
 * u8 [n][k/16]; blocks u8 [n][k/64][36]. */
ORACLE_API void oracle_cke_pack(const uint8_t *codes, const uint8_t *scales, int64_t n, int64_t k, uint8_t *blocks)
{
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < k / 64; ++b) {
            uint8_t *blk = blocks + (r * (k / 64) + b) * 36;
            for (int j = 0; j < 4; ++j) {
                blk[j] = scales[r * (k / 16) + 4 * b + j];
                const uint8_t *c = codes + r * k + 64 * b + 16 * j;
                for (int i = 0; i < 8; ++i)
                    blk[4 + 8 * j + i] = (uint8_t)((c[i] & 15u) | ((c[i + 8] & 15u) << 4));
            }
        }
}

ORACLE_API void oracle_cke_unpack(const uint8_t *blocks, int64_t n, int64_t k, uint8_t *codes, uint8_t *scales)
{
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < k / 64; ++b) {
            const uint8_t *blk = blocks + (r * (k / 64) + b) * 36;
            for (int j = 0; j < 4; ++j) {
                scales[r * (k / 16) + 4 * b + j] = blk[j];
                uint8_t *c = codes + r * k + 64 * b + 16 * j;
                for (int i = 0; i < 8; ++i) {
                    c[i] = blk[4 + 8 * j + i] & 15u;
                    c[i + 8] = blk[4 + 8 * j + i] >> 4;
                }
            }
        }
}

ORACLE_API void oracle_q4_0_pack(const uint8_t *q, const uint16_t *d_bits, int64_t K, int64_t N,
                                 uint8_t *blocks)
{
    int64_t nb = K / 32;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < nb; ++b) {
            uint8_t *blk = blocks + (n * nb + b) * 18;
            uint16_t d = d_bits[n * nb + b];
            blk[0] = (uint8_t)(d & 0xFF);
            blk[1] = (uint8_t)(d >> 8);
            for (int j = 0; j < 16; ++j) {
                unsigned lo = q[(32 * b + j) * N + n] & 15u;
                unsigned hi = q[(32 * b + j + 16) * N + n] & 15u;
                blk[2 + j] = (uint8_t)(lo | (hi << 4));
            }
        }
}

ORACLE_API void oracle_q4_0_unpack(const uint8_t *blocks, int64_t K, int64_t N, uint8_t *q, uint16_t *d_bits)
{
    int64_t nb = K / 32;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = blocks + (n * nb + b) * 18;
            if (d_bits)
                d_bits[n * nb + b] = (uint16_t)rd_u16(blk);
            for (int j = 0; j < 16; ++j) {
                q[(32 * b + j) * N + n] = blk[2 + j] & 15u;
                q[(32 * b + j + 16) * N + n] = blk[2 + j] >> 4;
            }
        }
}

/* Affine int4 dequantization of the logical matrix: w = s * (q - z) with
 * fp16 s and integer zero point z per group of g rows along K; exact in
 * binary32. [BP] "Repacking between formats", step 2. Output [K][N]. */
ORACLE_API void oracle_affine_dequant(const uint8_t *q, const uint16_t *scale_bits, const uint8_t *zeros,
                                      int64_t K, int64_t N, int64_t g, float *out)
{
    for (int64_t kk = 0; kk < K; ++kk)
        for (int64_t n = 0; n < N; ++n) {
            double s = oracle_f16(scale_bits[(kk / g) * N + n]);
            double z = (double)zeros[(kk / g) * N + n];
            out[kk * N + n] = (float)(s * ((double)q[kk * N + n] - z));
        }
}

/* ------------------------------------------------------------------ */
/* Format dispatch: dequantize chosen rows of an n x k weight          */
/* ------------------------------------------------------------------ */

enum { OR_MXFP4 = 1, OR_NVFP4 = 2, OR_Q4_K = 3, OR_Q4_0 = 4, OR_NVFP4_CKE = 8 };

static int row_dequant(int fmt, const uint8_t *data, const uint8_t *scales, float scale2, int64_t k,
                       int64_t r, float *out)
{
    switch (fmt) {
    case OR_MXFP4: mxfp4_row(data, scales, k, r, out); return 0;
    case OR_NVFP4: nvfp4_row(data, scales, scale2, k, r, out); return 0;
    case OR_Q4_K: q4k_row(data, k, r, out); return 0;
    case OR_Q4_0: q4_0_row(data, k, r, out); return 0;
    case OR_NVFP4_CKE: nvfp4_cke_row(data, scale2, k, r, out); return 0;
    default: return -1;
    }
}

/* out[i][0..k) = dequantized row rows[i]. Returns 0, or -1 on a bad format. */
ORACLE_API int oracle_dequant_rows(int fmt, const uint8_t *data, const uint8_t *scales, float scale2, int64_t k,
                                   const int64_t *rows, int64_t nrows, float *out)
{
    for (int64_t i = 0; i < nrows; ++i)
        if (row_dequant(fmt, data, scales, scale2, k, rows[i], out + i * k))
            return -1;
    return 0;
}

/* ------------------------------------------------------------------ */
/* Dot products                                                        */
/* ------------------------------------------------------------------ */

/* The value of a Neumaier sum: the running sum plus its compensation. The
 * compensation only exists for finite sums; once the running sum is an
 * infinity or NaN (weights beyond binary32's range decode to +-inf), the
 * IEEE sum itself is the value: +inf plus finite terms stays +inf, and
 * infinities of both signs give NaN. */
static double neumaier_value(double sum, double comp)
{
    return isfinite(sum) ? sum + comp : sum;
}

/* Neumaier-compensated binary64 sum of w[i]*x[i] (each product exact in
 * binary64 since both factors carry at most 24 significant bits), and the
 * plain binary64 sum of |w[i]*x[i]|. */
static void dot_f64(const float *w, const double *x, int64_t k, double *y, double *sabs)
{
    double sum = 0.0, comp = 0.0, a = 0.0;
    for (int64_t i = 0; i < k; ++i) {
        double p = (double)w[i] * x[i];
        double t = sum + p;
        if (fabs(sum) >= fabs(p))
            comp += (sum - t) + p;
        else
            comp += (p - t) + sum;
        sum = t;
        a += fabs(p);
    }
    *y = neumaier_value(sum, comp);
    *sabs = a;
}

/* Activation vector values: xdtype 0 = binary32, 1 = bfloat16 bits. */
static void load_x(const void *x, int xdtype, int64_t k, double *xv)
{
    for (int64_t i = 0; i < k; ++i) {
        if (xdtype == 1)
            xv[i] = oracle_bf16_value(((const uint16_t *)x)[i]);
        else
            xv[i] = (double)((const float *)x)[i];
    }
}

/* y[i] = sum_k w[rows[i]][k] * x[k] and s[i] = sum_k |w x| for the chosen
 * rows. scratch must hold k floats + k doubles (caller-provided so the
 * oracle itself never allocates). A fused kernel never materializes w;
 * this definition does, one row at a time. [WK] sections 1 and 7b. */
ORACLE_API int oracle_gemv_rows(int fmt, const uint8_t *data, const uint8_t *scales, float scale2, int64_t k,
                                const void *x, int xdtype, const int64_t *rows, int64_t nrows, double *y,
                                double *sabs, float *wscratch, double *xscratch)
{
    load_x(x, xdtype, k, xscratch);
    for (int64_t i = 0; i < nrows; ++i) {
        if (row_dequant(fmt, data, scales, scale2, k, rows[i], wscratch))
            return -1;
        dot_f64(wscratch, xscratch, k, &y[i], &sabs[i]);
    }
    return 0;
}

/* GEMV over a K x N weight stored input-major, as the GPTQ / AWQ logical
 * matrix is ([BP] "Real layouts compared"): y[i] = sum_k W[k][cols[i]] *
 * x[k] and s[i] = sum_k |W x|, with W the binary32 values of
 * oracle_affine_dequant. xscratch holds K doubles (caller-provided). */
ORACLE_API void oracle_gemv_kn(const float *W, int64_t K, int64_t N, const void *x, int xdtype,
                               const int64_t *cols, int64_t ncols, double *y, double *sabs, double *xscratch)
{
    load_x(x, xdtype, K, xscratch);
    for (int64_t i = 0; i < ncols; ++i) {
        double sum = 0.0, comp = 0.0, a = 0.0;
        for (int64_t kk = 0; kk < K; ++kk) {
            double p = (double)W[kk * N + cols[i]] * xscratch[kk];
            double t = sum + p;
            if (fabs(sum) >= fabs(p))
                comp += (sum - t) + p;
            else
                comp += (p - t) + sum;
            sum = t;
            a += fabs(p);
        }
        y[i] = neumaier_value(sum, comp);
        sabs[i] = a;
    }
}

/* Sampled GEMM entries: Y[m][n] = sum_k X[m][k] * w[n][k] for the pairs
 * (ms[i], ns[i]); X is bfloat16 bits [M][ldx]. Entries are grouped by the
 * caller; each weight row is decoded once per call of this function for
 * every pair (plain and slow by design). */
ORACLE_API int oracle_gemm_entries(int fmt, const uint8_t *data, const uint8_t *scales, float scale2, int64_t k,
                                   const uint16_t *X, int64_t ldx, const int64_t *ms, const int64_t *ns,
                                   int64_t npairs, double *y, double *sabs, float *wscratch, double *xscratch)
{
    int64_t cur_n = -1;
    for (int64_t i = 0; i < npairs; ++i) {
        if (ns[i] != cur_n) {
            if (row_dequant(fmt, data, scales, scale2, k, ns[i], wscratch))
                return -1;
            cur_n = ns[i];
        }
        load_x(X + ms[i] * ldx, 1, k, xscratch);
        dot_f64(wscratch, xscratch, k, &y[i], &sabs[i]);
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* W4A8: Q4_K weights times int8-quantized activations                 */
/* ------------------------------------------------------------------ */

/* One activation code: the binary32 product x * iscale rounded to the
 * nearest integer (ties to even), limited to at most 127. [NV] section 7.4.2
 * (round to nearest even, clamp at 127); [WK] section 7 (eight-bit codes). */
ORACLE_API int oracle_q8_code(float x, float iscale)
{
    float t = x * iscale; /* binary32 product, rounded to nearest */
    double r = nearbyint((double)t);
    if (r > 127.0)
        r = 127.0;
    return (int)r;
}

/* Q8_K-style activation quantization ([NV] section 7.4.2; the Q8_K
 * activations of [WK] section 7c), one scale per 256-element block:
 *   mx = the first element (lowest index) of largest magnitude, with its
 *        sign; iscale = RN32(-127 / mx); q = oracle_q8_code(x, iscale);
 *   d  = RN32(1 / iscale), so that x ~ d * q (d has the opposite sign of mx
 *        and the code of mx itself is -127).
 * A block with |mx| < 2^-118 (all zeros included) has d = 0 and q = 0: the
 * pages give no rule there, and below that bound 127 / |mx| is no longer
 * safely inside binary32's range (0 * inf would leave a code undefined).
 * bsums[j] = sum of the 32 codes of sub-block j.
 * x: finite binary32 (xdtype 0) or bfloat16 bits (1); k a multiple of 256. */
ORACLE_API void oracle_q8_quantize(const void *x, int xdtype, int64_t k, int8_t *q, float *d, int32_t *bsums)
{
    for (int64_t b = 0; b < k / 256; ++b) {
        float v[256];
        float mx = 0.0f;
        for (int i = 0; i < 256; ++i) {
            int64_t e = 256 * b + i;
            v[i] = xdtype == 1 ? (float)oracle_bf16_value(((const uint16_t *)x)[e]) : ((const float *)x)[e];
            if (fabsf(v[i]) > fabsf(mx))
                mx = v[i];
        }
        if (fabsf(mx) < 0x1p-118f) {
            d[b] = 0.0f;
            for (int i = 0; i < 256; ++i)
                q[256 * b + i] = 0;
        } else {
            float iscale = -127.0f / mx;
            d[b] = 1.0f / iscale;
            for (int i = 0; i < 256; ++i)
                q[256 * b + i] = (int8_t)oracle_q8_code(v[i], iscale);
        }
        for (int j = 0; j < 8; ++j) {
            int32_t t = 0;
            for (int i = 0; i < 32; ++i)
                t += q[256 * b + 32 * j + i];
            bsums[8 * b + j] = t;
        }
    }
}

/* The W4A8 contribution of one Q4_K sub-block, written as the integer dot
 * and the activation-code sum: s_x * step * sum(q_w q_x) - s_x * offset *
 * sum(q_x), in binary64. [WK] section 7 (the identity and its worked
 * example), section 7b step 4 and section 7c. idot and csum return the two
 * integer sums. */
ORACLE_API double oracle_w4a8_term(double step, double offset, double sx, const int *qw, const int *qx, int n,
                                   int64_t *idot, int64_t *csum)
{
    int64_t a = 0, c = 0;
    for (int i = 0; i < n; ++i) {
        a += (int64_t)qw[i] * qx[i];
        c += qx[i];
    }
    *idot = a;
    *csum = c;
    return sx * step * (double)a - sx * offset * (double)c;
}

/* W4A8 Q4_K GEMV rows: y[i] = sum over the row's weights of w * x_hat,
 * where w = (d*s_j)*q - dmin*m_j is the weight before any binary32 rounding
 * (the value the integer route computes) and x_hat = d_b * q_x. Each product
 * and the compensated sum are formed in binary64; s[i] = sum |w x_hat|. */
ORACLE_API void oracle_q4k_w4a8_rows(const uint8_t *blocks, int64_t k, const int8_t *qx, const float *dx,
                                     const int64_t *rows, int64_t nrows, double *y, double *sabs)
{
    int64_t nb = k / 256;
    for (int64_t ri = 0; ri < nrows; ++ri) {
        double sum = 0.0, comp = 0.0, sa = 0.0;
        for (int64_t b = 0; b < nb; ++b) {
            const uint8_t *blk = blocks + (rows[ri] * nb + b) * 144;
            double d = oracle_f16(rd_u16(blk + 0));
            double dmin = oracle_f16(rd_u16(blk + 2));
            unsigned sc[8], mn[8];
            oracle_q4k_unpack_scales(blk + 4, sc, mn);
            const uint8_t *qs = blk + 16;
            for (int c = 0; c < 4; ++c) {
                for (int l = 0; l < 32; ++l) {
                    for (int half = 0; half < 2; ++half) {
                        int j = 2 * c + half;
                        unsigned q = half ? (qs[32 * c + l] >> 4) : (qs[32 * c + l] & 15u);
                        int64_t e = b * 256 + 64 * c + 32 * half + l;
                        double w = d * (double)sc[j] * (double)q - dmin * (double)mn[j];
                        double p = w * ((double)dx[b] * (double)qx[e]);
                        double t = sum + p;
                        if (fabs(sum) >= fabs(p))
                            comp += (sum - t) + p;
                        else
                            comp += (p - t) + sum;
                        sum = t;
                        sa += fabs(p);
                    }
                }
            }
        }
        y[ri] = neumaier_value(sum, comp);
        sabs[ri] = sa;
    }
}

/* ------------------------------------------------------------------ */
/* NVFP4 x Q8_K, integer-exact ("a16_q8")                              */
/* ------------------------------------------------------------------ */

/* E2M1 element as an integer in units of 2^-1 (Q1): 2 * e2m1(code), one of
 * 0, +-1, +-2, +-3, +-4, +-6, +-8, +-12. [NV] section 7.4.2. */
ORACLE_API int oracle_e2m1_q1(unsigned code) { return (int)(2.0 * oracle_e2m1(code & 15u)); }

/* E4M3FN scale as an integer in units of 2^-9 (Q9): every finite E4M3FN
 * value is a multiple of 2^-9 (the smallest subnormal), up to 448 * 512.
 * The two NaN encodings have no Q9 value; they give 0 here and are rejected
 * by load-time validation. [NV] section 7.4.2. */
ORACLE_API int64_t oracle_e4m3fn_q9(unsigned b)
{
    double v = oracle_e4m3fn(b);
    if (v != v)
        return 0;
    return (int64_t)(v * 512.0);
}

/* binary32 to IEEE binary16 bits, round to nearest even; magnitudes from
 * 65520 up become infinity; subnormals are kept; NaN stays NaN (quiet). */
ORACLE_API unsigned oracle_f16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    unsigned sign = (u >> 16) & 0x8000u;
    double a = fabs((double)f);
    if (a != a)
        return sign | 0x7E00u;
    if (a >= 65520.0)
        return sign | 0x7C00u;
    if (a < 0x1p-14) {
        /* subnormal range: an integer count of 2^-24; 1024 is the smallest normal */
        return sign | (unsigned)nearbyint(a * 0x1p24);
    }
    int e;
    double m = frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
    double frac = nearbyint((m * 2.0 - 1.0) * 1024.0);
    e -= 1; /* a = (1 + frac / 1024) * 2^e */
    if (frac == 1024.0) {
        frac = 0.0;
        e += 1;
    }
    if (e + 15 >= 31)
        return sign | 0x7C00u;
    return sign | ((unsigned)(e + 15) << 10) | (unsigned)frac;
}

/* Rows of the integer-exact NVFP4 decode of [NV] section 7.4.2 against
 * Q8_K activations (q int8 [k], d = 1 / iscale per 256, from
 * oracle_q8_quantize): for each 256-element block b of the row,
 *   total_b = sum over its 16 groups g of
 *             (sum over the group of Q1(code) * q) * Q9(scale_g)
 * in int64 (exact, so the order of the additions does not matter), then
 * exactly these binary32 steps, blocks in ascending order from +0:
 *   c = fma(float(total_b), 2^-10, 0)     (Q1 x Q9 units)
 *   c = fma(c, d_b, 0)                     (activation scale 1 / iscale)
 *   c = fma(c, scale2, 0)                  (tensor scale)
 *   acc = fma(1, c, acc)
 * y32[i] = acc, y16[i] = binary16 bits of acc (round to nearest even).
 * Codes u8 [n][k/2] (low nibble = even element), scales u8 [n][k/16];
 * k a multiple of 256. */
ORACLE_API void oracle_nvfp4_a16q8_rows(const uint8_t *codes, const uint8_t *scales, float scale2, int64_t k,
                                        const int8_t *q, const float *d, const int64_t *rows, int64_t nrows,
                                        float *y32, uint16_t *y16)
{
    for (int64_t ri = 0; ri < nrows; ++ri) {
        const uint8_t *crow = codes + rows[ri] * (k / 2);
        const uint8_t *srow = scales + rows[ri] * (k / 16);
        float acc = 0.0f;
        for (int64_t b = 0; b < k / 256; ++b) {
            int64_t total = 0;
            for (int g = 0; g < 16; ++g) {
                int64_t dot = 0;
                for (int i = 0; i < 16; ++i) {
                    int64_t e = 256 * b + 16 * g + i;
                    dot += (int64_t)oracle_e2m1_q1(nibble_lo_even(crow, e)) * q[e];
                }
                total += dot * oracle_e4m3fn_q9(srow[16 * b + g]);
            }
            float c = fmaf((float)total, 0x1p-10f, 0.0f);
            c = fmaf(c, d[b], 0.0f);
            c = fmaf(c, scale2, 0.0f);
            acc = fmaf(1.0f, c, acc);
        }
        y32[ri] = acc;
        y16[ri] = (uint16_t)oracle_f16_rne(acc);
    }
}

/* ------------------------------------------------------------------ */
/* MX activations (OCP MX: E8M0 scale per 32) and the MX x MX product  */
/* ------------------------------------------------------------------ */

/* Nearest E2M1 code to v (already divided by the block scale), ties to the
 * even code (the OCP MX conversion rounds ties to even), magnitudes above
 * 6 saturate to 6. The sign of zero follows v. [FB] section 1 (the grid). */
ORACLE_API unsigned oracle_e2m1_rne(double v)
{
    static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    unsigned sign = signbit(v) ? 8u : 0u;
    double a = fabs(v);
    if (a > 6.0)
        a = 6.0; /* saturate first: for huge a every distance rounds to the same value */
    unsigned best = 0;
    for (unsigned c = 1; c < 8; ++c) {
        double dc = fabs(a - grid[c]), db = fabs(a - grid[best]);
        if (dc < db || (dc == db && (c & 1u) == 0))
            best = c;
    }
    return sign | best;
}

/* Nearest E4M3FN byte to v, ties to even, magnitudes above 448 saturate to
 * 448 (0x7E); subnormals kept. [FB] section 4 (the format). */
ORACLE_API unsigned oracle_e4m3fn_rne(double v)
{
    unsigned sign = signbit(v) ? 0x80u : 0u;
    double a = fabs(v);
    if (a >= 448.0)
        return sign | 0x7Eu;
    if (a < 0x1p-6) /* subnormal range: a multiple of 2^-9 */
        return sign | (unsigned)nearbyint(a * 512.0); /* 8 -> 0x08, the smallest normal */
    int e;
    double m = frexp(a, &e); /* a = m * 2^e, m in [0.5, 1) */
    double f = nearbyint((m * 2.0 - 1.0) * 8.0);
    e -= 1;
    if (f == 8.0) {
        f = 0.0;
        e += 1;
    }
    if (e > 8)
        return sign | 0x7Eu;
    return sign | ((unsigned)(e + 7) << 3) | (unsigned)f;
}

/* MX quantization of the rows of X [m][k] (binary32 or bfloat16 bits, row
 * stride ldx elements), k a multiple of 32, following the OCP MX
 * specification that [FB] section 3 and [WK] section 5 name as the contract:
 * per 32 consecutive elements, shared exponent e = floor(log2(max |x|)) -
 * emax (emax 2 for E2M1, 8 for E4M3), clamped to [-127, 127] (-127 for an
 * all-zero block); scale byte e + 127; each element quantized from x / 2^e to
 * the element grid with ties to even and saturation.
 * xfmt 1: E2M1 elements, codes [m][k/2] (low nibble = even element);
 * xfmt 7: E4M3FN elements, codes [m][k]. Scales [m][k/32]. */
ORACLE_API int oracle_mx_quantize(const void *x, int xdtype, int64_t m, int64_t k, int64_t ldx, int xfmt,
                                  uint8_t *codes, uint8_t *scales)
{
    if (xfmt != 1 && xfmt != 7)
        return 1;
    int emax = xfmt == 1 ? 2 : 8;
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t b = 0; b < k / 32; ++b) {
            double v[32];
            double amax = 0.0;
            for (int j = 0; j < 32; ++j) {
                int64_t e = i * ldx + 32 * b + j;
                v[j] = xdtype == 1 ? oracle_bf16_value(((const uint16_t *)x)[e]) : (double)((const float *)x)[e];
                if (fabs(v[j]) > amax)
                    amax = fabs(v[j]);
            }
            int se = -127;
            if (amax > 0.0) {
                int fe;
                frexp(amax, &fe); /* amax = f * 2^fe, f in [0.5, 1): floor(log2 amax) = fe - 1 */
                se = fe - 1 - emax;
                if (se < -127)
                    se = -127;
                if (se > 127)
                    se = 127;
            }
            scales[i * (k / 32) + b] = (uint8_t)(se + 127);
            for (int j = 0; j < 32; ++j) {
                double t = ldexp(v[j], -se);
                int64_t e = 32 * b + j;
                if (xfmt == 1) {
                    unsigned c = oracle_e2m1_rne(t);
                    uint8_t *p = codes + i * (k / 2) + e / 2;
                    if (e % 2 == 0)
                        *p = (uint8_t)((*p & 0xF0u) | c);
                    else
                        *p = (uint8_t)((*p & 0x0Fu) | (c << 4));
                } else {
                    codes[i * k + e] = (uint8_t)oracle_e4m3fn_rne(t);
                }
            }
        }
    }
    return 0;
}

/* Value of element e of an MX-quantized row (exact in binary64). */
static double mx_value(int xfmt, const uint8_t *codes_row, const uint8_t *scales_row, int64_t e)
{
    double s = oracle_e8m0(scales_row[e / 32]);
    if (xfmt == 1)
        return oracle_e2m1(nibble_lo_even(codes_row, e)) * s;
    return oracle_e4m3fn(codes_row[e]) * s;
}

/* Entries (ms[i], ns[i]) of Y = X_hat W_hat^T for MX-quantized activations
 * (xfmt 1 or 7, as above) and MXFP4 weights W [n][k/2] + E8M0 [n][k/32]:
 * every product is exact in binary64 and the sum is compensated; s[i] =
 * sum |x_hat w_hat|. */
ORACLE_API int oracle_mx_gemm_entries(const uint8_t *wcodes, const uint8_t *wscales, int64_t k, int xfmt,
                                      const uint8_t *xcodes, const uint8_t *xscales, const int64_t *ms,
                                      const int64_t *ns, int64_t count, double *y, double *sabs)
{
    if (xfmt != 1 && xfmt != 7)
        return 1;
    int64_t xrow = xfmt == 1 ? k / 2 : k;
    for (int64_t t = 0; t < count; ++t) {
        const uint8_t *xc = xcodes + ms[t] * xrow, *xs = xscales + ms[t] * (k / 32);
        const uint8_t *wc = wcodes + ns[t] * (k / 2), *ws = wscales + ns[t] * (k / 32);
        double sum = 0.0, comp = 0.0, sa = 0.0;
        for (int64_t e = 0; e < k; ++e) {
            double p = mx_value(xfmt, xc, xs, e) * (oracle_e2m1(nibble_lo_even(wc, e)) * oracle_e8m0(ws[e / 32]));
            double u = sum + p;
            if (fabs(sum) >= fabs(p))
                comp += (sum - u) + p;
            else
                comp += (p - u) + sum;
            sum = u;
            sa += fabs(p);
        }
        y[t] = neumaier_value(sum, comp);
        sabs[t] = sa;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* Encode-side helpers used only to reproduce the pages' worked facts  */
/* ------------------------------------------------------------------ */

/* Nearest scaled E2M1 code to w at scale s; on an exact tie the lowest
 * unsigned code wins (the lab convention of [FB] section 2). */
ORACLE_API unsigned oracle_e2m1_nearest(double w, double s)
{
    unsigned best = 0;
    double best_err = INFINITY;
    for (unsigned c = 0; c < 16; ++c) {
        double err = fabs(oracle_e2m1(c) * s - w);
        if (err < best_err) {
            best_err = err;
            best = c;
        }
    }
    return best;
}

/* Symmetric signed int4: q = clip(round(w/s), -8, 7) with round half to even,
 * stored as the 4-bit two's complement pattern. [WK] section 1. */
ORACLE_API unsigned oracle_int4_sym_code(double w, double s)
{
    double q = nearbyint(w / s);
    if (q < -8.0)
        q = -8.0;
    if (q > 7.0)
        q = 7.0;
    return (unsigned)((int)q & 15);
}

ORACLE_API int oracle_int4_sym_value(unsigned code)
{
    code &= 15u;
    return (code & 8u) ? (int)code - 16 : (int)code;
}

/* ------------------------------------------------------------------ */
/* Encode side: E2M1 with the two tie rules, NVFP4, INT4 symmetric,    */
/* bit planes                                                          */
/* ------------------------------------------------------------------ */

/* Nearest E2M1 code to v, magnitudes above 6 saturating to 6. tie 0: ties
 * to the even code (ModelOpt's midpoints, [NV] section 7.2); tie 1: the
 * lowest unsigned code ([FB] section 2, the lab convention). The sign of
 * zero follows v. */
ORACLE_API unsigned oracle_e2m1_round(double v, int tie)
{
    static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    unsigned sign = signbit(v) ? 8u : 0u;
    double a = fabs(v);
    if (a > 6.0)
        a = 6.0;
    unsigned best = 0;
    for (unsigned c = 1; c < 8; ++c) {
        double dc = fabs(a - grid[c]), db = fabs(a - grid[best]);
        if (dc < db || (dc == db && tie == 0 && (c & 1u) == 0))
            best = c; /* tie 1 keeps the lower code on an exact tie */
    }
    return sign | best;
}

/* NVFP4 quantization of the rows of X [m][k] (binary32 or bfloat16 bits,
 * row stride ldx), k a multiple of 16, for a given positive scale2 ([WK]
 * section 5: x = q_E2M1 * s_block(E4M3) * s_global; [NV] sections 7.1-7.2).
 * Per block of 16, in binary32 arithmetic:
 *   amax = max |x|; s = E4M3FN_RNE(RN32(amax / RN32(6 * scale2))) (the block
 *   maximum lands on the top E2M1 magnitude 6; saturating at 448);
 *   t = RN32(E4M3FN(s) * scale2);
 *   if t == 0 every code is +0; else code_i = E2M1(RN32(x_i / t)) with the
 *   tie rule (0 ties-to-even, 1 lowest code).
 * Codes [m][k/2] (low nibble = even element), scale bytes [m][k/16]. */
ORACLE_API int oracle_nvfp4_quantize(const void *x, int xdtype, int64_t m, int64_t k, int64_t ldx, float scale2,
                                     int tie, uint8_t *codes, uint8_t *scales)
{
    if (tie != 0 && tie != 1)
        return 1;
    const float den = 6.0f * scale2;
    for (int64_t i = 0; i < m; ++i)
        for (int64_t b = 0; b < k / 16; ++b) {
            float v[16], amax = 0.0f;
            for (int j = 0; j < 16; ++j) {
                int64_t e = i * ldx + 16 * b + j;
                v[j] = xdtype == 1 ? (float)oracle_bf16_value(((const uint16_t *)x)[e]) : ((const float *)x)[e];
                if (fabsf(v[j]) > amax)
                    amax = fabsf(v[j]);
            }
            const float qs = amax / den;
            const unsigned sb = oracle_e4m3fn_rne((double)qs) & 0x7Fu;
            scales[i * (k / 16) + b] = (uint8_t)sb;
            const float t = (float)oracle_e4m3fn(sb) * scale2;
            for (int j = 0; j < 16; j += 2) {
                unsigned lo = 0, hi = 0;
                if (t != 0.0f) {
                    lo = oracle_e2m1_round((double)(v[j] / t), tie);
                    hi = oracle_e2m1_round((double)(v[j + 1] / t), tie);
                }
                codes[i * (k / 2) + 8 * b + j / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    return 0;
}

/* Signed INT4 symmetric quantization ([WK] section 1): per group of `group`
 * consecutive elements of a row, s = RN32(max |w| / 7) and
 * q = clip(round_half_even(RN32(w / s)), -8, 7) (a zero group has s = 0 and
 * q = 0); codes two's-complement nibbles [m][k/2], the earlier element in
 * the low nibble; scales binary32 [m][k/group]. */
ORACLE_API void oracle_int4_sym_quantize(const void *w, int wdtype, int64_t m, int64_t k, int64_t ldw,
                                         int64_t group, uint8_t *codes, float *scales)
{
    for (int64_t i = 0; i < m; ++i)
        for (int64_t g = 0; g < k / group; ++g) {
            float amax = 0.0f;
            for (int64_t j = 0; j < group; ++j) {
                int64_t e = i * ldw + g * group + j;
                float v = wdtype == 1 ? (float)oracle_bf16_value(((const uint16_t *)w)[e]) : ((const float *)w)[e];
                if (fabsf(v) > amax)
                    amax = fabsf(v);
            }
            const float sc = amax / 7.0f;
            scales[i * (k / group) + g] = sc;
            for (int64_t j = 0; j < group; ++j) {
                int64_t e = i * ldw + g * group + j;
                float v = wdtype == 1 ? (float)oracle_bf16_value(((const uint16_t *)w)[e]) : ((const float *)w)[e];
                int q = 0;
                if (sc != 0.0f) {
                    double r = nearbyint((double)(v / sc));
                    q = r < -8.0 ? -8 : r > 7.0 ? 7 : (int)r;
                }
                int64_t c = g * group + j;
                uint8_t *byte = &codes[i * (k / 2) + c / 2];
                unsigned nib = (unsigned)q & 15u;
                *byte = (c & 1) ? (uint8_t)((*byte & 0x0Fu) | (nib << 4)) : (uint8_t)((*byte & 0xF0u) | nib);
            }
        }
}

/* Bit-plane split of b-bit codes ([BP] "Odd widths"): the low `lo` bits of
 * every value form one little-endian word stream and the high b - lo bits
 * another, each packed as oracle_pack_bits does (GGUF's Q6_K keeps 4 + 2).
 * count * lo and count * (b - lo) must be multiples of 32. */
ORACLE_API void oracle_pack_planes(const uint32_t *vals, int64_t count, int bits, int lo, uint32_t *lo_words,
                                   uint32_t *hi_words, uint32_t *scratch)
{
    for (int64_t i = 0; i < count; ++i)
        scratch[i] = vals[i] & ((1u << lo) - 1u);
    oracle_pack_bits(scratch, count, lo, lo_words);
    for (int64_t i = 0; i < count; ++i)
        scratch[i] = vals[i] >> lo;
    oracle_pack_bits(scratch, count, bits - lo, hi_words);
}

ORACLE_API void oracle_unpack_planes(const uint32_t *lo_words, const uint32_t *hi_words, int64_t count, int bits,
                                     int lo, uint32_t *vals, uint32_t *scratch)
{
    oracle_unpack_bits(lo_words, count, lo, vals);
    oracle_unpack_bits(hi_words, count, bits - lo, scratch);
    for (int64_t i = 0; i < count; ++i)
        vals[i] |= scratch[i] << lo;
}
