/*
 * kvq_oracle.c -- plain CPU reference for thought-adaptive quantised,
 * evictable paged-KV decode attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the slow, obviously-correct model that
 * the GPU library is checked against.  Only the test suite, the smoke check
 * and the CPU-baseline leg of the benchmark may load it; the product path
 * never does.  It shares no code, header or table with the GPU library: the
 * cache format is re-derived here from its written definition.
 *
 * Sources (web pages, cited by title and section):
 *  [ThinKV]   "ThinKV: Thought-Adaptive KV Cache Compression for Efficient
 *             Reasoning Models", technical summary, Methodology:
 *             - "Thought-Adaptive Quantization (TBQ)": per-token precision
 *               chosen by thought type, R > E > T, via group quantisation;
 *             - "System Implementation: Continuous Thinking (CT)": a paged
 *               block table that records thought type, start index and
 *               eviction mask, and lets new tokens of the same thought type
 *               overwrite evicted slots in place, without gather compaction.
 *  [DynTS]    "Dynamic Thinking-Token Selection ..." technical summary,
 *             section 2.3 (dual-window KV selection): question window never
 *             evicted, local window of recent tokens kept, top-k by
 *             importance kept inside the selection window.
 *  [TAM]      "Thought-Aware KV Cache Compaction for Reasoning via Adaptive
 *             Attention Matching", sections 1 and 2.B: attention mass
 *             received by a token is its importance signal.
 *  [Surprise] "Back from the Future: Key-Value Cache Management by
 *             Counter-Causal Surprise", Problem Statement: scaled
 *             dot-product attention over the KV cache; H2O-style cumulative
 *             attention scores.
 *
 * Readings where the pages are silent (all listed in the design notes):
 *  - bits per thought type: R=8, E=4, T=2; asymmetric min/max integer
 *    codes, group of 32 channels, fp16 (scale, zero) per group;
 *  - scale is the smallest fp16 >= (max-min)/(2^b-1) computed in fp32,
 *    zero is the group minimum, codes are
 *    rint((x-zero)/scale) (ties to even) clamped to [0, 2^b-1], all in fp32;
 *    a -0 group minimum or maximum is taken as +0;
 *  - query head h reads kv head h / (Hq/Hkv);
 *  - mass of a position = sum over all Hq query heads of its softmax
 *    probability; importance' = decay * importance + mass;
 *  - append takes the first free slot (table order, then slot order) of a
 *    block of the token's own type, else pops the type's free stack
 *    (sequences in batch order) and appends that block to the table;
 *  - eviction keeps positions < q_window and >= seq_len - recent_window,
 *    plus the keep_k best (importance desc, position asc) of the rest;
 *    afterwards every table entry whose mask is empty is removed (order
 *    kept) and its block id pushed on its pool's free stack (table order,
 *    sequences in batch order).
 *
 * Parity pins: every function here is exercised against closed forms,
 * numpy's float16 conversion, torch's scaled-dot-product attention in
 * fp64, brute-force lexsort top-k and hand-derived tiny scenarios by the
 * CPU test suite.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define HD 128  /* head dimension */
#define BLK 16  /* slots per block */
#define GS 32   /* channels per quantisation group */
#define NGRP (HD / GS)
#define TAG_SKIP 0xFF

#define ST_OK 0
#define ST_EINVAL (-1)
#define ST_ENOSPC (-4)

/* ------------------------------------------------------------------ */
/* IEEE 754 binary16, written out from its definition                   */
/* ------------------------------------------------------------------ */

double orc_half_to_double(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);               /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);   /* 1.m * 2^(e-15) */
    return sign ? -v : v;
}

/* Round a float to binary16, ties to even. */
uint16_t orc_float_to_half(float f)
{
    double v = (double)f;                        /* exact */
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return (uint16_t)(sign | 0x7e00);
    if (a >= 65520.0)                            /* at or past the midpoint above 65504 */
        return (uint16_t)(sign | 0x7c00);
    if (a < ldexp(1.0, -14)) {                   /* subnormal range, step 2^-24 */
        double q = nearbyint(ldexp(a, 24));      /* default mode: ties to even */
        return (uint16_t)(sign | (uint16_t)q);   /* q == 1024 is the least normal */
    }
    int ex;
    frexp(a, &ex);                               /* a in [2^(ex-1), 2^ex) */
    int E = ex - 1;
    double q = nearbyint(ldexp(a, 10 - E));      /* 11 significant bits: [1024, 2048] */
    if (q == 2048.0) {
        q = 1024.0;
        E += 1;
    }
    if (E > 15)
        return (uint16_t)(sign | 0x7c00);
    return (uint16_t)(sign | ((E + 15) << 10) | (int)(q - 1024.0));
}

/* ------------------------------------------------------------------ */
/* TBQ: asymmetric group quantisation [ThinKV, Methodology, TBQ]         */
/* ------------------------------------------------------------------ */

int orc_pool_bits(int pool) { return 8 >> pool; }  /* R=0:8, E=1:4, T=2:2 */

void orc_quantize_group(const uint16_t *x, int bits, uint16_t *scale_h,
                        uint16_t *zero_h, uint8_t *codes)
{
    const int lv = (1 << bits) - 1;
    float mn = (float)orc_half_to_double(x[0]);
    float mx = mn;
    for (int i = 1; i < GS; ++i) {
        float v = (float)orc_half_to_double(x[i]);
        if (v < mn) mn = v;
        if (v > mx) mx = v;
    }
    if (mn == 0.0f)
        mn = fabsf(mn);                          /* -0 counts as +0 */
    if (mx == 0.0f)
        mx = fabsf(mx);
    float s32 = (mx - mn) / (float)lv;           /* fp32 subtract, fp32 divide */
    uint16_t sh = orc_float_to_half(s32);
    if (orc_half_to_double(sh) < (double)s32)
        sh = (uint16_t)(sh + 1);                 /* next binary16 up (s32 >= 0) */
    *scale_h = sh;
    *zero_h = orc_float_to_half(mn);             /* exact: mn is a binary16 value */
    float sc = (float)orc_half_to_double(sh);
    for (int i = 0; i < GS; ++i) {
        if (sc == 0.0f) {
            codes[i] = 0;
            continue;
        }
        float t = ((float)orc_half_to_double(x[i]) - mn) / sc;
        t = rintf(t);                            /* ties to even */
        if (t < 0.0f) t = 0.0f;
        if (t > (float)lv) t = (float)lv;
        codes[i] = (uint8_t)t;
    }
}

/* ------------------------------------------------------------------ */
/* ThinKV's own formats [ThinKV, Methodology, TBQ]: FP8 for Reasoning,  */
/* FP4 for Execution, ternary for Transition                          */
/* ------------------------------------------------------------------ */

/* A sign-magnitude minifloat with E exponent bits (bias), M mantissa bits,
 * subnormals at exponent field 0 and no infinities: the OCP formats
 * E4M3 (bias 7, largest magnitude code 0x7E = 448; 0x7F is NaN) and E2M1
 * (bias 1, largest 7 = 6).  Value of a magnitude code. */
double orc_mini_value(unsigned mag, int E, int M, int bias)
{
    unsigned e = mag >> M, m = mag & ((1u << M) - 1);
    if (e == 0)
        return ldexp((double)m, 1 - bias - M);
    return ldexp(1.0 + ldexp((double)m, -M), (int)e - bias);
}

/* Nearest code to y (ties to the even code), magnitudes above the largest
 * code saturating to it; the sign bit is set only for a nonzero magnitude
 * of a negative y. */
unsigned orc_mini_encode(float y, int E, int M, int bias, unsigned max_mag)
{
    double a = fabs((double)y);
    unsigned mag;
    double emin_pow = ldexp(1.0, 1 - bias);        /* least normal magnitude */
    if (a < emin_pow) {
        /* subnormal grid, step 2^(1 - bias - M); q == 2^M is the least normal */
        mag = (unsigned)nearbyint(ldexp(a, bias - 1 + M));
    } else {
        int ex;
        frexp(a, &ex);                             /* a in [2^(ex-1), 2^ex) */
        int e = ex - 1;
        double q = nearbyint(ldexp(a, M - e));     /* M+1 significant bits */
        if (q == ldexp(1.0, M + 1)) {
            q = ldexp(1.0, M);
            e += 1;
        }
        long eb = (long)e + bias;
        if (eb > (1L << E) - 1)
            mag = max_mag;
        else
            mag = (unsigned)((eb << M) | (long)(q - ldexp(1.0, M)));
    }
    if (mag > max_mag)
        mag = max_mag;
    unsigned sign = (y < 0.0f && mag != 0) ? 1u : 0u;
    return (sign << (E + M)) | mag;
}

static const int MINI_E[2] = {4, 2}, MINI_M[2] = {3, 1}, MINI_BIAS[2] = {7, 1};
static const unsigned MINI_MAX[2] = {0x7e, 0x7};
static const float MINI_TOP[2] = {448.0f, 6.0f};

/* Value of a native code of pool 0 (E4M3) or 1 (E2M1), before the scale. */
double orc_native_value(int pool, unsigned code)
{
    int E = MINI_E[pool], M = MINI_M[pool];
    double v = orc_mini_value(code & ((1u << (E + M)) - 1), E, M, MINI_BIAS[pool]);
    return (code >> (E + M)) & 1 ? -v : v;
}

/* Symmetric group quantisation in the native formats.  amax = max |x|
 * (-0 as +0); scale = the least fp16 >= amax / top in fp32 (top = 448, 6,
 * 1 for E4M3, E2M1, ternary); y = x / scale in fp32.  Pools 0 and 1 store
 * the minifloat code of y and zero 0 (x^ = value(code) * scale).  Pool 2
 * stores t + 1 for t = rint(y) clamped to [-1, 1] (ties to even) and
 * zero = -scale, so that x^ = code * scale + zero is -scale, 0 or +scale.
 * A group of zeros stores scale 0, zero 0 and the code of 0. */
void orc_quantize_group_native(const uint16_t *x, int pool, uint16_t *scale_h, uint16_t *zero_h,
                               uint8_t *codes)
{
    float amax = 0.0f;
    for (int i = 0; i < GS; ++i) {
        float v = fabsf((float)orc_half_to_double(x[i]));
        if (v > amax) amax = v;
    }
    float top = pool == 2 ? 1.0f : MINI_TOP[pool];
    float s32 = amax / top;
    uint16_t sh = orc_float_to_half(s32);
    if (orc_half_to_double(sh) < (double)s32)
        sh = (uint16_t)(sh + 1);
    *scale_h = sh;
    *zero_h = (pool == 2 && sh != 0) ? (uint16_t)(sh | 0x8000) : 0;
    float sc = (float)orc_half_to_double(sh);
    for (int i = 0; i < GS; ++i) {
        if (sc == 0.0f) {
            codes[i] = pool == 2 ? 1 : 0;
            continue;
        }
        float y = (float)orc_half_to_double(x[i]) / sc;
        if (pool == 2) {
            float t = rintf(y);
            if (t < -1.0f) t = -1.0f;
            if (t > 1.0f) t = 1.0f;
            codes[i] = (uint8_t)(t + 1.0f);
        } else {
            codes[i] = (uint8_t)orc_mini_encode(y, MINI_E[pool], MINI_M[pool], MINI_BIAS[pool], MINI_MAX[pool]);
        }
    }
}

/* ------------------------------------------------------------------ */
/* Cache format (one region per (pool, block, kv head))                 */
/*   [K codes 256*b B][V codes 256*b B][K (scale,zero) 256 B][V ... ]    */
/* ------------------------------------------------------------------ */

long orc_region_bytes(int bits) { return 512L * bits + 512L; }

/* Index (in codes) of K channel d inside a token's 128-code K row. */
int orc_k_row_index(int bits, int d)
{
    int g = d >> 5, kb = (d >> 3) & 3, e = d & 7;
    if (bits == 8)
        return 32 * kb + 8 * g + e;
    if (bits == 4)
        return 32 * kb + 8 * g + 4 * (e & 1) + (e >> 1);
    return 32 * kb + 16 * (g >> 1) + 8 * (e & 1) + 4 * (g & 1) + (e >> 1);
}

/* Bit offset of K code (t, d) inside the K-code area of a region. */
long orc_k_bit_offset(int bits, int t, int d)
{
    return ((long)t * HD + orc_k_row_index(bits, d)) * bits;
}

/* Bit offset of V code (t, d) inside the V-code area of a region. */
long orc_v_bit_offset(int bits, int t, int d)
{
    int r = t >> 2, tt = t & 3, n = d >> 4, j = d & 15;
    int L = 16 * r + j;
    int per = 8 / bits;                          /* 16-channel tiles per dword */
    int w = n / per, m = n % per;
    int c = (tt & 1) * (16 / bits) + 2 * m + (tt >> 1);
    long byte;
    if (bits == 8)
        byte = (long)(w >> 2) * 1024 + L * 16 + (w & 3) * 4;
    else if (bits == 4)
        byte = (long)L * 16 + w * 4;
    else
        byte = (long)L * 8 + w * 4;
    return byte * 8 + (long)c * bits;
}

static unsigned get_code(const uint8_t *area, long bit, int bits)
{
    return (area[bit >> 3] >> (bit & 7)) & ((1u << bits) - 1);
}

static void put_code(uint8_t *area, long bit, int bits, unsigned code)
{
    unsigned msk = ((1u << bits) - 1) << (bit & 7);
    area[bit >> 3] = (uint8_t)((area[bit >> 3] & ~msk) | ((code << (bit & 7)) & msk));
}

/* (scale, zero) of group g of token t: K at 512*b, V at 512*b + 256. */
static const uint16_t *sz_ptr(const uint8_t *region, int bits, int is_v, int t, int g)
{
    return (const uint16_t *)(region + 512L * bits + (is_v ? 256 : 0) + (t * NGRP + g) * 4);
}

/* ------------------------------------------------------------------ */
/* Cache state: the same arrays the GPU library works on                */
/* ------------------------------------------------------------------ */

typedef struct {
    int32_t B, Hq, Hkv, max_blocks, n_cap;
    int32_t pool_blocks[3];
    int32_t codec;           /* 0 integer min/max, 1 ThinKV's formats */
    uint8_t *kv[3];          /* [pool_blocks][Hkv] regions            */
    uint16_t *mask[3];       /* [pool_blocks] valid-slot bitmask      */
    int32_t *pos[3];         /* [pool_blocks][16] logical positions   */
    uint32_t *table;         /* [B][max_blocks]  (pool << 30) | id    */
    int32_t *n_blocks;       /* [B]                                   */
    int32_t *seq_len;        /* [B]  next logical position            */
    uint32_t *free_ids[3];   /* [pool_blocks] LIFO stacks             */
    int32_t *free_top;       /* [3]                                   */
    int32_t *status;         /* [1]                                   */
} orc_cache;

static uint8_t *region_of(const orc_cache *c, int pool, uint32_t id, int h)
{
    return c->kv[pool] + ((long)id * c->Hkv + h) * orc_region_bytes(orc_pool_bits(pool));
}

/* Quantise one token's K and V rows for kv head h and store them in slot t. */
static void write_token(orc_cache *c, int pool, uint32_t id, int h, int t,
                        const uint16_t *k, const uint16_t *v)
{
    int bits = orc_pool_bits(pool);
    uint8_t *reg = region_of(c, pool, id, h);
    uint8_t *kc = reg, *vc = reg + 256L * bits;
    for (int g = 0; g < NGRP; ++g) {
        uint16_t sc, zr;
        uint8_t codes[GS];
        uint16_t *kz = (uint16_t *)sz_ptr(reg, bits, 0, t, g);
        if (c->codec == 1)
            orc_quantize_group_native(k + g * GS, pool, &sc, &zr, codes);
        else
            orc_quantize_group(k + g * GS, bits, &sc, &zr, codes);
        kz[0] = sc;
        kz[1] = zr;
        for (int i = 0; i < GS; ++i)
            put_code(kc, orc_k_bit_offset(bits, t, g * GS + i), bits, codes[i]);
        uint16_t *vz = (uint16_t *)sz_ptr(reg, bits, 1, t, g);
        if (c->codec == 1)
            orc_quantize_group_native(v + g * GS, pool, &sc, &zr, codes);
        else
            orc_quantize_group(v + g * GS, bits, &sc, &zr, codes);
        vz[0] = sc;
        vz[1] = zr;
        for (int i = 0; i < GS; ++i)
            put_code(vc, orc_v_bit_offset(bits, t, g * GS + i), bits, codes[i]);
    }
}

/* Dequantised K and V of slot t for kv head h, in fp64: x = code*scale + zero,
 * or for the native formats of pools 0 and 1, value(code)*scale + zero. */
void orc_dequant_slot(const orc_cache *c, int pool, uint32_t id, int h, int t,
                      double *k_out, double *v_out)
{
    int bits = orc_pool_bits(pool);
    const uint8_t *reg = region_of(c, pool, id, h);
    const uint8_t *kc = reg, *vc = reg + 256L * bits;
    for (int d = 0; d < HD; ++d) {
        const uint16_t *kz = sz_ptr(reg, bits, 0, t, d / GS);
        const uint16_t *vz = sz_ptr(reg, bits, 1, t, d / GS);
        unsigned ck = get_code(kc, orc_k_bit_offset(bits, t, d), bits);
        unsigned cv = get_code(vc, orc_v_bit_offset(bits, t, d), bits);
        double qk = ck, qv = cv;
        if (c->codec == 1 && pool < 2) {
            qk = orc_native_value(pool, ck);
            qv = orc_native_value(pool, cv);
        }
        if (k_out) k_out[d] = qk * orc_half_to_double(kz[0]) + orc_half_to_double(kz[1]);
        if (v_out) v_out[d] = qv * orc_half_to_double(vz[0]) + orc_half_to_double(vz[1]);
    }
}

/* Raw codes of slot t (logical channel order), for byte-level checks. */
void orc_slot_codes(const orc_cache *c, int pool, uint32_t id, int h, int t,
                    uint8_t *k_codes, uint8_t *v_codes, uint16_t *k_sz, uint16_t *v_sz)
{
    int bits = orc_pool_bits(pool);
    const uint8_t *reg = region_of(c, pool, id, h);
    for (int d = 0; d < HD; ++d) {
        k_codes[d] = (uint8_t)get_code(reg, orc_k_bit_offset(bits, t, d), bits);
        v_codes[d] = (uint8_t)get_code(reg + 256L * bits, orc_v_bit_offset(bits, t, d), bits);
    }
    for (int g = 0; g < NGRP; ++g) {
        memcpy(k_sz + 2 * g, sz_ptr(reg, bits, 0, t, g), 4);
        memcpy(v_sz + 2 * g, sz_ptr(reg, bits, 1, t, g), 4);
    }
}

/* Store given codes into slot t (used by the pack/unpack pins). */
void orc_put_slot_codes(orc_cache *c, int pool, uint32_t id, int h, int t,
                        const uint8_t *k_codes, const uint8_t *v_codes)
{
    int bits = orc_pool_bits(pool);
    uint8_t *reg = region_of(c, pool, id, h);
    for (int d = 0; d < HD; ++d) {
        put_code(reg, orc_k_bit_offset(bits, t, d), bits, k_codes[d]);
        put_code(reg + 256L * bits, orc_v_bit_offset(bits, t, d), bits, v_codes[d]);
    }
}

/* ------------------------------------------------------------------ */
/* Append one token per sequence [ThinKV, Methodology, CT]               */
/* ------------------------------------------------------------------ */

/*
 * k_new, v_new: fp16 [B][Hkv][128]; tags: [B], 0=R 1=E 2=T, 0xFF = no token.
 * Sequences are served in batch order.  A sequence that cannot be served
 * (pool or table exhausted, position space full) is left untouched and the
 * status word is set to ENOSPC; a bad tag sets EINVAL.
 */
void orc_append(orc_cache *c, const uint16_t *k_new, const uint16_t *v_new, const uint8_t *tags)
{
    for (int b = 0; b < c->B; ++b) {
        int tag = tags[b];
        if (tag == TAG_SKIP)
            continue;
        if (tag > 2) {
            *c->status = ST_EINVAL;
            continue;
        }
        int pool = tag;
        if (c->seq_len[b] >= c->n_cap) {
            *c->status = ST_ENOSPC;
            continue;
        }
        uint32_t *row = c->table + (long)b * c->max_blocks;
        long id = -1;
        int slot = -1;
        /* first free slot of a same-type block, in table order then slot order */
        for (int e = 0; e < c->n_blocks[b] && id < 0; ++e) {
            if ((int)(row[e] >> 30) != pool)
                continue;
            uint32_t bid = row[e] & 0x3fffffffu;
            uint16_t m = c->mask[pool][bid];
            if (m == 0xffff)
                continue;
            for (slot = 0; (m >> slot) & 1; ++slot)
                ;
            id = bid;
        }
        if (id < 0) {
            if (c->n_blocks[b] >= c->max_blocks || c->free_top[pool] == 0) {
                *c->status = ST_ENOSPC;
                continue;
            }
            id = c->free_ids[pool][--c->free_top[pool]];
            row[c->n_blocks[b]++] = ((uint32_t)pool << 30) | (uint32_t)id;
            c->mask[pool][id] = 0;
            slot = 0;
        }
        for (int h = 0; h < c->Hkv; ++h)
            write_token(c, pool, (uint32_t)id, h, slot,
                        k_new + ((long)b * c->Hkv + h) * HD,
                        v_new + ((long)b * c->Hkv + h) * HD);
        c->mask[pool][id] |= (uint16_t)(1u << slot);
        c->pos[pool][id * BLK + slot] = c->seq_len[b];
        c->seq_len[b] += 1;
    }
}

/* ------------------------------------------------------------------ */
/* Decode attention, mass and importance                                 */
/* [Surprise, Problem Statement] scaled dot-product attention;           */
/* [TAM, 1 and 2.B] attention mass; [Surprise] H2O cumulative score.     */
/* ------------------------------------------------------------------ */

typedef struct {
    int pool;
    uint32_t id;
    int slot, pos;
} valid_slot;

static int list_valid(const orc_cache *c, int b, valid_slot *out)
{
    const uint32_t *row = c->table + (long)b * c->max_blocks;
    int n = 0;
    for (int e = 0; e < c->n_blocks[b]; ++e) {
        int pool = (int)(row[e] >> 30);
        uint32_t id = row[e] & 0x3fffffffu;
        uint16_t m = c->mask[pool][id];
        for (int s = 0; s < BLK; ++s)
            if ((m >> s) & 1) {
                out[n].pool = pool;
                out[n].id = id;
                out[n].slot = s;
                out[n].pos = c->pos[pool][id * BLK + s];
                ++n;
            }
    }
    return n;
}

/*
 * q: fp16 [B][Hq][128].  out: fp64 [B][Hq][128].  mass: fp64 [B][n_cap],
 * written for positions < seq_len (0 where no valid slot holds the
 * position).  If imp_in is non-null, imp_out[b][pos] =
 * float(decay*imp_in + mass) at valid positions and imp_in elsewhere.
 * want: optional [B] flags; sequences with want[b]==0 are skipped.
 *
 * Each (sequence, kv head) is independent, so OpenMP runs over those
 * pairs.  A pair sums the probabilities its G query heads give each valid
 * slot (heads in order); the mass of a position is then the sum of those
 * per-kv-head sums in kv-head order, i.e. the sum over all Hq heads.
 */
void orc_decode(const orc_cache *c, const uint16_t *q, double sm_scale,
                double *out, double *mass, const float *imp_in, float *imp_out,
                double decay, const uint8_t *want)
{
    const int G = c->Hq / c->Hkv, B = c->B, Hkv = c->Hkv;
    valid_slot **vs = calloc((size_t)B, sizeof(valid_slot *));
    int *nv = calloc((size_t)B, sizeof(int));
    double **mslot = calloc((size_t)B, sizeof(double *));   /* [Hkv][n] per sequence */
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        if (want && !want[b])
            continue;
        long cap = (long)c->n_blocks[b] * BLK + 1;
        vs[b] = malloc(sizeof(valid_slot) * cap);
        nv[b] = list_valid(c, b, vs[b]);
        mslot[b] = calloc((size_t)Hkv * (nv[b] + 1), sizeof(double));
    }
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        for (int kh = 0; kh < Hkv; ++kh) {
            if (want && !want[b])
                continue;
            const int n = nv[b];
            const valid_slot *sl = vs[b];
            double *K = malloc(sizeof(double) * HD * (n + 1));
            double *V = malloc(sizeof(double) * HD * (n + 1));
            double *s = malloc(sizeof(double) * (n + 1));
            double *ms = mslot[b] + (long)kh * (n + 1);
            for (int t = 0; t < n; ++t)
                orc_dequant_slot(c, sl[t].pool, sl[t].id, kh, sl[t].slot, K + (long)t * HD,
                                 V + (long)t * HD);
            for (int h = kh * G; h < (kh + 1) * G; ++h) {
                const uint16_t *qh = q + ((long)b * c->Hq + h) * HD;
                double *oh = out + ((long)b * c->Hq + h) * HD;
                double qd[HD];
                for (int d = 0; d < HD; ++d)
                    qd[d] = orc_half_to_double(qh[d]);
                double M = -INFINITY;
                for (int t = 0; t < n; ++t) {
                    double acc = 0.0;
                    for (int d = 0; d < HD; ++d)
                        acc += qd[d] * K[(long)t * HD + d];
                    s[t] = acc * sm_scale;
                    if (s[t] > M) M = s[t];
                }
                double L = 0.0;
                for (int t = 0; t < n; ++t) {
                    s[t] = exp(s[t] - M);
                    L += s[t];
                }
                for (int d = 0; d < HD; ++d)
                    oh[d] = 0.0;
                for (int t = 0; t < n; ++t) {
                    double p = s[t] / L;
                    for (int d = 0; d < HD; ++d)
                        oh[d] += p * V[(long)t * HD + d];
                    ms[t] += p;
                }
            }
            free(K);
            free(V);
            free(s);
        }
    }
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        if (want && !want[b])
            continue;
        const int n = nv[b];
        double *mrow = mass + (long)b * c->n_cap;
        for (int p = 0; p < c->seq_len[b]; ++p)
            mrow[p] = 0.0;
        for (int t = 0; t < n; ++t) {
            double m = 0.0;
            for (int kh = 0; kh < Hkv; ++kh)
                m += mslot[b][(long)kh * (n + 1) + t];
            mrow[vs[b][t].pos] = m;
        }
        if (imp_in && imp_out) {
            const float *ii = imp_in + (long)b * c->n_cap;
            float *io = imp_out + (long)b * c->n_cap;
            for (int p = 0; p < c->n_cap; ++p)
                io[p] = ii[p];
            for (int t = 0; t < n; ++t)
                io[vs[b][t].pos] = (float)(decay * (double)ii[vs[b][t].pos] + mrow[vs[b][t].pos]);
        }
        free(vs[b]);
        free(mslot[b]);
    }
    free(vs);
    free(nv);
    free(mslot);
}

/* ------------------------------------------------------------------ */
/* Windowed top-k eviction and metadata-only compaction                  */
/* [DynTS, 2.3]; [ThinKV, Methodology, CT]                               */
/* ------------------------------------------------------------------ */

typedef struct {
    float imp;
    int pos;
    int pool;
    uint32_t id;
    int slot;
} cand;

static int cand_cmp(const void *a, const void *b)
{
    const cand *x = a, *y = b;
    if (x->imp > y->imp) return -1;   /* larger importance first */
    if (x->imp < y->imp) return 1;
    return (x->pos > y->pos) - (x->pos < y->pos);  /* then lower position */
}

/*
 * importance: fp32 [B][n_cap] indexed by position; keep_k: [B].
 * Per sequence: positions < q_window and >= seq_len - recent_window are
 * protected; of the other valid slots the keep_k best survive.  Then all
 * table entries with an empty mask are dropped (order kept) and their
 * ids pushed on their pool's free stack (table order, batch order).
 */
void orc_evict(orc_cache *c, const float *importance, const int32_t *keep_k,
               int q_window, int recent_window)
{
    for (int b = 0; b < c->B; ++b) {
        uint32_t *row = c->table + (long)b * c->max_blocks;
        const float *imp = importance + (long)b * c->n_cap;
        int lo = q_window, hi = c->seq_len[b] - recent_window;
        long cap = (long)c->n_blocks[b] * BLK + 1;
        cand *cs = malloc(sizeof(cand) * cap);
        int n = 0;
        for (int e = 0; e < c->n_blocks[b]; ++e) {
            int pool = (int)(row[e] >> 30);
            uint32_t id = row[e] & 0x3fffffffu;
            uint16_t m = c->mask[pool][id];
            for (int s = 0; s < BLK; ++s) {
                if (!((m >> s) & 1))
                    continue;
                int p = c->pos[pool][id * BLK + s];
                if (p < lo || p >= hi)
                    continue;
                cs[n].imp = imp[p];
                cs[n].pos = p;
                cs[n].pool = pool;
                cs[n].id = id;
                cs[n].slot = s;
                ++n;
            }
        }
        int k = keep_k[b] < 0 ? 0 : keep_k[b];
        if (n > k) {
            qsort(cs, n, sizeof(cand), cand_cmp);
            for (int i = k; i < n; ++i)
                c->mask[cs[i].pool][cs[i].id] &= (uint16_t)~(1u << cs[i].slot);
        }
        free(cs);
        int kept = 0;
        for (int e = 0; e < c->n_blocks[b]; ++e) {
            int pool = (int)(row[e] >> 30);
            uint32_t id = row[e] & 0x3fffffffu;
            if (c->mask[pool][id] == 0)
                c->free_ids[pool][c->free_top[pool]++] = id;
            else
                row[kept++] = row[e];
        }
        c->n_blocks[b] = kept;
    }
}

/* Table compaction after mask changes: entries with an empty mask leave
 * the row (order kept) and their ids go on their pool's free stack. */
static void compact_row(orc_cache *c, int b)
{
    uint32_t *row = c->table + (long)b * c->max_blocks;
    int kept = 0;
    for (int e = 0; e < c->n_blocks[b]; ++e) {
        int pool = (int)(row[e] >> 30);
        uint32_t id = row[e] & 0x3fffffffu;
        if (c->mask[pool][id] == 0)
            c->free_ids[pool][c->free_top[pool]++] = id;
        else
            row[kept++] = row[e];
    }
    c->n_blocks[b] = kept;
}

static int pos_cmp(const void *a, const void *b)
{
    const cand *x = a, *y = b;
    return (x->pos > y->pos) - (x->pos < y->pos);
}

/*
 * Thought-adaptive eviction ("ThinKV", Methodology, think-before-evict):
 * once a Transition thought starts, earlier Reasoning / Execution segments
 * are pruned at segment granularity on an annealing schedule, and a small
 * safety net of every earlier Transition segment stays.
 *
 * Per sequence: the candidates are the valid slots with q_window <= pos <
 * seq_len - recent_window.  Taken in position order they form segments,
 * maximal runs of one thought type.  A segment followed by k Transition
 * segments keeps everything if k == 0; otherwise it keeps
 * max(r_min, r0 >> (k - 1)) slots if it is a Reasoning or Execution segment
 * (r0 after the first later Transition, r0 / 2 after the second, ...) and
 * t_keep slots if it is a Transition segment.  A segment keeps its best
 * slots: larger importance first, then lower position.  Then the table is
 * compacted as in orc_evict.  seq_mask (NULL: every sequence) names the
 * sequences the eviction fires for; the others are skipped whole.
 */
void orc_evict_tbe(orc_cache *c, const float *importance, const uint8_t *seq_mask, int r0,
                   int r_min, int t_keep, int q_window, int recent_window)
{
    for (int b = 0; b < c->B; ++b) {
        /* the eviction fires per sequence, where a Transition thought was
         * detected ("ThinKV", Methodology, think-before-evict); the others
         * stay exactly as they are */
        if (seq_mask && !seq_mask[b])
            continue;
        uint32_t *row = c->table + (long)b * c->max_blocks;
        const float *imp = importance + (long)b * c->n_cap;
        int lo = q_window, hi = c->seq_len[b] - recent_window;
        long cap = (long)c->n_blocks[b] * BLK + 1;
        cand *cs = malloc(sizeof(cand) * cap);
        int n = 0;
        for (int e = 0; e < c->n_blocks[b]; ++e) {
            int pool = (int)(row[e] >> 30);
            uint32_t id = row[e] & 0x3fffffffu;
            uint16_t m = c->mask[pool][id];
            for (int s = 0; s < BLK; ++s) {
                if (!((m >> s) & 1))
                    continue;
                int p = c->pos[pool][id * BLK + s];
                if (p < lo || p >= hi)
                    continue;
                cs[n].imp = imp[p];
                cs[n].pos = p;
                cs[n].pool = pool;
                cs[n].id = id;
                cs[n].slot = s;
                ++n;
            }
        }
        qsort(cs, n, sizeof(cand), pos_cmp);
        /* segments: [start, end) runs of one type; count the Transition
         * segments after each one from the end */
        int *seg_start = malloc(sizeof(int) * (n + 1));
        int n_seg = 0;
        for (int i = 0; i < n; ++i)
            if (i == 0 || cs[i].pool != cs[i - 1].pool)
                seg_start[n_seg++] = i;
        seg_start[n_seg] = n;
        int later_t = 0;
        for (int sg = n_seg - 1; sg >= 0; --sg) {
            int a = seg_start[sg], e = seg_start[sg + 1];
            int is_t = cs[a].pool == 2;
            if (later_t > 0) {
                long keep;
                if (is_t) {
                    keep = t_keep;
                } else {
                    long r = later_t - 1 >= 31 ? 0 : ((long)r0 >> (later_t - 1));
                    keep = r > r_min ? r : r_min;
                }
                if (keep < 0) keep = 0;
                if (keep < e - a) {
                    qsort(cs + a, e - a, sizeof(cand), cand_cmp);
                    for (int i = a + (int)keep; i < e; ++i)
                        c->mask[cs[i].pool][cs[i].id] &= (uint16_t)~(1u << cs[i].slot);
                }
            }
            later_t += is_t;
        }
        free(seg_start);
        free(cs);
        compact_row(c, b);
    }
}

/* Window score in fixed point, 16 fractional bits: floor(score * 2^16) for
 * 0 < score < 2^16, 2^32 - 1 from 2^16 up, 0 for score <= 0 or NaN. */
static uint32_t tam_fix(float score)
{
    if (!(score > 0.0f))
        return 0;
    if (score >= 65536.0f)
        return 0xffffffffu;
    return (uint32_t)(score * 65536.0f);
}

/* floor(sqrt(x)) for x < 2^64, by bisection on the root. */
static uint64_t isqrt_u64(uint64_t x)
{
    uint64_t lo = 0, hi = 1ull << 32;
    while (hi - lo > 1) {
        uint64_t mid = lo + (hi - lo) / 2;
        if (mid * mid <= x)
            lo = mid;
        else
            hi = mid;
    }
    return lo;
}

/*
 * Thought-aware budgets ("Thought-Aware KV Cache Compaction ... (TAM)",
 * section 2: A segmentation, B adaptive budget allocation, C pivotal-token
 * protection), with compaction read as keeping a subset of the cached
 * tokens.
 *
 * Per sequence, the candidates are the valid slots with q_window <= pos <
 * seq_len - recent_window; the others are kept.  score[p] is the attention
 * mass position p received from the selection window (the R most recent
 * queries), taken in fixed point s = tam_fix(score).
 *  C. A candidate is pivotal when s * N > pivot_c * S (in doubles), N the
 *     candidates and S the sum of their s: its mass is above pivot_c times
 *     the mean.  Pivotal candidates are all kept; the budget left,
 *     T = max(0, keep_k - pivotal), goes to the others.
 *  A. In position order the candidates form runs of one thought type; a
 *     run of at least min_seg candidates opens a new segment, a shorter run
 *     merges into the segment before it (the first run always opens one).
 *  B. Segment i has n_i candidates, m_i of them not pivotal, and the sum S_i
 *     of their s.  Its weight is a_i = isqrt(floor(S_i / n_i) * 2^16) * m_i,
 *     i.e. sqrt(w_i) * m_i with w_i its mean window score.  Budgets are
 *     t_i = T a_i / A (A the sum of the weights) except that a segment whose
 *     share reaches m_i is capped at m_i and the rest shared again among the
 *     others, until no share reaches its segment's size.  Integer budgets
 *     come from the running sums C_j of the uncapped weights in position
 *     order: t = floor(T' C_j / A) - floor(T' C_(j-1) / A), T' the budget
 *     left after the capped segments; they add up to T' exactly.  With A = 0
 *     the uncapped segments get nothing.
 * Each segment keeps its pivotal candidates and its t_i others of largest
 * score (ties: lower position); then the table is compacted as in orc_evict.
 */
void orc_evict_tam(orc_cache *c, const float *score, const int32_t *keep_k, float pivot_c, int min_seg,
                   int q_window, int recent_window)
{
    if (min_seg < 1)
        min_seg = 1;
    for (int b = 0; b < c->B; ++b) {
        uint32_t *row = c->table + (long)b * c->max_blocks;
        const float *sc = score + (long)b * c->n_cap;
        int lo = q_window, hi = c->seq_len[b] - recent_window;
        long cap = (long)c->n_blocks[b] * BLK + 1;
        cand *cs = malloc(sizeof(cand) * cap);
        int n = 0;
        for (int e = 0; e < c->n_blocks[b]; ++e) {
            int pool = (int)(row[e] >> 30);
            uint32_t id = row[e] & 0x3fffffffu;
            uint16_t m = c->mask[pool][id];
            for (int s = 0; s < BLK; ++s) {
                if (!((m >> s) & 1))
                    continue;
                int p = c->pos[pool][id * BLK + s];
                if (p < lo || p >= hi)
                    continue;
                cs[n].imp = sc[p];
                cs[n].pos = p;
                cs[n].pool = pool;
                cs[n].id = id;
                cs[n].slot = s;
                ++n;
            }
        }
        qsort(cs, n, sizeof(cand), pos_cmp);

        /* C. pivotal candidates */
        uint64_t s_all = 0;
        for (int i = 0; i < n; ++i)
            s_all += tam_fix(cs[i].imp);
        char *piv = calloc(n + 1, 1);
        long n_piv = 0;
        for (int i = 0; i < n; ++i) {
            piv[i] = (double)tam_fix(cs[i].imp) * (double)n > (double)pivot_c * (double)s_all;
            n_piv += piv[i];
        }
        long T = (long)keep_k[b] - n_piv;
        if (T < 0)
            T = 0;

        /* A. segments: runs, then the short ones merged */
        int *seg_start = malloc(sizeof(int) * (n + 1));
        int n_seg = 0;
        for (int i = 0; i < n;) {
            int j = i + 1;
            while (j < n && cs[j].pool == cs[i].pool)
                ++j;
            if (i == 0 || j - i >= min_seg)
                seg_start[n_seg++] = i;
            i = j;
        }
        seg_start[n_seg] = n;

        /* B. weights, capped shares, cumulative rounding */
        uint64_t *a = malloc(sizeof(uint64_t) * (n_seg + 1));
        long *mm = malloc(sizeof(long) * (n_seg + 1));
        long *t = malloc(sizeof(long) * (n_seg + 1));
        char *capped = calloc(n_seg + 1, 1);
        for (int sg = 0; sg < n_seg; ++sg) {
            uint64_t ssum = 0;
            long nn = seg_start[sg + 1] - seg_start[sg], m = 0;
            for (int i = seg_start[sg]; i < seg_start[sg + 1]; ++i) {
                ssum += tam_fix(cs[i].imp);
                m += !piv[i];
            }
            mm[sg] = m;
            a[sg] = isqrt_u64((ssum / (uint64_t)nn) << 16) * (uint64_t)m;
            capped[sg] = m == 0;
            t[sg] = 0;
        }
        long t_left = T;
        for (;;) {
            t_left = T;
            unsigned __int128 A = 0;
            for (int sg = 0; sg < n_seg; ++sg) {
                if (capped[sg])
                    t_left -= mm[sg];
                else
                    A += a[sg];
            }
            int more = 0;
            if (A > 0) {
                for (int sg = 0; sg < n_seg; ++sg) {
                    if (!capped[sg] && (unsigned __int128)t_left * a[sg] >= (unsigned __int128)mm[sg] * A) {
                        capped[sg] = 1;
                        more = 1;
                    }
                }
            }
            if (!more) {
                unsigned __int128 run = 0, q_prev = 0;
                for (int sg = 0; sg < n_seg; ++sg) {
                    if (capped[sg]) {
                        t[sg] = mm[sg];
                    } else if (A > 0) {
                        run += a[sg];
                        unsigned __int128 q = (unsigned __int128)t_left * run / A;
                        t[sg] = (long)(q - q_prev);
                        q_prev = q;
                    }
                }
                break;
            }
        }

        /* each segment: pivotal kept, t others by score */
        cand *np = malloc(sizeof(cand) * (n + 1));
        for (int sg = 0; sg < n_seg; ++sg) {
            int k = 0;
            for (int i = seg_start[sg]; i < seg_start[sg + 1]; ++i)
                if (!piv[i])
                    np[k++] = cs[i];
            qsort(np, k, sizeof(cand), cand_cmp);
            for (int i = (int)t[sg]; i < k; ++i)
                c->mask[np[i].pool][np[i].id] &= (uint16_t)~(1u << np[i].slot);
        }
        free(np);
        free(capped);
        free(t);
        free(mm);
        free(a);
        free(seg_start);
        free(piv);
        free(cs);
        compact_row(c, b);
    }
}

/* ------------------------------------------------------------------ */
/* Array forms of the scalar routines above, for the test suite         */
/* ------------------------------------------------------------------ */

void orc_half_to_double_array(const uint16_t *h, double *out, long n)
{
    for (long i = 0; i < n; ++i)
        out[i] = orc_half_to_double(h[i]);
}

void orc_float_to_half_array(const float *f, uint16_t *out, long n)
{
    for (long i = 0; i < n; ++i)
        out[i] = orc_float_to_half(f[i]);
}

/* Native formats, array forms (pool 0 E4M3, 1 E2M1, 2 ternary). */
void orc_quantize_groups_native(const uint16_t *x, long n_groups, int pool, uint16_t *scale,
                                uint16_t *zero, uint8_t *codes)
{
    for (long i = 0; i < n_groups; ++i)
        orc_quantize_group_native(x + i * GS, pool, scale + i, zero + i, codes + i * GS);
}

void orc_native_values(int pool, const uint8_t *codes, long n, double *out)
{
    for (long i = 0; i < n; ++i)
        out[i] = orc_native_value(pool, codes[i]);
}

void orc_mini_encode_array(const float *y, long n, int pool, uint8_t *out)
{
    for (long i = 0; i < n; ++i)
        out[i] = (uint8_t)orc_mini_encode(y[i], MINI_E[pool], MINI_M[pool], MINI_BIAS[pool], MINI_MAX[pool]);
}

/* x: fp16 [n_groups][32] -> scale, zero [n_groups], codes [n_groups][32] */
void orc_quantize_groups(const uint16_t *x, long n_groups, int bits, uint16_t *scale,
                         uint16_t *zero, uint8_t *codes)
{
    for (long i = 0; i < n_groups; ++i)
        orc_quantize_group(x + i * GS, bits, scale + i, zero + i, codes + i * GS);
}
