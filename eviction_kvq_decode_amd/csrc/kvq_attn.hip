// kvq_attn.hip -- single-query decode attention over the typed, paged,
// quantised cache, with per-position attention mass and decayed importance.
//
// "Back from the Future", Problem Statement: scaled dot-product attention
// over the cached K/V.  "TAM", sections 1 and 2.B: the attention mass a
// position receives (summed over query heads) is the importance signal;
// accumulated H2O-style with a decay.  "ThinKV", Continuous Thinking: the
// kernel walks a block table whose blocks carry an eviction mask.
//
// attn_split: a persistent grid; each workgroup takes one contiguous range
//   of the flat (sequence, kv-head pack, table entry) list and records where
//   it starts.  Online softmax in base 2; writes one partial (max, sum,
//   unnormalised output) per (sequence, pack) unit its range meets, and every
//   score it computed (needed later for the mass, whose normaliser is only
//   known once all ranges are done).
// attn_finalize: a resident grid over items of 16 table entries of one
//   sequence: merges each head's partials (log-sum-exp), turns the stored
//   scores into mass / importance in a fixed head order (no float atomics),
//   and writes the output rows.
#include <math.h>

#include <algorithm>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

constexpr int E = 256;  // table entries a segment walks at a time (64 per wave)
constexpr int MAX_HQ = 256;
constexpr int MAX_B = 1024;   // the largest batch the library accepts
constexpr float LOG2E = 1.4426950408889634f;

// Table entries of a sequence, as the kernels read them (a count outside
// [0, max_blocks] in a corrupt cache is clamped).
__device__ inline int table_entries(const kvq_cache &c, int b) {
    return min(max(c.n_blocks[b], 0), c.max_blocks);
}

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef unsigned short ushort2v __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

#ifndef KVQ_WAVES
#define KVQ_WAVES 4          // waves per split workgroup
#endif
#ifndef KVQ_MIN_WAVES_PER_SIMD
#define KVQ_MIN_WAVES_PER_SIMD 2
#endif
constexpr int WAVES = KVQ_WAVES;

// kv heads packed into one wave: the 16 MFMA columns hold PACK(G) * G query heads
__host__ __device__ constexpr int PACK(int G) { return 16 / G < 4 ? 16 / G : 4; }
constexpr float P_HEADROOM = 60000.0f;    // P' = p * v_scale * mult must stay below fp16 max

// Codes become exact integer-valued fp16 MFMA operands, each as B + c for a
// power-of-two bias B whose exponent puts the code's bits at the top of the
// mantissa: B = 1024 for 8-bit codes (0x64 high byte, code in the low byte),
// 16 for 4-bit codes (0x4C00 | c << 6) and 4 for 2-bit codes (0x4400 |
// c << 8).  B is then about the size of the codes, so for K the bias can
// stay in the operand and be taken out of the fp32 sums at no cost in
// precision, through the q sums (B * sum q).  Only 8-bit K codes are
// unbiased before the product (one packed fp16 subtract), because the
// scores feed the per-token mass, whose tolerance is tighter than the 8 : 1
// bias-to-code ratio allows.  V codes are centred instead (Code::MID).  (Operands
// with a zero exponent, c * 2^-24 subnormals, would need no bias but lose
// precision in the MFMA products on this hardware.)
template <int BITS>
struct Code {
    static constexpr float BIAS = BITS == 8 ? 1024.0f : BITS == 4 ? 16.0f : 4.0f;
    // V operands are centred: c - MID, MID = 2^(BITS - 1), from B + c by one
    // exact packed subtract of B + MID (both sides and the result are exact
    // fp16).  The rounding of P' then multiplies a code of either sign and
    // half the magnitude, so with few tokens it stays inside the output
    // tolerance (with B + c, or c alone, it multiplies x - min >= 0).
    static constexpr float MID = BITS == 8 ? 128.0f : BITS == 4 ? 8.0f : 2.0f;
    static constexpr uint32_t BIAS2 = BITS == 8 ? 0x64006400u : BITS == 4 ? 0x4C004C00u : 0x44004400u;
    static constexpr uint32_t FIELDS = BITS == 4 ? 0x03C003C0u : 0x03000300u;   // mantissa top field
    static constexpr int TOP = BITS == 4 ? 6 : 8;                              // its lowest bit
};
__device__ inline uint32_t unbias1024(uint32_t x) {
    half2v h = __builtin_bit_cast(half2v, x);
    h = h - (half2v){(_Float16)1024.0f, (_Float16)1024.0f};
    return __builtin_bit_cast(uint32_t, h);
}
// Bytes i and j of w as the fp16 pair (1024 + w.byte[i], 1024 + w.byte[j]).
__device__ inline uint32_t byte_pair(uint32_t w, int i, int j) {
    const uint32_t sel = (uint32_t)(4 + i) | ((uint32_t)(4 + j) << 16);  // selector 0: a 0x64 byte
    return __builtin_amdgcn_perm(w, 0x64646464u, sel);
}
__device__ inline uint32_t shift_signed(uint32_t w, int s) { return s >= 0 ? w << s : w >> -s; }
// The 4- or 2-bit fields at bit offsets sh and sh+16 of w as the fp16 pair
// (B + c0, B + c1): one shift and one v_and_or_b32.  vb holds BIAS2 in a
// vector register the compiler cannot see through (a VOP3 instruction takes
// neither a literal nor two scalar operands here).
template <int BITS>
__device__ inline uint32_t field_pair(uint32_t w, int sh, uint32_t vb) {
    return (shift_signed(w, Code<BITS>::TOP - sh) & Code<BITS>::FIELDS) | vb;
}
template <int BITS>
__device__ inline uint32_t opaque_bias() {
    uint32_t vb = Code<BITS>::BIAS2;
    asm volatile("" : "+v"(vb));
    return vb;
}

// ThinKV's own formats (the native codec) as exact fp16 operands, no bias:
// a code's sign goes to bit 15 and its exponent and mantissa bits to the
// top of fp16's, which reads as value * 2^-8 (E4M3) or value * 2^-14
// (E2M1), a subnormal for the formats' subnormals; one packed multiply by
// the power of two then gives the value itself, a normal fp16 (every E4M3
// and E2M1 value is one), so no operand reaches the MFMA subnormal.
__device__ inline uint32_t scale_pair(uint32_t x, float f) {
    half2v h = __builtin_bit_cast(half2v, x);
    h = h * (half2v){(_Float16)f, (_Float16)f};
    return __builtin_bit_cast(uint32_t, h);
}
// E4M3 codes in bytes i and j of w as an fp16 pair.
__device__ inline uint32_t e4m3_pair(uint32_t w, int i, int j) {
    const uint32_t sel = 0x0Cu | ((uint32_t)(4 + i) << 8) | (0x0Cu << 16) | ((uint32_t)(4 + j) << 24);
    const uint32_t t = __builtin_amdgcn_perm(w, 0u, sel);  // codes in the high bytes
    return scale_pair(((t >> 1) & 0x3F803F80u) | (t & 0x80008000u), 256.0f);
}
// E2M1 codes in the 4-bit fields at bit offsets sh and sh+16 of w as an fp16 pair.
__device__ inline uint32_t e2m1_pair(uint32_t w, int sh) {
    const uint32_t x = (shift_signed(w, 9 - sh) & 0x0E000E00u) | (shift_signed(w, 12 - sh) & 0x80008000u);
    return scale_pair(x, 16384.0f);
}

// QK A operand: the eight codes of group g held by this lane's K slice,
// in channel order e0..e7 (see the K row layout); 8-bit codes exact, 4- and
// 2-bit codes as B + c; native E4M3 / E2M1 codes as their values.
template <int BITS, bool NAT>
__device__ inline half8 k_operand(const uint32_t *kw, int g, uint32_t vb) {
    uint32_t r[4];
    if constexpr (NAT && BITS == 8) {
        r[0] = e4m3_pair(kw[2 * g], 0, 1);
        r[1] = e4m3_pair(kw[2 * g], 2, 3);
        r[2] = e4m3_pair(kw[2 * g + 1], 0, 1);
        r[3] = e4m3_pair(kw[2 * g + 1], 2, 3);
    } else if constexpr (NAT && BITS == 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) r[k] = e2m1_pair(kw[g], 4 * k);
    } else if constexpr (BITS == 8) {
        r[0] = unbias1024(byte_pair(kw[2 * g], 0, 1));
        r[1] = unbias1024(byte_pair(kw[2 * g], 2, 3));
        r[2] = unbias1024(byte_pair(kw[2 * g + 1], 0, 1));
        r[3] = unbias1024(byte_pair(kw[2 * g + 1], 2, 3));
    } else if constexpr (BITS == 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) r[k] = field_pair<4>(kw[g], 4 * k, vb);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) r[k] = field_pair<2>(kw[g >> 1], 2 * (4 * (g & 1) + k), vb);
    }
    return __builtin_bit_cast(half8, r);
}

// (B + c0, B + c1) -> (c0 - MID, c1 - MID), exact
template <int BITS>
__device__ inline uint32_t center_pair(uint32_t x) {
    constexpr _Float16 k = (_Float16)(Code<BITS>::BIAS + Code<BITS>::MID);
    half2v h = __builtin_bit_cast(half2v, x);
    h = h - (half2v){k, k};
    return __builtin_bit_cast(uint32_t, h);
}

// PV B operand: codes of tokens 4r..4r+3 at this lane's channel of tile n,
// as c - MID (native E4M3 / E2M1 codes: their values).
template <int BITS, bool NAT>
__device__ inline half4 v_operand(const uint32_t *vw, int n, uint32_t vb) {
    uint32_t r[2];
    if constexpr (NAT && BITS == 8) {
        r[0] = e4m3_pair(vw[n], 0, 2);
        r[1] = e4m3_pair(vw[n], 1, 3);
    } else if constexpr (NAT && BITS == 4) {
        const int m = n & 1;
        r[0] = e2m1_pair(vw[n >> 1], 8 * m);
        r[1] = e2m1_pair(vw[n >> 1], 8 * m + 4);
    } else if constexpr (BITS == 8) {
        const uint32_t w = vw[n];
        r[0] = __builtin_amdgcn_perm(w, 0x64646464u, 4u | (6u << 16));
        r[1] = __builtin_amdgcn_perm(w, 0x64646464u, 5u | (7u << 16));
    } else if constexpr (BITS == 4) {
        const int m = n & 1;
        r[0] = field_pair<4>(vw[n >> 1], 8 * m, vb);
        r[1] = field_pair<4>(vw[n >> 1], 8 * m + 4, vb);
    } else {
        const int m = n & 3;
        r[0] = field_pair<2>(vw[n >> 2], 4 * m, vb);
        r[1] = field_pair<2>(vw[n >> 2], 4 * m + 2, vb);
    }
    if constexpr (!NAT) {
        r[0] = center_pair<BITS>(r[0]);
        r[1] = center_pair<BITS>(r[1]);
    }
    return __builtin_bit_cast(half4, r);
}

// 2^x by the hardware instruction (results below the normal range flush to
// zero, which no probability here needs)
__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline float lo_h(uint32_t x) { return h2f((uint16_t)(x & 0xffff)); }
__device__ inline float hi_h(uint32_t x) { return h2f((uint16_t)(x >> 16)); }

// Per-wave running state for the G query heads of each kv head in the pack.
// Lane (rho = lane % 16, r = lane / 16) owns head rho and, inside a block,
// tokens 4r..4r+3; the PV accumulators O[n] hold heads 4r..4r+3 at
// channel 16n + lane % 16.
struct WaveState {
    float m;         // running max of head rho (base-2 scaled scores)
    float l;         // this lane's share of the running sum
    float z[NGRP];   // this lane's share of sum p * (v_zero + MID * v_scale) per group
    floatx4 o[8];    // sum P' * (code - MID), P' = p * v_scale * mult: head rho, channels
                     // 16 n + 4 r .. + 3 of tile n
    float mult;      // power-of-two headroom factor applied to P'
    float4 sc;       // the last block's scores in tile layout (slot 4 r + rho % 4,
                     // heads 4 (rho / 4) ..), stored once the next block has landed
};

// The score rows of a block whose entry's tile is `tile` and valid slots m16:
// lane (lo, hi) writes the 16 bytes of slot 4 hi + lo % 4, heads 4 (lo / 4)
// .. + 3.  A block's rows are written at the start of the wave's next block,
// right after its loads have landed, so the write completes under that
// block's work instead of holding up the wait for its loads (the wait counts
// stores too).
__device__ inline void store_scores(float *tile, uint32_t m16, float4 v) {
    const int lane = threadIdx.x & 63, lo = lane & 15, hi = lane >> 4;
    const int slot = 4 * hi + (lo & 3);
    if ((m16 >> slot) & 1u) *reinterpret_cast<float4 *>(tile + slot * 16 + 4 * (lo >> 2)) = v;
}

// ---------------------------------------------------------------------------
// Block staging.  Each wave owns an LDS stage that holds one block-pack: the
// (scale, zero) areas of its kv heads at a * 512, kv head a's K codes
// at kcode0(P) + 2048 a and its V codes at vcode0(P) + 2048 a, whatever the
// bit width (an 8-bit block fills them; 4- and 2-bit blocks use the first
// half or quarter).  The areas of one part sit at the same place for every
// bit width, so the next block's V part can land while this block's K codes
// are read.  Loads go straight from HBM to LDS, 1 KB per instruction (lane
// i's 16 bytes land at base + 16 i), and skip the 16-byte chunks that belong
// only to evicted slots; those bytes keep stale contents.  The (scale, zero)
// areas only ever hold zeros or pairs of valid slots: finite fp16, which a
// cleared slot (p = 0) turns into exact zeros.
constexpr int STAGE_REGION = 4096 + 512;                        // 8-bit region
constexpr int CODE_AREA = 2048;                                 // per part and kv head
__host__ __device__ constexpr int stage_bytes(int P) { return P * STAGE_REGION; }
__host__ __device__ constexpr int kcode0(int P) { return P * 512; }
__host__ __device__ constexpr int vcode0(int P) { return kcode0(P) + P * CODE_AREA; }

typedef __attribute__((address_space(3))) void lds_void;

// lane i: 16 bytes from gptr (its own address) + GOFF to lds_dst + 16 i.
// Written as an instruction the compiler does not track: its waits would
// otherwise drain every store behind these loads before any later LDS read
// (it cannot tell the stage from other LDS data).  The kernel waits for the
// loads itself.  The instruction has no register result; m0 carries the LDS
// base and needs one wait state before the load.  The loads are marked
// non-temporal: the cache is read once, and streaming it through the caches
// at normal priority evicts the score tiles being written (the long-trace
// decode took 232 us with plain loads and 197 us with these, for the same
// HBM byte counts).
template <int GOFF = 0>
__device__ inline void lds_load16(const void *gptr, uint8_t *lds_dst) {
    const uint32_t lds = (uint32_t)(size_t)(lds_void *)lds_dst;
    const uint8_t *g = static_cast<const uint8_t *>(gptr) + GOFF;
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt" : : "v"(g), "s"(lds)
                 : "memory", "m0");
}
// s_waitcnt encodings (gfx9): vmcnt(0), and lgkmcnt(0) alone
__device__ inline void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Issue the loads of one block-pack into `stage`, in two parts: PART_V
// (V codes and both (scale, zero) areas) and PART_K (K codes).  blk = the
// pack's first region (kv head kh0) in HBM; np kv heads are real.
constexpr int PART_V = 1, PART_K = 2;
template <int BITS, int P, int PART>
__device__ inline void issue_block(uint8_t *stage, const uint8_t *blk, int np, uint32_t m16) {
    constexpr uint32_t CB = 512u * BITS, RB = CB + 512u;
    const int lane = threadIdx.x & 63;
    const uint32_t live4 = ((m16 & 0x000fu) ? 1u : 0u) | ((m16 & 0x00f0u) ? 2u : 0u) |
                           ((m16 & 0x0f00u) ? 4u : 0u) | ((m16 & 0xf000u) ? 8u : 0u);
    // addresses: a wave-uniform base plus a 32-bit lane offset; loads that
    // share a lane predicate are issued under one exec mask
    const uint32_t loff = (uint32_t)lane * 16u;
    if constexpr (PART == PART_K) {
        // K rows are swizzled in LDS: a token's 16-byte chunks are stored in
        // an order that depends on the token (chunk j of token t at chunk
        // position j ^ k_swz(t)), so the sixteen token lanes that read the
        // same chunk of their rows meet different banks.  Lane i lands at
        // chunk position i and therefore loads the chunk stored there.
        if constexpr (BITS == 8) {
            // token (1024 j + 16 lane) / 128 = 8 j + lane / 8
            const uint32_t koff = (((uint32_t)lane & ~7u) | (((uint32_t)lane ^ ((uint32_t)lane >> 3)) & 7u)) * 16u;
            if ((m16 >> (lane >> 3)) & 1u) {
#pragma unroll
                for (int a = 0; a < P; ++a)
                    if (a < np) lds_load16<0>(blk + (a * RB + koff), stage + kcode0(P) + a * CODE_AREA);
            }
            if ((m16 >> (8 + (lane >> 3))) & 1u) {
#pragma unroll
                for (int a = 0; a < P; ++a)
                    if (a < np) lds_load16<1024>(blk + (a * RB + koff), stage + kcode0(P) + a * CODE_AREA + 1024);
            }
        } else if constexpr (BITS == 4) {
            const uint32_t koff = (((uint32_t)lane & ~3u) | (((uint32_t)lane ^ ((uint32_t)lane >> 3)) & 3u)) * 16u;
            if ((m16 >> (lane >> 2)) & 1u) {                          // token lane / 4
#pragma unroll
                for (int a = 0; a < P; ++a)
                    if (a < np) lds_load16<0>(blk + (a * RB + koff), stage + kcode0(P) + a * CODE_AREA);
            }
        } else {
            const uint32_t koff = (((uint32_t)lane & ~1u) | (((uint32_t)lane ^ ((uint32_t)lane >> 3)) & 1u)) * 16u;
            if (lane < 32 && ((m16 >> (lane >> 1)) & 1u)) {           // token lane / 2
#pragma unroll
                for (int a = 0; a < P; ++a)
                    if (a < np) lds_load16<0>(blk + (a * RB + koff), stage + kcode0(P) + a * CODE_AREA);
            }
        }
    } else {
        if constexpr (BITS == 8) {
            // two 1 KB halves; a 16-byte chunk holds 4 consecutive tokens
            if ((live4 >> (lane >> 4)) & 1u) {
#pragma unroll
                for (int a = 0; a < P; ++a)
                    if (a < np) {
                        lds_load16<2048>(blk + (a * RB + loff), stage + vcode0(P) + a * CODE_AREA);
                        lds_load16<3072>(blk + (a * RB + loff), stage + vcode0(P) + a * CODE_AREA + 1024);
                    }
            }
        } else if constexpr (BITS == 4) {
            if ((live4 >> (lane >> 4)) & 1u) {
#pragma unroll
                for (int a = 0; a < P; ++a)
                    if (a < np) lds_load16<1024>(blk + (a * RB + loff), stage + vcode0(P) + a * CODE_AREA);
            }
        } else {
            // the V codes follow the 512 K bytes: lanes 32-63 of the region's
            // first 1 KB (group (lane - 32) / 8 of 4 tokens), landing at the
            // start of the V area
            if (lane >= 32 && ((live4 >> ((lane - 32) >> 3)) & 1u)) {
#pragma unroll
                for (int a = 0; a < P; ++a)
                    if (a < np) lds_load16<0>(blk + (a * RB + loff), stage + vcode0(P) + a * CODE_AREA - 512);
            }
        }
        // (scale, zero) areas, two kv heads per instruction: lane i < 32 takes
        // chunk i of head 2 a2, lane i >= 32 chunk i - 32 of head 2 a2 + 1;
        // chunk c < 16 holds token c's K pairs, c >= 16 token c - 16's V pairs
        if ((m16 >> (lane & 15)) & 1u) {
            const uint32_t soff = (uint32_t)(lane >> 5) * RB + CB + ((uint32_t)lane & 31u) * 16u;
#pragma unroll
            for (int a2 = 0; a2 < (P + 1) / 2; ++a2)
                if (2 * a2 + (lane >> 5) < np) lds_load16(blk + (2u * a2 * RB + soff), stage + a2 * 1024);
        }
    }
}

// 4x4 transpose across the four lanes of a group (lane bits 0-1 = i):
// lane i's element k becomes lane k's element i.  Two exchange stages, over
// lane bit 0 / element bit 0, then lane bit 1 / element bit 1 (DPP quad
// permutations: swap neighbours, swap pairs).
template <int CTRL>
__device__ inline float quad_perm(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
__device__ inline float4 quad_transpose(float4 r, int lane) {
    const bool b0 = lane & 1, b1 = (lane >> 1) & 1;
    // lane bit 0: even lanes send elements 1, 3 and receive the odd lane's 0, 2
    const float y0 = quad_perm<0xB1>(b0 ? r.x : r.y), y1 = quad_perm<0xB1>(b0 ? r.z : r.w);
    r = b0 ? make_float4(y0, r.y, y1, r.w) : make_float4(r.x, y0, r.z, y1);
    // lane bit 1: lanes 0, 1 send elements 2, 3 and receive lanes 2, 3's 0, 1
    const float z0 = quad_perm<0x4E>(b1 ? r.x : r.z), z1 = quad_perm<0x4E>(b1 ? r.y : r.w);
    return b1 ? make_float4(z0, z1, r.z, r.w) : make_float4(r.x, r.y, z0, z1);
}

// The next block-pack's loads, issued by attend_block in two parts: the V
// part once the current block's V codes, pairs and positions are in
// registers, the K part once its QK^T products have read the K codes.
struct NoNext {
    __device__ void operator()(int) const {}
};

// NAT: the block holds native E4M3 / E2M1 codes (symmetric, zero 0).
template <int G, int BITS, bool NAT, class Next>
__device__ inline void attend_block(const uint8_t *stage, int np, uint32_t m16, const uint4 *const *qa,
                                    const float *qsum, float scale2, WaveState &st,
                                    const Next &next) {
    constexpr int P = PACK(G);
    const int lane = threadIdx.x & 63, lo = lane & 15, hi = lane >> 4;
    const int a_rho = min(lo / G, np - 1);
    const bool row_ok = lo < np * G;
    const uint32_t vb = opaque_bias<BITS>();

    // -- the block-pack from the stage: K slice of token lo (channel slice
    //    hi), V slice of this lane, and the (scale, zero) pairs of tokens
    //    4hi..4hi+3 of this lane's kv head; a partial pack re-reads its last
    //    kv head, whose products meet zero q / P' operands
    constexpr int KW = BITS, VW = BITS;
    uint32_t vw[P][VW];
#pragma unroll
    for (int a = 0; a < P; ++a) {
        const uint8_t *lr = stage + vcode0(P) + (uint32_t)min(a, np - 1) * CODE_AREA;
        if constexpr (BITS == 8) {
            const uint4 v0 = *reinterpret_cast<const uint4 *>(lr + lane * 16);
            const uint4 v1 = *reinterpret_cast<const uint4 *>(lr + 1024 + lane * 16);
            vw[a][0] = v0.x; vw[a][1] = v0.y; vw[a][2] = v0.z; vw[a][3] = v0.w;
            vw[a][4] = v1.x; vw[a][5] = v1.y; vw[a][6] = v1.z; vw[a][7] = v1.w;
        } else if constexpr (BITS == 4) {
            const uint4 v0 = *reinterpret_cast<const uint4 *>(lr + lane * 16);
            vw[a][0] = v0.x; vw[a][1] = v0.y; vw[a][2] = v0.z; vw[a][3] = v0.w;
        } else {
            const uint2 v0 = *reinterpret_cast<const uint2 *>(lr + lane * 8);
            vw[a][0] = v0.x; vw[a][1] = v0.y;
        }
    }
    uint32_t ksz[16], vsz[16];
    {
        const uint8_t *own = stage + a_rho * 512 + 64 * hi;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 kq = reinterpret_cast<const uint4 *>(own)[i];
            const uint4 vq = reinterpret_cast<const uint4 *>(own + 256)[i];
            ksz[4 * i + 0] = kq.x; ksz[4 * i + 1] = kq.y; ksz[4 * i + 2] = kq.z; ksz[4 * i + 3] = kq.w;
            vsz[4 * i + 0] = vq.x; vsz[4 * i + 1] = vq.y; vsz[4 * i + 2] = vq.z; vsz[4 * i + 3] = vq.w;
        }
    }
    // -- those reads have landed: the next block-pack's V part may overwrite
    //    them while this one's K codes and positions are still read
    wait_lgkm0();
    next(PART_V);

    // -- QK^T per group: rows = tokens, columns = the pack's 16 query heads;
    //    a kv head's codes meet only its own heads (block-diagonal q: a
    //    column outside kv head a reads a zero operand).  Each kv head's K
    //    slice (token lo, channel slice hi) is read just before its MFMAs.
    floatx4 acc[NGRP];
#pragma unroll
    for (int g = 0; g < NGRP; ++g) acc[g] = (floatx4){0.f, 0.f, 0.f, 0.f};
    // this lane's K slice in the swizzled rows: chunk j of token lo sits at
    // chunk position j ^ k_swz(lo) of its row
    uint32_t koff;
    if constexpr (BITS == 8)
        koff = (uint32_t)lo * 128u + (((2u * hi) ^ ((uint32_t)lo & 7u)) << 4);
    else if constexpr (BITS == 4)
        koff = (uint32_t)lo * 64u + (((uint32_t)hi ^ (((uint32_t)lo >> 1) & 3u)) << 4);
    else
        koff = (uint32_t)lo * 32u + ((((uint32_t)hi >> 1) ^ (((uint32_t)lo >> 2) & 1u)) << 4) + (((uint32_t)hi & 1u) << 3);
#pragma unroll
    for (int a = 0; a < P; ++a) {
        const uint8_t *lr = stage + kcode0(P) + (uint32_t)min(a, np - 1) * CODE_AREA;
        uint32_t kw[KW];
        if constexpr (BITS == 8) {
            // the lane's two chunks differ only in the lowest position bit
            const uint4 k0 = *reinterpret_cast<const uint4 *>(lr + koff);
            const uint4 k1 = *reinterpret_cast<const uint4 *>(lr + (koff ^ 16u));
            kw[0] = k0.x; kw[1] = k0.y; kw[2] = k0.z; kw[3] = k0.w;
            kw[4] = k1.x; kw[5] = k1.y; kw[6] = k1.z; kw[7] = k1.w;
        } else if constexpr (BITS == 4) {
            const uint4 k0 = *reinterpret_cast<const uint4 *>(lr + koff);
            kw[0] = k0.x; kw[1] = k0.y; kw[2] = k0.z; kw[3] = k0.w;
        } else {
            const uint2 k0 = *reinterpret_cast<const uint2 *>(lr + koff);
            kw[0] = k0.x; kw[1] = k0.y;
        }
#pragma unroll
        for (int g = 0; g < NGRP; ++g) {
            const half8 qb = __builtin_bit_cast(half8, qa[a][65 * g]);
            acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand<BITS, NAT>(kw, g, vb), qb, acc[g], 0, 0, 0);
        }
    }
    // -- the K reads have landed: the next block-pack's K part, while the
    //    last products, the scores and their tile store proceed.  No stage
    //    read follows in this block; the next block waits for all of its
    //    wave's memory operations.
    wait_lgkm0();
    next(PART_K);

    // -- scores of tokens 4hi..4hi+3 for head lo: fold the group scales and
    //    zeros, base-2 scale, mask cleared slots (a cleared slot's stage
    //    bytes are stale: its score is replaced, never used)
    float s[4];
    bool tv[4];
    {
        // group by group, so each group's scale and zero terms (which largely
        // cancel) meet before the next group is added; the four tokens'
        // chains are independent and interleave
        // (4- and 2-bit products carry the code bias: B * sum q comes off;
        // native codes carry no bias and their zero is 0)
        constexpr float KB = BITS == 8 || NAT ? 0.f : Code<BITS>::BIAS;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < NGRP; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t sz = ksz[4 * i + g];
                if constexpr (NAT) {
                    v[i] = fmaf(lo_h(sz), acc[g][i], v[i]);
                } else {
                    // acc - B * sum q in one rounding (B * sum q is exact)
                    v[i] = fmaf(lo_h(sz), BITS == 8 ? acc[g][i] : fmaf(-KB, qsum[g], acc[g][i]), v[i]);
                    v[i] = fmaf(hi_h(sz), qsum[g], v[i]);
                }
            }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            tv[i] = (m16 >> (4 * hi + i)) & 1u;
            s[i] = row_ok && tv[i] ? v[i] * scale2 : -INFINITY;
        }
    }
    // -- the block's scores: the entry's 1 KB tile is [slot][head] (rows of
    //    cleared slots not written; heads past the pack unspecified).  Lane
    //    (head lo = 4a + i, hi) holds head lo's slots 4hi..4hi+3; a 4x4
    //    transpose inside each group of four lanes gives it slot 4hi + i's
    //    heads 4a..4a+3, kept for one 16-byte write (store_scores), so the
    //    wave writes the tile's valid rows at once (the mass pass reads only
    //    those).
    st.sc = quad_transpose(make_float4(s[0], s[1], s[2], s[3]), lo);

    // -- online softmax.  The PV accumulators hold this lane's own head (lo),
    //    so a rescale is a multiply by the lane's own factor; it is done on
    //    every block (a branch around it makes the compiler copy the
    //    accumulators at the join).
    float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    bm = fmaxf(bm, __shfl_xor(bm, 16));
    bm = fmaxf(bm, __shfl_xor(bm, 32));
    const float mn = fmaxf(st.m, bm);
    const float am = mn == st.m ? 1.f : (st.m == -INFINITY ? 0.f : exp2_fast(st.m - mn));
    st.m = mn;
    float p[4];
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p[i] = s[i] == -INFINITY ? 0.f : exp2_fast(s[i] - mn);
        psum += p[i];
    }
    st.l = fmaf(st.l, am, psum);
#pragma unroll
    for (int g = 0; g < NGRP; ++g) st.z[g] *= am;
    float ao = am;   // the accumulators' factor: am, and the headroom change

    // -- headroom: P' = p * v_scale * mult must stay inside fp16, and p <= 1,
    //    so the largest v_scale in the stage bounds it.  Scales are
    //    non-negative fp16, whose bit patterns order like their values: a
    //    packed unsigned max over the (scale, zero) words finds it in the low
    //    halves.  (Stale pairs of cleared tokens only make the bound safer.)
    {
        ushort2v vm = __builtin_bit_cast(ushort2v, vsz[0]);
#pragma unroll
        for (int j = 1; j < 16; ++j) vm = __builtin_elementwise_max(vm, __builtin_bit_cast(ushort2v, vsz[j]));
        float vmax = h2f(vm[0]);
        if (__ballot(vmax * st.mult > P_HEADROOM)) {
            for (int off = 1; off < 64; off <<= 1) vmax = fmaxf(vmax, __shfl_xor(vmax, off));
            float nm = st.mult;
            while (vmax * nm > P_HEADROOM) nm *= 0.5f;
            ao *= nm / st.mult;
            st.mult = nm;
        }
    }
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) st.o[n][i] *= ao;
    // -- P' per group in the PV A-operand layout (lane = head, 4 tokens), one
    //    rounding to fp16.  A cleared token has p = 0 and finite stale pairs,
    //    so it contributes exact zeros.
    float pm[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pm[i] = p[i] * st.mult;
    half4 pop[NGRP];
#pragma unroll
    for (int g = 0; g < NGRP; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) pop[g][i] = (_Float16)(pm[i] * lo_h(vsz[4 * i + g]));
    // zero-point term sum p * (v_zero + MID * v_scale): the centred
    // operands' offset joins the zero point (native codes: neither)
    if constexpr (!NAT) {
#pragma unroll
        for (int g = 0; g < NGRP; ++g) {
            float zg = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                zg = fmaf(p[i], fmaf(Code<BITS>::MID, lo_h(vsz[4 * i + g]), hi_h(vsz[4 * i + g])), zg);
            st.z[g] += zg;
        }
    }

    // -- PV: block-diagonal over the pack's kv heads
#pragma unroll
    for (int a = 0; a < P; ++a) {
        const bool mine = a_rho == a && row_ok;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const half4 pa = mine ? pop[n >> 1] : (half4){};
            st.o[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(v_operand<BITS, NAT>(vw[a], n, vb), pa, st.o[n], 0, 0, 0);
        }
    }

}

// Workgroup LDS of the split kernel.  A wave's merged output rows reuse its
// stage's code area once every wave has left its loop; the prologue's
// prefix sums share the stage area too.
template <int P>
struct SplitLds {
    uint32_t ent[E];         // non-empty table entries of the chunk, in order
    int eix[E];              // their table indices
    uint16_t msk[E];         // their masks
    int wcnt[WAVES];         // non-empty entries each wave found
    uint4 qb[NGRP][65];      // [g][lane]: q of column head lane % 16, channel
                             // slice lane / 16 of group g; [g][64] is zero
    // wave merge: row maxima and scaled row sums per wave
    float mm[WAVES][16], lw[WAVES][16];
    // merged rows: padded by 4 floats where the stage has room, so the 16
    // head rows written at once meet different banks
    static constexpr int MRS = P >= 3 ? HD + 4 : HD;
    // the stages; a wave's merged output rows go to its own stage's code
    // area (whose stale bytes are harmless), or after the stages when a
    // one-kv-head stage is too small for 16 rows
    union alignas(16) {
        uint8_t stage[WAVES * stage_bytes(P) + (P == 1 ? WAVES * 16 * HD * 4 : 0)];
        int scan[WAVES * 64 + 1025];
    } u;
    __device__ float *merge_rows(int w) {
        return reinterpret_cast<float *>(u.stage + (P == 1 ? WAVES * stage_bytes(P) + w * 16 * HD * 4
                                                           : w * stage_bytes(P) + kcode0(P)));
    }
};

// One segment: table entries [e_begin, e_end) of sequence b for kv-head pack
// `pack`, taken E entries at a time; writes its partial (max, sum, output)
// for the pack's heads to segment slot `seg`.
template <int G, bool NATIVE>
__device__ inline void split_segment(const kvq_cache &c, const uint16_t *q, float *mass, const DecodeWs &ws,
                                     float scale2, int b, int nb, int pack, int e_begin, int e_end, int seg,
                                     SplitLds<PACK(G)> &sh) {
    constexpr int P = PACK(G);
    const int n_packs = (c.Hkv + P - 1) / P;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lo = lane & 15, hi = lane >> 4;
    const int kh0 = pack * P, np = min(P, c.Hkv - kh0);
    const bool row_ok = lo < np * G;

    // -- the first chunk's table entries are loaded with q, and their masks
    //    once the entries are in, so that the walk below does not start a
    //    chain of its own after q
    const int k0 = 64 * wave + lane;
    const bool in0 = k0 < min(E, e_end - e_begin);
    uint32_t ent0 = 0, m0 = 0;
    if (in0) ent0 = c.table[(size_t)b * c.max_blocks + e_begin + k0];
    // -- q of the pack's heads into LDS (zero past the pack), and the
    //    per-group q sums of head lo in registers
    float qsum[NGRP];
    {
        const int h = kh0 * G + lo;
        uint4 qraw[NGRP];
#pragma unroll
        for (int g = 0; g < NGRP; ++g) {
            qraw[g] = make_uint4(0, 0, 0, 0);
            if (row_ok) qraw[g] = *reinterpret_cast<const uint4 *>(q + ((size_t)b * c.Hq + h) * HD + 32 * g + 8 * hi);
        }
        if (in0) m0 = pool_sel(c.mask, ent0 >> 30)[ent0 & 0x3fffffffu];
#pragma unroll
        for (int g = 0; g < NGRP; ++g) {
            const uint4 raw = qraw[g];
            if (wave == 0) {
                sh.qb[g][lane] = raw;
                if (lane == 0) sh.qb[g][64] = make_uint4(0, 0, 0, 0);
            }
            const half8 qv = __builtin_bit_cast(half8, raw);
            float sum = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) sum += (float)qv[i];
            sum += __shfl_xor(sum, 16);
            sum += __shfl_xor(sum, 32);
            qsum[g] = sum;
        }
    }
    // B operand rows: column lo reads its q for its own kv head, zeros else
    const uint4 *qa[P];
#pragma unroll
    for (int a = 0; a < P; ++a) qa[a] = row_ok && lo / G == a ? &sh.qb[0][lane] : &sh.qb[0][64];
    __syncthreads();

    WaveState st;
    st.m = -INFINITY;
    st.l = 0.f;
    st.mult = 4096.f;
#pragma unroll
    for (int g = 0; g < NGRP; ++g) st.z[g] = 0.f;
#pragma unroll
    for (int n = 0; n < 8; ++n) st.o[n] = (floatx4){0.f, 0.f, 0.f, 0.f};

    const int wv = __builtin_amdgcn_readfirstlane(wave);
    uint8_t *stg = sh.u.stage + wv * stage_bytes(P);
    float *const score_u = ws.score + ((size_t)b * n_packs + pack) * c.max_blocks * 256;
    for (int base = e_begin; base < e_end; base += E) {
        // -- the chunk's non-empty table entries, compacted in table order:
        //    wave w walks entries [64 w, 64 w + 64) of the chunk and places its
        //    non-empty ones after those of the waves before it
        {
            const int cnt = min(E, e_end - base);
            const int k = 64 * wave + lane;
            uint32_t ent = ent0, m = m0;
            if (base != e_begin) {
                ent = 0, m = 0;
                if (k < cnt) {
                    ent = c.table[(size_t)b * c.max_blocks + base + k];
                    m = pool_sel(c.mask, ent >> 30)[ent & 0x3fffffffu];
                }
            }
            const uint64_t bal = __ballot(m != 0);
            if (lane == 0) sh.wcnt[wave] = __popcll(bal);
            __syncthreads();
            int at = __popcll(bal & ((1ull << lane) - 1));
            for (int w = 0; w < wave; ++w) at += sh.wcnt[w];
            if (m != 0) {
                sh.ent[at] = ent;
                sh.msk[at] = (uint16_t)m;
                sh.eix[at] = base + k;
            }
        }
        int n_ent = 0;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) n_ent += sh.wcnt[w];
        n_ent = __builtin_amdgcn_readfirstlane(n_ent);
        __syncthreads();

        auto issue = [&](int k, int part) {
            // block metadata is wave-uniform: keep it in scalar registers
            const uint32_t ent = __builtin_amdgcn_readfirstlane(sh.ent[k]);
            const uint32_t msk = __builtin_amdgcn_readfirstlane(sh.msk[k]);
            const int pool = (int)(ent >> 30);
            const uint32_t id = ent & 0x3fffffffu;
            const uint8_t *blk0 = c.kv[0] + ((size_t)id * c.Hkv + kh0) * (512u * 8 + 512u);
            const uint8_t *blk1 = c.kv[1] + ((size_t)id * c.Hkv + kh0) * (512u * 4 + 512u);
            const uint8_t *blk2 = c.kv[2] + ((size_t)id * c.Hkv + kh0) * (512u * 2 + 512u);
            if (part == PART_V) {
                if (pool == 0) issue_block<8, P, PART_V>(stg, blk0, np, msk);
                else if (pool == 1) issue_block<4, P, PART_V>(stg, blk1, np, msk);
                else issue_block<2, P, PART_V>(stg, blk2, np, msk);
            } else {
                if (pool == 0) issue_block<8, P, PART_K>(stg, blk0, np, msk);
                else if (pool == 1) issue_block<4, P, PART_K>(stg, blk1, np, msk);
                else issue_block<2, P, PART_K>(stg, blk2, np, msk);
            }
        };
        if (wv < n_ent) {
            issue(wv, PART_V);
            issue(wv, PART_K);
        }
        float *pend = nullptr;   // tile of the scores held in st.sc (wave-uniform)
        uint32_t pend_m = 0;
        for (int k = wv; k < n_ent; k += WAVES) {
            // entry k is in the stage once its wave's memory operations are done
            // (the last ones issued are its K part)
            wait_vm0();
            if (pend) store_scores(pend, pend_m, st.sc);
            const uint32_t ent = __builtin_amdgcn_readfirstlane(sh.ent[k]);
            const uint32_t msk = __builtin_amdgcn_readfirstlane(sh.msk[k]);
            const int e = __builtin_amdgcn_readfirstlane(sh.eix[k]);
            const int pool = (int)(ent >> 30);
            const int kn = k + WAVES;
            auto next = [&](int part) {
                if (kn < n_ent) issue(kn, part);
            };
            if (pool == 0)
                attend_block<G, 8, NATIVE>(stg, np, msk, qa, qsum, scale2, st, next);
            else if (pool == 1)
                attend_block<G, 4, NATIVE>(stg, np, msk, qa, qsum, scale2, st, next);
            else
                attend_block<G, 2, false>(stg, np, msk, qa, qsum, scale2, st, next);
            pend = score_u + (size_t)e * 256;
            pend_m = msk;
        }
        if (pend) store_scores(pend, pend_m, st.sc);
        // every wave is done with the chunk's entries before the next chunk's
        // walk overwrites them
        __syncthreads();
    }

    // -- merge the waves of this workgroup and write the segment's partial.
    //    Each wave publishes its row maxima, then writes its output rows
    //    already rescaled to the workgroup maximum (zero-point term included)
    //    into its own stage; the rows are then summed over the waves in a
    //    fixed order.
    float lsum = st.l;
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);
    float zs[NGRP];
#pragma unroll
    for (int g = 0; g < NGRP; ++g) {
        zs[g] = st.z[g];
        zs[g] += __shfl_xor(zs[g], 16);
        zs[g] += __shfl_xor(zs[g], 32);
    }
    if (hi == 0) sh.mm[wave][lo] = st.m;
    __syncthreads();   // maxima of every wave
    {
        // this lane's output row is head lo, channels 16 n + 4 hi .. + 3
        const float inv_mult = 1.0f / st.mult;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) M = fmaxf(M, sh.mm[w][lo]);
        const float f = st.m == -INFINITY ? 0.f : exp2_fast(st.m - M);
        if (hi == 0) sh.lw[wave][lo] = f * lsum;
        float *rows_out = sh.merge_rows(wave) + lo * SplitLds<P>::MRS + 4 * hi;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const float zg = zs[n >> 1];
            *reinterpret_cast<float4 *>(rows_out + 16 * n) =
                make_float4(f * fmaf(st.o[n][0], inv_mult, zg), f * fmaf(st.o[n][1], inv_mult, zg),
                            f * fmaf(st.o[n][2], inv_mult, zg), f * fmaf(st.o[n][3], inv_mult, zg));
        }
    }
    __syncthreads();

    const int rows = np * G;
    for (int idx = tid; idx < rows * HD; idx += WAVES * 64) {
        const int rr = idx / HD, d = idx % HD;
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) o += sh.merge_rows(w)[rr * SplitLds<P>::MRS + d];
        ws.o[((size_t)seg * 16 + rr) * HD + d] = o;
        if (d == 0) {
            float M = -INFINITY, L = 0.f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) M = fmaxf(M, sh.mm[w][rr]);
#pragma unroll
            for (int w = 0; w < WAVES; ++w) L += sh.lw[w][rr];
            ws.ml[((size_t)seg * 16 + rr) * 2 + 0] = M;
            ws.ml[((size_t)seg * 16 + rr) * 2 + 1] = L;
        }
    }
    // -- pack 0's segments partition the sequence's table, so their shares of
    //    the positions below seq_len partition those: each starts its share
    //    at mass 0 (the finalize then writes the valid positions)
    if (pack == 0) {
        const int len = min(c.seq_len[b], c.n_cap);
        const int p0 = (int)((long)len * e_begin / nb), p1 = (int)((long)len * e_end / nb);
        for (int p = p0 + tid; p < p1; p += WAVES * 64) mass[(size_t)b * c.n_cap + p] = 0.f;
    }
    // the merge rows live in the stages: every wave has read them before the
    // next segment's loads land there
    __syncthreads();
}

// Split of the flat entry list over the grid.  With two workgroups per
// compute unit, workgroup j and j + n_first (n_first = the compute units)
// share one, and the first-dispatched one issues ahead of the other: on the
// long evicted trace it finished its equal share about 14% sooner, and the
// unit then ran the later one alone.  So the first n_first workgroups take
// (64 + SPLIT_SKEW) / 64 of the mean share and the rest (64 - SPLIT_SKEW) / 64
// (n_first = NW: equal shares).  Any split that keeps the ranges in
// workgroup order is correct: the finalize reads the starts the split kernel
// records.
constexpr long SPLIT_SKEW = 6;
// A range that crosses into another (sequence, pack) unit starts a second
// segment: its table walk, q and first blocks form a new chain of loads,
// which cost a workgroup about as much as SPLIT_GAP table entries (10.6 us
// on the long evicted trace, where a workgroup streams about one entry per
// us).  The list is therefore split in cost space, where each unit is
// followed by a gap of SPLIT_GAP: a range that takes in a unit boundary
// takes that many fewer entries.
constexpr long SPLIT_GAP = 10;
// A short list is split over fewer workgroups, each taking at least
// SPLIT_MIN units of cost space; the rest get empty ranges.  Every range adds
// a partial that the finalize merges per head, in rounds of dependent loads:
// a 64-entry list over 512 ranges of one entry or none cost the finalize
// about 14 such rounds per output row.  And below SPLIT_SHARED units per
// workgroup of the full grid, a second workgroup on a compute unit gains
// less than its partials cost: the list goes to the first-dispatched
// workgroups only, one per unit (a 32768-position sequence 48.6 -> 38.3 us;
// 16 to 32 units per workgroup lost 3-4 us when capped).
constexpr int SPLIT_MIN = 4;
constexpr int SPLIT_SHARED = 16;
__device__ inline int split_start(long N, int NW, int n_first, int j) {
    if (n_first >= NW) return (int)(N * j / NW);
    const long A = 64 + SPLIT_SKEW, Bw = 64 - SPLIT_SKEW;
    const long tot = n_first * A + (long)(NW - n_first) * Bw;
    const long u = j <= n_first ? (long)j * A : n_first * A + (long)(j - n_first) * Bw;
    return (int)(N * u / tot);
}

// The work is the flat list of (sequence b, kv-head pack p, table entry e),
// in that order: sequence b's entries for pack p sit at
// pre(b) + p nb(b) + e, where nb(b) is its table length and pre(b) =
// n_packs * (table entries of the sequences before it).  Workgroup j of the
// NW in the grid (what fits on the GPU at once) takes the contiguous range
// [split_start(j), split_start(j + 1)) of the N entries (over the first
// NWe <= NW workgroups, see SPLIT_MIN and SPLIT_SHARED; the others take
// empty ranges at the end), with no scheduling traffic, and records its
// start for the finalize.  Where its range crosses a (sequence, pack)
// boundary it writes one partial per side; the partial
// of workgroup j for unit u = b n_packs + p sits in slot j + u (unique,
// since both j and u grow along the list).
// NATIVE: the cache holds the native codec (Reasoning and Execution blocks
// in E4M3 / E2M1; Transition blocks are integer-coded in both codecs).
template <int G, bool NATIVE>
__global__ __launch_bounds__(WAVES * 64, KVQ_MIN_WAVES_PER_SIMD) void attn_split(kvq_cache c, const uint16_t *q,
                                                                                 float *mass, DecodeWs ws, float scale2,
                                                                                 int n_first) {
    constexpr int P = PACK(G);
    const int n_packs = (c.Hkv + P - 1) / P;
    const int tid = threadIdx.x;
    constexpr int NT = WAVES * 64;
    __shared__ SplitLds<P> lds;
    __shared__ int s_carry, s_loc[6];

    // -- pre(b) for every sequence (a scan over table lengths in the stage
    //    area), the total N, and where this workgroup's range starts
    int *s_scan = lds.u.scan, *s_pre = lds.u.scan + NT;
    if (tid == 0) s_carry = 0;
    __syncthreads();
    for (int b0 = 0; b0 < c.B; b0 += NT) {
        // inclusive scan of the counts: inside each wave by shuffles, then
        // the wave totals in LDS
        const int bb = b0 + tid, lane = tid & 63, wave = tid >> 6;
        const int cnt = bb < c.B ? table_entries(c, bb) * n_packs : 0;
        int incl = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(incl, d);
            if (lane >= d) incl += y;
        }
        if (lane == 63) s_scan[wave] = incl;
        __syncthreads();
        int before = s_carry;
        for (int w = 0; w < wave; ++w) before += s_scan[w];
        if (bb < c.B) s_pre[bb] = before + incl - cnt;
        __syncthreads();
        if (tid == NT - 1) s_carry = before + incl;
        __syncthreads();
    }
    const long N = s_carry;
    const int NW = gridDim.x, j = blockIdx.x;
    if (j == 0) {
        // for the finalize: where each sequence's entries start, and N
        for (int bb = tid; bb < c.B; bb += NT) ws.pre[bb] = s_pre[bb];
        if (tid == 0) ws.pre[c.B] = (int)N;
    }
    // -- this workgroup's range, found by two waves (wave w for its end w):
    //    the entry at cost position cpos, where unit (b, p) takes
    //    [cpre(b) + p (nb + gap), + nb) of cost space, cpre(b) = pre(b) +
    //    b n_packs gap, and a position in a gap maps to the next unit's first
    //    entry.  Both prefixes never decrease, so "the last b with prefix <=
    //    x" is the count of such b less one: a ballot per 64 sequences.
    //    Wave 0 also finds the sequence holding the range's first entry and
    //    the table lengths of it and the next (the stage area that holds the
    //    prefix is cleared below).
    if (tid < 128) {
        const int wv = tid >> 6, lane = tid & 63;
        const int NC = (int)N + c.B * n_packs * (int)SPLIT_GAP;
        int NWe = min(NW, max(1, (NC + SPLIT_MIN - 1) / SPLIT_MIN));
        if (NC < SPLIT_SHARED * NW) NWe = min(NWe, n_first);
        const int cpos = j + wv >= NWe ? NC : split_start(NC, NWe, min(n_first, NWe), j + wv);
        int cnt = 0;
        for (int b0 = 0; b0 < c.B; b0 += 64) {
            const int bb = b0 + lane;
            cnt += __popcll(__ballot(bb < c.B && s_pre[bb] + bb * n_packs * (int)SPLIT_GAP <= cpos));
        }
        const int sb = max(cnt - 1, 0);
        const int next = sb + 1 < c.B ? s_pre[sb + 1] : (int)N;
        const int nbb = (next - s_pre[sb]) / n_packs;
        const int off = cpos - (s_pre[sb] + sb * n_packs * (int)SPLIT_GAP);
        const int pp = off / (nbb + (int)SPLIT_GAP), o = off % (nbb + (int)SPLIT_GAP);
        const int f = min(s_pre[sb] + pp * nbb + min(o, nbb), (int)N);
        if (wv == 0) {
            // the sequence holding entry f: the last b with pre(b) <= f
            int cnt2 = 0;
            for (int b0 = 0; b0 < c.B; b0 += 64) {
                const int bb = b0 + lane;
                cnt2 += __popcll(__ballot(bb < c.B && s_pre[bb] <= f));
            }
            const int lb = max(cnt2 - 1, 0);
            if (lane == 0) {
                ws.rstart[j] = f;
                s_loc[0] = lb;
                s_loc[1] = f - s_pre[lb];
                s_loc[2] = f;
                const int n1 = lb + 1 < c.B ? s_pre[lb + 1] : (int)N;
                const int n2 = lb + 2 < c.B ? s_pre[lb + 2] : (int)N;
                s_loc[4] = (n1 - s_pre[lb]) / n_packs;
                s_loc[5] = lb + 1 < c.B ? (n2 - n1) / n_packs : 0;
            }
        } else if (lane == 0) {
            s_loc[3] = f;
            if (j == NW - 1) ws.rstart[NW] = f;
        }
    }
    __syncthreads();
    int b = __builtin_amdgcn_readfirstlane(s_loc[0]), r = __builtin_amdgcn_readfirstlane(s_loc[1]);
    const int f0 = __builtin_amdgcn_readfirstlane(s_loc[2]), f1 = __builtin_amdgcn_readfirstlane(s_loc[3]);
    const int b_first = b, nb_first = __builtin_amdgcn_readfirstlane(s_loc[4]),
              nb_second = __builtin_amdgcn_readfirstlane(s_loc[5]);
    __syncthreads();   // s_loc read before the stage area is cleared

    // -- stage bytes start finite: zero the shared area once (the scan used it;
    //    later only loaded pairs and merged rows in the code areas land there)
    for (int i = tid; i < (int)(sizeof(lds.u) / 16); i += NT)
        reinterpret_cast<uint4 *>(&lds.u)[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();


    // -- the range's segments
    for (int f = f0; f < f1 && b < c.B;) {
        // table lengths of the first two sequences come from the prefix
        const int nb = b == b_first ? nb_first : b == b_first + 1 ? nb_second : table_entries(c, b);
        if (nb == 0) {   // an empty sequence holds no entries of the list
            ++b;
            continue;
        }
        const int pack = r / nb, e = r % nb;
        const int cnt = min(nb - e, f1 - f);
        split_segment<G, NATIVE>(c, q, mass, ws, scale2, b, nb, pack, e, e + cnt, j + b * n_packs + pack, lds);
        f += cnt;
        r += cnt;
        if (r == nb * n_packs) {
            r = 0;
            ++b;
        }
    }
}

// The split workgroup whose range holds entry f of its list: the last j
// with rs[j] <= f, from the recorded starts rs[0..NW] (a workgroup with an
// empty range is never the answer).
__device__ inline int range_owner(const int *rs, int NW, int f) {
    int lo = 0, hi = NW - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (rs[mid] <= f) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Finalize: a grid of W workgroups that all fit on the device at once.
//  - Items: runs of FC consecutive table entries of one sequence, sequence
//    by sequence (ceil(nb / FC) each), taken in turn: item j, j + W, ...
//  - Per item, each wave loads the table entries, masks and positions of its
//    FB entries first; then, while they are in flight, the workgroup merges
//    (into the statistics buffer of the item's parity), per head of the sequence,
//    the partials of the head's unit (the split ranges that met the unit, in
//    order) into M_h, 1 / L_h; then lanes 4t .. 4t + 3 load slot t's row of
//    every pack's tile (16 B each, four heads), sum exp2(s - M_h) / L_h over
//    their heads, and a fixed two-step butterfly totals the slot; mass and
//    importance are written at the slot's position.
//  - Item k of a sequence also writes its output rows h = k, k + K, ...
//    (K = the sequence's items): channels merged over the unit's partials in
//    a fixed order.
//  - Sequences without table entries get mass 0 below their length and zero
//    output rows, by workgroup b mod W.
constexpr int FT = 256;
constexpr int FB = 4;                 // entries a wave takes per item
constexpr int FC = FB * (FT / 64);    // entries per item
// resident finalize workgroups per compute unit at most; a workgroup's FT / 64
// waves spread over the unit's four SIMDs, so this is also the waves per SIMD
// the kernel's registers must allow
constexpr int FIN_PER_CU = 6;

// M_h and 1 / L_h of every head of sequence b (whose split-list entries
// start at pre and number n_packs x nb), into Mh / Rh: tpg lanes per head,
// each over a stride of the unit's segments, then a butterfly.  Called by
// the whole workgroup.
__device__ inline void head_stats(const DecodeWs &ws, const int *rs, int NW, int b, long pre, int nb, int Hq,
                                  int PG, int n_packs, float *Mh, float *Rh) {
    const int tid = threadIdx.x;
    int tpg = 64;
    while (tpg > 1 && tpg * Hq > FT) tpg >>= 1;
    for (int h0 = 0; h0 < Hq; h0 += FT / tpg) {
        const int h = h0 + tid / tpg, jj = tid % tpg;
        float M = -INFINITY, L = 0.f;
        if (h < Hq && nb > 0) {
            const int p = h / PG, hh = h % PG, u = b * n_packs + p;
            const long U0 = pre + (long)p * nb;
            const int j0 = range_owner(rs, NW, (int)U0), j1 = range_owner(rs, NW, (int)(U0 + nb - 1));
            for (int jb = j0 + jj; jb <= j1; jb += 4 * tpg) {
                float2 v[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int jx = jb + q * tpg;
                    const bool live = jx <= j1 && rs[jx] < rs[jx + 1];
                    v[q] = live ? reinterpret_cast<const float2 *>(ws.ml)[((size_t)jx + u) * 16 + hh]
                                : make_float2(-INFINITY, 0.f);
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (v[q].x == -INFINITY) continue;
                    if (v[q].x > M) {
                        L = L * exp2f(M - v[q].x) + v[q].y;
                        M = v[q].x;
                    } else {
                        L += v[q].y * exp2f(v[q].x - M);
                    }
                }
            }
        }
        for (int w = 1; w < tpg; w <<= 1) {
            const float Mo = __shfl_xor(M, w), Lo = __shfl_xor(L, w);
            const float MM = fmaxf(M, Mo);
            L = (M == -INFINITY ? 0.f : L * exp2f(M - MM)) + (Mo == -INFINITY ? 0.f : Lo * exp2f(Mo - MM));
            M = MM;
        }
        if (jj == 0 && h < Hq) {
            Mh[h] = M;
            Rh[h] = L > 0.f ? 1.0f / L : 0.f;
        }
    }
}

__global__ __launch_bounds__(FT, FIN_PER_CU) void attn_finalize(kvq_cache c, float *out, float *mass, float *importance,
                                                    float decay, DecodeWs ws, int NW, int G, int P, int n_packs) {
    const int j = blockIdx.x, W = gridDim.x;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int Hq = c.Hq, PG = P * G;
    __shared__ float Mh2[2][MAX_HQ], Rh2[2][MAX_HQ];   // by item parity
    __shared__ float4 red[FT];
    __shared__ int s_pre[MAX_B + 1];          // sequences' first entries (no pack factor)
    __shared__ int s_item[MAX_B + 1];         // sequences' first items
    __shared__ int s_rs[MAX_SPLIT_WGS + 1];   // split ranges' starts
    __shared__ int s_wsum[FT / 64];

    // -- the sequences' entry prefix, the split ranges, and the item prefix
    //    (a block scan over ceil(nb / FC), SPT consecutive sequences per
    //    thread, so that the prefix at B is written too)
    constexpr int SPT = (MAX_B + FT) / FT;
    for (int bb = tid; bb <= c.B; bb += FT) s_pre[bb] = ws.pre[bb] / n_packs;
    for (int k = tid; k <= NW; k += FT) s_rs[k] = ws.rstart[k];
    __syncthreads();
    {
        int cnt[SPT], tot = 0;
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
            const int bb = SPT * tid + i;
            cnt[i] = bb < c.B ? (s_pre[bb + 1] - s_pre[bb] + FC - 1) / FC : 0;
            tot += cnt[i];
        }
        int incl = tot;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(incl, d);
            if (lane >= d) incl += y;
        }
        if (lane == 63) s_wsum[wave] = incl;
        __syncthreads();
        int run = incl - tot;
        for (int w = 0; w < wave; ++w) run += s_wsum[w];
#pragma unroll
        for (int i = 0; i < SPT; ++i) {
            const int bb = SPT * tid + i;
            if (bb <= c.B) s_item[bb] = run;
            run += cnt[i];
        }
        __syncthreads();
    }
    const int n_items = s_item[c.B];

    // -- sequences with no table entries: no split segment zeroed their
    //    positions, so every one below seq_len gets mass 0 here, and their
    //    output rows are 0
    for (int bb = j; bb < c.B; bb += W) {
        if (s_pre[bb + 1] > s_pre[bb]) continue;
        const int len = min(c.seq_len[bb], c.n_cap);
        for (int p = tid; p < len; p += FT) mass[(size_t)bb * c.n_cap + p] = 0.f;
        for (int i = tid; i < Hq * HD; i += FT) out[(size_t)bb * Hq * HD + i] = 0.f;
    }

    const int t = lane >> 2, hq = lane & 3;
    for (int it = j, par = 0; it < n_items; it += W, par ^= 1) {
        float *const Mh = Mh2[par], *const Rh = Rh2[par];
        // the sequence of item it: the last b with s_item[b] <= it
        int b = 0;
        {
            int lo_b = 0, hi_b = c.B - 1;
            while (lo_b < hi_b) {
                const int mid = (lo_b + hi_b + 1) >> 1;
                if (s_item[mid] <= it) lo_b = mid; else hi_b = mid - 1;
            }
            b = lo_b;
        }
        const int nb = s_pre[b + 1] - s_pre[b], k = it - s_item[b], K = s_item[b + 1] - s_item[b];
        const int e0 = k * FC + wave * FB;   // this wave's first entry
        const long pre = (long)s_pre[b] * n_packs;

        // -- this wave's entries: table, then masks and positions, issued
        //    before the head statistics so their latency overlaps
        bool valid[FB];
        int pos[FB];
#pragma unroll
        for (int q = 0; q < FB; ++q) {
            valid[q] = false;
            pos[q] = -1;
            if (e0 + q < nb) {
                const uint32_t ent = c.table[(size_t)b * c.max_blocks + e0 + q];
                const int pool = (int)(ent >> 30);
                const uint32_t id = ent & 0x3fffffffu;
                valid[q] = (pool_sel(c.mask, pool)[id] >> t) & 1u;
                pos[q] = pool_sel(c.pos, pool)[(size_t)id * BLK + t];
            }
            // a position outside the row stride (a corrupt cache) is skipped
            if (pos[q] < 0 || pos[q] >= c.n_cap) valid[q] = false;
        }
        // -- the first pack's score rows and the old importance of the valid
        //    slots, issued before the partials are merged so that the two
        //    sets of loads are in flight together
        const float *const score_b = ws.score + (size_t)b * n_packs * c.max_blocks * 256;
        float4 sv0[FB];
        float imp_old[FB];
#pragma unroll
        for (int q = 0; q < FB; ++q)
            sv0[q] = valid[q] ? reinterpret_cast<const float4 *>(score_b + (size_t)(e0 + q) * 256)[t * 4 + hq]
                              : make_float4(0.f, 0.f, 0.f, 0.f);
        if (importance && hq == 0) {
#pragma unroll
            for (int q = 0; q < FB; ++q) imp_old[q] = valid[q] ? importance[(size_t)b * c.n_cap + pos[q]] : 0.f;
        }
        // (no barrier before: the statistics of the item before last, in
        // this buffer, were read before the last item's barrier below, so
        // the loads above stay in flight while the partials are merged)
        head_stats(ws, s_rs, NW, b, pre, nb, Hq, PG, n_packs, Mh, Rh);
        __syncthreads();

        // -- mass (and importance) of the valid slots
        {
            float acc[FB];
#pragma unroll
            for (int q = 0; q < FB; ++q) acc[q] = 0.f;
            for (int p = 0; p < n_packs; ++p) {
                float4 sv[FB];
#pragma unroll
                for (int q = 0; q < FB; ++q)
                    sv[q] = p == 0 ? sv0[q]
                          : valid[q] ? reinterpret_cast<const float4 *>(
                                           score_b + ((size_t)p * c.max_blocks + e0 + q) * 256)[t * 4 + hq]
                                     : make_float4(0.f, 0.f, 0.f, 0.f);
                const int np = min(P, c.Hkv - p * P);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int hh = 4 * hq + i;
                    if (hh >= np * G) continue;
                    const int h = p * PG + hh;
                    const float Mx = Mh[h], Rx = Rh[h];
                    if (Mx == -INFINITY) continue;
#pragma unroll
                    for (int q = 0; q < FB; ++q) {
                        const float sx = i == 0 ? sv[q].x : i == 1 ? sv[q].y : i == 2 ? sv[q].z : sv[q].w;
                        if (valid[q]) acc[q] = fmaf(exp2_fast(sx - Mx), Rx, acc[q]);
                    }
                }
            }
#pragma unroll
            for (int q = 0; q < FB; ++q) {
                acc[q] += __shfl_xor(acc[q], 1);
                acc[q] += __shfl_xor(acc[q], 2);
            }
            if (hq == 0) {
#pragma unroll
                for (int q = 0; q < FB; ++q) {
                    if (!valid[q]) continue;
                    mass[(size_t)b * c.n_cap + pos[q]] = acc[q];
                    if (importance) importance[(size_t)b * c.n_cap + pos[q]] = fmaf(decay, imp_old[q], acc[q]);
                }
            }
        }

        // -- output rows h = k, k + K, ...: 32 channel quads x 8 segment
        //    groups, merged in a fixed order
        for (int h = k; h < Hq; h += K) {
            const int c4 = tid & 31, sg = tid >> 5;
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
            const float Mx = Mh[h];
            if (Mx != -INFINITY) {
                const int p = h / PG, hh = h % PG, u = b * n_packs + p;
                const long U0 = pre + (long)p * nb;
                const int j0 = range_owner(s_rs, NW, (int)U0), j1 = range_owner(s_rs, NW, (int)(U0 + nb - 1));
                for (int jb = j0 + sg; jb <= j1; jb += 4 * 8) {
                    float mv[4];
                    float4 ov[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int jx = jb + 8 * q;
                        const bool live = jx <= j1 && s_rs[jx] < s_rs[jx + 1];
                        const size_t r = ((size_t)jx + u) * 16 + hh;
                        mv[q] = live ? ws.ml[r * 2] : -INFINITY;
                        ov[q] = live ? reinterpret_cast<const float4 *>(ws.o + r * HD)[c4] : make_float4(0.f, 0.f, 0.f, 0.f);
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        if (mv[q] == -INFINITY) continue;
                        const float fq = exp2f(mv[q] - Mx);
                        acc.x = fmaf(ov[q].x, fq, acc.x);
                        acc.y = fmaf(ov[q].y, fq, acc.y);
                        acc.z = fmaf(ov[q].z, fq, acc.z);
                        acc.w = fmaf(ov[q].w, fq, acc.w);
                    }
                }
            }
            red[tid] = acc;
            __syncthreads();
            if (tid < 32) {
                float4 sum = red[tid];
#pragma unroll
                for (int q = 1; q < 8; ++q) {
                    const float4 rr = red[q * 32 + tid];
                    sum.x += rr.x; sum.y += rr.y; sum.z += rr.z; sum.w += rr.w;
                }
                const float R = Rh[h];
                reinterpret_cast<float4 *>(out + ((size_t)b * Hq + h) * HD)[tid] =
                    make_float4(sum.x * R, sum.y * R, sum.z * R, sum.w * R);
            }
            __syncthreads();
        }
    }
}

}  // namespace

// Workgroups of attn_split<G, native> that fit on the device at once, and
// per compute unit (cached per device, G and codec).
int persistent_grid(int G, bool native, const void *kernel, int *per_cu_out) {
    static int cache[64][2][KVQ_MAX_GQA + 1], cache_cu[64][2][KVQ_MAX_GQA + 1];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int &v = cache[dev][native][G];
    if (v == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, WAVES * 64, 0) != hipSuccess)
            return 0;
        cache_cu[dev][native][G] = per_cu > 0 ? per_cu : 1;
        v = cus * cache_cu[dev][native][G];
    }
    *per_cu_out = cache_cu[dev][native][G];
    return v;
}

// Finalize workgroups that fit on the device at once, at most six per
// compute unit (cached per device).
int finalize_grid() {
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int &v = cache[dev];
    if (v == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(attn_finalize),
                                                         FT, 0) != hipSuccess)
            return 0;
        v = cus * std::max(1, std::min(per_cu, FIN_PER_CU));
    }
    return v;
}

bool launch_decode(const kvq_cache &c, const void *q, float *out, float *mass, float *importance,
                   float decay, float sm_scale, void *ws_ptr, hipStream_t s) {
    DecodeWs ws(ws_ptr, c);
    const int G = c.Hq / c.Hkv;
    const uint16_t *qq = static_cast<const uint16_t *>(q);
    const float scale2 = sm_scale * LOG2E;
    int NW = 0;
    // the split's workgroups j and j + NW / 2 share a compute unit when two fit
    // on one; the first-dispatched half takes the larger shares (split_start)
    switch (G) {
#define KVQ_GN(g, nat)                                                                                   \
    {                                                                                                    \
        int per_cu = 0;                                                                                  \
        const int fit = persistent_grid(g, nat, reinterpret_cast<const void *>(attn_split<g, nat>), &per_cu); \
        NW = std::min(fit, MAX_SPLIT_WGS);                                                               \
        if (NW <= 0) return false;                                                                       \
        const int n_first = per_cu == 2 && NW == fit ? NW / 2 : NW;                                      \
        hipLaunchKernelGGL((attn_split<g, nat>), dim3(NW), dim3(WAVES * 64), 0, s, c, qq, mass, ws, scale2, \
                           n_first);                                                                     \
    }
#define KVQ_G(g)                                                    \
    case g:                                                         \
        if (c.codec == KVQ_CODEC_NATIVE) KVQ_GN(g, true) else KVQ_GN(g, false) \
        break;
        KVQ_G(1) KVQ_G(2) KVQ_G(3) KVQ_G(4) KVQ_G(5) KVQ_G(6) KVQ_G(7) KVQ_G(8)
        KVQ_G(9) KVQ_G(10) KVQ_G(11) KVQ_G(12) KVQ_G(13) KVQ_G(14) KVQ_G(15) KVQ_G(16)
#undef KVQ_G
#undef KVQ_GN
        default: return false;
    }
    {
        // every finalize workgroup resident at once, at most six per compute
        // unit, and no more than the items a full table would give
        const int W = std::min(finalize_grid(), c.B * ((c.max_blocks + FC - 1) / FC));
        if (W <= 0) return false;
        hipLaunchKernelGGL(attn_finalize, dim3(W), dim3(FT), 0, s, c, out, mass, importance, decay, ws, NW, G,
                           decode_pack(G), decode_n_packs(c));
    }
    return hipGetLastError() == hipSuccess;
}

}  // namespace kvq
