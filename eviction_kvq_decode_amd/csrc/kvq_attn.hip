// kvq_attn.hip -- single-query decode attention over the typed, paged,
// quantised cache, with per-position attention mass and decayed importance.
//
// "Back from the Future", Problem Statement: scaled dot-product attention
// over the cached K/V.  "TAM", sections 1 and 2.B: the attention mass a
// position receives (summed over query heads) is the importance signal;
// accumulated H2O-style with a decay.  "ThinKV", Continuous Thinking: the
// kernel walks a block table whose blocks carry an eviction mask.
//
// attn_split: persistent workgroups over (sequence, kv-head pack, run of
//   table entries) items; runs are shortened when a small batch would leave
//   workgroups idle.  Online softmax in base 2; writes the run's (max, sum,
//   unnormalised output) and every score it computed (needed later for the
//   mass, whose normaliser is only known once all runs are done).
// attn_finalize: two workgroups per (sequence, run of table entries): merges
//   the runs (log-sum-exp), writes the output rows, and turns the stored
//   scores into mass / importance in a fixed head order (no float atomics).
#include <math.h>

#include <algorithm>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

constexpr int E = ENTRIES_PER_SPLIT;
constexpr int MAX_HQ = 256;
constexpr float LOG2E = 1.4426950408889634f;

// Table entries of a sequence, as the kernels read them (a count outside
// [0, max_blocks] in a corrupt cache is clamped).
__device__ inline int table_entries(const kvq_cache &c, int b) {
    return min(max(c.n_blocks[b], 0), c.max_blocks);
}

// Runs of a sequence with nb table entries when a run holds at most ew of
// them: never fewer than E-entry runs need, never more than S (the partials
// held per sequence; S * MIN_RUN >= max_blocks >= nb).
__device__ inline int seq_runs(int nb, int ew, int S) {
    if (nb <= 0) return 0;
    const int lo = (nb + E - 1) / E, nr = (nb + ew - 1) / ew;
    return nr < lo ? lo : (nr > S ? S : nr);
}

// Run j holds entries j, j + nr, ...: at most ceil(nb / nr) of them.  Its
// scores start at group j * run_stride: E-entry runs keep E-aligned areas
// (nr E <= max_blocks rounded up to E); shorter runs are packed at their
// longest length (nr ceil(nb / nr) < nb + nr <= max_blocks + S).
__device__ inline int run_stride(int nb, int nr, int ew) {
    return ew == E ? E : (nb + nr - 1) / nr;
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
// c << 8).  B is then about the size of the codes, so the bias can stay in
// the operand and be taken out of the fp32 sums at no cost in precision:
// through the q sums for K (B * sum q) and through the zero-point sums for
// V (B * sum P').  Only 8-bit K codes are unbiased before the product (one
// packed fp16 subtract), because the scores feed the per-token mass, whose
// tolerance is tighter than the 8 : 1 bias-to-code ratio allows.  (Operands
// with a zero exponent, c * 2^-24 subnormals, would need no bias but lose
// precision in the MFMA products on this hardware.)
template <int BITS>
struct Code {
    static constexpr float BIAS = BITS == 8 ? 1024.0f : BITS == 4 ? 16.0f : 4.0f;
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

// PV B operand: codes of tokens 4r..4r+3 at this lane's channel of tile n,
// as B + c (native E4M3 / E2M1 codes: their values).
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
    float z[NGRP];   // this lane's share of sum p * v_zero - B * P' / mult per group
    floatx4 o[8];    // sum P' * (B + code), P' = p * v_scale * mult, per 16-channel tile
    float mult;      // power-of-two headroom factor applied to P'
};

// ---------------------------------------------------------------------------
// Block staging.  Each wave owns an LDS stage that holds one block-pack: the
// (scale, zero) areas of its kv heads at a * 512, the block's 16 slot
// positions at P * 512 (first pack of a sequence only), kv head a's K codes
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
__host__ __device__ constexpr int stage_bytes(int P) { return P * STAGE_REGION + 64; }
__host__ __device__ constexpr int kcode0(int P) { return P * 512 + 64; }
__host__ __device__ constexpr int vcode0(int P) { return kcode0(P) + P * CODE_AREA; }

typedef __attribute__((address_space(3))) void lds_void;

// lane i: 16 bytes from gptr (its own address) + GOFF to lds_dst + 16 i.
// Written as an instruction the compiler does not track: its waits would
// otherwise drain every store behind these loads before any later LDS read
// (it cannot tell the stage from other LDS data).  The kernel waits for the
// loads itself.  The instruction has no register result; m0 carries the LDS
// base and needs one wait state before the load.
template <int GOFF = 0>
__device__ inline void lds_load16(const void *gptr, uint8_t *lds_dst) {
    const uint32_t lds = (uint32_t)(size_t)(lds_void *)lds_dst;
    const uint8_t *g = static_cast<const uint8_t *>(gptr) + GOFF;
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(g), "s"(lds)
                 : "memory", "m0");
}
// s_waitcnt encodings (gfx9): vmcnt(0), and lgkmcnt(0) alone
__device__ inline void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Issue the loads of one block-pack into `stage`, in two parts: PART_V
// (V codes and both (scale, zero) areas) and PART_K (K codes and the
// positions).  blk = the pack's first region (kv head kh0) in HBM; np kv heads
// are real; posb = the block's positions or null.
constexpr int PART_V = 1, PART_K = 2;
template <int BITS, int P, int PART>
__device__ inline void issue_block(uint8_t *stage, const uint8_t *blk, int np, uint32_t m16, const int *posb) {
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
    if constexpr (PART == PART_K) {
        if (posb != nullptr && lane < 4 && ((m16 >> (4 * lane)) & 15u))
            lds_load16(reinterpret_cast<const uint8_t *>(posb) + loff, stage + P * 512);
    }
}

// The next block-pack's loads, issued by attend_block in two parts: the V
// part once the current block's V codes, pairs and positions are in
// registers, the K part once its QK^T products have read the K codes.
struct NoNext {
    __device__ void operator()(int) const {}
};

// NAT: the block holds native E4M3 / E2M1 codes (symmetric, zero 0).
template <int G, int BITS, bool NAT, class Next>
__device__ inline void attend_block(const uint8_t *stage, int np, uint32_t m16, float *score, int *spos,
                                    int off, bool has_pos, const uint4 *const *qa, const float *qsum, float scale2,
                                    WaveState &st, const Next &next) {
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
    // -- the valid slots' scores, and from the first pack their positions,
    //    in the split's compacted numbering: valid slot t of this block is
    //    number off + (valid slots of the block before t)
    {
        int4 pos4 = make_int4(0, 0, 0, 0);
        if (has_pos && lo == 0) pos4 = reinterpret_cast<const int4 *>(stage + P * 512)[hi];
        const int pp[4] = {pos4.x, pos4.y, pos4.z, pos4.w};
        int cn = off + __popc(m16 & ((1u << (4 * hi)) - 1u));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (tv[i]) {
                if (row_ok) score[(cn >> 4) * 256 + lo * 16 + (cn & 15)] = s[i];
                if (has_pos && lo == 0) spos[cn] = pp[i];
                ++cn;
            }
        }
    }

    // -- the K and position reads have landed: the next block-pack's K part.
    //    No LDS read follows in this block, and the stores above were issued
    //    before it, so the next block waits for all of its wave's memory
    //    operations.
    wait_lgkm0();
    next(PART_K);
    // -- online softmax; the max only moves when some score exceeds it
    float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    if (__ballot(bm > st.m)) {
        bm = fmaxf(bm, __shfl_xor(bm, 16));
        bm = fmaxf(bm, __shfl_xor(bm, 32));
        const float mn = fmaxf(st.m, bm);
        const float alpha = st.m == -INFINITY ? 0.f : exp2_fast(st.m - mn);
        st.m = mn;
        st.l *= alpha;
#pragma unroll
        for (int g = 0; g < NGRP; ++g) st.z[g] *= alpha;
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * hi + i);
#pragma unroll
        for (int n = 0; n < 8; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) st.o[n][i] *= al[i];
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p[i] = s[i] == -INFINITY ? 0.f : exp2_fast(s[i] - st.m);
        st.l += p[i];
    }

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
            const float f = nm / st.mult;
            st.mult = nm;
#pragma unroll
            for (int n = 0; n < 8; ++n)
#pragma unroll
                for (int i = 0; i < 4; ++i) st.o[n][i] *= f;
        }
    }
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
    // zero-point term sum p * v_zero, less the V operands' bias share
    // B * P' / mult (native codes: neither)
    if constexpr (!NAT) {
        const float kb = -Code<BITS>::BIAS / st.mult;
#pragma unroll
        for (int g = 0; g < NGRP; ++g) {
            float zg = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                zg = fmaf(p[i], hi_h(vsz[4 * i + g]), zg);
                zg = fmaf(kb, (float)pop[g][i], zg);
            }
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
            st.o[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, v_operand<BITS, NAT>(vw[a], n, vb), st.o[n], 0, 0, 0);
        }
    }

}

// Workgroup LDS of the split kernel.  A wave's merged output rows reuse its
// stage's code area once every wave has left its loop; the prologue's scan
// buffer shares the stage area too.
template <int P>
struct SplitLds {
    uint32_t ent[E];
    int off[E];              // valid slots before entry k (compacted numbering)
    uint32_t msk[E];
    int n;
    uint4 qb[NGRP][65];      // [g][lane]: q of column head lane % 16, channel
                             // slice lane / 16 of group g; [g][64] is zero
    // wave merge: row maxima, scaled row sums and zero-point sums per wave
    float mm[WAVES][16], lw[WAVES][16], zz[WAVES][16][NGRP];
    // the stages; a wave's merged output rows go to its own stage's code
    // area (whose stale bytes are harmless), or after the stages when a
    // one-kv-head stage is too small for 16 rows
    union alignas(16) {
        uint8_t stage[WAVES * stage_bytes(P) + (P == 1 ? WAVES * 16 * HD * 4 : 0)];
        int scan[WAVES * 64];
    } u;
    __device__ float *merge_rows(int w) {
        return reinterpret_cast<float *>(u.stage + (P == 1 ? WAVES * stage_bytes(P) + w * 16 * HD * 4
                                                           : w * stage_bytes(P) + kcode0(P)));
    }
};

// One work item (sequence, kv-head pack, run of at most E entries).
template <int G, bool NATIVE>
__device__ inline void split_item(const kvq_cache &c, const uint16_t *q, const DecodeWs &ws,
                                  float scale2, int S, int span, int ew, int item, const int *s_first,
                                  SplitLds<PACK(G)> &sh) {
    constexpr int P = PACK(G);
    const int n_packs = (c.Hkv + P - 1) / P;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lo = lane & 15, hi = lane >> 4;
    // decode the item: sequence by binary search over the item prefix
    int lo_b = 0, hi_b = c.B - 1;
    while (lo_b < hi_b) {
        const int mid = (lo_b + hi_b + 1) >> 1;
        if (s_first[mid] <= item) lo_b = mid; else hi_b = mid - 1;
    }
    // (item values read from LDS are uniform: keep them in scalar registers)
    const int b = __builtin_amdgcn_readfirstlane(lo_b);
    const int r = __builtin_amdgcn_readfirstlane(item - s_first[b]);
    const int pack = r % n_packs, split = r / n_packs;
    const int kh0 = pack * P, np = min(P, c.Hkv - kh0);
    const bool row_ok = lo < np * G;

    // -- non-empty table entries of this run, compacted (wave 0).  Run j of
    //    a sequence with nr runs holds table entries j, j + nr, j + 2 nr, ...
    //    (at most E): every run samples the whole sequence, so the runs of a
    //    sequence cost about the same whatever the order of its block widths.
    const int nb = table_entries(c, b);
    const int nr = __builtin_amdgcn_readfirstlane((s_first[b + 1] - s_first[b]) / n_packs);
    if (wave == 0) {
        int n = 0, slots = 0;
        for (int base = 0; base < E; base += 64) {
            const int e = split + nr * (base + lane);
            uint32_t ent = 0, m = 0;
            if (base + lane < E && e < nb) {
                ent = c.table[(size_t)b * c.max_blocks + e];
                m = c.mask[ent >> 30][ent & 0x3fffffffu];
            }
            const uint64_t bal = __ballot(m != 0);
            const int at = n + __popcll(bal & ((1ull << lane) - 1));
            // valid slots of the entries before this one: a wave prefix sum
            int cnt = __popc(m), incl = cnt;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int y = __shfl_up(incl, d);
                if (lane >= d) incl += y;
            }
            if (m != 0) {
                sh.ent[at] = ent;
                sh.msk[at] = m;
                sh.off[at] = slots + incl - cnt;
            }
            n += __popcll(bal);
            slots += __shfl(incl, 63);
        }
        if (lane == 0) {
            sh.n = n;
            if (pack == 0) ws.ents[(size_t)b * S + split] = slots;
        }
    }

    // -- q of the pack's heads into LDS (zero past the pack), and the
    //    per-group q sums of head lo in registers
    float qsum[NGRP];
    {
        const int h = kh0 * G + lo;
#pragma unroll
        for (int g = 0; g < NGRP; ++g) {
            uint4 raw = make_uint4(0, 0, 0, 0);
            if (row_ok) raw = *reinterpret_cast<const uint4 *>(q + ((size_t)b * c.Hq + h) * HD + 32 * g + 8 * hi);
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

    // -- this wave's entries k = wave, wave + WAVES, ...: the loads of entry
    //    k + WAVES run while entry k is computed
    const int n_ent = __builtin_amdgcn_readfirstlane(sh.n);
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    uint8_t *stg = sh.u.stage + wv * stage_bytes(P);
    auto issue = [&](int k, int part) {
        // block metadata is wave-uniform: keep it in scalar registers
        const uint32_t ent = __builtin_amdgcn_readfirstlane(sh.ent[k]);
        const uint32_t msk = __builtin_amdgcn_readfirstlane(sh.msk[k]);
        const int pool = (int)(ent >> 30);
        const uint32_t id = ent & 0x3fffffffu;
        const int *pb = pack == 0 ? c.pos[pool] + (size_t)id * BLK : nullptr;
        const uint8_t *blk0 = c.kv[0] + ((size_t)id * c.Hkv + kh0) * (512u * 8 + 512u);
        const uint8_t *blk1 = c.kv[1] + ((size_t)id * c.Hkv + kh0) * (512u * 4 + 512u);
        const uint8_t *blk2 = c.kv[2] + ((size_t)id * c.Hkv + kh0) * (512u * 2 + 512u);
        if (part == PART_V) {
            if (pool == 0) issue_block<8, P, PART_V>(stg, blk0, np, msk, pb);
            else if (pool == 1) issue_block<4, P, PART_V>(stg, blk1, np, msk, pb);
            else issue_block<2, P, PART_V>(stg, blk2, np, msk, pb);
        } else {
            if (pool == 0) issue_block<8, P, PART_K>(stg, blk0, np, msk, pb);
            else if (pool == 1) issue_block<4, P, PART_K>(stg, blk1, np, msk, pb);
            else issue_block<2, P, PART_K>(stg, blk2, np, msk, pb);
        }
    };
    if (wv < n_ent) {
        issue(wv, PART_V);
        issue(wv, PART_K);
    }
    // the run's compacted scores of this pack, and its slot positions
    const int rst = __builtin_amdgcn_readfirstlane(run_stride(nb, nr, ew));
    const size_t roff = (size_t)b * span + (size_t)split * rst;
    float *score = ws.score + (roff * n_packs + (size_t)pack * rst) * 256;
    int *spos = ws.spos + roff * 16;
    for (int k = wv; k < n_ent; k += WAVES) {
        // entry k is in the stage once its wave's memory operations are done
        // (the last ones issued are its K part)
        wait_vm0();
        const uint32_t ent = __builtin_amdgcn_readfirstlane(sh.ent[k]);
        const uint32_t msk = __builtin_amdgcn_readfirstlane(sh.msk[k]);
        const int off = __builtin_amdgcn_readfirstlane(sh.off[k]);
        const int pool = (int)(ent >> 30);
        const int kn = k + WAVES;
        auto next = [&](int part) {
            if (kn < n_ent) issue(kn, part);
        };
        if (pool == 0)
            attend_block<G, 8, NATIVE>(stg, np, msk, score, spos, off, pack == 0, qa, qsum, scale2, st, next);
        else if (pool == 1)
            attend_block<G, 4, NATIVE>(stg, np, msk, score, spos, off, pack == 0, qa, qsum, scale2, st, next);
        else
            attend_block<G, 2, false>(stg, np, msk, score, spos, off, pack == 0, qa, qsum, scale2, st, next);
    }
    // -- merge the waves of this workgroup and write the run's partial.  Each
    //    wave publishes its row maxima, then writes its output rows already
    //    rescaled to the workgroup maximum (zero-point term included) into its
    //    own stage; the rows are then summed over the waves in a fixed order.
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
    if (hi == 0) {
        sh.mm[wave][lo] = st.m;
#pragma unroll
        for (int g = 0; g < NGRP; ++g) sh.zz[wave][lo][g] = zs[g];
    }
    __syncthreads();   // maxima and zero-point sums of every wave
    {
        // this lane's output rows are 4hi..4hi+3
        const float inv_mult = 1.0f / st.mult;
        float f[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * hi + i;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) M = fmaxf(M, sh.mm[w][r]);
            const float mw = sh.mm[wave][r];
            f[i] = mw == -INFINITY ? 0.f : exp2_fast(mw - M);
        }
        if (hi == 0) {
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) M = fmaxf(M, sh.mm[w][lo]);
            sh.lw[wave][lo] = st.m == -INFINITY ? 0.f : lsum * exp2_fast(st.m - M);
        }
        float *rows_out = sh.merge_rows(wave);
#pragma unroll
        for (int n = 0; n < 8; ++n)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * hi + i;
                rows_out[r * HD + 16 * n + lo] = f[i] * fmaf(st.o[n][i], inv_mult, sh.zz[wave][r][n >> 1]);
            }
    }
    __syncthreads();

    const int rows = np * G;
    for (int idx = tid; idx < rows * HD; idx += WAVES * 64) {
        const int rr = idx / HD, d = idx % HD;
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) o += sh.merge_rows(w)[rr * HD + d];
        const size_t hrow = (size_t)b * c.Hq + (size_t)kh0 * G + rr;
        ws.o[(hrow * S + split) * HD + d] = o;
        if (d == 0) {
            float M = -INFINITY, L = 0.f;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) M = fmaxf(M, sh.mm[w][rr]);
#pragma unroll
            for (int w = 0; w < WAVES; ++w) L += sh.lw[w][rr];
            ws.ml[(hrow * S + split) * 2 + 0] = M;
            ws.ml[(hrow * S + split) * 2 + 1] = L;
        }
    }
}

// Work items are (sequence, kv-head pack, run of at most ew table entries),
// ordered by sequence, run, pack, for the runs that hold entries.  The kernel is
// persistent: gridDim.x workgroups (what fits on the GPU at once) take the
// items round-robin, so the dispatcher never has to refill slots and no
// workgroup is launched for a run past a sequence's end.  The item prefix
// (B + 1 ints) lives in dynamic LDS.
// The run length ew is E, unless E-entry runs give fewer items than there
// are workgroups: then it is the shortest length whose items still fit in
// the grid, so that a small batch is spread over every workgroup in one
// round.  (Shortening runs to fill a partly idle last round of a larger
// batch was measured slower than E-entry runs.)
// NATIVE: the cache holds the native codec (Reasoning and Execution blocks
// in E4M3 / E2M1; Transition blocks are integer-coded in both codecs).
template <int G, bool NATIVE>
__global__ __launch_bounds__(WAVES * 64, KVQ_MIN_WAVES_PER_SIMD) void attn_split(kvq_cache c, const uint16_t *q, float *mass,
                                                         DecodeWs ws, float scale2, int S, int span) {
    constexpr int P = PACK(G);
    const int n_packs = (c.Hkv + P - 1) / P;
    const int tid = threadIdx.x;
    constexpr int NT = WAVES * 64;
    extern __shared__ int s_first[];
    __shared__ SplitLds<P> lds;
    __shared__ int s_carry;
    __shared__ int s_red[WAVES];

    // -- run length (the same in every workgroup; workgroup 0 publishes it
    //    for the finalize).  s_first holds the table entries until the prefix.
    for (int bb = tid; bb < c.B; bb += NT) s_first[bb] = table_entries(c, bb);
    __syncthreads();
    auto items_for = [&](int ew) {
        int n = 0;
        for (int bb = tid; bb < c.B; bb += NT) n += seq_runs(s_first[bb], ew, S);
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) n += __shfl_xor(n, d);
        if ((tid & 63) == 0) s_red[tid >> 6] = n;
        __syncthreads();
        int t = 0;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) t += s_red[w];
        __syncthreads();   // s_red is reused by the next call
        return t * n_packs;
    };
    int ew = E;
    if (items_for(E) < (int)gridDim.x) {
        for (int lo_e = 1; lo_e < ew;) {
            const int mid = (lo_e + ew) >> 1;
            if (items_for(mid) <= (int)gridDim.x) ew = mid;
            else lo_e = mid + 1;
        }
    }
    if (blockIdx.x == 0 && tid == 0) *ws.run_len = ew;

    // -- item prefix: s_first[b] = first item of sequence b (items per
    //    sequence = active runs * packs)
    if (tid == 0) s_carry = 0;
    __syncthreads();
    int *s_scan = lds.u.scan;
    for (int b0 = 0; b0 < c.B; b0 += NT) {
        const int bb = b0 + tid;
        const int cnt = bb < c.B ? seq_runs(s_first[bb], ew, S) * n_packs : 0;
        // inclusive scan of cnt over the workgroup (Hillis-Steele in LDS)
        s_scan[tid] = cnt;
        __syncthreads();
        for (int off = 1; off < NT; off <<= 1) {
            const int v = tid >= off ? s_scan[tid - off] : 0;
            __syncthreads();
            s_scan[tid] += v;
            __syncthreads();
        }
        if (bb < c.B) s_first[bb] = s_carry + s_scan[tid] - cnt;
        __syncthreads();
        if (tid == NT - 1) s_carry += s_scan[NT - 1];
        __syncthreads();
    }
    if (tid == 0) s_first[c.B] = s_carry;
    __syncthreads();
    const int n_items = s_first[c.B];

    // -- stage bytes start finite: zero the shared area once (the scan used it;
    //    later only loaded pairs and merged rows in the code areas land there)
    for (int i = tid; i < (int)(sizeof(lds.u) / 16); i += NT)
        reinterpret_cast<uint4 *>(&lds.u)[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();

    // -- every position below seq_len starts at mass 0; the finalize pass
    //    writes the valid ones.  Grid-stride over (sequence, position).
    for (int bb = 0; bb < c.B; ++bb) {
        const int len = min(c.seq_len[bb], c.n_cap);
        for (int p = blockIdx.x * NT + tid; p < len; p += gridDim.x * NT) mass[(size_t)bb * c.n_cap + p] = 0.f;
    }

    for (int item = blockIdx.x; item < n_items; item += gridDim.x)
        split_item<G, NATIVE>(c, q, ws, scale2, S, span, ew, item, s_first, lds);
}

// Finalize: gridDim.x workgroups per sequence, FPART of them per run:
// workgroup x takes runs x / FPART + k gridDim.x / FPART, and writes the
// output rows of heads x, x + gridDim.x, ...  A run's valid slots were stored compacted, in groups of
// 16; the run's workgroups and their waves take whole groups in turn:
// a group's scores (one 1 KB block [head][16 slots] per kv-head pack) are
// read with 1 KB loads, each lane summing exp2(s - M_h) / L_h over its head
// of every pack for 4 slots, and a fixed 16-lane butterfly totals the heads
// of each slot.
constexpr int FT = 256;
constexpr int FB = 4;                         // groups a wave takes per round
constexpr int FPK = 2;                        // kv-head packs whose scores are loaded together (4: slower)
#ifndef KVQ_FPART
#define KVQ_FPART 2
#endif
constexpr int FPART = KVQ_FPART;              // workgroups sharing one run's groups
constexpr int FIN_RUNS = 32;

__global__ __launch_bounds__(FT) void attn_finalize(kvq_cache c, float *out, float *mass, float *importance,
                                                    float decay, DecodeWs ws, int S, int span, int G, int P,
                                                    int n_packs) {
    const int x = blockIdx.x, b = blockIdx.y, X = gridDim.x, XS = X / FPART;
    const int part = x % FPART;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lo = lane & 15, hi = lane >> 4;
    const int nb = table_entries(c, b);
    const int ew = *ws.run_len;
    const int s_act = seq_runs(nb, ew, S);
    const int Hq = c.Hq;
    const int split0 = x < XS * FPART ? x / FPART : s_act;   // first run of this workgroup
    if (split0 >= s_act && x >= Hq) return;   // no slots and no output head
    __shared__ float Mh[MAX_HQ], Rh[MAX_HQ];
    __shared__ float4 red[FT];

    // -- global max / sum per head: tpg lanes of one wave per head, each over
    //    a stride of splits with its loads issued together, then a butterfly
    int tpg = 64;
    while (tpg > 1 && tpg * Hq > FT) tpg >>= 1;
    for (int h0 = 0; h0 < Hq; h0 += FT / tpg) {
        const int h = h0 + tid / tpg, jj = tid % tpg;
        float M = -INFINITY, L = 0.f;
        if (h < Hq) {
            const float2 *ml = reinterpret_cast<const float2 *>(ws.ml + ((size_t)b * Hq + h) * S * 2);
            for (int s0 = jj; s0 < s_act; s0 += 8 * tpg) {
                float2 v[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int s = s0 + u * tpg;
                    v[u] = s < s_act ? ml[s] : make_float2(-INFINITY, 0.f);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    if (v[u].x == -INFINITY) continue;
                    if (v[u].x > M) {
                        L = L * exp2f(M - v[u].x) + v[u].y;
                        M = v[u].x;
                    } else {
                        L += v[u].y * exp2f(v[u].x - M);
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
    __syncthreads();

    // -- mass (and importance) of the valid slots of this run, 16 at a time
    //    (a group k: lane (head lo, hi) takes slots 16 k + 4 hi .. + 3)
    auto run_mass = [&](int split) {
        const int n_slots = ws.ents[(size_t)b * S + split];
        const int n_ent = (n_slots + 15) >> 4;
        const int rst = run_stride(nb, s_act, ew);
        const size_t off = (size_t)b * span + (size_t)split * rst;
        for (int k0 = (part * (FT / 64) + wave) * FB; k0 < n_ent; k0 += FPART * (FT / 64) * FB) {
            int4 pos[FB];
            float acc[FB][4];
#pragma unroll
            for (int e = 0; e < FB; ++e) {
                const int k = k0 + e;
                pos[e] = k < n_ent ? reinterpret_cast<const int4 *>(ws.spos + (off + k) * 16)[hi]
                                   : make_int4(-1, -1, -1, -1);
                // slots past the run's last are stale
                const int c0 = 16 * k + 4 * hi;
                if (c0 + 0 >= n_slots) pos[e].x = -1;
                if (c0 + 1 >= n_slots) pos[e].y = -1;
                if (c0 + 2 >= n_slots) pos[e].z = -1;
                if (c0 + 3 >= n_slots) pos[e].w = -1;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[e][i] = 0.f;
            }
            // the importance of these positions, loaded before the scores so that
            // its latency overlaps theirs (lanes lo == 0 write the slots)
            float imp_old[FB][4];
            if (importance && lo == 0) {
#pragma unroll
                for (int e = 0; e < FB; ++e) {
                    const int pp[4] = {pos[e].x, pos[e].y, pos[e].z, pos[e].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        imp_old[e][i] = pp[i] >= 0 && pp[i] < c.n_cap ? importance[(size_t)b * c.n_cap + pp[i]] : 0.f;
                }
            }
            for (int p0 = 0; p0 < n_packs; p0 += FPK) {
                // FPK packs' scores of the round's groups, loads issued together
                float4 t[FB][FPK];
#pragma unroll
                for (int e = 0; e < FB; ++e)
#pragma unroll
                    for (int q = 0; q < FPK; ++q) {
                        const int k = k0 + e, p = p0 + q;
                        t[e][q] = k < n_ent && p < n_packs
                                      ? reinterpret_cast<const float4 *>(ws.score + (off * n_packs + (size_t)p * rst + k) * 256)[lo * 4 + hi]
                                      : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
                    }
#pragma unroll
                for (int q = 0; q < FPK; ++q) {
                    const int p = p0 + q;
                    const int col = p * P * G + lo;
                    const bool cv = p < n_packs && lo < min(P, c.Hkv - p * P) * G && Mh[min(col, Hq - 1)] != -INFINITY;
                    if (!cv) continue;
                    const float Mx = Mh[col], Rx = Rh[col];
#pragma unroll
                    for (int e = 0; e < FB; ++e) {
                        acc[e][0] = fmaf(exp2_fast(t[e][q].x - Mx), Rx, acc[e][0]);
                        acc[e][1] = fmaf(exp2_fast(t[e][q].y - Mx), Rx, acc[e][1]);
                        acc[e][2] = fmaf(exp2_fast(t[e][q].z - Mx), Rx, acc[e][2]);
                        acc[e][3] = fmaf(exp2_fast(t[e][q].w - Mx), Rx, acc[e][3]);
                    }
                }
            }
#pragma unroll
            for (int e = 0; e < FB; ++e)
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int w = 1; w < 16; w <<= 1) acc[e][i] += __shfl_xor(acc[e][i], w);
            if (lo == 0) {
#pragma unroll
                for (int e = 0; e < FB; ++e) {
                    const int pp[4] = {pos[e].x, pos[e].y, pos[e].z, pos[e].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        // a position outside the row stride (a corrupt cache) is skipped
                        if (pp[i] < 0 || pp[i] >= c.n_cap) continue;
                        mass[(size_t)b * c.n_cap + pp[i]] = acc[e][i];
                        if (importance) importance[(size_t)b * c.n_cap + pp[i]] = fmaf(decay, imp_old[e][i], acc[e][i]);
                    }
                }
            }
        }
    };
    // (the first run straight, further ones in a loop: a loop around the
    // only run of the usual case was measured slower)
    if (split0 < s_act) run_mass(split0);
    for (int split = split0 + XS; split < s_act; split += XS) run_mass(split);

    // -- output rows of the heads this workgroup owns: 32 channel quads x
    //    8 split groups, merged in a fixed order
    for (int h = x; h < Hq; h += X) {
        const int c4 = tid & 31, sg = tid >> 5;
        const float *ml = ws.ml + ((size_t)b * Hq + h) * S * 2;
        const float4 *o = reinterpret_cast<const float4 *>(ws.o + ((size_t)b * Hq + h) * S * HD);
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        const float Mx = Mh[h];
        for (int s0 = sg; s0 < s_act; s0 += 4 * 8) {
            float mv[4];
            float4 ov[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int s = s0 + 8 * u;
                mv[u] = s < s_act ? ml[2 * s] : -INFINITY;
                ov[u] = s < s_act ? o[(size_t)s * (HD / 4) + c4] : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (mv[u] == -INFINITY) continue;
                const float f = exp2f(mv[u] - Mx);
                acc.x = fmaf(ov[u].x, f, acc.x);
                acc.y = fmaf(ov[u].y, f, acc.y);
                acc.z = fmaf(ov[u].z, f, acc.z);
                acc.w = fmaf(ov[u].w, f, acc.w);
            }
        }
        red[tid] = acc;
        __syncthreads();
        if (tid < 32) {
            float4 sum = red[tid];
#pragma unroll
            for (int k = 1; k < 8; ++k) {
                const float4 r = red[k * 32 + tid];
                sum.x += r.x; sum.y += r.y; sum.z += r.z; sum.w += r.w;
            }
            const float R = Rh[h];
            reinterpret_cast<float4 *>(out + ((size_t)b * Hq + h) * HD)[tid] =
                make_float4(sum.x * R, sum.y * R, sum.z * R, sum.w * R);
        }
        __syncthreads();
    }
}

}  // namespace

// Workgroups of attn_split<G, native> that fit on the device at once, for a
// given dynamic LDS size (cached per device, G and codec).
int persistent_grid(int G, bool native, const void *kernel, size_t dyn_lds) {
    static int cache[64][2][KVQ_MAX_GQA + 1];
    static size_t cache_lds[64][2][KVQ_MAX_GQA + 1];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int &v = cache[dev][native][G];
    if (v == 0 || cache_lds[dev][native][G] != dyn_lds) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, WAVES * 64, dyn_lds) != hipSuccess)
            return 0;
        v = cus * (per_cu > 0 ? per_cu : 1);
        cache_lds[dev][native][G] = dyn_lds;
    }
    return v;
}

bool launch_decode(const kvq_cache &c, const void *q, float *out, float *mass, float *importance,
                   float decay, float sm_scale, void *ws_ptr, hipStream_t s) {
    DecodeWs ws(ws_ptr, c);
    const int S = n_splits(c), span = score_span(c);
    const int G = c.Hq / c.Hkv;
    const uint16_t *qq = static_cast<const uint16_t *>(q);
    const float scale2 = sm_scale * LOG2E;
    const size_t dyn = sizeof(int) * ((size_t)c.B + 1);   // item prefix of the split kernel
    switch (G) {
#define KVQ_GN(g, nat)                                                                                   \
    {                                                                                                    \
        const int grid = persistent_grid(g, nat, reinterpret_cast<const void *>(attn_split<g, nat>), dyn); \
        if (grid <= 0) return false;                                                                     \
        hipLaunchKernelGGL((attn_split<g, nat>), dim3(grid), dim3(WAVES * 64), dyn, s, c, qq, mass, ws, scale2, S, span); \
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
        const int P = decode_pack(G);
        // FIN_RUNS runs per sequence at a time (more are taken in turn), and
        // a workgroup per output head.  An odd run count per row keeps the
        // rows' busy workgroups from landing on the same compute units (with
        // 64 or 128 workgroups per row the finalize was measured 27% slower).
        const int X = FPART * (std::max(std::min(S, FIN_RUNS), (c.Hq + FPART - 1) / FPART) | 1);
        hipLaunchKernelGGL(attn_finalize, dim3(X, c.B), dim3(FT), 0, s, c, out, mass, importance, decay, ws, S, span, G, P,
                           decode_n_packs(c));
    }
    return hipGetLastError() == hipSuccess;
}

}  // namespace kvq
