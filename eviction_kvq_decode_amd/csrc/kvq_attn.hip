// kvq_attn.hip -- single-query decode attention over the typed, paged,
// quantised cache, with per-position attention mass and decayed importance.
//
// "Back from the Future", Problem Statement: scaled dot-product attention
// over the cached K/V.  "TAM", sections 1 and 2.B: the attention mass a
// position receives (summed over query heads) is the importance signal;
// accumulated H2O-style with a decay.  "ThinKV", Continuous Thinking: the
// kernel walks a block table whose blocks carry an eviction mask.
//
// attn_split: one workgroup per (sequence, kv head, run of table entries).
//   Online softmax in base 2; writes the split's (max, sum, unnormalised
//   output) and every score it computed (needed later for the mass, whose
//   normaliser is only known once all splits are done).
// attn_finalize: one workgroup per (sequence, run of table entries): merges
//   the splits (log-sum-exp), writes the output rows, and turns the stored
//   scores into mass / importance in a fixed head order (no float atomics).
#include <math.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

constexpr int E = ENTRIES_PER_SPLIT;
constexpr int MAX_HQ = 256;
constexpr int MAX_B = 1024;       // sequences per call handled by the split kernel's item prefix
constexpr float LOG2E = 1.4426950408889634f;

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
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
constexpr uint32_t BIAS2 = 0x64006400u;   // two fp16 1024.0: (1024 + c) has c in its low bits

// Codes become exact integer-valued fp16 operands: the code bits are placed
// under the exponent of 1024 (0x64 high byte), giving 1024 + c, and 1024 is
// subtracted with one packed fp16 add.  (Operands with a zero exponent,
// i.e. c * 2^-24 subnormals, would save the subtract but lose precision in
// the MFMA products on this hardware.)
__device__ inline uint32_t unbias(uint32_t x) {
    half2v h = __builtin_bit_cast(half2v, x);
    h = h - (half2v){(_Float16)1024.0f, (_Float16)1024.0f};
    return __builtin_bit_cast(uint32_t, h);
}
// Bytes i and j of w as the exact fp16 pair (w.byte[i], w.byte[j]).
__device__ inline uint32_t byte_pair(uint32_t w, int i, int j) {
    const uint32_t sel = (uint32_t)(4 + i) | ((uint32_t)(4 + j) << 16);  // selector 0: a 0x64 byte
    return unbias(__builtin_amdgcn_perm(w, 0x64646464u, sel));
}
// Fields at bit offsets sh and sh+16 of w (mask m per field) as an exact fp16 pair.
__device__ inline uint32_t field_pair(uint32_t w, int sh, uint32_t m) {
    return unbias(((w >> sh) & m) | BIAS2);
}

// QK A operand: the eight codes of group g held by this lane's K slice,
// in channel order e0..e7 (see the K row layout).
template <int BITS>
__device__ inline half8 k_operand(const uint32_t *kw, int g) {
    uint32_t r[4];
    if constexpr (BITS == 8) {
        r[0] = byte_pair(kw[2 * g], 0, 1);
        r[1] = byte_pair(kw[2 * g], 2, 3);
        r[2] = byte_pair(kw[2 * g + 1], 0, 1);
        r[3] = byte_pair(kw[2 * g + 1], 2, 3);
    } else if constexpr (BITS == 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) r[k] = field_pair(kw[g], 4 * k, 0x000F000Fu);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) r[k] = field_pair(kw[g >> 1], 2 * (4 * (g & 1) + k), 0x00030003u);
    }
    return __builtin_bit_cast(half8, r);
}

// PV B operand: codes of tokens 4r..4r+3 at this lane's channel of tile n.
template <int BITS>
__device__ inline half4 v_operand(const uint32_t *vw, int n) {
    uint32_t r[2];
    if constexpr (BITS == 8) {
        r[0] = byte_pair(vw[n], 0, 2);
        r[1] = byte_pair(vw[n], 1, 3);
    } else if constexpr (BITS == 4) {
        const int m = n & 1;
        r[0] = field_pair(vw[n >> 1], 8 * m, 0x000F000Fu);
        r[1] = field_pair(vw[n >> 1], 8 * m + 4, 0x000F000Fu);
    } else {
        const int m = n & 3;
        r[0] = field_pair(vw[n >> 2], 4 * m, 0x00030003u);
        r[1] = field_pair(vw[n >> 2], 4 * m + 2, 0x00030003u);
    }
    return __builtin_bit_cast(half4, r);
}

__device__ inline float lo_h(uint32_t x) { return h2f((uint16_t)(x & 0xffff)); }
__device__ inline float hi_h(uint32_t x) { return h2f((uint16_t)(x >> 16)); }

// Per-wave running state for the G query heads of each kv head in the pack.
// Lane (rho = lane % 16, r = lane / 16) owns head rho and, inside a block,
// tokens 4r..4r+3; the PV accumulators O[n] hold heads 4r..4r+3 at
// channel 16n + lane % 16.
struct WaveState {
    float m;         // running max of head rho (base-2 scaled scores)
    float l;         // this lane's share of the running sum
    float z[NGRP];   // this lane's share of sum p * v_zero per group
    floatx4 o[8];    // sum p * v_scale * mult * code, per 16-channel tile
    float mult;      // power-of-two headroom factor applied to P'
};

// The block's slot positions, read by the first kv-head pack only.
__device__ inline const int *pos_blk(const kvq_cache &c, int pool, uint32_t id, int pack) {
    return pack == 0 ? c.pos[pool] + (size_t)id * BLK : nullptr;
}

template <int G, int BITS>
__device__ inline void attend_block(const kvq_cache &c, const uint8_t *pool_base, uint32_t id, int kh0,
                                    int np, uint32_t m16, float *srow, int *prow, const int *pos_blk,
                                    const uint4 (*qop)[NGRP][64], const float *qsum, float scale2,
                                    const DecodeWs &ws, WaveState &st) {
    constexpr int P = PACK(G);
    const int lane = threadIdx.x & 63, lo = lane & 15, hi = lane >> 4;
    const int a_rho = min(lo / G, np - 1);
    const bool row_ok = lo < np * G;
    const long RB = 512L * BITS + 512L;
    const uint8_t *blk = pool_base + (long)id * c.Hkv * RB;

    // -- loads: K and V code slices of every kv head in the pack, and the
    //    (scale, zero) pairs of this lane's four tokens for its own kv head
    constexpr int KW = BITS;          // dwords per K slice: 32 codes * BITS / 32
    constexpr int VW = BITS;          // dwords per V slice: 32 codes * BITS / 32
    // a lane skips the bytes of evicted slots: its K row if token lo is
    // cleared, its V slice and (scale, zero) pairs if all four tokens
    // 4hi..4hi+3 are cleared.  Skipped code registers keep stale values:
    // they are finite subnormals whose products are masked (K) or meet
    // P' = 0 (V); the (scale, zero) consumers select on g_live.
    const bool k_live = (m16 >> lo) & 1u;
    const bool g_live = (m16 >> (4 * hi)) & 15u;
    const uint32_t k_off = lo * 16 * BITS + hi * 4 * BITS;          // K slice of token lo
    const uint32_t v_off = 256 * BITS + lane * (BITS == 2 ? 8 : 16); // V slice of lane
    const uint32_t sz_off = 512 * BITS + 64 * hi;                   // tokens 4hi..4hi+3
    uint32_t kw[P][KW], vw[P][VW];
#pragma unroll
    for (int a = 0; a < P; ++a) {
        // a partial pack re-reads its last kv head; the zero q / P' operands
        // of the missing heads cancel those products
        const uint8_t *reg = blk + (uint32_t)(kh0 + min(a, np - 1)) * (uint32_t)RB;
        if constexpr (BITS == 8) {
            if (k_live) {
                const uint4 k0 = *reinterpret_cast<const uint4 *>(reg + k_off);
                const uint4 k1 = *reinterpret_cast<const uint4 *>(reg + k_off + 16);
                kw[a][0] = k0.x; kw[a][1] = k0.y; kw[a][2] = k0.z; kw[a][3] = k0.w;
                kw[a][4] = k1.x; kw[a][5] = k1.y; kw[a][6] = k1.z; kw[a][7] = k1.w;
            }
            if (g_live) {
                const uint4 v0 = *reinterpret_cast<const uint4 *>(reg + v_off);
                const uint4 v1 = *reinterpret_cast<const uint4 *>(reg + v_off + 1024);
                vw[a][0] = v0.x; vw[a][1] = v0.y; vw[a][2] = v0.z; vw[a][3] = v0.w;
                vw[a][4] = v1.x; vw[a][5] = v1.y; vw[a][6] = v1.z; vw[a][7] = v1.w;
            }
        } else if constexpr (BITS == 4) {
            if (k_live) {
                const uint4 k0 = *reinterpret_cast<const uint4 *>(reg + k_off);
                kw[a][0] = k0.x; kw[a][1] = k0.y; kw[a][2] = k0.z; kw[a][3] = k0.w;
            }
            if (g_live) {
                const uint4 v0 = *reinterpret_cast<const uint4 *>(reg + v_off);
                vw[a][0] = v0.x; vw[a][1] = v0.y; vw[a][2] = v0.z; vw[a][3] = v0.w;
            }
        } else {
            if (k_live) {
                const uint2 k0 = *reinterpret_cast<const uint2 *>(reg + k_off);
                kw[a][0] = k0.x; kw[a][1] = k0.y;
            }
            if (g_live) {
                const uint2 v0 = *reinterpret_cast<const uint2 *>(reg + v_off);
                vw[a][0] = v0.x; vw[a][1] = v0.y;
            }
        }
    }
    // positions of tokens 4hi..4hi+3 (one lane per token group, first pack
    // of the sequence only): copied next to the score rows
    int4 pos4 = make_int4(0, 0, 0, 0);
    if (pos_blk != nullptr && lo == 0 && g_live) pos4 = reinterpret_cast<const int4 *>(pos_blk)[hi];
    const uint8_t *own = blk + (uint32_t)(kh0 + a_rho) * (uint32_t)RB + sz_off;
    uint32_t ksz[16], vsz[16];
    if (g_live) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 kq = reinterpret_cast<const uint4 *>(own)[i];
            const uint4 vq = reinterpret_cast<const uint4 *>(own + 256)[i];
            ksz[4 * i + 0] = kq.x; ksz[4 * i + 1] = kq.y; ksz[4 * i + 2] = kq.z; ksz[4 * i + 3] = kq.w;
            vsz[4 * i + 0] = vq.x; vsz[4 * i + 1] = vq.y; vsz[4 * i + 2] = vq.z; vsz[4 * i + 3] = vq.w;
        }
    }

    // -- QK^T per group: rows = tokens, columns = the pack's 16 query heads;
    //    a kv head's codes meet only its own heads (block-diagonal q)
    floatx4 acc[NGRP];
#pragma unroll
    for (int g = 0; g < NGRP; ++g) acc[g] = (floatx4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int a = 0; a < P; ++a) {
#pragma unroll
        for (int g = 0; g < NGRP; ++g) {
            const half8 qb = __builtin_bit_cast(half8, qop[a][g][lane]);
            acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand<BITS>(kw[a], g), qb, acc[g], 0, 0, 0);
        }
    }

    // -- scores of tokens 4hi..4hi+3 for head lo: fold the group scales and
    //    zeros, base-2 scale, mask cleared slots
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // group by group, so each group's scale and zero terms (which largely
        // cancel) meet before the next group is added
        float v = 0.f;
#pragma unroll
        for (int g = 0; g < NGRP; ++g) {
            const uint32_t sz = ksz[4 * i + g];
            v = fmaf(lo_h(sz), acc[g][i], v);
            v = fmaf(hi_h(sz), qsum[g], v);
        }
        const bool valid = row_ok && ((m16 >> (4 * hi + i)) & 1u);
        s[i] = valid ? v * scale2 : -INFINITY;
    }
    {
        // score rows: valid slots only, in slot order from srow; the Hq
        // scores of a slot are contiguous
        const uint32_t below = m16 & ((1u << (4 * hi)) - 1u);
        float *sp = srow + (size_t)__popc(below) * c.Hq + (size_t)kh0 * G + lo;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (s[i] != -INFINITY) {
                *sp = s[i];
                sp += c.Hq;
            }
        if (pos_blk != nullptr && lo == 0) {
            int *pp = prow + __popc(below);
            const int pv[4] = {pos4.x, pos4.y, pos4.z, pos4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if ((m16 >> (4 * hi + i)) & 1u) *pp++ = pv[i];
        }
    }

    // -- online softmax; the max only moves when some score exceeds it
    float bm = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    if (__ballot(bm > st.m)) {
        bm = fmaxf(bm, __shfl_xor(bm, 16));
        bm = fmaxf(bm, __shfl_xor(bm, 32));
        const float mn = fmaxf(st.m, bm);
        const float alpha = st.m == -INFINITY ? 0.f : exp2f(st.m - mn);
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
        p[i] = s[i] == -INFINITY ? 0.f : exp2f(s[i] - st.m);
        st.l += p[i];
    }

    // -- headroom for P' = p * v_scale * mult in fp16
    {
        float vmax = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) vmax = fmaxf(vmax, lo_h(vsz[j]));
        vmax = g_live ? vmax : 0.f;
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

    // -- P' per group in the PV A-operand layout (lane = head, 4 tokens), and
    //    the zero-point term
    half4 pop[NGRP];
#pragma unroll
    for (int g = 0; g < NGRP; ++g) {
        half4 t;
        float zg = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t sz = vsz[4 * i + g];
            t[i] = (_Float16)(p[i] * lo_h(sz) * st.mult);
            zg = fmaf(p[i], hi_h(sz), zg);
        }
        st.z[g] += g_live ? zg : 0.f;
        pop[g] = g_live ? t : (half4){};
    }

    // -- PV: block-diagonal over the pack's kv heads
#pragma unroll
    for (int a = 0; a < P; ++a) {
        const bool mine = a_rho == a && row_ok;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const half4 pa = mine ? pop[n >> 1] : (half4){};
            st.o[n] = __builtin_amdgcn_mfma_f32_16x16x16f16(pa, v_operand<BITS>(vw[a], n), st.o[n], 0, 0, 0);
        }
    }
}

// Workgroup LDS of the split kernel.
template <int P>
struct SplitLds {
    uint32_t ent[E];
    uint32_t msk[E];
    int rb[E];         // first score row of the entry within the run
    int n;
    uint4 q[P][NGRP][64];
    float m[WAVES][16], l[WAVES][16], z[WAVES][16][NGRP];
    float o[WAVES][16][HD];
};

// One work item (sequence, kv-head pack, run of E entries).
template <int G>
__device__ inline void split_item(const kvq_cache &c, const uint16_t *q, const DecodeWs &ws,
                                        float scale2, int S, int item, const int *s_first,
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
    const int b = lo_b;
    const int r = item - s_first[b];
    const int pack = r % n_packs, split = r / n_packs;
    const int kh0 = pack * P, np = min(P, c.Hkv - kh0);
    const bool row_ok = lo < np * G;

    // -- non-empty table entries of this run, compacted (wave 0)
    const int nb = c.n_blocks[b];
    const int e0 = split * E;
    if (wave == 0) {
        int n = 0, rows = 0;
        for (int base = 0; base < E; base += 64) {
            const int e = e0 + base + lane;
            uint32_t ent = 0, m = 0;
            if (base + lane < E && e < nb) {
                ent = c.table[(size_t)b * c.max_blocks + e];
                m = c.mask[ent >> 30][ent & 0x3fffffffu];
            }
            const uint64_t bal = __ballot(m != 0);
            const int at = n + __popcll(bal & ((1ull << lane) - 1));
            // exclusive prefix of valid-slot counts: the entry's first row
            int cnt = __popc(m), incl = cnt;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int v = __shfl_up(incl, d);
                if (lane >= d) incl += v;
            }
            if (m != 0) {
                sh.ent[at] = ent;
                sh.msk[at] = m;
                sh.rb[at] = rows + incl - cnt;
            }
            n += __popcll(bal);
            rows += __shfl(incl, 63);
        }
        if (lane == 0) {
            sh.n = n;
            if (pack == 0) ws.rows[(size_t)b * S + split] = rows;
        }
    }

    // -- q operands: sh.q[a][g][lane] is q of head lo, channel slice hi of
    //    group g if head lo belongs to kv head a of the pack, else zero
    //    (block-diagonal columns); per-group q sums of head lo in registers
    float qsum[NGRP];
    {
        const int h = kh0 * G + lo;
        const int a_lo = lo / G;
#pragma unroll
        for (int g = 0; g < NGRP; ++g) {
            uint4 raw = make_uint4(0, 0, 0, 0);
            if (row_ok) raw = *reinterpret_cast<const uint4 *>(q + ((size_t)b * c.Hq + h) * HD + 32 * g + 8 * hi);
            if (wave == 0)
#pragma unroll
                for (int a = 0; a < P; ++a) sh.q[a][g][lane] = a == a_lo ? raw : make_uint4(0, 0, 0, 0);
            const half8 qv = __builtin_bit_cast(half8, raw);
            float sum = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) sum += (float)qv[i];
            sum += __shfl_xor(sum, 16);
            sum += __shfl_xor(sum, 32);
            qsum[g] = sum;
        }
    }
    __syncthreads();

    WaveState st;
    st.m = -INFINITY;
    st.l = 0.f;
    st.mult = 4096.f;
#pragma unroll
    for (int g = 0; g < NGRP; ++g) st.z[g] = 0.f;
#pragma unroll
    for (int n = 0; n < 8; ++n) st.o[n] = (floatx4){0.f, 0.f, 0.f, 0.f};

    const int n_ent = sh.n;
    for (int k = wave; k < n_ent; k += WAVES) {
        // block metadata is wave-uniform: keep it in scalar registers
        const uint32_t ent = __builtin_amdgcn_readfirstlane(sh.ent[k]);
        const uint32_t msk = __builtin_amdgcn_readfirstlane(sh.msk[k]);
        const size_t row0 = (size_t)(b * S + split) * (E * BLK) + (size_t)__builtin_amdgcn_readfirstlane(sh.rb[k]);
        float *srow = ws.score + row0 * c.Hq;
        int *prow = ws.spos + row0;
        const int pool = (int)(ent >> 30);
        const uint32_t id = ent & 0x3fffffffu;
        if (pool == 0)
            attend_block<G, 8>(c, c.kv[0], id, kh0, np, msk, srow, prow, pos_blk(c, 0, id, pack), sh.q, qsum, scale2, ws, st);
        else if (pool == 1)
            attend_block<G, 4>(c, c.kv[1], id, kh0, np, msk, srow, prow, pos_blk(c, 1, id, pack), sh.q, qsum, scale2, ws, st);
        else
            attend_block<G, 2>(c, c.kv[2], id, kh0, np, msk, srow, prow, pos_blk(c, 2, id, pack), sh.q, qsum, scale2, ws, st);
    }

    // -- merge the waves of this workgroup and write the run's partial
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
        sh.m[wave][lo] = st.m;
        sh.l[wave][lo] = lsum;
#pragma unroll
        for (int g = 0; g < NGRP; ++g) sh.z[wave][lo][g] = zs[g];
    }
    const float inv_mult = 1.0f / st.mult;
#pragma unroll
    for (int n = 0; n < 8; ++n)
#pragma unroll
        for (int i = 0; i < 4; ++i) sh.o[wave][4 * hi + i][16 * n + lo] = st.o[n][i] * inv_mult;
    __syncthreads();

    const int rows = np * G;
    for (int idx = tid; idx < rows * HD; idx += WAVES * 64) {
        const int rr = idx / HD, d = idx % HD;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) M = fmaxf(M, sh.m[w][rr]);
        float L = 0.f, o = 0.f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) {
            const float mw = sh.m[w][rr];
            const float f = mw == -INFINITY ? 0.f : exp2f(mw - M);
            L = fmaf(sh.l[w][rr], f, L);
            o = fmaf(sh.o[w][rr][d] + sh.z[w][rr][d / GS], f, o);
        }
        const size_t hrow = (size_t)b * c.Hq + (size_t)kh0 * G + rr;
        ws.o[(hrow * S + split) * HD + d] = o;
        if (d == 0) {
            ws.ml[(hrow * S + split) * 2 + 0] = M;
            ws.ml[(hrow * S + split) * 2 + 1] = L;
        }
    }
    __syncthreads();   // LDS is reused by the next item
}

// Work items are (sequence, kv-head pack, run of E table entries), ordered
// by sequence, pack, run, for the runs that hold entries.  The kernel is
// persistent: gridDim.x workgroups (what fits on the GPU at once) take the
// items round-robin, so the dispatcher never has to refill slots and no
// workgroup is launched for a run past a sequence's end.
template <int G>
__global__ __launch_bounds__(WAVES * 64, KVQ_MIN_WAVES_PER_SIMD) void attn_split(kvq_cache c, const uint16_t *q, float *mass,
                                                         DecodeWs ws, float scale2, int S) {
    constexpr int P = PACK(G);
    const int n_packs = (c.Hkv + P - 1) / P;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int lo = lane & 15, hi = lane >> 4;
    constexpr int NT = WAVES * 64;

    // -- item prefix: s_first[b] = first item of sequence b (items per
    //    sequence = active runs * packs)
    __shared__ int s_first[MAX_B + 1];
    __shared__ int s_carry;
    if (tid == 0) s_carry = 0;
    __syncthreads();
    for (int b0 = 0; b0 < c.B; b0 += NT) {
        const int bb = b0 + tid;
        const int cnt = bb < c.B ? ((c.n_blocks[bb] + E - 1) / E) * n_packs : 0;
        // inclusive scan of cnt over the workgroup (Hillis-Steele in LDS)
        __shared__ int s_scan[NT];
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

    // -- every position below seq_len starts at mass 0; the finalize pass
    //    writes the valid ones.  Grid-stride over (sequence, position).
    for (int bb = 0; bb < c.B; ++bb) {
        const int len = c.seq_len[bb];
        for (int p = blockIdx.x * NT + tid; p < len; p += gridDim.x * NT) mass[(size_t)bb * c.n_cap + p] = 0.f;
    }

    __shared__ SplitLds<P> lds;
    for (int item = blockIdx.x; item < n_items; item += gridDim.x)
        split_item<G>(c, q, ws, scale2, S, item, s_first, lds);
}

// Finalize: one workgroup per (run of E entries, sequence).  The run's
// valid slots are rows of Hq scores with their positions; RPL lanes share a
// row, each reading four heads.  Two dependent rounds of loads: the row
// count and split partials, then the rows.
constexpr int FT = 256;

template <int RPL>
__global__ __launch_bounds__(FT) void attn_finalize(kvq_cache c, float *out, float *mass,
                                                    float *importance, float decay, DecodeWs ws, int S) {
    constexpr int ROWS = FT / RPL;             // rows one pass of the workgroup covers
    constexpr int BATCH = 16;                  // passes whose loads are issued together
    static_assert(2 * RPL >= BATCH, "row positions: two passes per lane");
    const int split = blockIdx.x, b = blockIdx.y, X = gridDim.x;
    const int tid = threadIdx.x, j = tid % RPL;
    const int nb = c.n_blocks[b];
    const int s_act = (nb + E - 1) / E;
    const int Hq = c.Hq;
    if (split >= s_act && split >= Hq) return;   // no rows and no output head
    __shared__ float Mh[MAX_HQ], Rh[MAX_HQ];
    __shared__ float4 red[FT];

    // (1) row count, split (m, l) pairs of every head, and the partial
    //     outputs of the head this workgroup writes
    const int n_rows = split < s_act ? ws.rows[(size_t)b * S + split] : 0;
    int tpg = 64;
    while (tpg > 1 && tpg * Hq > FT) tpg >>= 1;
    float M = -INFINITY, L = 0.f;
    {
        // one pass of tpg lanes per head covers Hq <= FT / tpg heads; more
        // heads take more passes below
        const int h = tid / tpg, jj = tid % tpg;
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
    }

    // (2) score rows and positions of the first batch
    const bool vec = (Hq & 3) == 0 && Hq <= 4 * RPL;
    const size_t row0 = (size_t)(b * S + split) * (E * BLK);
    float4 sv[BATCH];
    int pv[2];          // positions of passes 2j and 2j + 1 of this lane's row group
    auto load_batch = [&](int r0) {
#pragma unroll
        for (int ps = 0; ps < BATCH; ++ps) {
            const int r = r0 + ps * ROWS + tid / RPL;
            sv[ps] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (r < n_rows && vec && 4 * j < Hq)
                sv[ps] = *reinterpret_cast<const float4 *>(ws.score + (row0 + r) * Hq + 4 * j);
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int ps = 2 * j + u;
            const int r = r0 + ps * ROWS + tid / RPL;
            pv[u] = ps < BATCH && r < n_rows ? ws.spos[row0 + r] : 0;
        }
    };
    load_batch(0);

    // (3) global max / sum per head (butterfly over the tpg lanes)
    for (int w = 1; w < tpg; w <<= 1) {
        const float Mo = __shfl_xor(M, w), Lo = __shfl_xor(L, w);
        const float MM = fmaxf(M, Mo);
        L = (M == -INFINITY ? 0.f : L * exp2f(M - MM)) + (Mo == -INFINITY ? 0.f : Lo * exp2f(Mo - MM));
        M = MM;
    }
    if (tid % tpg == 0 && tid / tpg < Hq) {
        Mh[tid / tpg] = M;
        Rh[tid / tpg] = L > 0.f ? 1.0f / L : 0.f;
    }
    for (int h0 = FT / tpg; h0 < Hq; h0 += FT / tpg) {   // heads beyond one pass
        const int h = h0 + tid / tpg, jj = tid % tpg;
        float Mx = -INFINITY, Lx = 0.f;
        if (h < Hq) {
            const float2 *ml = reinterpret_cast<const float2 *>(ws.ml + ((size_t)b * Hq + h) * S * 2);
            for (int s = jj; s < s_act; s += tpg) {
                const float2 v = ml[s];
                if (v.x == -INFINITY) continue;
                if (v.x > Mx) {
                    Lx = Lx * exp2f(Mx - v.x) + v.y;
                    Mx = v.x;
                } else {
                    Lx += v.y * exp2f(v.x - Mx);
                }
            }
        }
        for (int w = 1; w < tpg; w <<= 1) {
            const float Mo = __shfl_xor(Mx, w), Lo = __shfl_xor(Lx, w);
            const float MM = fmaxf(Mx, Mo);
            Lx = (Mx == -INFINITY ? 0.f : Lx * exp2f(Mx - MM)) + (Mo == -INFINITY ? 0.f : Lo * exp2f(Mo - MM));
            Mx = MM;
        }
        if (jj == 0 && h < Hq) {
            Mh[h] = Mx;
            Rh[h] = Lx > 0.f ? 1.0f / Lx : 0.f;
        }
    }
    __syncthreads();

    // (5) mass (and importance) of each row: partial sums over the lane's
    //     heads, then a fixed-order butterfly
    float4 m4 = make_float4(0.f, 0.f, 0.f, 0.f), r4 = m4;
    if (vec && 4 * j < Hq) {
        m4 = *reinterpret_cast<const float4 *>(&Mh[4 * j]);
        r4 = *reinterpret_cast<const float4 *>(&Rh[4 * j]);
    }
    for (int r0 = 0; r0 < n_rows; r0 += BATCH * ROWS) {
        if (r0 > 0) load_batch(r0);
#pragma unroll
        for (int ps = 0; ps < BATCH; ++ps) {
            const int r = r0 + ps * ROWS + tid / RPL;
            const bool valid = r < n_rows;
            float sum = 0.f;
            if (valid) {
                if (vec) {
                    sum = exp2f(sv[ps].x - m4.x) * r4.x;
                    sum += exp2f(sv[ps].y - m4.y) * r4.y;
                    sum += exp2f(sv[ps].z - m4.z) * r4.z;
                    sum += exp2f(sv[ps].w - m4.w) * r4.w;
                } else {
                    const float *sp = ws.score + (row0 + r) * Hq;
                    for (int h = j; h < Hq; h += RPL) sum += exp2f(sp[h] - Mh[h]) * Rh[h];
                }
            }
#pragma unroll
            for (int w = 1; w < RPL; w <<= 1) sum += __shfl_xor(sum, w);
            const int p = __shfl(pv[ps & 1], (tid & 63) - j + ps / 2);
            if (valid && j == 0) {
                mass[(size_t)b * c.n_cap + p] = sum;
                if (importance) {
                    float *ip = importance + (size_t)b * c.n_cap + p;
                    *ip = fmaf(decay, *ip, sum);
                }
            }
        }
    }
    // (4) output rows of the heads this workgroup owns: 32 channel quads x
    //     8 split groups, merged in a fixed order
    for (int h = split; h < Hq; h += X) {
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

// Workgroups of attn_split<G> that fit on the device at once (cached).
int persistent_grid(int G, const void *kernel) {
    static int cache[64][KVQ_MAX_GQA + 1];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int &v = cache[dev][G];
    if (v == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, WAVES * 64, 0) != hipSuccess) return 0;
        v = cus * (per_cu > 0 ? per_cu : 1);
    }
    return v;
}

bool launch_decode(const kvq_cache &c, const void *q, float *out, float *mass, float *importance,
                   float decay, float sm_scale, void *ws_ptr, hipStream_t s) {
    DecodeWs ws(ws_ptr, c);
    const int S = n_splits(c);
    const int G = c.Hq / c.Hkv;
    const uint16_t *qq = static_cast<const uint16_t *>(q);
    const float scale2 = sm_scale * LOG2E;
    switch (G) {
#define KVQ_G(g)                                                                                   \
    case g: {                                                                                      \
        const int grid = persistent_grid(g, reinterpret_cast<const void *>(attn_split<g>));         \
        if (grid <= 0) return false;                                                               \
        hipLaunchKernelGGL(attn_split<g>, dim3(grid), dim3(WAVES * 64), 0, s, c, qq, mass, ws, scale2, S); \
        break;                                                                                     \
    }
        KVQ_G(1) KVQ_G(2) KVQ_G(3) KVQ_G(4) KVQ_G(5) KVQ_G(6) KVQ_G(7) KVQ_G(8)
        KVQ_G(9) KVQ_G(10) KVQ_G(11) KVQ_G(12) KVQ_G(13) KVQ_G(14) KVQ_G(15) KVQ_G(16)
#undef KVQ_G
        default: return false;
    }
    // lanes per score row: enough float4s to cover Hq heads (8 when Hq is
    // not a multiple of four: that case reads rows head by head)
    int rpl = 8;
    if ((c.Hq & 3) == 0)
        while (rpl < 64 && 4 * rpl < c.Hq) rpl *= 2;
    switch (rpl) {
#define KVQ_FIN(r)                                                                                 \
    case r:                                                                                        \
        hipLaunchKernelGGL(attn_finalize<r>, dim3(S > c.Hq ? S : c.Hq, c.B), dim3(FT), 0, s, \
                           c, out, mass, importance, decay, ws, S);                                \
        break;
        KVQ_FIN(8)
        KVQ_FIN(16)
        KVQ_FIN(32)
        KVQ_FIN(64)
#undef KVQ_FIN
    }
    return hipGetLastError() == hipSuccess;
}

}  // namespace kvq
