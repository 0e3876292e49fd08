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
constexpr int THREADS = 256;
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

template <int G, int BITS>
__device__ inline void attend_block(const kvq_cache &c, const uint8_t *pool_base, uint32_t id, int kh0,
                                    int np, uint32_t m16, int e, int b, const uint4 (*qop)[NGRP][64],
                                    const float *qsum, float scale2, const DecodeWs &ws, WaveState &st) {
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
    if (row_ok) {
        float *sp = ws.score + ((size_t)b * c.Hq + (size_t)kh0 * G + lo) * ((size_t)c.max_blocks * BLK) +
                    (size_t)e * BLK + 4 * hi;
        *reinterpret_cast<float4 *>(sp) = make_float4(s[0], s[1], s[2], s[3]);
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
    int idx[E];
    uint32_t msk[E];
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
        int n = 0;
        for (int base = 0; base < E; base += 64) {
            const int e = e0 + base + lane;
            uint32_t ent = 0, m = 0;
            if (base + lane < E && e < nb) {
                ent = c.table[(size_t)b * c.max_blocks + e];
                m = c.mask[ent >> 30][ent & 0x3fffffffu];
            }
            const uint64_t bal = __ballot(m != 0);
            const int at = n + __popcll(bal & ((1ull << lane) - 1));
            if (m != 0) {
                sh.ent[at] = ent;
                sh.idx[at] = e;
                sh.msk[at] = m;
            }
            n += __popcll(bal);
        }
        if (lane == 0) sh.n = n;
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
        const int eix = __builtin_amdgcn_readfirstlane(sh.idx[k]);
        const int pool = (int)(ent >> 30);
        const uint32_t id = ent & 0x3fffffffu;
        if (pool == 0)
            attend_block<G, 8>(c, c.kv[0], id, kh0, np, msk, eix, b, sh.q, qsum, scale2, ws, st);
        else if (pool == 1)
            attend_block<G, 4>(c, c.kv[1], id, kh0, np, msk, eix, b, sh.q, qsum, scale2, ws, st);
        else
            attend_block<G, 2>(c, c.kv[2], id, kh0, np, msk, eix, b, sh.q, qsum, scale2, ws, st);
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

__global__ __launch_bounds__(THREADS) void attn_finalize(kvq_cache c, float *out, float *mass,
                                                         float *importance, float decay, DecodeWs ws,
                                                         int S) {
    const int chunk = blockIdx.x, b = blockIdx.y, C = gridDim.x;
    const int tid = threadIdx.x;
    const int nb = c.n_blocks[b];
    const int s_act = (nb + E - 1) / E;
    const int Hq = c.Hq;
    __shared__ float Mh[MAX_HQ], Rh[MAX_HQ];
    __shared__ float pm[THREADS], pl[THREADS];
    __shared__ uint32_t s_ent[E], s_msk[E];

    // stage this chunk's table entries and masks
    const int e0 = chunk * E;
    for (int k = tid; k < E; k += THREADS) {
        uint32_t ent = 0, m = 0;
        if (e0 + k < nb) {
            ent = c.table[(size_t)b * c.max_blocks + e0 + k];
            m = c.mask[ent >> 30][ent & 0x3fffffffu];
        }
        s_ent[k] = ent;
        s_msk[k] = m;
    }
    // global max / sum per head: TPH threads per head, each over a stride of splits
    int tph = 1;
    while (tph * 2 * Hq <= THREADS) tph *= 2;
    for (int h0 = 0; h0 < Hq; h0 += THREADS / tph) {
        const int h = h0 + tid / tph, j = tid % tph;
        float M = -INFINITY, L = 0.f;
        if (h < Hq) {
            const float *ml = ws.ml + ((size_t)b * Hq + h) * S * 2;
            for (int s = j; s < s_act; s += tph) {
                const float m = ml[2 * s], l = ml[2 * s + 1];
                if (m == -INFINITY) continue;
                if (m > M) {
                    L = L * exp2f(M - m) + l;
                    M = m;
                } else {
                    L += l * exp2f(m - M);
                }
            }
        }
        pm[tid] = M;
        pl[tid] = L;
        __syncthreads();
        if (j == 0 && h < Hq) {
            float MM = -INFINITY;
            for (int k = 0; k < tph; ++k) MM = fmaxf(MM, pm[tid + k]);
            float LL = 0.f;
            for (int k = 0; k < tph; ++k)
                if (pm[tid + k] != -INFINITY) LL += pl[tid + k] * exp2f(pm[tid + k] - MM);
            Mh[h] = MM;
            Rh[h] = LL > 0.f ? 1.0f / LL : 0.f;
        }
        __syncthreads();
    }

    // output rows of the heads this chunk owns
    for (int h = chunk; h < Hq; h += C) {
        if (tid >= HD) break;
        const float *ml = ws.ml + ((size_t)b * Hq + h) * S * 2;
        const float *o = ws.o + ((size_t)b * Hq + h) * S * HD;
        float acc = 0.f;
        for (int s = 0; s < s_act; ++s) {
            const float m = ml[2 * s];
            if (m != -INFINITY) acc = fmaf(o[(size_t)s * HD + tid], exp2f(m - Mh[h]), acc);
        }
        out[((size_t)b * Hq + h) * HD + tid] = acc * Rh[h];
    }

    // mass (and importance) of the valid slots of this chunk's entries
    const size_t score_row = (size_t)c.max_blocks * BLK;
    const float *sbase = ws.score + (size_t)b * Hq * score_row;
#pragma unroll 1
    for (int i = tid; i < E * BLK; i += THREADS) {
        const int k = i / BLK, t = i % BLK;
        const uint32_t m = s_msk[k];
        if (!((m >> t) & 1)) continue;
        const uint32_t ent = s_ent[k];
        const int p = c.pos[ent >> 30][(size_t)(ent & 0x3fffffffu) * BLK + t];
        const float *sp = sbase + (size_t)(e0 + k) * BLK + t;
        float sum = 0.f;
#pragma unroll 8
        for (int h = 0; h < Hq; ++h) sum += exp2f(sp[h * score_row] - Mh[h]) * Rh[h];
        mass[(size_t)b * c.n_cap + p] = sum;
        if (importance) {
            float *ip = importance + (size_t)b * c.n_cap + p;
            *ip = fmaf(decay, *ip, sum);
        }
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
    hipLaunchKernelGGL(attn_finalize, dim3(S, c.B), dim3(THREADS), 0, s, c, out, mass, importance,
                       decay, ws, S);
    return hipGetLastError() == hipSuccess;
}

}  // namespace kvq
