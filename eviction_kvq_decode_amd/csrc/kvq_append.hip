// kvq_append.hip -- append one token per sequence into the typed, paged,
// quantised cache.
//
// "ThinKV", Methodology, Thought-Adaptive Quantization (TBQ): the token's
// thought type picks the precision (R 8 bit, E 4 bit, T 2 bit) and the
// values are group-quantised.  Same page, System Implementation (Continuous
// Thinking): a new token of a type overwrites an evicted slot of a block of
// that type in place; only when none is free does a block come from the
// type's free list.
//
// Two launches: append_plan (one workgroup per sequence) finds the slot or
// decides on a pop; append_write (one wave per (sequence, kv head))
// quantises K and V, packs the codes into the cache layout and updates the
// block metadata.  Pops are ranked across sequences in batch order from a
// copy of the free-stack tops taken by the plan, so no cross-workgroup
// synchronisation is needed.
#include <limits.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

constexpr int PLAN_THREADS = 256;
constexpr int PLAN_UNROLL = 4;

__global__ __launch_bounds__(PLAN_THREADS) void append_plan(kvq_cache c, const uint8_t *tags,
                                                            AppendWs ws) {
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    if (b == 0 && tid < 3) ws.top[tid] = c.free_top[tid];
    const int tag = tags[b];
    if (tag == TAG_NONE || tag > 2 || c.seq_len[b] >= c.n_cap) {
        if (tid == 0) {
            ws.need[b] = -2;
            if (tag != TAG_NONE) *c.status = tag > 2 ? KVQ_EINVAL : KVQ_ENOSPC;
        }
        return;
    }
    __shared__ int first;
    if (tid == 0) first = INT_MAX;
    __syncthreads();
    const int nb = c.n_blocks[b];
    const uint32_t *row = c.table + (size_t)b * c.max_blocks;
    const uint16_t *mask = c.mask[tag];
    // Scan the table in rounds; each thread issues PLAN_UNROLL independent
    // loads per round so the dependent table -> mask chain overlaps.  The
    // thread holding the first entry with a free slot writes the plan from
    // its registers.
    for (int base = 0; base < nb; base += PLAN_THREADS * PLAN_UNROLL) {
        uint32_t ent[PLAN_UNROLL];
        uint32_t m[PLAN_UNROLL];
#pragma unroll
        for (int u = 0; u < PLAN_UNROLL; ++u) {
            const int e = base + u * PLAN_THREADS + tid;
            ent[u] = e < nb ? row[e] : 0xffffffffu;
        }
        int mine = INT_MAX;
#pragma unroll
        for (int u = 0; u < PLAN_UNROLL; ++u) {
            const int e = base + u * PLAN_THREADS + tid;
            m[u] = 0xffffu;
            if (e < nb && (int)(ent[u] >> 30) == tag) {
                m[u] = mask[ent[u] & 0x3fffffffu];
                if (m[u] != 0xffffu) mine = min(mine, e);
            }
        }
        if (mine != INT_MAX) atomicMin(&first, mine);
        __syncthreads();
        const int f = first;   // the same in every thread
        if (f != INT_MAX) {
#pragma unroll
            for (int u = 0; u < PLAN_UNROLL; ++u)
                if (base + u * PLAN_THREADS + tid == f) {
                    ws.need[b] = -1;
                    ws.entry[b] = (int32_t)ent[u];
                    ws.slot[b] = __builtin_ctz(~m[u]);
                }
            return;
        }
    }
    if (tid == 0) {
        if (nb >= c.max_blocks) {
            ws.need[b] = -2;
            *c.status = KVQ_ENOSPC;
        } else {
            ws.need[b] = tag;
        }
    }
}

// Group-quantise one 128-channel fp16 row held two channels per lane
// (lane l owns channels 2l, 2l+1; 16 lanes per 32-channel group).
// Matches the TBQ reading: zero = min, scale = least fp16 >= (max-min)/lv,
// code = clamp(rint((x - zero)/scale)), all in fp32.
__device__ inline void quantise_pair(uint32_t two, int bits, uint32_t &c0, uint32_t &c1,
                                     uint32_t &scale_zero) {
    const float x0 = h2f((uint16_t)(two & 0xffff)), x1 = h2f((uint16_t)(two >> 16));
    float mn = fminf(x0, x1), mx = fmaxf(x0, x1);
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, off));
        mx = fmaxf(mx, __shfl_xor(mx, off));
    }
    if (mn == 0.0f) mn = fabsf(mn);  // -0 counts as +0
    if (mx == 0.0f) mx = fabsf(mx);
    const float lv = (float)((1 << bits) - 1);
    const float s32 = (mx - mn) / lv;
    uint16_t sh = f2h_rn(s32);
    if (h2f(sh) < s32) sh = (uint16_t)(sh + 1);
    const float sc = h2f(sh);
    if (sc == 0.0f) {
        c0 = c1 = 0;
    } else {
        float t0 = rintf((x0 - mn) / sc), t1 = rintf((x1 - mn) / sc);
        c0 = (uint32_t)fminf(fmaxf(t0, 0.0f), lv);
        c1 = (uint32_t)fminf(fmaxf(t1, 0.0f), lv);
    }
    scale_zero = (uint32_t)sh | ((uint32_t)f2h_rn(mn) << 16);
}

// Nearest code of y in a sign-magnitude minifloat with E exponent bits, M
// mantissa bits and the given bias (subnormals at exponent field 0, no
// infinities), ties to the even code, magnitudes saturating at max_mag;
// the sign bit only for a nonzero magnitude of a negative y.  Normal range:
// the fp32 mantissa rounded to M bits on its bit pattern (a carry moves into
// the exponent); below it, the subnormal grid by an exact power-of-two
// scaling and rintf.
template <int E, int M, int BIAS>
__device__ inline uint32_t minifloat_code(float y, uint32_t max_mag) {
    const float a = fabsf(y);
    constexpr float least_normal = BIAS == 7 ? 0.015625f : 1.0f;  // 2^(1 - BIAS)
    constexpr float to_steps = BIAS == 7 ? 512.0f : 2.0f;         // 2^(BIAS - 1 + M)
    uint32_t mag;
    if (a < least_normal) {
        mag = (uint32_t)rintf(a * to_steps);
    } else {
        constexpr int drop = 23 - M;
        uint32_t u = __float_as_uint(a);
        u += (1u << (drop - 1)) - 1u + ((u >> drop) & 1u);
        const int eb = (int)(u >> 23) - 127 + BIAS;
        mag = eb > (1 << E) - 1 ? max_mag : ((uint32_t)eb << M) | ((u >> drop) & ((1u << M) - 1u));
    }
    mag = min(mag, max_mag);
    return (y < 0.0f && mag != 0u ? 1u << (E + M) : 0u) | mag;
}

// ThinKV's own formats ("ThinKV", Methodology, TBQ), same row layout:
// symmetric groups of 32 with scale = least fp16 >= max|x| / top (top 448,
// 6, 1); pool 0 stores E4M3 codes of x / scale, pool 1 E2M1 codes, both
// with zero 0; pool 2 stores t + 1 for t = rint(x / scale) in [-1, 1] with
// zero = -scale (so the integer decode gives -scale, 0, +scale).  A group
// of zeros stores scale 0, zero 0 and the code of 0.
__device__ inline void quantise_pair_native(uint32_t two, int pool, uint32_t &c0, uint32_t &c1,
                                            uint32_t &scale_zero) {
    const float x0 = h2f((uint16_t)(two & 0xffff)), x1 = h2f((uint16_t)(two >> 16));
    float amax = fmaxf(fabsf(x0), fabsf(x1));
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    const float top = pool == 0 ? 448.0f : pool == 1 ? 6.0f : 1.0f;
    const float s32 = amax / top;
    uint16_t sh = f2h_rn(s32);
    if (h2f(sh) < s32) sh = (uint16_t)(sh + 1);
    const float sc = h2f(sh);
    const uint16_t zh = pool == 2 && sh != 0 ? (uint16_t)(sh | 0x8000u) : (uint16_t)0;
    if (sc == 0.0f) {
        c0 = c1 = pool == 2 ? 1u : 0u;
    } else {
        const float y0 = x0 / sc, y1 = x1 / sc;
        if (pool == 0) {
            c0 = minifloat_code<4, 3, 7>(y0, 0x7eu);
            c1 = minifloat_code<4, 3, 7>(y1, 0x7eu);
        } else if (pool == 1) {
            c0 = minifloat_code<2, 1, 1>(y0, 0x7u);
            c1 = minifloat_code<2, 1, 1>(y1, 0x7u);
        } else {
            c0 = (uint32_t)(fminf(fmaxf(rintf(y0), -1.0f), 1.0f) + 1.0f);
            c1 = (uint32_t)(fminf(fmaxf(rintf(y1), -1.0f), 1.0f) + 1.0f);
        }
    }
    scale_zero = (uint32_t)sh | ((uint32_t)zh << 16);
}

__global__ __launch_bounds__(64) void append_write(kvq_cache c, const uint16_t *k_new,
                                                   const uint16_t *v_new, AppendWs ws) {
    const int b = blockIdx.x / c.Hkv, h = blockIdx.x % c.Hkv;
    const int lane = threadIdx.x;
    // this lane's two channels of the new K and V rows, loaded before the
    // plan so that the loads overlap the dependent plan/table reads
    const size_t row_off = ((size_t)b * c.Hkv + h) * HD;
    const uint32_t k_two = reinterpret_cast<const uint32_t *>(k_new + row_off)[lane];
    const uint32_t v_two = reinterpret_cast<const uint32_t *>(v_new + row_off)[lane];
    if (blockIdx.x == 0 && lane < 3) {
        int cnt = 0;
        for (int bb = 0; bb < c.B; ++bb) cnt += ws.need[bb] == lane;
        c.free_top[lane] = ws.top[lane] - min(cnt, ws.top[lane]);
    }
    const int need = ws.need[b];
    if (need == -2) return;
    int pool, slot;
    uint32_t id;
    bool fresh = false;
    if (need == -1) {
        const uint32_t ent = (uint32_t)ws.entry[b];
        pool = (int)(ent >> 30);
        id = ent & 0x3fffffffu;
        slot = ws.slot[b];
    } else {
        pool = need;
        int rank = 0;
        for (int bb = lane; bb < b; bb += 64) rank += ws.need[bb] == pool;
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) rank += __shfl_xor(rank, off);
        const int top = ws.top[pool];
        if (rank >= top) {
            if (h == 0 && lane == 0) *c.status = KVQ_ENOSPC;
            return;
        }
        id = c.free_ids[pool][top - 1 - rank];
        slot = 0;
        fresh = true;
    }
    const int bits = pool_bits(pool);
    uint8_t *reg = region_ptr(c.kv[pool], id, c.Hkv, h, pool);

    __shared__ uint8_t kcode[HD];  // by K-row code index
    __shared__ uint8_t vcode[HD];  // by channel
    uint32_t k0, k1, ksz, v0, v1, vsz;
    if (c.codec == KVQ_CODEC_NATIVE) {
        quantise_pair_native(k_two, pool, k0, k1, ksz);
        quantise_pair_native(v_two, pool, v0, v1, vsz);
    } else {
        quantise_pair(k_two, bits, k0, k1, ksz);
        quantise_pair(v_two, bits, v0, v1, vsz);
    }
    kcode[k_row_index(bits, 2 * lane)] = (uint8_t)k0;
    kcode[k_row_index(bits, 2 * lane + 1)] = (uint8_t)k1;
    vcode[2 * lane] = (uint8_t)v0;
    vcode[2 * lane + 1] = (uint8_t)v1;
    if ((lane & 15) == 0) {
        const int g = lane >> 4;
        reinterpret_cast<uint32_t *>(reg + 512 * bits)[slot * NGRP + g] = ksz;
        reinterpret_cast<uint32_t *>(reg + 512 * bits + 256)[slot * NGRP + g] = vsz;
    }
    __syncthreads();

    // K row: 4*bits dwords, LSB-first.
    const int per = 32 / bits;  // codes per dword
    if (lane < 4 * bits) {
        uint32_t w = 0;
        for (int i = 0; i < per; ++i) w |= (uint32_t)kcode[lane * per + i] << (i * bits);
        reinterpret_cast<uint32_t *>(reg + slot * 16 * bits)[lane] = w;
    }
    // V: the 16*bits dwords holding this token's codes; read-modify-write,
    // other tokens' codes in the same dwords are preserved.
    uint8_t *vbase = reg + 256 * bits;
    const int tiles_per_dword = 8 / bits;
    for (int qd = lane; qd < 16 * bits; qd += 64) {
        const int j = qd & 15, w = qd >> 4;
        const int d_first = 16 * (w * tiles_per_dword) + j;
        uint32_t *dw = reinterpret_cast<uint32_t *>(vbase + v_dword_byte(bits, slot, d_first));
        uint32_t val = *dw;
        const uint32_t lvmask = (1u << bits) - 1;
        for (int m = 0; m < tiles_per_dword; ++m) {
            const int d = 16 * (w * tiles_per_dword + m) + j;
            const int sh = v_code_slot(bits, slot, d) * bits;
            val = (val & ~(lvmask << sh)) | ((uint32_t)vcode[d] << sh);
        }
        *dw = val;
    }

    if (h == 0 && lane == 0) {
        if (fresh) {
            const int nb = c.n_blocks[b];
            c.table[(size_t)b * c.max_blocks + nb] = ((uint32_t)pool << 30) | id;
            c.n_blocks[b] = nb + 1;
            c.mask[pool][id] = 1;
        } else {
            c.mask[pool][id] = (uint16_t)(c.mask[pool][id] | (1u << slot));
        }
        const int p = c.seq_len[b];
        c.pos[pool][(size_t)id * BLK + slot] = p;
        c.seq_len[b] = p + 1;
    }
}

}  // namespace

bool launch_append(const kvq_cache &c, const void *k_new, const void *v_new, const uint8_t *tags,
                   void *ws_ptr, hipStream_t s) {
    AppendWs ws(ws_ptr, c);
    hipLaunchKernelGGL(append_plan, dim3(c.B), dim3(PLAN_THREADS), 0, s, c, tags, ws);
    hipLaunchKernelGGL(append_write, dim3(c.B * c.Hkv), dim3(64), 0, s, c,
                       static_cast<const uint16_t *>(k_new), static_cast<const uint16_t *>(v_new), ws);
    return hipGetLastError() == hipSuccess;
}

}  // namespace kvq
