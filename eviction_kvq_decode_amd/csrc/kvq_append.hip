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
// One launch, one workgroup per sequence: it finds the slot or decides on a
// pop, then quantises K and V for every kv head, packs the codes into the
// cache layout and updates the block metadata.  Pops are served in batch
// order (kvq_sync.h): each workgroup publishes its pops per pool, and a
// workgroup that pops sums the pops of the sequences before it for its rank;
// the last workgroup also sums all of them and lowers the free-stack tops.
#include <limits.h>

#include <mutex>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_sync.h"

namespace kvq {

namespace {

constexpr int PLAN_THREADS = 512;
constexpr int PLAN_UNROLL = 4;

// The plan of sequence b: -2 nothing to do (tag none, or the sequence cannot
// be served: status set), -1 reuse (entry, slot; m the entry's mask), p >= 0
// pop a block of pool p.  nb and len: the sequence's table length and
// seq_len, read once here for the metadata update.  The workgroup scans the
// table in rounds; each thread issues PLAN_UNROLL independent loads per
// round (unconditional, from clamped indices, so that they go out as one
// batch and the dependent table -> mask chain overlaps), and the first
// entry of the tag with a free slot wins.
struct Plan {
    int need;
    uint32_t entry;
    int slot;
    uint32_t m;
    int nb, len;
};
__device__ inline Plan plan_slot(const kvq_cache &c, int b, int tag, int *first, Plan *sh_plan) {
    const int tid = threadIdx.x;
    const int len = c.seq_len[b], nb = c.n_blocks[b];
    if (tag == TAG_NONE || tag > 2 || len >= c.n_cap) {
        if (tid == 0 && tag != TAG_NONE) *c.status = tag > 2 ? KVQ_EINVAL : KVQ_ENOSPC;
        return Plan{-2, 0u, 0, 0u, nb, len};
    }
    if (tid == 0) *first = INT_MAX;
    __syncthreads();
    const uint32_t *row = c.table + (size_t)b * c.max_blocks;
    for (int base = 0; base < nb; base += PLAN_THREADS * PLAN_UNROLL) {
        uint32_t ent[PLAN_UNROLL];
        uint32_t m[PLAN_UNROLL];
#pragma unroll
        for (int u = 0; u < PLAN_UNROLL; ++u) ent[u] = row[min(base + u * PLAN_THREADS + tid, nb - 1)];
#pragma unroll
        for (int u = 0; u < PLAN_UNROLL; ++u) m[u] = pool_sel(c.mask, ent[u] >> 30)[ent[u] & 0x3fffffffu];
        int mine = INT_MAX;
#pragma unroll
        for (int u = 0; u < PLAN_UNROLL; ++u) {
            const int e = base + u * PLAN_THREADS + tid;
            if (e < nb && (int)(ent[u] >> 30) == tag && m[u] != 0xffffu) mine = min(mine, e);
        }
        if (mine != INT_MAX) atomicMin(first, mine);
        __syncthreads();
        const int f = *first;   // the same in every thread
        if (f != INT_MAX) {
            // the thread holding the first free entry passes it on
#pragma unroll
            for (int u = 0; u < PLAN_UNROLL; ++u)
                if (base + u * PLAN_THREADS + tid == f)
                    *sh_plan = Plan{-1, ent[u], __builtin_ctz(~m[u]), m[u], nb, len};
            __syncthreads();
            return *sh_plan;
        }
        // every thread has read `first` before any thread of the next round
        // may lower it (f is uniform, so the barrier is too)
        __syncthreads();
    }
    if (nb >= c.max_blocks) {
        if (tid == 0) *c.status = KVQ_ENOSPC;
        return Plan{-2, 0u, 0, 0u, nb, len};
    }
    return Plan{tag, 0u, 0, 0u, nb, len};
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

// LDS written by some lanes of a wave is visible to the others after this
__device__ inline void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Quantise and pack one kv head's K and V rows of the token into slot `slot`
// of region `reg` (one wave; lane l holds channels 2l, 2l+1 of each row).
// kcode / vcode: the wave's own 128-byte LDS buffers.
__device__ inline void write_head(const kvq_cache &c, uint8_t *reg, int pool, int slot, uint32_t k_two,
                                  uint32_t v_two, uint8_t *kcode, uint8_t *vcode) {
    const int lane = threadIdx.x & 63;
    const int bits = pool_bits(pool);
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
    // the wave's code bytes are in LDS before any lane packs them
    wave_sync();

    // K row: 4*bits dwords, LSB-first.
    const int per = 32 / bits;  // codes per dword
    if (lane < 4 * bits) {
        uint32_t w = 0;
        for (int i = 0; i < per; ++i) w |= (uint32_t)kcode[lane * per + i] << (i * bits);
        reinterpret_cast<uint32_t *>(reg + slot * 16 * bits)[lane] = w;
    }
    // V: the 16*bits dwords holding this token's codes, whose other bits
    // are other tokens' codes: the token's fields are cleared and set with
    // two atomics per dword (in that order: same lane, same address), which
    // need no read back.
    uint8_t *vbase = reg + 256 * bits;
    const int tiles_per_dword = 8 / bits;
    for (int qd = lane; qd < 16 * bits; qd += 64) {
        const int j = qd & 15, w = qd >> 4;
        const int d_first = 16 * (w * tiles_per_dword) + j;
        uint32_t *dw = reinterpret_cast<uint32_t *>(vbase + v_dword_byte(bits, slot, d_first));
        const uint32_t lvmask = (1u << bits) - 1;
        uint32_t clr = 0, set = 0;
        for (int m = 0; m < tiles_per_dword; ++m) {
            const int d = 16 * (w * tiles_per_dword + m) + j;
            const int sh = v_code_slot(bits, slot, d) * bits;
            clr |= lvmask << sh;
            set |= (uint32_t)vcode[d] << sh;
        }
        __hip_atomic_fetch_and(dw, ~clr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_or(dw, set, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the buffers are reused by the wave's next head
    wave_sync();
}

// One workgroup per sequence: plan the slot, take a block id if the plan
// pops (ranked in batch order over the sequences' published pops), then
// quantise and write the token for every kv head (wave w takes heads w,
// w + 8, ...) and update the block metadata.
__global__ __launch_bounds__(PLAN_THREADS) void append_token(kvq_cache c, const uint16_t *k_new,
                                                             const uint16_t *v_new, const uint8_t *tags,
                                                             AppendWs sync) {
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int NWAVE = PLAN_THREADS / 64;
    __shared__ int first;
    __shared__ Plan sh_plan;
    __shared__ int s_id;
    __shared__ uint8_t kcode[NWAVE][HD], vcode[NWAVE][HD];
    // this lane's two channels of the first head's new K and V rows, loaded
    // first so that the loads overlap the plan
    const int h0 = wave;
    uint32_t k_two = 0, v_two = 0;
    if (h0 < c.Hkv) {
        const size_t row_off = ((size_t)b * c.Hkv + h0) * HD;
        k_two = reinterpret_cast<const uint32_t *>(k_new + row_off)[lane];
        v_two = reinterpret_cast<const uint32_t *>(v_new + row_off)[lane];
    }
    // wave 0 publishes and ranks: it reads the call's epoch and the
    // free-stack tops before this sequence's pops go out (only the last
    // workgroup moves the tops and the epoch, once every sequence's are in)
    uint32_t epoch = 0;
    int tops[3] = {0, 0, 0};
    if (wave == 0) {
        epoch = sync_epoch(sync);
        for (int p = 0; p < 3; ++p) tops[p] = c.free_top[p];
    }
    const Plan pl = plan_slot(c, b, tags[b], &first, &sh_plan);
    if (tid < 3) {
        wait_loads_done();
        sync_publish(sync, c.B, b, tid, epoch, pl.need == tid ? 1u : 0u);
    }
    const bool last = b == c.B - 1;
    if (pl.need >= 0 || last) {
        if (wave == 0) {
            int cnt[3];
            const bool ok = sync_counts_before(sync, c.B, b, epoch, last ? 7u : 1u << pl.need, cnt);
            if (lane == 0) {
                if (!ok) *c.status = KVQ_EHIP;
                if (last) {
                    for (int p = 0; p < 3; ++p) {
                        const int tot = cnt[p] + (pl.need == p ? 1 : 0);
                        c.free_top[p] = tops[p] - min(tot, tops[p]);
                    }
                    sync_close(sync, epoch);
                }
                int id = -1;
                if (pl.need >= 0) {
                    const int top = tops[pl.need], rank = cnt[pl.need];
                    if (rank >= top) *c.status = KVQ_ENOSPC;
                    else id = (int)pool_sel(c.free_ids, pl.need)[top - 1 - rank];
                }
                s_id = id;
            }
        }
        __syncthreads();
    }
    if (pl.need == -2) return;
    int pool, slot;
    uint32_t id;
    const bool fresh = pl.need >= 0;
    if (fresh) {
        if (s_id < 0) return;   // pool exhausted: the sequence is left unchanged
        pool = pl.need;
        id = (uint32_t)s_id;
        slot = 0;
    } else {
        pool = (int)(pl.entry >> 30);
        id = pl.entry & 0x3fffffffu;
        slot = pl.slot;
    }
    for (int h = h0; h < c.Hkv; h += NWAVE) {
        if (h != h0) {
            const size_t row_off = ((size_t)b * c.Hkv + h) * HD;
            k_two = reinterpret_cast<const uint32_t *>(k_new + row_off)[lane];
            v_two = reinterpret_cast<const uint32_t *>(v_new + row_off)[lane];
        }
        write_head(c, region_ptr(pool_sel(c.kv, pool), id, c.Hkv, h, pool), pool, slot, k_two, v_two, kcode[wave],
                   vcode[wave]);
    }
    if (tid == 0) {
        if (fresh) {
            c.table[(size_t)b * c.max_blocks + pl.nb] = ((uint32_t)pool << 30) | id;
            c.n_blocks[b] = pl.nb + 1;
            pool_sel(c.mask, pool)[id] = 1;
        } else {
            pool_sel(c.mask, pool)[id] = (uint16_t)(pl.m | (1u << slot));
        }
        pool_sel(c.pos, pool)[(size_t)id * BLK + slot] = pl.len;
        c.seq_len[b] = pl.len + 1;
    }
}

}  // namespace

// Scratch of the no-allocation append: the sync words (AppendWs) for up to
// APPEND_SCRATCH_BYTES, in a file-scope device array, zero when the code
// object loads, as the sync region must be before its first call.  Each GPU
// holds its own copy for the life of the process; its device address is
// looked up once per device (the array's name is only a host-side
// stand-in).  The words carry the epoch of the call that wrote them and the
// epoch itself lives in the array, so nothing needs clearing between calls
// (graph replays included); calls that overlap on one GPU share the array
// and race.
__device__ __align__(256) uint8_t scratch[APPEND_SCRATCH_BYTES];

void *append_scratch() {
    static std::mutex mu;
    static void *ptr[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        ptr[dev] = p;
    }
    return ptr[dev];
}

bool launch_append(const kvq_cache &c, const void *k_new, const void *v_new, const uint8_t *tags,
                   void *ws_ptr, hipStream_t s) {
    AppendWs ws(ws_ptr, c);
    hipLaunchKernelGGL(append_token, dim3(c.B), dim3(PLAN_THREADS), 0, s, c, static_cast<const uint16_t *>(k_new),
                       static_cast<const uint16_t *>(v_new), tags, ws);
    return hipGetLastError() == hipSuccess;
}

}  // namespace kvq
