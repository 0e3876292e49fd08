// kvq_evict.hip -- windowed top-k eviction with metadata-only compaction.
//
// "Dynamic Thinking-Token Selection ...", section 2.3: tokens of the
// question window are never evicted, the local window of recent tokens is
// kept, and inside the selection window the top-k by importance survive.
// "ThinKV", Continuous Thinking: eviction only clears mask bits -- the KV
// bytes never move; blocks that become empty leave the table and go back to
// their pool's free list for in-place reuse.
//
// evict_select: one 1024-thread workgroup per sequence, one thread per slot
//   in each pass.  Candidate keys (order-preserving importance bits, then
//   inverted position, so ties go to the lower position) are radix-selected
//   for the k-th largest; losers' mask bits are cleared; the table row is
//   compacted in order with a ballot prefix scan; freed entries are listed
//   in table order.
// evict_push: one workgroup per sequence pushes its freed ids at offsets
//   ranked across sequences in batch order.
#include <limits.h>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {

namespace {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int SEL_UNROLL = 16;  // slots a thread takes per batch
constexpr int RADIX_BITS = 11;  // digit width of the radix select
constexpr int RADIX = 1 << RADIX_BITS;

__device__ inline uint32_t order_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if (f == 0.0f) u = 0u;  // -0 counts as +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline uint64_t sel_key(float imp, int pos) {
    return ((uint64_t)order_bits(imp) << 32) | (uint64_t)(0xffffffffu - (uint32_t)pos);
}

// Exclusive prefix count of `flag` over the workgroup (thread order) and the
// total.  Uses per-wave ballots; all threads must call it.
__device__ inline int block_prefix(bool flag, int *wave_tot, int &total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const uint64_t bal = __ballot(flag);
    const int in_wave = __popcll(bal & ((1ull << lane) - 1));
    if (lane == 0) wave_tot[wv] = __popcll(bal);
    __syncthreads();
    int before = 0;
    total = 0;
    for (int w = 0; w < SEL_WAVES; ++w) {
        const int v = wave_tot[w];
        before += w < wv ? v : 0;
        total += v;
    }
    __syncthreads();
    return before + in_wave;
}

__global__ __launch_bounds__(SEL_THREADS) void evict_select(kvq_cache c, const float *importance,
                                                            const int32_t *keep_k, int q_window,
                                                            int recent_window, EvictWs ws) {
    const int b = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    if (b == 0 && tid < 3) ws.top[tid] = c.free_top[tid];
    const int nb = c.n_blocks[b];
    const int nslot = nb * BLK;
    const int lo = q_window, hi = c.seq_len[b] - recent_window;
    uint32_t *row = c.table + (size_t)b * c.max_blocks;
    const float *imp = importance + (size_t)b * c.n_cap;
    uint64_t *key = ws.cand + (size_t)b * c.max_blocks * BLK;

    __shared__ uint32_t hist[RADIX];
    __shared__ int s_digit, s_cum, s_ncand;
    __shared__ int wave_tot[SEL_WAVES];
    __shared__ int pool_cnt[4];
    if (tid == 0) s_ncand = 0;
    if (tid < 4) pool_cnt[tid] = 0;
    __syncthreads();

    // 1. one word per slot, thread per slot (slot s of entry e at 16 e + s):
    //    0 for a cleared slot, 1 for a valid slot in a window, else the
    //    candidate's key (a finite importance gives a key >= 2^55).
    //    SEL_UNROLL slots per thread and batch; the entry, then its mask and
    //    positions, then the importance, each level's loads issued together.
    int my_cand = 0;
    for (int i0 = 0; i0 < nslot; i0 += SEL_THREADS * SEL_UNROLL) {
        uint32_t ent[SEL_UNROLL], m[SEL_UNROLL];
        int p[SEL_UNROLL];
#pragma unroll
        for (int u = 0; u < SEL_UNROLL; ++u) {
            const int i = i0 + u * SEL_THREADS + tid;
            ent[u] = i < nslot ? row[i >> 4] : 0u;
        }
#pragma unroll
        for (int u = 0; u < SEL_UNROLL; ++u) {
            const int i = i0 + u * SEL_THREADS + tid;
            m[u] = i < nslot ? c.mask[ent[u] >> 30][ent[u] & 0x3fffffffu] : 0u;
            p[u] = i < nslot ? c.pos[ent[u] >> 30][(size_t)(ent[u] & 0x3fffffffu) * BLK + (i & 15)] : -1;
        }
#pragma unroll
        for (int u = 0; u < SEL_UNROLL; ++u) {
            const int i = i0 + u * SEL_THREADS + tid;
            uint64_t kk = 0;
            if ((m[u] >> (i & 15)) & 1u) {
                kk = 1;
                if (p[u] >= lo && p[u] < hi) {
                    kk = sel_key(imp[p[u]], p[u]);
                    ++my_cand;
                }
            }
            if (i < nslot) key[i] = kk;
        }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) my_cand += __shfl_xor(my_cand, off);
    if (lane == 0) atomicAdd(&s_ncand, my_cand);
    __syncthreads();
    const int n = s_ncand;
    const int k = max(keep_k[b], 0);
    const bool evicting = n > k;

    // 2. radix-select the k-th largest key, RADIX_BITS at a time from the
    //    top (the last digit is narrower), stopping as soon as the boundary
    //    digit's whole bin is kept.  Wide digits spread the keys, whose top
    //    bits (sign and exponent of the importance) take few values, over
    //    many bins: fewer passes and fewer same-bin atomics.
    uint64_t thr = 0;
    int thr_shift = 0;
    if (evicting && k > 0) {
        uint64_t prefix = 0;
        uint32_t need = (uint32_t)k;
        for (int top = 64;;) {
            const int width = top < RADIX_BITS ? top : RADIX_BITS;
            const int shift = top - width;
            const uint32_t dmask = (1u << width) - 1u;
            for (int i = tid; i < RADIX; i += SEL_THREADS) hist[i] = 0;
            __syncthreads();
            const uint64_t hmask = top == 64 ? 0ull : (~0ull << top);
            for (int i0 = 0; i0 < nslot; i0 += SEL_THREADS * SEL_UNROLL) {
                uint64_t kk[SEL_UNROLL];
#pragma unroll
                for (int u = 0; u < SEL_UNROLL; ++u) {
                    const int i = i0 + u * SEL_THREADS + tid;
                    kk[u] = i < nslot ? key[i] : 0ull;
                }
#pragma unroll
                for (int u = 0; u < SEL_UNROLL; ++u)
                    if (kk[u] > 1 && (kk[u] & hmask) == (prefix & hmask))
                        atomicAdd(&hist[(uint32_t)(kk[u] >> shift) & dmask], 1u);
            }
            __syncthreads();
            if (wv == 0) {
                // bins from the top: lane l holds RADIX-1 - BPL l - j, j < BPL
                constexpr int BPL = RADIX / 64;
                uint32_t sum = 0;
                for (int j = 0; j < BPL; ++j) sum += hist[RADIX - 1 - BPL * lane - j];
                uint32_t incl = sum;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const uint32_t y = __shfl_up(incl, off);
                    if (lane >= off) incl += y;
                }
                const uint32_t excl = incl - sum;
                // the boundary lane: its bins reach need, the bins above do not
                if (excl < need && incl >= need) {
                    uint32_t cum = excl;
                    int j = 0;
                    for (; j < BPL - 1; ++j) {
                        const uint32_t h = hist[RADIX - 1 - BPL * lane - j];
                        if (cum + h >= need) break;
                        cum += h;
                    }
                    s_digit = RADIX - 1 - BPL * lane - j;
                    s_cum = (int)cum;
                }
            }
            __syncthreads();
            const int dgt = s_digit;
            need -= (uint32_t)s_cum;
            prefix |= (uint64_t)dgt << shift;
            const bool done = hist[dgt] == need || shift == 0;
            __syncthreads();
            if (done) {
                thr = prefix;
                thr_shift = shift;
                break;
            }
            top = shift;
        }
    }

    // 3a. clear losers, thread per slot: 16-lane ballots give each entry's
    //     old and new masks; the entry's first slot's lane stores the new
    //     mask if it changed, and parks it in that slot's word for the
    //     compaction
#pragma unroll 1
    for (int i0 = 0; i0 < nslot; i0 += SEL_THREADS * SEL_UNROLL) {
        uint32_t ent[SEL_UNROLL];
        uint64_t kk[SEL_UNROLL];
#pragma unroll
        for (int u = 0; u < SEL_UNROLL; ++u) {
            const int i = i0 + u * SEL_THREADS + tid;
            ent[u] = i < nslot ? row[i >> 4] : 0u;
            kk[u] = i < nslot ? key[i] : 0ull;
        }
#pragma unroll
        for (int u = 0; u < SEL_UNROLL; ++u) {
            const int i = i0 + u * SEL_THREADS + tid;
            bool bit = kk[u] != 0;
            if (evicting && kk[u] > 1 && !(k > 0 && (kk[u] >> thr_shift) >= (thr >> thr_shift))) bit = false;
            const uint32_t oldm = (uint32_t)(__ballot(kk[u] != 0) >> (lane & 48)) & 0xffffu;
            const uint32_t newm = (uint32_t)(__ballot(bit) >> (lane & 48)) & 0xffffu;
            if (i < nslot && (i & 15) == 0) {
                if (newm != oldm) c.mask[ent[u] >> 30][ent[u] & 0x3fffffffu] = (uint16_t)newm;
                key[i] = newm;
            }
        }
    }
    __syncthreads();

    // 3b. compact the table row in order, list freed entries (thread per entry)
    int kept_base = 0, freed_base = 0;
    uint32_t *freed = ws.freed + (size_t)b * c.max_blocks;
    for (int c0 = 0; c0 < nb; c0 += SEL_THREADS) {
        const int e = c0 + tid;
        const bool has = e < nb;
        uint32_t ent = 0, newm = 0;
        if (has) {
            ent = row[e];
            newm = (uint32_t)key[(size_t)e * BLK];
        }
        int nkept, nfreed;
        const int kr = block_prefix(has && newm != 0, wave_tot, nkept);
        const int fr = block_prefix(has && newm == 0, wave_tot, nfreed);
        if (has) {
            if (newm != 0) {
                row[kept_base + kr] = ent;
            } else {
                freed[freed_base + fr] = ent;
                atomicAdd(&pool_cnt[ent >> 30], 1);
            }
        }
        kept_base += nkept;
        freed_base += nfreed;
        __syncthreads();
    }
    if (tid == 0) c.n_blocks[b] = kept_base;
    if (tid < 4) ws.nfreed[b * 4 + tid] = tid < 3 ? pool_cnt[tid] : freed_base;
}

__global__ __launch_bounds__(256) void evict_push(kvq_cache c, EvictWs ws) {
    const int b = blockIdx.x, tid = threadIdx.x;
    __shared__ int base[3];
    __shared__ int wave_cnt[4][3];
    if (tid < 3) {
        int s = ws.top[tid];
        for (int bb = 0; bb < b; ++bb) s += ws.nfreed[bb * 4 + tid];
        base[tid] = s;
        if (b == 0) {
            int tot = ws.top[tid];
            for (int bb = 0; bb < c.B; ++bb) tot += ws.nfreed[bb * 4 + tid];
            c.free_top[tid] = tot;
        }
    }
    __syncthreads();
    const int nf = ws.nfreed[b * 4 + 3];
    const uint32_t *freed = ws.freed + (size_t)b * c.max_blocks;
    const int lane = tid & 63, wv = tid >> 6;
    for (int c0 = 0; c0 < nf; c0 += 256) {
        const int i = c0 + tid;
        const uint32_t ent = i < nf ? freed[i] : 0xffffffffu;
        const int pool = i < nf ? (int)(ent >> 30) : 3;
        int rank = 0;
        for (int p = 0; p < 3; ++p) {
            const uint64_t bal = __ballot(pool == p);
            if (lane == 0) wave_cnt[wv][p] = __popcll(bal);
            if (pool == p) rank = __popcll(bal & ((1ull << lane) - 1));
        }
        __syncthreads();
        if (pool < 3) {
            int before = 0;
            for (int w = 0; w < wv; ++w) before += wave_cnt[w][pool];
            c.free_ids[pool][base[pool] + before + rank] = ent & 0x3fffffffu;
        }
        __syncthreads();
        if (tid < 3) {
            int tot = 0;
            for (int w = 0; w < 4; ++w) tot += wave_cnt[w][tid];
            base[tid] += tot;
        }
        __syncthreads();
    }
}

}  // namespace

bool launch_evict(const kvq_cache &c, const float *importance, const int32_t *keep_k, int q_window,
                  int recent_window, void *ws_ptr, hipStream_t s) {
    EvictWs ws(ws_ptr, c);
    hipLaunchKernelGGL(evict_select, dim3(c.B), dim3(SEL_THREADS), 0, s, c, importance, keep_k,
                       q_window, recent_window, ws);
    hipLaunchKernelGGL(evict_push, dim3(c.B), dim3(256), 0, s, c, ws);
    return hipGetLastError() == hipSuccess;
}

}  // namespace kvq
