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
// evict_tbe_select: thought-adaptive eviction by segment (below).
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

// Clear the slots the rule drops and compact the table row (one workgroup
// per sequence).  key holds one word per slot (0: cleared); keep(word) says
// whether a valid slot survives.  Thread per slot: 16-lane ballots give each
// entry's old and new masks; the entry's first slot's lane stores the new
// mask if it changed, and parks it in that slot's word.  Then, thread per
// entry, the entries that kept a slot are packed in order and the emptied
// ones listed for the free-stack pushes.
template <class Keep>
__device__ inline void clear_and_compact(const kvq_cache &c, int b, uint64_t *key, int nslot, int nb,
                                         uint32_t *row, EvictWs &ws, int *wave_tot, int *pool_cnt,
                                         const Keep &keep) {
    const int tid = threadIdx.x, lane = tid & 63;
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
            const bool bit = keep(kk[u]);
            const uint32_t oldm = (uint32_t)(__ballot(kk[u] != 0) >> (lane & 48)) & 0xffffu;
            const uint32_t newm = (uint32_t)(__ballot(bit) >> (lane & 48)) & 0xffffu;
            if (i < nslot && (i & 15) == 0) {
                if (newm != oldm) c.mask[ent[u] >> 30][ent[u] & 0x3fffffffu] = (uint16_t)newm;
                key[i] = newm;
            }
        }
    }
    __syncthreads();

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

// One word per slot (slot s of entry e at 16 e + s), thread per slot:
// 0 for a cleared slot, 1 for a valid slot outside [lo, hi), else the
// candidate's key (a finite importance gives a key >= 2^55).  SEL_UNROLL
// slots per thread and batch; the entry, then its mask and positions, then
// the importance, each level's loads issued together.  pmap, if given,
// receives the slot of each candidate position.  Returns this thread's
// candidate count.
__device__ inline int slot_keys(const kvq_cache &c, const uint32_t *row, const float *imp, int nslot, int lo,
                                int hi, uint64_t *key, int32_t *pmap) {
    const int tid = threadIdx.x;
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
                    if (pmap) pmap[p[u]] = i;
                }
            }
            if (i < nslot) key[i] = kk;
        }
    }
    return my_cand;
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

    // 1. one word per slot: the candidate keys
    int my_cand = slot_keys(c, row, imp, nslot, lo, hi, key, nullptr);
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

    // 3. clear losers, compact the table row, list freed entries
    clear_and_compact(c, b, key, nslot, nb, row, ws, wave_tot, pool_cnt,
                      [&](uint64_t kk) {
                          return kk != 0 && !(evicting && kk > 1 && !(k > 0 && (kk >> thr_shift) >= (thr >> thr_shift)));
                      });
}

// evict_tbe_select: thought-adaptive eviction ("ThinKV", Methodology,
// think-before-evict), one 1024-thread workgroup per sequence.  The
// candidates (valid slots with q_window <= pos < seq_len - recent_window),
// taken in position order, form segments: maximal runs of one thought type.
// A segment followed by k Transition segments keeps everything if k == 0,
// else its best max(r_min, r0 >> (k - 1)) slots (Reasoning, Execution) or
// t_keep slots (Transition): larger importance, then lower position.
//   1. one word per slot (as evict_select) and a position -> slot map;
//   2. the candidates in position order (a ballot prefix over positions);
//   3. segment starts where the type changes (a ballot prefix);
//   4. each segment's retention from the count of later Transition segments;
//   5. each candidate's rank in its segment, counted until it reaches the
//      retention;
//   6. clear and compact as evict_select.
__global__ __launch_bounds__(SEL_THREADS) void evict_tbe_select(kvq_cache c, const float *importance, int r0,
                                                                int r_min, int t_keep, int q_window,
                                                                int recent_window, EvictWs ws) {
    const int b = blockIdx.x, tid = threadIdx.x;
    if (b == 0 && tid < 3) ws.top[tid] = c.free_top[tid];
    const int nb = c.n_blocks[b];
    const int nslot = nb * BLK;
    const int lo = q_window, hi = min(c.seq_len[b] - recent_window, c.n_cap);
    uint32_t *row = c.table + (size_t)b * c.max_blocks;
    const float *imp = importance + (size_t)b * c.n_cap;
    const size_t ms = (size_t)c.max_blocks * BLK;
    uint64_t *key = ws.cand + (size_t)b * ms;
    int32_t *pmap = ws.pmap + (size_t)b * c.n_cap;
    int32_t *ord = ws.ord + (size_t)b * ms;
    uint64_t *okey = ws.okey + (size_t)b * ms;
    int32_t *segof = ws.segof + (size_t)b * ms;
    int32_t *segstart = ws.segstart + (size_t)b * (ms + 1);
    int32_t *segret = ws.segret + (size_t)b * ms;

    __shared__ int wave_tot[SEL_WAVES];
    __shared__ int pool_cnt[4];
    if (tid < 4) pool_cnt[tid] = 0;
    for (int p = lo + tid; p < hi; p += SEL_THREADS) pmap[p] = -1;
    __syncthreads();

    // 1. slot words and the position map of the candidates
    slot_keys(c, row, imp, nslot, lo, hi, key, pmap);
    __syncthreads();

    // 2. candidates in position order, with their keys
    int n = 0;
    for (int p0 = lo; p0 < hi; p0 += SEL_THREADS) {
        const int p = p0 + tid;
        const int v = p < hi ? pmap[p] : -1;
        int tot;
        const int r = block_prefix(v >= 0, wave_tot, tot);
        if (v >= 0) {
            ord[n + r] = v;
            okey[n + r] = key[v];
        }
        n += tot;
    }
    __syncthreads();

    // 3. segments; segof[k] = segment of candidate k, segret[s] = its type
    int nseg = 0;
    for (int k0 = 0; k0 < n; k0 += SEL_THREADS) {
        const int k = k0 + tid;
        bool start = false;
        int pool = 0;
        if (k < n) {
            pool = (int)(row[ord[k] >> 4] >> 30);
            start = k == 0 || (int)(row[ord[k - 1] >> 4] >> 30) != pool;
        }
        int tot;
        const int r = block_prefix(start, wave_tot, tot);
        if (start) {
            segstart[nseg + r] = k;
            segret[nseg + r] = pool;
        }
        if (k < n) segof[k] = nseg + r + (start ? 1 : 0) - 1;
        nseg += tot;
    }
    if (tid == 0) segstart[nseg] = n;
    __syncthreads();

    // 4. retention: Transition segments after each segment
    int n_t = 0;
    for (int s0 = 0; s0 < nseg; s0 += SEL_THREADS) {
        const int sg = s0 + tid;
        int tot;
        block_prefix(sg < nseg && segret[sg] == 2, wave_tot, tot);
        n_t += tot;
    }
    int t_before = 0;
    for (int s0 = 0; s0 < nseg; s0 += SEL_THREADS) {
        const int sg = s0 + tid;
        const bool is_t = sg < nseg && segret[sg] == 2;
        int tot;
        const int r = block_prefix(is_t, wave_tot, tot);
        if (sg < nseg) {
            const int later = n_t - (t_before + r + (is_t ? 1 : 0));
            int keep = INT_MAX;
            if (later > 0) {
                if (is_t) {
                    keep = t_keep;
                } else {
                    const int sh = later - 1;
                    keep = max(sh >= 31 ? 0 : (r0 >> sh), r_min);
                }
                keep = max(keep, 0);
            }
            segret[sg] = keep;
        }
        t_before += tot;
    }
    __syncthreads();

    // 5. each candidate's verdict: fewer than `retention` better candidates
    //    in its segment (keys are unique: the position is part of them)
    for (int k0 = 0; k0 < n; k0 += SEL_THREADS) {
        const int k = k0 + tid;
        if (k < n) {
            const int sg = segof[k];
            const int a = segstart[sg], e = segstart[sg + 1];
            const int keep = segret[sg];
            bool kept = true;
            if (keep < e - a) {
                const uint64_t kk = okey[k];
                int better = 0;
                for (int j = a; j < e && better < keep; ++j) better += okey[j] > kk ? 1 : 0;
                kept = better < keep;
            }
            segof[k] = kept ? 1 : 0;
        }
    }
    __syncthreads();
    for (int k0 = 0; k0 < n; k0 += SEL_THREADS) {
        const int k = k0 + tid;
        if (k < n) key[ord[k]] = segof[k] ? 1ull : 2ull;
    }
    __syncthreads();

    // 6. clear the dropped candidates (word 2), compact the table row
    clear_and_compact(c, b, key, nslot, nb, row, ws, wave_tot, pool_cnt,
                      [](uint64_t kk) { return kk != 0 && kk != 2; });
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

bool launch_evict_tbe(const kvq_cache &c, const float *importance, int r0, int r_min, int t_keep,
                      int q_window, int recent_window, void *ws_ptr, hipStream_t s) {
    EvictWs ws(ws_ptr, c);
    hipLaunchKernelGGL(evict_tbe_select, dim3(c.B), dim3(SEL_THREADS), 0, s, c, importance, r0, r_min,
                       t_keep, q_window, recent_window, ws);
    hipLaunchKernelGGL(evict_push, dim3(c.B), dim3(256), 0, s, c, ws);
    return hipGetLastError() == hipSuccess;
}

}  // namespace kvq
