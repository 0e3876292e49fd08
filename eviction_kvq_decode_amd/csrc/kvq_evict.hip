// kvq_evict.hip -- eviction with metadata-only compaction, three policies:
// windowed top-k, thought-adaptive eviction by segment, and thought-aware
// segment budgets.
//
// "Dynamic Thinking-Token Selection ...", section 2.3: tokens of the
// question window are never evicted, the local window of recent tokens is
// kept, and inside the selection window the top-k by importance survive.
// "ThinKV", Methodology, think-before-evict: earlier Reasoning / Execution
// segments are pruned on an annealing schedule as Transitions follow.
// "Thought-Aware KV Cache Compaction ... (TAM)", section 2: segment budgets
// proportional to sqrt(mean mass) * size, pivotal tokens kept.
// "ThinKV", Continuous Thinking: eviction only clears mask bits -- the KV
// bytes never move; blocks that become empty leave the table and go back to
// their pool's free list for in-place reuse.
//
// evict_keys + evict_select: eight workgroups per sequence build one key
//   word per slot; then one 1024-thread workgroup per sequence, one thread
//   per slot in each pass.  Candidate keys (order-preserving importance bits,
//   then inverted position, so ties go to the lower position) are radix-selected
//   for the k-th largest; losers' mask bits are cleared; the table row is
//   compacted in order with a ballot prefix scan; freed entries are listed
//   in table order.
// evict_tbe_prep / evict_tam_prep + evict_seg_drop + evict_seg_compact:
//   segment-granular eviction, thought-adaptive (TBE) or by thought-aware
//   budgets (TAM) (below).
// The compacting kernels (evict_select, evict_seg_compact) end by pushing
// each sequence's freed ids onto the free stacks, ranked across sequences in
// batch order (kvq_sync.h, push_freed).
#include <limits.h>

#include "kvq_device.h"
#include "kvq_internal.h"
#include "kvq_sync.h"

namespace kvq {

namespace {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int SEL_UNROLL = 17;  // slots a thread takes per batch (17 x 1024: rows of up to 1088 entries at once)
constexpr int RADIX_BITS = 11;  // digit width of the radix select
constexpr int RADIX = 1 << RADIX_BITS;
static_assert(RADIX == EVICT_RADIX, "top-k's first-digit histograms");
// segment eviction's selection: DROP_WGS workgroups of DROP_THREADS per
// sequence, DROP_WAVES waves in all
constexpr int DROP_THREADS = 256;
constexpr int DROP_WGS = 16;
constexpr int DROP_WAVES = DROP_WGS * DROP_THREADS / 64;
constexpr int TBE_RUN = 16;  // chunks of 64 positions / candidates a wave takes per pass
constexpr int TAM_FAST = 32768;  // budgets: rows up to this many candidates take the one-pass sums
// top-k's slot keys: KEY_WGS workgroups of KEY_THREADS per sequence
constexpr int KEY_WGS = EVICT_KEY_WGS;
constexpr int KEY_THREADS = 256;
constexpr int KEY_UNROLL = 8;

// Grids of `per` workgroups per sequence are laid out so that all of
// sequence b's run on the XCD that runs workgroup b of a grid of one per
// sequence (workgroups go to the 8 XCDs round-robin by id): id = 8 per
// (b / 8) + 8 j + b % 8 for the sequence's j-th workgroup.  What one kernel
// writes for a sequence is then read by the next from the same L2.
constexpr int XCDS = 8;
inline int xcd_grid(int per, int B) { return XCDS * per * ((B + XCDS - 1) / XCDS); }
__device__ inline bool xcd_part(int per, int B, int &b, int &j) {
    const int id = blockIdx.x, grp = id / (XCDS * per), r = id % (XCDS * per);
    j = r / XCDS;
    b = grp * XCDS + r % XCDS;
    return b < B;
}

// Batched loads: element i of a[0 .. n) for i < n, else dflt, loaded from
// the clamped index (n >= 1) so that the load has no branch around it and
// a thread's loads of one batch are all issued before the first wait.
template <class T>
__device__ inline T ld_clamped(const T *a, int i, int n, T dflt) {
    const T v = a[min(i, n - 1)];
    return i < n ? v : dflt;
}

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

// The start of a compacting kernel, before any of the workgroup's work: wave
// 0 takes the call's epoch and thread p < 3 the free-stack top of pool p
// (both read before the workgroup's counts are published; only the last
// workgroup moves them, once every sequence's counts are in).
__device__ inline uint32_t push_begin(const kvq_cache &c, const SyncWs &sync, int *top0) {
    uint32_t epoch = 0;
    if (threadIdx.x < 64) epoch = sync_epoch(sync);
    if (threadIdx.x < 3) top0[threadIdx.x] = c.free_top[threadIdx.x];
    return epoch;
}

// Publish sequence b's freed count per pool (pool_cnt, complete): threads
// 0 .. 2, after a barrier.
__device__ inline void push_publish(const kvq_cache &c, int b, const int *pool_cnt, const SyncWs &sync,
                                    uint32_t epoch) {
    if (threadIdx.x < 3) {
        wait_loads_done();   // this workgroup's reads of the tops are in
        sync_publish(sync, c.B, b, threadIdx.x, epoch, (uint32_t)pool_cnt[threadIdx.x]);
    }
}

// Push sequence b's freed ids (freed[0 .. nf), table order; pool_cnt per
// pool, already published) onto the free stacks, the sequences in batch
// order: sum the counts of the sequences before b (wave 0) and push each id
// at the pool's old top + that sum + its rank in table order.  The last
// sequence raises the tops and closes the call.  top0 and epoch from
// push_begin; every thread calls it, after a barrier.
__device__ inline void push_freed(const kvq_cache &c, int b, const uint32_t *freed, int nf, const int *pool_cnt,
                                  const int *top0, const SyncWs &sync, uint32_t epoch) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    __shared__ int base[3];
    __shared__ int wave_cnt[SEL_WAVES][3];
    const bool last = b == c.B - 1;
    if (nf == 0 && !last) return;
    if (wv == 0) {
        int cnt[3];
        const uint32_t pm = last ? 7u : (pool_cnt[0] ? 1u : 0u) | (pool_cnt[1] ? 2u : 0u) | (pool_cnt[2] ? 4u : 0u);
        const bool ok = sync_counts_before(sync, c.B, b, epoch, pm, cnt);
        if (lane < 3) {
            const int at = top0[lane] + (lane == 0 ? cnt[0] : lane == 1 ? cnt[1] : cnt[2]);
            base[lane] = at;
            if (last) c.free_top[lane] = at + pool_cnt[lane];
        }
        if (lane == 0) {
            if (!ok) *c.status = KVQ_EHIP;
            if (last) sync_close(sync, epoch);
        }
    }
    __syncthreads();
    for (int c0 = 0; c0 < nf; c0 += SEL_THREADS) {
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
            pool_sel(c.free_ids, pool)[base[pool] + before + rank] = ent & 0x3fffffffu;
        }
        __syncthreads();
        if (tid < 3) {
            int tot = 0;
            for (int w = 0; w < SEL_WAVES; ++w) tot += wave_cnt[w][tid];
            base[tid] += tot;
        }
        __syncthreads();
    }
}

// Clear the slots the rule drops, compact the table row and push the freed
// ids (one workgroup per sequence).  key holds one word per slot (0:
// cleared); keep(word) says whether a valid slot survives.  Thread per
// slot: 16-lane ballots give each entry's old and new masks; the entry's
// first slot's lane stores the new mask if it changed, parks it in that
// slot's word and, if it is 0, counts the entry as freed in its pool.  The
// counts are published at once; then, thread per entry, the entries that
// kept a slot are packed in order and the emptied ones listed, and the list
// is pushed (push_freed) once the earlier sequences' counts are in.
// pool_cnt must be zero and top0 / epoch taken (push_begin) before.  The
// row's entries are read from row_in (the row itself, or a copy) and the
// compacted row is written to row.
template <class Keep>
__device__ inline void clear_compact_push(const kvq_cache &c, int b, uint64_t *key, int nslot, int nb,
                                          const uint32_t *row_in, uint32_t *row, EvictWs &ws, int *wave_tot,
                                          int *pool_cnt, const int *top0, const SyncWs &sync, uint32_t epoch,
                                          const Keep &keep) {
    const int tid = threadIdx.x, lane = tid & 63;
#pragma unroll 1
    for (int i0 = 0; i0 < nslot; i0 += SEL_THREADS * SEL_UNROLL) {
        uint32_t ent[SEL_UNROLL];
        uint64_t kk[SEL_UNROLL];
#pragma unroll
        for (int u = 0; u < SEL_UNROLL; ++u) {
            const int i = i0 + u * SEL_THREADS + tid;
            ent[u] = ld_clamped(row_in, i >> 4, (nslot + BLK - 1) >> 4, 0u);
            kk[u] = ld_clamped(key, i, nslot, (uint64_t)0);
        }
#pragma unroll
        for (int u = 0; u < SEL_UNROLL; ++u) {
            const int i = i0 + u * SEL_THREADS + tid;
            const bool bit = keep(kk[u]);
            const uint32_t oldm = (uint32_t)(__ballot(kk[u] != 0) >> (lane & 48)) & 0xffffu;
            const uint32_t newm = (uint32_t)(__ballot(bit) >> (lane & 48)) & 0xffffu;
            if (i < nslot && (i & 15) == 0) {
                if (newm != oldm) pool_sel(c.mask, ent[u] >> 30)[ent[u] & 0x3fffffffu] = (uint16_t)newm;
                key[i] = newm;
                if (newm == 0) atomicAdd(&pool_cnt[ent[u] >> 30], 1);
            }
        }
    }
    __syncthreads();
    push_publish(c, b, pool_cnt, sync, epoch);

    int kept_base = 0, freed_base = 0;
    uint32_t *freed = ws.freed + (size_t)b * c.max_blocks;
    for (int c0 = 0; c0 < nb; c0 += SEL_THREADS) {
        const int e = c0 + tid;
        const bool has = e < nb;
        uint32_t ent = 0, newm = 0;
        if (has) {
            ent = row_in[e];
            newm = (uint32_t)key[(size_t)e * BLK];
        }
        int nkept, nfreed;
        const int kr = block_prefix(has && newm != 0, wave_tot, nkept);
        const int fr = block_prefix(has && newm == 0, wave_tot, nfreed);
        if (has) {
            if (newm != 0) row[kept_base + kr] = ent;
            else freed[freed_base + fr] = ent;
        }
        kept_base += nkept;
        freed_base += nfreed;
        __syncthreads();
    }
    if (tid == 0) c.n_blocks[b] = kept_base;
    push_freed(c, b, freed, freed_base, pool_cnt, top0, sync, epoch);
}

// One word per slot (slot s of entry e at 16 e + s), thread per slot, for
// the slots [i_begin, i_end) of a row: 0 for a cleared slot, 1 for a valid
// slot outside [lo, hi), else the candidate's key (a finite importance gives
// a key >= 2^55).  UNROLL slots per thread and batch of NT threads; the
// entry, then its mask and positions, then the importance, each level's
// loads issued together.  Without an importance a candidate's word is 3.
// pmap, if given, receives (pool << 30) | slot for each candidate position;
// hist1, if given (LDS), counts the candidates by their key's top
// RADIX_BITS bits.  Returns this thread's candidate count.
template <int NT, int UNROLL>
__device__ inline int slot_keys(const kvq_cache &c, const uint32_t *row, const float *imp, int i_begin,
                                int i_end, int lo, int hi, uint64_t *key, uint32_t *pmap,
                                uint32_t *hist1 = nullptr) {
    const int tid = threadIdx.x;
    int my_cand = 0;
    for (int i0 = i_begin; i0 < i_end; i0 += NT * UNROLL) {
        uint32_t ent[UNROLL], m[UNROLL];
        int p[UNROLL];
        // every level's loads unconditional (clamped slot, clamped
        // position), so that each level is issued as one batch
        float f[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int i = min(i0 + u * NT + tid, i_end - 1);
            ent[u] = row[i >> 4];
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int i = min(i0 + u * NT + tid, i_end - 1);
            m[u] = pool_sel(c.mask, ent[u] >> 30)[ent[u] & 0x3fffffffu];
            p[u] = pool_sel(c.pos, ent[u] >> 30)[(size_t)(ent[u] & 0x3fffffffu) * BLK + (i & 15)];
        }
        if (imp) {
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) f[u] = imp[min(max(p[u], 0), c.n_cap - 1)];
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int i = i0 + u * NT + tid;
            uint64_t kk = 0;
            if (i < i_end && ((m[u] >> (i & 15)) & 1u)) {
                kk = 1;
                if (p[u] >= lo && p[u] < hi) {
                    kk = imp ? sel_key(f[u], p[u]) : 3ull;
                    ++my_cand;
                    if (hist1) atomicAdd(&hist1[(uint32_t)(kk >> (64 - RADIX_BITS))], 1u);
                    if (pmap) pmap[p[u]] = (uint32_t)i | (ent[u] & 0xc0000000u);
                }
            }
            if (i < i_end) key[i] = kk;
        }
    }
    return my_cand;
}

// Top-k, step 1: one word per slot (slot_keys), a sequence's row shared by
// KEY_WGS workgroups (xcd_grid) in contiguous parts; each part's candidate
// count goes to ws.kcnt and its histogram of the candidates' first radix
// digit to ws.khist (the select's first pass, spread over the parts).
__global__ __launch_bounds__(KEY_THREADS) void evict_keys(kvq_cache c, const float *importance, int q_window,
                                                          int recent_window, EvictWs ws) {
    const int tid = threadIdx.x;
    int b, part;
    if (!xcd_part(KEY_WGS, c.B, b, part)) return;
    const int nslot = c.n_blocks[b] * BLK;
    const int share = (nslot + KEY_WGS - 1) / KEY_WGS;
    const int i0 = min(nslot, part * share), i1 = min(nslot, i0 + share);
    const int lo = q_window, hi = c.seq_len[b] - recent_window;
    __shared__ uint32_t hist1[RADIX];
    for (int i = tid; i < RADIX; i += KEY_THREADS) hist1[i] = 0;
    __syncthreads();
    int my_cand = slot_keys<KEY_THREADS, KEY_UNROLL>(c, c.table + (size_t)b * c.max_blocks,
                                                     importance + (size_t)b * c.n_cap, i0, i1, lo, hi,
                                                     ws.cand + (size_t)b * c.max_blocks * BLK, nullptr, hist1);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) my_cand += __shfl_xor(my_cand, off);
    __shared__ int wsum[KEY_THREADS / 64];
    if ((tid & 63) == 0) wsum[tid >> 6] = my_cand;
    __syncthreads();
    if (tid == 0) {
        int n = 0;
#pragma unroll
        for (int w = 0; w < KEY_THREADS / 64; ++w) n += wsum[w];
        ws.kcnt[b * KEY_WGS + part] = n;
    }
    uint32_t *h = ws.khist + ((size_t)b * KEY_WGS + part) * RADIX;
    for (int i = tid; i < RADIX; i += KEY_THREADS) h[i] = hist1[i];
}

// Top-k, step 2, on the row's slot keys at `keys` (in memory, or a copy in
// LDS): radix-select the k-th largest candidate key, RADIX_BITS at a time
// from the top, stopping as soon as the boundary digit's whole bin is kept;
// then clear the losers, compact the table row and push the freed ids
// (clear_compact_push).  Wide digits spread the keys, whose top bits (sign
// and exponent of the importance) take few values, over many bins: fewer
// passes and fewer same-bin atomics.  The digits split each 32-bit half of
// the key as 11 + 11 + 10 bits.
__device__ __attribute__((always_inline)) inline void select_and_compact(
    const kvq_cache &c, int b, uint64_t *keys, int nslot, int nb, const uint32_t *row_in, uint32_t *row,
    EvictWs &ws, int k,
    bool evicting, uint32_t *hist, int *s_digit, int *s_cum, int *wave_tot, int *pool_cnt, const int *top0,
    const SyncWs &sync, uint32_t epoch) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    uint64_t thr = 0;
    int thr_shift = 0;
    if (evicting && k > 0) {
        uint64_t prefix = 0;
        uint32_t need = (uint32_t)k;
        for (int top = 64;;) {
            const int width = min(RADIX_BITS, top > 32 ? top - 32 : top);
            const int shift = top - width;
            const uint32_t dmask = (1u << width) - 1u;
            if (top == 64) {
                // the first digit: the parts' histograms from evict_keys
                const uint32_t *kh = ws.khist + (size_t)b * KEY_WGS * RADIX;
                for (int i = tid; i < RADIX; i += SEL_THREADS) {
                    uint32_t h = 0;
#pragma unroll
                    for (int j = 0; j < KEY_WGS; ++j) h += kh[j * RADIX + i];
                    hist[i] = h;
                }
            } else {
                for (int i = tid; i < RADIX; i += SEL_THREADS) hist[i] = 0;
            }
            __syncthreads();
            const uint64_t hmask = top == 64 ? 0ull : (~0ull << top);
            for (int i0 = 0; i0 < nslot && top < 64; i0 += SEL_THREADS * SEL_UNROLL) {
                uint64_t kk[SEL_UNROLL];
#pragma unroll
                for (int u = 0; u < SEL_UNROLL; ++u) {
                    const int i = i0 + u * SEL_THREADS + tid;
                    kk[u] = ld_clamped(keys, i, nslot, (uint64_t)0);
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
                    *s_digit = RADIX - 1 - BPL * lane - j;
                    *s_cum = (int)cum;
                }
            }
            __syncthreads();
            const int dgt = *s_digit;
            need -= (uint32_t)*s_cum;
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
    clear_compact_push(c, b, keys, nslot, nb, row_in, row, ws, wave_tot, pool_cnt, top0, sync, epoch,
                       [&](uint64_t kk) {
        return kk != 0 && !(evicting && kk > 1 && !(k > 0 && (kk >> thr_shift) >= (thr >> thr_shift)));
    });
}

// Rows of up to this many slots (one batch of the workgroup) are selected
// from a copy of their keys in LDS (136 KiB); longer rows from the keys in
// memory.
constexpr int SEL_LDS_SLOTS = SEL_THREADS * SEL_UNROLL;

// Top-k, step 2 (one workgroup per sequence): the k-th largest key, then
// the losers cleared, the row compacted and the freed ids pushed.
__global__ __launch_bounds__(SEL_THREADS) void evict_select(kvq_cache c, const int32_t *keep_k, EvictWs ws,
                                                           SyncWs sync) {
    const int b = blockIdx.x, tid = threadIdx.x;
    __shared__ int top0[3];
    const uint32_t epoch = push_begin(c, sync, top0);
    const int nb = c.n_blocks[b];
    const int nslot = nb * BLK;
    uint32_t *row = c.table + (size_t)b * c.max_blocks;
    uint64_t *key = ws.cand + (size_t)b * c.max_blocks * BLK;

    __shared__ uint64_t lkeys[SEL_LDS_SLOTS];
    __shared__ uint32_t lrow[SEL_LDS_SLOTS / BLK];
    __shared__ uint32_t hist[RADIX];
    __shared__ int s_digit, s_cum;
    __shared__ int wave_tot[SEL_WAVES];
    __shared__ int pool_cnt[4];
    if (tid < 4) pool_cnt[tid] = 0;

    // 1. the candidates counted by evict_keys
    int n = 0;
#pragma unroll
    for (int j = 0; j < KEY_WGS; ++j) n += ws.kcnt[b * KEY_WGS + j];
    const int k = max(keep_k[b], 0);
    const bool evicting = n > k;

    // 2, 3. select, clear, compact, push
    if (nslot <= SEL_LDS_SLOTS) {
        for (int i0 = 0; i0 < nslot; i0 += SEL_THREADS * SEL_UNROLL) {
            uint64_t kk[SEL_UNROLL];
#pragma unroll
            for (int u = 0; u < SEL_UNROLL; ++u) {
                const int i = i0 + u * SEL_THREADS + tid;
                kk[u] = ld_clamped(key, i, nslot, (uint64_t)0);
            }
#pragma unroll
            for (int u = 0; u < SEL_UNROLL; ++u) {
                const int i = i0 + u * SEL_THREADS + tid;
                if (i < nslot) lkeys[i] = kk[u];
            }
        }
        for (int e = tid; e < nb; e += SEL_THREADS) lrow[e] = row[e];
        __syncthreads();
        select_and_compact(c, b, lkeys, nslot, nb, lrow, row, ws, k, evicting, hist, &s_digit, &s_cum, wave_tot,
                           pool_cnt, top0, sync, epoch);
    } else {
        __syncthreads();
        select_and_compact(c, b, key, nslot, nb, row, row, ws, k, evicting, hist, &s_digit, &s_cum, wave_tot,
                           pool_cnt, top0, sync, epoch);
    }
}

// Exclusive prefix sum over the waves of a value each wave holds
// (uniform within the wave), and the total.  All threads must call it.
__device__ inline int wave_offsets(int x, int *wave_tot, int &total) {
    const int wv = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) wave_tot[wv] = x;
    __syncthreads();
    int before = 0;
    total = 0;
    for (int w = 0; w < SEL_WAVES; ++w) {
        const int v = wave_tot[w];
        before += w < wv ? v : 0;
        total += v;
    }
    __syncthreads();
    return before;
}

// Drops of one segment [a, e) of position-ordered candidates, taken by one
// wave: all but the best `keep` of them (larger importance, then lower
// position) get word 2 in the slot words; the kept ones keep their word 3.
// ob[k] is candidate k's importance as 32 order bits, or 0 for a candidate
// that is never dropped and does not count toward `keep` (which is at most
// the number of the others).  The keep-th largest
// value t is found bit by bit from the top: the largest t with at least
// `keep` values >= t, counted with ballots.  Every value above t is kept,
// and of the values equal to t the first keep - #(above t) in position
// order.  A missing candidate holds 0, which no tested threshold (a bit
// set) or value above t counts.  R > 0: the segment's values and slots stay
// in registers, R chunks of 64 (L <= 64 R), loaded together; R == 0: any
// length, by 8-bit digits through the wave's 256-word LDS histogram hist.
template <int R>
__device__ inline void tbe_segment(const uint32_t *ob, const int32_t *ord, uint64_t *key, int a, int e,
                                   int keep, uint32_t *hist) {
    const int lane = threadIdx.x & 63;
    const uint64_t below = (1ull << lane) - 1ull;
    uint32_t t = 0;
    int above = 0, seen = 0;
    if constexpr (R > 0) {
        uint32_t v[R];
        int32_t sl[R];
        bool live[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int k = a + 64 * r + lane;
            live[r] = k < e;
            v[r] = live[r] ? ob[k] : 0u;
            sl[r] = live[r] ? ord[k] & 0x3fffffff : 0;
        }
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t c = t | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int r = 0; r < R; ++r) cnt += __popcll(__ballot(v[r] >= c));
            if (cnt >= keep) t = c;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) above += __popcll(__ballot(v[r] > t));
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint64_t eq = __ballot(live[r] && v[r] == t);
            const int rk = seen + __popcll(eq & below);
            if (live[r] && v[r] != 0 && !(v[r] > t || (v[r] == t && rk < keep - above))) key[sl[r]] = 2ull;
            seen += __popcll(eq);
        }
    } else {
        // any length: radix select on 8-bit digits from the top, one
        // 256-bin LDS histogram per wave (hist), 4 passes over the values
        // and one for the keep or drop decisions.  need = how many of the values that
        // match the digits chosen so far are still to be kept.
        int need = keep;
        uint32_t pre = 0, pre_mask = 0;
        for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
            for (int i = 0; i < 4; ++i) hist[4 * lane + i] = 0;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            for (int k = a + lane; k < e; k += 64) {
                const uint32_t x = ob[k];
                if (x != 0 && (x & pre_mask) == pre) atomicAdd(&hist[(x >> shift) & 255u], 1u);
            }
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // suffix counts: S(d) = matching values with digit >= d; lane
            // holds digits 4 lane .. 4 lane + 3
            uint32_t h[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) h[i] = hist[4 * lane + i];
            const int tot = (int)(h[0] + h[1] + h[2] + h[3]);
            int incl = tot;  // sum over lanes >= this one
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int y = __shfl_down(incl, d);
                incl += lane + d < 64 ? y : 0;
            }
            int sfx[4];
            sfx[3] = incl - tot + (int)h[3];
            sfx[2] = sfx[3] + (int)h[2];
            sfx[1] = sfx[2] + (int)h[1];
            sfx[0] = sfx[1] + (int)h[0];
            // digit = largest d with S(d) >= need (S falls as d rises)
            int ge = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) ge += __popcll(__ballot(sfx[i] >= need));
            const int dig = ge - 1;
            // matching values with a larger digit are all kept
            int gt = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) gt += 4 * lane + i > dig ? (int)h[i] : 0;
#pragma unroll
            for (int d = 32; d > 0; d >>= 1) gt += __shfl_xor(gt, d);
            need -= gt;
            pre |= (uint32_t)dig << shift;
            pre_mask |= 255u << shift;
        }
        t = pre;
        above = keep - need;
        for (int k = a + lane; k - lane < e; k += 64) {
            const bool live = k < e;
            const uint32_t v = live ? ob[k] : 0u;
            const uint64_t eq = __ballot(live && v == t);
            const int rk = seen + __popcll(eq & below);
            if (live && v != 0 && !(v > t || (v == t && rk < keep - above))) key[ord[k] & 0x3fffffff] = 2ull;
            seen += __popcll(eq);
        }
    }
}

// One segment: nothing to do when everything is kept (keep >= L), every
// droppable candidate dropped when keep is 0, else the selection above: in registers
// up to 512 candidates, by LDS histogram beyond.
__device__ inline void tbe_segment_any(const uint32_t *ob, const int32_t *ord, uint64_t *key, int a, int e,
                                       int keep, uint32_t *hist) {
    const int lane = threadIdx.x & 63;
    const int L = e - a;
    if (keep >= L) return;
    if (keep <= 0) {
        for (int k = a + lane; k < e; k += 64)
            if (ob[k] != 0) key[ord[k] & 0x3fffffff] = 2ull;
    } else if (L <= 64) {
        tbe_segment<1>(ob, ord, key, a, e, keep, hist);
    } else if (L <= 128) {
        tbe_segment<2>(ob, ord, key, a, e, keep, hist);
    } else if (L <= 256) {
        tbe_segment<4>(ob, ord, key, a, e, keep, hist);
    } else if (L <= 512) {
        tbe_segment<8>(ob, ord, key, a, e, keep, hist);
    } else {
        tbe_segment<0>(ob, ord, key, a, e, keep, hist);
    }
}

// Window score in fixed point, 16 fractional bits: floor(score * 2^16) for
// 0 < score < 2^16, 2^32 - 1 from 2^16 up, 0 for score <= 0 or NaN.
__device__ inline uint32_t tam_fix(float score) {
    if (!(score > 0.0f)) return 0u;
    if (score >= 65536.0f) return 0xffffffffu;
    return (uint32_t)(score * 65536.0f);
}

// One DPP step of a 64-bit wave scan: x of the lane CTRL selects (0 where
// there is none, or in a row outside RM).
template <int CTRL, int RM>
__device__ inline uint64_t dpp_u64(uint64_t x) {
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, CTRL, RM, 0xf, false);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(x >> 32), CTRL, RM, 0xf, false);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
// Inclusive sum of x over lanes 0 .. this one (all 64 lanes active): shifts
// of 1, 2, 4, 8 inside each 16-lane row, then each row's last lane added to
// the rows after it (row broadcasts of lanes 15 and 31).
__device__ inline uint64_t wave_incl_scan_u64(uint64_t x) {
    x += dpp_u64<0x111, 0xf>(x);
    x += dpp_u64<0x112, 0xf>(x);
    x += dpp_u64<0x114, 0xf>(x);
    x += dpp_u64<0x118, 0xf>(x);
    x += dpp_u64<0x142, 0xa>(x);
    x += dpp_u64<0x143, 0xc>(x);
    return x;
}

// floor(sqrt(x)), by bisection on the root (exact integer arithmetic).
__device__ inline uint64_t isqrt_u64(uint64_t x) {
    uint64_t lo = 0, hi = 1ull << 32;
    while (hi - lo > 1) {
        const uint64_t mid = lo + (hi - lo) / 2;
        if (mid * mid <= x) lo = mid;
        else hi = mid;
    }
    return lo;
}

// Sum of a 64-bit value over the workgroup (all threads get it).
__device__ inline uint64_t block_sum_u64(uint64_t x, uint64_t *wave_u64) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int d = 32; d > 0; d >>= 1) x += __shfl_xor(x, d);
    if (lane == 0) wave_u64[wv] = x;
    __syncthreads();
    uint64_t t = 0;
    for (int w = 0; w < SEL_WAVES; ++w) t += wave_u64[w];
    __syncthreads();
    return t;
}

// Inclusive prefix sum of a 64-bit value over the workgroup (thread order)
// and the total.
__device__ inline uint64_t block_scan_u64(uint64_t x, uint64_t *wave_u64, uint64_t &total) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    uint64_t incl = x;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint64_t y = __shfl_up(incl, d);
        incl += lane >= d ? y : 0ull;
    }
    if (lane == 63) wave_u64[wv] = incl;
    __syncthreads();
    uint64_t before = 0;
    total = 0;
    for (int w = 0; w < SEL_WAVES; ++w) {
        const uint64_t v = wave_u64[w];
        before += w < wv ? v : 0ull;
        total += v;
    }
    __syncthreads();
    return before + incl;
}

// Segment-granular eviction, two policies on one pipeline: a prep kernel
// per policy (one 1024-thread workgroup per sequence) orders the candidates
// (valid slots with q_window <= pos < seq_len - recent_window) by position,
// cuts them into segments and gives each segment the number of its
// droppable candidates it keeps (segkeep); evict_seg_drop then drops the
// rest of each segment, lowest value first (ties: higher position first),
// and evict_seg_compact clears, compacts and frees the emptied blocks.

struct SegOrder {
    int n, nseg, n_t;
    uint64_t s_all;  // sum of the fixed-point scores (when sfx is written)
};

// Steps shared by the prep kernels:
//   1. one word per slot (3 for a candidate, kept unless evict_seg_drop
//      drops it) and a position -> (pool, slot) map of the candidates;
//   2. the candidates in position order, each wave taking TBE_RUN chunks of
//      64 consecutive positions (ballots number them inside the wave, one
//      scan of the wave totals places the waves): their (pool, slot) words,
//      their value's order bits and, if sfx is given, its fixed point;
//   3. runs of one thought type, laid out the same way over the
//      candidates: the first candidate of each run and the Transition runs
//      up to and including it (segstart, segtc), then the counts.
__device__ inline SegOrder seg_order(const kvq_cache &c, int b, const float *value, int q_window,
                                     int recent_window, EvictWs &ws, uint32_t *sfx, int *wave_tot,
                                     uint64_t *wave_u64) {
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int nb = c.n_blocks[b];
    const int nslot = nb * BLK;
    const int lo = q_window, hi = min(c.seq_len[b] - recent_window, c.n_cap);
    const uint32_t *row = c.table + (size_t)b * c.max_blocks;
    const float *val = value + (size_t)b * c.n_cap;
    const size_t ms = (size_t)c.max_blocks * BLK;
    uint64_t *key = ws.cand + (size_t)b * ms;
    uint32_t *pmap = ws.pmap + (size_t)b * c.n_cap;
    int32_t *ord = ws.ord + (size_t)b * ms;
    uint32_t *ob = ws.ob + (size_t)b * ms;
    int32_t *segstart = ws.segstart + (size_t)b * (ms + 1);
    int32_t *segtc = ws.segtc + (size_t)b * ms;

    for (int p = lo + tid; p < hi; p += SEL_THREADS) pmap[p] = 0xffffffffu;
    __syncthreads();

    // 1.
    slot_keys<SEL_THREADS, SEL_UNROLL>(c, row, nullptr, 0, nslot, lo, hi, key, pmap);
    __syncthreads();

    // 2.
    const uint64_t below = (1ull << lane) - 1ull;
    int n = 0;
    uint64_t my_s = 0;
    for (int p0 = lo; p0 < hi; p0 += SEL_THREADS * TBE_RUN) {
        const int wb = p0 + wv * 64 * TBE_RUN;
        uint32_t v[TBE_RUN];
        float im[TBE_RUN];
#pragma unroll
        for (int u = 0; u < TBE_RUN; ++u) {
            const int p = wb + 64 * u + lane;
            v[u] = ld_clamped(pmap, p, hi, 0xffffffffu);
            im[u] = ld_clamped(val, p, hi, 0.0f);
        }
        int cnt = 0;
#pragma unroll
        for (int u = 0; u < TBE_RUN; ++u) cnt += __popcll(__ballot(v[u] != 0xffffffffu));
        int tot;
        int at = n + wave_offsets(cnt, wave_tot, tot);
#pragma unroll
        for (int u = 0; u < TBE_RUN; ++u) {
            const uint64_t bal = __ballot(v[u] != 0xffffffffu);
            if (v[u] != 0xffffffffu) {
                const int i = at + __popcll(bal & below);
                ord[i] = (int32_t)v[u];
                ob[i] = order_bits(im[u]);
                if (sfx) {
                    const uint32_t f = tam_fix(im[u]);
                    sfx[i] = f;
                    my_s += f;
                }
            }
            at += __popcll(bal);
        }
        n += tot;
    }
    const uint64_t s_all = sfx ? block_sum_u64(my_s, wave_u64) : 0ull;
    __syncthreads();

    // 3. a run starts at a pool change from the previous candidate; the
    //    starts and the Transition starts are counted together (16 bits
    //    each) for the wave scan
    int nseg = 0, n_t = 0;
    for (int k0 = 0; k0 < n; k0 += SEL_THREADS * TBE_RUN) {
        const int wb = k0 + wv * 64 * TBE_RUN;
        int pool[TBE_RUN];
#pragma unroll
        for (int u = 0; u < TBE_RUN; ++u) {
            const int k = wb + 64 * u + lane;
            const int32_t o = ld_clamped(ord, k, n, 0);
            pool[u] = k < n ? (int)((uint32_t)o >> 30) : -1;
        }
        const int before0 = wb > 0 && wb <= n ? (int)((uint32_t)ord[wb - 1] >> 30) : -1;
        uint32_t stm = 0;  // bit u: candidate of chunk u starts a run
        int cnt = 0;
#pragma unroll
        for (int u = 0; u < TBE_RUN; ++u) {
            const int up = __shfl_up(pool[u], 1);
            const int carry = u == 0 ? before0 : __builtin_amdgcn_readlane(pool[u > 0 ? u - 1 : 0], 63);
            const int prev = lane == 0 ? carry : up;
            const bool st = pool[u] >= 0 && pool[u] != prev;
            stm |= (uint32_t)st << u;
            cnt += __popcll(__ballot(st)) + (__popcll(__ballot(st && pool[u] == 2)) << 16);
        }
        int tot;
        const int off = wave_offsets(cnt, wave_tot, tot);
        int sg = nseg + (off & 0xffff), tc = n_t + (off >> 16);
#pragma unroll
        for (int u = 0; u < TBE_RUN; ++u) {
            const bool st = (stm >> u) & 1u;
            const uint64_t bs = __ballot(st);
            const uint64_t bt = __ballot(st && pool[u] == 2);
            if (st) {
                const int i = sg + __popcll(bs & below);
                segstart[i] = wb + 64 * u + lane;
                segtc[i] = tc + __popcll(bt & below) + (pool[u] == 2 ? 1 : 0);
            }
            sg += __popcll(bs);
            tc += __popcll(bt);
        }
        nseg += tot & 0xffff;
        n_t += tot >> 16;
    }
    if (tid == 0) segstart[nseg] = n;
    __syncthreads();
    return SegOrder{n, nseg, n_t, s_all};
}

// evict_tbe_prep: thought-adaptive eviction ("ThinKV", Methodology,
// think-before-evict).  Segments are the runs of one thought type.  A
// segment followed by k Transition segments keeps everything if k == 0,
// else its best max(r_min, r0 >> (k - 1)) slots (Reasoning, Execution) or
// t_keep slots (Transition), by importance.
// A sequence outside seq_mask gets segn = -1: no segment to drop, and the
// compaction leaves it as it is.
__global__ __launch_bounds__(SEL_THREADS) void evict_tbe_prep(kvq_cache c, const float *importance,
                                                              const uint8_t *seq_mask, int r0, int r_min,
                                                              int t_keep, int q_window, int recent_window,
                                                              EvictWs ws) {
    const int b = blockIdx.x, tid = threadIdx.x;
    if (seq_mask && seq_mask[b] == 0) {
        if (tid == 0) ws.segn[2 * b] = -1;
        return;
    }
    __shared__ int wave_tot[SEL_WAVES];
    __shared__ uint64_t wave_u64[SEL_WAVES];
    const SegOrder so = seg_order(c, b, importance, q_window, recent_window, ws, nullptr, wave_tot, wave_u64);
    const size_t ms = (size_t)c.max_blocks * BLK;
    const int32_t *ord = ws.ord + (size_t)b * ms;
    const int32_t *segstart = ws.segstart + (size_t)b * (ms + 1);
    const int32_t *segtc = ws.segtc + (size_t)b * ms;
    int32_t *segkeep = ws.segkeep + (size_t)b * ms;
    for (int sg = tid; sg < so.nseg; sg += SEL_THREADS) {
        const int later = so.n_t - segtc[sg];
        const bool is_t = ((uint32_t)ord[segstart[sg]] >> 30) == 2u;
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
        segkeep[sg] = keep;
    }
    if (tid == 0) ws.segn[2 * b] = so.nseg;
}

// evict_tam_prep: thought-aware budgets ("Thought-Aware KV Cache Compaction
// ... (TAM)", section 2), compaction read as keeping a subset of the cache.
// value = the window score (mass from the R most recent queries), taken in
// fixed point s (tam_fix).
//   C. pivotal: s * N > pivot_c * S in doubles (N candidates, S the sum of
//      their s); their order bits become 0, so they are never dropped.
//      The budget left is T = max(0, keep_k - pivotal).
//   A. segments: a run of one thought type with at least min_seg
//      candidates opens a segment; a shorter run merges into the segment
//      before it (the first run always opens one).
//   B. per segment: n_i candidates, m_i droppable, S_i the sum of s (from
//      running sums over the candidates); weight
//      a_i = isqrt(floor(S_i / n_i) * 2^16) * m_i.  Rounds of
//      capped shares: a segment with T' a_i >= m_i A (T' the budget left
//      after the capped ones, A the sum of the uncapped weights) keeps all
//      m_i and leaves the pool; then the uncapped ones get
//      floor(T' C_j / A) - floor(T' C_(j-1) / A) from the running sums C_j
//      of their weights in position order (nothing when A = 0).  All of it
//      in integers (128-bit products), as exact as the rule.

__global__ __launch_bounds__(SEL_THREADS) void evict_tam_prep(kvq_cache c, const float *score,
                                                              const int32_t *keep_k, float pivot_c, int min_seg,
                                                              int q_window, int recent_window, EvictWs ws) {
    const int b = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    __shared__ int wave_tot[SEL_WAVES];
    __shared__ uint64_t wave_u64[SEL_WAVES];
    __shared__ int s_any;
    const size_t ms = (size_t)c.max_blocks * BLK;
    uint32_t *sfx = ws.sfx + (size_t)b * ms;
    const SegOrder so = seg_order(c, b, score, q_window, recent_window, ws, sfx, wave_tot, wave_u64);
    const int n = so.n;
    uint32_t *ob = ws.ob + (size_t)b * ms;
    int32_t *segstart = ws.segstart + (size_t)b * (ms + 1);
    int32_t *segkeep = ws.segkeep + (size_t)b * ms;
    uint64_t *sega = ws.sega + (size_t)b * ms;
    int32_t *segm = ws.segm + (size_t)b * ms;
    uint64_t *psum = ws.psum + (size_t)b * (ms + 1);
    int32_t *pcnt = ws.pcnt + (size_t)b * (ms + 1);


    // A. a run of at least min_seg candidates opens a segment, a shorter one
    //    merges into the segment before it: a block prefix over the runs
    //    compacts the run starts that open one (each chunk reads its starts
    //    before the prefix's barrier and writes below them after it)
    int nseg = so.nseg;
    if (min_seg > 1 && nseg > 1) {
        int out = 0;
        for (int r0 = 0; r0 < so.nseg; r0 += SEL_THREADS) {
            const int j = r0 + tid;
            const bool in = j < so.nseg;
            const int st = in ? segstart[j] : 0, en = in ? segstart[j + 1] : 0;
            const bool opens = in && (j == 0 || en - st >= min_seg);
            int tot;
            const int r = block_prefix(opens, wave_tot, tot);
            if (opens) segstart[out + r] = st;
            out += tot;
        }
        nseg = out;
        __syncthreads();
        if (tid == 0) segstart[nseg] = n;
        __syncthreads();
    }

    // B. weights from running sums over the candidates, packed in one word
    //    (s in the low 48 bits, the droppable count above), at the segments'
    //    first candidates only (the weights read nothing else).
    //    Rows of up to TAM_FAST candidates, one pass: each wave takes TBE_RUN
    //    coalesced chunks of 64 candidates, loads them at once, scans each
    //    chunk (DPP), stores the in-chunk prefix at segment starts (marked in
    //    an LDS bitmap) and the chunk's total in LDS; a block scan of the
    //    chunk totals then gives each chunk's offset (sums stay below 2^47,
    //    counts below 2^15).
    //    Longer rows: psum[k] = sum of s before candidate k, pcnt[k] =
    //    droppable candidates before it, for every candidate, in passes of
    //    SEL_THREADS * TBE_RUN (the totals carried across passes kept apart).
    //    Then a thread per segment.
    constexpr uint64_t LOW = (1ull << 48) - 1;
    __shared__ uint32_t segbits[TAM_FAST / 32];
    __shared__ uint64_t chunk_ex[TAM_FAST / 64];
    const bool fast = n <= TAM_FAST;
    uint64_t total_packed = 0;
    // C. pivotal candidates (s N > c S, in doubles): their order bits become
    //    0, so they are neither dropped nor counted as droppable.  In the
    //    one-pass sums the test is taken as each candidate is loaded.
    const double piv_rhs = (double)pivot_c * (double)so.s_all;
    int my_piv = 0;
    if (!fast) {
        for (int k = tid; k < n; k += SEL_THREADS) {
            if ((double)sfx[k] * (double)n > piv_rhs) {
                ob[k] = 0u;
                ++my_piv;
            }
        }
        __syncthreads();
    }
    if (fast) {
        for (int i = tid; i < (n + 31) / 32; i += SEL_THREADS) segbits[i] = 0u;
        __syncthreads();
        for (int sg = tid; sg < nseg; sg += SEL_THREADS) {
            const int k = segstart[sg];
            atomicOr(&segbits[k >> 5], 1u << (k & 31));
        }
        __syncthreads();
        constexpr int HALF = TBE_RUN / 2;   // chunks loaded at once (registers)
        for (int k0 = 0; k0 < n; k0 += SEL_THREADS * TBE_RUN) {
            const int wb = k0 + wv * 64 * TBE_RUN;
            for (int h = 0; h < TBE_RUN; h += HALF) {
                uint64_t v[HALF];
#pragma unroll
                for (int u = 0; u < HALF; ++u) {
                    const int k = wb + 64 * (h + u) + lane;
                    const uint32_t sv = ld_clamped(sfx, k, n, 0u), ov = ld_clamped(ob, k, n, 0u);
                    const bool piv = k < n && (double)sv * (double)n > piv_rhs;
                    if (piv) {
                        ob[k] = 0u;
                        ++my_piv;
                    }
                    v[u] = k < n ? ((uint64_t)sv | ((uint64_t)(ov != 0u && !piv ? 1 : 0) << 48)) : 0ull;
                }
#pragma unroll
                for (int u = 0; u < HALF; ++u) {
                    const int k = wb + 64 * (h + u) + lane;
                    const uint64_t incl = wave_incl_scan_u64(v[u]);
                    if (k < n && ((segbits[k >> 5] >> (k & 31)) & 1u)) psum[k] = incl - v[u];
                    if (lane == 63 && wb + 64 * (h + u) < n) chunk_ex[(wb + 64 * (h + u)) >> 6] = incl;
                }
            }
        }
        __syncthreads();
        const int nch = (n + 63) >> 6;   // <= TAM_FAST / 64 <= SEL_THREADS
        const uint64_t x = tid < nch ? chunk_ex[tid] : 0ull;
        const uint64_t incl = block_scan_u64(x, wave_u64, total_packed);
        if (tid < nch) chunk_ex[tid] = incl - x;
    } else {
        uint64_t carry_s = 0;
        int carry_c = 0;
        for (int k0 = 0; k0 < n; k0 += SEL_THREADS * TBE_RUN) {
            const int wb = k0 + wv * 64 * TBE_RUN;
            uint64_t mine = 0;
#pragma unroll
            for (int u = 0; u < TBE_RUN; ++u) {
                const int k = wb + 64 * u + lane;
                if (k < n) mine += (uint64_t)sfx[k] | ((uint64_t)(ob[k] != 0u ? 1 : 0) << 48);
            }
#pragma unroll
            for (int d = 32; d > 0; d >>= 1) mine += __shfl_xor(mine, d);
            if (lane == 0) wave_u64[wv] = mine;
            __syncthreads();
            uint64_t run = 0, tot = 0;
            for (int w = 0; w < SEL_WAVES; ++w) {
                const uint64_t v = wave_u64[w];
                run += w < wv ? v : 0ull;
                tot += v;
            }
            __syncthreads();
#pragma unroll 4
            for (int u = 0; u < TBE_RUN; ++u) {
                const int k = wb + 64 * u + lane;
                const uint64_t v = k < n ? ((uint64_t)sfx[k] | ((uint64_t)(ob[k] != 0u ? 1 : 0) << 48)) : 0ull;
                const uint64_t incl = wave_incl_scan_u64(v);
                if (k < n) {
                    const uint64_t ex = run + incl - v;
                    psum[k] = carry_s + (ex & LOW);
                    pcnt[k] = carry_c + (int32_t)(ex >> 48);
                }
                run += ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(incl >> 32), 63) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)incl, 63);
            }
            carry_s += tot & LOW;
            carry_c += (int32_t)(tot >> 48);
        }
        if (tid == 0) {
            psum[n] = carry_s;
            pcnt[n] = carry_c;
        }
    }
    __syncthreads();
    const long n_piv = (long)block_sum_u64((uint64_t)my_piv, wave_u64);
    const long T = max((long)keep_k[b] - n_piv, 0L);
    // (sum of s, droppable count) before candidate k, k a segment start or n
    auto prefix = [&](int k, uint64_t &sum, int &cnt) {
        if (fast) {
            const uint64_t w = k < n ? chunk_ex[k >> 6] + psum[k] : total_packed;
            sum = w & LOW;
            cnt = (int)(w >> 48);
        } else {
            sum = psum[k];
            cnt = pcnt[k];
        }
    };
    for (int sg = tid; sg < nseg; sg += SEL_THREADS) {
        const int a = segstart[sg], e = segstart[sg + 1];
        uint64_t sa, se;
        int ca, ce;
        prefix(a, sa, ca);
        prefix(e, se, ce);
        const uint64_t ssum = se - sa;
        const int m = ce - ca;
        sega[sg] = isqrt_u64((ssum / (uint64_t)(e - a)) << 16) * (uint64_t)m;
        segm[sg] = m > 0 ? m : -1;  // -m-1: capped (an empty segment keeps its 0)
    }
    __syncthreads();

    // B. rounds of capped shares
    uint64_t A;
    long t_left;
    for (;;) {
        uint64_t my_a = 0, my_cap = 0;
        for (int sg = tid; sg < nseg; sg += SEL_THREADS) {
            const int m = segm[sg];
            if (m >= 0) my_a += sega[sg];
            else my_cap += (uint64_t)(-m - 1);
        }
        A = block_sum_u64(my_a, wave_u64);
        t_left = T - (long)block_sum_u64(my_cap, wave_u64);
        if (tid == 0) s_any = 0;
        __syncthreads();
        if (A > 0) {
            for (int sg = tid; sg < nseg; sg += SEL_THREADS) {
                const int m = segm[sg];
                if (m >= 0 && (unsigned __int128)(uint64_t)t_left * sega[sg] >=
                                  (unsigned __int128)(uint64_t)m * A) {
                    segm[sg] = -m - 1;
                    s_any = 1;
                }
            }
        }
        __syncthreads();
        const int any = s_any;
        __syncthreads();
        if (!any) break;
    }

    // B. cumulative rounding over the uncapped weights, in segment order
    uint64_t carry = 0;
    for (int s0 = 0; s0 < nseg; s0 += SEL_THREADS) {
        const int sg = s0 + tid;
        const int m = sg < nseg ? segm[sg] : -1;
        const uint64_t w = m >= 0 ? sega[sg] : 0ull;
        uint64_t tot;
        const uint64_t run = carry + block_scan_u64(w, wave_u64, tot);
        if (sg < nseg) {
            long t = (long)(-m - 1);
            if (m >= 0) {
                t = 0;
                if (A > 0) {
                    const unsigned __int128 tl = (uint64_t)t_left;
                    const uint64_t q = (uint64_t)(tl * run / A), q0 = (uint64_t)(tl * (run - w) / A);
                    t = (long)(q - q0);
                }
            }
            segkeep[sg] = (int32_t)t;
        }
        carry += tot;
    }
    if (tid == 0) ws.segn[2 * b] = nseg;
}

// evict_seg_drop: DROP_WGS workgroups per sequence (xcd_grid), one wave per
// segment (segments gw, gw + DROP_WAVES, ... for the sequence's wave gw): each lane
// loads the bounds and retention of one of the wave's next 64 segments,
// then the wave takes them in turn (tbe_segment_any).  Spreading a
// sequence's segments over many workgroups puts the selection, which is
// bound by instruction issue, on every compute unit.
__global__ __launch_bounds__(DROP_THREADS) void evict_seg_drop(kvq_cache c, EvictWs ws) {
    int b, j;
    if (!xcd_part(DROP_WGS, c.B, b, j)) return;
    const int gw = j * (DROP_THREADS / 64) + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const size_t ms = (size_t)c.max_blocks * BLK;
    uint64_t *key = ws.cand + (size_t)b * ms;
    const int32_t *ord = ws.ord + (size_t)b * ms;
    const uint32_t *ob = ws.ob + (size_t)b * ms;
    const int32_t *segstart = ws.segstart + (size_t)b * (ms + 1);
    const int32_t *segkeep = ws.segkeep + (size_t)b * ms;
    const int nseg = ws.segn[2 * b];
    __shared__ uint32_t s_hist[DROP_THREADS / 64][256];
    for (int s0 = gw; s0 < nseg; s0 += DROP_WAVES * 64) {
        const int my = s0 + DROP_WAVES * lane;
        int ma = 0, me = 0, mkeep = 0;
        if (my < nseg) {
            ma = segstart[my];
            me = segstart[my + 1];
            mkeep = segkeep[my];
        }
        const int cnt = min(64, (nseg - s0 + DROP_WAVES - 1) / DROP_WAVES);
        for (int j = 0; j < cnt; ++j) {
            const int a = __builtin_amdgcn_readlane(ma, j);
            const int e = __builtin_amdgcn_readlane(me, j);
            const int keep = __builtin_amdgcn_readlane(mkeep, j);
            tbe_segment_any(ob, ord, key, a, e, keep, s_hist[threadIdx.x >> 6]);
        }
    }
}

// evict_seg_compact: clear the dropped slots (word 2) and compact the table
// row as evict_select does, one workgroup per sequence, then push the freed
// ids.  A sequence left as it is frees nothing but still takes its part in
// the batch-order push.
__global__ __launch_bounds__(SEL_THREADS) void evict_seg_compact(kvq_cache c, EvictWs ws, SyncWs sync) {
    const int b = blockIdx.x, tid = threadIdx.x;
    __shared__ int wave_tot[SEL_WAVES];
    __shared__ int pool_cnt[4];
    __shared__ int top0[3];
    const uint32_t epoch = push_begin(c, sync, top0);
    if (tid < 4) pool_cnt[tid] = 0;
    __syncthreads();
    if (ws.segn[2 * b] >= 0) {
        const int nb = c.n_blocks[b];
        uint32_t *row = c.table + (size_t)b * c.max_blocks;
        uint64_t *key = ws.cand + (size_t)b * c.max_blocks * BLK;
        clear_compact_push(c, b, key, nb * BLK, nb, row, row, ws, wave_tot, pool_cnt, top0, sync, epoch,
                           [](uint64_t kk) { return kk != 0 && kk != 2; });
    } else {
        // nothing freed (pool_cnt zero)
        push_publish(c, b, pool_cnt, sync, epoch);
        push_freed(c, b, nullptr, 0, pool_cnt, top0, sync, epoch);
    }
}

}  // namespace

bool launch_evict(const kvq_cache &c, const float *importance, const int32_t *keep_k, int q_window,
                  int recent_window, void *ws_ptr, hipStream_t s) {
    EvictWs ws(ws_ptr, c);
    SyncWs sync(ws_ptr, c);
    hipLaunchKernelGGL(evict_keys, dim3(xcd_grid(KEY_WGS, c.B)), dim3(KEY_THREADS), 0, s, c, importance, q_window,
                       recent_window, ws);
    hipLaunchKernelGGL(evict_select, dim3(c.B), dim3(SEL_THREADS), 0, s, c, keep_k, ws, sync);
    return hipGetLastError() == hipSuccess;
}

bool launch_evict_tbe(const kvq_cache &c, const float *importance, const uint8_t *seq_mask, int r0, int r_min,
                      int t_keep, int q_window, int recent_window, void *ws_ptr, hipStream_t s) {
    EvictWs ws(ws_ptr, c);
    hipLaunchKernelGGL(evict_tbe_prep, dim3(c.B), dim3(SEL_THREADS), 0, s, c, importance, seq_mask, r0, r_min,
                       t_keep, q_window, recent_window, ws);
    hipLaunchKernelGGL(evict_seg_drop, dim3(xcd_grid(DROP_WGS, c.B)), dim3(DROP_THREADS), 0, s, c, ws);
    hipLaunchKernelGGL(evict_seg_compact, dim3(c.B), dim3(SEL_THREADS), 0, s, c, ws, SyncWs(ws_ptr, c));
    return hipGetLastError() == hipSuccess;
}

bool launch_evict_tam(const kvq_cache &c, const float *score, const int32_t *keep_k, float pivot_c,
                      int min_seg, int q_window, int recent_window, void *ws_ptr, hipStream_t s) {
    EvictWs ws(ws_ptr, c);
    hipLaunchKernelGGL(evict_tam_prep, dim3(c.B), dim3(SEL_THREADS), 0, s, c, score, keep_k, pivot_c, min_seg,
                       q_window, recent_window, ws);
    hipLaunchKernelGGL(evict_seg_drop, dim3(xcd_grid(DROP_WGS, c.B)), dim3(DROP_THREADS), 0, s, c, ws);
    hipLaunchKernelGGL(evict_seg_compact, dim3(c.B), dim3(SEL_THREADS), 0, s, c, ws, SyncWs(ws_ptr, c));
    return hipGetLastError() == hipSuccess;
}

}  // namespace kvq
