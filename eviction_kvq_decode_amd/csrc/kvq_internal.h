// kvq_internal.h -- host-side contract between the C ABI and the kernels.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

// Decode split-K: a run (split) covers at most this many table entries of
// one sequence and kv-head pack (a sequence with nr runs gives run j the
// entries j, j + nr, j + 2 nr, ...).  The decode shortens the runs when the
// batch leaves workgroups idle, down to MIN_RUN entries for a sequence that
// fills its table, so a sequence has at most n_splits runs.
#ifndef KVQ_ENTRIES_PER_SPLIT
#define KVQ_ENTRIES_PER_SPLIT 64
#endif
constexpr int ENTRIES_PER_SPLIT = KVQ_ENTRIES_PER_SPLIT;
constexpr int MIN_RUN = 16;

inline int n_splits(const kvq_cache &c) { return (c.max_blocks + MIN_RUN - 1) / MIN_RUN; }

// Score groups (of 16 slots) reserved per sequence and kv-head pack: runs
// of E entries each take E groups at E-group offsets, like any run layout
// up to max_blocks + n_splits groups (see run_stride); rounded up to E.
inline int score_span(const kvq_cache &c) {
    const int e64 = (c.max_blocks + ENTRIES_PER_SPLIT - 1) / ENTRIES_PER_SPLIT * ENTRIES_PER_SPLIT;
    return (e64 + n_splits(c) + ENTRIES_PER_SPLIT - 1) / ENTRIES_PER_SPLIT * ENTRIES_PER_SPLIT;
}

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace carve-up.  Calls are stream-ordered, so they share one buffer.
struct AppendWs {
    int32_t *need;     // [B] -2 nothing, -1 reuse slot, p >= 0 pop pool p
    int32_t *entry;    // [B] table entry (pool << 30 | id) of the reused block
    int32_t *slot;     // [B]
    int32_t *top;      // [4] free_top before the call
    static size_t bytes(const kvq_cache &c) { return align256(16 * 4) + 3 * align256(4L * c.B); }
    AppendWs(void *ws, const kvq_cache &c) {
        char *p = (char *)ws;
        top = (int32_t *)p;   p += align256(16 * 4);
        need = (int32_t *)p;  p += align256(4L * c.B);
        entry = (int32_t *)p; p += align256(4L * c.B);
        slot = (int32_t *)p;
    }
};

// The no-allocation append keeps AppendWs in a static device array of this
// size: enough for every batch the library accepts (B <= 1024).
constexpr size_t APPEND_SCRATCH_BYTES = 16384;
// Its device address on the current device (looked up once per device), or
// null if the lookup failed.
void *append_scratch();

// kv heads whose query heads share one 16-column MFMA tile in decode
inline int decode_pack(int G) { return 16 / G < 4 ? 16 / G : 4; }
inline int decode_n_packs(const kvq_cache &c) {
    const int P = decode_pack(c.Hq / c.Hkv);
    return (c.Hkv + P - 1) / P;
}

struct DecodeWs {
    float *ml;         // [B][Hq][S][2]  split max (base-2 units), split sum
    float *o;          // [B][Hq][S][128] split output, unnormalised
    // The valid slots of a run, in table and slot order, are numbered
    // 0 .. n-1 (n <= 16 x its entries); their scores and positions are
    // stored compacted in groups of 16, run j of a sequence from group
    // j * st (st: the run stride, at least the entries of any of its runs).
    int32_t *ents;     // [B][S] valid slots n of the run
    int32_t *run_len;  // [1] most entries per run, chosen by the split kernel
    int32_t *spos;     // [B][span][16] position of valid slot c at [j st + c / 16][c % 16]
    float *score;      // [B][span][n_packs][16 heads][16]: the base-2 scaled score
                       // of valid slot c of pack p at group (j st) n_packs + p st +
                       // c / 16, [head][c % 16] (a run's packs adjacent)
    static size_t bytes(const kvq_cache &c) {
        const size_t S = n_splits(c), SP = score_span(c);
        return align256(8L * c.B * c.Hq * S) + align256(512L * c.B * c.Hq * S) + align256(4L * c.B * S) +
               align256(4) + align256(64L * c.B * SP) + align256(1024L * c.B * SP * decode_n_packs(c));
    }
    DecodeWs(void *ws, const kvq_cache &c) {
        const size_t S = n_splits(c), SP = score_span(c);
        char *p = (char *)ws;
        ml = (float *)p;      p += align256(8L * c.B * c.Hq * S);
        o = (float *)p;       p += align256(512L * c.B * c.Hq * S);
        ents = (int32_t *)p;  p += align256(4L * c.B * S);
        run_len = (int32_t *)p; p += align256(4);
        spos = (int32_t *)p;  p += align256(64L * c.B * SP);
        score = (float *)p;
    }
};

constexpr int EVICT_KEY_WGS = 8;   // workgroups per sequence building top-k's slot keys

struct EvictWs {
    uint64_t *cand;    // [B][max_blocks*16] selection keys, one word per slot
    int32_t *kcnt;     // [B][EVICT_KEY_WGS] candidates per part of a row (top-k)
    uint32_t *freed;   // [B][max_blocks] freed table entries, table order
    int32_t *nfreed;   // [B][4] freed per pool
    int32_t *top;      // [4] free_top before the call
    // segment-granular eviction only: candidates in position order
    uint32_t *pmap;    // [B][n_cap] (pool << 30) | slot of the candidate at a position, or ~0
    int32_t *ord;      // [B][max_blocks*16] (pool << 30) | slot of the candidates, by position
    uint32_t *ob;      // [B][max_blocks*16] their importance as order bits (0: never dropped)
    uint32_t *sfx;     // [B][max_blocks*16] their window score in fixed point (budgets)
    int32_t *segstart; // [B][max_blocks*16 + 1] first candidate of each segment
    int32_t *segtc;    // [B][max_blocks*16] Transition segments up to and including each segment
    int32_t *segkeep;  // [B][max_blocks*16] how many droppable candidates each segment keeps
    uint64_t *sega;    // [B][max_blocks*16] budget weight of each segment
    int32_t *segm;     // [B][max_blocks*16] droppable candidates of each segment (-m-1: capped)
    uint64_t *psum;    // [B][max_blocks*16 + 1] running sum of sfx before each candidate
    int32_t *pcnt;     // [B][max_blocks*16 + 1] droppable candidates before each candidate
    int32_t *segn;     // [B][2] segments, Transition segments
    static size_t bytes(const kvq_cache &c) {
        const size_t ms = (size_t)c.max_blocks * 16, slot4 = align256(4L * c.B * ms);
        return align256(8L * c.B * ms) + align256(4L * EVICT_KEY_WGS * c.B) + align256(4L * c.B * c.max_blocks) +
               align256(16L * c.B) +
               align256(16) + align256(4L * c.B * c.n_cap) + 3 * slot4 + align256(4L * c.B * (ms + 1)) +
               2 * slot4 + align256(8L * c.B * ms) + slot4 + align256(8L * c.B * (ms + 1)) +
               align256(4L * c.B * (ms + 1)) + align256(8L * c.B);
    }
    EvictWs(void *ws, const kvq_cache &c) {
        const size_t ms = (size_t)c.max_blocks * 16, slot4 = align256(4L * c.B * ms);
        char *p = (char *)ws;
        cand = (uint64_t *)p;     p += align256(8L * c.B * ms);
        kcnt = (int32_t *)p;      p += align256(4L * EVICT_KEY_WGS * c.B);
        freed = (uint32_t *)p;    p += align256(4L * c.B * c.max_blocks);
        nfreed = (int32_t *)p;    p += align256(16L * c.B);
        top = (int32_t *)p;       p += align256(16);
        pmap = (uint32_t *)p;     p += align256(4L * c.B * c.n_cap);
        ord = (int32_t *)p;       p += slot4;
        ob = (uint32_t *)p;       p += slot4;
        sfx = (uint32_t *)p;      p += slot4;
        segstart = (int32_t *)p;  p += align256(4L * c.B * (ms + 1));
        segtc = (int32_t *)p;     p += slot4;
        segkeep = (int32_t *)p;   p += slot4;
        sega = (uint64_t *)p;     p += align256(8L * c.B * ms);
        segm = (int32_t *)p;      p += slot4;
        psum = (uint64_t *)p;     p += align256(8L * c.B * (ms + 1));
        pcnt = (int32_t *)p;      p += align256(4L * c.B * (ms + 1));
        segn = (int32_t *)p;
    }
};

// Launchers (one per kernel file); return false if a launch failed.
bool launch_append(const kvq_cache &c, const void *k_new, const void *v_new, const uint8_t *tags,
                   void *ws, hipStream_t s);
bool launch_decode(const kvq_cache &c, const void *q, float *out, float *mass, float *importance,
                   float decay, float sm_scale, void *ws, hipStream_t s);
bool launch_evict(const kvq_cache &c, const float *importance, const int32_t *keep_k, int q_window,
                  int recent_window, void *ws, hipStream_t s);
bool launch_evict_tbe(const kvq_cache &c, const float *importance, int r0, int r_min, int t_keep,
                      int q_window, int recent_window, void *ws, hipStream_t s);
bool launch_evict_tam(const kvq_cache &c, const float *score, const int32_t *keep_k, float pivot_c,
                      int min_seg, int q_window, int recent_window, void *ws, hipStream_t s);

}  // namespace kvq
