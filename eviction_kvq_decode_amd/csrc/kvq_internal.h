// kvq_internal.h -- host-side contract between the C ABI and the kernels.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "kvq.h"

namespace kvq {

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace carve-up.  Calls are stream-ordered, so they share one buffer.
//
// Its first SyncWs::bytes belong to the calls that rank work across
// workgroups in batch order (append's pops, eviction's pushes) and no other
// call writes them: the epoch of the last such call, then one word per pool
// and sequence, (epoch << 32) | count, of the call that wrote it.  A call
// takes epoch + 1 (never 0), so words of earlier calls and zeroed memory
// never pass for its own; its last workgroup stores the new epoch once every
// word is in.  The region must be zero before the first call.
struct SyncWs {
    uint32_t *epoch;           // [1] epoch of the last call that ended
    unsigned long long *words; // [3][B] per pool, per sequence
    static size_t bytes(const kvq_cache &c) { return 256 + align256(24L * c.B); }
    SyncWs(void *ws, const kvq_cache &c) {
        epoch = (uint32_t *)ws;
        words = (unsigned long long *)((char *)ws + 256);
    }
};

// The append needs nothing beyond the sync words.
using AppendWs = SyncWs;

// The no-allocation append keeps AppendWs in a static device array of this
// size: enough for every batch the library accepts (B <= 1024).
constexpr size_t APPEND_SCRATCH_BYTES = 32768;
// Its device address on the current device (looked up once per device), or
// null if the lookup failed.
void *append_scratch();

// kv heads whose query heads share one 16-column MFMA tile in decode
inline int decode_pack(int G) { return 16 / G < 4 ? 16 / G : 4; }
inline int decode_n_packs(const kvq_cache &c) {
    const int P = decode_pack(c.Hq / c.Hkv);
    return (c.Hkv + P - 1) / P;
}

// The decode split kernel's grid holds at most this many workgroups.  Each
// takes a contiguous range of the flat (sequence, kv-head pack, table entry)
// list and writes one partial per (sequence, pack) unit its range touches,
// in slot (workgroup + unit): fewer than MAX_SPLIT_WGS + B * n_packs slots.
constexpr int MAX_SPLIT_WGS = 1024;

struct DecodeWs {
    float *ml;         // [slots][16 heads][2] segment max (base-2 units) and sum
    float *o;          // [slots][16 heads][128] segment output, unnormalised
    float *score;      // [B][n_packs][max_blocks][16 slots][16 heads]: the base-2
                       // scaled scores of table entry e (-inf at cleared slots),
                       // written by the split kernel, read by the finalize
    int32_t *pre;      // [B + 1] where each sequence's entries start in the split
                       // kernel's flat list (n_packs x the entries before it); [B]: N
    int32_t *rstart;   // [grid + 1] where each split workgroup's range of that list
                       // starts; [grid]: N
    static size_t slots(const kvq_cache &c) { return MAX_SPLIT_WGS + (size_t)c.B * decode_n_packs(c); }
    static size_t bytes(const kvq_cache &c) {
        const size_t S = slots(c);
        return SyncWs::bytes(c) + align256(4L * (c.B + 1)) + align256(4L * (MAX_SPLIT_WGS + 1)) +
               align256(128L * S) + align256(8192L * S) + align256(1024L * c.B * c.max_blocks * decode_n_packs(c));
    }
    DecodeWs(void *ws, const kvq_cache &c) {
        const size_t S = slots(c);
        char *p = (char *)ws + SyncWs::bytes(c);
        pre = (int32_t *)p;   p += align256(4L * (c.B + 1));
        rstart = (int32_t *)p; p += align256(4L * (MAX_SPLIT_WGS + 1));
        ml = (float *)p;      p += align256(128L * S);
        o = (float *)p;       p += align256(8192L * S);
        score = (float *)p;
    }
};

constexpr int EVICT_KEY_WGS = 8;   // workgroups per sequence building top-k's slot keys
constexpr int EVICT_RADIX = 2048;  // bins of top-k's radix select (11-bit digits)

struct EvictWs {
    uint64_t *cand;    // [B][max_blocks*16] selection keys, one word per slot
    int32_t *kcnt;     // [B][EVICT_KEY_WGS] candidates per part of a row (top-k)
    uint32_t *khist;   // [B][EVICT_KEY_WGS][EVICT_RADIX] per part, candidates by their key's top 11 bits
    uint32_t *freed;   // [B][max_blocks] freed table entries, table order
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
    int32_t *segn;     // [B][2] segments (-1: the sequence is left as it is), Transition segments
    static size_t bytes(const kvq_cache &c) {
        const size_t ms = (size_t)c.max_blocks * 16, slot4 = align256(4L * c.B * ms);
        return SyncWs::bytes(c) + align256(8L * c.B * ms) + align256(4L * EVICT_KEY_WGS * c.B) +
               align256(4L * EVICT_KEY_WGS * EVICT_RADIX * c.B) +
               align256(4L * c.B * c.max_blocks) + align256(4L * c.B * c.n_cap) + 3 * slot4 + align256(4L * c.B * (ms + 1)) +
               2 * slot4 + align256(8L * c.B * ms) + slot4 + align256(8L * c.B * (ms + 1)) +
               align256(4L * c.B * (ms + 1)) + align256(8L * c.B);
    }
    EvictWs(void *ws, const kvq_cache &c) {
        const size_t ms = (size_t)c.max_blocks * 16, slot4 = align256(4L * c.B * ms);
        char *p = (char *)ws + SyncWs::bytes(c);
        cand = (uint64_t *)p;     p += align256(8L * c.B * ms);
        kcnt = (int32_t *)p;      p += align256(4L * EVICT_KEY_WGS * c.B);
        khist = (uint32_t *)p;    p += align256(4L * EVICT_KEY_WGS * EVICT_RADIX * c.B);
        freed = (uint32_t *)p;    p += align256(4L * c.B * c.max_blocks);
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
bool launch_evict_tbe(const kvq_cache &c, const float *importance, const uint8_t *seq_mask, int r0, int r_min,
                      int t_keep, int q_window, int recent_window, void *ws, hipStream_t s);
bool launch_evict_tam(const kvq_cache &c, const float *score, const int32_t *keep_k, float pivot_c,
                      int min_seg, int q_window, int recent_window, void *ws, hipStream_t s);

}  // namespace kvq
