/*
 * kvq.h -- C ABI of libkvq: decode attention over a paged KV cache whose
 * tokens are stored at 8, 4 or 2 bits according to their thought type, with
 * evicted slots reused in place, on AMD Instinct MI355X (gfx950).
 *
 * The method (web pages, cited by title and section):
 *  - "ThinKV: Thought-Adaptive KV Cache Compression for Efficient Reasoning
 *    Models", Methodology, "Thought-Adaptive Quantization (TBQ)": each token's
 *    K/V precision follows its thought type (Reasoning > Execution >
 *    Transition), by group quantisation.
 *  - same page, Methodology, "System Implementation: Continuous Thinking":
 *    a PagedAttention-style block table that records thought type and an
 *    eviction mask; new tokens of the same type overwrite evicted slots in
 *    place; no gather compaction.
 *  - "Dynamic Thinking-Token Selection ...", section 2.3: question window,
 *    local window, and top-k by importance inside the selection window.
 *  - "Thought-Aware KV Cache Compaction ... (TAM)", sections 1 and 2.B, and
 *    "Back from the Future ...", Problem Statement: the attention mass a
 *    token receives (H2O-style cumulative score) is the importance signal;
 *    attention itself is scaled dot-product attention over the cache.
 *
 * Conventions for every call:
 *  - All pointers are DEVICE pointers owned by the caller, except the
 *    kvq_cache struct itself, which is read on the host during the call.
 *    The library never allocates, frees or synchronises; all work is
 *    enqueued on `stream` and returns immediately.
 *  - A host-detectable problem (null pointer, unsupported shape, workspace
 *    too small) returns an error and enqueues nothing.  A failed launch
 *    returns KVQ_EHIP.  Data-dependent problems found on the device (a pool
 *    or table full, a bad tag) store a negative kvq_status into *status and
 *    leave the affected sequence unchanged; the library never clears
 *    *status.
 *  - Calls on one cache must be ordered on one stream; calls on disjoint
 *    caches may run concurrently.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KVQ_OK = 0,
    KVQ_EINVAL = -1,       /* bad argument                          */
    KVQ_EUNSUPPORTED = -2, /* shape outside what the kernels handle */
    KVQ_EHIP = -3,         /* a HIP launch failed                   */
    KVQ_ENOSPC = -4        /* pool, table or position space full    */
} kvq_status;

enum { KVQ_HEAD_DIM = 128, KVQ_BLOCK = 16, KVQ_GROUP = 32, KVQ_MAX_GQA = 16 };

/* Thought types; the pool index equals the tag.  R -> 8 bit, E -> 4 bit,
 * T -> 2 bit ("ThinKV", TBQ: precision ordered R > E > T). */
enum { KVQ_TAG_R = 0, KVQ_TAG_E = 1, KVQ_TAG_T = 2, KVQ_TAG_NONE = 255 };

/*
 * Codecs ("ThinKV", Methodology, TBQ: precision by thought type), chosen per
 * cache in kvq_cache.codec; both keep the same code widths and layout:
 *   KVQ_CODEC_INT    asymmetric integer codes per group of 32 channels:
 *                    zero = group min, scale = least fp16 >= (max-min) /
 *                    (2^b - 1), code = rint((x - zero) / scale);
 *   KVQ_CODEC_NATIVE ThinKV's own formats, symmetric per group of 32 with
 *                    scale = least fp16 >= max|x| / top: Reasoning rows hold
 *                    OCP E4M3 codes of x / scale (top 448), Execution rows
 *                    E2M1 codes (top 6), both nearest with ties to even and
 *                    zero = 0, dequantised as value(code) * scale; Transition
 *                    rows hold t + 1 for t = rint(x / scale) in [-1, 1]
 *                    (top 1) with zero = -scale, dequantised as code * scale
 *                    + zero (ternary).
 */
enum { KVQ_CODEC_INT = 0, KVQ_CODEC_NATIVE = 1 };

/*
 * The cache.  One pool per bit width; a block holds 16 slots of one thought
 * type.  For pool p (bits b = 8 >> p) and block id, kv head h, the region at
 *     kv[p] + (id * Hkv + h) * kvq_region_bytes(p)
 * holds, in order:
 *     K codes  256*b bytes : token t's K row is 16*b contiguous bytes at t*16*b;
 *                            channel d = 32g + 8k + e sits at code index
 *                            (b=8) 32k + 8g + e, (b=4) 32k + 8g + 4(e&1) + (e>>1),
 *                            (b=2) 32k + 16(g>>1) + 8(e&1) + 4(g&1) + (e>>1)
 *     V codes  256*b bytes : tiles for a 16x16x16 MFMA; for token t = 4r + u
 *                            and channel d = 16n + j, lane L = 16r + j owns
 *                            dword w = n*b/8 of a slice at byte
 *                            (b=8) (w>>2)*1024 + 16L + 4(w&3), (b=4) 16L + 4w,
 *                            (b=2) 8L + 4w; inside it the code sits at slot
 *                            (u&1)*(16/b) + 2*(n mod 8/b) + (u>>1)
 *     K (scale, zero) 256 B: fp16 pair for token t, group g at (t*4 + g)*4
 *     V (scale, zero) 256 B: same layout
 * Codes are packed LSB first.  A dequantised value is code * scale + zero
 * (KVQ_CODEC_NATIVE, Reasoning and Execution rows: value(code) * scale).
 * Bytes of slots whose mask bit is clear are unspecified.
 *
 * table[b * max_blocks + e] = (pool << 30) | id, for e < n_blocks[b], in
 * logical order.  pos[p][id * 16 + s] is the logical position held by slot
 * s of block id (meaningful where mask bit s is set).  free_ids[p][0 ..
 * free_top[p]) is pool p's stack of unused block ids; pops take the top.
 */
typedef struct kvq_cache {
    int32_t B;            /* sequences                                   */
    int32_t Hq;           /* query heads                                 */
    int32_t Hkv;          /* kv heads; Hq % Hkv == 0, Hq/Hkv <= 16       */
    int32_t head_dim;     /* must be 128                                 */
    int32_t max_blocks;   /* table row capacity per sequence             */
    int32_t n_cap;        /* row stride (positions) of mass / importance */
    int32_t pool_blocks[3];
    int32_t codec;        /* KVQ_CODEC_INT or KVQ_CODEC_NATIVE           */
    uint8_t *kv[3];       /* [pool_blocks][Hkv] regions                  */
    uint16_t *mask[3];    /* [pool_blocks] valid-slot bitmask            */
    int32_t *pos[3];      /* [pool_blocks][16]                           */
    uint32_t *table;      /* [B][max_blocks]                             */
    int32_t *n_blocks;    /* [B]                                         */
    int32_t *seq_len;     /* [B] next logical position                   */
    uint32_t *free_ids[3];/* [pool_blocks]                               */
    int32_t *free_top;    /* [3]                                         */
    int32_t *status;      /* [1] device error word                       */
} kvq_cache;

/* Bytes of one (block, kv head) region of pool p (0, 1, 2): 512*b + 512. */
size_t kvq_region_bytes(int pool);

/* Workspace bytes that every call below needs for this cache, so that one
 * buffer serves them all (device memory, 256-byte aligned; calls ordered on
 * one stream may share it).  0 if the cache description is rejected.
 * Zero-fill a workspace once, before its first call; from then on its
 * contents belong to the library (do not write it between calls).  Its
 * first bytes hold what the append and the evictions use to rank pops and
 * pushes across sequences in batch order within one launch: the epoch of
 * the last such call and, per pool and sequence, a count tagged with the
 * epoch of the call that wrote it.  Each call takes the next epoch on the
 * device, so the calls also work when captured in a graph and replayed. */
size_t kvq_workspace_bytes(const kvq_cache *cache);

/* Workspace bytes kvq_decode_attention needs for this cache (a buffer this
 * size serves the decode alone; <= kvq_workspace_bytes).  It holds the split
 * partials (max, sum, output per head), the base-2 scores of every table
 * entry's slots for the mass pass, the sequence prefix of the work list and
 * where each split workgroup's part of it starts.
 * 0 if the cache description is rejected. */
size_t kvq_decode_workspace_bytes(const kvq_cache *cache);

/*
 * Append one token per sequence ("ThinKV", TBQ and Continuous Thinking).
 *   k_new, v_new : fp16 [B][Hkv][128]
 *   tags         : uint8 [B]; KVQ_TAG_R/E/T, or KVQ_TAG_NONE to skip b
 * Per kv head and per 32-channel group, K and V are quantised to b bits:
 * zero = group min, scale = least fp16 >= (max - min)/(2^b - 1) (fp32),
 * code = clamp(rint((x - zero)/scale), 0, 2^b - 1) (fp32, ties to even).
 * The token goes to the first free slot of a block of its own type, in table
 * order then slot order; otherwise a block is popped from that pool's free
 * stack (sequences served in batch order) and appended to the table.  It
 * gets position seq_len[b], which then grows by one.  Sequences that cannot
 * be served (pool empty, table full, seq_len == n_cap) set *status =
 * KVQ_ENOSPC and are left unchanged; a tag > 2 sets KVQ_EINVAL.
 */
kvq_status kvq_append_quantize(const kvq_cache *cache, const void *k_new, const void *v_new,
                               const uint8_t *tags, void *workspace, size_t workspace_bytes,
                               hipStream_t stream);

/*
 * kvq_append_quantize without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same semantics and kernel; the words
 * that rank pops across sequences in batch order (an epoch, and one tagged
 * count per pool and sequence) live in a static device array of the library
 * (32 KiB per GPU, zero when the library loads, held until the process
 * ends), enough for every B the library accepts (<= 1024).  The words carry
 * the epoch of the call that wrote them, so nothing is cleared between calls.
 * A cache whose words would not fit returns KVQ_EUNSUPPORTED.  Nothing
 * is allocated or freed.  Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (concurrent streams) race and must not be
 * issued; calls ordered on one stream are safe.
 */
kvq_status kvq_append_quantize_noalloc(const kvq_cache *cache, const void *k_new, const void *v_new,
                                       const uint8_t *tags, hipStream_t stream);

/*
 * Decode attention for one query token per sequence ("Back from the
 * Future", Problem Statement: scaled dot-product attention over the cache),
 * plus the per-position attention mass ("TAM", sections 1 and 2.B).
 *   q          : fp16 [B][Hq][128]
 *   out        : fp32 [B][Hq][128] = sum_t p_ht * v_t over valid slots of the
 *                sequence, p = softmax(sm_scale * q_h . k_t); query head h
 *                reads kv head h / (Hq / Hkv).  Zero if no slot is valid.
 *   mass       : fp32 [B][n_cap]; for positions < seq_len[b]:
 *                sum over all Hq heads of p_ht for the slot holding the
 *                position, 0 if no valid slot holds it.  Other entries are
 *                not written.
 *   importance : fp32 [B][n_cap] or NULL; at valid positions
 *                importance = decay * importance + mass (H2O-style
 *                cumulative score); other entries are not touched.
 */
kvq_status kvq_decode_attention(const kvq_cache *cache, const void *q, float *out, float *mass,
                                float *importance, float decay, float sm_scale, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * Windowed top-k eviction ("Dynamic Thinking-Token Selection ...", 2.3) with
 * metadata-only compaction ("ThinKV", Continuous Thinking).
 *   importance : fp32 [B][n_cap], read at the positions of valid slots
 *                (finite values; -0 counts as +0)
 *   keep_k     : int32 [B]
 * Per sequence, valid slots with position < q_window or >= seq_len -
 * recent_window are kept; of the others, the keep_k with the largest
 * importance (ties: lower position) are kept and the rest are evicted
 * (mask bit cleared; the bytes stay in place).  Then every table entry whose
 * mask is empty is removed from the table, order kept, and its id pushed on
 * its pool's free stack, in table order, sequences in batch order.
 */
kvq_status kvq_evict_topk(const kvq_cache *cache, const float *importance, const int32_t *keep_k,
                          int32_t q_window, int32_t recent_window, void *workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * Thought-adaptive eviction by segment ("ThinKV", Methodology,
 * think-before-evict): once a Transition thought starts, earlier Reasoning
 * and Execution segments are pruned at segment granularity on an annealing
 * schedule, and a small safety net of every earlier Transition segment stays.
 *   importance : fp32 [B][n_cap], read at the positions of valid slots
 *                (finite values; -0 counts as +0)
 *   seq_mask   : uint8 [B] or NULL; a sequence with seq_mask[b] == 0 is left
 *                exactly as it is (no eviction, no compaction): the caller
 *                fires the eviction only for the sequences in which a
 *                Transition thought was detected.  NULL: every sequence.
 *   r0, r_min, t_keep : >= 0
 * Per sequence, the valid slots with q_window <= pos < seq_len -
 * recent_window are the candidates; the others are kept.  In position order
 * the candidates form segments: maximal runs of one thought type.  A segment
 * followed by k Transition segments keeps all its slots if k == 0;
 * otherwise it keeps max(r_min, r0 >> (k - 1)) slots if it is a Reasoning or
 * Execution segment (r0, r0 / 2, r0 / 4, ... as Transitions follow) and
 * t_keep slots if it is a Transition segment.  A segment keeps its slots of
 * largest importance (ties: lower position).  The rest are evicted, and the
 * table is compacted and emptied blocks are freed as in kvq_evict_topk (pushes
 * ranked over the sequences in the mask, in batch order).
 */
kvq_status kvq_evict_tbe(const kvq_cache *cache, const float *importance, const uint8_t *seq_mask,
                         int32_t r0, int32_t r_min, int32_t t_keep, int32_t q_window,
                         int32_t recent_window, void *workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * Thought-aware segment budgets ("Thought-Aware KV Cache Compaction for
 * Reasoning via Adaptive Attention Matching (TAM)", section 2: A thought
 * segmentation, B adaptive budget allocation, C pivotal-token protection),
 * with compaction read as keeping a subset of the cached tokens.
 *   score   : fp32 [B][n_cap], the attention mass each position received
 *             from the selection window (the R most recent queries; e.g.
 *             the importance accumulated by R decode calls with decay 1
 *             from zero), read at the positions of valid slots; taken in
 *             fixed point s = floor(score * 2^16) for 0 < score < 2^16,
 *             2^32 - 1 above, 0 for score <= 0
 *   keep_k  : int32 [B] token budget per sequence (the windows aside)
 *   pivot_c : >= 0 (+inf: no pivotal tokens)
 *   min_seg : >= 1
 * Per sequence, the valid slots with q_window <= pos < seq_len -
 * recent_window are the candidates; the others are kept.  A candidate is
 * pivotal if s * N > pivot_c * S (in doubles; N candidates, S the sum of
 * their s) and is kept; the budget left, T = max(0, keep_k - pivotal), goes
 * to the others.  In position order the candidates form runs of one thought
 * type; a run of at least min_seg candidates opens a new segment and a
 * shorter run joins the segment before it (the first run always opens one;
 * the pages merge short segments, and the cache's only segment structure is
 * the thought type).  Segment i (n_i candidates, m_i not pivotal, S_i the sum of
 * their s) has weight a_i = isqrt(floor(S_i / n_i) * 2^16) * m_i, that is
 * sqrt(mean score) * m_i.  A segment whose share T' a_i / A reaches m_i
 * (T' the budget left after such segments, A the sum of the others'
 * weights) keeps all m_i, and the shares are recomputed without it until
 * none does; the others keep floor(T' C_j / A) - floor(T' C_(j-1) / A),
 * C_j the running sum of their weights in position order (none if A = 0).
 * A segment keeps its pivotal candidates and that many others of largest
 * score (ties: lower position).  The rest are evicted, and the table is
 * compacted and emptied blocks are freed as in kvq_evict_topk.
 */
kvq_status kvq_evict_tam(const kvq_cache *cache, const float *score, const int32_t *keep_k,
                         float pivot_c, int32_t min_seg, int32_t q_window, int32_t recent_window,
                         void *workspace, size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
