// kvq_api.hip -- the extern "C" entry points declared in include/kvq.h:
// host-side argument checks, workspace sizing, and kernel dispatch.  No
// allocation, no synchronisation: every call only enqueues work on `stream`.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kvq_internal.h"

namespace {

kvq_status check_cache(const kvq_cache *c) {
    if (!c) return KVQ_EINVAL;
    if (c->head_dim != KVQ_HEAD_DIM) return KVQ_EUNSUPPORTED;
    if (c->B < 1 || c->Hkv < 1 || c->Hq < 1 || c->Hq % c->Hkv != 0) return KVQ_EINVAL;
    if (c->Hq / c->Hkv > KVQ_MAX_GQA || c->Hq > 256 || c->B > 1024) return KVQ_EUNSUPPORTED;
    if (c->max_blocks < 1 || c->n_cap < 1) return KVQ_EINVAL;
    if (c->codec != KVQ_CODEC_INT && c->codec != KVQ_CODEC_NATIVE) return KVQ_EINVAL;
    for (int p = 0; p < 3; ++p) {
        if (c->pool_blocks[p] < 0 || c->pool_blocks[p] >= (1 << 30)) return KVQ_EINVAL;
        if (c->pool_blocks[p] > 0 && (!c->kv[p] || !c->mask[p] || !c->pos[p] || !c->free_ids[p]))
            return KVQ_EINVAL;
    }
    if (!c->table || !c->n_blocks || !c->seq_len || !c->free_top || !c->status) return KVQ_EINVAL;
    return KVQ_OK;
}

// each call checks the workspace against its own need
kvq_status check_ws(const void *ws, size_t bytes, size_t need) {
    if (!ws || (reinterpret_cast<uintptr_t>(ws) & 255) != 0) return KVQ_EINVAL;
    return bytes >= need ? KVQ_OK : KVQ_EINVAL;
}

}  // namespace

extern "C" size_t kvq_region_bytes(int pool) {
    if (pool < 0 || pool > 2) return 0;
    return 512u * (8u >> pool) + 512u;
}

extern "C" size_t kvq_workspace_bytes(const kvq_cache *c) {
    if (check_cache(c) != KVQ_OK) return 0;
    return std::max({kvq::AppendWs::bytes(*c), kvq::DecodeWs::bytes(*c), kvq::EvictWs::bytes(*c)});
}

extern "C" size_t kvq_decode_workspace_bytes(const kvq_cache *c) {
    if (check_cache(c) != KVQ_OK) return 0;
    return kvq::DecodeWs::bytes(*c);
}

extern "C" kvq_status kvq_append_quantize(const kvq_cache *c, const void *k_new, const void *v_new,
                                          const uint8_t *tags, void *ws, size_t ws_bytes,
                                          hipStream_t stream) {
    kvq_status st = check_cache(c);
    if (st != KVQ_OK) return st;
    if (!k_new || !v_new || !tags) return KVQ_EINVAL;
    if ((st = check_ws(ws, ws_bytes, kvq::AppendWs::bytes(*c))) != KVQ_OK) return st;
    return kvq::launch_append(*c, k_new, v_new, tags, ws, stream) ? KVQ_OK : KVQ_EHIP;
}

extern "C" kvq_status kvq_append_quantize_noalloc(const kvq_cache *c, const void *k_new,
                                                  const void *v_new, const uint8_t *tags,
                                                  hipStream_t stream) {
    kvq_status st = check_cache(c);
    if (st != KVQ_OK) return st;
    if (!k_new || !v_new || !tags) return KVQ_EINVAL;
    if (kvq::AppendWs::bytes(*c) > kvq::APPEND_SCRATCH_BYTES) return KVQ_EUNSUPPORTED;
    void *ws = kvq::append_scratch();
    if (!ws) return KVQ_EHIP;
    return kvq::launch_append(*c, k_new, v_new, tags, ws, stream) ? KVQ_OK : KVQ_EHIP;
}

extern "C" kvq_status kvq_decode_attention(const kvq_cache *c, const void *q, float *out,
                                           float *mass, float *importance, float decay,
                                           float sm_scale, void *ws, size_t ws_bytes,
                                           hipStream_t stream) {
    kvq_status st = check_cache(c);
    if (st != KVQ_OK) return st;
    if (!q || !out || !mass) return KVQ_EINVAL;
    if ((st = check_ws(ws, ws_bytes, kvq::DecodeWs::bytes(*c))) != KVQ_OK) return st;
    return kvq::launch_decode(*c, q, out, mass, importance, decay, sm_scale, ws, stream) ? KVQ_OK
                                                                                         : KVQ_EHIP;
}

extern "C" kvq_status kvq_evict_topk(const kvq_cache *c, const float *importance,
                                     const int32_t *keep_k, int32_t q_window,
                                     int32_t recent_window, void *ws, size_t ws_bytes,
                                     hipStream_t stream) {
    kvq_status st = check_cache(c);
    if (st != KVQ_OK) return st;
    if (!importance || !keep_k || q_window < 0 || recent_window < 0) return KVQ_EINVAL;
    if ((st = check_ws(ws, ws_bytes, kvq::EvictWs::bytes(*c))) != KVQ_OK) return st;
    return kvq::launch_evict(*c, importance, keep_k, q_window, recent_window, ws, stream) ? KVQ_OK
                                                                                           : KVQ_EHIP;
}

extern "C" kvq_status kvq_evict_tbe(const kvq_cache *c, const float *importance, const uint8_t *seq_mask,
                                    int32_t r0, int32_t r_min, int32_t t_keep, int32_t q_window,
                                    int32_t recent_window, void *ws, size_t ws_bytes,
                                    hipStream_t stream) {
    kvq_status st = check_cache(c);
    if (st != KVQ_OK) return st;
    if (!importance || r0 < 0 || r_min < 0 || t_keep < 0 || q_window < 0 || recent_window < 0)
        return KVQ_EINVAL;
    if ((st = check_ws(ws, ws_bytes, kvq::EvictWs::bytes(*c))) != KVQ_OK) return st;
    return kvq::launch_evict_tbe(*c, importance, seq_mask, r0, r_min, t_keep, q_window, recent_window, ws,
                                  stream)
               ? KVQ_OK
               : KVQ_EHIP;
}

extern "C" kvq_status kvq_evict_tam(const kvq_cache *c, const float *score, const int32_t *keep_k,
                                    float pivot_c, int32_t min_seg, int32_t q_window,
                                    int32_t recent_window, void *ws, size_t ws_bytes,
                                    hipStream_t stream) {
    kvq_status st = check_cache(c);
    if (st != KVQ_OK) return st;
    if (!score || !keep_k || !(pivot_c >= 0.0f) || min_seg < 1 || q_window < 0 || recent_window < 0)
        return KVQ_EINVAL;
    if ((st = check_ws(ws, ws_bytes, kvq::EvictWs::bytes(*c))) != KVQ_OK) return st;
    return kvq::launch_evict_tam(*c, score, keep_k, pivot_c, min_seg, q_window, recent_window, ws, stream)
               ? KVQ_OK
               : KVQ_EHIP;
}
