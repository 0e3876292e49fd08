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
constexpr float LOG2E = 1.4426950408889634f;

// Dequantised K code (t, d) and V code (t, d) of a region.
__device__ inline uint32_t k_code(const uint8_t *reg, int bits, int t, int d) {
    const int bit = (t * HD + k_row_index(bits, d)) * bits;
    return (reg[bit >> 3] >> (bit & 7)) & ((1u << bits) - 1);
}
__device__ inline uint32_t v_code(const uint8_t *reg, int bits, int t, int d) {
    const uint8_t *dw = reg + 256 * bits + v_dword_byte(bits, t, d);
    const int bit = v_code_slot(bits, t, d) * bits;
    return (dw[bit >> 3] >> (bit & 7)) & ((1u << bits) - 1);
}

__global__ __launch_bounds__(THREADS) void attn_split(kvq_cache c, const uint16_t *q, float *mass,
                                                      DecodeWs ws, float scale2) {
    const int split = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
    const int S = gridDim.x, G = c.Hq / c.Hkv;
    const int tid = threadIdx.x;

    // Positions of this sequence start at mass 0; the finalize pass adds the
    // valid ones.  All workgroups of the sequence share the fill.
    {
        const int w = split * c.Hkv + kh, W = S * c.Hkv, len = c.seq_len[b];
        for (int p = w * THREADS + tid; p < len; p += W * THREADS) mass[(size_t)b * c.n_cap + p] = 0.f;
    }

    __shared__ float qs[KVQ_MAX_GQA][HD];
    __shared__ float sc[BLK][KVQ_MAX_GQA];
    __shared__ float pb[BLK][KVQ_MAX_GQA];
    __shared__ float m_run[KVQ_MAX_GQA], l_run[KVQ_MAX_GQA], alpha[KVQ_MAX_GQA];
    for (int i = tid; i < G * HD; i += THREADS)
        qs[i / HD][i % HD] = h2f(q[((size_t)b * c.Hq + kh * G) * HD + i]);
    if (tid < G) {
        m_run[tid] = -INFINITY;
        l_run[tid] = 0.f;
    }
    float acc[KVQ_MAX_GQA / 2];
#pragma unroll
    for (int k = 0; k < KVQ_MAX_GQA / 2; ++k) acc[k] = 0.f;
    __syncthreads();

    const int nb = c.n_blocks[b];
    const int e0 = split * E, e1 = min(nb, e0 + E);
    const size_t score_row = (size_t)c.max_blocks * BLK;
    for (int e = e0; e < e1; ++e) {
        const uint32_t ent = c.table[(size_t)b * c.max_blocks + e];
        const int pool = (int)(ent >> 30);
        const uint32_t id = ent & 0x3fffffffu;
        const uint32_t m = c.mask[pool][id];
        if (m == 0) continue;
        const int bits = pool_bits(pool);
        const uint8_t *reg = region_ptr(c.kv[pool], id, c.Hkv, kh, pool);
        const uint32_t *ksz = reinterpret_cast<const uint32_t *>(reg + 512 * bits);
        const uint32_t *vsz = reinterpret_cast<const uint32_t *>(reg + 512 * bits + 256);
        {   // scores: 16 threads per token, 8 channels each
            const int t = tid >> 4, sub = tid & 15, g = sub >> 2;
            const uint32_t sz = ksz[t * NGRP + g];
            const float s = h2f((uint16_t)(sz & 0xffff)), z = h2f((uint16_t)(sz >> 16));
            float kv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) kv[i] = (float)k_code(reg, bits, t, 8 * sub + i) * s + z;
            for (int hh = 0; hh < G; ++hh) {
                float part = 0.f;
#pragma unroll
                for (int i = 0; i < 8; ++i) part += qs[hh][8 * sub + i] * kv[i];
#pragma unroll
                for (int off = 1; off < 16; off <<= 1) part += __shfl_xor(part, off);
                if (sub == 0) sc[t][hh] = part * scale2;
            }
        }
        __syncthreads();
        if (tid < G) {
            float mx = m_run[tid];
            for (int t = 0; t < BLK; ++t)
                if ((m >> t) & 1) mx = fmaxf(mx, sc[t][tid]);
            const float a = exp2f(m_run[tid] - mx);
            float lsum = 0.f;
            for (int t = 0; t < BLK; ++t) {
                const float p = ((m >> t) & 1) ? exp2f(sc[t][tid] - mx) : 0.f;
                pb[t][tid] = p;
                lsum += p;
            }
            l_run[tid] = l_run[tid] * a + lsum;
            m_run[tid] = mx;
            alpha[tid] = a;
        }
        for (int i = tid; i < BLK * G; i += THREADS) {
            const int t = i / G, hh = i % G;
            ws.score[((size_t)b * c.Hq + kh * G + hh) * score_row + (size_t)e * BLK + t] = sc[t][hh];
        }
        __syncthreads();
        {   // PV: thread owns channel d for heads hh = (tid >> 7) + 2k
            const int d = tid & (HD - 1), h0 = tid >> 7;
            for (int k = 0; 2 * k + h0 < G; ++k) acc[k] *= alpha[2 * k + h0];
            const int g = d / GS;
            for (int t = 0; t < BLK; ++t) {
                if (!((m >> t) & 1)) continue;
                const uint32_t sz = vsz[t * NGRP + g];
                const float v = (float)v_code(reg, bits, t, d) * h2f((uint16_t)(sz & 0xffff)) +
                                h2f((uint16_t)(sz >> 16));
                for (int k = 0; 2 * k + h0 < G; ++k) acc[k] += pb[t][2 * k + h0] * v;
            }
        }
        __syncthreads();
    }

    const size_t base = (size_t)b * c.Hq + kh * G;
    if (tid < G) {
        ws.ml[((base + tid) * S + split) * 2 + 0] = m_run[tid];
        ws.ml[((base + tid) * S + split) * 2 + 1] = l_run[tid];
    }
    {
        const int d = tid & (HD - 1), h0 = tid >> 7;
        for (int k = 0; 2 * k + h0 < G; ++k)
            ws.o[((base + 2 * k + h0) * S + split) * HD + d] = acc[k];
    }
}

__global__ __launch_bounds__(THREADS) void attn_finalize(kvq_cache c, float *out, float *mass,
                                                         float *importance, float decay, DecodeWs ws,
                                                         int S) {
    const int chunk = blockIdx.x, b = blockIdx.y, C = gridDim.x;
    const int tid = threadIdx.x;
    const int nb = c.n_blocks[b];
    const int s_act = (nb + E - 1) / E;
    __shared__ float Mh[MAX_HQ], Rh[MAX_HQ];
    for (int h = tid; h < c.Hq; h += THREADS) {
        const float *ml = ws.ml + ((size_t)b * c.Hq + h) * S * 2;
        float M = -INFINITY;
        for (int s = 0; s < s_act; ++s) M = fmaxf(M, ml[2 * s]);
        float L = 0.f;
        for (int s = 0; s < s_act; ++s)
            if (ml[2 * s] != -INFINITY) L += ml[2 * s + 1] * exp2f(ml[2 * s] - M);
        Mh[h] = M;
        Rh[h] = L > 0.f ? 1.0f / L : 0.f;
    }
    __syncthreads();
    for (int h = chunk; h < c.Hq; h += C) {
        if (tid >= HD) break;
        const float *ml = ws.ml + ((size_t)b * c.Hq + h) * S * 2;
        const float *o = ws.o + ((size_t)b * c.Hq + h) * S * HD;
        float acc = 0.f;
        for (int s = 0; s < s_act; ++s)
            if (ml[2 * s] != -INFINITY) acc += o[(size_t)s * HD + tid] * exp2f(ml[2 * s] - Mh[h]);
        out[((size_t)b * c.Hq + h) * HD + tid] = acc * Rh[h];
    }
    const size_t score_row = (size_t)c.max_blocks * BLK;
    for (int i = tid; i < E * BLK; i += THREADS) {
        const int e = chunk * E + i / BLK, t = i % BLK;
        if (e >= nb) break;
        const uint32_t ent = c.table[(size_t)b * c.max_blocks + e];
        const int pool = (int)(ent >> 30);
        const uint32_t id = ent & 0x3fffffffu;
        if (!((c.mask[pool][id] >> t) & 1)) continue;
        const int p = c.pos[pool][(size_t)id * BLK + t];
        const float *sp = ws.score + (size_t)b * c.Hq * score_row + (size_t)e * BLK + t;
        float sum = 0.f;
        for (int h = 0; h < c.Hq; ++h) sum += exp2f(sp[h * score_row] - Mh[h]) * Rh[h];
        mass[(size_t)b * c.n_cap + p] = sum;
        if (importance) {
            float *ip = importance + (size_t)b * c.n_cap + p;
            *ip = fmaf(decay, *ip, sum);
        }
    }
}

}  // namespace

bool launch_decode(const kvq_cache &c, const void *q, float *out, float *mass, float *importance,
                   float decay, float sm_scale, void *ws_ptr, hipStream_t s) {
    DecodeWs ws(ws_ptr, c);
    const int S = n_splits(c);
    hipLaunchKernelGGL(attn_split, dim3(S, c.Hkv, c.B), dim3(THREADS), 0, s, c,
                       static_cast<const uint16_t *>(q), mass, ws, sm_scale * LOG2E);
    hipLaunchKernelGGL(attn_finalize, dim3(S, c.B), dim3(THREADS), 0, s, c, out, mass, importance,
                       decay, ws, S);
    return hipGetLastError() == hipSuccess;
}

}  // namespace kvq
