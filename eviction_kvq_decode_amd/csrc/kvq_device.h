// kvq_device.h -- device-side view of the compressed KV cache format.
//
// One region per (pool, block, kv head): [K codes 256b B][V codes 256b B]
// [K (scale,zero) 256 B][V (scale,zero) 256 B], b = 8 >> pool.
//
// K rows are token-major so that a 16x16x32 MFMA A-operand (lane = token,
// lane-group kb) reads its eight channels of every 32-channel group with
// contiguous loads: lane-group kb owns channels {32g + 8kb + e}.  Within a
// group the eight codes are ordered so that one shift+mask of a dword yields
// fp16 pairs (e0,e1), (e2,e3), ... (extraction pairs codes 16 bits apart).
//
// V is channel-tiled for the PV MFMA B-operand (lane = channel j of a
// 16-channel tile n, lane-group r = tokens 4r..4r+3): lane L = 16r + j keeps
// all eight tiles of its (j, r) in consecutive dwords; within a dword codes
// are ordered so that shift+mask yields (tt0,tt1), (tt2,tt3) pairs.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int HD = 128;     // head dimension
constexpr int BLK = 16;     // slots per block
constexpr int GS = 32;      // channels per quantisation group
constexpr int NGRP = 4;     // groups per row
constexpr int TAG_NONE = 255;

__host__ __device__ inline int pool_bits(int pool) { return 8 >> pool; }
__host__ __device__ inline long region_bytes_of(int pool) { return 512L * pool_bits(pool) + 512L; }

// Code index of channel d inside a K row.
__host__ __device__ inline int k_row_index(int bits, int d) {
    const int g = d >> 5, kb = (d >> 3) & 3, e = d & 7;
    if (bits == 8) return 32 * kb + 8 * g + e;
    if (bits == 4) return 32 * kb + 8 * g + 4 * (e & 1) + (e >> 1);
    return 32 * kb + 16 * (g >> 1) + 8 * (e & 1) + 4 * (g & 1) + (e >> 1);
}

// Byte offset (inside the V-code area) of the dword that holds V code
// (t, d), and the code slot of (t, d) within that dword.
__host__ __device__ inline int v_dword_byte(int bits, int t, int d) {
    const int r = t >> 2, n = d >> 4, j = d & 15, L = 16 * r + j;
    const int w = (n * bits) >> 3;          // dword index within lane L's slice
    if (bits == 8) return (w >> 2) * 1024 + L * 16 + (w & 3) * 4;
    if (bits == 4) return L * 16 + w * 4;
    return L * 8 + w * 4;
}
__host__ __device__ inline int v_code_slot(int bits, int t, int d) {
    const int tt = t & 3, n = d >> 4;
    const int m = n % (8 / bits);
    return (tt & 1) * (16 / bits) + 2 * m + (tt >> 1);
}

__device__ inline uint8_t *region_ptr(uint8_t *base, uint32_t id, int Hkv, int h, int pool) {
    return base + ((long)id * Hkv + h) * region_bytes_of(pool);
}

// One of a cache's three per-pool pointers for a pool index held in a
// vector register: a select among the three (kept in scalar registers), not
// an indexed read of the kernel-argument array, which costs a dependent
// memory load.
template <class T>
__device__ inline T *pool_sel(T *const (&a)[3], uint32_t pool) {
    return pool == 0 ? a[0] : (pool == 1 ? a[1] : a[2]);
}

__device__ inline float h2f(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }
__device__ inline uint16_t f2h_rn(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

}  // namespace kvq
