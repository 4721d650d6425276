// q8kv_tile.hpp -- the blocked-KV tile walk shared by the decode kernel and
// the partials test hook.
//
// Layout ("9-2 flash_attn_single_q_q8_neon" §2 segment 2): token t of a
// sequence sits in physical block block_table[t / kv_bs] at row t % kv_bs;
// a row holds every KV head, head kh at bytes [128 kh, 128 kh + 128).
//
// A wave works on one KV head and walks the sequence in tiles of 32 tokens.
// Lane (slot, c) = (lane / 8, lane % 8) loads bytes [16c, 16c + 16) of the
// head's row for token t0 + 8 k + slot, k = 0..3: eight lanes cover one
// 128-byte row, so every 16-byte load is part of a fully used 128-byte line.
#pragma once

#include "q8kv_device.hpp"

namespace q8kv {

struct CacheView {
    const int8_t *k_codes;
    const int8_t *v_codes;
    const float *k_scale;
    const float *v_scale;
    int32_t nkv;
    int32_t kv_bs_log2;
    int32_t num_blocks;
};

struct Tile {
    uint4 k[4];
    uint4 v[4];
    float ks[4];
    float vs[4];
    uint32_t valid;   // bit k: this lane's token of sub-tile k is inside the sequence
};

// Loads tile [t0, t0 + 32) of one sequence (length n) for KV head kh.  Sub-
// tiles that start at or past n are not touched (their block may not exist).
// Rows past n inside a loaded sub-tile are read (they lie inside a real block)
// and masked by `valid`.  A block id outside [0, num_blocks) is reported in
// *status and its sub-tile is masked.
template <bool WithV>
__device__ __forceinline__ void load_tile(const CacheView &cv, const int32_t *__restrict__ bt,
                                          int kh, int lane, int t0, int n, int32_t *status,
                                          Tile &t)
{
    const int slot = lane >> 3, c = lane & 7;
    const int bs_mask = (1 << cv.kv_bs_log2) - 1;
    t.valid = 0;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int tk = t0 + kSub * kk;
        bool ok = tk < n;
        int blk = 0;
        if (ok) {
            blk = uniform(bt[tk >> cv.kv_bs_log2]);
            if (blk < 0 || blk >= cv.num_blocks) {
                if (lane == 0 && status) atomicOr(status, kDevBadBlockId);
                ok = false;
            }
        }
        if (ok) {
            const size_t row = ((size_t)blk << cv.kv_bs_log2) + (size_t)((tk & bs_mask) + slot);
            const size_t s = row * (size_t)cv.nkv + kh;
            t.k[kk] = *reinterpret_cast<const uint4 *>(cv.k_codes + s * kHeadDim + 16 * c);
            t.ks[kk] = cv.k_scale[s];
            if (WithV) {
                t.v[kk] = *reinterpret_cast<const uint4 *>(cv.v_codes + s * kHeadDim + 16 * c);
                t.vs[kk] = cv.v_scale[s];
            }
            t.valid |= (tk + slot < n) ? (1u << kk) : 0u;
        } else {
            t.k[kk] = make_uint4(0, 0, 0, 0);
            t.ks[kk] = 0.0f;
            if (WithV) {
                t.v[kk] = make_uint4(0, 0, 0, 0);
                t.vs[kk] = 0.0f;
            }
        }
    }
}

}  // namespace q8kv
