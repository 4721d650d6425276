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
//
// No K/V load of the tile walk waits on another vector load: the block ids
// come from scalar loads issued a tile ahead, and each lane loads one scale
// per tile -- lane (slot, c) the K (c < 4) or V (c >= 4) scale of token
// t0 + 8 (c % 4) + slot -- which DPP moves then hand to the lanes that need
// them.  Scales are stored [block][kv head][row], so the 32 scales of one
// head in a tile are one 128-byte line per array: a wave reads only its own
// head's lines, and every scale line is fetched once.
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

using const_i32 = const __attribute__((address_space(4))) int32_t;

// Buffer resource over [base, base + bytes): loads at offsets >= bytes
// return 0 without touching memory (raw buffer, stride 0).
constexpr int kRsrcWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, kRsrcWord3);
}

// Cache policy of the K/V code and scale loads: the SLC bit, which gfx950
// encodes as `nt` (non-temporal).  Every cache byte is read once per call,
// and streaming loads keep it from displacing lines in L2 and the Infinity
// Cache; on an MI355X a plain read of 0.5-2 GiB runs 15-20% faster with the
// hint (5.8 -> 6.7-7.0 TB/s), and the decode kernel 12% faster.
constexpr int kStreamPolicy = 2;

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStreamPolicy));
}

__device__ __forceinline__ float buf_load4(__amdgpu_buffer_rsrc_t r, int voff, int soff)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kStreamPolicy));
}

constexpr int kOutOfRange = 0x7ffffff0;   // a lane offset past any resource

struct Tile {
    uint4 k[4];
    uint4 v[4];
    float sk, sv;     // this lane's scale: K (c < 4, sv = 0) or V (c >= 4, sk = 0) of token t0 + 8 (c % 4) + slot
    uint32_t valid;   // bit k: token t0 + 8 k + slot is inside the sequence (and its block id is good)
    // matrix-core score layout only (load_tile_mf): K scales of tokens
    // t0 + j and t0 + 16 + j, and their validity in bits 0 and 1
    float ksm[2];
    uint32_t svalid;
};

// Physical block ids of the 4 sub-tiles of tile [t0, t0 + 32), read with
// scalar loads (the table is read-only for the kernel's lifetime; scalar
// loads are counted apart from the vector loads, so waiting for them never
// drains the K/V loads in flight).  Sub-tiles at or past n get -1.
struct TileBlocks {
    int id[4];
};

__device__ __forceinline__ void fetch_blocks(const int32_t *bt, int log2bs, int t0, int n, TileBlocks &b)
{
    const_i32 *sbt = (const_i32 *)bt;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int tk = t0 + kSub * kk;
        b.id[kk] = (tk < n) ? sbt[tk >> log2bs] : -1;
    }
}

// The same for the decode walk, branch-free: every scalar load reads an
// entry of the sequence's own table row (token index clamped to the last
// token; n >= 1 for a walked piece, and n <= max_seq_len <=
// max_blocks_per_seq * kv_bs), so a tile's loads issue together and the
// compiler can hoist them above other work.  BigBlocks (kv_bs >= 32): the
// four sub-tiles of a tile lie in one block, read once.
template <bool BigBlocks>
__device__ __forceinline__ void fetch_blocks_ahead(const int32_t *bt, int log2bs, int t0, int n, TileBlocks &b)
{
    const_i32 *sbt = (const_i32 *)bt;
    const int last = max(n - 1, 0);
    if (BigBlocks) {
        const int id = sbt[min(t0, last) >> log2bs];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) b.id[kk] = (t0 + kSub * kk < n) ? id : -1;
    } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int tk = t0 + kSub * kk;
            const int id = sbt[min(tk, last) >> log2bs];
            b.id[kk] = (tk < n) ? id : -1;
        }
    }
}

// Per-lane constants of the tile walk (loop invariant).
struct LaneOffsets {
    int code;     // byte offset of this lane's 16 bytes inside an 8-row sub-tile
    int scale_k;  // byte offset of this lane's K scale among the head's 32 tile rows, or out of range
    int scale_v;  // same for V
    int scale_sub;// byte offset of this lane's scale inside an 8-row sub-tile
    int kh;       // the wave's KV head
    int kmf;      // matrix-core score layout: bytes [32 lg, 32 lg + 32) of token row j (lane = 16 lg + j)
    int ksmf;     // and that row's scale
};

__device__ __forceinline__ LaneOffsets lane_offsets(const CacheView &cv, int kh, int lane)
{
    const int slot = lane >> 3, c = lane & 7;
    const int row_bytes = cv.nkv * kHeadDim;
    LaneOffsets o;
    o.code = slot * row_bytes + kh * kHeadDim + 16 * c;
    const int in_tile = (kSub * (c & 3) + slot) * 4;
    o.scale_k = (c < 4) ? in_tile : kOutOfRange;
    o.scale_v = (c < 4) ? kOutOfRange : in_tile;
    o.scale_sub = slot * 4;
    o.kh = uniform(kh);   // wave-uniform: the scale resources live in SGPRs
    o.kmf = (lane & 15) * row_bytes + kh * kHeadDim + 32 * (lane >> 4);
    o.ksmf = (lane & 15) * 4;
    return o;
}

// Loads tile [t0, t0 + 32) of one sequence for KV head kh, given its block
// ids; tokens at or past n are masked by `valid`.  Every call issues the
// same number of loads whatever the tile holds, so the compiler waits for
// exactly the loads a tile needs and leaves the next tile's in flight: a
// sub-tile that starts at or past n, or whose block id is outside
// [0, num_blocks) (reported in *status), gets an empty buffer resource and
// reads zeros without touching memory.  Rows past n inside a real sub-tile
// are read (they lie inside a real block) and masked.
//
// BigBlocks (kv_bs >= 32): a tile lies inside one block, so one resource per
// array covers it (sub-tiles are 8-row steps of the SGPR offset) and the
// scales come in two loads.  Otherwise every sub-tile has its own resources.
template <bool WithV, bool BigBlocks>
__device__ __forceinline__ void load_tile(const CacheView &cv, const TileBlocks &tb, const LaneOffsets &lo,
                                          int lane, int t0, int n, int32_t *status, Tile &t)
{
    const int slot = lane >> 3, c = lane & 7;
    const int bs_mask = (1 << cv.kv_bs_log2) - 1;
    const int row_bytes = cv.nkv * kHeadDim;
    bool ok[4];
    bool bad = false;
    t.valid = 0;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int tk = t0 + kSub * kk;
        const bool want = tk < n;
        const bool good = (unsigned)tb.id[kk] < (unsigned)cv.num_blocks;
        ok[kk] = want && good;
        bad = bad || (want && !good);
        t.valid |= (ok[kk] && tk + slot < n) ? (1u << kk) : 0u;
    }
    if (bad && lane == 0 && status) atomicOr(status, kDevBadBlockId);
    if (BigBlocks) {
        const bool tok = ok[0];   // the tile's sub-tiles share block tb.id[0]
        const size_t row0 = ((size_t)(tok ? tb.id[0] : 0) << cv.kv_bs_log2) + (size_t)(t0 & bs_mask);
        const int bytes = tok ? kTile * row_bytes : 0;
        if (WithV) {
            // the head's 32 scales of the tile ([block][kv head][row])
            const size_t s0 = ((((size_t)(tok ? tb.id[0] : 0) * cv.nkv + lo.kh) << cv.kv_bs_log2) +
                               (size_t)(t0 & bs_mask));
            const int sbytes = tok ? kTile * 4 : 0;
            const auto sk = make_rsrc(cv.k_scale + s0, sbytes);
            const auto sv = make_rsrc(cv.v_scale + s0, sbytes);
            // kept apart: adding them here would make the loop wait for them
            t.sk = buf_load4(sk, lo.scale_k, 0);
            t.sv = buf_load4(sv, lo.scale_v, 0);
        }
        const auto rk = make_rsrc(cv.k_codes + row0 * row_bytes, bytes);
        const auto rv = make_rsrc(cv.v_codes + row0 * row_bytes, bytes);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            t.k[kk] = buf_load16(rk, lo.code, kk * kSub * row_bytes);
            if (WithV) t.v[kk] = buf_load16(rv, lo.code, kk * kSub * row_bytes);
        }
    } else {
        float sk = 0.0f, sv = 0.0f;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int tk = t0 + kSub * kk;
            const size_t row0 = ((size_t)(ok[kk] ? tb.id[kk] : 0) << cv.kv_bs_log2) + (size_t)(tk & bs_mask);
            const int bytes = ok[kk] ? kSub * row_bytes : 0;
            t.k[kk] = buf_load16(make_rsrc(cv.k_codes + row0 * row_bytes, bytes), lo.code, 0);
            if (WithV) {
                t.v[kk] = buf_load16(make_rsrc(cv.v_codes + row0 * row_bytes, bytes), lo.code, 0);
                const size_t s0 = ((((size_t)(ok[kk] ? tb.id[kk] : 0) * cv.nkv + lo.kh) << cv.kv_bs_log2) +
                                   (size_t)(tk & bs_mask));
                const int sbytes = ok[kk] ? kSub * 4 : 0;
                const int mine = ((c & 3) == kk) ? lo.scale_sub : kOutOfRange;
                sk += buf_load4(make_rsrc(cv.k_scale + s0, sbytes), (c < 4) ? mine : kOutOfRange, 0);
                sv += buf_load4(make_rsrc(cv.v_scale + s0, sbytes), (c < 4) ? kOutOfRange : mine, 0);
            }
        }
        if (WithV) {
            t.sk = sk;
            t.sv = sv;
        }
    }
}

// load_tile for the matrix-core score path (kv_bs >= 32, so a tile lies in
// one block): V, the spread scales and `valid` as load_tile, but K in the
// layout of v_mfma_i32_16x16x64_i8's B operand -- lane (lg, j) holds bytes
// [32 lg, 32 lg + 32) of token t0 + j in k[0], k[1] and of token t0 + 16 + j
// in k[2], k[3] -- plus those two tokens' K scales.
__device__ __forceinline__ void load_tile_mf(const CacheView &cv, const TileBlocks &tb, const LaneOffsets &lo,
                                             int lane, int t0, int n, int32_t *status, Tile &t)
{
    const int slot = lane >> 3, j = lane & 15;
    const int bs_mask = (1 << cv.kv_bs_log2) - 1;
    const int row_bytes = cv.nkv * kHeadDim;
    const bool want = t0 < n;
    const bool good = (unsigned)tb.id[0] < (unsigned)cv.num_blocks;
    const bool tok = want && good;
    if (want && !good && lane == 0 && status) atomicOr(status, kDevBadBlockId);
    t.valid = 0;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) t.valid |= (tok && t0 + kSub * kk + slot < n) ? (1u << kk) : 0u;
    t.svalid = ((tok && t0 + j < n) ? 1u : 0u) | ((tok && t0 + 16 + j < n) ? 2u : 0u);
    const size_t row0 = ((size_t)(tok ? tb.id[0] : 0) << cv.kv_bs_log2) + (size_t)(t0 & bs_mask);
    const int bytes = tok ? kTile * row_bytes : 0;
    const size_t s0 =
        ((((size_t)(tok ? tb.id[0] : 0) * cv.nkv + lo.kh) << cv.kv_bs_log2) + (size_t)(t0 & bs_mask));
    const int sbytes = tok ? kTile * 4 : 0;
    const auto sk = make_rsrc(cv.k_scale + s0, sbytes);
    const auto sv = make_rsrc(cv.v_scale + s0, sbytes);
    t.sk = buf_load4(sk, lo.scale_k, 0);
    t.sv = buf_load4(sv, lo.scale_v, 0);
    t.ksm[0] = buf_load4(sk, lo.ksmf, 0);
    t.ksm[1] = buf_load4(sk, lo.ksmf, 16 * 4);
    const auto rk = make_rsrc(cv.k_codes + row0 * row_bytes, bytes);
    const auto rv = make_rsrc(cv.v_codes + row0 * row_bytes, bytes);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        t.k[2 * m] = buf_load16(rk, lo.kmf, 16 * m * row_bytes);
        t.k[2 * m + 1] = buf_load16(rk, lo.kmf + 16, 16 * m * row_bytes);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) t.v[kk] = buf_load16(rv, lo.code, kk * kSub * row_bytes);
}

// ------------------------------------- four query heads per KV head, MFMA --
// The score path of q8_decode_attn when nq / nkv == 4 and kv_bs >= 32 (and
// of the partials test hook on those shapes): v_mfma_i32_16x16x64_i8 with
// A = the four heads' query codes -- row 4 g + beta holds head g's codes of
// 32-block beta, placed in k-group beta only, zeros elsewhere -- and B = 16
// K rows in load_tile_mf's layout.  Lane (lg, j) = (lane / 16, lane % 16)
// then holds the exact int32 partials of head lg with token j of the
// 16-token half, block beta in register beta ("9-2 flash_attn_single_q_q8_neon"
// §2 segments 1-2: one exact int32 sum per 32-block).
typedef int v4i_mf __attribute__((ext_vector_type(4)));

struct MfQuery {
    v4i_mf a[2];   // A operand: 32 code bytes of (head (lane % 16) / 4, block lane % 4) in k-group lane / 16 only
    float qs[4];   // qscale of head lane / 16, blocks 0..3
};

// The query block lane (lg, j) quantizes: head j / 4 of the group, 32-block
// j % 4 (q_group: the group's first query row; 128 fp32 per head).
__device__ __forceinline__ void mf_load_query(const float *q_group, int lane, float4 (&qv)[8])
{
    const int j = lane & 15;
    const float4 *qp = reinterpret_cast<const float4 *>(q_group + (j >> 2) * kHeadDim + 32 * (j & 3));
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[i] = qp[i];
}

// Quantizes the lane's block ("9-2" §2 segment 1, one lane per 32-block) and
// forms the A operands and the per-lane block scales; lo, hi, step are the
// lane's own codes and scale.
__device__ __forceinline__ void mf_query_operands(const float4 (&qv)[8], int lane, MfQuery &mq, uint4 &lo,
                                                  uint4 &hi, float &step)
{
    const int j = lane & 15, lg = lane >> 4;
    quantize_q_block_vals(qv, lo, hi, step);
    const bool mine = lg == (j & 3);
    mq.a[0] = __builtin_bit_cast(v4i_mf, mine ? lo : make_uint4(0, 0, 0, 0));
    mq.a[1] = __builtin_bit_cast(v4i_mf, mine ? hi : make_uint4(0, 0, 0, 0));
#pragma unroll
    for (int r = 0; r < 4; ++r) mq.qs[r] = __shfl(step, 4 * lg + r, 64);
}

// The exact int32 block partials of 16 tokens (m = 0: t0 .. t0 + 15, m = 1:
// t0 + 16 .. t0 + 31) of a tile loaded by load_tile_mf.
__device__ __forceinline__ v4i_mf mf_block_partials(const MfQuery &mq, const uint4 (&k)[4], int m)
{
    v4i_mf acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(mq.a[0], __builtin_bit_cast(v4i_mf, k[2 * m]),
                                                       v4i_mf{0, 0, 0, 0}, 0, 0, 0);
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(mq.a[1], __builtin_bit_cast(v4i_mf, k[2 * m + 1]), acc, 0, 0, 0);
}

// K and V scales of this lane's token in sub-tile kk, from the lanes of the
// same 8-lane group that loaded them (see Tile::sc).
template <int KK>
__device__ __forceinline__ void tile_scales(const Tile &t, int c, float &ks, float &vs)
{
    const float sc = t.sk + t.sv;              // one of the two is 0
    const float b = dpp_f<0x55 * KK>(sc);       // quad_perm [KK, KK, KK, KK]
    const float m = dpp_f<kDppHalfMirror>(b);   // the other quad's value
    ks = (c < 4) ? b : m;
    vs = (c < 4) ? m : b;
}

}  // namespace q8kv
