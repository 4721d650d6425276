// q8kv_decode.hip -- single-query decode attention over the blocked q8 cache.
//
// Method ("9-2 flash_attn_single_q_q8_neon -- 单 q 单遍扫全 KV"):
//   §2 segment 1: the query is quantized once, in 32-element blocks;
//   §2 segment 2: per token, int8 dot products give one int32 sum per block,
//     rescaled by the block's Q scale, then by the K row scale and the
//     softmax scale; an online softmax keeps the running max M and sum S and
//     rescales what has been accumulated whenever M rises; V is accumulated
//     as int8 code times (weight x V row scale), weights staying fp32;
//   §2 segment 3: one division by S at the end.
// §1 and §3 of the same page: the cache is read exactly once.
//
// GPU organisation (gfx950, wave64):
//   * The batch's tiles (32 tokens of one sequence) are laid end to end and
//     cut into `nparts` equal contiguous ranges; one workgroup per range (and
//     per group of up to 8 KV heads) walks its range.  Each KV head is one wave, so
//     the K/V rows of a head are read once for all of its G = nq/nkv query
//     heads, and a workgroup's waves together read whole token rows.
//   * Per tile the rescale is applied once with the tile's max (the online
//     softmax in blocked form, "online softmax 分块语义" in §2 segment 2):
//     exactly the per-token recurrence up to fp32 rounding.
//   * Scores are kept in the log2 domain (scale * log2 e folded into the
//     per-token factor) so the weights are single v_exp_f32 instructions.
//   * A sequence cut by a range boundary leaves (M, S, acc) partial states
//     in the workspace; the merge kernel combines them with the same rescale
//     rule and divides once.  A sequence inside one range is finished in place.
#include <atomic>
#include "q8kv_ranges.hpp"

namespace q8kv {

// Register tiles per wave.  Two keep the memory system saturated here: a
// third tile (room for it exists at two query heads per KV head) measured
// 1.5% slower on the ragged 2B batch.
template <int G> struct PipeDepth { static constexpr int value = 2; };

// Where a wave's state goes after the slot sums (slot_reduce_scatter): token
// slot s holds 2 G consecutive dims, from 16 c + (s 2 G) % 16, of head s G / 8
// of its KV head, with that head's M and S.  key >= 0: record `key` of the
// workspace; key < 0: output row -key - 1 (z already divided by S).
template <int G>
__device__ __forceinline__ void write_state(const DecodeParams &p, int kh, int lane, int key,
                                            const float (&z)[2 * G], float mr, float sr)
{
    constexpr int P = 2 * G;
    const int c = lane & 7, tslot = lane >> 3;
    const int j0 = (tslot * P) & 15, h = kh * G + ((tslot * G) >> 3);
    if (key >= 0) {
        const size_t idx = (size_t)key * p.nq + h;
        store_floats<P>(p.ws_acc + idx * kHeadDim + 16 * c + j0, z);
        if (c == 0 && j0 == 0) p.ws_ms[idx] = make_float2(mr, sr);
    } else {
        store_floats<P>(p.out + ((size_t)(-key - 1) * p.nq + h) * kHeadDim + 16 * c + j0, z);
    }
}

// A wave's finished states waiting in LDS (lane-private slots of P + 3 words:
// the dims, M, S and the key) until the slots are full or the workgroup's walk
// ends.  Stores issued between tile loads would hold up every later tile wait
// (the vector memory counter counts in order), so a state is written only
// after the wave's last tile, unless the slots run out first.  slots = 0:
// every state is written at once.
template <int G>
struct HeldStates {
    static constexpr int P = 2 * G, W = P + 3;
    float *buf;   // [slots][W][64]
    int slots;
    int n;        // held (uniform)

    __device__ __forceinline__ void drain(const DecodeParams &p, int kh, int lane)
    {
        for (int i = 0; i < n; ++i) {
            float z[P];
#pragma unroll
            for (int k = 0; k < P; ++k) z[k] = buf[(i * W + k) * 64 + lane];
            write_state<G>(p, kh, lane, __float_as_int(buf[(i * W + P + 2) * 64 + lane]), z,
                           buf[(i * W + P) * 64 + lane], buf[(i * W + P + 1) * 64 + lane]);
        }
        n = 0;
    }
    __device__ __forceinline__ void put(const DecodeParams &p, int kh, int lane, int key, const float (&z)[P],
                                        float mr, float sr)
    {
        if (slots == 0) {
            write_state<G>(p, kh, lane, key, z, mr, sr);
            return;
        }
        if (n == slots) drain(p, kh, lane);
#pragma unroll
        for (int k = 0; k < P; ++k) buf[(n * W + k) * 64 + lane] = z[k];
        buf[(n * W + P) * 64 + lane] = mr;
        buf[(n * W + P + 1) * 64 + lane] = sr;
        buf[(n * W + P + 2) * 64 + lane] = __int_as_float(key);
        ++n;
    }
};

// One wave: attention of the G query heads of KV head kh over tiles
// [lt0, lt1) of sequence b (length n).  The state goes to the output rows
// (whole) or to slot `slot` of record `part`, i.e. to record 2 part + slot.
// With Runs, [lt0, lt1) is a run of chunks of `chunk` tiles each (lt0 a
// multiple of chunk): the state is written to record 2 part + slot + i at the
// end of the run's chunk i and started afresh, while the next chunk's first
// tile loads are already in flight, so each chunk's record is the one a piece
// of that chunk alone would leave.
template <int G, bool Big, bool Runs>
__device__ __forceinline__ void attend_piece(const DecodeParams &p, int b, int kh, int lane,
                                             int lt0, int lt1, int n, bool whole, int part,
                                             int slot, const TileBlocks *first, int chunk, HeldStates<G> &held)
{
    const int c = lane & 7, tslot = lane >> 3;
    const uint32_t m1 = (c & 1) ? 0xffffffffu : 0u, m2 = (c & 2) ? 0xffffffffu : 0u;

    const int32_t *bt = p.block_table + (size_t)b * p.max_blocks_per_seq;
    const int log2bs = p.cache.kv_bs_log2;
    const int ne = min(n, lt1 * kTile);
    constexpr int D = PipeDepth<G>::value;
    Tile t[D];
    TileBlocks bl[D];
    // The query rows and the first tile's block ids are loaded together, and
    // the first tile's loads go out before the query is quantized (the
    // scheduling barrier keeps the compiler from moving them below it): a
    // piece starts after two memory round trips (block id, tile), not three.
    float4 qv[G][4];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float4 *qp = reinterpret_cast<const float4 *>(p.q + ((size_t)b * p.nq + kh * G + g) * kHeadDim + 16 * c);
#pragma unroll
        for (int i = 0; i < 4; ++i) qv[g][i] = qp[i];
    }
    if (first)   // the block ids a step plan holds for this piece
        planned_first_blocks<Big>(*first, lt0 * kTile, ne, bl[0]);
    else
        fetch_blocks_ahead<Big>(bt, log2bs, lt0 * kTile, ne, bl[0]);
    const LaneOffsets lo = lane_offsets(p.cache, kh, lane);
#pragma unroll
    for (int d = 0; d < D - 1; ++d) {
        if (d > 0) fetch_blocks_ahead<Big>(bt, log2bs, (lt0 + d) * kTile, ne, bl[d]);
        load_tile<true, Big>(p.cache, bl[d], lo, lane, (lt0 + d) * kTile, ne, p.dev_status, t[d]);
    }
    fetch_blocks_ahead<Big>(bt, log2bs, (lt0 + D - 1) * kTile, ne, bl[D - 1]);
    __builtin_amdgcn_sched_barrier(0);

    // Q quantized once per (sequence, head) ("9-2" §2 segment 1).
    uint4 qc[G];
    float qs[G];
#pragma unroll
    for (int g = 0; g < G; ++g) quantize_q_quarter_vals(qv[g][0], qv[g][1], qv[g][2], qv[g][3], qc[g], qs[g]);

    // PV on the matrix cores for groups of four heads: lane (slot, c) is in
    // the 4-lane block of token slot and bytes [16c, 16c + 16); with the
    // weight of head 4q + c % 4 as its a operand and its byte j as its b
    // operand, one v_mfma_f32_4x4x1 adds w[4q + i] * v[16c + j] to register
    // i of accm[q][j] -- the same per-lane accumulators as the VALU path,
    // with the 64 fp32 multiply-adds per lane and sub-tile moved off the
    // VALU.  (Groups of 8 would take two MFMAs per byte; that variant spills
    // and stays on the VALU path.)
    constexpr bool kPvMfma = G == 4;
    constexpr int NQ = kPvMfma ? G / 4 : 1;
    float M[G], S[G], acc[G][16];
    v4f accm[NQ][16];
    auto fresh = [&]() {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            M[g] = -INFINITY;
            S[g] = 0.0f;
            if constexpr (!kPvMfma) {
#pragma unroll
                for (int j = 0; j < 16; ++j) acc[g][j] = 0.0f;
            }
        }
        if constexpr (kPvMfma) {
#pragma unroll
            for (int q = 0; q < NQ; ++q)
#pragma unroll
                for (int j = 0; j < 16; ++j) accm[q][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        }
    };
    fresh();

    auto process = [&](const Tile &t) {
        float ks[4], vs[4];
        tile_scales<0>(t, c, ks[0], vs[0]);
        tile_scales<1>(t, c, ks[1], vs[1]);
        tile_scales<2>(t, c, ks[2], vs[2]);
        tile_scales<3>(t, c, ks[3], vs[3]);
        float s[4][G];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bool ok = (t.valid >> kk) & 1u;
            const float f = ks[kk] * p.sc;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                // exact int32 block sum, then x Q block scale, summed over the 4 blocks
                float x = (float)block_partial(t.k[kk], qc[g]) * qs[g];
                x += dpp_f<kDppQuadXor2>(x);
                x += dpp_f<kDppHalfMirror>(x);
                s[kk][g] = ok ? x * f : -INFINITY;
            }
        }
        // Tile max, rescale of what has accumulated if M rises.
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float m = fmaxf(fmaxf(s[0][g], s[1][g]), fmaxf(s[2][g], s[3][g]));
            m = max_over_slots(m);
            if (m > M[g]) {
                const float a = __builtin_amdgcn_exp2f(M[g] - m);
                S[g] *= a;
                if constexpr (kPvMfma) {
#pragma unroll
                    for (int j = 0; j < 16; ++j) accm[g >> 2][j][g & 3] *= a;
                } else {
#pragma unroll
                    for (int j = 0; j < 16; ++j) acc[g][j] *= a;
                }
                M[g] = m;
            }
        }
        // Weights and V accumulation: acc += code_v * (w * vs).
        float Mf[G];   // M, or 0 while no token has been seen (then every weight is 0)
#pragma unroll
        for (int g = 0; g < G; ++g) Mf[g] = M[g] == -INFINITY ? 0.0f : M[g];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bool ok = (t.valid >> kk) & 1u;
            const uint32_t words[4] = {t.v[kk].x, t.v[kk].y, t.v[kk].z, t.v[kk].w};
            // masked tokens contribute nothing (their scale may be any bit pattern)
            if constexpr (kPvMfma) {
                // branch-free: a masked token's score is -inf, so its weight
                // is exp2(-inf) = 0 against the finite reference Mf
                float pw[G];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    pw[g] = __builtin_amdgcn_exp2f(s[kk][g] - Mf[g]);
                    S[g] += pw[g];
                }
                const uint32_t okm = ok ? 0xffffffffu : 0u;
                float wa[NQ];
#pragma unroll
                for (int q = 0; q < NQ; ++q) {
                    // the weight of head 4q + c % 4, picked with bit masks
                    const uint32_t lo2 = bitsel(m1, __float_as_uint(pw[4 * q + 1]), __float_as_uint(pw[4 * q]));
                    const uint32_t hi2 = bitsel(m1, __float_as_uint(pw[4 * q + 3]), __float_as_uint(pw[4 * q + 2]));
                    const float w = __uint_as_float(bitsel(m2, hi2, lo2)) * vs[kk];
                    wa[q] = __uint_as_float(__float_as_uint(w) & okm);
                }
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float vf = byte_f(words[j >> 2], j & 3);
#pragma unroll
                    for (int q = 0; q < NQ; ++q) accm[q][j] = mfma_outer4(wa[q], vf, accm[q][j]);
                }
            } else {
                float pw[G];
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    pw[g] = ok ? __builtin_amdgcn_exp2f(s[kk][g] - M[g]) : 0.0f;
                    S[g] += pw[g];
                }
                float w[G];
#pragma unroll
                for (int g = 0; g < G; ++g) w[g] = ok ? pw[g] * vs[kk] : 0.0f;
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const float vf = byte_f(words[j >> 2], j & 3);
#pragma unroll
                    for (int g = 0; g < G; ++g) acc[g][j] = fmaf(w[g], vf, acc[g][j]);
                }
            }
        }
    };

    // The state's sums over the token slots, scattered (slot_reduce_scatter):
    // token slot s ends with 2 G consecutive dims of head s G / 8, which its 8
    // lanes hold in z, with the head's M and S.
    constexpr int P = 2 * G;
    const int gh = (tslot * G) >> 3;   // the head whose dims the lane ends with
    auto sums = [&](float (&z)[P], float &mr, float &sr) {
        float v[16 * G];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                if constexpr (kPvMfma)
                    v[16 * g + j] = accm[g >> 2][j][g & 3];
                else
                    v[16 * g + j] = acc[g][j];
            }
        slot_reduce_scatter<16 * G>(v, z, lane);
        sr = 0.0f;
        mr = 0.0f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float sg = sum_over_slots(S[g]);
            sr = gh == g ? sg : sr;
            mr = gh == g ? M[g] : mr;
        }
    };
    // the state to the output rows (divided by S) or to record `rec`, through
    // the wave's held states
    auto emit = [&](bool to_out, int rec) {
        float z[P], mr, sr;
        sums(z, mr, sr);
        if (to_out) {
            // one division at the end ("9-2" §2 segment 3)
#pragma unroll
            for (int k = 0; k < P; ++k) z[k] = sr > 0.0f ? z[k] / sr : 0.0f;
        }
        held.put(p, kh, lane, to_out ? -(b + 1) : rec, z, mr, sr);
    };

    // D register tiles (the first D - 1 loaded above): while tile i is
    // processed, the loads of tiles i + 1 .. i + D - 1 are in flight and the
    // block ids of tile i + D are being read.  Tile i lives in t[i % D].
    // Tokens past the piece count as past the end, so the tiles loaded
    // beyond the piece cost no HBM traffic.  Rounds of D tiles, the last one
    // possibly short: the loop's only exit is its count, and a chunk
    // boundary of a run (after a whole round: D divides the chunk length) is
    // handled inside the round's last step, so no path that leaves the loop
    // or skips a step runs into the flush (the compiler would make the flush
    // wait there for loads still in flight).
    int lt = lt0, rec = 2 * part + slot, cut = Runs ? lt0 + chunk : lt1;
    for (int r = (lt1 - lt0 + D - 1) / D; r > 0; --r) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (d > 0 && lt >= lt1) continue;   // the last round may be short
            // here lt % D == (lt0 + d) % D relative to the prologue's slots
            const int nxt = (d + D - 1) % D;
            load_tile<true, Big>(p.cache, bl[nxt], lo, lane, (lt + D - 1) * kTile, ne, p.dev_status, t[nxt]);
            fetch_blocks_ahead<Big>(bt, log2bs, (lt + D) * kTile, ne, bl[d]);
            process(t[d]);
            ++lt;
            if constexpr (Runs) {
                if (d == D - 1 && lt == cut && lt < lt1) {   // a chunk of the run ends
                    emit(false, rec++);
                    fresh();
                    cut += chunk;
                }
            }
        }
    }
    emit(whole, rec);
}

// Four query heads per KV head, kv_bs >= 32: the scores on the matrix cores
// (mf_query_operands / mf_block_partials in q8kv_tile.hpp): lane (lg, j)
// receives the exact int32 partials of head lg with token j, four blocks in
// four registers, two instructions per 16 tokens.  The score is then formed
// once per (head, token) instead of in eight lanes: x_b = P_b * qscale_b,
// y = (x0 + x1) + (x3 + x2), s = y * (kscale * sc).  The per-head tile max is
// a row-of-16 reduction; each V lane (slot, c) receives its head's (c % 4)
// weights with ds_bpermute and the value path is the 4x4x1 matrix-core outer
// product of attend_piece.

__device__ __forceinline__ float row16_max(float v)
{
    v = fmaxf(v, dpp_f<kDppQuadXor1>(v));
    v = fmaxf(v, dpp_f<kDppQuadXor2>(v));
    v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    return fmaxf(v, dpp_f<kDppRor8>(v));
}

__device__ __forceinline__ float row16_sum(float v)
{
    v += dpp_f<kDppQuadXor1>(v);
    v += dpp_f<kDppQuadXor2>(v);
    v += dpp_f<kDppHalfMirror>(v);
    return v + dpp_f<kDppRor8>(v);
}

template <bool Runs>
__device__ __forceinline__ void attend_piece_mf(const DecodeParams &p, int b, int kh, int lane, int lt0, int lt1,
                                                int n, bool whole, int part, int slot, const TileBlocks *first,
                                                int chunk, HeldStates<4> &held)
{
    constexpr int G = 4;
    const int c = lane & 7, tslot = lane >> 3;
    const int lg = lane >> 4;
    const uint32_t m1 = (c & 1) ? 0xffffffffu : 0u, m2 = (c & 2) ? 0xffffffffu : 0u;

    // A operands: head g = j / 4's codes of block beta = j % 4 in k-group
    // beta (this lane's group lg), 16 bytes per MFMA; qs[r] = head lg's step
    // of block r
    const int32_t *bt = p.block_table + (size_t)b * p.max_blocks_per_seq;
    const int log2bs = p.cache.kv_bs_log2;
    const LaneOffsets lo = lane_offsets(p.cache, kh, lane);
    constexpr int D = 2;
    const int ne = min(n, lt1 * kTile);
    Tile t[D];
    TileBlocks bl[D];
    // the query block and the first tile's block id together, the first
    // tile's loads before the quantization (as in attend_piece)
    float4 qv[8];
    mf_load_query(p.q + ((size_t)b * p.nq + kh * G) * kHeadDim, lane, qv);
    if (first)
        planned_first_blocks<true>(*first, lt0 * kTile, ne, bl[0]);
    else
        fetch_blocks_ahead<true>(bt, log2bs, lt0 * kTile, ne, bl[0]);
    load_tile_mf(p.cache, bl[0], lo, lane, lt0 * kTile, ne, p.dev_status, t[0]);
    fetch_blocks_ahead<true>(bt, log2bs, (lt0 + 1) * kTile, ne, bl[1]);
    __builtin_amdgcn_sched_barrier(0);

    MfQuery mq;
    {
        uint4 qlo, qhi;
        float step;
        mf_query_operands(qv, lane, mq, qlo, qhi, step);
    }
    const float *qs = mq.qs;

    float M[G], Sl;   // M per head (uniform); Sl: this lane's share of head lg's sum
    v4f accm[16];
    auto fresh = [&]() {
        Sl = 0.0f;
#pragma unroll
        for (int g = 0; g < G; ++g) M[g] = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) accm[jj] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    };
    fresh();

    // ds_bpermute byte addresses of the score lanes holding head c % 4's
    // weight of token slot (+ 8)
    const int src_lo = (16 * (c & 3) + tslot) * 4, src_hi = src_lo + 32;

    auto process = [&](const Tile &t) {
        float ks[4], vs[4];
        tile_scales<0>(t, c, ks[0], vs[0]);
        tile_scales<1>(t, c, ks[1], vs[1]);
        tile_scales<2>(t, c, ks[2], vs[2]);
        tile_scales<3>(t, c, ks[3], vs[3]);
        float s[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const v4i_mf acc_i = mf_block_partials(mq, t.k, m);
            const float x0 = (float)acc_i[0] * qs[0], x1 = (float)acc_i[1] * qs[1];
            const float x2 = (float)acc_i[2] * qs[2], x3 = (float)acc_i[3] * qs[3];
            const float y = (x0 + x1) + (x3 + x2);
            const uint32_t keep = ((t.svalid >> m) & 1u) ? 0xffffffffu : 0u;
            // a masked token's scale may be any bit pattern
            s[m] = __uint_as_float(bitsel(keep, __float_as_uint(y * (t.ksm[m] * p.sc)), 0xff800000u));
        }
        // tile max per head: lanes 16 g .. 16 g + 15 hold head g
        const float mrow = row16_max(fmaxf(s[0], s[1]));
        float mg[G];
#pragma unroll
        for (int g = 0; g < G; ++g) mg[g] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mrow), 16 * g));
        float alpha[G];
        bool rise = false;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            alpha[g] = 1.0f;
            if (mg[g] > M[g]) {
                alpha[g] = __builtin_amdgcn_exp2f(M[g] - mg[g]);
                M[g] = mg[g];
                rise = true;
            }
        }
        if (rise) {
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int jj = 0; jj < 16; ++jj) accm[jj][g] *= alpha[g];
        }
        // this lane's head: alpha, reference max
        const float a_l = lg == 0 ? alpha[0] : lg == 1 ? alpha[1] : lg == 2 ? alpha[2] : alpha[3];
        const float M_l = lg == 0 ? M[0] : lg == 1 ? M[1] : lg == 2 ? M[2] : M[3];
        const float Mf = M_l == -INFINITY ? 0.0f : M_l;   // then every weight of the head is 0
        const float p0 = __builtin_amdgcn_exp2f(s[0] - Mf), p1 = __builtin_amdgcn_exp2f(s[1] - Mf);
        Sl = Sl * a_l + (p0 + p1);
        // weights to the V lanes: token slot + 8 kk of head c % 4 sits in
        // lane 16 (c % 4) + (slot + 8 kk) % 16, register kk / 2
        float pw[4];
        pw[0] = __int_as_float(__builtin_amdgcn_ds_bpermute(src_lo, __float_as_int(p0)));
        pw[1] = __int_as_float(__builtin_amdgcn_ds_bpermute(src_hi, __float_as_int(p0)));
        pw[2] = __int_as_float(__builtin_amdgcn_ds_bpermute(src_lo, __float_as_int(p1)));
        pw[3] = __int_as_float(__builtin_amdgcn_ds_bpermute(src_hi, __float_as_int(p1)));
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const uint32_t okm = ((t.valid >> kk) & 1u) ? 0xffffffffu : 0u;
            const float wa = __uint_as_float(__float_as_uint(pw[kk] * vs[kk]) & okm);
            const uint32_t words[4] = {t.v[kk].x, t.v[kk].y, t.v[kk].z, t.v[kk].w};
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) accm[jj] = mfma_outer4(wa, byte_f(words[jj >> 2], jj & 3), accm[jj]);
        }
        (void)m1;
        (void)m2;
    };

    // the state's sums over the token slots, scattered (as in attend_piece):
    // slot s holds dims 8 (s & 1) + k of head s / 2 = lg, whose sum
    // row16_sum(Sl) gives in the same lanes
    constexpr int P = 2 * G;
    auto sums = [&](float (&z)[P], float &mr, float &sr) {
        float v[16 * G];
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int jj = 0; jj < 16; ++jj) v[16 * g + jj] = accm[jj][g];
        slot_reduce_scatter<16 * G>(v, z, lane);
        sr = row16_sum(Sl);
        mr = lg == 0 ? M[0] : lg == 1 ? M[1] : lg == 2 ? M[2] : M[3];
    };
    auto emit = [&](bool to_out, int rec) {
        float z[P], mr, sr;
        sums(z, mr, sr);
        if (to_out) {
            // one division at the end ("9-2" §2 segment 3)
#pragma unroll
            for (int k = 0; k < P; ++k) z[k] = sr > 0.0f ? z[k] / sr : 0.0f;
        }
        held.put(p, kh, lane, to_out ? -(b + 1) : rec, z, mr, sr);
    };

    // rounds and the chunk boundaries of a run as in attend_piece
    int lt = lt0, rec = 2 * part + slot, cut = Runs ? lt0 + chunk : lt1;
    for (int r = (lt1 - lt0 + D - 1) / D; r > 0; --r) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            if (d > 0 && lt >= lt1) continue;
            const int nxt = (d + D - 1) % D;
            load_tile_mf(p.cache, bl[nxt], lo, lane, (lt + D - 1) * kTile, ne, p.dev_status, t[nxt]);
            fetch_blocks_ahead<true>(bt, log2bs, (lt + D) * kTile, ne, bl[d]);
            process(t[d]);
            ++lt;
            if constexpr (Runs) {
                if (d == D - 1 && lt == cut && lt < lt1) {
                    emit(false, rec++);
                    fresh();
                    cut += chunk;
                }
            }
        }
    }
    emit(whole, rec);
}

// Ints of dynamic LDS before the waves' held states (the batch arrays,
// rounded up to 16 bytes).
__host__ __device__ inline int run_buf_offset(int batch) { return (2 * batch + 1 + 3) & ~3; }

// The partial kernel of either cut: Chunked walks the invariant cut
// (p.chunk_tiles > 0) in chunk runs, else the balanced cut or a step plan.
static_assert(kInvariantChunkTiles % 2 == 0, "a chunk boundary must fall after a whole round of D = 2 tiles");

template <int G, bool Big, bool Chunked>
__global__ __launch_bounds__(64 * kMaxWavesPerWG) void q8_attn_partial_kernel(DecodeParams p)
{
    // [batch + 1] tile prefix, [batch] lengths, then (invariant cut) each
    // wave's run_slots held chunk records of 2 G + 2 floats per lane
    extern __shared__ int lds_batch[];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    HeldStates<G> held{reinterpret_cast<float *>(lds_batch + run_buf_offset(p.batch)) +
                           wave * p.run_slots * HeldStates<G>::W * 64,
                       p.run_slots, 0};
    auto attend = [&](int b, int kh, int lane, int lt0, int lt1, int n, bool whole, int part, int slot,
                      const TileBlocks *first, int chunk) __attribute__((always_inline)) {
        // the matrix-core score path exactly where decode_uses_mfma_scores(G, kv_bs) holds
        if constexpr (G == 4 && Big)
            attend_piece_mf<Chunked>(p, b, kh, lane, lt0, lt1, n, whole, part, slot, first, chunk, held);
        else
            attend_piece<G, Big, Chunked>(p, b, kh, lane, lt0, lt1, n, whole, part, slot, first, chunk, held);
    };
    if constexpr (Chunked)
        walk_chunks<true>(p, lds_batch, lds_batch + p.batch + 1, attend);
    else
        walk_balanced(p, lds_batch, lds_batch + p.batch + 1, attend);
    // the held states, once the wave's last tile is in (its KV head as in the walks)
    const int hg = blockIdx.x % p.head_groups;
    held.drain(p, hg * (int)(blockDim.x >> 6) + wave, lane);
}

// ---------------------------------------------------------------- merge ----
struct MergeParams {
    const int32_t *ws_prefix;   // [batch + 1] cut-axis prefix (a negative total: no records)
    const float2 *ws_ms;
    const float *ws_acc;
    float *out;
    int32_t batch;
    int32_t nq;
    int32_t nparts;
    int32_t piece_cost;
    // batch-invariant cut (walk_chunks), or 0: tiles per chunk and records per
    // sequence; the chunk count comes from seq_lens
    int32_t chunk_tiles;
    int32_t max_chunks;
    const int32_t *seq_lens;
    int32_t max_seq_len;
};

constexpr int kMaxMergeWaves = 16;
constexpr int kMergeBatch = 16;  // loads a lane has in flight together

// Two partial states combined with the rescale rule of "9-2" §2 segment 2
// (M the larger, S and the accumulators rescaled to it and summed).  Every
// operation is symmetric in the two states (max, and sums of two products --
// IEEE addition is commutative), so the two lanes of a swapped pair end with
// the same bits whichever of them holds which state.
__device__ __forceinline__ void merge_states(float &m, float &s, float &ax, float &ay, float m2, float s2, float ax2,
                                             float ay2)
{
    const float mn = fmaxf(m, m2);
    if (mn == -INFINITY) return;   // neither has seen a token
    const float f1 = __builtin_amdgcn_exp2f(m - mn), f2 = __builtin_amdgcn_exp2f(m2 - mn);   // 0 for -inf
    m = mn;
    s = s * f1 + s2 * f2;
    ax = ax * f1 + ax2 * f2;
    ay = ay * f1 + ay2 * f2;
}

// The state of the lane 16 (Rows = 16) or 32 (Rows = 32) lanes away,
// combined into this lane's: a v_permlane16/32_swap of a register with itself
// leaves this lane's value and the partner's in the two results.
template <int Rows>
__device__ __forceinline__ void merge_across_rows(float &m, float &s, float &ax, float &ay)
{
    auto swap = [](float v) {
        if constexpr (Rows == 16)
            return __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        else
            return __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    };
    const auto rm = swap(m), rs = swap(s), rx = swap(ax), ry = swap(ay);
    float m0 = __uint_as_float(rm[0]), s0 = __uint_as_float(rs[0]);
    float x0 = __uint_as_float(rx[0]), y0 = __uint_as_float(ry[0]);
    merge_states(m0, s0, x0, y0, __uint_as_float(rm[1]), __uint_as_float(rs[1]), __uint_as_float(rx[1]),
                 __uint_as_float(ry[1]));
    m = m0;
    s = s0;
    ax = x0;
    ay = y0;
}

// Merge of the pieces of every (sequence, query head) whose tiles span
// several ranges: their (M, S, acc) records combined with the online-softmax
// rescale rule ("9-2" §2 segment 2 applied to whole partial states) and one
// division.  Workgroup = (sequence b, query head h, slice of 128 / Slices
// dims); a lane holds two dims of one piece, so a wave reads 64 / (64 /
// Slices) = Slices pieces per load and each lane has kMergeBatch loads in
// flight.  Wave w takes piece groups w, w + waves, ...; the lanes' states are
// combined across the lane rows (permlane swaps) and then the waves' states
// in wave order through LDS, so the result does not depend on timing.  More
// slices give small batches more workgroups (a batch-1 128K sequence has 32
// (sequence, head) rows of 256 pieces each).
template <int Slices>
__global__ __launch_bounds__(64 * kMaxMergeWaves) void q8_attn_merge_kernel(MergeParams p)
{
    constexpr int kLanesPerPiece = 64 / Slices;   // 64, 32, 16
    const int row = blockIdx.x / Slices, sl = blockIdx.x - row * Slices;
    const int b = row / p.nq, h = row - b * p.nq;
    int np, i0 = 0, slot0 = 0, total = 0;
    bool may_be_empty = false;
    if (p.chunk_tiles > 0) {
        // batch-invariant cut: the sequence's chunks, records b * max_chunks + c
        int n = p.seq_lens[b];
        if (n < 0 || n > p.max_seq_len) n = 0;   // reported by the partial kernel
        const int tiles = (n + kTile - 1) / kTile, L = chunk_tiles_of(tiles, p.chunk_tiles);
        np = (tiles + L - 1) / L;
        if (np <= 1) return;   // one chunk: finished in place
        i0 = b * p.max_chunks;
    } else {
        const int a0 = p.ws_prefix[b], e0 = p.ws_prefix[b + 1];
        total = p.ws_prefix[p.batch];
        // a negative total: the partial kernel refused its step plan (made for
        // another cut) and wrote no records
        if (e0 == a0 || total < 0) return;
        // ranges of the first and the last tile (before the first tile of a
        // sequence other than 0 lie piece_cost units that hold none)
        const int first = a0 + (b > 0 ? p.piece_cost : 0);
        i0 = part_of(first, total, p.nparts);
        const int i1 = part_of(e0 - 1, total, p.nparts);
        if (i0 == i1) return;
        np = i1 - i0 + 1;
        // the first piece sits in slot 1 of its range when the range starts in an earlier sequence
        slot0 = part_start(i0, total, p.nparts) < a0 ? 1 : 0;
        // a range can be empty (and write no record) only when there are more
        // ranges than cut-axis units; otherwise skip the two divisions per
        // record (a range strictly between the first and the last tile's holds
        // only tiles of this sequence)
        may_be_empty = p.nparts > total;
    }
    // record of piece j: (range i0 + j, slot) = index (2 (i0 + j) + slot) nq + h,
    // or chunk record i0 + j = index (i0 + j) nq + h
    const bool chunked = p.chunk_tiles > 0;
    auto record = [&](int j) {
        return chunked ? (size_t)(i0 + j) * p.nq + h : ((size_t)(i0 + j) * 2 + (j == 0 ? slot0 : 0)) * p.nq + h;
    };
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, waves = blockDim.x >> 6;
    const int pg = lane / kLanesPerPiece, dl = lane - pg * kLanesPerPiece;
    const int dim2 = sl * kLanesPerPiece + dl;   // this lane's float2 of the 64 in a row

    float m = -INFINITY, s = 0.0f, ax = 0.0f, ay = 0.0f;
    const int stride = waves * Slices;   // piece groups per round of one load
    for (int j0 = wave * Slices + pg; j0 < np; j0 += kMergeBatch * stride) {
        float2 ms[kMergeBatch], av[kMergeBatch];
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
            const int j = j0 + u * stride, i = i0 + j;
            const bool have = j < np && (!may_be_empty || part_start(i, total, p.nparts) !=
                                                              part_start(i + 1, total, p.nparts));
            if (have) {
                const size_t r = record(j);
                ms[u] = p.ws_ms[r];
                av[u] = reinterpret_cast<const float2 *>(p.ws_acc + r * kHeadDim)[dim2];
            } else {
                ms[u] = make_float2(-INFINITY, 0.0f);
                av[u] = make_float2(0.0f, 0.0f);
            }
        }
        float mn = m;
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) mn = fmaxf(mn, ms[u].x);
        if (mn == -INFINITY) continue;   // nothing visible yet
        const float fo = __builtin_amdgcn_exp2f(m - mn);   // 0 while m is -inf
        s *= fo;
        ax *= fo;
        ay *= fo;
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
            const float f = __builtin_amdgcn_exp2f(ms[u].x - mn);   // 0 for an empty piece
            s = fmaf(ms[u].y, f, s);
            ax = fmaf(av[u].x, f, ax);
            ay = fmaf(av[u].y, f, ay);
        }
        m = mn;
    }
    // the wave's piece groups: rows of 16 lanes (Slices = 4) or halves (2)
    if constexpr (Slices == 4) merge_across_rows<16>(m, s, ax, ay);
    if constexpr (Slices >= 2) merge_across_rows<32>(m, s, ax, ay);

    __shared__ float sh_m[kMaxMergeWaves], sh_s[kMaxMergeWaves];
    __shared__ float2 sh_a[kMaxMergeWaves][64];
    if (lane == 0) {
        sh_m[wave] = m;
        sh_s[wave] = s;
    }
    sh_a[wave][lane] = make_float2(ax, ay);
    __syncthreads();
    if (wave != 0 || pg != 0) return;
    float mx = -INFINITY;
    for (int w = 0; w < waves; ++w) mx = fmaxf(mx, sh_m[w]);
    s = 0.0f;
    ax = ay = 0.0f;
    if (mx != -INFINITY) {
        for (int w = 0; w < waves; ++w) {
            const float f = __builtin_amdgcn_exp2f(sh_m[w] - mx);   // 0 for a wave that saw nothing
            const float2 aw = sh_a[w][lane];
            s = fmaf(sh_s[w], f, s);
            ax = fmaf(aw.x, f, ax);
            ay = fmaf(aw.y, f, ay);
        }
    }
    float2 *o = reinterpret_cast<float2 *>(p.out + ((size_t)b * p.nq + h) * kHeadDim);
    o[dim2] = s > 0.0f ? make_float2(ax / s, ay / s) : make_float2(0.0f, 0.0f);
}

// ----------------------------------------------------------------- host ----
static size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

template <int G, bool Big>
static const void *partial_fn(bool chunked)
{
    return chunked ? reinterpret_cast<const void *>(&q8_attn_partial_kernel<G, Big, true>)
                   : reinterpret_cast<const void *>(&q8_attn_partial_kernel<G, Big, false>);
}

static const void *partial_kernel(int group, bool big, bool chunked)
{
    switch (group) {
    case 1: return big ? partial_fn<1, true>(chunked) : partial_fn<1, false>(chunked);
    case 2: return big ? partial_fn<2, true>(chunked) : partial_fn<2, false>(chunked);
    case 4: return big ? partial_fn<4, true>(chunked) : partial_fn<4, false>(chunked);
    default: return big ? partial_fn<8, true>(chunked) : partial_fn<8, false>(chunked);
    }
}

// LDS of one partial workgroup: the batch's tile prefix and lengths, and
// (slots > 0) each wave's held states (HeldStates) after them.
static size_t partial_lds_bytes(int batch, int waves = 0, int group = 0, int slots = 0)
{
    if (slots <= 0) return (size_t)(2 * batch + 1) * sizeof(int);
    return (size_t)run_buf_offset(batch) * sizeof(int) + (size_t)slots * waves * 64 * (2 * group + 3) * sizeof(float);
}

int decode_blocks_per_cu(int group, int waves, int batch)
{
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, partial_kernel(group, true, false), waves * 64,
                                                     partial_lds_bytes(batch)) != hipSuccess || nb < 1)
        nb = 1;
    return nb;
}

// Waves per SIMD that the partial kernel for (group, block size, cut) can
// hold (its registers decide): the resident 4-wave workgroups per CU, one
// wave per SIMD each.  Cached per device.
static int partial_waves_per_simd(int group, bool big, bool chunked)
{
    static std::atomic<int> cache[kMaxDevices][4][2][2];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
    const int gi = group == 1 ? 0 : group == 2 ? 1 : group == 4 ? 2 : 3;
    if (dev >= 0) {
        const int v = cache[dev][gi][big][chunked].load(std::memory_order_relaxed);
        if (v > 0) return v;
    }
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, partial_kernel(group, big, chunked), 256, 0) != hipSuccess ||
        nb < 1)
        nb = 1;
    if (dev >= 0) cache[dev][gi][big][chunked].store(nb, std::memory_order_relaxed);
    return nb;
}

// Workgroup width (KV heads per workgroup, one wave each): at most 8, and at
// most 4 where the kernel holds three or more waves per SIMD (G <= 2 with
// blocks of 32 positions or more).  The narrow workgroups spread a range's KV
// heads over two CUs' worth of slots: A-B-B-A on one box, ragged 2B batch
// 105.4 -> 101.8-102.3 us per layer-step at 256 ranges (384 ranges: 102.4-102.6,
// 512: 103.8), 2B batch 1 at n = 4059 12.6 -> 11.2 us; at two waves per SIMD
// (G = 4) they were slower (stress batch 102.8 -> 106.7 us).
static void choose_width(const q8_kv_layer &layer, int group, bool chunked, int &waves, int &head_groups)
{
    const int maxw =
        partial_waves_per_simd(group, layer.kv_bs >= kTile, chunked) >= 3 ? kMaxWavesPerWG / 2 : kMaxWavesPerWG;
    head_groups = (layer.nkv_heads + maxw - 1) / maxw;
    waves = (layer.nkv_heads + head_groups - 1) / head_groups;
}

// One range per CU for every whole multiple of the batch's KV heads that the
// CU's resident waves cover (at least one; fewer ranges than CUs when a
// range's heads take more than a CU), at most one per tile.
int auto_parts(const q8_kv_layer &layer, const q8_batch &batch, int nq)
{
    const int group = nq / layer.nkv_heads;
    int waves, head_groups;
    choose_width(layer, group, (batch.flags & Q8_BATCH_INVARIANT) != 0, waves, head_groups);
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
            cus = v;
    }
    const long long resident = (long long)decode_blocks_per_cu(group, waves, batch.batch) * waves;   // per CU
    const long long slots = resident >= layer.nkv_heads ? (long long)cus * (resident / layer.nkv_heads)
                                                        : (long long)cus * resident / layer.nkv_heads;
    const long long tiles_ub = (long long)batch.batch * ((batch.max_seq_len + kTile - 1) / kTile);
    long long parts = slots < tiles_ub ? slots : tiles_ub;
    if (parts < 1) parts = 1;
    return (int)parts;
}

DecodePlan make_plan(const q8_kv_layer &layer, const q8_batch &batch, int nq, int nparts)
{
    DecodePlan pl;
    pl.nparts = nparts > 0 ? nparts : auto_parts(layer, batch, nq);
    pl.piece_cost = kPieceCost;
    choose_width(layer, nq / layer.nkv_heads, (batch.flags & Q8_BATCH_INVARIANT) != 0, pl.waves, pl.head_groups);
    // merge: few (sequence, query head) rows get each row's dims split over
    // up to four workgroups, so a small batch still spreads its merge over
    // many CUs; waves: enough that a sequence cut into about twice the average
    // number of pieces is read in one round (kMergeBatch loads per lane, a
    // wave reading `slices` pieces per load); more pieces take more rounds
    const long long rows = (long long)batch.batch * nq;
    pl.merge_slices = rows >= 256 ? 1 : rows >= 64 ? 2 : 4;
    const long long per_seq = 2LL * pl.nparts / (batch.batch > 0 ? batch.batch : 1) + 2;
    int mw = 1;
    while (mw < kMaxMergeWaves && (long long)mw * kMergeBatch * pl.merge_slices < per_seq) mw <<= 1;
    pl.merge_waves = mw;
    pl.chunk_tiles = 0;
    pl.max_chunks = 0;
    pl.run_slots = 0;
    size_t records = 2 * (size_t)pl.nparts;   // (range, slot) records per query head
    if (batch.flags & Q8_BATCH_INVARIANT) {
        // chunks counted from each sequence's start, no units charged per
        // sequence, one record per chunk; the merge's shape is fixed, so the
        // order in which it combines a sequence's chunk states depends on
        // their number only
        pl.piece_cost = 0;
        pl.chunk_tiles = kInvariantChunkTiles;
        // the most chunks a sequence of at most max_seq_len positions has
        pl.max_chunks = max_chunks_of((batch.max_seq_len + kTile - 1) / kTile, kInvariantChunkTiles);
        pl.merge_slices = 1;
        pl.merge_waves = 4;
        records = (size_t)batch.batch * pl.max_chunks;
    }
    // states a wave holds in LDS until its walk ends (HeldStates): up to 8 (3
    // at G = 4, none at G = 8), as many as keep the workgroup's LDS within 64
    // KB; none where a range walks about one piece (one sequence; or, for the
    // invariant cut, no more chunks than ranges), since the larger LDS
    // request then measured slower
    {
        const int group = nq / layer.nkv_heads;
        int slots = group <= 2 ? 8 : group == 4 ? 3 : 0;
        if (pl.chunk_tiles > 0 ? (long long)batch.batch * pl.max_chunks <= pl.nparts : batch.batch <= 1) slots = 0;
        while (slots > 0 && partial_lds_bytes(batch.batch, pl.waves, group, slots) > 65536) --slots;
        pl.run_slots = slots;
    }
    pl.off_prefix = 0;
    pl.off_ms = align_up(sizeof(int32_t) * ((size_t)batch.batch + 1), 256);
    pl.off_acc = pl.off_ms + align_up(sizeof(float) * 2 * records * nq, 256);
    pl.bytes = pl.off_acc + sizeof(float) * records * nq * kHeadDim;
    return pl;
}

DecodeParams fill_decode_params(const q8_kv_layer &layer, const q8_batch &batch, int nq, const float *q,
                                float scale, float *out, const DecodePlan &plan, void *workspace,
                                int32_t *dev_status)
{
    DecodeParams p;
    p.cache.k_codes = layer.k_codes;
    p.cache.v_codes = layer.v_codes;
    p.cache.k_scale = layer.k_scale;
    p.cache.v_scale = layer.v_scale;
    p.cache.nkv = layer.nkv_heads;
    p.cache.kv_bs_log2 = ilog2(layer.kv_bs);
    p.cache.num_blocks = layer.num_blocks;
    p.k_f32 = layer.k_f32;
    p.v_f32 = layer.v_f32;
    p.block_table = batch.block_table;
    p.seq_lens = batch.seq_lens;
    p.q = q;
    p.out = out;
    char *ws = static_cast<char *>(workspace);
    p.ws_prefix = ws ? reinterpret_cast<int32_t *>(ws + plan.off_prefix) : nullptr;
    p.ws_ms = ws ? reinterpret_cast<float2 *>(ws + plan.off_ms) : nullptr;
    p.ws_acc = ws ? reinterpret_cast<float *>(ws + plan.off_acc) : nullptr;
    p.dev_status = dev_status;
    p.k_new = nullptr;
    p.v_new = nullptr;
    p.plan = static_cast<const int32_t *>(batch.plan);
    p.batch = batch.batch;
    p.nq = nq;
    p.max_blocks_per_seq = batch.max_blocks_per_seq;
    p.max_seq_len = batch.max_seq_len;
    p.nparts = plan.nparts;
    p.head_groups = plan.head_groups;
    p.piece_cost = plan.piece_cost;
    p.chunk_tiles = plan.chunk_tiles;
    p.max_chunks = plan.max_chunks;
    p.run_slots = plan.run_slots;
    p.sc = (float)((double)scale * 1.4426950408889634);
    return p;
}

hipError_t launch_decode_partial(const q8_kv_layer &layer, const q8_batch &batch, int nq,
                                 const float *q, float scale, float *out, const DecodePlan &plan,
                                 void *workspace, int32_t *dev_status, hipStream_t stream,
                                 const float *k_new, const float *v_new)
{
    DecodeParams p = fill_decode_params(layer, batch, nq, q, scale, out, plan, workspace, dev_status);
    p.k_new = k_new;
    p.v_new = v_new;
    const dim3 grid(plan.nparts * plan.head_groups), block(plan.waves * 64);
    const void *fn = partial_kernel(nq / layer.nkv_heads, layer.kv_bs >= kTile, plan.chunk_tiles > 0);
    void *args[] = {&p};
    const size_t lds = partial_lds_bytes(batch.batch, plan.waves, nq / layer.nkv_heads, plan.run_slots);
    const hipError_t e = hipLaunchKernel(fn, grid, block, args, lds, stream);
    return e != hipSuccess ? e : hipGetLastError();
}

hipError_t launch_decode_merge(const q8_kv_layer &layer, const q8_batch &batch, int nq, float *out,
                               const DecodePlan &plan, void *workspace, hipStream_t stream)
{
    (void)layer;
    if (plan.nparts <= 1 && plan.chunk_tiles == 0) return hipSuccess;
    MergeParams p;
    char *ws = static_cast<char *>(workspace);
    // the cut-axis prefix, which the partial kernel wrote to the workspace
    // (from its own scan, or copied from the step plan)
    p.ws_prefix = reinterpret_cast<const int32_t *>(ws + plan.off_prefix);
    p.ws_ms = reinterpret_cast<const float2 *>(ws + plan.off_ms);
    p.ws_acc = reinterpret_cast<const float *>(ws + plan.off_acc);
    p.out = out;
    p.batch = batch.batch;
    p.nq = nq;
    p.nparts = plan.nparts;
    p.piece_cost = plan.piece_cost;
    p.chunk_tiles = plan.chunk_tiles;
    p.max_chunks = plan.max_chunks;
    p.seq_lens = batch.seq_lens;
    p.max_seq_len = batch.max_seq_len;
    const dim3 grid((unsigned)((long long)batch.batch * nq * plan.merge_slices)), block(plan.merge_waves * 64);
    if (plan.merge_slices == 4)
        hipLaunchKernelGGL(q8_attn_merge_kernel<4>, grid, block, 0, stream, p);
    else if (plan.merge_slices == 2)
        hipLaunchKernelGGL(q8_attn_merge_kernel<2>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(q8_attn_merge_kernel<1>, grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace q8kv
