// q8kv_ranges.hpp -- what the decode partial kernels share: their launch
// parameters, the cut of the batch's tiles into contiguous ranges, and
// the walk of one range piece by piece.
//
// The batch's 32-token tiles are laid end to end on a cut axis; every
// non-empty sequence but sequence 0 is preceded by piece_cost units that hold
// no tile.  They stand for the fixed cost of starting a piece inside a range
// (the query load and the first block-id and tile loads), so a range that
// starts many sequences gets fewer tiles; sequence 0 starts with range 0
// anyway.  Range i covers units [i*T/nparts, (i+1)*T/nparts) of the T units,
// and a tile belongs to the range that holds its unit.  A piece is the part of
// one sequence inside one range: a sequence inside a single range is finished
// in place, the pieces of a cut sequence leave (M, S, acc) states for the
// merge kernel ("9-2 flash_attn_single_q_q8_neon" §2 segment 2, the rescale
// rule applied to whole partial states).
#pragma once

#include "q8kv_tile.hpp"
#include "q8kv_internal.hpp"

namespace q8kv {

struct DecodeParams {
    CacheView cache;
    const float *k_f32;   // fp32 mirror codes layout, or null
    const float *v_f32;
    const int32_t *block_table;
    const int32_t *seq_lens;
    const float *q;
    float *out;
    int32_t *ws_prefix;   // [batch + 1] tile prefix over the batch
    float2 *ws_ms;        // [nparts][2][nq] (M, S) of cut pieces
    float *ws_acc;        // [nparts][2][nq][128] accumulators of cut pieces
    int32_t *dev_status;
    // fused append (or null): the token at position seq_lens[b] - 1 of every
    // sequence, [batch][nkv][128] fp32, quantized into the cache first
    const float *k_new;
    const float *v_new;
    // the step plan (q8kv_plan.hpp), or null: the cut is then made here
    const int32_t *plan;
    int32_t batch;
    int32_t nq;
    int32_t max_blocks_per_seq;
    int32_t max_seq_len;
    int32_t nparts;
    int32_t head_groups;
    int32_t piece_cost;   // cut-axis units in front of every non-empty sequence's tiles
    // batch-invariant cut (walk_chunks), or 0: tiles per chunk, and the chunk
    // records per sequence (record of chunk c of sequence b: b * max_chunks + c)
    int32_t chunk_tiles;
    int32_t max_chunks;
    // chunk records a wave of the invariant cut's kernel holds in LDS (after
    // the batch arrays) before writing them out, or 0
    int32_t run_slots;
    float sc;             // softmax scale * log2(e)
};

// Range bounds take one integer division; it is a 32-bit one whenever
// nparts * total < 2^31 (every product below is at most that), which is far
// cheaper than the 64-bit form and runs at the start of every workgroup.
__device__ __forceinline__ bool narrow_cut(int total, int nparts)
{
    return (long long)total * nparts < (1LL << 31);
}

__device__ __forceinline__ int part_start(int i, int total, int nparts)
{
    if (narrow_cut(total, nparts)) return (int)((unsigned)(i * total) / (unsigned)nparts);
    return (int)(((long long)i * total) / nparts);
}

// The range that holds tile x (0 <= x < total).
__device__ __forceinline__ int part_of(int x, int total, int nparts)
{
    if (narrow_cut(total, nparts)) return (int)((unsigned)((x + 1) * nparts - 1) / (unsigned)total);
    return (int)((((long long)x + 1) * nparts - 1) / total);
}

// Number of entries i in [0, count) with v[i] <= u, for v non-decreasing
// (LDS); 64 entries per step, so a batch of up to 64 sequences takes one
// LDS read and a ballot instead of a binary search's dependent reads.  The
// whole wave calls it with the same arguments.
__device__ __forceinline__ int count_le(const int *v, int count, int u, int lane)
{
    int n = 0;
    for (int base = 0; base < count; base += 64) {
        const int i = base + lane;
        const uint64_t m = __builtin_amdgcn_ballot_w64(i < count && v[i] <= u);
        n += __builtin_popcountll(m);
        if (m != ~0ull) break;   // no later entry is <= u
    }
    return uniform(n);
}

// Cut-axis prefix over the batch into LDS: pref[b] = units of the sequences
// before b (tiles, plus piece_cost per non-empty sequence after sequence 0);
// and, if lens is given, the lengths.  A length outside [0, max_seq_len]
// counts as empty.
__device__ inline void build_prefix(const DecodeParams &p, int *pref, int *lens, bool report)
{
    for (int b = threadIdx.x; b < p.batch; b += blockDim.x) {
        int n = p.seq_lens[b];
        if (n < 0 || n > p.max_seq_len) {
            if (report && p.dev_status) atomicOr(p.dev_status, kDevBadSeqLen);
            n = 0;
        }
        pref[b + 1] = (n + kTile - 1) / kTile;
        if (lens) lens[b] = n;
    }
    if (threadIdx.x == 0) pref[0] = 0;
    __syncthreads();
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int carry = 0;
        for (int base = 1; base <= p.batch; base += 64) {
            const int idx = base + lane;
            const int tiles = (idx <= p.batch) ? pref[idx] : 0;
            int v = tiles + ((idx > 1 && tiles > 0) ? p.piece_cost : 0);
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int u = __shfl_up(v, off, 64);
                if (lane >= off) v += u;
            }
            if (idx <= p.batch) pref[idx] = v + carry;
            carry += __shfl(v, 63, 64);
        }
    }
    __syncthreads();
}

// The first tile's block ids of a planned piece, masked like
// fetch_blocks_ahead: sub-tiles at or past ne (the piece's end) get -1.
template <bool BigBlocks>
__device__ __forceinline__ void planned_first_blocks(const TileBlocks &raw, int t0, int ne, TileBlocks &b)
{
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) b.id[kk] = (t0 + kSub * kk < ne) ? raw.id[BigBlocks ? 0 : kk] : -1;
}

// walk_balanced over a step plan: the same pieces, appends and zeroed rows,
// read from the plan (every piece's fields with scalar loads) instead of
// found by a length scan and lookups.  A plan made for another batch size,
// partition count, block size, cost or length bound sets Q8_DEV_BAD_PLAN
// and the workgroup does nothing.
template <class Attend>
__device__ __forceinline__ void walk_plan(const DecodeParams &p, Attend &&attend)
{
    const_i32 *pl = (const_i32 *)p.plan;
    const int part = blockIdx.x / p.head_groups;
    const int hg = blockIdx.x - part * p.head_groups;
    const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int kh = hg * (int)(blockDim.x >> 6) + wave;
    // the header's fields in one round of loads (no short-circuit between them)
    const bool ok = (pl[kPhMagic] == kPlanMagic) & (pl[kPhBatch] == p.batch) & (pl[kPhParts] == p.nparts) &
                    (pl[kPhKvBsLog2] == p.cache.kv_bs_log2) & (pl[kPhPieceCost] == p.piece_cost) &
                    (pl[kPhMaxSeqLen] == p.max_seq_len);
    if (!ok) {
        if (threadIdx.x == 0 && p.dev_status) atomicOr(p.dev_status, kDevBadPlan);
        // the merge reads a negative total as "no records"
        if (blockIdx.x == 0 && threadIdx.x == 0 && p.ws_prefix) p.ws_prefix[p.batch] = -1;
        return;
    }
    const StepPlanLayout L = step_plan_layout(p.batch, p.nparts);
    // the plan's cut-axis prefix to the workspace, where the merge reads it
    // (one entry per workgroup, so no workgroup's start waits on more)
    if (p.ws_prefix && threadIdx.x == 0)
        for (int b = blockIdx.x; b <= p.batch; b += gridDim.x) p.ws_prefix[b] = pl[L.pref + b];
    const int r0 = pl[L.range + part], r1 = pl[L.range + part + 1];
    const int bs_mask = (1 << p.cache.kv_bs_log2) - 1;

    if (p.k_new && kh < p.cache.nkv) {
        // fused append: the newest token of every sequence whose last tile
        // lies in this range, before any tile is loaded (ordering as in
        // walk_balanced); four rows' loads in flight at a time
        bool wrote = false;
        for (int j0 = r0; j0 < r1; j0 += 4) {
            float2 k[4], v[4];
            int seq[4], blk[4], row[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int j = j0 + u;
                seq[u] = -1;
                if (j < r1) {
                    const_i32 *pc = pl + L.pieces + (size_t)j * kPieceInts;
                    if (pc[kPfFlags] & kPieceAppend) {
                        seq[u] = pc[kPfSeq];
                        blk[u] = pc[kPfAppendBlk];
                        row[u] = (pc[kPfLen] - 1) & bs_mask;
                        const size_t src = ((size_t)seq[u] * p.cache.nkv + kh) * kHeadDim + 2 * lane;
                        k[u] = *reinterpret_cast<const float2 *>(p.k_new + src);
                        v[u] = *reinterpret_cast<const float2 *>(p.v_new + src);
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (seq[u] < 0) continue;
                if ((unsigned)blk[u] >= (unsigned)p.cache.num_blocks) {
                    if (lane == 0 && p.dev_status) atomicOr(p.dev_status, kDevBadBlockId);
                    continue;
                }
                append_row_vals(const_cast<int8_t *>(p.cache.k_codes), const_cast<int8_t *>(p.cache.v_codes),
                                const_cast<float *>(p.cache.k_scale), const_cast<float *>(p.cache.v_scale),
                                const_cast<float *>(p.k_f32), const_cast<float *>(p.v_f32), p.cache.nkv,
                                p.cache.kv_bs_log2, blk[u], row[u], kh, k[u], v[u], lane);
                wrote = true;
            }
        }
        if (wrote) __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    }

    if (kh < p.cache.nkv) {
        for (int j = r0; j < r1; ++j) {
            const_i32 *pc = pl + L.pieces + (size_t)j * kPieceInts;
            const int b = pc[kPfSeq], lt0 = pc[kPfT0], lt1 = pc[kPfT1], n = pc[kPfLen], fl = pc[kPfFlags];
            TileBlocks first;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) first.id[kk] = pc[kPfFirstBlk + kk];
            attend(b, kh, lane, lt0, lt1, n, (fl & kPieceWhole) != 0, part, (fl & kPieceSlot1) ? 1 : 0, &first, 0);
        }
    }

    if (hg == 0) {
        const int n_empty = pl[kPhEmpty];
        for (int e = part; e < n_empty; e += p.nparts) {
            const int b = pl[L.empty + e];
            float4 *o = reinterpret_cast<float4 *>(p.out + (size_t)b * p.nq * kHeadDim);
            for (int i = threadIdx.x; i < p.nq * (kHeadDim / 4); i += blockDim.x)
                o[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
}

// Fused append of walk_balanced / walk_chunks: the new token of every
// sequence b >= lo with owns(b), for this wave's KV head kh, before the wave
// loads any tile; groups of 64 sequences from lo until past(first of the
// group).  The owning range is the one whose wave reads the token's tile, so
// the wave reads back only rows it wrote itself.  Lane i looks up sequence
// b0 + i's block while the rows of the first four owned sequences are read;
// rows are written four at a time.  A wave's vector memory operations are
// performed in order, so a wavefront-scope fence (no wait; it keeps the
// compiler from moving the tile loads above the stores) is all the ordering
// needed.  An agent-scope fence would write back and invalidate L2 in every
// workgroup.
template <class Owns, class Past>
__device__ __forceinline__ void append_rows(const DecodeParams &p, const int *lens, int kh, int lane, int lo,
                                            Owns &&owns, Past &&past)
{
    bool wrote = false;
    for (int b0 = lo; b0 < p.batch && !past(b0); b0 += 64) {
        const int b = b0 + lane;
        const bool own = b < p.batch && owns(b);
        const int pos = own ? lens[b] - 1 : 0;
        int blk = 0;
        if (own) blk = p.block_table[(size_t)b * p.max_blocks_per_seq + (pos >> p.cache.kv_bs_log2)];
        uint64_t todo = __builtin_amdgcn_ballot_w64(own);
        int idx[4];
        float2 k[4], v[4];
        auto load_group = [&]() {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                idx[j] = todo ? __builtin_ctzll(todo) : -1;
                todo &= todo - 1;
                if (idx[j] >= 0) {
                    const size_t src = ((size_t)(b0 + idx[j]) * p.cache.nkv + kh) * kHeadDim + 2 * lane;
                    k[j] = *reinterpret_cast<const float2 *>(p.k_new + src);
                    v[j] = *reinterpret_cast<const float2 *>(p.v_new + src);
                }
            }
        };
        if (!todo) continue;
        load_group();
        const uint64_t bad = __builtin_amdgcn_ballot_w64(own && (unsigned)blk >= (unsigned)p.cache.num_blocks);
        if (bad != 0 && lane == 0 && p.dev_status) atomicOr(p.dev_status, kDevBadBlockId);
        for (;;) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (idx[j] < 0) break;
                if ((bad >> idx[j]) & 1) continue;
                const int ps = __builtin_amdgcn_readlane(pos, idx[j]);
                const int bk = __builtin_amdgcn_readlane(blk, idx[j]);
                append_row_vals(const_cast<int8_t *>(p.cache.k_codes), const_cast<int8_t *>(p.cache.v_codes),
                                const_cast<float *>(p.cache.k_scale), const_cast<float *>(p.cache.v_scale),
                                const_cast<float *>(p.k_f32), const_cast<float *>(p.v_f32), p.cache.nkv,
                                p.cache.kv_bs_log2, bk, ps & ((1 << p.cache.kv_bs_log2) - 1), kh, k[j], v[j],
                                lane);
                wrote = true;
            }
            if (!todo) break;
            load_group();
        }
    }
    if (wrote) __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// Output rows of the empty sequences whose cut-axis position falls in units
// [start, end) of range `part` (the last range also takes those at the very
// end), zeroed by the whole workgroup.
__device__ __forceinline__ void zero_empty_rows(const DecodeParams &p, const int *pref, int part, int start, int end,
                                                int lane)
{
    const int total = pref[p.batch];
    // first b with pref[b] >= start (start <= total = pref[batch])
    const int lo = p.batch == 1 ? (start > 0 ? 1 : 0) : count_le(pref, p.batch + 1, start - 1, lane);
    const bool last = (part == p.nparts - 1);
    for (int b = lo; b < p.batch && (pref[b] < end || (last && pref[b] <= total)); ++b) {
        if (pref[b + 1] != pref[b]) continue;
        float4 *o = reinterpret_cast<float4 *>(p.out + (size_t)b * p.nq * kHeadDim);
        for (int i = threadIdx.x; i < p.nq * (kHeadDim / 4); i += blockDim.x)
            o[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

// The batch-invariant walk (p.chunk_tiles > 0): every sequence is cut into
// chunks of chunk_tiles_of(its tiles, chunk_tiles) tiles counted from its own
// start, and a range takes the chunks whose first tile lies in it (units
// [start, end) of the tile prefix, which here charges no units per
// sequence).  Every chunk is attended with a fresh state: a sequence of one
// chunk is finished in place, the chunks of a longer one leave their states
// in records b * max_chunks + c, which the merge kernel combines in chunk
// order.  Nothing of this depends on the other sequences or the partition
// count, so neither do the bits.  The fused append is done by the range that
// walks the sequence's last chunk.  With Runs, a range's consecutive chunks
// of one sequence go to one attend call with chunk = their length in tiles
// (the callee restarts its state at every chunk boundary but keeps its loads
// in flight across it); without, one call per chunk with chunk = 0.
template <bool Runs, class Attend>
__device__ __forceinline__ void walk_chunks(const DecodeParams &p, int *pref, int *lens, Attend &&attend)
{
    const int part = blockIdx.x / p.head_groups;
    const int hg = blockIdx.x - part * p.head_groups;
    const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int kh = hg * (int)(blockDim.x >> 6) + wave;
    build_prefix(p, pref, lens, blockIdx.x == 0);
    const int total = pref[p.batch];
    const int start = part_start(part, total, p.nparts);
    const int end = part_start(part + 1, total, p.nparts);
    // first tile of sequence b's last chunk (tiles > 0)
    auto last_chunk = [&](int b) {
        const int tiles = pref[b + 1] - pref[b], L = chunk_tiles_of(tiles, p.chunk_tiles);
        return pref[b] + ((tiles - 1) / L) * L;
    };

    if (p.k_new && lens && kh < p.cache.nkv && start < end) {
        const int lo = p.batch == 1 ? 0 : count_le(pref + 1, p.batch, start, lane);
        append_rows(p, lens, kh, lane, lo,
                    [&](int b) {
                        if (pref[b + 1] == pref[b]) return false;
                        const int c = last_chunk(b);
                        return start <= c && c < end;
                    },
                    [&](int b0) { return pref[b0] >= end; });
    }

    if (kh < p.cache.nkv && start < end) {
        // the sequence holding tile `start`, then every later one that starts before `end`
        int b = p.batch == 1 ? 0 : count_le(pref, p.batch, start, lane) - 1;
        for (; b < p.batch && pref[b] < end; ++b) {
            b = uniform(b);
            const int a0 = uniform(pref[b]), tiles = uniform(pref[b + 1]) - a0;
            if (tiles == 0) continue;
            const int L = chunk_tiles_of(tiles, p.chunk_tiles);
            const int nch = (tiles + L - 1) / L;
            const int n = uniform(lens ? lens[b] : p.seq_lens[b]);
            // chunks [c0, c1) start in [start, end) (a0 < end)
            const int c0 = a0 >= start ? 0 : (start - a0 + L - 1) / L;
            const int c1 = min(nch, (end - a0 + L - 1) / L);
            if constexpr (Runs) {
                if (c0 < c1) {
                    const int rec = b * p.max_chunks + c0;
                    attend(b, kh, lane, c0 * L, min(tiles, c1 * L), n, nch == 1, rec >> 1, rec & 1,
                           static_cast<const TileBlocks *>(nullptr), L);
                }
            } else {
                for (int c = c0; c < c1; ++c) {
                    const int rec = b * p.max_chunks + c;
                    attend(b, kh, lane, c * L, min(tiles, (c + 1) * L), n, nch == 1, rec >> 1, rec & 1,
                           static_cast<const TileBlocks *>(nullptr), 0);
                }
            }
        }
    }

    if (hg == 0) zero_empty_rows(p, pref, part, start, end, lane);
}

// The whole job of one workgroup of a partial kernel under the balanced cut:
// range blockIdx.x / head_groups, KV heads hg * waves + wave.  attend(b, kh,
// lane, lt0, lt1, n, whole, part, slot, first, chunk) runs one wave over
// tiles [lt0, lt1) of sequence b (length n); `whole` says the piece is the
// whole sequence, else its state goes to slot `slot` (0: first piece of the
// range, 1: later) of record `part`; `first` holds the raw block ids of the
// first tile (from a step plan), or is null; chunk is 0 (walk_chunks passes
// its chunk length).  Afterwards the output rows of empty sequences whose
// tile position falls in this range are zeroed (the last range also takes
// those at the very end).  With p.k_new set, `lens` (LDS, batch entries) is
// required and the range's new tokens are appended first.  With a step plan
// (p.plan) the same work is read from it (walk_plan).
template <class Attend>
__device__ __forceinline__ void walk_balanced(const DecodeParams &p, int *pref, int *lens, Attend &&attend)
{
    if (p.plan) {
        walk_plan(p, attend);
        return;
    }
    const int part = blockIdx.x / p.head_groups;
    const int hg = blockIdx.x - part * p.head_groups;
    const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int kh = hg * (int)(blockDim.x >> 6) + wave;

    build_prefix(p, pref, lens, blockIdx.x == 0);
    if (blockIdx.x == 0)
        for (int b = threadIdx.x; b <= p.batch; b += blockDim.x) p.ws_prefix[b] = pref[b];

    const int total = pref[p.batch];
    const int start = part_start(part, total, p.nparts);
    const int end = part_start(part + 1, total, p.nparts);

    if (p.k_new && lens && kh < p.cache.nkv && start < end) {
        // the sequences whose last tile lies in this range (their position
        // n - 1 is in that tile, which no other range reads), starting with
        // the first sequence whose tiles end after `start` (one exists:
        // start < total)
        const int lo = p.batch == 1 ? 0 : count_le(pref + 1, p.batch, start, lane);
        append_rows(p, lens, kh, lane, lo,
                    [&](int b) { return pref[b + 1] <= end && pref[b + 1] > pref[b]; },
                    [&](int b0) { return pref[b0 + 1] > end; });
    }

    if (kh < p.cache.nkv && start < end) {
        // the sequence holding tile `start`: the largest b with pref[b] <= start
        // (pref[0] = 0, so there is one)
        int b = p.batch == 1 ? 0 : count_le(pref, p.batch, start, lane) - 1;
        int x = start;
        while (x < end) {
            while (pref[b + 1] <= x) ++b;
            b = uniform(b);
            const int a0 = uniform(pref[b]), e0 = uniform(pref[b + 1]);
            const int f = a0 + (b > 0 ? p.piece_cost : 0);   // unit of the sequence's first tile
            const int x0 = max(x, f), x1 = min(end, e0);
            if (x0 < x1) {   // else the range ends before the sequence's first tile
                const bool whole = (x0 == f) && (x1 == e0);
                // slot 0 unless a piece of an earlier sequence lies in this range
                const int slot = (start >= a0) ? 0 : 1;
                int n = lens ? lens[b] : p.seq_lens[b];
                n = uniform(n);
                attend(b, kh, lane, x0 - f, x1 - f, n, whole, part, slot, static_cast<const TileBlocks *>(nullptr), 0);
            }
            x = x1;
        }
    }

    if (hg == 0) zero_empty_rows(p, pref, part, start, end, lane);
}

// Either cut, chosen at run time from p.chunk_tiles (one attend call per
// chunk under the invariant cut).
template <class Attend>
__device__ __forceinline__ void walk_ranges(const DecodeParams &p, int *pref, int *lens, Attend &&attend)
{
    if (p.chunk_tiles > 0)
        walk_chunks<false>(p, pref, lens, attend);
    else
        walk_balanced(p, pref, lens, attend);
}

// Host: the kernel arguments of one decode call.
DecodeParams fill_decode_params(const q8_kv_layer &layer, const q8_batch &batch, int nq, const float *q,
                                float scale, float *out, const DecodePlan &plan, void *workspace,
                                int32_t *dev_status);

}  // namespace q8kv
