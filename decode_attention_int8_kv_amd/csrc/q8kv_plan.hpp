// q8kv_plan.hpp -- the launch plan of one q8 decode call (ranges, workgroup
// shape, workspace layout), shared by the decode kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "q8kv.h"

namespace q8kv {

// Resolved launch plan of one decode call.
struct DecodePlan {
    int nparts;          // equal ranges of the batch's tile sequence
    int head_groups;     // workgroups per range (`waves` KV heads each)
    int waves;           // waves per decode workgroup
    int merge_waves;     // waves per merge workgroup
    int merge_slices;    // merge workgroups per (sequence, query head): dim slices 1, 2 or 4
    int piece_cost;      // cut-axis units charged per non-empty sequence (see q8kv_ranges.hpp)
    int chunk_tiles;     // batch-invariant cut: tiles per chunk (walk_chunks), or 0
    int max_chunks;      // batch-invariant cut: chunk records per sequence
    int run_slots;       // batch-invariant cut: chunk records a wave holds in LDS within a run (0: none)
    size_t off_prefix, off_ms, off_acc, bytes;
};

// Units charged per non-empty sequence when the batch is cut into ranges: a
// piece start costs about one tile's time (its query, block-id and first tile
// loads are dependent round trips), so ranges that start many sequences get
// fewer tiles.
constexpr int kPieceCost = 2;

// The batch-invariant cut (Q8_BATCH_INVARIANT): chunks of this many 32-token
// tiles counted from each sequence's start (Q8_INVARIANT_CHUNK_TOKENS
// positions) for sequences under 32 such chunks, twice as long up to 128 and
// four times as long beyond (chunk_tiles_of).  Short chunks spread a short
// sequence over many ranges (its latency at batch 1); long sequences get
// longer chunks, whose fewer starts, flushes and records cost less on a full
// batch, and still at least 32 of them.
constexpr int kInvariantChunkTiles = 4;

// Tiles per chunk of a sequence of `tiles` tiles under the batch-invariant
// cut with base chunk length `base` (a function of the sequence's own length
// only).
// Chunks of the base length up to kChunkBand1 chunks' worth of tiles, then
// twice as long up to kChunkBand2 base chunks' worth, then four times.
constexpr int kChunkBand1 = 32, kChunkBand2 = 128;
__host__ __device__ inline int chunk_tiles_of(int tiles, int base)
{
    return tiles >= kChunkBand2 * base ? 4 * base : tiles >= kChunkBand1 * base ? 2 * base : base;
}

// The most chunks a sequence of at most tiles_ub tiles has (the count grows
// with the length inside each band and drops where the chunk length doubles,
// so it is the largest of the bands' tops).
__host__ __device__ inline int max_chunks_of(int tiles_ub, int base)
{
    auto ceil_div = [](int a, int b) { return (a + b - 1) / b; };
    int m = ceil_div(tiles_ub < kChunkBand1 * base ? tiles_ub : kChunkBand1 * base - 1, base);
    if (tiles_ub >= kChunkBand1 * base) {
        const int c = ceil_div(tiles_ub < kChunkBand2 * base ? tiles_ub : kChunkBand2 * base - 1, 2 * base);
        m = c > m ? c : m;
    }
    if (tiles_ub >= kChunkBand2 * base) {
        const int c = ceil_div(tiles_ub, 4 * base);
        m = c > m ? c : m;
    }
    return m > 1 ? m : 1;
}

DecodePlan make_plan(const q8_kv_layer &layer, const q8_batch &batch, int nq, int nparts);
int auto_parts(const q8_kv_layer &layer, const q8_batch &batch, int nq);

// ------------------------------------------------------------ step plan --
// The cut of one decode step, made once by q8_decode_plan (one small kernel)
// and read by every layer's partial kernel instead of scanning the lengths
// and looking up block ids at the start of every workgroup.  It lists, per
// range, its pieces in walk order; per piece the sequence, its tile interval
// and length, whether it is the whole sequence, its record slot, whether it
// holds the sequence's newest token, and the block ids a piece starts with.
// int32 words, in order:
//   header  [kPlanHeader]                       (kPlanMagic, batch, nparts, ...)
//   pref    [batch + 1]   cut-axis prefix (the merge kernel reads it)
//   range   [nparts + 1]  first piece of every range (prefix of piece counts)
//   empty   [batch]       the sequences of length 0 (their output rows are zeroed)
//   pieces  [(nparts + batch) * kPieceInts], 64-byte aligned
// A range holds at most one piece more than the sequences that start inside
// it, so nparts + batch pieces always suffice.
constexpr int32_t kPlanMagic = 0x51384B50;   // tag of a finished plan
constexpr int kPlanHeader = 16;
constexpr int kPieceInts = 16;
enum PlanHeader { kPhMagic, kPhBatch, kPhParts, kPhKvBsLog2, kPhPieceCost, kPhTotal, kPhEmpty, kPhMaxSeqLen };
enum PieceField {
    kPfSeq,        // sequence b
    kPfT0,         // first tile (of the sequence's 32-token tiles)
    kPfT1,         // one past the last tile
    kPfLen,        // the sequence's length n (>= 1)
    kPfFlags,      // bit 0: whole sequence; bit 1: record slot 1; bit 2: holds position n - 1
    kPfAppendBlk,  // block id of position n - 1
    kPfFirstBlk    // 4 words: block ids of the first tile's 8-token sub-tiles (tokens clamped to n - 1)
};
constexpr int kPieceWhole = 1, kPieceSlot1 = 2, kPieceAppend = 4;

struct StepPlanLayout {
    size_t pref, range, empty, pieces, words;   // word offsets and total
};

__host__ __device__ inline StepPlanLayout step_plan_layout(int batch, int nparts)
{
    StepPlanLayout l;
    l.pref = kPlanHeader;
    l.range = l.pref + (size_t)batch + 1;
    l.empty = l.range + (size_t)nparts + 1;
    l.pieces = (l.empty + (size_t)batch + 15) / 16 * 16;
    l.words = l.pieces + ((size_t)nparts + batch) * kPieceInts;
    return l;
}

}  // namespace q8kv
