// q8kv_plan.hpp -- the launch plan of one q8 decode call (ranges, workgroup
// shape, workspace layout), shared by the decode kernels and the C-ABI layer.
#pragma once

#include <stddef.h>

#include "q8kv.h"

namespace q8kv {

// Resolved launch plan of one decode call.
struct DecodePlan {
    int nparts;          // equal ranges of the batch's tile sequence
    int head_groups;     // workgroups per range (8 KV heads each)
    int waves;           // waves per decode workgroup
    int merge_waves;     // waves per merge workgroup
    int piece_cost;      // cut-axis units charged per non-empty sequence (see q8kv_ranges.hpp)
    size_t off_prefix, off_ms, off_acc, bytes;
};

// Units charged per non-empty sequence when the batch is cut into ranges: a
// piece start costs about one tile's time (its query, block-id and first tile
// loads are dependent round trips), so ranges that start many sequences get
// fewer tiles.
constexpr int kPieceCost = 2;

DecodePlan make_plan(const q8_kv_layer &layer, const q8_batch &batch, int nq, int nparts);
int auto_parts(const q8_kv_layer &layer, const q8_batch &batch, int nq);

}  // namespace q8kv
