// q8kv_stepplan.hip -- q8_decode_plan: the cut of one decode step into
// ranges and pieces, made once per step and read by every layer's decode
// partial kernel (layout in q8kv_plan.hpp).
//
// The cut is the one the partial kernels make on their own (q8kv_ranges.hpp):
// the batch's 32-token tiles laid end to end with piece_cost units in front
// of every non-empty sequence but the first, cut into nparts equal ranges.
// Here it is made once, by one workgroup, with the very same prefix and walk,
// so a layer that reads the plan walks exactly the pieces it would have found
// itself -- its results are bit for bit those of the unplanned call -- but
// starts its first tile loads one memory round trip after launch (the plan
// read) instead of after the length scan, the range lookup and the block-id
// loads, and starts every later piece without a block-id load.
#include "q8kv_ranges.hpp"

namespace q8kv {

constexpr int kPlanThreads = 1024;

// Pieces of range i, in walk order (the loop of walk_balanced); emit(b, x0, x1,
// f, e0, slot) for each.  pref: the cut-axis prefix (LDS).
template <class Emit>
__device__ __forceinline__ void range_pieces(const int *pref, int batch, int cost, int start, int end, Emit &&emit)
{
    if (start >= end) return;
    // the sequence holding unit `start`: the largest b with pref[b] <= start
    int lo = 0, hi = batch - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pref[mid] <= start) lo = mid; else hi = mid - 1;
    }
    int b = lo, x = start;
    while (x < end) {
        while (pref[b + 1] <= x) ++b;
        const int a0 = pref[b], e0 = pref[b + 1];
        const int f = a0 + (b > 0 ? cost : 0);
        const int x0 = max(x, f), x1 = min(end, e0);
        if (x0 < x1) emit(b, x0, x1, f, e0, start >= a0 ? 0 : 1);
        x = x1;
    }
}

__device__ __forceinline__ int block_scan_exclusive(int v, int *tmp, int &total)
{
    // Hillis-Steele over the workgroup through LDS (once per step; simple)
    const int t = threadIdx.x;
    tmp[t] = v;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
        const int u = t >= off ? tmp[t - off] : 0;
        __syncthreads();
        tmp[t] += u;
        __syncthreads();
    }
    const int incl = tmp[t];
    total = tmp[kPlanThreads - 1];
    __syncthreads();
    return incl - v;
}

__global__ __launch_bounds__(kPlanThreads) void q8_step_plan_kernel(DecodeParams p, int32_t *plan)
{
    __shared__ int pref[kMaxBatch + 1];
    __shared__ int lens[kMaxBatch];
    __shared__ int scan_tmp[kPlanThreads];
    const StepPlanLayout L = step_plan_layout(p.batch, p.nparts);
    build_prefix(p, pref, lens, true);
    const int total = pref[p.batch];
    for (int b = threadIdx.x; b <= p.batch; b += blockDim.x) plan[L.pref + b] = pref[b];

    // the empty sequences, in order (one wave, 64 at a time with ballots)
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        int count = 0;
        for (int b0 = 0; b0 < p.batch; b0 += 64) {
            const int b = b0 + lane;
            const bool empty = b < p.batch && pref[b + 1] == pref[b];
            const uint64_t m = __builtin_amdgcn_ballot_w64(empty);
            if (empty) plan[L.empty + count + __builtin_popcountll(m & ((1ull << lane) - 1))] = b;
            count += __builtin_popcountll(m);
        }
        if (lane == 0) plan[kPhEmpty] = count;
    }

    // pass 1: pieces per range, scanned into the range offsets
    int carry = 0;
    for (int i0 = 0; i0 < p.nparts; i0 += kPlanThreads) {
        const int i = i0 + (int)threadIdx.x;
        int c = 0;
        if (i < p.nparts)
            range_pieces(pref, p.batch, p.piece_cost, part_start(i, total, p.nparts), part_start(i + 1, total, p.nparts),
                         [&](int, int, int, int, int, int) { ++c; });
        int chunk;
        const int off = block_scan_exclusive(c, scan_tmp, chunk);
        if (i < p.nparts) plan[L.range + i] = carry + off;
        carry += chunk;
    }
    if (threadIdx.x == 0) plan[L.range + p.nparts] = carry;
    __syncthreads();

    // pass 2: the pieces and the block ids they start with
    const int log2bs = p.cache.kv_bs_log2;
    for (int i = threadIdx.x; i < p.nparts; i += blockDim.x) {
        int j = plan[L.range + i];
        range_pieces(pref, p.batch, p.piece_cost, part_start(i, total, p.nparts), part_start(i + 1, total, p.nparts),
                     [&](int b, int x0, int x1, int f, int e0, int slot) {
                         const int n = lens[b];
                         const int lt0 = x0 - f;
                         const int32_t *bt = p.block_table + (size_t)b * p.max_blocks_per_seq;
                         int32_t *pc = plan + L.pieces + (size_t)j * kPieceInts;
                         pc[kPfSeq] = b;
                         pc[kPfT0] = lt0;
                         pc[kPfT1] = x1 - f;
                         pc[kPfLen] = n;
                         pc[kPfFlags] = ((x0 == f && x1 == e0) ? kPieceWhole : 0) | (slot ? kPieceSlot1 : 0) |
                                        (x1 == e0 ? kPieceAppend : 0);
                         pc[kPfAppendBlk] = bt[(n - 1) >> log2bs];
                         for (int kk = 0; kk < 4; ++kk)
                             pc[kPfFirstBlk + kk] = bt[min(lt0 * kTile + kSub * kk, n - 1) >> log2bs];
                         ++j;
                     });
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        plan[kPhBatch] = p.batch;
        plan[kPhParts] = p.nparts;
        plan[kPhKvBsLog2] = p.cache.kv_bs_log2;
        plan[kPhPieceCost] = p.piece_cost;
        plan[kPhTotal] = total;
        plan[kPhMaxSeqLen] = p.max_seq_len;
        plan[kPhMagic] = kPlanMagic;   // written last: a plan cut short is refused
    }
}

size_t step_plan_bytes(const q8_batch &batch, int nparts)
{
    return step_plan_layout(batch.batch, nparts).words * sizeof(int32_t);
}

hipError_t launch_step_plan(const q8_kv_layer &layer, const q8_batch &batch, int nq, const DecodePlan &plan,
                            void *plan_buf, int32_t *dev_status, hipStream_t stream)
{
    q8_batch unplanned = batch;
    unplanned.plan = nullptr;
    DecodeParams p = fill_decode_params(layer, unplanned, nq, nullptr, 1.0f, nullptr, plan, nullptr, dev_status);
    hipLaunchKernelGGL(q8_step_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, p, static_cast<int32_t *>(plan_buf));
    return hipGetLastError();
}

}  // namespace q8kv
