// q8kv_hooks.hip -- test hooks that expose intermediate integers of the
// decode path, computed by the same device routines the decode kernel runs:
//   q8_quantize_q       : the 32-block query quantizer ("9-2
//                         flash_attn_single_q_q8_neon" §2 segment 1);
//   q8_qk_block_partials: the exact int32 block sums of Q codes against the
//                         K codes of every visible token (§2 segment 2).
#include "q8kv_tile.hpp"
#include "q8kv_internal.hpp"

namespace q8kv {

// One wave per 128-element row, lane layout of the decode kernel: lane
// (slot, c) quantizes elements [16c, 16c + 16); slot-0 lanes write.
__global__ __launch_bounds__(256) void q8_quantize_q_kernel(const float *__restrict__ q, int32_t rows,
                                                             int8_t *__restrict__ codes,
                                                             float *__restrict__ qscale)
{
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, c = lane & 7;
    if (row >= rows) return;
    uint4 cd;
    float qs;
    quantize_q_quarter(q + (size_t)row * kHeadDim, c, cd, qs);
    if (lane < 8) {
        *reinterpret_cast<uint4 *>(codes + (size_t)row * kHeadDim + 16 * c) = cd;
        if ((c & 1) == 0) qscale[(size_t)row * (kHeadDim / kQBlock) + (c >> 1)] = qs;
    }
}

hipError_t launch_quantize_q(const float *q, int32_t rows, int8_t *codes, float *qscale,
                             hipStream_t stream)
{
    hipLaunchKernelGGL(q8_quantize_q_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, q, rows, codes,
                       qscale);
    return hipGetLastError();
}

struct PartialsParams {
    CacheView cache;
    const int32_t *block_table;
    const int32_t *seq_lens;
    const float *q;
    int32_t *partials;
    int32_t *dev_status;
    int32_t nq;
    int32_t group;
    int32_t max_blocks_per_seq;
    int32_t max_seq_len;
};

// Grid: (batch * nkv, tiles of max_seq_len).  One wave per (sequence, KV head,
// tile); for each of the G query heads, lanes with even c hold the exact sum
// of block c/2 for their token after block_partial.
__global__ __launch_bounds__(64) void q8_qk_partials_kernel(PartialsParams p)
{
    const int b = blockIdx.x / p.cache.nkv, kh = blockIdx.x - b * p.cache.nkv;
    const int lane = threadIdx.x, c = lane & 7, slot = lane >> 3;
    const int t0 = blockIdx.y * kTile;
    int n = p.seq_lens[b];
    if (n < 0 || n > p.max_seq_len) {
        if (lane == 0 && p.dev_status && blockIdx.y == 0 && kh == 0) atomicOr(p.dev_status, kDevBadSeqLen);
        n = 0;
    }
    n = uniform(n);
    TileBlocks tb;
    fetch_blocks(p.block_table + (size_t)b * p.max_blocks_per_seq, p.cache.kv_bs_log2, t0, n, tb);
    Tile t;
    const LaneOffsets lo = lane_offsets(p.cache, kh, lane);
    load_tile<false, false>(p.cache, tb, lo, lane, t0, n, p.dev_status, t);
    for (int g = 0; g < p.group; ++g) {
        const int h = kh * p.group + g;
        uint4 qc;
        float qs;
        quantize_q_quarter(p.q + ((size_t)b * p.nq + h) * kHeadDim, c, qc, qs);
        int32_t *dst = p.partials + ((size_t)b * p.nq + h) * (size_t)p.max_seq_len * (kHeadDim / kQBlock);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int tok = t0 + kSub * kk + slot;
            const int pb = block_partial(t.k[kk], qc);
            if ((c & 1) == 0 && tok < p.max_seq_len)
                dst[(size_t)tok * (kHeadDim / kQBlock) + (c >> 1)] = ((t.valid >> kk) & 1u) ? pb : 0;
        }
    }
}

hipError_t launch_qk_partials(const q8_kv_layer &layer, const q8_batch &batch, int nq,
                              const float *q, int32_t *partials, int32_t *dev_status,
                              hipStream_t stream)
{
    PartialsParams p;
    p.cache.k_codes = layer.k_codes;
    p.cache.v_codes = layer.v_codes;
    p.cache.k_scale = layer.k_scale;
    p.cache.v_scale = layer.v_scale;
    p.cache.nkv = layer.nkv_heads;
    p.cache.kv_bs_log2 = ilog2(layer.kv_bs);
    p.cache.num_blocks = layer.num_blocks;
    p.block_table = batch.block_table;
    p.seq_lens = batch.seq_lens;
    p.q = q;
    p.partials = partials;
    p.dev_status = dev_status;
    p.nq = nq;
    p.group = nq / layer.nkv_heads;
    p.max_blocks_per_seq = batch.max_blocks_per_seq;
    p.max_seq_len = batch.max_seq_len;
    const dim3 grid(batch.batch * layer.nkv_heads, (batch.max_seq_len + kTile - 1) / kTile);
    if (grid.y == 0) return hipSuccess;
    hipLaunchKernelGGL(q8_qk_partials_kernel, grid, dim3(64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace q8kv
