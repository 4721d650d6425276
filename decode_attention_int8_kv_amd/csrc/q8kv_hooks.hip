// q8kv_hooks.hip -- test hooks that expose intermediate integers of the
// decode path, computed by the same device routines the decode kernel runs:
//   q8_quantize_q       : the 32-block query quantizer ("9-2
//                         flash_attn_single_q_q8_neon" §2 segment 1), in
//                         either of the decode's two lane layouts;
//   q8_qk_block_partials: the exact int32 block sums of Q codes against the
//                         K codes of every visible token (§2 segment 2), and
//                         the Q codes and scales behind them, by the routine
//                         and operand layout q8_decode_attn uses for the
//                         shape: sdot4 over two lanes per 32-block, or the
//                         i8 matrix-core path at four query heads per KV
//                         head with kv_bs >= 32.
#include "q8kv_tile.hpp"
#include "q8kv_internal.hpp"

namespace q8kv {

// One wave per 128-element row.  Two lanes per block (Q8_QPATH_VALU): lane
// (slot, c) quantizes elements [16c, 16c + 16), slot-0 lanes write.  One lane
// per block (Q8_QPATH_MFMA): the four rows of a group of four query heads
// share a wave, lane (lg, j) with lg = 0 quantizes block j % 4 of row j / 4
// (the decode's A-operand layout).
__global__ __launch_bounds__(256) void q8_quantize_q_kernel(const float *__restrict__ q, int32_t rows, int32_t path,
                                                             int8_t *__restrict__ codes, float *__restrict__ qscale)
{
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (path == Q8_QPATH_VALU) {
        const int row = wave, c = lane & 7;
        if (row >= rows) return;
        uint4 cd;
        float qs;
        quantize_q_quarter(q + (size_t)row * kHeadDim, c, cd, qs);
        if (lane < 8) {
            *reinterpret_cast<uint4 *>(codes + (size_t)row * kHeadDim + 16 * c) = cd;
            if ((c & 1) == 0) qscale[(size_t)row * (kHeadDim / kQBlock) + (c >> 1)] = qs;
        }
        return;
    }
    // four rows per wave; a group past the end reads row 0 and writes nothing
    const int r0 = 4 * wave;
    if (r0 >= rows) return;
    const int j = lane & 15, row = r0 + (j >> 2);
    const bool live = row < rows;
    float4 qv[8];
    mf_load_query(q + (size_t)(live ? r0 : 0) * kHeadDim, live ? lane : (lane & 3), qv);
    MfQuery mq;
    uint4 lo, hi;
    float step;
    mf_query_operands(qv, lane, mq, lo, hi, step);
    if (lane < 16 && live) {
        uint4 *dst = reinterpret_cast<uint4 *>(codes + (size_t)row * kHeadDim + 32 * (j & 3));
        dst[0] = lo;
        dst[1] = hi;
        qscale[(size_t)row * (kHeadDim / kQBlock) + (j & 3)] = step;
    }
}

hipError_t launch_quantize_q(const float *q, int32_t rows, int32_t path, int8_t *codes, float *qscale,
                             hipStream_t stream)
{
    const int waves = path == Q8_QPATH_VALU ? rows : (rows + 3) / 4;
    hipLaunchKernelGGL(q8_quantize_q_kernel, dim3((waves + 3) / 4), dim3(256), 0, stream, q, rows, path, codes,
                       qscale);
    return hipGetLastError();
}

struct PartialsParams {
    CacheView cache;
    const int32_t *block_table;
    const int32_t *seq_lens;
    const float *q;
    int32_t *partials;
    int8_t *qcodes;     // [batch][nq][128], or null
    float *qscale;      // [batch][nq][4], or null
    int32_t *dev_status;
    int32_t nq;
    int32_t group;
    int32_t max_blocks_per_seq;
    int32_t max_seq_len;
};

__device__ __forceinline__ int hook_len(const PartialsParams &p, int b, int kh, int lane)
{
    int n = p.seq_lens[b];
    if (n < 0 || n > p.max_seq_len) {
        if (lane == 0 && p.dev_status && blockIdx.y == 0 && kh == 0) atomicOr(p.dev_status, kDevBadSeqLen);
        n = 0;
    }
    return uniform(n);
}

// The decode's two-lanes-per-block path.  Grid: (batch * nkv, tiles of
// max_seq_len).  One wave per (sequence, KV head, tile); for each of the G
// query heads, lanes with even c hold the exact sum of block c/2 for their
// token after block_partial.
__global__ __launch_bounds__(64) void q8_qk_partials_kernel(PartialsParams p)
{
    const int b = blockIdx.x / p.cache.nkv, kh = blockIdx.x - b * p.cache.nkv;
    const int lane = threadIdx.x, c = lane & 7, slot = lane >> 3;
    const int t0 = blockIdx.y * kTile;
    const int n = hook_len(p, b, kh, lane);
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
        if (p.qcodes && blockIdx.y == 0 && lane < 8) {
            *reinterpret_cast<uint4 *>(p.qcodes + ((size_t)b * p.nq + h) * kHeadDim + 16 * c) = qc;
            if ((c & 1) == 0) p.qscale[((size_t)b * p.nq + h) * (kHeadDim / kQBlock) + (c >> 1)] = qs;
        }
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

// The decode's matrix-core path (four query heads per KV head, kv_bs >= 32):
// the same query operands, tile loads and i8 MFMAs as the decode kernel;
// lane (lg, j) writes the four partials of head lg with tokens t0 + j and
// t0 + 16 + j.
__global__ __launch_bounds__(64) void q8_qk_partials_mf_kernel(PartialsParams p)
{
    const int b = blockIdx.x / p.cache.nkv, kh = blockIdx.x - b * p.cache.nkv;
    const int lane = threadIdx.x, j = lane & 15, lg = lane >> 4;
    const int t0 = blockIdx.y * kTile;
    const int n = hook_len(p, b, kh, lane);
    TileBlocks tb;
    fetch_blocks(p.block_table + (size_t)b * p.max_blocks_per_seq, p.cache.kv_bs_log2, t0, n, tb);
    Tile t;
    const LaneOffsets lo = lane_offsets(p.cache, kh, lane);
    load_tile_mf(p.cache, tb, lo, lane, t0, n, p.dev_status, t);
    float4 qv[8];
    mf_load_query(p.q + ((size_t)b * p.nq + kh * 4) * kHeadDim, lane, qv);
    MfQuery mq;
    uint4 qlo, qhi;
    float step;
    mf_query_operands(qv, lane, mq, qlo, qhi, step);
    if (p.qcodes && blockIdx.y == 0 && lane < 16) {
        const size_t h = (size_t)b * p.nq + kh * 4 + (j >> 2);
        uint4 *dst = reinterpret_cast<uint4 *>(p.qcodes + h * kHeadDim + 32 * (j & 3));
        dst[0] = qlo;
        dst[1] = qhi;
        p.qscale[h * (kHeadDim / kQBlock) + (j & 3)] = step;
    }
    int32_t *dst = p.partials + ((size_t)b * p.nq + kh * 4 + lg) * (size_t)p.max_seq_len * (kHeadDim / kQBlock);
#pragma unroll
    for (int m = 0; m < 2; ++m) {
        const v4i_mf acc = mf_block_partials(mq, t.k, m);
        const int tok = t0 + 16 * m + j;
        if (tok < p.max_seq_len) {
            const bool ok = (t.svalid >> m) & 1u;
            *reinterpret_cast<int4 *>(dst + (size_t)tok * (kHeadDim / kQBlock)) =
                ok ? make_int4(acc[0], acc[1], acc[2], acc[3]) : make_int4(0, 0, 0, 0);
        }
    }
}

hipError_t launch_qk_partials(const q8_kv_layer &layer, const q8_batch &batch, int nq, const float *q,
                              int32_t *partials, int8_t *qcodes, float *qscale, int32_t *dev_status,
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
    p.qcodes = qcodes;
    p.qscale = qscale;
    p.dev_status = dev_status;
    p.nq = nq;
    p.group = nq / layer.nkv_heads;
    p.max_blocks_per_seq = batch.max_blocks_per_seq;
    p.max_seq_len = batch.max_seq_len;
    // at least one tile row, so the Q codes are written even when every sequence is empty
    const dim3 grid(batch.batch * layer.nkv_heads, (batch.max_seq_len + kTile - 1) / kTile + (batch.max_seq_len == 0));
    if (decode_uses_mfma_scores(p.group, layer.kv_bs))
        hipLaunchKernelGGL(q8_qk_partials_mf_kernel, grid, dim3(64), 0, stream, p);
    else
        hipLaunchKernelGGL(q8_qk_partials_kernel, grid, dim3(64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace q8kv
