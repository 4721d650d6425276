// q8kv_append.hip -- kv_quantize_per_head append into the blocked q8 cache.
//
// "9-3 q8 KV 精度对照实验" §2: each new (token, KV head) row of 128 values
// shares one scale, scale = max-abs/127, code = round(v / scale) clamped to
// [-127, 127].  The codes go to block block_table[seq][pos / kv_bs], row
// pos % kv_bs, head offset kh * 128 ("9-2 flash_attn_single_q_q8_neon" §2
// segment 2 layout); the stored scale is the step d.
//
// One wave per (token, group of H KV heads): the group's K and V rows are
// loaded first (2 values per lane and row), while the token's sequence,
// position and block id come from scalar loads on the side, so the
// destination lookups and the row loads overlap.  Per row, a wave max gives
// the exact max-abs, and every lane writes its 2 codes (a 128-byte coalesced
// row).  H grows with the number of rows (more bytes in flight per wave for
// bulk appends, more waves for a decode step's few tokens).  Append traffic
// is tiny next to attention (2112 bytes written per token and layer for 8 KV
// heads).
#include "q8kv_device.hpp"
#include "q8kv_internal.hpp"

namespace q8kv {

struct AppendParams {
    int8_t *k_codes;
    int8_t *v_codes;
    float *k_scale;
    float *v_scale;
    float *k_f32;          // fp32 mirror, or null
    float *v_f32;
    const int32_t *block_table;
    const int32_t *seq_lens;
    const int32_t *tok_seq;
    const int32_t *tok_pos;
    const float *k_new;
    const float *v_new;
    int32_t *dev_status;
    int32_t n_tokens;
    int32_t nkv;
    int32_t kv_bs_log2;
    int32_t num_blocks;
    int32_t batch;
    int32_t max_blocks_per_seq;
};

constexpr int kAppendWaves = 4;   // waves per workgroup

template <int H>
__global__ __launch_bounds__(64 * kAppendWaves) void q8_append_kernel(AppendParams p)
{
    using const_i32 = const __attribute__((address_space(4))) int32_t;
    const int lane = threadIdx.x & 63;
    const int groups = (p.nkv + H - 1) / H;
    const int w = uniform(blockIdx.x * kAppendWaves + (int)(threadIdx.x >> 6));
    if (w >= p.n_tokens * groups) return;
    const int tok = w / groups;
    const int h0 = (w - tok * groups) * H;
    const size_t src = (size_t)tok * p.nkv * kHeadDim + 2 * lane;

    // the rows first (branch-free: a slot past the last head re-reads it)
    float2 k[H], v[H];
#pragma unroll
    for (int j = 0; j < H; ++j) {
        const size_t off = src + (size_t)min(h0 + j, p.nkv - 1) * kHeadDim;
        k[j] = *reinterpret_cast<const float2 *>(p.k_new + off);
        v[j] = *reinterpret_cast<const float2 *>(p.v_new + off);
    }

    // destination of the token (read-only metadata: scalar loads)
    const int seq = ((const_i32 *)p.tok_seq)[tok];
    const int pos = ((const_i32 *)p.tok_pos)[tok];
    int32_t bad = 0;
    int blk = -1;
    if (seq < 0 || seq >= p.batch) {
        bad = kDevBadToken;
    } else {
        const int len = ((const_i32 *)p.seq_lens)[seq];
        const int cap = p.max_blocks_per_seq << p.kv_bs_log2;
        if (pos < 0 || pos >= len || pos >= cap) {
            bad = kDevBadToken;
        } else {
            blk = ((const_i32 *)p.block_table)[(size_t)seq * p.max_blocks_per_seq + (pos >> p.kv_bs_log2)];
            if (blk < 0 || blk >= p.num_blocks) bad = kDevBadBlockId;
        }
    }
    if (bad) {
        if (lane == 0 && p.dev_status) atomicOr(p.dev_status, bad);
        return;
    }

    const int row_in_blk = pos & ((1 << p.kv_bs_log2) - 1);
#pragma unroll
    for (int j = 0; j < H; ++j)
        if (h0 + j < p.nkv)
            append_row_vals(p.k_codes, p.v_codes, p.k_scale, p.v_scale, p.k_f32, p.v_f32, p.nkv, p.kv_bs_log2,
                            blk, row_in_blk, h0 + j, k[j], v[j], lane);
}

// Heads per wave: the most (up to 8) that still leave about 8192 waves.
static int append_heads(long long rows)
{
    int h = 1;
    while (h < 8 && rows / (2 * h) >= 8192) h *= 2;
    return h;
}

hipError_t launch_append(const q8_kv_layer &layer, const q8_batch &batch, int32_t n_tokens,
                         const int32_t *tok_seq, const int32_t *tok_pos, const float *k_new,
                         const float *v_new, int32_t *dev_status, hipStream_t stream)
{
    AppendParams p;
    p.k_codes = layer.k_codes;
    p.v_codes = layer.v_codes;
    p.k_scale = layer.k_scale;
    p.v_scale = layer.v_scale;
    p.k_f32 = layer.k_f32;
    p.v_f32 = layer.v_f32;
    p.block_table = batch.block_table;
    p.seq_lens = batch.seq_lens;
    p.tok_seq = tok_seq;
    p.tok_pos = tok_pos;
    p.k_new = k_new;
    p.v_new = v_new;
    p.dev_status = dev_status;
    p.n_tokens = n_tokens;
    p.nkv = layer.nkv_heads;
    p.kv_bs_log2 = ilog2(layer.kv_bs);
    p.num_blocks = layer.num_blocks;
    p.batch = batch.batch;
    p.max_blocks_per_seq = batch.max_blocks_per_seq;
    const int h = append_heads((long long)n_tokens * layer.nkv_heads);
    const long long waves = (long long)n_tokens * ((layer.nkv_heads + h - 1) / h);
    const dim3 grid((unsigned)((waves + kAppendWaves - 1) / kAppendWaves)), block(64 * kAppendWaves);
    switch (h) {
    case 1: hipLaunchKernelGGL(q8_append_kernel<1>, grid, block, 0, stream, p); break;
    case 2: hipLaunchKernelGGL(q8_append_kernel<2>, grid, block, 0, stream, p); break;
    case 4: hipLaunchKernelGGL(q8_append_kernel<4>, grid, block, 0, stream, p); break;
    default: hipLaunchKernelGGL(q8_append_kernel<8>, grid, block, 0, stream, p); break;
    }
    return hipGetLastError();
}

}  // namespace q8kv
