// q8kv_append.hip -- kv_quantize_per_head append into the blocked q8 cache.
//
// "9-3 q8 KV 精度对照实验" §2: each new (token, KV head) row of 128 values
// shares one scale, scale = max-abs/127, code = round(v / scale) clamped to
// [-127, 127].  The codes go to block block_table[seq][pos / kv_bs], row
// pos % kv_bs, head offset kh * 128 ("9-2 flash_attn_single_q_q8_neon" §2
// segment 2 layout); the stored scale is the step d.
//
// One wave per (token, KV head): each lane holds 2 of the 128 K values and 2
// of the V values, a wave max gives the exact max-abs, and every lane writes
// its 2 codes (a 128-byte coalesced row per wave).  Append traffic is tiny
// next to attention (2112 bytes written per token and layer for 8 KV heads).
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
    int32_t n_rows;        // n_tokens * nkv
    int32_t nkv;
    int32_t kv_bs_log2;
    int32_t num_blocks;
    int32_t batch;
    int32_t max_blocks_per_seq;
};

constexpr int kAppendWaves = 4;

__global__ __launch_bounds__(64 * kAppendWaves) void q8_append_kernel(AppendParams p)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * kAppendWaves + (threadIdx.x >> 6);
    if (row >= p.n_rows) return;
    const int tok = row / p.nkv;
    const int kh = row - tok * p.nkv;

    const int seq = p.tok_seq[tok];
    const int pos = p.tok_pos[tok];
    int32_t bad = 0;
    int blk = -1;
    if (seq < 0 || seq >= p.batch) {
        bad = kDevBadToken;
    } else {
        const int len = p.seq_lens[seq];
        const int cap = p.max_blocks_per_seq << p.kv_bs_log2;
        if (pos < 0 || pos >= len || pos >= cap) {
            bad = kDevBadToken;
        } else {
            blk = p.block_table[(size_t)seq * p.max_blocks_per_seq + (pos >> p.kv_bs_log2)];
            if (blk < 0 || blk >= p.num_blocks) bad = kDevBadBlockId;
        }
    }
    if (bad) {
        if (lane == 0 && p.dev_status) atomicOr(p.dev_status, bad);
        return;
    }

    const size_t src = (size_t)row * kHeadDim;
    append_row(p.k_codes, p.v_codes, p.k_scale, p.v_scale, p.k_f32, p.v_f32, p.nkv, p.kv_bs_log2, blk,
               pos & ((1 << p.kv_bs_log2) - 1), kh, p.k_new + src, p.v_new + src, lane);
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
    p.n_rows = n_tokens * layer.nkv_heads;
    p.nkv = layer.nkv_heads;
    p.kv_bs_log2 = ilog2(layer.kv_bs);
    p.num_blocks = layer.num_blocks;
    p.batch = batch.batch;
    p.max_blocks_per_seq = batch.max_blocks_per_seq;
    const int grid = (p.n_rows + kAppendWaves - 1) / kAppendWaves;
    hipLaunchKernelGGL(q8_append_kernel, dim3(grid), dim3(64 * kAppendWaves), 0, stream, p);
    return hipGetLastError();
}

}  // namespace q8kv
