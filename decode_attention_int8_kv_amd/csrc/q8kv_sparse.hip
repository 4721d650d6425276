// q8kv_sparse.hip -- block-sparse decode attention over the q8 cache.
//
// Method ("why long context must be sparse" §1-§2): the history is cut into
// 32-token blocks; a cheap probe finds, per query head, the k blocks most
// worth attending to (8 probe rows per block, "max-dot fusion"); exact
// attention then runs over the tokens of those k blocks only.  Sequences of
// at most k blocks (which includes every sequence of at most two blocks, the
// page's gate, since k >= 2) keep every block.  Readings where the page
// defers to another: probe rows 0, 4, ..., 28 of a block; a block's
// importance is the largest q8 attention score of its probe rows, computed
// with the decode kernel's fp32 score formula; selection per query head,
// ties to the lower block index, nothing forced in.
//
// Kernels:
//   probe  -- one wave per (sequence, KV head, 16 blocks): lane (slot, c)
//             reads bytes [16c, 16c + 16) of probe row 4 slot, so one load
//             covers a block's 8 probes; every query head of the KV head
//             gets the block's score (max over the 8 probes).
//   attend -- one 4-wave workgroup per (sequence, query head): top-k by an
//             8-pass radix select on 64-bit keys (score, then lower index),
//             the chosen blocks sorted ascending, each wave attends over
//             every fourth chosen block (the q8 single pass of "9-2
//             flash_attn_single_q_q8_neon" §2), and the four partial states
//             are combined in wave order (the same rescale rule) and divided
//             once.
#include "q8kv_tile.hpp"
#include "q8kv_internal.hpp"

namespace q8kv {

constexpr int kSparseBlock = 32;        // positions per sparse block
constexpr int kProbeStride = 4;         // probe rows 0, 4, ..., 28
constexpr int kProbeBlocksPerWave = 16;
constexpr int kSparseWaves = 4;

struct SparseParams {
    CacheView cache;
    const int32_t *block_table;
    const int32_t *seq_lens;
    const float *q;
    float *out;
    float *scores;        // [batch][nq][max_nb] block scores
    int32_t *selected;    // [batch][nq][topk] chosen blocks, or null
    int32_t *dev_status;
    int32_t batch, nq, max_blocks_per_seq, max_seq_len, max_nb, topk;
    float sc;             // softmax scale * log2(e)
};

__device__ __forceinline__ int sparse_len(const SparseParams &p, int b)
{
    const int n = p.seq_lens[b];
    return (n < 0 || n > p.max_seq_len) ? 0 : n;
}

// ------------------------------------------------------------------ probe --
template <int G>
__global__ __launch_bounds__(64 * kSparseWaves) void q8_sparse_probe_kernel(SparseParams p)
{
    const int nkv = p.cache.nkv;
    const int b = blockIdx.x / nkv, kh = blockIdx.x - (blockIdx.x / nkv) * nkv;
    const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int slot = lane >> 3, c = lane & 7;
    const int n = uniform(sparse_len(p, b));
    const int nb = (n + kSparseBlock - 1) / kSparseBlock;
    if (nb <= p.topk) return;   // every block is kept: nothing to probe
    const int j0 = (blockIdx.y * kSparseWaves + wave) * kProbeBlocksPerWave;
    if (j0 >= nb) return;

    uint4 qc[G];
    float qs[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
        quantize_q_quarter(p.q + ((size_t)b * p.nq + kh * G + g) * kHeadDim, c, qc[g], qs[g]);

    const int32_t *bt = p.block_table + (size_t)b * p.max_blocks_per_seq;
    const int log2bs = p.cache.kv_bs_log2, mask = (1 << log2bs) - 1;
    const int row_bytes = nkv * kHeadDim;
    int blk[kProbeBlocksPerWave];
#pragma unroll
    for (int i = 0; i < kProbeBlocksPerWave; ++i) {
        const int t = (j0 + i) * kSparseBlock + kProbeStride * slot;
        blk[i] = (t < n) ? bt[t >> log2bs] : -1;
    }
    uint4 kc[kProbeBlocksPerWave];
    float ks[kProbeBlocksPerWave];
    bool bad = false;
#pragma unroll
    for (int i = 0; i < kProbeBlocksPerWave; ++i) {
        const int t = (j0 + i) * kSparseBlock + kProbeStride * slot;
        const bool good = (unsigned)blk[i] < (unsigned)p.cache.num_blocks;
        bad = bad || (t < n && !good);
        if (t < n && good) {
            const size_t row = ((size_t)blk[i] << log2bs) + (t & mask);
            kc[i] = *reinterpret_cast<const uint4 *>(p.cache.k_codes + row * row_bytes + kh * kHeadDim + 16 * c);
            ks[i] = p.cache.k_scale[(((size_t)blk[i] * nkv + kh) << log2bs) + (t & mask)];
        } else {
            kc[i] = make_uint4(0, 0, 0, 0);
            ks[i] = 0.0f;
            blk[i] = -1;
        }
    }
    if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0 && p.dev_status) atomicOr(p.dev_status, kDevBadBlockId);

#pragma unroll
    for (int i = 0; i < kProbeBlocksPerWave; ++i) {
        const int j = j0 + i;
        if (j >= nb) break;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            // the decode kernel's score, step for step: per 32-block
            // x = P * qscale, y = (x0 + x1) + (x3 + x2), s = y * (kscale * sc)
            float x = (float)block_partial(kc[i], qc[g]) * qs[g];
            x += dpp_f<kDppQuadXor2>(x);
            x += dpp_f<kDppHalfMirror>(x);
            const float f = ks[i] * p.sc;
            const float s = blk[i] >= 0 ? x * f : -INFINITY;
            const float m = max_over_slots(s);
            if (lane == 0) p.scores[((size_t)b * p.nq + kh * G + g) * p.max_nb + j] = m;
        }
    }
}

// ----------------------------------------------------------------- attend --
__device__ __forceinline__ uint64_t block_key(float s, int j)
{
    const uint32_t u = __float_as_uint(s);
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // order-preserving
    return ((uint64_t)ord << 32) | (uint64_t)(0xffffffffu - (uint32_t)j);   // ties: lower index first
}

template <bool Big>
__global__ __launch_bounds__(64 * kSparseWaves) void q8_sparse_attend_kernel(SparseParams p)
{
    __shared__ uint32_t hist[256];
    __shared__ uint64_t s_prefix;
    __shared__ int s_need, s_cnt;
    __shared__ int sel[64];
    __shared__ float sh_m[kSparseWaves], sh_s[kSparseWaves];
    __shared__ float sh_acc[kSparseWaves][kHeadDim];

    const int b = blockIdx.x / p.nq, h = blockIdx.x - (blockIdx.x / p.nq) * p.nq;
    const int G = p.nq / p.cache.nkv, kh = h / G;
    const int tid = threadIdx.x;
    const int wave = uniform(tid >> 6), lane = tid & 63, tslot = lane >> 3, c = lane & 7;
    int n = p.seq_lens[b];
    if (n < 0 || n > p.max_seq_len) {
        if (h == 0 && tid == 0 && p.dev_status) atomicOr(p.dev_status, kDevBadSeqLen);
        n = 0;
    }
    n = uniform(n);
    float *o = p.out + ((size_t)b * p.nq + h) * kHeadDim;
    const int nb = (n + kSparseBlock - 1) / kSparseBlock;

    // ---- which blocks
    if (nb <= p.topk) {
        if (tid < 64) sel[tid] = tid;
        if (tid == 0) s_cnt = nb;
    } else {
        const float *sc = p.scores + ((size_t)b * p.nq + h) * p.max_nb;
        if (tid == 0) {
            s_prefix = 0;
            s_need = p.topk;
        }
        uint64_t mask = 0;
        for (int pass = 0; pass < 8; ++pass) {
            const int shift = 56 - 8 * pass;
            hist[tid] = 0;
            __syncthreads();
            const uint64_t prefix = s_prefix;
            for (int j = tid; j < nb; j += 64 * kSparseWaves) {
                const uint64_t key = block_key(sc[j], j);
                if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xff], 1u);
            }
            __syncthreads();
            if (tid == 0) {
                // the digit of the need-th largest key among those matching the prefix
                int need = s_need, d = 255;
                for (; d > 0; --d) {
                    const int hcount = (int)hist[d];
                    if (hcount >= need) break;
                    need -= hcount;
                }
                s_need = need;
                s_prefix = prefix | ((uint64_t)d << shift);
            }
            mask |= (uint64_t)0xff << shift;
            __syncthreads();
        }
        // keys are distinct, so exactly topk keys are >= the topk-th largest
        const uint64_t kth = s_prefix;
        if (tid == 0) s_cnt = 0;
        __syncthreads();
        for (int j = tid; j < nb; j += 64 * kSparseWaves)
            if (block_key(sc[j], j) >= kth) sel[atomicAdd(&s_cnt, 1)] = j;
        __syncthreads();
        if (tid < 64) {
            // ascending block order: bitonic sort over the 64 lanes of wave 0
            int v = tid < s_cnt ? sel[tid] : 0x7fffffff;
            for (int k = 2; k <= 64; k <<= 1)
                for (int jj = k >> 1; jj > 0; jj >>= 1) {
                    const int u = __shfl_xor(v, jj, 64);
                    const bool up = ((tid & k) == 0);
                    const bool lower = (tid & jj) == 0;
                    v = (lower == up) ? min(v, u) : max(v, u);
                }
            sel[tid] = v;
        }
    }
    __syncthreads();
    const int cnt = s_cnt;
    if (p.selected && tid < p.topk)
        p.selected[((size_t)b * p.nq + h) * p.topk + tid] = tid < cnt ? sel[tid] : -1;

    // ---- exact attention over the chosen blocks: wave w takes every fourth
    uint4 qc;
    float qs;
    quantize_q_quarter(p.q + ((size_t)b * p.nq + h) * kHeadDim, c, qc, qs);
    const LaneOffsets lo = lane_offsets(p.cache, kh, lane);
    const int32_t *bt = p.block_table + (size_t)b * p.max_blocks_per_seq;
    const int log2bs = p.cache.kv_bs_log2;
    float M = -INFINITY, S = 0.0f, acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = 0.0f;

    auto process = [&](const Tile &t) {
        float ks[4], vs[4];
        tile_scales<0>(t, c, ks[0], vs[0]);
        tile_scales<1>(t, c, ks[1], vs[1]);
        tile_scales<2>(t, c, ks[2], vs[2]);
        tile_scales<3>(t, c, ks[3], vs[3]);
        float s[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bool ok = (t.valid >> kk) & 1u;
            float x = (float)block_partial(t.k[kk], qc) * qs;
            x += dpp_f<kDppQuadXor2>(x);
            x += dpp_f<kDppHalfMirror>(x);
            s[kk] = ok ? x * (ks[kk] * p.sc) : -INFINITY;
        }
        float m = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
        m = max_over_slots(m);
        if (m > M) {
            const float a = __builtin_amdgcn_exp2f(M - m);
            S *= a;
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[j] *= a;
            M = m;
        }
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bool ok = (t.valid >> kk) & 1u;
            // masked tokens contribute nothing (their scale may be any bit pattern)
            const float pw = ok ? __builtin_amdgcn_exp2f(s[kk] - M) : 0.0f;
            S += pw;
            const float w = ok ? pw * vs[kk] : 0.0f;
            const uint32_t words[4] = {t.v[kk].x, t.v[kk].y, t.v[kk].z, t.v[kk].w};
#pragma unroll
            for (int j = 0; j < 16; ++j) acc[j] = fmaf(w, byte_f(words[j >> 2], j & 3), acc[j]);
        }
    };

    // this wave's blocks: sel[wave], sel[wave + 4], ...; tile i of the wave is
    // block sel[wave + 4 i]; a tile past the list loads nothing
    const int mine = cnt > wave ? (cnt - wave + kSparseWaves - 1) / kSparseWaves : 0;
    auto tile_t0 = [&](int i) { return i < mine ? sel[wave + kSparseWaves * i] * kSparseBlock : 0; };
    auto tile_n = [&](int i) { return i < mine ? n : 0; };
    Tile ta, tb;
    TileBlocks ba, bb;
    if (mine > 0) {
        fetch_blocks(bt, log2bs, tile_t0(0), tile_n(0), ba);
        load_tile<true, Big>(p.cache, ba, lo, lane, tile_t0(0), tile_n(0), p.dev_status, ta);
        fetch_blocks(bt, log2bs, tile_t0(1), tile_n(1), bb);
        int i = 0;
        while (true) {
            load_tile<true, Big>(p.cache, bb, lo, lane, tile_t0(i + 1), tile_n(i + 1), p.dev_status, tb);
            fetch_blocks(bt, log2bs, tile_t0(i + 2), tile_n(i + 2), ba);
            process(ta);
            if (++i >= mine) break;
            load_tile<true, Big>(p.cache, ba, lo, lane, tile_t0(i + 1), tile_n(i + 1), p.dev_status, ta);
            fetch_blocks(bt, log2bs, tile_t0(i + 2), tile_n(i + 2), bb);
            process(tb);
            if (++i >= mine) break;
        }
    }
    S = sum_over_slots(S);
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = sum_over_slots(acc[j]);

    // ---- combine the waves in wave order, divide once
    if (lane == 0) {
        sh_m[wave] = M;
        sh_s[wave] = S;
    }
    if (tslot == 0) {
#pragma unroll
        for (int j = 0; j < 16; ++j) sh_acc[wave][16 * c + j] = acc[j];
    }
    __syncthreads();
    if (tid >= 64) return;
    float mx = -INFINITY;
    for (int w = 0; w < kSparseWaves; ++w) mx = fmaxf(mx, sh_m[w]);
    float st = 0.0f, a0 = 0.0f, a1 = 0.0f;
    if (mx != -INFINITY) {
        for (int w = 0; w < kSparseWaves; ++w) {
            const float f = __builtin_amdgcn_exp2f(sh_m[w] - mx);   // 0 for a wave with no tokens
            st = fmaf(sh_s[w], f, st);
            a0 = fmaf(sh_acc[w][2 * lane], f, a0);
            a1 = fmaf(sh_acc[w][2 * lane + 1], f, a1);
        }
    }
    reinterpret_cast<float2 *>(o)[lane] = st > 0.0f ? make_float2(a0 / st, a1 / st) : make_float2(0.0f, 0.0f);
}

// ------------------------------------------------------------------- host --
size_t sparse_workspace_bytes(const q8_batch &batch, int nq)
{
    const size_t max_nb = (size_t)((batch.max_seq_len + kSparseBlock - 1) / kSparseBlock);
    return ((size_t)batch.batch * nq * (max_nb > 0 ? max_nb : 1) * sizeof(float) + 255) / 256 * 256;
}

hipError_t launch_sparse(const q8_kv_layer &layer, const q8_batch &batch, int nq, const float *q, float scale,
                         float *out, int topk, int32_t *selected, void *workspace, int32_t *dev_status,
                         hipStream_t stream)
{
    SparseParams p;
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
    p.out = out;
    p.scores = static_cast<float *>(workspace);
    p.selected = selected;
    p.dev_status = dev_status;
    p.batch = batch.batch;
    p.nq = nq;
    p.max_blocks_per_seq = batch.max_blocks_per_seq;
    p.max_seq_len = batch.max_seq_len;
    p.max_nb = (batch.max_seq_len + kSparseBlock - 1) / kSparseBlock;
    if (p.max_nb < 1) p.max_nb = 1;
    p.topk = topk;
    p.sc = (float)((double)scale * 1.4426950408889634);

    if (p.max_nb > topk) {
        const dim3 grid(batch.batch * layer.nkv_heads,
                        (p.max_nb + kSparseWaves * kProbeBlocksPerWave - 1) / (kSparseWaves * kProbeBlocksPerWave));
        const void *fn;
        switch (nq / layer.nkv_heads) {
        case 1: fn = reinterpret_cast<const void *>(&q8_sparse_probe_kernel<1>); break;
        case 2: fn = reinterpret_cast<const void *>(&q8_sparse_probe_kernel<2>); break;
        case 4: fn = reinterpret_cast<const void *>(&q8_sparse_probe_kernel<4>); break;
        default: fn = reinterpret_cast<const void *>(&q8_sparse_probe_kernel<8>); break;
        }
        void *args[] = {&p};
        const hipError_t e = hipLaunchKernel(fn, grid, dim3(64 * kSparseWaves), args, 0, stream);
        if (e != hipSuccess) return e;
    }
    const void *fa = layer.kv_bs >= kTile ? reinterpret_cast<const void *>(&q8_sparse_attend_kernel<true>)
                                          : reinterpret_cast<const void *>(&q8_sparse_attend_kernel<false>);
    void *args[] = {&p};
    const hipError_t e = hipLaunchKernel(fa, dim3(batch.batch * nq), dim3(64 * kSparseWaves), args, 0, stream);
    return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace q8kv
