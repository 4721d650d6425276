// q8kv_sparse.hip -- block-sparse decode attention over the q8 cache.
//
// Method ("why long context must be sparse" §1-§2): the history is cut into
// 32-token blocks; a cheap probe finds, per query head, the k blocks most
// worth attending to (8 probe rows per block, "max-dot fusion"); exact
// attention then runs over the tokens of those k blocks only.  Sequences of
// at most k blocks (which includes every sequence of at most two blocks, the
// page's gate, since k >= 2) keep every block.  Readings where the page
// defers to another: probe rows 0, 4, ..., 28 of a block; a block's
// importance is the largest q8 attention score of its probe rows ("9-2
// flash_attn_single_q_q8_neon" §2 segment 2: s = (sum over 32-blocks of
// P_b * qscale_b) * kscale * scale); selection per query head, ties to the
// lower block index, nothing forced in.  The probe evaluates s in fp32 with
// every product and sum rounded on its own (x_b = P_b * qscale_b exact
// partials, y = (x0 + x1) + (x3 + x2), s = y * (kscale * sc), sc = scale *
// log2 e, a positive factor common to all blocks), so its value lies within
// about 5 * 2^-24 * scale * kscale * sum_b |x_b| of the exact score, and the
// kept set is the exact top k up to blocks whose scores lie that close.
//
// Kernels (one call enqueues them in this order):
//   probe  -- one wave per (sequence, KV head, 16 blocks), the waves of a
//             workgroup being up to 4 KV heads of the same 16 blocks.  The int8 dot products of the
//             probe rows with up to 4 query heads at once run on the matrix
//             cores (i8 MFMA, one 32-block per k-group, so every 32-block
//             partial comes out exact and separate); the fp32 score and the
//             max over a block's 8 probe rows follow in the lanes.
//   select -- one wave per (sequence, query head): a lower bound of the
//             k-th largest score from the 64 lanes' maxima keeps only a few
//             candidates; the k-th largest of those is found bit by bit
//             with ballot counts (no atomics); the blocks above it and the
//             lowest-index ones equal to it are written in ascending order.
//   attend -- P workgroups of 4 waves per (sequence, query head), P chosen
//             from batch x heads so that small batches still fill the GPU;
//             workgroup p takes a contiguous share of the kept blocks, its
//             waves every fourth of them (the q8 single pass of "9-2
//             flash_attn_single_q_q8_neon" §2), and their states are
//             combined in wave order.  With P = 1 the result is written
//             directly, else as a partial (M, S, acc) record.
//   merge  -- P > 1 only: the records of each (sequence, query head)
//             combined in order with the same rescale rule, divided once.
#include "q8kv_tile.hpp"
#include "q8kv_internal.hpp"

namespace q8kv {

constexpr int kSparseBlock = 32;        // positions per sparse block
constexpr int kProbeStride = 4;         // probe rows 0, 4, ..., 28
constexpr int kProbeBlocksPerWave = 16;
constexpr int kProbeWaves = 4;         // KV heads per probe workgroup
constexpr int kSparseWaves = 4;
constexpr int kMaxTopk = 64;
constexpr int kSelLdsKeys = 8192;       // keys the select wave keeps in LDS (32 KB); more are re-read
constexpr int kSelSurvivors = 1024;     // keys at or above the select's lower bound kept in LDS (8 KB)
constexpr int kMaxSparseParts = 8;

struct SparseParams {
    CacheView cache;
    const int32_t *block_table;
    const int32_t *seq_lens;
    const float *q;
    float *out;
    float *scores;        // [batch * nq][max_nb] block scores
    int32_t *sel;         // [batch * nq][kMaxTopk] kept blocks, ascending
    int32_t *cnt;         // [batch * nq] number kept
    float2 *rec_ms;       // [batch * nq][parts] (M, S) of partial states (parts > 1)
    float *rec_acc;       // [batch * nq][parts][128]
    int32_t *selected;    // user copy [batch][nq][topk], or null
    int32_t *dev_status;
    int32_t batch, nq, max_blocks_per_seq, max_seq_len, max_nb, topk, parts;
    int32_t probe_waves, probe_groups;   // probe workgroup: waves = KV heads [g * waves, (g + 1) * waves)
    float sc;             // softmax scale * log2(e)
};

__device__ __forceinline__ int sparse_len(const SparseParams &p, int b)
{
    const int n = p.seq_lens[b];
    return (n < 0 || n > p.max_seq_len) ? 0 : n;
}

// ------------------------------------------------------------------ probe --
typedef int v4i __attribute__((ext_vector_type(4)));

// One wave scores 16 blocks (8 pairs) of one KV head for its G query heads
// with v_mfma_i32_16x16x64_i8 (C = A x B, 16 x 16, k = 64 per step):
//   B (K rows): column j = lane % 16 is probe row 4 (j % 8) of block
//     2 q + j / 8 of the pair; lane group lg = lane / 16 holds bytes
//     [32 lg, 32 lg + 32) of the head's 128, 16 per step;
//   A (queries): row i = 4 g + beta holds query head g's codes of 32-block
//     beta, placed in k-group beta only (zeros elsewhere);
//   so C[4 g + beta][j] is the exact int32 partial of block beta, and lane
//   (lg, j) ends up holding the 4 partials of head lg for its own row j.
// The score then follows the decode formula in one lane: x_beta = P_beta *
// qscale_beta, y = (x0 + x1) + (x3 + x2), s = y * (kscale * sc); the block's
// max over its 8 probe rows is taken across the 8 lanes j % 8 with DPP.
template <int G>
__global__ __launch_bounds__(64 * kProbeWaves) void q8_sparse_probe_kernel(SparseParams p)
{
    constexpr int kSets = G > 4 ? 2 : 1;   // 4 query heads per MFMA
    constexpr int kPairs = kProbeBlocksPerWave / 2;
    const int nkv = p.cache.nkv;
    const int b = blockIdx.x / p.probe_groups, hg = blockIdx.x - (blockIdx.x / p.probe_groups) * p.probe_groups;
    const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int kh = hg * p.probe_waves + wave;
    if (kh >= nkv) return;
    const int n = uniform(sparse_len(p, b));
    const int nb = (n + kSparseBlock - 1) / kSparseBlock;
    if (nb <= p.topk) return;   // every block is kept: nothing to probe
    const int j0 = blockIdx.y * kProbeBlocksPerWave;
    if (j0 >= nb) return;
    const int j = lane & 15, lg = lane >> 4;

    // Rows at or past n are read at the sequence's last row and a bad block
    // id as block 0, so every load is in bounds and all are issued before the
    // first wait; such rows are masked to -inf.
    const int32_t *bt = p.block_table + (size_t)b * p.max_blocks_per_seq;
    const int log2bs = p.cache.kv_bs_log2, mask = (1 << log2bs) - 1;
    const int row_bytes = nkv * kHeadDim;
    auto token = [&](int q) { return (j0 + 2 * q + (j >> 3)) * kSparseBlock + kProbeStride * (j & 7); };
    int id[kPairs];
#pragma unroll
    for (int q = 0; q < kPairs; ++q) id[q] = bt[min(token(q), n - 1) >> log2bs];
    uint4 k0[kPairs], k1[kPairs];
    float ks[kPairs];
    uint32_t valid = 0;
    bool bad = false;
#pragma unroll
    for (int q = 0; q < kPairs; ++q) {
        const int tr = token(q), t = min(tr, n - 1);
        const bool good = (unsigned)id[q] < (unsigned)p.cache.num_blocks;
        bad = bad || (tr < n && !good);
        valid |= (tr < n && good) ? (1u << q) : 0u;
        const size_t blk = good ? (size_t)id[q] : 0;
        const size_t row = (blk << log2bs) + (size_t)(t & mask);
        const int8_t *src = p.cache.k_codes + row * row_bytes + kh * kHeadDim + 32 * lg;
        k0[q] = *reinterpret_cast<const uint4 *>(src);
        k1[q] = *reinterpret_cast<const uint4 *>(src + 16);
        ks[q] = p.cache.k_scale[((blk * nkv + kh) << log2bs) + (size_t)(t & mask)];
    }
    if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0 && p.dev_status) atomicOr(p.dev_status, kDevBadBlockId);

    // the queries are read and quantized while the rows are in flight
    uint4 qa0[kSets], qa1[kSets];
    float qsc[kSets][4];
#pragma unroll
    for (int st = 0; st < kSets; ++st) {
        const int gi = 4 * st + (j >> 2), beta = j & 3;
        uint4 lo = make_uint4(0, 0, 0, 0), hi = lo;
        float step = 0.0f;
        if (gi < G) quantize_q_block(p.q + ((size_t)b * p.nq + kh * G + gi) * kHeadDim + 32 * beta, lo, hi, step);
        const bool mine = lg == beta;
        qa0[st] = mine ? lo : make_uint4(0, 0, 0, 0);
        qa1[st] = mine ? hi : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) qsc[st][r] = __shfl(step, 4 * lg + r, 64);   // head 4 st + lg, block r
    }

#pragma unroll
    for (int q = 0; q < kPairs; ++q) {
        const float f = ks[q] * p.sc;
        const bool ok = (valid >> q) & 1u;
        const int jb = j0 + 2 * q + (j >> 3);
#pragma unroll
        for (int st = 0; st < kSets; ++st) {
            v4i c = {0, 0, 0, 0};
            c = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, qa0[st]), __builtin_bit_cast(v4i, k0[q]),
                                                      c, 0, 0, 0);
            c = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, qa1[st]), __builtin_bit_cast(v4i, k1[q]),
                                                      c, 0, 0, 0);
            float sv;
            {
                // every product and sum rounded on its own (no fused
                // multiply-add), so the error against the exact score stays
                // within the bound stated at the top of this file
#pragma clang fp contract(off)
                const float x0 = (float)c[0] * qsc[st][0], x1 = (float)c[1] * qsc[st][1];
                const float x2 = (float)c[2] * qsc[st][2], x3 = (float)c[3] * qsc[st][3];
                const float y = (x0 + x1) + (x3 + x2);
                sv = ok ? y * f : -INFINITY;
            }
            sv = fmaxf(sv, dpp_f<kDppQuadXor1>(sv));
            sv = fmaxf(sv, dpp_f<kDppQuadXor2>(sv));
            sv = fmaxf(sv, dpp_f<kDppHalfMirror>(sv));   // max over the block's 8 probe rows
            const int g = 4 * st + lg;
            if (g < G && (j & 7) == 0 && jb < nb) p.scores[((size_t)b * p.nq + kh * G + g) * p.max_nb + jb] = sv;
        }
    }
}

// ----------------------------------------------------------------- select --
__device__ __forceinline__ uint32_t score_ord(float s)
{
    const uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);   // -0 ties with +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);   // unsigned order = float order
}

__device__ __forceinline__ int count_true(bool pred) { return __builtin_popcountll(__builtin_amdgcn_ballot_w64(pred)); }

__device__ __forceinline__ int lanes_before(uint64_t mask)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
}

// The largest T with at least k of the list's keys >= T (the k-th largest
// key), found bit by bit; a list item is key(i), i < len.
template <class Key>
__device__ __forceinline__ uint32_t kth_largest(int len, int k, int lane, Key key)
{
    uint32_t T = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand = T | (1u << bit);
        int c = 0;
        for (int i0 = 0; i0 < len && c < k; i0 += 64) c += count_true(i0 + lane < len && key(i0 + lane) >= cand);
        if (c >= k) T = cand;
    }
    return T;
}

// One wave per (sequence, query head).
//  1. Each lane takes the maximum of the keys j = lane mod 64.  The k-th
//     largest of these 64 maxima, L, is at most the k-th largest key T (the
//     k lanes with the largest maxima each hold a key >= L).
//  2. The keys >= L (few, except when many scores are equal) are compacted
//     in index order; T is the k-th largest of them.
//  3. Kept: every key > T, then the lowest-index keys equal to T up to k,
//     written in ascending block order.
// If more than kSelSurvivors keys are >= L, steps 2-3 run over all keys.
__global__ __launch_bounds__(64) void q8_sparse_select_kernel(SparseParams p)
{
    extern __shared__ uint32_t keys[];   // min(max_nb, kSelLdsKeys) score keys when blocks are probed
    __shared__ uint32_t surv_key[kSelSurvivors];
    __shared__ int32_t surv_idx[kSelSurvivors];
    const int bh = blockIdx.x, b = bh / p.nq, h = bh - (bh / p.nq) * p.nq;
    const int lane = threadIdx.x;
    int n = p.seq_lens[b];
    if (n < 0 || n > p.max_seq_len) {
        if (h == 0 && lane == 0 && p.dev_status) atomicOr(p.dev_status, kDevBadSeqLen);
        n = 0;
    }
    n = uniform(n);
    const int nb = (n + kSparseBlock - 1) / kSparseBlock;
    int32_t *sel = p.sel + (size_t)bh * kMaxTopk;
    int32_t *user = p.selected ? p.selected + (size_t)bh * p.topk : nullptr;
    const int k = p.topk;
    int count;
    if (nb <= k) {
        for (int i = lane; i < nb; i += 64) {
            sel[i] = i;
            if (user) user[i] = i;
        }
        count = nb;
    } else {
        const float *sc = p.scores + (size_t)bh * p.max_nb;
        const bool in_lds = nb <= kSelLdsKeys;
        uint32_t lmax = 0;
        for (int j0 = 0; j0 < nb; j0 += 16 * 64) {   // 16 loads in flight per lane
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int jj = j0 + 64 * u + lane;
                v[u] = jj < nb ? sc[jj] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int jj = j0 + 64 * u + lane;
                const uint32_t kj = score_ord(v[u]);
                if (jj < nb) {
                    if (in_lds) keys[jj] = kj;
                    lmax = kj > lmax ? kj : lmax;
                }
            }
        }
        __syncthreads();
        auto key = [&](int j) { return in_lds ? keys[j] : score_ord(sc[j]); };
        // 1. the lower bound L
        uint32_t L = 0;
        for (int bit = 31; bit >= 0; --bit) {
            const uint32_t cand = L | (1u << bit);
            if (count_true(lmax >= cand) >= k) L = cand;
        }
        // 2. survivors in index order
        int ns = 0;
        for (int j0 = 0; j0 < nb; j0 += 4 * 64) {   // 4 reads in flight per lane
            uint32_t kv[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int jj = j0 + 64 * u + lane;
                kv[u] = jj < nb ? key(jj) : 0u;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int jj = j0 + 64 * u + lane;
                const bool keep = jj < nb && kv[u] >= L;
                const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
                const int at = ns + lanes_before(bal);
                if (keep && at < kSelSurvivors) {
                    surv_key[at] = kv[u];
                    surv_idx[at] = jj;
                }
                ns += __builtin_popcountll(bal);
            }
        }
        __syncthreads();
        const bool few = ns <= kSelSurvivors;
        const int len = few ? ns : nb;
        auto item_key = [&](int i) { return few ? surv_key[i] : key(i); };
        auto item_idx = [&](int i) { return few ? surv_idx[i] : i; };
        uint32_t T;
        if (len <= 64) {   // one candidate per lane: the search runs on ballots of a register
            const uint32_t kr = lane < len ? item_key(lane) : 0u;
            T = kth_largest(len, k, lane, [&](int) { return kr; });
        } else {
            T = kth_largest(len, k, lane, item_key);
        }
        // 3. the kept blocks in ascending order
        int above = 0;
        for (int i0 = 0; i0 < len; i0 += 64) above += count_true(i0 + lane < len && item_key(i0 + lane) > T);
        int ties = k - above;   // items equal to T still to take, lowest index first
        int base = 0;
        for (int i0 = 0; i0 < len && base < k; i0 += 64) {
            const int i = i0 + lane;
            const uint32_t ki = i < len ? item_key(i) : 0u;
            const uint64_t eqb = __builtin_amdgcn_ballot_w64(i < len && ki == T);
            const bool take = i < len && (ki > T || (ki == T && lanes_before(eqb) < ties));
            const uint64_t bal = __builtin_amdgcn_ballot_w64(take);
            if (take) {
                const int at = base + lanes_before(bal);
                const int j = item_idx(i);
                sel[at] = j;
                if (user) user[at] = j;
            }
            base += __builtin_popcountll(bal);
            const int eq_n = __builtin_popcountll(eqb);
            ties -= eq_n < ties ? eq_n : ties;
        }
        count = k;
    }
    if (lane == 0) p.cnt[bh] = count;
    if (user)
        for (int i = count + lane; i < k; i += 64) user[i] = -1;
}

// ----------------------------------------------------------------- attend --
template <bool Big>
__global__ __launch_bounds__(64 * kSparseWaves) void q8_sparse_attend_kernel(SparseParams p)
{
    __shared__ int sel[kMaxTopk];
    __shared__ float sh_m[kSparseWaves], sh_s[kSparseWaves];
    __shared__ float sh_acc[kSparseWaves][kHeadDim];

    const int bh = blockIdx.x / p.parts, part = blockIdx.x - (blockIdx.x / p.parts) * p.parts;
    const int b = bh / p.nq, h = bh - (bh / p.nq) * p.nq;
    const int G = p.nq / p.cache.nkv, kh = h / G;
    const int tid = threadIdx.x;
    const int wave = uniform(tid >> 6), lane = tid & 63, tslot = lane >> 3, c = lane & 7;
    const int n = uniform(sparse_len(p, b));
    const int cnt = uniform(p.cnt[bh]);
    if (tid < kMaxTopk) sel[tid] = tid < cnt ? p.sel[(size_t)bh * kMaxTopk + tid] : 0;
    __syncthreads();
    const int k0 = (int)(((long long)part * cnt) / p.parts), k1 = (int)(((long long)(part + 1) * cnt) / p.parts);

    uint4 qc;
    float qs;
    quantize_q_quarter(p.q + (size_t)bh * kHeadDim, c, qc, qs);
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

    // this wave's blocks: kept positions k0 + wave, k0 + wave + 4, ... < k1;
    // a tile past the list loads nothing
    const int span = k1 - k0;
    const int mine = span > wave ? (span - wave + kSparseWaves - 1) / kSparseWaves : 0;
    auto tile_t0 = [&](int i) { return i < mine ? sel[k0 + wave + kSparseWaves * i] * kSparseBlock : 0; };
    auto tile_n = [&](int i) { return i < mine ? n : 0; };
    if (mine > 0) {
        Tile ta, tb;
        TileBlocks ba, bb;
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

    // combine the waves in wave order
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
    if (p.parts == 1) {
        float2 *o = reinterpret_cast<float2 *>(p.out + (size_t)bh * kHeadDim);
        o[lane] = st > 0.0f ? make_float2(a0 / st, a1 / st) : make_float2(0.0f, 0.0f);
    } else {
        const size_t r = (size_t)bh * p.parts + part;
        reinterpret_cast<float2 *>(p.rec_acc + r * kHeadDim)[lane] = make_float2(a0, a1);
        if (lane == 0) p.rec_ms[r] = make_float2(mx, st);
    }
}

// ------------------------------------------------------------------ merge --
__global__ __launch_bounds__(64) void q8_sparse_merge_kernel(SparseParams p)
{
    const size_t bh = blockIdx.x;
    const int lane = threadIdx.x;
    float mx = -INFINITY;
    for (int i = 0; i < p.parts; ++i) mx = fmaxf(mx, p.rec_ms[bh * p.parts + i].x);
    float st = 0.0f, a0 = 0.0f, a1 = 0.0f;
    if (mx != -INFINITY) {
        for (int i = 0; i < p.parts; ++i) {
            const float2 ms = p.rec_ms[bh * p.parts + i];
            const float f = __builtin_amdgcn_exp2f(ms.x - mx);   // 0 for a part with no tokens
            const float2 a = reinterpret_cast<const float2 *>(p.rec_acc + (bh * p.parts + i) * kHeadDim)[lane];
            st = fmaf(ms.y, f, st);
            a0 = fmaf(a.x, f, a0);
            a1 = fmaf(a.y, f, a1);
        }
    }
    reinterpret_cast<float2 *>(p.out + bh * kHeadDim)[lane] =
        st > 0.0f ? make_float2(a0 / st, a1 / st) : make_float2(0.0f, 0.0f);
}

// ------------------------------------------------------------------- host --
// Workgroups per (sequence, query head): enough that a small batch still
// spreads over ~512 workgroups; a function of the shape only, so the
// workspace size and the result do not depend on the device.
static int sparse_parts(const q8_batch &batch, int nq)
{
    const long long rows = (long long)batch.batch * nq;
    long long parts = 512 / (rows > 0 ? rows : 1);
    if (parts < 1) parts = 1;
    if (parts > kMaxSparseParts) parts = kMaxSparseParts;
    return (int)parts;
}

struct SparseLayout {
    size_t scores, sel, cnt, ms, acc, bytes;
    int max_nb, parts;
};

static SparseLayout sparse_layout(const q8_batch &batch, int nq)
{
    auto up = [](size_t v) { return (v + 255) / 256 * 256; };
    SparseLayout l;
    l.max_nb = (batch.max_seq_len + kSparseBlock - 1) / kSparseBlock;
    if (l.max_nb < 1) l.max_nb = 1;
    l.parts = sparse_parts(batch, nq);
    const size_t rows = (size_t)batch.batch * nq;
    l.scores = 0;
    l.sel = up(rows * l.max_nb * sizeof(float));
    l.cnt = l.sel + up(rows * kMaxTopk * sizeof(int32_t));
    l.ms = l.cnt + up(rows * sizeof(int32_t));
    const size_t recs = l.parts > 1 ? rows * l.parts : 0;
    l.acc = l.ms + up(recs * sizeof(float2));
    l.bytes = l.acc + up(recs * kHeadDim * sizeof(float));
    return l;
}

size_t sparse_workspace_bytes(const q8_batch &batch, int nq) { return sparse_layout(batch, nq).bytes; }

hipError_t launch_sparse(const q8_kv_layer &layer, const q8_batch &batch, int nq, const float *q, float scale,
                         float *out, int topk, int32_t *selected, void *workspace, int32_t *dev_status,
                         hipStream_t stream)
{
    const SparseLayout l = sparse_layout(batch, nq);
    char *ws = static_cast<char *>(workspace);
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
    p.scores = reinterpret_cast<float *>(ws + l.scores);
    p.sel = reinterpret_cast<int32_t *>(ws + l.sel);
    p.cnt = reinterpret_cast<int32_t *>(ws + l.cnt);
    p.rec_ms = reinterpret_cast<float2 *>(ws + l.ms);
    p.rec_acc = reinterpret_cast<float *>(ws + l.acc);
    p.selected = selected;
    p.dev_status = dev_status;
    p.batch = batch.batch;
    p.nq = nq;
    p.max_blocks_per_seq = batch.max_blocks_per_seq;
    p.max_seq_len = batch.max_seq_len;
    p.max_nb = l.max_nb;
    p.topk = topk;
    p.parts = l.parts;
    p.sc = (float)((double)scale * 1.4426950408889634);
    p.probe_groups = (layer.nkv_heads + kProbeWaves - 1) / kProbeWaves;
    p.probe_waves = (layer.nkv_heads + p.probe_groups - 1) / p.probe_groups;
    const bool big = layer.kv_bs >= kTile;
    void *args[] = {&p};
    hipError_t e;

    const bool probing = l.max_nb > topk;
    if (probing) {
        const dim3 grid(batch.batch * p.probe_groups, (l.max_nb + kProbeBlocksPerWave - 1) / kProbeBlocksPerWave);
        const void *fn;
        switch (nq / layer.nkv_heads) {
        case 1: fn = reinterpret_cast<const void *>(&q8_sparse_probe_kernel<1>); break;
        case 2: fn = reinterpret_cast<const void *>(&q8_sparse_probe_kernel<2>); break;
        case 4: fn = reinterpret_cast<const void *>(&q8_sparse_probe_kernel<4>); break;
        default: fn = reinterpret_cast<const void *>(&q8_sparse_probe_kernel<8>); break;
        }
        if ((e = hipLaunchKernel(fn, grid, dim3(64 * p.probe_waves), args, 0, stream)) != hipSuccess) return e;
    }
    const size_t lds = probing ? (size_t)(l.max_nb < kSelLdsKeys ? l.max_nb : kSelLdsKeys) * sizeof(uint32_t) : 0;
    if ((e = hipLaunchKernel(reinterpret_cast<const void *>(&q8_sparse_select_kernel), dim3(batch.batch * nq),
                             dim3(64), args, lds, stream)) != hipSuccess)
        return e;
    const void *fa = big ? reinterpret_cast<const void *>(&q8_sparse_attend_kernel<true>)
                         : reinterpret_cast<const void *>(&q8_sparse_attend_kernel<false>);
    if ((e = hipLaunchKernel(fa, dim3(batch.batch * nq * l.parts), dim3(64 * kSparseWaves), args, 0, stream)) !=
        hipSuccess)
        return e;
    if (l.parts > 1 &&
        (e = hipLaunchKernel(reinterpret_cast<const void *>(&q8_sparse_merge_kernel), dim3(batch.batch * nq),
                             dim3(64), args, 0, stream)) != hipSuccess)
        return e;
    return hipGetLastError();
}

}  // namespace q8kv
