// q8kv_prefill.hip -- batched prefill attention over the q8 cache on the
// matrix cores.
//
// Method ("why long context must be sparse" §1-§2: the exact batched prefill
// path; a batch of nb new tokens scores against the whole history): the new
// tokens of sequence b are the last nb_b positions of its cache (appended
// before the call); query row r at position p attends to positions 0..p.
// Each query row is quantized like the decode query (per 32-block step
// m * fl(1/127), codes truncated), and its attention is the decode's:
// s_t = ((sum_beta float(P_beta) * qs_beta) * ks_t) * scale with exact int32
// block partials P_beta, softmax over t <= p, weights times V codes and V
// steps, one division at the end ("9-2 flash_attn_single_q_q8_neon" §2).
//
// A wave owns 32 query rows of one KV head (two sets of 16): row rho =
// position * G + head of the flattened (position, query head) list.  It
// walks the keys 0..p_max of its rows in tiles of 16 tokens (for a fresh
// prompt, a quarter of them: see prefill_segments); each tile's loads, V
// transpose and V operands serve both sets:
//   scores  S^T = K Q^T with v_mfma_i32_16x16x32_i8, one instruction per
//           32-block beta (A: token j's bytes 32 beta + [8 lg, 8 lg + 8) in
//           lane (lg, j); B: the query codes in the same places), so lane
//           (lg, j) receives the exact partials of query j with tokens
//           4 lg .. 4 lg + 3 and forms their fp32 scores in place;
//   softmax online per query (log2 domain): the tile max across the 4 lane
//           groups with v_permlane16/32_swap, one rescale of S and the
//           accumulators per tile;
//   values  O^T += V^T P^T on the bf16 matrix cores.  P^T arrives in
//           exactly the B layout (query j, tokens 4 lg + e); each weight
//           w = p * vs is split exactly into three bf16 terms
//           (w = hi + mid + lo by truncation; the "bf16x3" form of an fp32
//           product), and V codes (|code| <= 127) are exact in bf16, so the
//           products are exact and only the fp32 accumulation order differs
//           from a scalar loop.  The hi and mid terms go through one
//           v_mfma_f32_16x16x32_bf16 (same cost as a K = 16 product, twice
//           the work): its A operand holds the lane's 4 V values twice and its
//           B operand the 4 hi then the 4 mid weights, so each k slot pairs a
//           token's V code with one of its terms (A and B hold the same k
//           slots in a lane, whatever their order); lo uses
//           v_mfma_f32_16x16x16_bf16.  V^T is staged per tile through LDS: each
//           lane loads 4 bytes of 8 token rows, transposes them with v_perm
//           and writes one dword (4 tokens of one dim) per dim.
#include "q8kv_tile.hpp"
#include "q8kv_internal.hpp"

namespace q8kv {

typedef int v4i_t __attribute__((ext_vector_type(4)));
typedef float v4f_t __attribute__((ext_vector_type(4)));
typedef short v4s_t __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));

// Eight bf16 from two groups of four (the operand of a K = 32 product).
__device__ __forceinline__ v8bf_t cat_bf16(v4s_t a, v4s_t b)
{
    const uint2 x = __builtin_bit_cast(uint2, a), y = __builtin_bit_cast(uint2, b);
    return __builtin_bit_cast(v8bf_t, make_uint4(x.x, x.y, y.x, y.y));
}

constexpr int kPrefillWaves = 4;   // query tiles per workgroup
constexpr int kSets = 2;           // 16-row query sets per wave (share each key tile's loads and V operands)
constexpr int kPrefillRows = 16 * kSets;   // query rows per wave
constexpr int kKeyTile = 16;       // tokens per step
constexpr int kVtStride = 5;       // dwords per dim row of the staged V^T tile (4 token quads + 1 pad)

struct PrefillParams {
    CacheView cache;
    const int32_t *block_table;
    const int32_t *seq_lens;
    const int32_t *q_start;
    const float *q;
    float *out;
    int32_t *dev_status;
    int32_t nq, max_blocks_per_seq, max_seq_len, max_new, total_q, log2g;
    int32_t ks;   // key segments per query tile (1, 2 or 4 waves of a workgroup)
    float sc;     // softmax scale * log2(e)
};

// Partial states of the key segments other than the first, per lane:
// [slot][set][32 accumulators, M, S][lane].
constexpr int kCombVals = 8 * 4 + 2;
// Waves that split one query tile's keys when at least half of them are new
// (prefill_segments).  The launch halves it (to 2, then 1) only while the
// grid would exceed 65535 rows of workgroups, i.e. for prompts of more than
// 2^21 query rows; chunks after a long history use 1.
constexpr int kPrefillSplit = 4;

// 4 int8 codes (one dword) -> 4 bf16 (exact: |code| <= 127 has 7 bits).
__device__ __forceinline__ v4s_t codes_to_bf16(uint32_t w)
{
    const uint32_t f0 = __float_as_uint((float)(int)(int8_t)(w & 0xff));
    const uint32_t f1 = __float_as_uint((float)(int)(int8_t)((w >> 8) & 0xff));
    const uint32_t f2 = __float_as_uint((float)(int)(int8_t)((w >> 16) & 0xff));
    const uint32_t f3 = __float_as_uint((float)(int)(int8_t)(w >> 24));
    const uint32_t lo = __builtin_amdgcn_perm(f1, f0, 0x07060302u);   // upper halves of f0, f1
    const uint32_t hi = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
    return __builtin_bit_cast(v4s_t, make_uint2(lo, hi));
}

// Exact split of 4 fp32 weights into three bf16 terms each (truncation: the
// first term keeps the top 8 significant bits, the second the next 8, the
// third the rest; both subtractions are exact).
__device__ __forceinline__ void split_bf16x3(const float (&w)[4], v4s_t &hi, v4s_t &mid, v4s_t &lo)
{
    uint32_t h[4], m[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        h[e] = __float_as_uint(w[e]) & 0xffff0000u;
        const float r1 = w[e] - __uint_as_float(h[e]);
        m[e] = __float_as_uint(r1) & 0xffff0000u;
        const float r2 = r1 - __uint_as_float(m[e]);
        l[e] = __float_as_uint(r2);
    }
    hi = __builtin_bit_cast(v4s_t, make_uint2(__builtin_amdgcn_perm(h[1], h[0], 0x07060302u),
                                              __builtin_amdgcn_perm(h[3], h[2], 0x07060302u)));
    mid = __builtin_bit_cast(v4s_t, make_uint2(__builtin_amdgcn_perm(m[1], m[0], 0x07060302u),
                                               __builtin_amdgcn_perm(m[3], m[2], 0x07060302u)));
    lo = __builtin_bit_cast(v4s_t, make_uint2(__builtin_amdgcn_perm(l[1], l[0], 0x07060302u),
                                              __builtin_amdgcn_perm(l[3], l[2], 0x07060302u)));
}

// Loads of one 16-token key tile: K bytes for the score MFMAs, the K and V
// steps of tokens t0 + 4 lg + e, and 4 bytes of 8 V rows for the transpose.
struct KeyTile {
    long ka[4];
    float ks[4], vs[4];
    uint32_t vw[8];
    bool good_lo, good_hi;   // block ids of tokens t0 .. t0 + 7 and t0 + 8 .. t0 + 15 are valid
};

// Big (kv_bs >= 16): the tile lies in one physical block, which holds only
// this sequence's rows; the bases are scalar, the lane offsets fixed, and
// rows past the sequence end inside the block are read (they may hold any
// bytes) and masked by the caller.  Otherwise (kv_bs = 8) the tile spans
// two blocks and tokens are clamped to n - 1.
template <bool Big>
__device__ __forceinline__ void load_key_tile(const PrefillParams &p, const const_i32 *sbt, int kh, int t0, int n,
                                              int j, int lg, int vh, int vd, KeyTile &kt)
{
    const int nkv = p.cache.nkv, row_bytes = nkv * kHeadDim;
    const int log2bs = p.cache.kv_bs_log2, bmask = (1 << log2bs) - 1;
    if (Big) {
        const int id = sbt[t0 >> log2bs];   // t0 <= n - 1
        const bool good = (unsigned)id < (unsigned)p.cache.num_blocks;
        kt.good_lo = kt.good_hi = good;
        const size_t row0 = ((size_t)(good ? id : 0) << log2bs) + (size_t)(t0 & bmask);
        const int8_t *kb = p.cache.k_codes + row0 * row_bytes + kh * kHeadDim;
        const int8_t *vb = p.cache.v_codes + row0 * row_bytes + kh * kHeadDim;
        const size_t s0 = (((size_t)(good ? id : 0) * nkv + kh) << log2bs) + (size_t)(t0 & bmask);
#pragma unroll
        for (int beta = 0; beta < 4; ++beta)
            kt.ka[beta] = *reinterpret_cast<const long *>(kb + j * row_bytes + 32 * beta + 8 * lg);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kt.ks[e] = p.cache.k_scale[s0 + 4 * lg + e];
            kt.vs[e] = p.cache.v_scale[s0 + 4 * lg + e];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            kt.vw[u] = *reinterpret_cast<const uint32_t *>(vb + (8 * vh + u) * row_bytes + 4 * vd);
    } else {
        int id0 = sbt[min(t0, n - 1) >> log2bs];
        int id1 = sbt[min(t0 + 8, n - 1) >> log2bs];
        kt.good_lo = (unsigned)id0 < (unsigned)p.cache.num_blocks;
        kt.good_hi = (unsigned)id1 < (unsigned)p.cache.num_blocks;
        id0 = kt.good_lo ? id0 : 0;
        id1 = kt.good_hi ? id1 : 0;
        auto row_of = [&](int t) {   // t in [t0, t0 + 16), clamped to n - 1
            const int id = ((t - t0) >> 3) ? id1 : id0;
            return ((size_t)id << log2bs) + (size_t)(t & bmask);
        };
        const int8_t *krow = p.cache.k_codes + row_of(min(t0 + j, n - 1)) * row_bytes + kh * kHeadDim + 8 * lg;
#pragma unroll
        for (int beta = 0; beta < 4; ++beta) kt.ka[beta] = *reinterpret_cast<const long *>(krow + 32 * beta);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const size_t row = row_of(min(t0 + 4 * lg + e, n - 1));
            const size_t sidx = (((row >> log2bs) * nkv + kh) << log2bs) + (row & bmask);
            kt.ks[e] = p.cache.k_scale[sidx];
            kt.vs[e] = p.cache.v_scale[sidx];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const size_t row = row_of(min(t0 + 8 * vh + u, n - 1));
            kt.vw[u] = *reinterpret_cast<const uint32_t *>(p.cache.v_codes + row * row_bytes + kh * kHeadDim + 4 * vd);
        }
    }
}

template <bool Big>
__global__ __launch_bounds__(64 * kPrefillWaves) void q8_prefill_kernel(PrefillParams p)
{
    __shared__ uint32_t vt_all[kPrefillWaves][kHeadDim * kVtStride];
    __shared__ float comb[kPrefillWaves - 1][kSets][kCombVals][64];
    const int nkv = p.cache.nkv;
    const int b = blockIdx.x / nkv, kh = blockIdx.x - (blockIdx.x / nkv) * nkv;
    const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
    uint32_t *vt = vt_all[wave];
    // With ks > 1 the ks waves of a group share one query tile, each taking a
    // contiguous segment of its key tiles; their states are combined at the
    // end.  The last query tiles (the longest key ranges under the causal
    // mask) are dispatched first, so the short ones fill in behind them.
    const int ks = p.ks, seg = wave % ks;
    const int tile = (gridDim.y - 1 - blockIdx.y) * (kPrefillWaves / ks) + wave / ks;
    const int G = 1 << p.log2g;
    const int j = lane & 15, lg = lane >> 4;
    // every wave meets the combine barrier (ks > 1), so nothing returns
    // early: waves without work skip to it
    bool active = true;

    const int r0 = uniform(p.q_start[b]), r1 = uniform(p.q_start[b + 1]);
    const int n = uniform(p.seq_lens[b]);
    const bool range_ok = 0 <= r0 && r0 <= r1 && r1 <= p.total_q;
    const int nn = r1 - r0;
    if (!range_ok || n < nn || n > p.max_seq_len || nn > p.max_new) {
        // a bad sequence: reported; its rows that this wave covers are zeros
        active = false;
        if (kh == 0 && tile == 0 && lane == 0 && p.dev_status) atomicOr(p.dev_status, kDevBadSeqLen);
        if (range_ok && seg == 0) {
#pragma unroll
            for (int st = 0; st < kSets; ++st) {
                const int rho = tile * kPrefillRows + 16 * st + j;
                if (rho < (nn << p.log2g)) {
                    const int i = rho >> p.log2g, g = rho & (G - 1);
                    float *o = p.out + ((size_t)(r0 + i) * p.nq + kh * G + g) * kHeadDim;
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt)
                        reinterpret_cast<float4 *>(o + 16 * dt + 4 * lg)[0] = make_float4(0.f, 0.f, 0.f, 0.f);
                }
            }
        }
    }
    const int rows = nn << p.log2g;
    if (tile * kPrefillRows >= rows) active = false;

    // state of this wave (declared for the combine; set by active waves)
    bool live[kSets] = {};
    int qi[kSets] = {}, qg[kSets] = {}, pos[kSets] = {};
    // M is a reference max per query: the weights exp2(s - M) may exceed 1 by
    // up to 2^kLazyRescale, and S and the accumulators are rescaled only when
    // some query's tile max rises above its M by more than that (the result
    // is the same quantity; only rounding differs)
    constexpr float kLazyRescale = 8.0f;
    float M[kSets], S[kSets];
    v4f_t acc[kSets][8];
#pragma unroll
    for (int st = 0; st < kSets; ++st) {
        M[st] = -INFINITY;
        S[st] = 0.0f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) acc[st][dt] = v4f_t{0.f, 0.f, 0.f, 0.f};
    }

    if (active) {
    // this lane's query row in each set (clamped to a real row; lanes past the
    // end are computed and discarded) and its position
#pragma unroll
    for (int st = 0; st < kSets; ++st) {
        const int rho = tile * kPrefillRows + 16 * st + j;
        live[st] = rho < rows;
        const int rr = live[st] ? rho : rows - 1;
        qi[st] = rr >> p.log2g;
        qg[st] = rr & (G - 1);
        pos[st] = n - nn + qi[st];
    }
    const int p_hi = n - nn + (min(tile * kPrefillRows + kPrefillRows - 1, rows - 1) >> p.log2g);
    const int pos_lo = n - nn + ((tile * kPrefillRows) >> p.log2g);   // the wave's smallest position
    const int nkt = p_hi / kKeyTile + 1;

    // query codes, the B operands of the score MFMAs: bytes 32 beta + [8 lg, 8 lg + 8)
    long qb[kSets][4];
    float qs[kSets][4];
#pragma unroll
    for (int st = 0; st < kSets; ++st) {
        const size_t qrow = ((size_t)(r0 + qi[st]) * p.nq + kh * G + qg[st]) * kHeadDim;
#pragma unroll
        for (int beta = 0; beta < 4; ++beta) {
            const float4 *src = reinterpret_cast<const float4 *>(p.q + qrow + 32 * beta + 8 * lg);
            const float4 a = src[0], c = src[1];
            const float x[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
            float m = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(x[e]));
            m = max_rows32(max_rows16(m));   // the 32-block's max over the four lane groups
            const BlockQuant bq = q_block_params(m);
            int cd[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) cd[e] = q_code(x[e], bq.recip);
            const uint32_t w0 = pack4_i8(cd[0], cd[1], cd[2], cd[3]), w1 = pack4_i8(cd[4], cd[5], cd[6], cd[7]);
            qb[st][beta] = (long)(((uint64_t)w1 << 32) | w0);
            qs[st][beta] = bq.qscale;
        }
    }

    const const_i32 *sbt = (const const_i32 *)(p.block_table + (size_t)b * p.max_blocks_per_seq);
    const int vh = lane >> 5, vd = lane & 31;   // V staging: tokens 8 vh + u, dims 4 vd .. 4 vd + 3

    bool bad = false;
    // tile kt + 1 (block id, K, steps, V rows) is in flight while tile kt is
    // computed; past the end the last tile is reloaded, unused.  (Loading the
    // V rows at the start of their own tile, or two tiles used in turn
    // without the copy, both measured slower.)
    // this wave's key segment: tiles [kt_lo, kt_hi) of the nkt, split evenly
    // over the ks waves of the query tile (possibly empty: then nothing is
    // loaded, since tile positions past the sequence have no table entry)
    const int kt_lo = (seg * nkt) / ks, kt_hi = ((seg + 1) * nkt) / ks;
    KeyTile nxt;
    if (kt_lo < kt_hi) load_key_tile<Big>(p, sbt, kh, kt_lo * kKeyTile, n, j, lg, vh, vd, nxt);
    for (int kt = kt_lo; kt < kt_hi; ++kt) {
        const int t0 = kt * kKeyTile;
        const KeyTile tl = nxt;
        load_key_tile<Big>(p, sbt, kh, min(kt + 1, kt_hi - 1) * kKeyTile, n, j, lg, vh, vd, nxt);
        bad = bad || !tl.good_lo || (t0 + 8 <= p_hi && !tl.good_hi);
        // every row of the wave sees all 16 tokens of the tile: no masks
        const bool full = t0 + kKeyTile - 1 <= pos_lo && tl.good_lo && tl.good_hi;

        // V^T tile through LDS: dword (dim, token quad) = 4 tokens of one dim;
        // the bf16 A operands are formed once and serve both query sets
        uint32_t tq[8];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const uint32_t a0 = tl.vw[4 * half], a1 = tl.vw[4 * half + 1], a2 = tl.vw[4 * half + 2],
                           a3 = tl.vw[4 * half + 3];
            const uint32_t x01l = __builtin_amdgcn_perm(a1, a0, 0x05010400u);   // a0.b0 a1.b0 a0.b1 a1.b1
            const uint32_t x01h = __builtin_amdgcn_perm(a1, a0, 0x07030602u);   // a0.b2 a1.b2 a0.b3 a1.b3
            const uint32_t x23l = __builtin_amdgcn_perm(a3, a2, 0x05010400u);
            const uint32_t x23h = __builtin_amdgcn_perm(a3, a2, 0x07030602u);
            tq[4 * half + 0] = __builtin_amdgcn_perm(x23l, x01l, 0x05040100u);  // byte 0 of a0..a3
            tq[4 * half + 1] = __builtin_amdgcn_perm(x23l, x01l, 0x07060302u);  // byte 1
            tq[4 * half + 2] = __builtin_amdgcn_perm(x23h, x01h, 0x05040100u);  // byte 2
            tq[4 * half + 3] = __builtin_amdgcn_perm(x23h, x01h, 0x07060302u);  // byte 3
        }
        asm volatile("" ::: "memory");   // the previous tile's V^T reads come first
#pragma unroll
        for (int dd = 0; dd < 4; ++dd) {
            vt[(4 * vd + dd) * kVtStride + 2 * vh] = tq[dd];
            vt[(4 * vd + dd) * kVtStride + 2 * vh + 1] = tq[4 + dd];
        }
        asm volatile("" ::: "memory");
        v4s_t va[8];
        v8bf_t va2[8];   // the same 4 values twice: the A operand of the paired hi + mid product
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            va[dt] = codes_to_bf16(vt[(16 * dt + j) * kVtStride + lg]);
            va2[dt] = cat_bf16(va[dt], va[dt]);
        }

#pragma unroll
        for (int st = 0; st < kSets; ++st) {
            // scores of query j of this set with tokens t0 + 4 lg + e
            v4i_t c[4];
#pragma unroll
            for (int beta = 0; beta < 4; ++beta)
                c[beta] = __builtin_amdgcn_mfma_i32_16x16x32_i8(tl.ka[beta], qb[st][beta], v4i_t{0, 0, 0, 0}, 0, 0, 0);
            float s[4];
            uint32_t keep[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float x0 = (float)c[0][e] * qs[st][0], x1 = (float)c[1][e] * qs[st][1];
                const float x2 = (float)c[2][e] * qs[st][2], x3 = (float)c[3][e] * qs[st][3];
                const float y = (x0 + x1) + (x3 + x2);
                s[e] = y * (tl.ks[e] * p.sc);
            }
            if (!full) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int t = t0 + 4 * lg + e;
                    keep[e] = (t <= pos[st] && ((e + 4 * lg) < 8 ? tl.good_lo : tl.good_hi)) ? 0xffffffffu : 0u;
                    // branch-free mask (a select here becomes a divergent
                    // branch); a masked token's step may be any bits, even NaN
                    s[e] = __uint_as_float(bitsel(keep[e], __float_as_uint(s[e]), 0xff800000u));
                }
            }
            float m = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
            m = max_rows32(max_rows16(m));   // the tile max of query j over the four lane groups
            const bool grow = m > M[st] + kLazyRescale;   // also true on the first tile with a finite max
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {
                const float Mn = grow ? m : M[st];
                const float alpha = Mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(M[st] - Mn);
                M[st] = Mn;
                S[st] *= alpha;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) acc[st][dt] *= alpha;
            }
            float w[4], psum = 0.0f;
            if (full) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float pw = __builtin_amdgcn_exp2f(s[e] - M[st]);
                    psum += pw;
                    w[e] = pw * tl.vs[e];
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    // masked: weight 0 (M may still be -inf, and the step may be NaN)
                    const float pw =
                        __uint_as_float(bitsel(keep[e], __float_as_uint(__builtin_amdgcn_exp2f(s[e] - M[st])), 0u));
                    psum += pw;
                    w[e] = __uint_as_float(bitsel(keep[e], __float_as_uint(pw * tl.vs[e]), 0u));
                }
            }
            S[st] += psum;
            v4s_t whi, wmid, wlo;
            split_bf16x3(w, whi, wmid, wlo);
            const v8bf_t whm = cat_bf16(whi, wmid);
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                acc[st][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va2[dt], whm, acc[st][dt], 0, 0, 0);
                acc[st][dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[dt], wlo, acc[st][dt], 0, 0, 0);
            }
        }
    }
    if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0 && p.dev_status) atomicOr(p.dev_status, kDevBadBlockId);

    }

    // the other segments' states into the first's: M the largest, S and the
    // accumulators rescaled to it and summed in segment order ("9-2" §2
    // segment 2 rule applied to partial states); deterministic
    if (ks > 1) {
        const int slot = (wave / ks) * (ks - 1) + seg - 1;
        if (active && seg > 0) {
#pragma unroll
            for (int st = 0; st < kSets; ++st) {
#pragma unroll
                for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) comb[slot][st][4 * dt + e][lane] = acc[st][dt][e];
                comb[slot][st][32][lane] = M[st];
                comb[slot][st][33][lane] = S[st];
            }
        }
        __syncthreads();
        if (active && seg == 0) {
#pragma unroll
            for (int st = 0; st < kSets; ++st) {
                float Mn = M[st];
                for (int w = 1; w < ks; ++w) Mn = fmaxf(Mn, comb[slot + w][st][32][lane]);
                const float a0 = M[st] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M[st] - Mn);
                S[st] *= a0;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) acc[st][dt] *= a0;
                for (int w = 1; w < ks; ++w) {
                    const float Mw = comb[slot + w][st][32][lane];
                    const float aw = Mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(Mw - Mn);
                    S[st] = fmaf(comb[slot + w][st][33][lane], aw, S[st]);
#pragma unroll
                    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            acc[st][dt][e] = fmaf(comb[slot + w][st][4 * dt + e][lane], aw, acc[st][dt][e]);
                }
                M[st] = Mn;
            }
        }
    }
    if (!active || seg != 0) return;

    float Ssum[kSets];
#pragma unroll
    for (int st = 0; st < kSets; ++st) Ssum[st] = sum_rows32(sum_rows16(S[st]));   // lane groups hold different tokens
#pragma unroll
    for (int st = 0; st < kSets; ++st) {
        const float Sst = Ssum[st];
        if (!live[st]) continue;
        float *o = p.out + ((size_t)(r0 + qi[st]) * p.nq + kh * G + qg[st]) * kHeadDim;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            // one division at the end, per element
            const v4f_t a = acc[st][dt];
            reinterpret_cast<float4 *>(o + 16 * dt + 4 * lg)[0] =
                Sst > 0.0f ? make_float4(a[0] / Sst, a[1] / Sst, a[2] / Sst, a[3] / Sst)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
}

// Key segments per query tile.  When at least half of the keys are new (a
// fresh prompt, or a chunk as long as its history), the causal triangle makes
// the last query tiles' key ranges about twice the average, and the waves
// that walk them alone set the launch time: their keys are split over four
// waves.  Chunks after a long history have query tiles of nearly equal
// length and keep one wave per tile.  The grid stays within 65535 rows of
// workgroups.
static int prefill_segments(int max_new, int max_seq_len, long long rows)
{
    int ks = (2LL * max_new >= max_seq_len) ? kPrefillSplit : 1;
    while (ks > 1 && (rows + (long long)kPrefillRows * (kPrefillWaves / ks) - 1) /
                             ((long long)kPrefillRows * (kPrefillWaves / ks)) > 65535)
        ks >>= 1;
    return ks;
}

hipError_t launch_prefill(const q8_kv_layer &layer, const q8_batch &batch, int nq, const int32_t *q_start,
                          int total_q, int max_new, const float *q, float scale, float *out, int32_t *dev_status,
                          hipStream_t stream)
{
    PrefillParams p;
    p.cache.k_codes = layer.k_codes;
    p.cache.v_codes = layer.v_codes;
    p.cache.k_scale = layer.k_scale;
    p.cache.v_scale = layer.v_scale;
    p.cache.nkv = layer.nkv_heads;
    p.cache.kv_bs_log2 = ilog2(layer.kv_bs);
    p.cache.num_blocks = layer.num_blocks;
    p.block_table = batch.block_table;
    p.seq_lens = batch.seq_lens;
    p.q_start = q_start;
    p.q = q;
    p.out = out;
    p.dev_status = dev_status;
    p.nq = nq;
    p.max_blocks_per_seq = batch.max_blocks_per_seq;
    p.max_seq_len = batch.max_seq_len;
    p.max_new = max_new;
    p.total_q = total_q;
    p.log2g = ilog2(nq / layer.nkv_heads);
    p.sc = (float)((double)scale * 1.4426950408889634);
    const long long rows = (long long)max_new * (nq / layer.nkv_heads);
    p.ks = prefill_segments(max_new, batch.max_seq_len, rows);
    const long long rows_per_wg = (long long)kPrefillRows * (kPrefillWaves / p.ks);
    const dim3 grid(batch.batch * layer.nkv_heads, (unsigned)((rows + rows_per_wg - 1) / rows_per_wg));
    void *args[] = {&p};
    const void *fn = layer.kv_bs >= kKeyTile ? reinterpret_cast<const void *>(&q8_prefill_kernel<true>)
                                             : reinterpret_cast<const void *>(&q8_prefill_kernel<false>);
    const hipError_t e = hipLaunchKernel(fn, grid,
                                         dim3(64 * kPrefillWaves), args, 0, stream);
    return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace q8kv
