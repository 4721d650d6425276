// q8kv_decode_f32.hip -- exact decode attention over the fp32 mirror cache.
//
// Method ("9-3 q8 KV 精度对照实验" §1, the exact baseline: scores of the raw
// fp32 q and K, max-subtracted softmax, weighted raw V; §3 closing note: the
// float cache kept beside the q8 one): s_t = scale * <q, k_t> in fp32, an
// online softmax with running max M and sum S that rescales what has
// accumulated whenever M rises, V accumulated in fp32, one division at the
// end ("9-2 flash_attn_single_q_q8_neon" §2 segments 2-3, with fp32 rows in
// place of int8 codes).  The batch is cut into the same ranges as the q8
// kernel and cut sequences leave the same (M, S, acc) records, which the
// same merge kernel finishes.
//
// A wave is one KV head and serves its G query heads.  A head's row is 128
// floats (512 bytes): lane (h, c) = (lane / 32, lane % 32) holds floats
// [4c, 4c + 4) of token 2 kk + h of an 8-token step, kk = 0..3, so one
// 16-byte load per lane reads two whole rows.  The dot product of a token is
// summed over its 32 lanes with DPP moves and v_permlane16_swap, so all 32
// lanes hold the same bits.  Two steps are in registers: the next step's
// loads are in flight while one is processed; block ids run a step ahead.
#include "q8kv_ranges.hpp"

namespace q8kv {

constexpr int kFStep = 8;   // tokens per step (a step never straddles a block: kv_bs >= 8)

struct FStep {
    float4 k[4];
    float4 v[4];
    uint32_t valid;   // bit kk: token t0 + 2 kk + h is inside the sequence and its block id is good
};

// Sum over the 32 lanes of this lane's half of the wave; every lane of the
// half gets the same bits (each stage adds a pair symmetrically).
__device__ __forceinline__ float sum_half(float x)
{
    x += dpp_f<kDppQuadXor1>(x);
    x += dpp_f<kDppQuadXor2>(x);
    x += dpp_f<kDppHalfMirror>(x);
    x += dpp_f<kDppRor8>(x);
    return sum_rows16(x);
}

// Loads step [t0, t0 + 8) of one sequence for the wave's KV head, given the
// step's block id; tokens at or past n are masked and read as zeros.  Every
// call issues the same 8 loads: a step at or past n, or with a block id
// outside [0, num_blocks) (reported in *status), gets an empty buffer
// resource; a masked token inside a real step gets an offset past the
// resource (kOutOfRange plus at most 6 rows stays below 2^32).
__device__ __forceinline__ void load_step(const DecodeParams &p, int blk, int kh, int lane, int t0, int n,
                                          FStep &s)
{
    const int h = lane >> 5, c = lane & 31;
    const int nkv = p.cache.nkv;
    const bool want = t0 < n;
    const bool good = (unsigned)blk < (unsigned)p.cache.num_blocks;
    if (want && !good && lane == 0 && p.dev_status) atomicOr(p.dev_status, kDevBadBlockId);
    const bool ok = want && good;
    s.valid = 0;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) s.valid |= (ok && t0 + 2 * kk + h < n) ? (1u << kk) : 0u;
    const size_t row0 = ((size_t)(ok ? blk : 0) << p.cache.kv_bs_log2) +
                        (size_t)(t0 & ((1 << p.cache.kv_bs_log2) - 1));
    const int row_bytes = nkv * kHeadDim * 4;
    const int bytes = ok ? kFStep * row_bytes : 0;
    const auto rk = make_rsrc(p.k_f32 + row0 * nkv * kHeadDim, bytes);
    const auto rv = make_rsrc(p.v_f32 + row0 * nkv * kHeadDim, bytes);
    const int off = h * row_bytes + kh * kHeadDim * 4 + 16 * c;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        // a token past the end reads zeros: its row may hold any bits (even
        // NaN), and a zero weight times NaN would still be NaN
        const int o = ((s.valid >> kk) & 1u) ? off : kOutOfRange;
        s.k[kk] = __builtin_bit_cast(float4, buf_load16(rk, o, kk * 2 * row_bytes));
        s.v[kk] = __builtin_bit_cast(float4, buf_load16(rv, o, kk * 2 * row_bytes));
    }
}

__device__ __forceinline__ int fetch_step_block(const int32_t *bt, int log2bs, int t0, int n)
{
    const const_i32 *sbt = (const const_i32 *)bt;
    return t0 < n ? sbt[t0 >> log2bs] : -1;
}

// One wave: exact attention of the G query heads of KV head kh over tiles
// [lt0, lt1) (32 tokens each) of sequence b (length n).
template <int G>
__device__ __forceinline__ void attend_piece_f32(const DecodeParams &p, int b, int kh, int lane, int lt0,
                                                 int lt1, int n, bool whole, int part, int slot)
{
    const int h = lane >> 5, c = lane & 31;
    float4 qv[G];
#pragma unroll
    for (int g = 0; g < G; ++g)
        qv[g] = reinterpret_cast<const float4 *>(p.q + ((size_t)b * p.nq + kh * G + g) * kHeadDim)[c];

    float M[G], S[G], acc[G][4];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        M[g] = -INFINITY;
        S[g] = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[g][j] = 0.0f;
    }

    auto process = [&](const FStep &st) {
        float s[4][G];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const bool ok = (st.valid >> kk) & 1u;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float d = st.k[kk].x * qv[g].x;
                d = fmaf(st.k[kk].y, qv[g].y, d);
                d = fmaf(st.k[kk].z, qv[g].z, d);
                d = fmaf(st.k[kk].w, qv[g].w, d);
                d = sum_half(d);
                s[kk][g] = ok ? d * p.sc : -INFINITY;   // log2 domain: scale * log2(e) folded in
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float m = fmaxf(fmaxf(s[0][g], s[1][g]), fmaxf(s[2][g], s[3][g]));
            m = max_rows32(m);   // with the other half: the step max, the same in every lane
            if (m > M[g]) {
                const float a = __builtin_amdgcn_exp2f(M[g] - m);
                S[g] *= a;
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[g][j] *= a;
                M[g] = m;
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            // a masked token's score is -inf: weight exp2(-inf) = 0 against a finite reference
            const float mf = M[g] == -INFINITY ? 0.0f : M[g];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const float w = __builtin_amdgcn_exp2f(s[kk][g] - mf);
                S[g] += w;
                acc[g][0] = fmaf(w, st.v[kk].x, acc[g][0]);
                acc[g][1] = fmaf(w, st.v[kk].y, acc[g][1]);
                acc[g][2] = fmaf(w, st.v[kk].z, acc[g][2]);
                acc[g][3] = fmaf(w, st.v[kk].w, acc[g][3]);
            }
        }
    };

    const int32_t *bt = p.block_table + (size_t)b * p.max_blocks_per_seq;
    const int log2bs = p.cache.kv_bs_log2;
    const int ne = min(n, lt1 * kTile);
    const int s0 = lt0 * (kTile / kFStep), s1 = lt1 * (kTile / kFStep);
    // Two register steps; step i lives in st[i % 2]; tokens past the piece
    // count as past the end, so the step loaded beyond it costs no traffic.
    FStep st[2];
    int blk[2];
    blk[0] = fetch_step_block(bt, log2bs, s0 * kFStep, ne);
    load_step(p, blk[0], kh, lane, s0 * kFStep, ne, st[0]);
    blk[1] = fetch_step_block(bt, log2bs, (s0 + 1) * kFStep, ne);
    int si = s0;
    while (true) {
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            load_step(p, blk[d ^ 1], kh, lane, (si + 1) * kFStep, ne, st[d ^ 1]);
            blk[d] = fetch_step_block(bt, log2bs, (si + 2) * kFStep, ne);
            process(st[d]);
            if (++si >= s1) goto piece_done;
        }
    }
piece_done:

    // combine the two halves (different tokens)
#pragma unroll
    for (int g = 0; g < G; ++g) {
        S[g] = sum_rows32(S[g]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[g][j] = sum_rows32(acc[g][j]);
    }
    if (h != 0) return;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int hq = kh * G + g;
        if (whole) {
            // one division at the end
            const float sg = S[g];
            float4 r;
            r.x = sg > 0.0f ? acc[g][0] / sg : 0.0f;
            r.y = sg > 0.0f ? acc[g][1] / sg : 0.0f;
            r.z = sg > 0.0f ? acc[g][2] / sg : 0.0f;
            r.w = sg > 0.0f ? acc[g][3] / sg : 0.0f;
            reinterpret_cast<float4 *>(p.out + ((size_t)b * p.nq + hq) * kHeadDim)[c] = r;
        } else {
            const size_t idx = ((size_t)part * 2 + slot) * p.nq + hq;
            reinterpret_cast<float4 *>(p.ws_acc + idx * kHeadDim)[c] =
                make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
            if (c == 0) p.ws_ms[idx] = make_float2(M[g], S[g]);
        }
    }
}

template <int G>
__global__ __launch_bounds__(64 * kMaxWavesPerWG) void q8_attn_f32_partial_kernel(DecodeParams p)
{
    __shared__ int pref[kMaxBatch + 1];
    // walk_ranges calls the lambda from each of its walks (one piece per
    // call: chunk is always 0 there); without always_inline the compiler
    // makes it a real call, with a stack frame in scratch and twice the VGPRs
    walk_ranges(p, pref, nullptr,
                [&](int b, int kh, int lane, int lt0, int lt1, int n, bool whole, int part, int slot,
                    const TileBlocks *, int) __attribute__((always_inline)) {
                    attend_piece_f32<G>(p, b, kh, lane, lt0, lt1, n, whole, part, slot);
                });
}

hipError_t launch_decode_partial_f32(const q8_kv_layer &layer, const q8_batch &batch, int nq,
                                     const float *q, float scale, float *out, const DecodePlan &plan,
                                     void *workspace, int32_t *dev_status, hipStream_t stream)
{
    DecodeParams p = fill_decode_params(layer, batch, nq, q, scale, out, plan, workspace, dev_status);
    const dim3 grid(plan.nparts * plan.head_groups), block(plan.waves * 64);
    const void *fn;
    switch (nq / layer.nkv_heads) {
    case 1: fn = reinterpret_cast<const void *>(&q8_attn_f32_partial_kernel<1>); break;
    case 2: fn = reinterpret_cast<const void *>(&q8_attn_f32_partial_kernel<2>); break;
    case 4: fn = reinterpret_cast<const void *>(&q8_attn_f32_partial_kernel<4>); break;
    default: fn = reinterpret_cast<const void *>(&q8_attn_f32_partial_kernel<8>); break;
    }
    void *args[] = {&p};
    const hipError_t e = hipLaunchKernel(fn, grid, block, args, 0, stream);
    return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace q8kv
