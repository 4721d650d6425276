// q8kv_device.hpp -- device routines shared by every kernel of libq8kv (gfx950).
//
// The quantizer routines follow two pages (cited by title and section):
//   "9-2 flash_attn_single_q_q8_neon -- 单 q 单遍扫全 KV" §2 segment 1 (the
//   query is cut into 32-element blocks, each with its own max-abs scale) and
//   "9-3 q8 KV 精度对照实验" §2 (one max-abs/127 scale per (token, KV head)
//   row, codes rounded and clamped to +-127).
// Every fp32 step of the two quantizers is one IEEE operation (the products
// use __fmul_rn so that nothing can be fused into them; fp32 division is the
// correctly rounded default lowering), so codes and scales are reproducible
// bit for bit by any IEEE implementation of the same steps.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8kv {

constexpr int kHeadDim = 128;     // supported head_dim
constexpr int kQBlock = 32;       // query block length
constexpr int kTile = 32;         // tokens per decode tile
constexpr int kSub = 8;           // tokens per wave load (8 lanes x 16 bytes per token row)
constexpr int kMaxBatch = 4096;
constexpr int kMaxWavesPerWG = 8; // KV heads handled by one decode workgroup
constexpr float kInv127 = 1.0f / 127.0f;   // fl(1/127) = 0x3C010204
constexpr float kGuard = 1e-6f;            // max-abs below this counts as 1
constexpr float kLog2e = 1.4426950408889634f;

constexpr int32_t kDevBadSeqLen = 0x1;
constexpr int32_t kDevBadBlockId = 0x2;
constexpr int32_t kDevBadToken = 0x4;
constexpr int32_t kDevBadPlan = 0x8;

// ------------------------------------------------------------------ quantizers
// K/V row: given the row's max-abs a, the stored step d and the reciprocal r.
struct RowQuant {
    float step;
    float recip;
};

__device__ __forceinline__ RowQuant kv_row_params(float amax)
{
    float a = (amax < kGuard) ? 1.0f : amax;
    RowQuant q;
    q.step = __fmul_rn(a, kInv127);
    q.recip = 127.0f / a;   // IEEE division (div_scale / div_fmas / div_fixup)
    return q;
}

// code = clamp(roundf(x * r), -127, 127); roundf rounds halves away from zero.
__device__ __forceinline__ int kv_code(float x, float r)
{
    float y = roundf(__fmul_rn(x, r));
    y = fminf(fmaxf(y, -127.0f), 127.0f);
    return (int)y;
}

// Q block: given the block's max-abs m, the block scale and the reciprocal.
struct BlockQuant {
    float qscale;
    float recip;
};

__device__ __forceinline__ BlockQuant q_block_params(float mabs)
{
    float m = (mabs < kGuard) ? 1.0f : mabs;
    BlockQuant q;
    q.qscale = __fmul_rn(m, kInv127);
    q.recip = 127.0f / m;
    return q;
}

// code = conversion toward zero of clamp(q * r, -128, 127).
__device__ __forceinline__ int q_code(float x, float r)
{
    float y = __fmul_rn(x, r);
    y = fminf(fmaxf(y, -128.0f), 127.0f);
    return (int)y;    // v_cvt_i32_f32 truncates toward zero
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d)
{
    return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
           ((uint32_t)(d & 0xff) << 24);
}

// ------------------------------------------------------------ lane exchanges
// DPP controls (within rows of 16 lanes).
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;   // lane i of each 8 reads lane 7-i
constexpr int kDppRor8 = 0x128;         // lane i of each 16 reads lane (i+8) mod 16

template <int Ctrl>
__device__ __forceinline__ int dpp_i(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, Ctrl, 0xF, 0xF, false);
}

template <int Ctrl>
__device__ __forceinline__ float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), Ctrl, 0xF, 0xF, false));
}

// Across rows: v_permlane16_swap / v_permlane32_swap (VALU, no LDS round
// trip).  Swapping a register with itself leaves, in every lane, its own
// value and the value of the lane 16 (32) away, one in each result; the
// reductions below combine the two symmetrically, so every lane gets the
// same bits.
__device__ __forceinline__ float sum_rows16(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_rows32(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_rows16(float v)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_rows32(float v)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sums over the 8 token slots of a wave (lane 8 s + c is slot s) of N values
// per lane, scattered over the slots: slot s ends with the sums of values
// [s N / 8, (s + 1) N / 8) in z.  Three halving steps, each pairing a value
// of the kept half with one of the given-away half: the 32-lane halves
// (v_permlane32_swap of the pair leaves, in every lane, its own kept value in
// one result and the partner's in the other), then the 16-lane rows
// (v_permlane16_swap), then slots s and s ^ 1, 8 lanes apart in a row (DPP
// row rotation by 8).  N / 2 + N / 4 + N / 8 exchanges, against 3 N for a
// full sum of every value in every lane.
template <int N>
__device__ __forceinline__ void slot_reduce_scatter(const float (&v)[N], float (&z)[N / 8], int lane)
{
    static_assert(N % 8 == 0, "eight slots");
    float w[N / 2], u[N / 4];
    // lanes 0-31 keep values [0, N/2), lanes 32-63 [N/2, N): the swap moves
    // the upper lanes of its first operand and the lower lanes of its second
#pragma unroll
    for (int k = 0; k < N / 2; ++k) {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[k]), __float_as_uint(v[k + N / 2]),
                                                        false, false);
        w[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    // even rows of a half keep [0, N/4), odd rows [N/4, N/2): the swap moves
    // the odd rows of its first operand and the even rows of its second
#pragma unroll
    for (int k = 0; k < N / 4; ++k) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(w[k]), __float_as_uint(w[k + N / 4]),
                                                        false, false);
        u[k] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    // even slots keep [0, N/8), odd slots [N/8, N/4)
    const bool odd = (lane >> 3) & 1;
#pragma unroll
    for (int k = 0; k < N / 8; ++k) {
        const float keep = odd ? u[k + N / 8] : u[k], give = odd ? u[k] : u[k + N / 8];
        z[k] = keep + dpp_f<kDppRor8>(give);
    }
}

// P consecutive floats to dst (P = 2, 4, 8 or 16; dst aligned to 4 P bytes).
template <int P>
__device__ __forceinline__ void store_floats(float *dst, const float (&x)[P])
{
    if constexpr (P == 2) {
        *reinterpret_cast<float2 *>(dst) = make_float2(x[0], x[1]);
    } else {
#pragma unroll
        for (int i = 0; i < P / 4; ++i)
            reinterpret_cast<float4 *>(dst)[i] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
    }
}

// Sum / max over the 8 token slots of a wave (lanes that share lane % 8).
__device__ __forceinline__ float sum_over_slots(float v)
{
    v += dpp_f<kDppRor8>(v);
    return sum_rows32(sum_rows16(v));
}

__device__ __forceinline__ float max_over_slots(float v)
{
    v = fmaxf(v, dpp_f<kDppRor8>(v));
    return max_rows32(max_rows16(v));
}

__device__ __forceinline__ float wave_max(float v)
{
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// ------------------------------------------------------------ int8 dot helpers
// Sum of 16 int8 x int8 products (one lane's quarter of a 32-block pair).
__device__ __forceinline__ int dot16_i8(const uint4 &k, const uint4 &q)
{
    int acc = 0;
    acc = __builtin_amdgcn_sdot4((int)k.x, (int)q.x, acc, false);
    acc = __builtin_amdgcn_sdot4((int)k.y, (int)q.y, acc, false);
    acc = __builtin_amdgcn_sdot4((int)k.z, (int)q.z, acc, false);
    acc = __builtin_amdgcn_sdot4((int)k.w, (int)q.w, acc, false);
    return acc;
}

// Exact 32-block sum: each block is held by two neighbouring lanes (c, c^1).
__device__ __forceinline__ int block_partial(const uint4 &k, const uint4 &q)
{
    int p = dot16_i8(k, q);
    return p + dpp_i<kDppQuadXor1>(p);
}

// int8 byte b of word w, sign-extended, as float (one v_cvt_f32_i32 with SDWA).
__device__ __forceinline__ float byte_f(uint32_t w, int b)
{
    return (float)(int)(int8_t)((w >> (8 * b)) & 0xff);
}

// Bits of a where m is set, of b elsewhere (v_bfi_b32).
__device__ __forceinline__ uint32_t bitsel(uint32_t m, uint32_t a, uint32_t b)
{
    return (m & a) | (~m & b);
}

// --------------------------------------------------------- matrix cores
typedef float v4f __attribute__((ext_vector_type(4)));

// v_mfma_f32_4x4x1_16b_f32: the wave is 16 blocks of 4 lanes; in block b,
// register i of lane 4b + j gains a(lane 4b + i) * b(lane 4b + j) -- an fp32
// outer product of the block's 4 a values and 4 b values.
__device__ __forceinline__ v4f mfma_outer4(float a, float b, v4f c)
{
    return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------ query quantization
// Lane (slot, c) of a wave owns elements [16c, 16c+16) of a 128-element query
// row; the 32-block of those elements is shared with lane c^1.  Quantizes the
// lane's 16 elements, given in registers (a, b, d, e in element order, so a
// caller can issue other loads between loading them and this call), and
// returns their codes (16 bytes) and the block scale.
__device__ __forceinline__ void quantize_q_quarter_vals(const float4 &a, const float4 &b, const float4 &d,
                                                        const float4 &e, uint4 &codes, float &qscale)
{
    float x[16] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w, d.x, d.y, d.z, d.w, e.x, e.y, e.z, e.w};
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(x[i]));
    m = fmaxf(m, dpp_f<kDppQuadXor1>(m));   // max over the whole 32-block
    BlockQuant bq = q_block_params(m);
    int cd[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) cd[i] = q_code(x[i], bq.recip);
    codes.x = pack4_i8(cd[0], cd[1], cd[2], cd[3]);
    codes.y = pack4_i8(cd[4], cd[5], cd[6], cd[7]);
    codes.z = pack4_i8(cd[8], cd[9], cd[10], cd[11]);
    codes.w = pack4_i8(cd[12], cd[13], cd[14], cd[15]);
    qscale = bq.qscale;
}

// The same, loading the lane's 16 elements of query row `qrow`.
__device__ __forceinline__ void quantize_q_quarter(const float *__restrict__ qrow, int c,
                                                   uint4 &codes, float &qscale)
{
    const float4 *p = reinterpret_cast<const float4 *>(qrow + 16 * c);
    quantize_q_quarter_vals(p[0], p[1], p[2], p[3], codes, qscale);
}

// Codes and step of one 32-float block of a query row, in one lane: the
// decode kernel's query quantizer (step = max|x| * fl(1/127), code =
// clamp(x * 127 / max|x|) truncated toward zero).
__device__ __forceinline__ void quantize_q_block_vals(const float4 (&p)[8], uint4 &lo, uint4 &hi, float &qscale)
{
    float x[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 v = p[i];
        x[4 * i] = v.x;
        x[4 * i + 1] = v.y;
        x[4 * i + 2] = v.z;
        x[4 * i + 3] = v.w;
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(x[i]));
    const BlockQuant bq = q_block_params(m);
    int cd[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) cd[i] = q_code(x[i], bq.recip);
    lo = make_uint4(pack4_i8(cd[0], cd[1], cd[2], cd[3]), pack4_i8(cd[4], cd[5], cd[6], cd[7]),
                    pack4_i8(cd[8], cd[9], cd[10], cd[11]), pack4_i8(cd[12], cd[13], cd[14], cd[15]));
    hi = make_uint4(pack4_i8(cd[16], cd[17], cd[18], cd[19]), pack4_i8(cd[20], cd[21], cd[22], cd[23]),
                    pack4_i8(cd[24], cd[25], cd[26], cd[27]), pack4_i8(cd[28], cd[29], cd[30], cd[31]));
    qscale = bq.qscale;
}

// The same, loading the block from q32.
__device__ __forceinline__ void quantize_q_block(const float *q32, uint4 &lo, uint4 &hi, float &qscale)
{
    const float4 *p = reinterpret_cast<const float4 *>(q32);
    float4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = p[i];
    quantize_q_block_vals(v, lo, hi, qscale);
}

// One (token, KV head) row of the append, one wave: each lane holds 2 of the
// 128 K and V values (k, v: dims 2 lane, 2 lane + 1), the wave max gives the
// exact max-abs, every lane writes its 2 codes (a 128-byte row per wave) and
// lane 0 the steps.  The codes go to cache row `cache_row` (= block * kv_bs +
// row in block), head kh; steps are stored [block][kv head][row]; the fp32
// mirror, if any, gets the row as is.
__device__ __forceinline__ void append_row_vals(int8_t *k_codes, int8_t *v_codes, float *k_scale, float *v_scale,
                                                float *k_f32, float *v_f32, int nkv, int kv_bs_log2, int blk,
                                                int row_in_blk, int kh, float2 k, float2 v, int lane)
{
    const float ka = wave_max(fmaxf(fabsf(k.x), fabsf(k.y)));
    const float va = wave_max(fmaxf(fabsf(v.x), fabsf(v.y)));
    const RowQuant kq = kv_row_params(ka);
    const RowQuant vq = kv_row_params(va);
    const size_t cache_row = ((size_t)blk << kv_bs_log2) + row_in_blk;
    const size_t dst = (cache_row * nkv + kh) * kHeadDim + 2 * lane;
    const size_t sdst = (((size_t)blk * nkv + kh) << kv_bs_log2) + row_in_blk;
    const uint16_t kc = (uint16_t)((kv_code(k.x, kq.recip) & 0xff) | ((kv_code(k.y, kq.recip) & 0xff) << 8));
    const uint16_t vc = (uint16_t)((kv_code(v.x, vq.recip) & 0xff) | ((kv_code(v.y, vq.recip) & 0xff) << 8));
    *reinterpret_cast<uint16_t *>(k_codes + dst) = kc;
    *reinterpret_cast<uint16_t *>(v_codes + dst) = vc;
    if (k_f32) {   // the fp32 mirror keeps the row unchanged
        *reinterpret_cast<float2 *>(k_f32 + dst) = k;
        *reinterpret_cast<float2 *>(v_f32 + dst) = v;
    }
    if (lane == 0) {
        k_scale[sdst] = kq.step;
        v_scale[sdst] = vq.step;
    }
}

// append_row_vals with the row read from k_src / v_src (128 fp32 each).
__device__ __forceinline__ void append_row(int8_t *k_codes, int8_t *v_codes, float *k_scale, float *v_scale,
                                           float *k_f32, float *v_f32, int nkv, int kv_bs_log2, int blk,
                                           int row_in_blk, int kh, const float *k_src, const float *v_src, int lane)
{
    const float2 k = *reinterpret_cast<const float2 *>(k_src + 2 * lane);
    const float2 v = *reinterpret_cast<const float2 *>(v_src + 2 * lane);
    append_row_vals(k_codes, v_codes, k_scale, v_scale, k_f32, v_f32, nkv, kv_bs_log2, blk, row_in_blk, kh, k, v,
                    lane);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

}  // namespace q8kv
