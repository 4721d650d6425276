// q8kv_prefill.hip -- batched prefill attention over the q8 cache on the
// matrix cores.
//
// Method ("why long context must be sparse" §1-§2: the exact batched prefill
// path; a batch of nb new tokens scores against the whole history): the new
// tokens of sequence b are the last nb_b positions of its cache (appended
// before the call); query row r at position p attends to positions 0..p.
// Each query row is quantized like the decode query (per 32-block step
// m * fl(1/127), codes truncated), and its attention is the decode's:
// s_t = ((sum_beta float(P_beta) * qs_beta) * ks_t) * scale with exact
// block partials P_beta, softmax over t <= p, weights times V codes and V
// steps, one division at the end ("9-2 flash_attn_single_q_q8_neon" §2).
//
// A workgroup owns 128 query rows of one KV head (row rho = position * G +
// head of the flattened (position, query head) list) and splits their key
// range 0..p_max in two: each half is walked by a group of four waves, one
// wave per 32 rows.  The four waves of a group walk the same 32-token key
// tiles, so each tile is loaded from HBM once per group and converted once
// into matrix-core operands in LDS, which all four read:
//   K  as fp16 codes (exact; two codes per byte permute and one packed fp16
//      subtraction, below);
//   V^T as bf16 (codes are exact in bf16), each dim row holding the 32 tokens
//      in the order of the weight operand below.
// Per tile, with 32x32 matrix-core products (lane l: query j = l % 32, half
// hf = l / 32):
//   scores  S^T = K Q^T with v_mfma_f32_32x32x16_f16, two k-steps of 16 dims
//           per 32-block beta: every product and partial sum is an integer of
//           magnitude below 2^19, so the result is the exact block partial
//           P_beta, as an int32 product would give it; the lane then holds
//           query j's partials with tokens 8 g + 4 hf + e (g, e = 0..3);
//   softmax online per query (log2 domain) with a reference max (below);
//   values  O^T += V^T P^T with v_mfma_f32_32x32x16_bf16: the lane's 16
//           weights are already its slots of the B operands of the two
//           16-token k-steps; each fp32 weight w = p * vs is split exactly
//           into three bf16 terms (w = hi + mid + lo by truncation, the
//           "bf16x3" form of an fp32 product) and V codes are exact in bf16,
//           so every product is exact and only the fp32 accumulation order
//           differs from a scalar loop: six products per 32 dims.
// The second group's states are folded into the first's at the end through
// LDS (the decode merge rule), so the result is deterministic.
#include "q8kv_tile.hpp"
#include "q8kv_internal.hpp"

namespace q8kv {

typedef _Float16 v8h_t __attribute__((ext_vector_type(8)));
typedef _Float16 v2h_t __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

constexpr int kPfGroups = 2;                          // key-range halves per workgroup
constexpr int kPfRowWaves = 4;                        // waves per half, one per 32 rows
constexpr int kPfWaves = kPfGroups * kPfRowWaves;
constexpr int kPfRows = 32;                           // query rows per wave
constexpr int kPfBlockRows = kPfRowWaves * kPfRows;   // query rows per workgroup
constexpr int kKeyTile = 32;                          // tokens per step
constexpr int kKRow = 136;                            // halves per staged K row (128 + 8 pad)
constexpr int kVRow = 40;                             // halves per staged V^T row (32 + 8 pad)

// One staged key tile of one group.
struct Stage {
    uint16_t k[kKeyTile * kKRow];     // K rows, fp16 codes, dims in order
    uint16_t vt[kHeadDim * kVRow];    // V^T rows, bf16 codes; chunk 2 r + hf, slot 4 g + e = token
                                      // 16 r + 8 g + 4 hf + e (chunk c stored at vt_chunk(d, c))
    float kss[kKeyTile];              // ks * scale * log2(e)
    float vs[kKeyTile];
    uint32_t good;                    // bit t: token t's block id is valid
    uint32_t pad[3];
};
// Second group's per-lane states for the fold: [row wave][64 accumulators, M, S][lane].
constexpr int kCombVals = 4 * 16 + 2;
constexpr size_t kStageBytes = sizeof(Stage) * kPfGroups * 2;
constexpr size_t kCombBytes = sizeof(float) * kPfRowWaves * kCombVals * 64;
constexpr size_t kPfLds = kStageBytes > kCombBytes ? kStageBytes : kCombBytes;
static_assert(sizeof(Stage) % 16 == 0, "stages stay 16-byte aligned");

struct PrefillParams {
    CacheView cache;
    const int32_t *block_table;
    const int32_t *seq_lens;
    const int32_t *q_start;
    const float *q;
    float *out;
    int32_t *dev_status;
    int32_t nq, max_blocks_per_seq, max_seq_len, max_new, total_q, log2g;
    float sc;     // softmax scale * log2(e)
};

// One thread's share of a key tile as loaded: 16 K bytes of one token, 4 V
// bytes of 4 tokens, and (lanes 0..31 of the group's first two waves) the K
// or V step of token lane.
struct TileRaw {
    uint4 k;
    uint32_t v[4];
    float s;
    bool good;   // the block id behind the step is valid
    bool bad;    // some block id behind this thread's loads is not
};

// The V share of thread gt: token quad a (tokens 4 a .. 4 a + 3, a = 4 r +
// 2 g + hf for tokens 16 r + 8 g + 4 hf + e) and dim quad c (dims 4 c ..
// 4 c + 3).  Sixteen neighbouring lanes read 64 contiguous bytes of a row,
// and each sixteen write 16 different bank quads of the staged V^T (below).
__device__ __forceinline__ int v_quad(int gt) { return (((gt >> 4) & 1) << 2) | (gt >> 6); }
__device__ __forceinline__ int v_dims(int gt) { return (gt & 15) | (((gt >> 5) & 1) << 4); }

// V^T row d keeps its four 16-byte chunks (one k-step and lane half's 8
// token slots) at chunk c ^ ((d / 16) % 4): the readers of a chunk (rows
// 32 dt + j) keep distinct banks within each 16 rows, and the writers of one
// dim of four tokens (rows 4 c + dd) spread over every bank.
__device__ __forceinline__ int vt_chunk(int d, int c) { return c ^ ((d >> 4) & 3); }

// Block ids of a tile, fetched one tile ahead of its loads.  Big (kv_bs >= 32):
// the tile lies in one block, one wave-uniform id; otherwise each thread
// looks up the blocks of its own tokens (tokens past the workgroup's last
// position are clamped to it: no row attends to them).
struct TileIds {
    int k, v, s;
};

template <bool Big>
__device__ __forceinline__ TileIds tile_ids(const PrefillParams &p, const int32_t *bt, int t0, int p_hi, int gt)
{
    const int log2bs = p.cache.kv_bs_log2;
    TileIds ids;
    if (Big) {
        ids.k = ids.v = ids.s = uniform(((const_i32 *)bt)[t0 >> log2bs]);
    } else {
        ids.k = bt[min(t0 + (gt >> 3), p_hi) >> log2bs];
        ids.v = bt[min(t0 + 4 * v_quad(gt), p_hi) >> log2bs];
        ids.s = bt[min(t0 + (gt & 31), p_hi) >> log2bs];
    }
    return ids;
}

// A thread's byte offsets inside a tile, from the tile's first row: K row
// gt / 8, bytes 16 (gt % 8); V rows 4 v_quad + u, bytes 4 v_dims.
struct TileOffsets {
    uint32_t k, v;
};

template <bool Big>
__device__ __forceinline__ void load_tile(const PrefillParams &p, int kh, int t0, int p_hi, int gt,
                                          const TileOffsets &off, const TileIds &ids, TileRaw &r)
{
    const int nkv = p.cache.nkv, row_bytes = nkv * kHeadDim;
    const int log2bs = p.cache.kv_bs_log2, bmask = (1 << log2bs) - 1;
    const unsigned nb = (unsigned)p.cache.num_blocks;
    if (Big) {
        // one block: buffer resources over the tile's rows (uniform), fixed
        // per-thread offsets; default caching, since the other row blocks of
        // the sequence read the same tile from L2
        r.good = (unsigned)ids.s < nb;
        r.bad = !r.good;
        const int id = r.good ? ids.s : 0;
        const size_t row0 = ((size_t)id << log2bs) + (size_t)(t0 & bmask);
        const int tile_bytes = kKeyTile * row_bytes;
        const __amdgpu_buffer_rsrc_t kr = make_rsrc(p.cache.k_codes + row0 * row_bytes, tile_bytes);
        const __amdgpu_buffer_rsrc_t vr = make_rsrc(p.cache.v_codes + row0 * row_bytes, tile_bytes);
        r.k = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, (int)off.k, 0, 0));
#pragma unroll
        for (int u = 0; u < 4; ++u)
            r.v[u] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(vr, (int)off.v, u * row_bytes, 0));
        // steps: wave 0 of the group the K steps (lane t: token t), wave 1
        // the V steps (one wave-uniform resource each)
        const int sw = uniform(gt >> 6);
        if (sw < 2) {
            const size_t s0 = (((size_t)id * nkv + kh) << log2bs) + (size_t)(t0 & bmask);
            r.s = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                make_rsrc((sw == 0 ? p.cache.k_scale : p.cache.v_scale) + s0, 4 * kKeyTile),
                                                4 * (gt & 31), 0, 0));
        }
        return;
    }
    auto row_of = [&](int id, int t) {   // physical row of token t in block id (0 for a bad id)
        return ((size_t)((unsigned)id < nb ? id : 0) << log2bs) + (size_t)(t & bmask);
    };
    {
        const int t = min(t0 + (gt >> 3), p_hi);
        r.k = *reinterpret_cast<const uint4 *>(p.cache.k_codes + row_of(ids.k, t) * row_bytes + kh * kHeadDim +
                                               16 * (gt & 7));
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int t = min(t0 + 4 * v_quad(gt) + u, p_hi);
        r.v[u] = *reinterpret_cast<const uint32_t *>(p.cache.v_codes + row_of(ids.v, t) * row_bytes +
                                                     kh * kHeadDim + 4 * v_dims(gt));
    }
    r.good = (unsigned)ids.s < nb;
    r.bad = !r.good || (unsigned)ids.k >= nb || (unsigned)ids.v >= nb;
    if ((gt >> 6) < 2) {
        const int t = min(t0 + (gt & 31), p_hi);
        const size_t sidx = ((((size_t)(r.good ? ids.s : 0)) * nkv + kh) << log2bs) + (size_t)(t & bmask);
        r.s = ((gt >> 6) == 0 ? p.cache.k_scale : p.cache.v_scale)[sidx];
    }
}

// Converts a thread's loaded share into the stage's operand layouts.
__device__ __forceinline__ void stage_tile(const PrefillParams &p, const TileRaw &r, int gt, Stage &s)
{
    // K: code c -> fp16 c, as (1024 + (c + 128)) - 1152: the code plus 128 is
    // the low byte of an fp16 whose exponent field makes it 1024 plus that
    // byte (one byte permute per two codes), and one packed fp16 subtraction
    // per two codes is exact
    const uint32_t kx[4] = {r.k.x ^ 0x80808080u, r.k.y ^ 0x80808080u, r.k.z ^ 0x80808080u, r.k.w ^ 0x80808080u};
    uint32_t kh16[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        kh16[2 * i] = __builtin_amdgcn_perm(0x64646464u, kx[i], 0x04010400u);
        kh16[2 * i + 1] = __builtin_amdgcn_perm(0x64646464u, kx[i], 0x04030402u);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const v2h_t x = __builtin_bit_cast(v2h_t, kh16[i]) - v2h_t{(_Float16)1152.0f, (_Float16)1152.0f};
        kh16[i] = __builtin_bit_cast(uint32_t, x);
    }
    uint4 *kd = reinterpret_cast<uint4 *>(s.k + (gt >> 3) * kKRow + 16 * (gt & 7));
    kd[0] = make_uint4(kh16[0], kh16[1], kh16[2], kh16[3]);
    kd[1] = make_uint4(kh16[4], kh16[5], kh16[6], kh16[7]);
    // V^T: dims 4 c + dd, tokens 4 a .. 4 a + 3 (a = 4 r + 2 g + hf: chunk 2 r + hf, slots 4 g ..)
    const int a = v_quad(gt), c = v_dims(gt);
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) {
        const int d = 4 * c + dd;
        const uint32_t f0 = __float_as_uint(byte_f(r.v[0], dd)), f1 = __float_as_uint(byte_f(r.v[1], dd));
        const uint32_t f2 = __float_as_uint(byte_f(r.v[2], dd)), f3 = __float_as_uint(byte_f(r.v[3], dd));
        *reinterpret_cast<uint2 *>(s.vt + d * kVRow + 8 * vt_chunk(d, 2 * (a >> 2) + (a & 1)) + 4 * ((a >> 1) & 1)) =
            make_uint2(__builtin_amdgcn_perm(f1, f0, 0x07060302u), __builtin_amdgcn_perm(f3, f2, 0x07060302u));
    }
    if ((gt >> 6) == 0) {
        if (gt < 32) s.kss[gt] = r.s * p.sc;
        const uint64_t g = __builtin_amdgcn_ballot_w64(r.good);
        if (gt == 0) s.good = (uint32_t)g;
    } else if ((gt >> 6) == 1 && (gt & 63) < 32) {
        s.vs[gt & 31] = r.s;
    }
}

// Exact split of 8 fp32 weights into three bf16 terms each (truncation: the
// first term keeps the top 8 significant bits, the second the next 8, the
// third the rest; both subtractions are exact).
__device__ __forceinline__ void split_bf16x3(const float (&w)[8], v8bf_t &hi, v8bf_t &mid, v8bf_t &lo)
{
    uint32_t h[8], m[8], l[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        h[e] = __float_as_uint(w[e]) & 0xffff0000u;
        const float r1 = w[e] - __uint_as_float(h[e]);
        m[e] = __float_as_uint(r1) & 0xffff0000u;
        const float r2 = r1 - __uint_as_float(m[e]);
        l[e] = __float_as_uint(r2);
    }
    uint32_t ph[4], pm[4], pl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        ph[i] = __builtin_amdgcn_perm(h[2 * i + 1], h[2 * i], 0x07060302u);
        pm[i] = __builtin_amdgcn_perm(m[2 * i + 1], m[2 * i], 0x07060302u);
        pl[i] = __builtin_amdgcn_perm(l[2 * i + 1], l[2 * i], 0x07060302u);
    }
    hi = __builtin_bit_cast(v8bf_t, make_uint4(ph[0], ph[1], ph[2], ph[3]));
    mid = __builtin_bit_cast(v8bf_t, make_uint4(pm[0], pm[1], pm[2], pm[3]));
    lo = __builtin_bit_cast(v8bf_t, make_uint4(pl[0], pl[1], pl[2], pl[3]));
}

template <bool Big>
__global__ __launch_bounds__(64 * kPfWaves) void q8_prefill_kernel(PrefillParams p)
{
    __shared__ __align__(16) unsigned char lds[kPfLds];
    // each wave's query operands, k-step s (dims 16 s + 8 hf ..), read back by the same lanes every tile
    __shared__ __align__(16) v8h_t q_lds[kPfWaves][8][64];
    Stage *stages = reinterpret_cast<Stage *>(lds);   // [group][buffer]
    const int nkv = p.cache.nkv;
    const int b = blockIdx.x / nkv, kh = blockIdx.x - (blockIdx.x / nkv) * nkv;
    const int wave = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int grp = wave / kPfRowWaves, rw = wave % kPfRowWaves;
    const int gt = (int)threadIdx.x - grp * 64 * kPfRowWaves;   // thread within the group
    // the last row blocks (the longest key ranges under the causal mask) are
    // dispatched first, so the short ones fill in behind them
    const int rb = gridDim.y - 1 - blockIdx.y;
    const int G = 1 << p.log2g;
    const int j = lane & 31, hf = lane >> 5;   // the lane's query row in the wave, and its half

    const int r0 = uniform(p.q_start[b]), r1 = uniform(p.q_start[b + 1]);
    const int n = uniform(p.seq_lens[b]);
    const bool range_ok = 0 <= r0 && r0 <= r1 && r1 <= p.total_q;
    const int nn = r1 - r0;
    const int wrow0 = rb * kPfBlockRows + rw * kPfRows;   // this wave's first row
    if (!range_ok || n < nn || n > p.max_seq_len || nn > p.max_new) {
        // a bad sequence (uniform over the workgroup): reported; its rows
        // that this workgroup covers are zeros
        if (kh == 0 && rb == 0 && threadIdx.x == 0 && p.dev_status) atomicOr(p.dev_status, kDevBadSeqLen);
        const int rho = wrow0 + j;
        if (range_ok && grp == 0 && rho < (nn << p.log2g)) {
            const int i = rho >> p.log2g, g = rho & (G - 1);
            float *o = p.out + ((size_t)(r0 + i) * p.nq + kh * G + g) * kHeadDim;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4)
                    reinterpret_cast<float4 *>(o + 32 * dt + 8 * q4 + 4 * hf)[0] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        return;
    }
    const int rows = nn << p.log2g;
    if (rb * kPfBlockRows >= rows) return;   // uniform over the workgroup

    // the workgroup's key range, cut into two halves of (almost) equal tile counts
    const int p0 = n - nn;   // position of the first new token
    const int p_hi = p0 + (min(rb * kPfBlockRows + kPfBlockRows - 1, rows - 1) >> p.log2g);
    const int nkt = p_hi / kKeyTile + 1;
    const int half = nkt >> 1;
    const int kt_lo = grp == 0 ? 0 : half, cnt = grp == 0 ? half : nkt - half;
    const int iters = nkt - half;   // the same for every wave: the barrier count

    // this lane's row, clamped to a real row (lanes past the end are computed
    // and discarded), and its position
    const bool active = wrow0 < rows;
    const int rho = wrow0 + j;
    const bool live = rho < rows;
    const int rr = live ? rho : rows - 1;
    const int qi = rr >> p.log2g, qg = rr & (G - 1);
    const int pos = p0 + qi;
    const int pw_hi = p0 + (min(wrow0 + kPfRows - 1, rows - 1) >> p.log2g);   // the wave's largest position
    const int pw_lo = p0 + (wrow0 >> p.log2g);                                 // and smallest

    // query codes as fp16, the B operands of the score products (k-step s:
    // dims 16 s + 8 hf .. + 7 of query j), kept in LDS, and their block steps;
    // the two halves of a 32-block sit in lanes j and j + 32
    v8h_t (*qb)[64] = q_lds[wave];
    float qs[4];
    {
        const float *qrow = p.q + ((size_t)(r0 + qi) * p.nq + kh * G + qg) * kHeadDim;
#pragma unroll
        for (int beta = 0; beta < 4; ++beta) {
            const float4 a0 = *reinterpret_cast<const float4 *>(qrow + 32 * beta + 8 * hf);
            const float4 a1 = *reinterpret_cast<const float4 *>(qrow + 32 * beta + 8 * hf + 4);
            const float4 b0 = *reinterpret_cast<const float4 *>(qrow + 32 * beta + 16 + 8 * hf);
            const float4 b1 = *reinterpret_cast<const float4 *>(qrow + 32 * beta + 16 + 8 * hf + 4);
            const float x[16] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w,
                                 b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
            float m = 0.0f;
#pragma unroll
            for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(x[e]));
            m = max_rows32(m);   // the 32-block's max over the two halves
            const BlockQuant bq = q_block_params(m);
            v8h_t c0, c1;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                c0[e] = (_Float16)q_code(x[e], bq.recip);
                c1[e] = (_Float16)q_code(x[8 + e], bq.recip);
            }
            qb[2 * beta][lane] = c0;
            qb[2 * beta + 1][lane] = c1;
            qs[beta] = bq.qscale;
        }
    }

    // M is a reference max per query: the weights exp2(s - M) may exceed 1 by
    // up to 2^kLazyRescale, and S and the accumulators are rescaled only when
    // the query's tile max rises above its M by more than that (the result is
    // the same quantity; only rounding differs)
    constexpr float kLazyRescale = 8.0f;
    float M = -INFINITY, S = 0.0f;
    v16f_t acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[dt][v] = 0.0f;

    const int32_t *bt = p.block_table + (size_t)b * p.max_blocks_per_seq;
    bool bad = false;
    // pipeline: while tile i is computed, tile i + 1 is converted into the
    // other buffer (before the computation, in the same iteration), tile
    // i + 2's loads and tile i + 3's block ids are in flight
    const int row_bytes = nkv * kHeadDim;
    const TileOffsets off = {(uint32_t)((gt >> 3) * row_bytes + kh * kHeadDim + 16 * (gt & 7)),
                             (uint32_t)(4 * v_quad(gt) * row_bytes + kh * kHeadDim + 4 * v_dims(gt))};
    TileRaw raw;
    TileIds ids_next = {0, 0, 0};
    // stage tile k of the group into its buffer and start the loads of tile k + 1
    auto advance = [&](int k) {
        stage_tile(p, raw, gt, stages[2 * grp + (k & 1)]);
        bad = bad || raw.bad;
        if (k + 1 < cnt) {
            const TileIds ids = ids_next;
            if (k + 2 < cnt) ids_next = tile_ids<Big>(p, bt, (kt_lo + k + 2) * kKeyTile, p_hi, gt);
            load_tile<Big>(p, kh, (kt_lo + k + 1) * kKeyTile, p_hi, gt, off, ids, raw);
        }
    };
    if (cnt > 0) {
        const TileIds ids0 = tile_ids<Big>(p, bt, kt_lo * kKeyTile, p_hi, gt);
        if (cnt > 1) ids_next = tile_ids<Big>(p, bt, (kt_lo + 1) * kKeyTile, p_hi, gt);
        load_tile<Big>(p, kh, kt_lo * kKeyTile, p_hi, gt, off, ids0, raw);
        advance(0);
    }
    // the lane's K operand row: token j, dims 16 s + 8 hf ..
    const int krow = j * kKRow + 8 * hf;
    for (int i = 0; i < iters; ++i) {
        // tile i is staged (buffer i % 2); buffer (i + 1) % 2 is free: its
        // readers finished tile i - 1 before this barrier
        __syncthreads();
        const Stage &sg = stages[2 * grp + (i & 1)];
        const int t0 = (kt_lo + i) * kKeyTile;
        const bool work = i < cnt && active && t0 <= pw_hi;
        if (i + 1 < cnt) advance(i + 1);
        if (!work) continue;

        const uint32_t gmask = sg.good;
        // every row of the wave sees all 32 tokens of the tile: no masks
        const bool full = t0 + kKeyTile - 1 <= pw_lo && gmask == 0xffffffffu;
        // block partials: c[beta][v] for token 8 (v / 4) + 4 hf + v % 4 of
        // query j (two k-steps of 16 dims per block)
        v16f_t c[4];
#pragma unroll
        for (int st = 0; st < 8; ++st) {
            const v8h_t ka = *reinterpret_cast<const v8h_t *>(sg.k + krow + 16 * st);
            const v8h_t qv = qb[st][lane];
            v16f_t z;
            if (st & 1) z = c[st >> 1];
            else
#pragma unroll
                for (int v = 0; v < 16; ++v) z[v] = 0.0f;
            c[st >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka, qv, z, 0, 0, 0);
        }
        // V operands: dims 32 dt + j, k-step r = tokens 16 r + 8 g + 4 hf + e
        // (chunk 2 r + hf); read now, the softmax covers their latency
        v8bf_t va[8];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int d = 32 * dt + j;
                va[2 * dt + r] = *reinterpret_cast<const v8bf_t *>(sg.vt + d * kVRow + 8 * vt_chunk(d, 2 * r + hf));
            }
        float kss[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float4 k4 = *reinterpret_cast<const float4 *>(sg.kss + 8 * q4 + 4 * hf);
            kss[4 * q4] = k4.x; kss[4 * q4 + 1] = k4.y; kss[4 * q4 + 2] = k4.z; kss[4 * q4 + 3] = k4.w;
        }
        __builtin_amdgcn_sched_barrier(0);
        float s[16];
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            // (P0 qs0 + P1 qs1) + (P3 qs3 + P2 qs2), the second product of each pair fused
            const float y01 = fmaf(c[1][v], qs[1], c[0][v] * qs[0]);
            const float y23 = fmaf(c[2][v], qs[2], c[3][v] * qs[3]);
            s[v] = (y01 + y23) * kss[v];
        }
        uint32_t keep[16];
        if (!full) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int tt = 8 * (v >> 2) + 4 * hf + (v & 3);   // token within the tile
                keep[v] = (t0 + tt <= pos && ((gmask >> tt) & 1u)) ? 0xffffffffu : 0u;
                // branch-free mask (a select here becomes a divergent
                // branch); a masked token's step may be any bits, even NaN
                s[v] = __uint_as_float(bitsel(keep[v], __float_as_uint(s[v]), 0xff800000u));
            }
        }
        float m = s[0];
#pragma unroll
        for (int v = 1; v < 16; ++v) m = fmaxf(m, s[v]);
        m = max_rows32(m);   // the tile max of query j over both halves
        const bool grow = m > M + kLazyRescale;   // also true on the first tile with a finite max
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            const float Mn = grow ? m : M;
            const float alpha = Mn == -INFINITY ? 1.0f : __builtin_amdgcn_exp2f(M - Mn);
            M = Mn;
            S *= alpha;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) acc[dt] *= alpha;
        }
        float vsv[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            const float4 v4 = *reinterpret_cast<const float4 *>(sg.vs + 8 * q4 + 4 * hf);
            vsv[4 * q4] = v4.x; vsv[4 * q4 + 1] = v4.y; vsv[4 * q4 + 2] = v4.z; vsv[4 * q4 + 3] = v4.w;
        }
        float w[16], psum = 0.0f;
        if (full) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float pw = __builtin_amdgcn_exp2f(s[v] - M);
                psum += pw;
                w[v] = pw * vsv[v];
            }
        } else {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                // masked: weight 0 (M may still be -inf, and the step may be NaN)
                const float pw =
                    __uint_as_float(bitsel(keep[v], __float_as_uint(__builtin_amdgcn_exp2f(s[v] - M)), 0u));
                psum += pw;
                w[v] = __uint_as_float(bitsel(keep[v], __float_as_uint(pw * vsv[v]), 0u));
            }
        }
        S += psum;
        v8bf_t wt[3][2];   // [term][k-step]: the lane's weights v = 8 r .. 8 r + 7
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const float w8[8] = {w[8 * r], w[8 * r + 1], w[8 * r + 2], w[8 * r + 3],
                                 w[8 * r + 4], w[8 * r + 5], w[8 * r + 6], w[8 * r + 7]};
            split_bf16x3(w8, wt[0][r], wt[1][r], wt[2][r]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int term = 0; term < 3; ++term)
#pragma unroll
            for (int r = 0; r < 2; ++r)
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
                    acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[2 * dt + r], wt[term][r], acc[dt], 0, 0, 0);
    }
    if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0 && p.dev_status) atomicOr(p.dev_status, kDevBadBlockId);

    // the second half's states into the first's: M the larger, S and the
    // accumulators rescaled to it and summed in key order ("9-2" §2 segment 2
    // rule applied to partial states); deterministic
    __syncthreads();   // every wave is done with the stages
    float(*comb)[kCombVals][64] = reinterpret_cast<float(*)[kCombVals][64]>(lds);
    if (active && grp == 1) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int v = 0; v < 16; ++v) comb[rw][16 * dt + v][lane] = acc[dt][v];
        comb[rw][64][lane] = M;
        comb[rw][65][lane] = S;
    }
    __syncthreads();
    if (!active || grp != 0) return;
    {
        const float M1 = comb[rw][64][lane];
        const float Mn = fmaxf(M, M1);
        const float a0 = M == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M - Mn);
        const float a1 = M1 == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(M1 - Mn);
        S = fmaf(comb[rw][65][lane], a1, S * a0);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[dt][v] = fmaf(comb[rw][16 * dt + v][lane], a1, acc[dt][v] * a0);
    }
    const float Ssum = sum_rows32(S);   // the two halves hold different tokens
    if (!live) return;
    float *o = p.out + ((size_t)(r0 + qi) * p.nq + kh * G + qg) * kHeadDim;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            // dims 32 dt + 8 q4 + 4 hf + e; one division at the end, per element
            const v16f_t &a = acc[dt];
            reinterpret_cast<float4 *>(o + 32 * dt + 8 * q4 + 4 * hf)[0] =
                Ssum > 0.0f ? make_float4(a[4 * q4] / Ssum, a[4 * q4 + 1] / Ssum, a[4 * q4 + 2] / Ssum,
                                          a[4 * q4 + 3] / Ssum)
                            : make_float4(0.f, 0.f, 0.f, 0.f);
        }
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
    const dim3 grid(batch.batch * layer.nkv_heads, (unsigned)((rows + kPfBlockRows - 1) / kPfBlockRows));
    void *args[] = {&p};
    const void *fn = layer.kv_bs >= kKeyTile ? reinterpret_cast<const void *>(&q8_prefill_kernel<true>)
                                             : reinterpret_cast<const void *>(&q8_prefill_kernel<false>);
    const hipError_t e = hipLaunchKernel(fn, grid, dim3(64 * kPfWaves), args, 0, stream);
    return e != hipSuccess ? e : hipGetLastError();
}

}  // namespace q8kv
