/*
 * q8kv.h -- C ABI of the MI355X (gfx950) q8 single-query decode-attention
 * library (libq8kv.so).
 *
 * What it computes (pages cited by title and section):
 *   - "9-3 q8 KV 精度对照实验" §2: every new (token, KV head) row of K and V is
 *     quantized on append with one fp32 scale per row (max-abs/127) and int8
 *     codes (round, clamp to +-127).
 *   - "9-2 flash_attn_single_q_q8_neon -- 单 q 单遍扫全 KV" §2: decode attention
 *     for one query per sequence and head, in one pass over that sequence's
 *     blocked int8 KV: Q quantized once in 32-element blocks (segment 1), int8
 *     dot products with int32 block sums rescaled by the Q block scale, the K
 *     row scale and the softmax scale, an online softmax with running max M and
 *     sum S that rescales the accumulator whenever M rises, V accumulated as
 *     int8 code times (weight x V row scale) (segment 2), and a single
 *     division by S at the end (segment 3).
 *
 * Data layout (device memory, owned by the caller; one pool per layer):
 *   k_codes, v_codes : int8  [num_blocks][kv_bs][nkv_heads * head_dim]
 *   k_scale, v_scale : fp32  [num_blocks][nkv_heads][kv_bs]
 *     Token t of sequence b lives in physical block block_table[b][t / kv_bs]
 *     at row t % kv_bs; head kh occupies bytes [kh*head_dim, (kh+1)*head_dim)
 *     of that row ("9-2" §2 segment 2), and its scale is element
 *     [block][kh][t % kv_bs] -- per block, one head's scales side by side.
 *     The scale stored for a row is the step d = max-abs * fl(1/127); a
 *     dequantized value is code * d.
 *   block_table : int32 [batch][max_blocks_per_seq] (physical block ids)
 *   seq_lens    : int32 [batch] (tokens visible to attention, including the
 *                 token appended this step)
 *   q, out      : fp32  [batch][nq_heads][head_dim]
 *   Query head h reads KV head h / (nq_heads / nkv_heads).
 *
 * Supported shapes: head_dim == 128; kv_bs a power of two in [8, 1024];
 * nkv_heads in [1, 16]; nq_heads / nkv_heads in {1, 2, 4, 8}; batch in
 * [1, 4096].  Everything else returns Q8_EUNSUPPORTED.
 *
 * Execution: every call only validates its host-visible arguments and
 * enqueues kernels on `stream` (a hipStream_t; NULL = the null stream).  No
 * call allocates device memory, synchronizes, or keeps state between calls,
 * so calls are re-entrant; calls that write the same buffers must be ordered
 * by the caller.  Inputs must be finite.
 *
 * Errors: host-detected errors return before anything is enqueued.  Errors
 * only the device can see (a sequence length outside [0, max_seq_len], a
 * block id outside [0, num_blocks), an append position outside its sequence)
 * OR a Q8_DEV_* bit into *dev_status (if non-NULL; the caller zeroes it and
 * reads it after synchronizing).  The affected work is skipped: an appended
 * row is not written; a sequence with a bad length reads as empty (its output
 * row is zeros); a block with a bad id is left out of the attention.
 */
#ifndef Q8KV_H
#define Q8KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q8KV_ABI_VERSION 7

typedef enum q8_status {
    Q8_OK = 0,
    Q8_EINVAL = -1,        /* NULL or misaligned pointer, negative or inconsistent size */
    Q8_EUNSUPPORTED = -2,  /* shape outside the supported set listed above */
    Q8_EWORKSPACE = -3,    /* workspace NULL or smaller than q8_decode_attn_workspace_bytes() */
    Q8_EHIP = -4           /* a HIP runtime call failed; q8_last_error() holds its text */
} q8_status;

/* Bits OR-ed into *dev_status by the device. */
#define Q8_DEV_BAD_SEQ_LEN  0x1  /* seq_lens[b] < 0 or > max_seq_len */
#define Q8_DEV_BAD_BLOCK_ID 0x2  /* block_table entry outside [0, num_blocks) */
#define Q8_DEV_BAD_TOKEN    0x4  /* append: tok_seq outside [0, batch) or tok_pos outside [0, seq_lens[seq]) */
#define Q8_DEV_BAD_PLAN     0x8  /* decode: batch->plan was not made by q8_decode_plan for this call's shape */

/* One layer's physical block pool (pointers to device memory).
 * Alignment: k_codes and v_codes 16 bytes, k_scale and v_scale 4 bytes.
 * k_f32, v_f32: the optional fp32 mirror ("9-3 q8 KV 精度对照实验" §3,
 * closing note: the write path also keeps every new K/V row in a float
 * cache, so quantized and exact attention coexist) -- both NULL, or both
 * fp32 [num_blocks][kv_bs][nkv_heads * head_dim] (the code layout with fp32
 * elements), 16-byte aligned. */
typedef struct q8_kv_layer {
    int32_t nkv_heads;
    int32_t head_dim;
    int32_t kv_bs;
    int32_t num_blocks;
    int8_t *k_codes;
    int8_t *v_codes;
    float *k_scale;
    float *v_scale;
    float *k_f32;
    float *v_f32;
} q8_kv_layer;

/* Per-step batch metadata, shared by all layers.  batch, max_blocks_per_seq
 * and max_seq_len are host values; the arrays are device memory.
 * max_seq_len must not exceed max_blocks_per_seq * kv_bs.
 * plan: NULL, or a step plan made by q8_decode_plan for these arrays (with
 * their current contents), the decode call's nq_heads and nparts and the
 * layer's nkv_heads and kv_bs (64-byte aligned device memory).  The decode
 * entry points (q8_decode_attn and its phases, q8_decode_step and its
 * partial, q8_decode_step_static, q8_decode_attn_f32 and its partial) then
 * read the cut from it instead of making it in every workgroup, with
 * bit-identical results; the other entry points ignore it.  A plan made for
 * another batch size, partition count, kv_bs or max_seq_len is detected on
 * the device (Q8_DEV_BAD_PLAN, no output written); one made before the
 * arrays changed is not -- make a new plan whenever they change.
 * flags: 0, or Q8_BATCH_INVARIANT: the decode entry points then cut every
 * sequence into chunks of Q8_INVARIANT_CHUNK_TOKENS positions counted from its
 * start (twice that for a sequence of 4096 positions or more, four times for
 * 16384 or more; the last chunk shorter), give every chunk its own partial
 * state and
 * combine a sequence's chunk states in chunk order with a fixed association
 * -- the online-softmax rescale rule of "9-2 flash_attn_single_q_q8_neon"
 * §2 segment 2 applied to partial states, one division at the end -- so a
 * sequence's output bits depend on nothing but its own length, K, V and q:
 * not on the other sequences of the batch, their order, the partition count
 * or the placement of its blocks.  Chunks are shared out over the ranges by
 * their first position, which balances the work less evenly than the default
 * cut.  The workspace holds up to batch * max(64, ceil(max_seq_len / 512))
 * records per query head.  Such a batch carries no step plan (Q8_EINVAL). */
#define Q8_BATCH_INVARIANT 0x1
#define Q8_INVARIANT_CHUNK_TOKENS 128
typedef struct q8_batch {
    int32_t batch;
    int32_t max_blocks_per_seq;
    int32_t max_seq_len;
    const int32_t *block_table;
    const int32_t *seq_lens;
    const void *plan;
    int32_t flags;
} q8_batch;

/* kv_quantize_per_head append ("9-3" §2; stored layout "9-2" §2 segment 2).
 * For each of n_tokens new tokens j and each KV head kh, quantizes the row
 * k_new[j][kh][0:head_dim] (and likewise v_new): a = max |x| (a := 1 when
 * a < 1e-6), d = a * fl(1/127), r = 127 / a (IEEE fp32 division),
 * code = clamp(roundf(x * r), -127, 127) with roundf rounding halves away
 * from zero; writes the codes and d at sequence tok_seq[j], position
 * tok_pos[j] of the cache.  tok_seq, tok_pos: device int32 [n_tokens];
 * k_new, v_new: device fp32 [n_tokens][nkv_heads][head_dim], 16-byte
 * aligned.  When the layer has an fp32 mirror, the rows are also written
 * there unchanged.  n_tokens == 0 is a no-op.  Positions must lie inside
 * [0, seq_lens[seq]); a decode step appends tok_pos = seq_lens - 1 and then
 * calls q8_decode_attn.  Two tokens with the same (seq, pos) race. */
q8_status q8_kv_append(const q8_kv_layer *layer, const q8_batch *batch,
                       int32_t n_tokens, const int32_t *tok_seq, const int32_t *tok_pos,
                       const float *k_new, const float *v_new,
                       int32_t *dev_status, void *stream);

/* Number of work partitions q8_decode_attn uses when asked for nparts = 0:
 * one per workgroup slot resident on the current device, capped at the
 * batch's largest possible tile count (tiles are 32 tokens). */
int32_t q8_decode_attn_auto_parts(const q8_kv_layer *layer, const q8_batch *batch,
                                  int32_t nq_heads);

/* Device workspace q8_decode_attn needs for this shape and partition count
 * (nparts = 0: the automatic count above).  Returns 0 on invalid arguments. */
size_t q8_decode_attn_workspace_bytes(const q8_kv_layer *layer, const q8_batch *batch,
                                      int32_t nq_heads, int32_t nparts);

/* The step plan (see q8_batch.plan): the cut of the batch into ranges and
 * pieces that every decode call of this step would otherwise make at the
 * start of every workgroup -- the length prefix, the ranges' pieces and the
 * block ids each piece starts with -- made once by one small kernel and
 * shared by all layers of the step.  The plan depends on the batch arrays'
 * contents, nq_heads (through the automatic partition count), nparts, and
 * the layer's nkv_heads and kv_bs; make it after the step's seq_lens and
 * block_table are final (after the appends' positions are counted in
 * seq_lens) and before the first decode of the step.  plan: device memory of
 * at least q8_decode_plan_bytes() bytes, 64-byte aligned; batch->plan is
 * ignored.  Bad lengths set Q8_DEV_BAD_SEQ_LEN here (the planned decode calls
 * then treat those sequences as empty without reporting again).  A batch with
 * Q8_BATCH_INVARIANT has no plan: Q8_EINVAL (and 0 bytes). */
size_t q8_decode_plan_bytes(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                            int32_t nparts);
q8_status q8_decode_plan(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads, int32_t nparts,
                         void *plan, size_t plan_bytes, int32_t *dev_status, void *stream);

/* Decode attention ("9-2" §2, all three segments) for every sequence b and
 * query head h of the batch:
 *   out[b][h] = sum_t softmax_t(s) * vhat_t,  s_t = scale * <qhat, khat_t>,
 * over t < seq_lens[b], where qhat, khat, vhat are the dequantized query
 * (32-blocks, see q8_quantize_q) and cache rows, computed in one pass with an
 * online softmax.  `scale` is the caller's softmax scale (1/sqrt(head_dim) in
 * the pages).  The batch's 32-token tiles, with two extra units of cost in
 * front of every non-empty sequence after the first (the cost of starting a
 * piece), are cut into `nparts` equal contiguous ranges (nparts = 0:
 * automatic), one workgroup each; a sequence
 * cut across ranges is finished by a merge of the partial (M, S, acc) states
 * with the same rescale rule ("9-2" §2 segment 2 applied to whole partial
 * states).  A sequence of length 0 gives a zero row.  Results are
 * deterministic for a given nparts.  workspace: device memory of at least
 * q8_decode_attn_workspace_bytes(..., nparts) bytes, 256-byte aligned, no
 * initialization needed; it must not be shared by calls that may overlap. */
q8_status q8_decode_attn(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                         const float *q, float scale, float *out, int32_t nparts,
                         void *workspace, size_t workspace_bytes,
                         int32_t *dev_status, void *stream);

/* The two kernels q8_decode_attn enqueues, exposed so a caller can time them
 * or interleave other work; calling _partial then _merge with identical
 * arguments is exactly q8_decode_attn.  _merge is a no-op when the resolved
 * nparts is 1. */
q8_status q8_decode_attn_partial(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                                 const float *q, float scale, float *out, int32_t nparts,
                                 void *workspace, size_t workspace_bytes,
                                 int32_t *dev_status, void *stream);
q8_status q8_decode_attn_merge(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                               const float *q, float scale, float *out, int32_t nparts,
                               void *workspace, size_t workspace_bytes,
                               int32_t *dev_status, void *stream);

/* One decode step of a layer in one call: exactly q8_kv_append of the
 * token at position seq_lens[b] - 1 of every sequence b with seq_lens[b] >= 1
 * (K/V rows k_new[b], v_new[b]: device fp32 [batch][nkv_heads][head_dim],
 * 8-byte aligned; the fp32 mirror too, if the layer has one), followed by
 * q8_decode_attn with the same arguments ("9-3" §2 append, "9-2" §2
 * attention).  The append is done inside the decode's partial kernel by the
 * workgroup that reads that token's tile, so the step needs no separate
 * append launch; the codes and steps written are bit-identical to
 * q8_kv_append's and the outputs to q8_decode_attn's.  A bad block id for
 * position seq_lens[b] - 1 sets Q8_DEV_BAD_BLOCK_ID and the row is not
 * written.  Workspace, nparts and errors as q8_decode_attn. */
q8_status q8_decode_step(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                         const float *k_new, const float *v_new, const float *q, float scale, float *out,
                         int32_t nparts, void *workspace, size_t workspace_bytes,
                         int32_t *dev_status, void *stream);

/* The step's first launch alone (append + cache walk): _step_partial
 * followed by q8_decode_attn_merge with the same layer, batch, heads, q,
 * scale, out, nparts and workspace is exactly q8_decode_step. */
q8_status q8_decode_step_partial(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                                 const float *k_new, const float *v_new, const float *q, float scale,
                                 float *out, int32_t nparts, void *workspace, size_t workspace_bytes,
                                 int32_t *dev_status, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): exactly
 * q8_decode_step -- same kernels, results bit-identical for the same nparts
 * -- with no workspace argument.  The partial records live in a device
 * array of the library (q8_decode_step_static_scratch_bytes() = 16 MiB on
 * every GPU it runs on, held until the process ends); nothing is allocated,
 * freed or initialized by the call, and the array needs no clearing (every
 * byte a call reads it has written first in the same call).  The first call
 * on a device looks up the array's device address (hipGetSymbolAddress);
 * make one call outside graph capture before capturing.  Every call on one
 * GPU uses the same array: calls that may overlap on a GPU (different
 * streams without ordering) race and must be ordered by the caller.
 * Q8_EWORKSPACE if the plan for this shape and nparts needs more than the
 * array holds (with nparts = 0 on an MI355X: up to 32 query heads); other
 * errors as q8_decode_step. */
size_t q8_decode_step_static_scratch_bytes(void);
q8_status q8_decode_step_static(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                                const float *k_new, const float *v_new, const float *q, float scale, float *out,
                                int32_t nparts, int32_t *dev_status, void *stream);

/* Exact decode attention over the layer's fp32 mirror ("9-3" §1: scores of
 * the raw fp32 q and K, max-subtracted softmax, weighted raw V), for every
 * sequence b and query head h:
 *   out[b][h] = sum_t softmax_t(s) * v_t,  s_t = scale * <q, k_t>,
 * in fp32 with an online softmax, over t < seq_lens[b].  Same batch, head
 * map, range cut, merge, workspace (q8_decode_attn_workspace_bytes), length-0
 * and error behaviour as q8_decode_attn.  Q8_EINVAL if the layer has no
 * fp32 mirror. */
q8_status q8_decode_attn_f32(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                             const float *q, float scale, float *out, int32_t nparts,
                             void *workspace, size_t workspace_bytes,
                             int32_t *dev_status, void *stream);

/* The exact decode's cache walk alone: _f32_partial followed by
 * q8_decode_attn_merge with identical arguments is exactly
 * q8_decode_attn_f32 (both paths leave the same partial-state records). */
q8_status q8_decode_attn_f32_partial(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                                     const float *q, float scale, float *out, int32_t nparts,
                                     void *workspace, size_t workspace_bytes,
                                     int32_t *dev_status, void *stream);

/* Block-sparse decode ("why long context must be sparse" §1-§2): per
 * sequence b and query head h, the history is cut into 32-token blocks; each
 * block is probed at its rows 0, 4, ..., 28 and scored by the largest q8
 * attention score among them ("9-2" §2 segment 2: s = (sum over 32-blocks of
 * P_b * qscale_b) * kscale * scale, evaluated in fp32 with each product and
 * sum rounded on its own, within about 5 * 2^-24 * scale * kscale *
 * sum_b |P_b * qscale_b| of the exact value); the `topk`
 * highest-scoring blocks (ties: lower block index) are kept, and out[b][h]
 * is the exact q8 single-pass attention ("9-2" §2) over the tokens of those
 * blocks.  A sequence of at most topk blocks keeps every block (the result
 * is then the full attention of q8_decode_attn up to rounding order).
 * topk in [2, 64] (the pages' default is 32).  selected: NULL, or device
 * int32 [batch][nq_heads][topk] receiving the kept block indices in
 * ascending order, -1 after the last.  workspace: at least
 * q8_decode_attn_sparse_workspace_bytes() bytes, 256-byte aligned, any
 * contents.  Errors as q8_decode_attn. */
size_t q8_decode_attn_sparse_workspace_bytes(const q8_kv_layer *layer, const q8_batch *batch,
                                             int32_t nq_heads, int32_t topk);
q8_status q8_decode_attn_sparse(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                                const float *q, float scale, float *out, int32_t topk,
                                int32_t *selected, void *workspace, size_t workspace_bytes,
                                int32_t *dev_status, void *stream);

/* Batched prefill attention over the q8 cache ("why long context must be
 * sparse" §1-§2: the exact batched path; a batch of new tokens scores against
 * the whole history).  For each sequence b, its nb_b = q_start[b + 1] -
 * q_start[b] new tokens are the last nb_b positions of its cache (appended
 * with q8_kv_append before this call, so seq_lens[b] counts them).  Query row
 * r, q_start[b] <= r < q_start[b + 1], sits at position
 *     p = seq_lens[b] - nb_b + (r - q_start[b])
 * and attends causally to positions 0..p: for every query head h,
 *     out[r][h] = the q8 single-pass attention ("9-2" §2) of q[r][h] over
 *                 tokens 0..p of KV head h / (nq_heads / nkv_heads),
 * with the decode's Q quantizer, scores, softmax and one final division
 * (products on the matrix cores; the value products are exact, only the fp32
 * summation order differs from q8_decode_attn over the same tokens).
 *   q_start : device int32 [batch + 1], q_start[0] = 0, nondecreasing,
 *             q_start[batch] = total_q;
 *   q, out  : device fp32 [total_q][nq_heads][head_dim], 16-byte aligned;
 *   max_new : host bound on every nb_b (sizes the launch), in [0, max_seq_len].
 * Device-detected: a sequence with q_start out of order or outside
 * [0, total_q], nb_b > seq_lens[b], nb_b > max_new, or seq_lens[b] outside
 * [0, max_seq_len] sets Q8_DEV_BAD_SEQ_LEN and its rows (when its q_start
 * range is inside [0, total_q], up to max_new of them) are zeros; a bad block
 * id sets Q8_DEV_BAD_BLOCK_ID and its tokens are left out.  No workspace;
 * nothing allocated; total_q == 0 or max_new == 0 enqueues nothing. */
q8_status q8_prefill_attn(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                          const int32_t *q_start, int32_t total_q, int32_t max_new,
                          const float *q, float scale, float *out, int32_t *dev_status, void *stream);

/* Test hook: the Q quantizer of the decode kernel ("9-2" §2 segment 1) on
 * `rows` rows of head_dim (== 128) values: per 32-block, m = max |q| (m := 1
 * when m < 1e-6), qscale = m * fl(1/127), r = 127 / m,
 * code = (int8) truncation toward zero of clamp(q * r, -128, 127).
 * path selects which of the decode's two device routines runs (they compute
 * the same codes in different lane layouts):
 *   Q8_QPATH_VALU -- two lanes per 32-block; q8_decode_attn and
 *                    q8_decode_step use it unless nq/nkv == 4 with
 *                    kv_bs >= 32, and so does the sparse attention;
 *   Q8_QPATH_MFMA -- one lane per 32-block, four rows per wave (the A-operand
 *                    layout of the i8 matrix-core scores); the decode uses it
 *                    at nq/nkv == 4 with kv_bs >= 32, and the sparse probe.
 * q: device fp32 [rows][head_dim] (16-byte aligned); codes: device int8
 * [rows][head_dim]; qscale: device fp32 [rows][head_dim / 32].  Q8_EINVAL
 * for an unknown path. */
#define Q8_QPATH_VALU 0
#define Q8_QPATH_MFMA 1
q8_status q8_quantize_q(const float *q, int32_t rows, int32_t head_dim, int32_t path,
                        int8_t *codes, float *qscale, void *stream);

/* Test hook: the exact int32 block sums the decode kernel forms ("9-2" §2
 * segment 2), P[b][h][t][blk] = sum over i in block blk of qcode[i] *
 * kcode_t[i], for every sequence b, query head h and t < seq_lens[b];
 * entries with seq_lens[b] <= t < max_seq_len are written as 0.
 * partials: device int32 [batch][nq_heads][max_seq_len][head_dim / 32],
 * 16-byte aligned.  qcodes, qscale: both NULL, or device int8
 * [batch][nq_heads][head_dim] (16-byte aligned) and fp32
 * [batch][nq_heads][head_dim / 32] receiving the query codes and scales the
 * partials were formed with.  Runs the device routines and operand layout
 * q8_decode_attn uses for this shape: the i8 matrix cores
 * (v_mfma_i32_16x16x64_i8, query quantized one lane per 32-block) at
 * nq/nkv == 4 with kv_bs >= 32, else sdot4 with the query quantized two
 * lanes per 32-block. */
q8_status q8_qk_block_partials(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                               const float *q, int32_t *partials, int8_t *qcodes, float *qscale,
                               int32_t *dev_status, void *stream);

/* Measurement hook: reads `bytes` (a multiple of 16) of device memory at buf
 * (16-byte aligned) exactly once with 16-byte loads -- the buffer split
 * evenly over `workgroups` workgroups of 512 lanes, four loads in flight per
 * lane, plain (nontemporal = 0) or non-temporal (1, the hint the decode's
 * cache loads carry) -- and writes *sink (device uint32) only if a value
 * folded from all loads equals a fixed constant.  The time it takes is the
 * read ceiling the decode kernel is measured against: the decode must read
 * every byte of the cache once ("why long context must be sparse" §1).
 * bytes == 0 is a no-op; workgroups in [1, 65536]. */
q8_status q8_stream_read(const void *buf, size_t bytes, int32_t workgroups, int32_t nontemporal,
                         uint32_t *sink, void *stream);

/* Measurement hook: instruction issue on the matrix cores and the VALU.  Each
 * of `workgroups` workgroups (512 lanes; 1024 in mode 4) runs, in waves 0-3,
 * eight independent fp32 FMA chains for valu_iters rounds (8 FMAs per round)
 * and, in waves 4-7, four independent v_mfma_f32_32x32x16_bf16 chains for
 * mfma_iters rounds (4 products per round); waves w and w + 4 share a SIMD.
 * mode 0: VALU waves only (one per SIMD); 1: matrix-core waves only; 2: both;
 * 3: all eight waves VALU (two per SIMD); 4: sixteen VALU waves (four per
 * SIMD).  The times of the modes show the VALU rate one wave reaches, the
 * rate several waves reach, and whether a SIMD overlaps one wave's
 * matrix-core products with another wave's VALU -- what bounds the batched
 * prefill, whose waves alternate between the two.  out: device fp32 scratch
 * of workgroups * 1024 elements (4-byte aligned; written, values
 * meaningless).  mode in [0, 4], iteration counts in [1, 2^20], workgroups
 * in [1, 65536]. */
q8_status q8_issue_probe(float *out, int32_t mode, int32_t valu_iters, int32_t mfma_iters, int32_t workgroups,
                         void *stream);

/* Short English name of a status code (static string). */
const char *q8_status_string(int32_t status);
/* Text of the last Q8_EHIP error on the calling thread ("" if none). */
const char *q8_last_error(void);
/* Q8KV_ABI_VERSION of the loaded library. */
int32_t q8_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* Q8KV_H */
