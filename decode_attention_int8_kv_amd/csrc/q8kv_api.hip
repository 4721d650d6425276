// q8kv_api.hip -- the extern "C" entry points declared in include/q8kv.h:
// argument validation, launch planning and error reporting.  No entry point
// allocates device memory or synchronizes; all kernels go on the caller's
// stream.
#include <stdio.h>

#include <string>

#include "q8kv_device.hpp"
#include "q8kv_internal.hpp"

namespace {

thread_local std::string g_last_error;

q8_status hip_fail(hipError_t e, const char *where)
{
    g_last_error = std::string(where) + ": " + hipGetErrorName(e) + " (" + hipGetErrorString(e) + ")";
    return Q8_EHIP;
}

bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

q8_status check_layer(const q8_kv_layer *l)
{
    if (!l) return Q8_EINVAL;
    if (l->head_dim != q8kv::kHeadDim) return Q8_EUNSUPPORTED;
    if (l->nkv_heads < 1 || l->nkv_heads > 16) return Q8_EUNSUPPORTED;
    if (!is_pow2(l->kv_bs) || l->kv_bs < 8 || l->kv_bs > 1024) return Q8_EUNSUPPORTED;
    if (l->num_blocks < 1) return Q8_EINVAL;
    if ((long long)l->num_blocks * l->kv_bs * l->nkv_heads * q8kv::kHeadDim > (1LL << 47)) return Q8_EINVAL;
    if (!l->k_codes || !l->v_codes || !l->k_scale || !l->v_scale) return Q8_EINVAL;
    if (!aligned(l->k_codes, 16) || !aligned(l->v_codes, 16)) return Q8_EINVAL;
    if (!aligned(l->k_scale, 4) || !aligned(l->v_scale, 4)) return Q8_EINVAL;
    // the fp32 mirror is optional, but all or nothing
    if (!l->k_f32 != !l->v_f32) return Q8_EINVAL;
    if (l->k_f32 && (!aligned(l->k_f32, 16) || !aligned(l->v_f32, 16))) return Q8_EINVAL;
    return Q8_OK;
}

q8_status check_batch(const q8_batch *b, const q8_kv_layer *l)
{
    if (!b) return Q8_EINVAL;
    if (b->batch < 1) return Q8_EINVAL;
    if (b->batch > q8kv::kMaxBatch) return Q8_EUNSUPPORTED;
    if (b->max_blocks_per_seq < 1 || b->max_seq_len < 0) return Q8_EINVAL;
    if ((long long)b->max_seq_len > (long long)b->max_blocks_per_seq * l->kv_bs) return Q8_EINVAL;
    // the batch's cut-axis units (tiles plus the units charged per sequence) must fit int32
    if ((long long)b->batch * ((b->max_seq_len + q8kv::kTile - 1) / q8kv::kTile + q8kv::kPieceCost) > 0x7fffffffLL)
        return Q8_EUNSUPPORTED;
    if (!b->block_table || !b->seq_lens) return Q8_EINVAL;
    if (!aligned(b->block_table, 4) || !aligned(b->seq_lens, 4)) return Q8_EINVAL;
    if (b->plan && !aligned(b->plan, 64)) return Q8_EINVAL;
    if (b->flags & ~Q8_BATCH_INVARIANT) return Q8_EINVAL;
    if ((b->flags & Q8_BATCH_INVARIANT) && b->plan) return Q8_EINVAL;   // an invariant batch is not planned
    return Q8_OK;
}

q8_status check_heads(const q8_kv_layer *l, int32_t nq)
{
    if (nq < 1 || nq % l->nkv_heads) return Q8_EINVAL;
    const int g = nq / l->nkv_heads;
    if (g != 1 && g != 2 && g != 4 && g != 8) return Q8_EUNSUPPORTED;
    return Q8_OK;
}

q8_status check_decode(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq, const float *q,
                       float *out, int32_t nparts, void *workspace, size_t workspace_bytes,
                       q8kv::DecodePlan *plan)
{
    q8_status s;
    if ((s = check_layer(layer)) != Q8_OK) return s;
    if ((s = check_batch(batch, layer)) != Q8_OK) return s;
    if ((s = check_heads(layer, nq)) != Q8_OK) return s;
    if (!q || !out || !aligned(q, 16) || !aligned(out, 16)) return Q8_EINVAL;
    if (nparts < 0) return Q8_EINVAL;
    *plan = q8kv::make_plan(*layer, *batch, nq, nparts);
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < plan->bytes) return Q8_EWORKSPACE;
    return Q8_OK;
}

}  // namespace

extern "C" {

q8_status q8_kv_append(const q8_kv_layer *layer, const q8_batch *batch, int32_t n_tokens,
                       const int32_t *tok_seq, const int32_t *tok_pos, const float *k_new,
                       const float *v_new, int32_t *dev_status, void *stream)
{
    q8_status s;
    if ((s = check_layer(layer)) != Q8_OK) return s;
    if ((s = check_batch(batch, layer)) != Q8_OK) return s;
    if (n_tokens < 0 || (long long)n_tokens * layer->nkv_heads > 0x7fffffffLL) return Q8_EINVAL;
    if (n_tokens == 0) return Q8_OK;
    if (!tok_seq || !tok_pos || !k_new || !v_new) return Q8_EINVAL;
    if (!aligned(tok_seq, 4) || !aligned(tok_pos, 4) || !aligned(k_new, 16) || !aligned(v_new, 16))
        return Q8_EINVAL;
    if (dev_status && !aligned(dev_status, 4)) return Q8_EINVAL;
    hipError_t e = q8kv::launch_append(*layer, *batch, n_tokens, tok_seq, tok_pos, k_new, v_new,
                                       dev_status, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8_OK : hip_fail(e, "q8_kv_append");
}

int32_t q8_decode_attn_auto_parts(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads)
{
    if (check_layer(layer) != Q8_OK || check_batch(batch, layer) != Q8_OK ||
        check_heads(layer, nq_heads) != Q8_OK)
        return 0;
    return q8kv::auto_parts(*layer, *batch, nq_heads);
}

size_t q8_decode_attn_workspace_bytes(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                                      int32_t nparts)
{
    if (check_layer(layer) != Q8_OK || check_batch(batch, layer) != Q8_OK ||
        check_heads(layer, nq_heads) != Q8_OK || nparts < 0)
        return 0;
    return q8kv::make_plan(*layer, *batch, nq_heads, nparts).bytes;
}

size_t q8_decode_plan_bytes(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads, int32_t nparts)
{
    if (check_layer(layer) != Q8_OK || check_batch(batch, layer) != Q8_OK ||
        check_heads(layer, nq_heads) != Q8_OK || nparts < 0 || (batch->flags & Q8_BATCH_INVARIANT))
        return 0;
    return q8kv::step_plan_bytes(*batch, q8kv::make_plan(*layer, *batch, nq_heads, nparts).nparts);
}

q8_status q8_decode_plan(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads, int32_t nparts,
                         void *plan, size_t plan_bytes, int32_t *dev_status, void *stream)
{
    q8_status s;
    if ((s = check_layer(layer)) != Q8_OK) return s;
    if ((s = check_batch(batch, layer)) != Q8_OK) return s;
    if ((s = check_heads(layer, nq_heads)) != Q8_OK) return s;
    if (nparts < 0 || (batch->flags & Q8_BATCH_INVARIANT)) return Q8_EINVAL;
    if (dev_status && !aligned(dev_status, 4)) return Q8_EINVAL;
    const q8kv::DecodePlan pl = q8kv::make_plan(*layer, *batch, nq_heads, nparts);
    const size_t need = q8kv::step_plan_bytes(*batch, pl.nparts);
    if (need > (size_t)0x7fffffff * 4) return Q8_EUNSUPPORTED;   // word offsets stay in int32 range
    if (!plan || !aligned(plan, 64) || plan_bytes < need) return Q8_EWORKSPACE;
    hipError_t e = q8kv::launch_step_plan(*layer, *batch, nq_heads, pl, plan, dev_status,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8_OK : hip_fail(e, "q8_decode_plan");
}

q8_status q8_decode_attn_partial(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                                 const float *q, float scale, float *out, int32_t nparts,
                                 void *workspace, size_t workspace_bytes, int32_t *dev_status,
                                 void *stream)
{
    q8kv::DecodePlan plan;
    q8_status s = check_decode(layer, batch, nq_heads, q, out, nparts, workspace, workspace_bytes, &plan);
    if (s != Q8_OK) return s;
    if (dev_status && !aligned(dev_status, 4)) return Q8_EINVAL;
    hipError_t e = q8kv::launch_decode_partial(*layer, *batch, nq_heads, q, scale, out, plan, workspace,
                                               dev_status, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8_OK : hip_fail(e, "q8_decode_attn_partial");
}

q8_status q8_decode_attn_merge(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                               const float *q, float scale, float *out, int32_t nparts,
                               void *workspace, size_t workspace_bytes, int32_t *dev_status,
                               void *stream)
{
    (void)scale;
    q8kv::DecodePlan plan;
    q8_status s = check_decode(layer, batch, nq_heads, q, out, nparts, workspace, workspace_bytes, &plan);
    if (s != Q8_OK) return s;
    if (dev_status && !aligned(dev_status, 4)) return Q8_EINVAL;
    hipError_t e = q8kv::launch_decode_merge(*layer, *batch, nq_heads, out, plan, workspace,
                                             static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8_OK : hip_fail(e, "q8_decode_attn_merge");
}

q8_status q8_decode_attn(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                         const float *q, float scale, float *out, int32_t nparts, void *workspace,
                         size_t workspace_bytes, int32_t *dev_status, void *stream)
{
    q8_status s = q8_decode_attn_partial(layer, batch, nq_heads, q, scale, out, nparts, workspace,
                                         workspace_bytes, dev_status, stream);
    if (s != Q8_OK) return s;
    return q8_decode_attn_merge(layer, batch, nq_heads, q, scale, out, nparts, workspace,
                                workspace_bytes, dev_status, stream);
}

q8_status q8_decode_step_partial(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                                 const float *k_new, const float *v_new, const float *q, float scale,
                                 float *out, int32_t nparts, void *workspace, size_t workspace_bytes,
                                 int32_t *dev_status, void *stream)
{
    q8kv::DecodePlan plan;
    q8_status s = check_decode(layer, batch, nq_heads, q, out, nparts, workspace, workspace_bytes, &plan);
    if (s != Q8_OK) return s;
    if (!k_new || !v_new || !aligned(k_new, 8) || !aligned(v_new, 8)) return Q8_EINVAL;
    if (dev_status && !aligned(dev_status, 4)) return Q8_EINVAL;
    hipError_t e = q8kv::launch_decode_partial(*layer, *batch, nq_heads, q, scale, out, plan, workspace, dev_status,
                                               static_cast<hipStream_t>(stream), k_new, v_new);
    return e == hipSuccess ? Q8_OK : hip_fail(e, "q8_decode_step_partial");
}

q8_status q8_decode_step(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads, const float *k_new,
                         const float *v_new, const float *q, float scale, float *out, int32_t nparts,
                         void *workspace, size_t workspace_bytes, int32_t *dev_status, void *stream)
{
    q8_status s = q8_decode_step_partial(layer, batch, nq_heads, k_new, v_new, q, scale, out, nparts, workspace,
                                         workspace_bytes, dev_status, stream);
    if (s != Q8_OK) return s;
    return q8_decode_attn_merge(layer, batch, nq_heads, q, scale, out, nparts, workspace, workspace_bytes,
                                dev_status, stream);
}

q8_status q8_decode_step_static(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                                const float *k_new, const float *v_new, const float *q, float scale, float *out,
                                int32_t nparts, int32_t *dev_status, void *stream)
{
    q8_status s;
    if ((s = check_layer(layer)) != Q8_OK) return s;
    if ((s = check_batch(batch, layer)) != Q8_OK) return s;
    if ((s = check_heads(layer, nq_heads)) != Q8_OK) return s;
    if (!q || !out || !aligned(q, 16) || !aligned(out, 16)) return Q8_EINVAL;
    if (!k_new || !v_new || !aligned(k_new, 8) || !aligned(v_new, 8)) return Q8_EINVAL;
    if (dev_status && !aligned(dev_status, 4)) return Q8_EINVAL;
    if (nparts < 0) return Q8_EINVAL;
    const q8kv::DecodePlan plan = q8kv::make_plan(*layer, *batch, nq_heads, nparts);
    if (plan.bytes > q8kv::static_scratch_bytes()) return Q8_EWORKSPACE;
    void *ws = nullptr;
    hipError_t e = q8kv::static_scratch(&ws);
    if (e != hipSuccess) return hip_fail(e, "q8_decode_step_static (scratch address)");
    const hipStream_t st = static_cast<hipStream_t>(stream);
    e = q8kv::launch_decode_partial(*layer, *batch, nq_heads, q, scale, out, plan, ws, dev_status, st, k_new, v_new);
    if (e != hipSuccess) return hip_fail(e, "q8_decode_step_static");
    e = q8kv::launch_decode_merge(*layer, *batch, nq_heads, out, plan, ws, st);
    return e == hipSuccess ? Q8_OK : hip_fail(e, "q8_decode_step_static");
}

size_t q8_decode_step_static_scratch_bytes(void) { return q8kv::static_scratch_bytes(); }

q8_status q8_decode_attn_f32_partial(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                                     const float *q, float scale, float *out, int32_t nparts,
                                     void *workspace, size_t workspace_bytes, int32_t *dev_status,
                                     void *stream)
{
    q8kv::DecodePlan plan;
    q8_status s = check_decode(layer, batch, nq_heads, q, out, nparts, workspace, workspace_bytes, &plan);
    if (s != Q8_OK) return s;
    if (!layer->k_f32) return Q8_EINVAL;
    if (dev_status && !aligned(dev_status, 4)) return Q8_EINVAL;
    hipError_t e = q8kv::launch_decode_partial_f32(*layer, *batch, nq_heads, q, scale, out, plan, workspace,
                                                   dev_status, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8_OK : hip_fail(e, "q8_decode_attn_f32_partial");
}

q8_status q8_decode_attn_f32(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                             const float *q, float scale, float *out, int32_t nparts, void *workspace,
                             size_t workspace_bytes, int32_t *dev_status, void *stream)
{
    q8_status s = q8_decode_attn_f32_partial(layer, batch, nq_heads, q, scale, out, nparts, workspace,
                                             workspace_bytes, dev_status, stream);
    if (s != Q8_OK) return s;
    return q8_decode_attn_merge(layer, batch, nq_heads, q, scale, out, nparts, workspace, workspace_bytes,
                                dev_status, stream);
}

size_t q8_decode_attn_sparse_workspace_bytes(const q8_kv_layer *layer, const q8_batch *batch,
                                             int32_t nq_heads, int32_t topk)
{
    if (check_layer(layer) != Q8_OK || check_batch(batch, layer) != Q8_OK ||
        check_heads(layer, nq_heads) != Q8_OK || topk < 2 || topk > 64)
        return 0;
    return q8kv::sparse_workspace_bytes(*batch, nq_heads);
}

q8_status q8_decode_attn_sparse(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                                const float *q, float scale, float *out, int32_t topk, int32_t *selected,
                                void *workspace, size_t workspace_bytes, int32_t *dev_status, void *stream)
{
    q8_status s;
    if ((s = check_layer(layer)) != Q8_OK) return s;
    if ((s = check_batch(batch, layer)) != Q8_OK) return s;
    if ((s = check_heads(layer, nq_heads)) != Q8_OK) return s;
    if (topk < 2 || topk > 64) return Q8_EINVAL;
    if (!q || !out || !aligned(q, 16) || !aligned(out, 16)) return Q8_EINVAL;
    if (selected && !aligned(selected, 4)) return Q8_EINVAL;
    if (dev_status && !aligned(dev_status, 4)) return Q8_EINVAL;
    if ((long long)batch->batch * nq_heads > 0x7fffffffLL) return Q8_EUNSUPPORTED;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < q8kv::sparse_workspace_bytes(*batch, nq_heads))
        return Q8_EWORKSPACE;
    hipError_t e = q8kv::launch_sparse(*layer, *batch, nq_heads, q, scale, out, topk, selected, workspace,
                                       dev_status, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8_OK : hip_fail(e, "q8_decode_attn_sparse");
}

q8_status q8_prefill_attn(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                          const int32_t *q_start, int32_t total_q, int32_t max_new, const float *q, float scale,
                          float *out, int32_t *dev_status, void *stream)
{
    q8_status s;
    if ((s = check_layer(layer)) != Q8_OK) return s;
    if ((s = check_batch(batch, layer)) != Q8_OK) return s;
    if ((s = check_heads(layer, nq_heads)) != Q8_OK) return s;
    if (total_q < 0 || max_new < 0 || max_new > batch->max_seq_len) return Q8_EINVAL;
    if (!q_start || !aligned(q_start, 4)) return Q8_EINVAL;
    if (dev_status && !aligned(dev_status, 4)) return Q8_EINVAL;
    if (total_q == 0 || max_new == 0) return Q8_OK;
    if (!q || !out || !aligned(q, 16) || !aligned(out, 16)) return Q8_EINVAL;
    if ((long long)total_q * nq_heads * q8kv::kHeadDim > (1LL << 40)) return Q8_EUNSUPPORTED;
    // launch rows: max_new * G per (sequence, KV head), 64 per workgroup, grid y <= 65535
    if (((long long)max_new * (nq_heads / layer->nkv_heads) + 63) / 64 > 65535) return Q8_EUNSUPPORTED;
    hipError_t e = q8kv::launch_prefill(*layer, *batch, nq_heads, q_start, total_q, max_new, q, scale, out,
                                        dev_status, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8_OK : hip_fail(e, "q8_prefill_attn");
}

q8_status q8_quantize_q(const float *q, int32_t rows, int32_t head_dim, int32_t path, int8_t *codes,
                        float *qscale, void *stream)
{
    if (head_dim != q8kv::kHeadDim) return Q8_EUNSUPPORTED;
    if (rows < 0 || (path != Q8_QPATH_VALU && path != Q8_QPATH_MFMA)) return Q8_EINVAL;
    if (rows == 0) return Q8_OK;
    if (!q || !codes || !qscale || !aligned(q, 16) || !aligned(codes, 16) || !aligned(qscale, 4))
        return Q8_EINVAL;
    if ((long long)rows > 0x7fffffffLL / 4) return Q8_EUNSUPPORTED;
    hipError_t e = q8kv::launch_quantize_q(q, rows, path, codes, qscale, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8_OK : hip_fail(e, "q8_quantize_q");
}

q8_status q8_qk_block_partials(const q8_kv_layer *layer, const q8_batch *batch, int32_t nq_heads,
                               const float *q, int32_t *partials, int8_t *qcodes, float *qscale,
                               int32_t *dev_status, void *stream)
{
    q8_status s;
    if ((s = check_layer(layer)) != Q8_OK) return s;
    if ((s = check_batch(batch, layer)) != Q8_OK) return s;
    if ((s = check_heads(layer, nq_heads)) != Q8_OK) return s;
    if (!q || !partials || !aligned(q, 16) || !aligned(partials, 16)) return Q8_EINVAL;
    if (!qcodes != !qscale) return Q8_EINVAL;
    if (qcodes && (!aligned(qcodes, 16) || !aligned(qscale, 4))) return Q8_EINVAL;
    if (dev_status && !aligned(dev_status, 4)) return Q8_EINVAL;
    if ((batch->max_seq_len + q8kv::kTile - 1) / q8kv::kTile > 65535) return Q8_EUNSUPPORTED;
    if ((long long)batch->batch * layer->nkv_heads > 0x7fffffffLL) return Q8_EUNSUPPORTED;
    hipError_t e = q8kv::launch_qk_partials(*layer, *batch, nq_heads, q, partials, qcodes, qscale, dev_status,
                                            static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8_OK : hip_fail(e, "q8_qk_block_partials");
}

q8_status q8_stream_read(const void *buf, size_t bytes, int32_t workgroups, int32_t nontemporal, uint32_t *sink,
                         void *stream)
{
    if (bytes == 0) return Q8_OK;
    if (!buf || !sink || !aligned(buf, 16) || !aligned(sink, 4) || bytes % 16) return Q8_EINVAL;
    if (workgroups < 1 || workgroups > 65536 || (nontemporal != 0 && nontemporal != 1)) return Q8_EINVAL;
    hipError_t e = q8kv::launch_stream_read(buf, bytes, workgroups, nontemporal, sink,
                                            static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8_OK : hip_fail(e, "q8_stream_read");
}

q8_status q8_issue_probe(float *out, int32_t mode, int32_t valu_iters, int32_t mfma_iters, int32_t workgroups,
                         void *stream)
{
    if (!out || !aligned(out, 4) || mode < 0 || mode > 4) return Q8_EINVAL;
    if (valu_iters < 1 || valu_iters > (1 << 20) || mfma_iters < 1 || mfma_iters > (1 << 20)) return Q8_EINVAL;
    if (workgroups < 1 || workgroups > 65536) return Q8_EINVAL;
    hipError_t e = q8kv::launch_issue_probe(out, mode, valu_iters, mfma_iters, workgroups,
                                            static_cast<hipStream_t>(stream));
    return e == hipSuccess ? Q8_OK : hip_fail(e, "q8_issue_probe");
}

const char *q8_status_string(int32_t status)
{
    switch (status) {
    case Q8_OK: return "ok";
    case Q8_EINVAL: return "invalid argument";
    case Q8_EUNSUPPORTED: return "unsupported shape";
    case Q8_EWORKSPACE: return "workspace missing or too small";
    case Q8_EHIP: return "HIP runtime error";
    default: return "unknown status";
    }
}

const char *q8_last_error(void) { return g_last_error.c_str(); }

int32_t q8_abi_version(void) { return Q8KV_ABI_VERSION; }

}  // extern "C"
