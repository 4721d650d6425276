// q8kv_internal.hpp -- launchers shared between the kernel translation units
// and the C-ABI layer (not part of the public interface).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "q8kv.h"
#include "q8kv_plan.hpp"

namespace q8kv {

inline int ilog2(int v)
{
    int r = 0;
    while ((1 << (r + 1)) <= v) ++r;
    return r;
}

hipError_t launch_append(const q8_kv_layer &layer, const q8_batch &batch, int32_t n_tokens,
                         const int32_t *tok_seq, const int32_t *tok_pos, const float *k_new,
                         const float *v_new, int32_t *dev_status, hipStream_t stream);

// k_new / v_new (or null): the token at position seq_lens[b] - 1 of every
// sequence, appended by the partial kernel before it reads the cache.
hipError_t launch_decode_partial(const q8_kv_layer &layer, const q8_batch &batch, int nq,
                                 const float *q, float scale, float *out, const DecodePlan &plan,
                                 void *workspace, int32_t *dev_status, hipStream_t stream,
                                 const float *k_new = nullptr, const float *v_new = nullptr);

hipError_t launch_decode_partial_f32(const q8_kv_layer &layer, const q8_batch &batch, int nq,
                                     const float *q, float scale, float *out, const DecodePlan &plan,
                                     void *workspace, int32_t *dev_status, hipStream_t stream);

size_t sparse_workspace_bytes(const q8_batch &batch, int nq);
hipError_t launch_sparse(const q8_kv_layer &layer, const q8_batch &batch, int nq, const float *q, float scale,
                         float *out, int topk, int32_t *selected, void *workspace, int32_t *dev_status,
                         hipStream_t stream);

hipError_t launch_prefill(const q8_kv_layer &layer, const q8_batch &batch, int nq, const int32_t *q_start,
                          int total_q, int max_new, const float *q, float scale, float *out, int32_t *dev_status,
                          hipStream_t stream);

hipError_t launch_decode_merge(const q8_kv_layer &layer, const q8_batch &batch, int nq, float *out,
                               const DecodePlan &plan, void *workspace, hipStream_t stream);

// Devices a process's per-device tables cover (device ordinals 0 .. 63).
constexpr int kMaxDevices = 64;

// Resident workgroups per CU of the decode kernel for this group size.
int decode_blocks_per_cu(int group, int waves, int batch);

// The decode's score path for a shape: the i8 matrix cores at four query
// heads per KV head when a 32-token tile lies in one block (kv_bs >= 32),
// else sdot4 over two lanes per 32-block.
inline bool decode_uses_mfma_scores(int group, int kv_bs) { return group == 4 && kv_bs >= 32; }

hipError_t launch_quantize_q(const float *q, int32_t rows, int32_t path, int8_t *codes, float *qscale,
                             hipStream_t stream);

hipError_t launch_qk_partials(const q8_kv_layer &layer, const q8_batch &batch, int nq, const float *q,
                              int32_t *partials, int8_t *qcodes, float *qscale, int32_t *dev_status,
                              hipStream_t stream);

// The library's own device scratch (q8kv_static.hip): its size, and this
// device's address of it.
size_t static_scratch_bytes();
hipError_t static_scratch(void **ptr);

// The step plan (q8kv_stepplan.hip).
size_t step_plan_bytes(const q8_batch &batch, int nparts);
hipError_t launch_step_plan(const q8_kv_layer &layer, const q8_batch &batch, int nq, const DecodePlan &plan,
                            void *plan_buf, int32_t *dev_status, hipStream_t stream);

hipError_t launch_stream_read(const void *buf, size_t bytes, int workgroups, int nontemporal, uint32_t *sink,
                              hipStream_t stream);
hipError_t launch_issue_probe(float *out, int mode, int valu_iters, int mfma_iters, int workgroups,
                              hipStream_t stream);

}  // namespace q8kv
