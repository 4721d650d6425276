// q8kv_probe.hip -- measurement hook: the read ceiling the decode kernel is
// judged against.  The q8 decode reads its cache exactly once ("why long
// context must be sparse" §1: decode attention is bounded by the bytes of
// the cache it must read), so the fastest it can be is the time this GPU
// takes to stream the same bytes once.  This kernel does only that: a
// contiguous buffer split statically over `workgroups` workgroups of 512
// lanes, every lane four 16-byte loads in flight, plain or non-temporal (the
// hint the decode's cache loads carry), and a value folded from every load
// written only if it equals a constant (so no load can be dropped).
#include "q8kv_internal.hpp"

namespace q8kv {

constexpr int kProbeLanes = 512;
constexpr int kProbeInFlight = 4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <bool NonTemporal>
__global__ __launch_bounds__(kProbeLanes) void q8_stream_read_kernel(const u32x4 *__restrict__ buf, size_t n16,
                                                                     uint32_t *sink)
{
    const size_t lo = (size_t)blockIdx.x * n16 / gridDim.x;
    const size_t hi = (size_t)(blockIdx.x + 1) * n16 / gridDim.x;
    uint32_t acc = 0;
    for (size_t i = lo + threadIdx.x; i < hi; i += (size_t)kProbeInFlight * kProbeLanes) {
        u32x4 v[kProbeInFlight];
#pragma unroll
        for (int u = 0; u < kProbeInFlight; ++u) {
            const size_t idx = i + (size_t)u * kProbeLanes;
            if (idx < hi)
                v[u] = NonTemporal ? __builtin_nontemporal_load(buf + idx) : buf[idx];
            else
                v[u] = u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kProbeInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

hipError_t launch_stream_read(const void *buf, size_t bytes, int workgroups, int nontemporal, uint32_t *sink,
                              hipStream_t stream)
{
    const u32x4 *b = static_cast<const u32x4 *>(buf);
    const size_t n16 = bytes / 16;
    if (nontemporal)
        hipLaunchKernelGGL(q8_stream_read_kernel<true>, dim3(workgroups), dim3(kProbeLanes), 0, stream, b, n16, sink);
    else
        hipLaunchKernelGGL(q8_stream_read_kernel<false>, dim3(workgroups), dim3(kProbeLanes), 0, stream, b, n16,
                           sink);
    return hipGetLastError();
}

}  // namespace q8kv
