// probe.hip -- diagnostics: the HBM read ceiling for the access policy of the
// decode kernels (non-temporal 16-byte loads), measured with nothing but the
// read, to set the kernels' achieved bandwidth beside what the memory system
// delivers for the same bytes per launch.
#include <hip/hip_runtime.h>

#include "dev_common.h"
#include "../../include/sffn_diag.h"

namespace sffn {

// Streams n16 16-byte words with non-temporal loads, 8 in flight per thread,
// and folds them with xor into one word per workgroup (so the loads are kept).
__global__ __launch_bounds__(256) void k_read_probe(const uint4 *__restrict__ p, size_t n16,
                                                    uint32_t *__restrict__ out)
{
    const size_t stride = (size_t)gridDim.x * 256;
    uint32_t acc = 0;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 7 * stride < n16; i += 8 * stride) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = ld16_nt(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += stride) {
        const uint4 v = ld16_nt(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    __shared__ uint32_t r[256];
    r[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t x = 0;
        for (int k = 0; k < 256; ++k) x ^= r[k];
        out[blockIdx.x] = x;
    }
}

}  // namespace sffn

extern "C" sffn_status sffn_read_probe(const void *buf, size_t bytes, int32_t workgroups, uint32_t *out, void *stream)
{
    if (!buf || !out || bytes < 16 || (bytes & 15) || ((uintptr_t)buf & 15) || workgroups < 1 || workgroups > 65536)
        return SFFN_ERR_INVALID_ARG;
    hipLaunchKernelGGL(sffn::k_read_probe, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, (const uint4 *)buf,
                       bytes / 16, out);
    return hipGetLastError() == hipSuccess ? SFFN_OK : SFFN_ERR_HIP;
}
