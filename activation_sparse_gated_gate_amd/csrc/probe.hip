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

// The same read with a chosen access pattern: IF 16-byte loads in flight per
// thread, non-temporal (NTP) or default cache policy; PAT 0 = grid-stride words
// (the whole grid sweeps the buffer together), PAT 1 = workgroup b reads one
// contiguous block of the buffer (the pattern of the batch-1 decode kernel,
// whose workgroups each own consecutive rows).
template <int IF, bool NTP, int PAT>
__global__ __launch_bounds__(1024) void k_read_probe_cfg(const uint4 *__restrict__ p, size_t n16,
                                                         uint32_t *__restrict__ out)
{
    const size_t nt = blockDim.x;
    size_t i0, i1, stride;
    if (PAT == 0) {
        i0 = (size_t)blockIdx.x * nt + threadIdx.x;
        i1 = n16;
        stride = (size_t)gridDim.x * nt;
    } else {
        const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
        const size_t b0 = min(n16, (size_t)blockIdx.x * per);
        i0 = b0 + threadIdx.x;
        i1 = min(n16, b0 + per);
        stride = nt;
    }
    uint32_t acc = 0;
    size_t i = i0;
    for (; i + (IF - 1) * stride < i1; i += IF * stride) {
        uint4 v[IF];
#pragma unroll
        for (int u = 0; u < IF; ++u) v[u] = NTP ? ld16_nt(p + i + u * stride) : ld16(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < IF; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < i1; i += stride) {
        const uint4 v = NTP ? ld16_nt(p + i) : ld16(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    __shared__ uint32_t r[1024];
    r[threadIdx.x] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t x = 0;
        for (size_t k = 0; k < nt; ++k) x ^= r[k];
        out[blockIdx.x] = x;
    }
}

// Latency of isolated row reads: one wave reads n rows of row_bytes (<= 1024)
// at the given byte offsets one after another, each read finished before the
// next is issued; out[i] = core clock cycles of read i, out[n] / out[n + 1] =
// core cycles / 100 MHz reference ticks over the whole loop (the clock rate).
// Offsets past the buffer are clamped to its last row.
__global__ __launch_bounds__(64) void k_latency_probe(const uint8_t *__restrict__ buf, size_t bytes, int row_bytes,
                                                      const uint64_t *__restrict__ offsets, int n,
                                                      unsigned long long *__restrict__ out)
{
    const int lane = threadIdx.x;
    const unsigned long long c0 = clock64(), w0 = wall_clock64();
    uint32_t acc = 0;
    for (int i = 0; i < n; ++i) {
        const uint64_t off = min((uint64_t)offsets[i], (uint64_t)(bytes - row_bytes)) & ~(uint64_t)15;
        const unsigned long long t0 = clock64();
        uint4 v = make_uint4(0, 0, 0, 0);
        if (lane * 16 < row_bytes) v = ld16_nt(buf + off + lane * 16);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
        // the wave's reads complete before the clock is read again
        acc = __builtin_amdgcn_readfirstlane(acc) ^ acc;
        const unsigned long long t1 = clock64();
        if (lane == 0) out[i] = (t1 - t0) + (acc == 0x9E3779B9u ? 1ull : 0ull);
    }
    const unsigned long long c1 = clock64(), w1 = wall_clock64();
    if (lane == 0) {
        out[n] = c1 - c0;
        out[n + 1] = w1 - w0;
    }
}

}  // namespace sffn

extern "C" sffn_status sffn_read_probe_cfg(const void *buf, size_t bytes, const sffn_probe_cfg *cfg, uint32_t *out,
                                           void *stream)
{
    if (!buf || !out || !cfg || bytes < 16 || (bytes & 15) || ((uintptr_t)buf & 15)) return SFFN_ERR_INVALID_ARG;
    const sffn_probe_cfg c = *cfg;
    if (c.workgroups < 1 || c.workgroups > 65536 || (c.threads != 256 && c.threads != 512 && c.threads != 1024) ||
        (c.pattern != 0 && c.pattern != 1) || (c.in_flight != 4 && c.in_flight != 8 && c.in_flight != 16) ||
        (c.nontemporal != 0 && c.nontemporal != 1))
        return SFFN_ERR_INVALID_ARG;
    const hipStream_t st = (hipStream_t)stream;
    const uint4 *p = (const uint4 *)buf;
    const size_t n16 = bytes / 16;
    hipEvent_t evb = nullptr, eve = nullptr;
    sffn::free_timer().take(&evb, &eve);   // armed by sffn_set_kernel_timer(NULL, ...)
#define SFFN_PROBE(IF, NTP, PAT)                                                                                  \
    if (c.in_flight == IF && c.nontemporal == NTP && c.pattern == PAT)                                            \
        SFFN_LAUNCH((sffn::k_read_probe_cfg<IF, NTP != 0, PAT>), dim3(c.workgroups), dim3(c.threads), 0, st, evb, eve, \
                    p, n16, out);
    SFFN_PROBE(4, 0, 0) SFFN_PROBE(4, 0, 1) SFFN_PROBE(4, 1, 0) SFFN_PROBE(4, 1, 1)
    SFFN_PROBE(8, 0, 0) SFFN_PROBE(8, 0, 1) SFFN_PROBE(8, 1, 0) SFFN_PROBE(8, 1, 1)
    SFFN_PROBE(16, 0, 0) SFFN_PROBE(16, 0, 1) SFFN_PROBE(16, 1, 0) SFFN_PROBE(16, 1, 1)
#undef SFFN_PROBE
    return hipGetLastError() == hipSuccess ? SFFN_OK : SFFN_ERR_HIP;
}

extern "C" sffn_status sffn_read_latency_probe(const void *buf, size_t bytes, int32_t row_bytes,
                                               const uint64_t *offsets, int32_t n, unsigned long long *out,
                                               void *stream)
{
    if (!buf || !offsets || !out || n < 1 || row_bytes < 16 || row_bytes > 1024 || (row_bytes & 15) ||
        bytes < (size_t)row_bytes || ((uintptr_t)buf & 15))
        return SFFN_ERR_INVALID_ARG;
    hipLaunchKernelGGL(sffn::k_latency_probe, dim3(1), dim3(64), 0, (hipStream_t)stream, (const uint8_t *)buf, bytes,
                       row_bytes, offsets, n, out);
    return hipGetLastError() == hipSuccess ? SFFN_OK : SFFN_ERR_HIP;
}

extern "C" sffn_status sffn_read_probe(const void *buf, size_t bytes, int32_t workgroups, uint32_t *out, void *stream)
{
    if (!buf || !out || bytes < 16 || (bytes & 15) || ((uintptr_t)buf & 15) || workgroups < 1 || workgroups > 65536)
        return SFFN_ERR_INVALID_ARG;
    hipLaunchKernelGGL(sffn::k_read_probe, dim3(workgroups), dim3(256), 0, (hipStream_t)stream, (const uint4 *)buf,
                       bytes / 16, out);
    return hipGetLastError() == hipSuccess ? SFFN_OK : SFFN_ERR_HIP;
}
