// reorder.hip -- neuron reordering by activation frequency (WiSparse
// reproduction notes, section 5, second trick: count how often each neuron is
// active, sort the neurons by that frequency and store the weights in the new
// order, so that the neurons read together lie together in memory).
//
// A permutation perm of the d_ff neurons (new neuron j = original neuron
// perm[j]) is applied once at layer creation: rows of W_gate and W_up and
// columns of W_down are gathered into the persistent natural-layout copies
// (W_gate and W_up only exist there with the DECODE layout; a prefill-only
// layer's interleave reads them through perm instead), and every other
// decode / batched / prefill layout is built from those.  The
// permuted layer computes the same FFN; selections and g' refer to the new
// neuron numbering.  int4 layers are excluded: W_down's scale groups run along
// d_ff, so moving a neuron to another 128-neuron group would change its
// quantisation.
//
// Two orders are provided (host logic, run once after calibration):
//   CLUSTER  neurons by (count desc, index asc): the frequently active
//            neurons share 16-row tiles, so the batched tile path finds more
//            W_up tiles with no selected neuron to skip.
//   BALANCE  ranks dealt in a snake over the batch-1 kernel's blocks of
//            consecutive neurons (one workgroup each), every block sorted by
//            index: each workgroup gets the same share of hot and cold
//            neurons, so no workgroup carries most of the gathers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "sffn_internal.h"

namespace sffn {

// dst row j = src row perm[j] (rows of rb bytes, rb a multiple of 16)
__global__ __launch_bounds__(256) void k_perm_rows(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst,
                                                   const int32_t *__restrict__ perm, size_t rb)
{
    const size_t j = blockIdx.x;
    const uint4 *s = (const uint4 *)(src + (size_t)perm[j] * rb);
    uint4 *o = (uint4 *)(dst + j * rb);
    for (size_t i = threadIdx.x; i < rb / 16; i += 256) o[i] = s[i];
}

// dst[i][j] = src[i][perm[j]] for one row i per workgroup of a [rows][cols] matrix
template <typename T>
__global__ __launch_bounds__(256) void k_perm_cols(const T *__restrict__ src, T *__restrict__ dst,
                                                   const int32_t *__restrict__ perm, int cols)
{
    const size_t i = blockIdx.x;
    for (int j = threadIdx.x; j < cols; j += 256) dst[i * cols + j] = src[i * cols + perm[j]];
}

// counts[idx[q]] += 1 for q < min(*count, f); integer adds, so the totals do
// not depend on their order
__global__ __launch_bounds__(256) void k_neuron_counts(const int32_t *__restrict__ idx,
                                                       const int32_t *__restrict__ count, int f,
                                                       int32_t *__restrict__ counts)
{
    const int n = min(*count, f);
    for (int q = blockIdx.x * 256 + threadIdx.x; q < n; q += gridDim.x * 256) {
        const int j = idx[q];
        if (j >= 0 && j < f) atomicAdd(&counts[j], 1);
    }
}

hipError_t launch_permute_weights(const sffn_layer_desc &D, const void *w_gate, const void *w_up,
                                  const void *w_down, const int32_t *perm, uint8_t *base, hipStream_t st)
{
    const PersistentLayout P = persistent_layout(D);
    const int d = D.d_model, f = D.d_ff;
    const size_t rb = row_bytes(D.wtype, d);
    if (D.layouts & SFFN_LAYOUT_DECODE) {
        hipLaunchKernelGGL(k_perm_rows, dim3(f), dim3(256), 0, st, (const uint8_t *)w_gate, base + P.wg, perm, rb);
        hipLaunchKernelGGL(k_perm_rows, dim3(f), dim3(256), 0, st, (const uint8_t *)w_up, base + P.wu, perm, rb);
    }
    if (D.wtype == SFFN_W_F32)
        hipLaunchKernelGGL(k_perm_cols<float>, dim3(d), dim3(256), 0, st, (const float *)w_down,
                           (float *)(base + P.wd), perm, f);
    else
        hipLaunchKernelGGL(k_perm_cols<uint16_t>, dim3(d), dim3(256), 0, st, (const uint16_t *)w_down,
                           (uint16_t *)(base + P.wd), perm, f);
    return hipGetLastError();
}

}  // namespace sffn

using namespace sffn;

extern "C" {

sffn_status sffn_neuron_counts(const int32_t *idx, const int32_t *count, int32_t d_ff, int32_t *counts,
                               void *stream)
{
    if (!idx || !count || !counts || d_ff < 1 || d_ff > 65536) return SFFN_ERR_INVALID_ARG;
    hipLaunchKernelGGL(k_neuron_counts, dim3((d_ff + 255) / 256), dim3(256), 0, (hipStream_t)stream, idx, count,
                       (int)d_ff, counts);
    return hipGetLastError() == hipSuccess ? SFFN_OK : SFFN_ERR_HIP;
}

int32_t sffn_decode_block_rows(int32_t d_ff) { return d_ff < 1 ? 0 : fused_rows_per_wg(d_ff); }

sffn_status sffn_frequency_order(const int32_t *counts, int32_t d_ff, int32_t mode, int32_t block, int32_t *perm)
{
    if (!counts || !perm || d_ff < 1) return SFFN_ERR_INVALID_ARG;
    if (mode != SFFN_ORDER_CLUSTER && mode != SFFN_ORDER_BALANCE) return SFFN_ERR_INVALID_ARG;
    if (mode == SFFN_ORDER_BALANCE && (block < 1 || block > d_ff)) return SFFN_ERR_INVALID_ARG;
    const int f = d_ff;
    for (int j = 0; j < f; ++j)
        if (counts[j] < 0) return SFFN_ERR_INVALID_ARG;
    std::vector<int32_t> rank(f);
    for (int j = 0; j < f; ++j) rank[j] = j;
    std::stable_sort(rank.begin(), rank.end(), [&](int32_t a, int32_t b) { return counts[a] > counts[b]; });
    if (mode == SFFN_ORDER_CLUSTER) {
        std::copy(rank.begin(), rank.end(), perm);
        return SFFN_OK;
    }
    // snake over the blocks 0, 1, ..., G-1, G-1, ..., 0, 0, 1, ...; full blocks are passed over
    const int G = (f + block - 1) / block;
    std::vector<std::vector<int32_t>> grp(G);
    long long p = 0;
    for (int r = 0; r < f; ++r) {
        for (;; ++p) {
            const int q = (int)(p % G);
            const int g = ((p / G) & 1) ? G - 1 - q : q;
            const int cap = g == G - 1 ? f - (G - 1) * block : block;
            if ((int)grp[g].size() < cap) {
                grp[g].push_back(rank[r]);
                ++p;
                break;
            }
        }
    }
    int o = 0;
    for (int g = 0; g < G; ++g) {
        std::sort(grp[g].begin(), grp[g].end());
        for (int32_t j : grp[g]) perm[o++] = j;
    }
    return SFFN_OK;
}

}  // extern "C"
