// relayout.hip -- one-time weight preparation at layer creation (gfx950).
//
// Decode reads W_up rows and W_down columns of active neurons only.  A column
// of the row-major W_down [d][f] is strided, so the decode layout stores
// W_down^T [f][d]: neuron j's down weights become one contiguous row that the
// gather kernel reads with 16-byte loads.  int4 W_down has its scale groups
// along d_ff (its input dimension); in the transposed layout the scale of
// element (j, i) is S[j/128][i].  The fp64 column norms ||W_down[:, j]||_2 used
// by the weight-aware score (WiSparse notes, section 2.3) are computed here
// once, as an ascending fp64 sum of squares and an IEEE square root.  Prefill
// interleaves W_gate and W_up in blocks of 32 rows so that one GEMM tile holds
// the gate and up columns of the same neurons.
#include <hip/hip_runtime.h>

#include "dev_common.h"

namespace sffn {

// out[j][i] = in[i][j] for 2- or 4-byte elements, 64 x 64 tiles through LDS
template <typename T>
__global__ __launch_bounds__(256) void k_transpose(const T *__restrict__ in, T *__restrict__ out, int rows,
                                                   int cols)
{
    __shared__ T tile[64][65];
    const int c0 = blockIdx.x * 64, r0 = blockIdx.y * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int r = ty; r < 64; r += 4)
        if (r0 + r < rows && c0 + tx < cols) tile[r][tx] = in[(size_t)(r0 + r) * cols + c0 + tx];
    __syncthreads();
    for (int c = ty; c < 64; c += 4)
        if (c0 + c < cols && r0 + tx < rows) out[(size_t)(c0 + c) * rows + r0 + tx] = tile[tx][c];
}

// int4 transpose of packed nibbles: in [rows][cols/2] -> out [cols][rows/2]
__global__ __launch_bounds__(256) void k_transpose_i4(const uint8_t *__restrict__ in, uint8_t *__restrict__ out,
                                                      int rows, int cols)
{
    const size_t n = (size_t)cols * (rows / 2);
    for (size_t o = (size_t)blockIdx.x * 256 + threadIdx.x; o < n; o += (size_t)gridDim.x * 256) {
        const int j = (int)(o / (rows / 2));       // output row = input column
        const int ib = (int)(o - (size_t)j * (rows / 2));
        const int i0 = 2 * ib, i1 = 2 * ib + 1;
        const uint8_t b0 = in[(size_t)i0 * (cols / 2) + j / 2];
        const uint8_t b1 = in[(size_t)i1 * (cols / 2) + j / 2];
        const uint8_t n0 = (j & 1) ? (b0 >> 4) : (b0 & 15);
        const uint8_t n1 = (j & 1) ? (b1 >> 4) : (b1 & 15);
        out[o] = (uint8_t)(n0 | (n1 << 4));
    }
}

// n_j = sqrt(sum_i w_ij^2), fp64, i ascending; W_down natural [d][f]
template <int WT>
__global__ __launch_bounds__(256) void k_col_norms(const uint8_t *__restrict__ wd, const uint16_t *__restrict__ sd,
                                                   int d, int f, double *__restrict__ out)
{
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= f) return;
    double s = 0.0;
    for (int i = 0; i < d; ++i) {
        double w;
        if constexpr (WT == SFFN_W_F32) {
            w = (double)((const float *)wd)[(size_t)i * f + j];
        } else if constexpr (WT == SFFN_W_BF16) {
            w = (double)bf16_lo(((const uint16_t *)wd)[(size_t)i * f + j]);
        } else {
            const uint8_t b = wd[(size_t)i * (f / 2) + j / 2];
            const int q = (j & 1) ? ((int)(b >> 4) ^ 8) - 8 : ((int)(b & 15) ^ 8) - 8;
            w = (double)((float)q * half_bits_to_float(sd[(size_t)i * (f / 128) + j / 128]));
        }
        s = s + w * w;
    }
    out[j] = sqrt(s);
}

// prefill interleave: dst block b = [gate rows 32b..32b+31][up rows 32b..32b+31]
// (neuron n read from source row perm[n] when a permutation is given)
__global__ __launch_bounds__(256) void k_interleave(const uint16_t *__restrict__ wg, const uint16_t *__restrict__ wu,
                                                    uint16_t *__restrict__ dst, int f, int d,
                                                    const int32_t *__restrict__ perm)
{
    const int r = blockIdx.x;  // destination row, 0..2f-1
    const int b = r / (2 * kIlvRows), w = (r / kIlvRows) & 1, rr = r % kIlvRows;
    const int n = b * kIlvRows + rr;
    const uint16_t *src = (w ? wu : wg) + (size_t)(perm ? perm[n] : n) * d;
    uint16_t *o = dst + (size_t)r * d;
    for (int i = threadIdx.x * 8; i < d; i += 256 * 8) *(uint4 *)(o + i) = *(const uint4 *)(src + i);
}

// [R][C] bf16 row-major -> 16 x 32 MFMA operand tiles [R/16][C/32][64][8]: lane l of tile (t, s)
// holds row 16t + (l & 15), columns 32s + 8(l >> 4) .. +8 (R % 16 == 0, C % 32 == 0).  One thread
// per 16-byte lane slot; reads are 16 bytes of one row, writes are contiguous.
__global__ __launch_bounds__(256) void k_tile_mfma(const uint16_t *__restrict__ src, uint16_t *__restrict__ dst,
                                                   int R, int C)
{
    const size_t nslot = (size_t)R * C / 8;
    const int ks = C / 32;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < nslot; i += (size_t)gridDim.x * 256) {
        const int l = (int)(i & 63);
        const size_t ts = i >> 6;
        const int s = (int)(ts % ks);
        const size_t t = ts / ks;
        const size_t r = t * 16 + (l & 15);
        const int c = s * 32 + 8 * (l >> 4);
        *(uint4 *)(dst + i * 8) = *(const uint4 *)(src + r * C + c);
    }
}

// W_gate [f][d] bf16 -> [4 classes][K][f][16][8] with K = ceil(d / 512): entry (m, k, j, i)
// is chunk m + 4i + 64k (8 values) of row j, zero where that chunk is past the row.
__global__ __launch_bounds__(256) void k_tile_gate_cls(const uint16_t *__restrict__ src, uint16_t *__restrict__ dst,
                                                       int f, int d)
{
    const int nch = d / 8, K = (nch + 63) / 64;
    const size_t nslot = (size_t)4 * K * f * 16;
    for (size_t s = (size_t)blockIdx.x * 256 + threadIdx.x; s < nslot; s += (size_t)gridDim.x * 256) {
        const int i = (int)(s & 15);
        const size_t rest = s >> 4;
        const size_t j = rest % f;
        const size_t mk = rest / f;
        const int k = (int)(mk % K), m = (int)(mk / K);
        const int ch = m + 4 * i + 64 * k;
        *(uint4 *)(dst + s * 8) = ch < nch ? *(const uint4 *)(src + j * d + (size_t)ch * 8) : make_uint4(0, 0, 0, 0);
    }
}

hipError_t launch_relayout(const Layer &L, const void *w_gate, const void *w_up, const void *w_down,
                           const void *s_gate, const void *s_up, const void *s_down, uint8_t *base,
                           hipStream_t st, const int32_t *ilv_perm)
{
    const sffn_layer_desc &D = L.desc;
    const int d = D.d_model, f = D.d_ff, wt = D.wtype;
    const PersistentLayout P = persistent_layout(D);
    hipError_t e;
    const size_t mat = row_bytes(wt, d) * (size_t)f;  // bytes of one [f][d] (or [d][f]) matrix
    const size_t scl = (size_t)f * (d / 128) * 2;     // bytes of its int4 scales
    const size_t scl_d = (size_t)d * (f / 128) * 2;

    if (D.layouts & SFFN_LAYOUT_DECODE) {
        // (a permuted layer's copies are already in place)
        if (w_gate != base + P.wg)
            if ((e = hipMemcpyAsync(base + P.wg, w_gate, mat, hipMemcpyDeviceToDevice, st)) != hipSuccess) return e;
        if (w_up != base + P.wu)
            if ((e = hipMemcpyAsync(base + P.wu, w_up, mat, hipMemcpyDeviceToDevice, st)) != hipSuccess) return e;
        if (wt == SFFN_W_INT4_G128) {
            if ((e = hipMemcpyAsync(base + P.sg, s_gate, scl, hipMemcpyDeviceToDevice, st)) != hipSuccess) return e;
            if ((e = hipMemcpyAsync(base + P.su, s_up, scl, hipMemcpyDeviceToDevice, st)) != hipSuccess) return e;
        }
        // W_down^T [f][d]
        if (wt == SFFN_W_F32) {
            hipLaunchKernelGGL(k_transpose<float>, dim3((f + 63) / 64, (d + 63) / 64), dim3(256), 0, st,
                               (const float *)w_down, (float *)(base + P.wdt), d, f);
        } else if (wt == SFFN_W_BF16) {
            hipLaunchKernelGGL(k_transpose<uint16_t>, dim3((f + 63) / 64, (d + 63) / 64), dim3(256), 0, st,
                               (const uint16_t *)w_down, (uint16_t *)(base + P.wdt), d, f);
        } else {
            hipLaunchKernelGGL(k_transpose_i4, dim3(4096), dim3(256), 0, st, (const uint8_t *)w_down,
                               (uint8_t *)(base + P.wdt), d, f);
            // scales [d][f/128] -> [f/128][d]
            hipLaunchKernelGGL(k_transpose<uint16_t>, dim3((f / 128 + 63) / 64, (d + 63) / 64), dim3(256), 0, st,
                               (const uint16_t *)s_down, (uint16_t *)(base + P.sdt), d, f / 128);
        }
        if ((e = hipGetLastError()) != hipSuccess) return e;
        // column norms
        if (wt == SFFN_W_F32)
            hipLaunchKernelGGL(k_col_norms<SFFN_W_F32>, dim3((f + 255) / 256), dim3(256), 0, st,
                               (const uint8_t *)w_down, (const uint16_t *)s_down, d, f, (double *)(base + P.wdn));
        else if (wt == SFFN_W_BF16)
            hipLaunchKernelGGL(k_col_norms<SFFN_W_BF16>, dim3((f + 255) / 256), dim3(256), 0, st,
                               (const uint8_t *)w_down, (const uint16_t *)s_down, d, f, (double *)(base + P.wdn));
        else
            hipLaunchKernelGGL(k_col_norms<SFFN_W_INT4_G128>, dim3((f + 255) / 256), dim3(256), 0, st,
                               (const uint8_t *)w_down, (const uint16_t *)s_down, d, f, (double *)(base + P.wdn));
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    // W_down natural [d][f]: dense baseline (decode) and prefill
    if (w_down != base + P.wd)
        if ((e = hipMemcpyAsync(base + P.wd, w_down, mat, hipMemcpyDeviceToDevice, st)) != hipSuccess) return e;
    if (wt == SFFN_W_INT4_G128)
        if ((e = hipMemcpyAsync(base + P.sd, s_down, scl_d, hipMemcpyDeviceToDevice, st)) != hipSuccess) return e;

    if ((D.layouts & SFFN_LAYOUT_DECODE) && (D.layouts & SFFN_LAYOUT_BATCH)) {
        hipLaunchKernelGGL(k_tile_mfma, dim3(4096), dim3(256), 0, st, (const uint16_t *)w_up,
                           (uint16_t *)(base + P.wut), f, d);
        hipLaunchKernelGGL(k_tile_mfma, dim3(4096), dim3(256), 0, st, (const uint16_t *)w_down,
                           (uint16_t *)(base + P.wdtl), d, f);
        hipLaunchKernelGGL(k_tile_gate_cls, dim3(4096), dim3(256), 0, st, (const uint16_t *)w_gate,
                           (uint16_t *)(base + P.wgt), f, d);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }

    if (D.layouts & SFFN_LAYOUT_PREFILL) {
        hipLaunchKernelGGL(k_interleave, dim3(2 * f), dim3(256), 0, st,
                           (const uint16_t *)w_gate, (const uint16_t *)w_up, (uint16_t *)(base + P.wgu), f, d,
                           ilv_perm);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace sffn
