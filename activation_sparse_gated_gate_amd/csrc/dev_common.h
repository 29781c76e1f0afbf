// dev_common.h -- device helpers shared by the gfx950 kernels of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sffn_internal.h"

namespace sffn {

// elements per 16-byte weight chunk
template <int WT> struct Chunk;
template <> struct Chunk<SFFN_W_F32> { static constexpr int E = 4; };
template <> struct Chunk<SFFN_W_BF16> { static constexpr int E = 8; };
template <> struct Chunk<SFFN_W_INT4_G128> { static constexpr int E = 32; };

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

__device__ __forceinline__ float half_bits_to_float(uint16_t h)
{
    _Float16 v;
    __builtin_memcpy(&v, &h, 2);
    return (float)v;
}

// signed nibble e (0..7) of a 32-bit word, low nibble first
__device__ __forceinline__ int nib(uint32_t w, int e) { return ((int)(w << (28 - 4 * e))) >> 28; }

__device__ __forceinline__ uint4 ld16(const void *p) { return *(const uint4 *)p; }

// 16-byte load with the non-temporal (streaming) cache policy, for weights
// that are read once per call
typedef unsigned int sffn_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16_nt(const void *p)
{
    const sffn_u32x4 v = __builtin_nontemporal_load((const sffn_u32x4 *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Unpack a 16-byte chunk of fp32 or bf16 weights into E floats (int4 is
// consumed nibble by nibble by its callers).
template <int WT>
__device__ __forceinline__ void unpack(const uint4 &v, float *w)
{
    if constexpr (WT == SFFN_W_F32) {
        w[0] = __uint_as_float(v.x);
        w[1] = __uint_as_float(v.y);
        w[2] = __uint_as_float(v.z);
        w[3] = __uint_as_float(v.w);
    } else {
        w[0] = bf16_lo(v.x); w[1] = bf16_hi(v.x);
        w[2] = bf16_lo(v.y); w[3] = bf16_hi(v.y);
        w[4] = bf16_lo(v.z); w[5] = bf16_hi(v.z);
        w[6] = bf16_lo(v.w); w[7] = bf16_hi(v.w);
    }
}

// One chunk of the fixed-order dot product: acc <- chunk(w) . x, element by
// element with fused multiply-adds (fp32 / bf16), or for int4
// t = sum q_e x_e from +0 then acc <- fma(scale, t, acc).
template <int WT>
__device__ __forceinline__ float chunk_dot(const uint4 &v, float scale, const float *x, float acc)
{
    if constexpr (WT == SFFN_W_INT4_G128) {
        float t = 0.0f;
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) t = __builtin_fmaf((float)nib(wd[q], e), x[q * 8 + e], t);
        return __builtin_fmaf(scale, t, acc);
    } else {
        constexpr int E = Chunk<WT>::E;
        float w[E];
        unpack<WT>(v, w);
#pragma unroll
        for (int e = 0; e < E; ++e) acc = __builtin_fmaf(w[e], x[e], acc);
        return acc;
    }
}

// Halving tree over the 64 lane accumulators: at offset o = 32, 16, ..., 1
// lane p adds lane p ^ o.  For p < o this is acc_p + acc_{p+o}; the upper
// lanes compute the same sums with the operands swapped, which is bitwise
// identical, so every lane ends with the tree's result.
__device__ __forceinline__ float wave_tree_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = v + __shfl_xor(v, off, 64);
    return v;
}

// The same halving tree without LDS traffic: xor 32 and xor 16 through the
// gfx950 lane swaps (each returns both halves; a lane takes its partner's),
// xor 8 as a rotation by 8 inside a row of 16, then a rotation by 4, which
// reads lane i + 4 or i - 4 -- after the xor-8 step both hold the value of
// lane i ^ 4 -- and xor 2, xor 1 as quad permutations.  Each step adds the
// partner's value exactly as the shuffle tree does, so the result is the same
// bit for bit.  Every lane of the wave must be active.
__device__ __forceinline__ float wave_tree_sum_dpp(float v)
{
    const int lane = threadIdx.x & 63;
    {
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = v + __uint_as_float(lane < 32 ? p[1] : p[0]);
    }
    {
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = v + __uint_as_float((lane & 16) ? p[0] : p[1]);
    }
    v = v + __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x128, 0xf, 0xf, false));  // row_ror:8
    v = v + __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x124, 0xf, 0xf, false));  // row_ror:4
    v = v + __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0x4E, 0xf, 0xf, false));   // quad [2,3,0,1]
    v = v + __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(v), 0xB1, 0xf, 0xf, false));   // quad [1,0,3,2]
    return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

// Inclusive prefix sum over the 64 lanes of a wave through DPP: shifts by 1, 2,
// 4, 8 inside each row of 16 (lanes whose source lies outside the row add 0),
// then lane 15 of rows 0 / 2 into rows 1 / 3 and lane 31 into rows 2 / 3.
// Every lane of the wave must be active.
__device__ __forceinline__ int wave_incl_scan(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);   // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);   // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);   // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);   // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);   // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);   // row_bcast:31
    return v;
}

// maximum over the wave, in every lane: lane swaps for xor 32 and 16, row
// rotations by 8 and 4 (after the first, lanes i and i ^ 8 agree, so the
// rotation by 4 reads the value of lane i ^ 4), quad permutations for 2 and 1.
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t v)
{
    const int lane = threadIdx.x & 63;
    {
        const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        v = max(v, (uint32_t)(lane < 32 ? p[1] : p[0]));
    }
    {
        const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        v = max(v, (uint32_t)((lane & 16) ? p[0] : p[1]));
    }
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false));   // row_ror:8
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false));   // row_ror:4
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, false));    // quad [2,3,0,1]
    v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, false));    // quad [1,0,3,2]
    return v;
}

// one step of a DPP prefix over 64-bit values (both halves moved, 0 where the
// source lane lies outside the pattern)
template <int CTRL, int ROWS>
__device__ __forceinline__ uint64_t dpp_add_u64(uint64_t v)
{
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, ROWS, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, ROWS, 0xf, false);
    return v + (((uint64_t)hi << 32) | lo);
}

// inclusive prefix over the 64 lanes (the steps of wave_incl_scan on 64 bits)
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v)
{
    v = dpp_add_u64<0x111, 0xf>(v);   // row_shr:1
    v = dpp_add_u64<0x112, 0xf>(v);   // row_shr:2
    v = dpp_add_u64<0x114, 0xf>(v);   // row_shr:4
    v = dpp_add_u64<0x118, 0xf>(v);   // row_shr:8
    v = dpp_add_u64<0x142, 0xa>(v);   // row_bcast:15
    v = dpp_add_u64<0x143, 0xc>(v);   // row_bcast:31
    return v;
}

__device__ __forceinline__ int mbcnt64(uint64_t m)
{
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

// activation on the offset gate value
__device__ __forceinline__ float act_f32(int act, float z)
{
    return act == SFFN_ACT_RELU ? fmaxf(z, 0.0f) : z / (1.0f + expf(-z));
}

// selection predicate on g' = fl(g + b)
__device__ __forceinline__ bool gate_pred(int mode, float gp, float theta)
{
    return mode == SFFN_MODE_EXACT ? (gp > 0.0f) : mode == SFFN_MODE_THRESH ? (gp > theta) : true;
}

// Block-wide exclusive scan of one int per thread (blockDim.x <= 1024).
// `tmp` needs 17 ints of shared memory.  Returns the exclusive prefix; *total
// receives the block total.
__device__ __forceinline__ int block_exclusive_scan(int v, int *tmp, int *total)
{
    const int lane = lane_id(), wave = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
    int incl = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        int o = __shfl_up(incl, off, 64);
        if (lane >= off) incl += o;
    }
    if (lane == 63) tmp[wave] = incl;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int w = 0; w < nw; ++w) {
            int t = tmp[w];
            tmp[w] = run;
            run += t;
        }
        tmp[16] = run;
    }
    __syncthreads();
    int res = tmp[wave] + incl - v;
    *total = tmp[16];
    __syncthreads();
    return res;
}

}  // namespace sffn
