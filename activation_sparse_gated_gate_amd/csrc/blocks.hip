// blocks.hip -- block-granular token selection over a batch of sequences (gfx950).
//
// RedKnot article: at least min_keep tokens per sequence (section on the
// token-selective sparse FFN); token-level bounds min_full_ratio /
// max_full_ratio and a fixed-budget top-K over blocks of 128 tokens, so that
// the kept rows form a few contiguous runs, all on the GPU with no host
// synchronisation (last paragraph of the section on adaptive expert top-K).
// Per sequence [cu[q], cu[q+1]) split into nb blocks from its first token:
//   S_b  = fp64 sum of the block's token scores in token order;
//   rank the blocks by (S_b desc, b asc); c_k = fp64 sum of the k top-ranked
//   S_b in rank order; mass >= 1, c_nb == 0 or a non-finite block mass keeps
//   every block; otherwise
//   K = smallest k with c_k >= mass * c_nb (0 for mass <= 0), capped at
//   floorf(nb * max_full) and then raised to ceilf(nb * min_full); the top K
//   blocks, every block holding one of the last recent_n tokens, and further
//   blocks in rank order until min(min_keep, length) tokens are kept.
// Two launches, one workgroup per sequence: k_blk_select decides the kept
// blocks and counts their tokens; k_blk_emit writes the kept token indices
// at the sequence's offset in the batch-wide ascending list (the sum of the
// earlier sequences' counts) and the total count.
#include <hip/hip_runtime.h>

#include "dev_common.h"
#include "sffn_internal.h"

namespace sffn {

// Sequence q's token range with the offsets clamped to [0, rows] and made
// non-decreasing (running maximum), so the ranges are disjoint, ascending and
// inside the batch whatever the offsets hold.  Called by every thread.
// integer reductions and scans over the 256 threads of a workgroup: inside
// each wave through lane exchanges, then the four wave results through LDS
// (red, at least 4 words); integer arithmetic, so the order does not matter
__device__ __forceinline__ int block256_max(int v, int *red)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = max(v, __shfl_xor(v, off, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = max(max(red[0], red[1]), max(red[2], red[3]));
    __syncthreads();   // red may be reused
    return v;
}

__device__ __forceinline__ int block256_sum(int v, int *red)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    v = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return v;
}

// exclusive prefix sum in thread order
__device__ __forceinline__ int block256_exclusive(int v, int *red)
{
    const int w = threadIdx.x >> 6;
    const int incl = wave_incl_scan(v);
    if ((threadIdx.x & 63) == 63) red[w] = incl;
    __syncthreads();
    int base = 0;
#pragma unroll
    for (int w2 = 0; w2 < 3; ++w2) base += w2 < w ? red[w2] : 0;
    __syncthreads();
    return base + incl - v;
}

__device__ __forceinline__ void seq_range(const int32_t *__restrict__ cu, int q, int rows, int *o0, int *o1,
                                          int *red)
{
    int m = 0;
    for (int p = threadIdx.x; p <= q; p += blockDim.x) m = max(m, min(max(cu[p], 0), rows));
    const int a = block256_max(m, red);
    *o0 = a;
    *o1 = max(a, min(max(cu[q + 1], 0), rows));
}

struct BlkArgs {
    const float *s;          // token scores [rows]
    const int32_t *cu;       // [nseq + 1]
    int rows, nseq, block;
    double mass;
    float min_full, max_full;
    int recent_n, min_keep;
    uint8_t *flags;          // kept flag per block, sequence q's at o0 / block + q
    int32_t *counts;         // kept tokens per sequence [nseq]
    int32_t *idx_out, *count_out;
    int32_t *keep_copy, *count_copy;   // the same list and count in the scratch (for forward without a list)
};

__global__ __launch_bounds__(256) void k_blk_select(const BlkArgs a)
{
    __shared__ double S[kMaxBlocksPerSeq];
    __shared__ double cum[kMaxBlocksPerSeq];
    __shared__ int ord[kMaxBlocksPerSeq];
    __shared__ uint8_t kept[kMaxBlocksPerSeq];
    __shared__ int red[4];
    const int q = blockIdx.x, tid = threadIdx.x, B = a.block;
    __shared__ int s_bad;   // a non-finite block mass (from a NaN or infinite score)
    int o0, o1;
    if (tid == 0) s_bad = 0;
    seq_range(a.cu, q, a.rows, &o0, &o1, red);
    const int Lq = o1 - o0;
    const int nb = (Lq + B - 1) / B;   // <= kMaxBlocksPerSeq (block >= 16, rows <= 16384)
    for (int b = tid; b < nb; b += 256) {
        const int t1 = min((b + 1) * B, Lq);
        double m = 0.0;
        // 32 scores loaded at a time, then added in token order
        for (int t0 = b * B; t0 < t1; t0 += 32) {
            float v[32];
#pragma unroll
            for (int i = 0; i < 32; ++i) v[i] = a.s[o0 + min(t0 + i, t1 - 1)];
#pragma unroll
            for (int i = 0; i < 32; ++i)
                if (t0 + i < t1) m = m + (double)v[i];
        }
        S[b] = m;
        kept[b] = 0;
        if (!isfinite(m)) s_bad = 1;
    }
    __syncthreads();
    // rank of each block by counting; the masses are also stored in rank order
    for (int b = tid; b < nb; b += 256) {
        const double m = S[b];
        int r = 0;
        for (int b2 = 0; b2 < nb; ++b2) {
            const double m2 = S[b2];
            r += (m2 > m) || (m2 == m && b2 < b);
        }
        ord[r] = b;
        cum[r] = m;
    }
    __syncthreads();
    if (tid == 0) {
        // cumulative mass in rank order, in place; 16 masses read at a time
        double c = 0.0;
        for (int k0 = 0; k0 < nb; k0 += 16) {
            double v[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i] = cum[min(k0 + i, nb - 1)];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                if (k0 + i < nb) {
                    c = c + v[i];
                    cum[k0 + i] = c;
                }
        }
    }
    __syncthreads();
    const double total = nb > 0 ? cum[nb - 1] : 0.0;
    // a non-finite total keeps the sequence.  It is taken from the block masses
    // themselves: a NaN mass has no rank, so the rank-order sums above do not
    // hold it (the fp64 sum of finite fp32 scores cannot overflow)
    const bool dense = a.mass >= 1.0 || total == 0.0 || s_bad != 0;
    if (dense) {
        for (int b = tid; b < nb; b += 256) kept[b] = 1;
    } else {
        int K = 0;
        if (a.mass > 0.0) {
            // first k (0-based) with cum[k] >= thr; cum is non-decreasing
            const double thr = a.mass * total;
            int lo = 0, hi = nb - 1;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (cum[mid] >= thr) hi = mid;
                else lo = mid + 1;
            }
            K = lo + 1;
        }
        const int kl = (int)ceilf((float)nb * a.min_full);
        const int kh = (int)floorf((float)nb * a.max_full);
        K = max(min(K, kh), kl);
        K = min(K, nb);
        for (int k = tid; k < K; k += 256) kept[ord[k]] = 1;
        if (a.recent_n > 0) {
            const int first = max(Lq - a.recent_n, 0) / B;
            for (int b = first + tid; b < nb; b += 256) kept[b] = 1;
        }
    }
    __syncthreads();
    int part = 0;
    for (int b = tid; b < nb; b += 256)
        if (kept[b]) part += min(B, Lq - b * B);
    const int kept_tokens = block256_sum(part, red);
    if (tid == 0) {
        int cnt = kept_tokens;
        if (!dense) {
            const int need = min(a.min_keep, Lq);
            for (int k = 0; k < nb && cnt < need; ++k) {
                const int b = ord[k];
                if (!kept[b]) {
                    kept[b] = 1;
                    cnt += min(B, Lq - b * B);
                }
            }
        }
        a.counts[q] = cnt;
    }
    __syncthreads();
    uint8_t *fl = a.flags + (size_t)(o0 / B + q);
    for (int b = tid; b < nb; b += 256) fl[b] = kept[b];
}

__global__ __launch_bounds__(256) void k_blk_emit(const BlkArgs a)
{
    __shared__ int pos[kMaxBlocksPerSeq + 1];
    __shared__ int red[4];
    const int q = blockIdx.x, tid = threadIdx.x, B = a.block;
    int o0, o1;
    seq_range(a.cu, q, a.rows, &o0, &o1, red);
    const int Lq = o1 - o0;
    const int nb = (Lq + B - 1) / B;
    // offset of this sequence in the list: the earlier sequences' counts
    int acc = 0;
    for (int p = tid; p < q; p += 256) acc += a.counts[p];
    const int base_out = block256_sum(acc, red);
    if (q == a.nseq - 1 && tid == 0) {
        *a.count_out = base_out + a.counts[q];
        *a.count_copy = base_out + a.counts[q];
    }
    // exclusive prefix of kept block sizes: 4 blocks per thread, then the 256 partials
    const uint8_t *fl = a.flags + (size_t)(o0 / B + q);
    int v[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int b = tid * 4 + i;
        v[i] = (b < nb && fl[b]) ? min(B, Lq - b * B) : 0;
        sum += v[i];
    }
    // pos[b] = kept tokens of the blocks before b, for b = 0..nb
    int run = block256_exclusive(sum, red);
    if (tid == 0) pos[0] = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int b = tid * 4 + i;
        run += v[i];
        if (b < nb) pos[b + 1] = run;
    }
    __syncthreads();
    for (int t = tid; t < Lq; t += 256) {
        const int b = t / B;
        if (pos[b + 1] != pos[b]) {
            a.idx_out[base_out + pos[b] + (t - b * B)] = o0 + t;
            a.keep_copy[base_out + pos[b] + (t - b * B)] = o0 + t;
        }
    }
}

hipError_t launch_block_select(const BlockSelectCall &c)
{
    const Layer &L = *c.L;
    const ScratchLayout S = scratch_layout(L.desc);
    float *sc = (float *)(c.scratch + S.tscore);
    hipError_t e = launch_token_norms(c.A, c.rows, L.desc.d_model, sc, c.stream);
    if (e != hipSuccess) return e;
    BlkArgs a{sc, c.cu, c.rows, c.nseq, c.block, c.mass, c.min_full, c.max_full, c.recent_n, c.min_keep,
              c.scratch + S.tkeys, (int32_t *)(c.scratch + S.tflag), c.idx_out, c.count_out,
              (int32_t *)(c.scratch + S.tkeep), (int32_t *)(c.scratch + S.tkcnt)};
    hipLaunchKernelGGL(k_blk_select, dim3(c.nseq), dim3(256), 0, c.stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_blk_emit, dim3(c.nseq), dim3(256), 0, c.stream, a);
    return hipGetLastError();
}

}  // namespace sffn
