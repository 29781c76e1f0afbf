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
    int emit_here;           // one sequence: k_blk_select writes the list itself (offset 0), no k_blk_emit
};

// Exact block masses.  Let u be the ulp of the sequence's smallest nonzero
// score: every score, block mass and sum of block masses is an integer
// multiple of u.  When the sequence's total is below 2^53 u, every partial sum
// of scores is an fp64 number, so every fp64 addition of them is exact and its
// result does not depend on the order: the block masses are then summed with
// all tokens at once and the rank-order sums by a scan.  Otherwise (a
// negative, infinite or NaN score, more than 2^26 between the largest and the
// smallest nonzero score, or a total of 2^52 u or more as summed here -- an
// fp64 sum in any order, within a factor 1 + 2^-38 of the true one) the block
// masses are added in token order and their rank-order sums in rank order.
constexpr int kBlkPer = kMaxPrefillRows / 256;   // tokens per thread

// a sum over the wave (a bound check only: any grouping will do)
__device__ __forceinline__ double wave_tree_sum_f64(double v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// inclusive prefix of doubles over the 64 lanes (exact sums: any grouping)
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_add_f64(double v)
{
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, CTRL, ROWS, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), CTRL, ROWS, 0xf, false);
    return v + __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// The sequence's block masses into S[0, nb), summed with all tokens at once;
// false (S not usable) when the scores break the condition.  The mass of a run
// of a thread's consecutive tokens inside one block goes in with one atomic.
__device__ bool blk_masses_exact(const BlkArgs &a, int o0, int Lq, int nb, double *S, int *red, double *wsum)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, B = a.block;
    if (Lq == 0) return false;
    // the sequence's scores through LDS: coalesced loads (all in flight,
    // clamped), then thread t takes tokens 64 t .. 64 t + 63; one pad word per
    // 64 puts a wave's 64 reads of one step in 64 different banks
    __shared__ uint32_t stage[kMaxPrefillRows + kMaxPrefillRows / 64];
    uint32_t b[kBlkPer];
#pragma unroll
    for (int k = 0; k < kBlkPer; ++k) b[k] = __float_as_uint(a.s[o0 + min(k * 256 + tid, Lq - 1)]);
#pragma unroll
    for (int k = 0; k < kBlkPer; ++k) {
        const int i = k * 256 + tid;
        stage[i + (i >> 6)] = b[k];
    }
    for (int bb = tid; bb < nb; bb += 256) S[bb] = 0.0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kBlkPer; ++k) {
        const int i = kBlkPer * tid + k;
        b[k] = stage[i + (i >> 6)];
    }
    const int nv = min(max(Lq - kBlkPer * tid, 0), kBlkPer);
    uint32_t bmax = 0, emn = 255;
#pragma unroll
    for (int k = 0; k < kBlkPer; ++k) {
        if (k < nv) {
            bmax = max(bmax, b[k]);
            if (b[k] - 1u < 0x7F7FFFFFu) emn = min(emn, (uint32_t)max((int)(b[k] >> 23), 1));
        }
    }
    // block masses: this thread's tokens fall in a few consecutive blocks.  In
    // chunks of 16 tokens, which hold at most one block start (B >= 16): the
    // masked sums before and from that start, without branches per token
    double tsum = 0.0;
    if (nv > 0) {
        double run = 0.0;
        int cur = (kBlkPer * tid) / B;
        int next = (cur + 1) * B;   // the first token of the next block
#pragma unroll
        for (int c = 0; c < kBlkPer / 16; ++c) {
            const int p = next - (kBlkPer * tid + 16 * c);   // >= 0; < 16: a block starts here
            double lo = 0.0, hi = 0.0;
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const double v = 16 * c + k < nv ? (double)__uint_as_float(b[16 * c + k]) : 0.0;
                lo += k < p ? v : 0.0;
                hi += k < p ? 0.0 : v;
            }
            run += lo;
            if (p < 16) {
                // cur may pass nb only after the sequence's last token, with run = 0
                if (cur < nb) atomicAdd(&S[cur], run);
                tsum += run;
                run = hi;
                ++cur;
                next += B;
            }
        }
        // the last block's run (a start past the sequence's end opens no block)
        if (cur < nb) atomicAdd(&S[cur], run);
        tsum += run;
    }
    bmax = wave_max_dpp(bmax);
    const uint32_t nemn = wave_max_dpp(255u - emn);
    tsum = wave_tree_sum_f64(tsum);
    if (lane == 0) {
        red[wave] = (int)bmax;
        red[4 + wave] = (int)nemn;
        wsum[wave] = tsum;
    }
    __syncthreads();
    uint32_t gmax = 0, gne = 0;
    double total = 0.0;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
        gmax = max(gmax, (uint32_t)red[w2]);
        gne = max(gne, (uint32_t)red[4 + w2]);
        total += wsum[w2];
    }
    const int emin = 255 - (int)gne, emax = max((int)(gmax >> 23), 1);
    if (gmax > 0x7F7FFFFFu || (gmax != 0u && emax - emin > 26)) return false;
    // total < 2^52 u, u = 2^(emin - 150)
    if (gmax != 0u && !(total < __longlong_as_double((long long)(emin - 98 + 1023) << 52))) return false;
    return true;
}

// rank-order sums of the masses in cum[0, nb) (in rank order), in place, by a
// scan: 4 consecutive ranks per thread (nb <= 1024); exact sums only
__device__ void blk_rank_sums_exact(double *cum, int nb, double *wsum)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    double v[4], sum = 0.0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int r = tid * 4 + k;
        v[k] = r < nb ? cum[r] : 0.0;
        sum += v[k];
    }
    double incl = sum;
    incl = dpp_add_f64<0x111, 0xf>(incl);   // row_shr:1
    incl = dpp_add_f64<0x112, 0xf>(incl);   // row_shr:2
    incl = dpp_add_f64<0x114, 0xf>(incl);   // row_shr:4
    incl = dpp_add_f64<0x118, 0xf>(incl);   // row_shr:8
    incl = dpp_add_f64<0x142, 0xa>(incl);   // row_bcast:15
    incl = dpp_add_f64<0x143, 0xc>(incl);   // row_bcast:31
    __syncthreads();   // wsum is free again
    if (lane == 63) wsum[wave] = incl;
    __syncthreads();
    double c = incl - sum;
#pragma unroll
    for (int w2 = 0; w2 < 3; ++w2) c += w2 < wave ? wsum[w2] : 0.0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int r = tid * 4 + k;
        c += v[k];
        if (r < nb) cum[r] = c;
    }
}

// The kept blocks' token count, further blocks in rank order until
// min(min_keep, Lq) tokens are kept (not for a dense sequence), the count and
// the flags out.
__device__ void blk_finish(const BlkArgs &a, int q, int o0, int Lq, int nb, bool dense, const int *ord,
                           uint8_t *kept, int *red)
{
    const int tid = threadIdx.x, B = a.block;
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

__device__ int emit_blocks(const BlkArgs &a, int o0, int Lq, int nb, const uint8_t *kept, int base_out, int *pos,
                           int *red);

__global__ __launch_bounds__(256) void k_blk_select(const BlkArgs a)
{
    __shared__ double S[kMaxBlocksPerSeq];
    __shared__ double cum[kMaxBlocksPerSeq];
    __shared__ int ord[kMaxBlocksPerSeq];
    __shared__ uint8_t kept[kMaxBlocksPerSeq];
    __shared__ int red[8];
    __shared__ double wsum[4];
    const int q = blockIdx.x, tid = threadIdx.x, B = a.block;
    __shared__ int s_bad;   // a non-finite block mass (from a NaN or infinite score)
    int o0, o1;
    if (tid == 0) s_bad = 0;
    seq_range(a.cu, q, a.rows, &o0, &o1, red);
    const int Lq = o1 - o0;
    const int nb = (Lq + B - 1) / B;   // <= kMaxBlocksPerSeq (block >= 16, rows <= 16384)
    for (int bb = tid; bb < nb; bb += 256) kept[bb] = 0;
    const bool exact = blk_masses_exact(a, o0, Lq, nb, S, red, wsum);
    if (!exact) {
        __syncthreads();
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
            if (!isfinite(m)) s_bad = 1;
        }
    }
    __syncthreads();
    // rank of each block by counting (mass desc, index asc): with nb < 256 the
    // comparisons of a block are split over P = 256 / nb threads, whose counts
    // are added in LDS; the masses then go in rank order
    {
        const int P = nb >= 256 ? 1 : 256 / max(nb, 1);
        for (int bb = tid; bb < nb; bb += 256) ord[bb] = 0;   // the counts, for now
        __syncthreads();
        for (int w = tid; w < nb * P; w += 256) {
            const int bb = w % nb, part = w / nb;
            const int c0 = part * nb / P, c1 = (part + 1) * nb / P;
            const double m = S[bb];
            int r = 0;
            for (int b0 = c0; b0 < c1; b0 += 8) {
                double m2[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) m2[i] = S[min(b0 + i, c1 - 1)];
#pragma unroll
                for (int i = 0; i < 8; ++i)   // bitwise, not short-circuit: no branch per comparison
                r += (int)((b0 + i < c1) & ((m2[i] > m) | ((m2[i] == m) & (b0 + i < bb))));
            }
            if (r) atomicAdd(&ord[bb], r);
        }
        __syncthreads();
        int rk[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) rk[k] = tid + 256 * k < nb ? ord[tid + 256 * k] : 0;
        __syncthreads();
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int bb = tid + 256 * k;
            if (bb < nb) {
                ord[rk[k]] = bb;
                cum[rk[k]] = S[bb];
            }
        }
    }
    __syncthreads();
    if (exact) {
        blk_rank_sums_exact(cum, nb, wsum);
    } else if (tid == 0) {
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
    blk_finish(a, q, o0, Lq, nb, dense, ord, kept, red);
    if (a.emit_here) {
        // one sequence: the list starts at 0 and its length is the kept total
        __shared__ int pos[kMaxBlocksPerSeq + 1];
        const int n = emit_blocks(a, o0, Lq, nb, kept, 0, pos, red);
        if (tid == 0) {
            *a.count_out = n;
            *a.count_copy = n;
        }
    }
}

// The sequence's kept token indices at base_out in the batch-wide list: an
// exclusive prefix of the kept block sizes (4 blocks per thread, then the 256
// partials) in pos, then every wave writes whole kept blocks, its lanes over
// the block's tokens.  kept: one byte per block (LDS or global).  Returns the
// sequence's kept tokens (every thread).
__device__ int emit_blocks(const BlkArgs &a, int o0, int Lq, int nb, const uint8_t *kept, int base_out, int *pos,
                           int *red)
{
    const int tid = threadIdx.x, B = a.block;
    int v[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int b = tid * 4 + i;
        v[i] = (b < nb && kept[b]) ? min(B, Lq - b * B) : 0;
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
    const int lane = tid & 63, wave = tid >> 6;
    for (int b = wave; b < nb; b += 4) {
        const int p0 = pos[b], len = pos[b + 1] - p0;   // 0: not kept
        for (int j = lane; j < len; j += 64) {
            a.idx_out[base_out + p0 + j] = o0 + b * B + j;
            a.keep_copy[base_out + p0 + j] = o0 + b * B + j;
        }
    }
    return pos[nb];
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
    emit_blocks(a, o0, Lq, nb, a.flags + (size_t)(o0 / B + q), base_out, pos, red);
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
    a.emit_here = c.nseq == 1 ? 1 : 0;
    hipLaunchKernelGGL(k_blk_select, dim3(c.nseq), dim3(256), 0, c.stream, a);
    if ((e = hipGetLastError()) != hipSuccess || a.emit_here) return e;
    hipLaunchKernelGGL(k_blk_emit, dim3(c.nseq), dim3(256), 0, c.stream, a);
    return hipGetLastError();
}

}  // namespace sffn
