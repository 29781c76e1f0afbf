// decode.hip -- gfx950 kernels of the decode path (batch of 1..16 tokens).
//
// Path (one layer, all launches on the caller's stream, no host sync):
//   [rmsnorm]  x_hat = x / sqrt(mean(x^2) + eps) in the fixed fp32 order
//   gate       g'_j = fl(W_gate[j,:] . x_hat + b) for every neuron j, in the fixed
//              fp32 order (64 lane accumulators, chunk c -> lane c mod 64, halving
//              tree), fused with the selection predicate and a per-workgroup
//              compaction (wave ballot + mbcnt) into ascending active lists.
//              Exact ReLU gating and the gate threshold follow denseflux
//              (sections 3, 4.1, 5.1-5.3): the gate is read in full, W_up rows and
//              W_down columns only for active neurons.
//   topk       (weight-aware top-k, WiSparse notes, sections 2.3 / 3.2) the gate
//              kernel also produces u in the fixed order; one workgroup per token
//              ranks score = |silu(g') u| * ||W_down[:, j]||_2 (fp64) with an exact
//              radix select, ties to the lower index; the union over the batch is
//              compacted into the same ascending lists.
//   gather     the active list is cut into equal shares; each workgroup reads
//              only its neurons' W_up rows (u, then h = act(g') u) and W_down^T
//              rows, accumulating a partial y with coalesced 16-byte loads.
//   reduce     y = sum of the partials in a fixed order (+ x for the residual).
// The dense baseline (mode DENSE) at batch 1 is the fused kernel over every
// neuron without a selection; at other batch sizes and for int4 it is two
// plain fixed-order GEMV launches: gate + up (h for every neuron), then the
// rows of the natural W_down dotted with h.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "dev_common.h"

namespace sffn {

enum { OUT_GATE = 0, OUT_GATE_UP = 1, OUT_DENSE_GU = 2, OUT_DENSE_DOWN = 3 };

constexpr int kFusedMaxRB = 48;   // neurons per workgroup of the batch-1 streaming kernels
constexpr int kGuI4Waves = 8;     // waves per workgroup of the batch-1 int4 gate + up kernel

// ---------------------------------------------------------------------------
// launch configuration per weight type and batch bucket
// ---------------------------------------------------------------------------
// Batched bf16 decode with the BATCH layout: the row gather reads only the
// union's rows but its work per row grows with the batch, while the MFMA tiles
// stream whole matrices at nearly the same cost for 5..16 tokens.  Union
// fraction (per mille) below which the gather was measured faster, per batch
// size, at 3584 x 18944 (a layer larger than the Infinity Cache): 5 tokens
// about 0.25, 8 tokens about 0.18, 16 tokens never.
static int gather_below_permille(int B)
{
    static const int t[17] = {0, 0, 0, 0, 0, 250, 220, 200, 180, 0, 0, 0, 0, 0, 0, 0, 0};
    return B >= 0 && B <= 16 ? t[B] : 0;
}

template <int WT, int BT> struct Cfg;
// waves and rows per wave of k_rowdot: as Cfg, except that the gate + up
// kernel with int4 weights at 8..16 tokens runs 8 waves of 2 rows (16 rows
// per workgroup), so the staged x slices (all tokens, in every workgroup)
// serve twice the weight rows: measured 6 us faster per 2048 x 11008 layer at
// 8 tokens than 4 waves; 4 rows per wave (the dequantised chunks of every row
// stay in registers across the tokens) was slower at 256 registers
template <int WT, int BT, int OUT> struct RdCfg {
    static constexpr bool TWO = (OUT == OUT_GATE_UP || OUT == OUT_DENSE_GU);
    static constexpr bool WIDE = TWO && WT == SFFN_W_INT4_G128 && BT >= 8;
    static constexpr int NW = WIDE ? 8 : Cfg<WT, BT>::NW;
    static constexpr int RPW = WIDE ? 2 : TWO ? (Cfg<WT, BT>::RPW > 1 ? Cfg<WT, BT>::RPW / 2 : 1) : Cfg<WT, BT>::RPW;
};

template <int WT, int BT> struct Cfg {
    static constexpr int E = Chunk<WT>::E;
    // chunk-columns staged per slice: keeps x in LDS at <= 32 KB (64 KB int4 x 8)
    static constexpr int KMAX =
        WT == SFFN_W_F32 ? (BT == 1 ? 4 : BT == 4 ? 2 : 1)
        : WT == SFFN_W_BF16 ? (BT == 1 ? 8 : BT == 4 ? 2 : 1)
                            : (BT == 1 ? 2 : 1);
    // rows per wave: each lane reuses its x values (read from LDS) over RPW rows,
    // which keeps the LDS reads below the FMA rate at 8-16 tokens
    static constexpr int RPW = (BT == 1 || BT >= 8) ? 4 : 2;
    static constexpr int NW = 4;                     // waves per workgroup
    static constexpr int CPT = (WT == SFFN_W_BF16 && BT == 1) ? 16 : (WT == SFFN_W_F32 ? 4 : 8);
    // down rows in flight per thread: an int4 row gives a thread 4 bytes, so it
    // keeps 16 rows in flight (fewer only costs latency: one workgroup per CU)
    static constexpr int UNR = WT == SFFN_W_INT4_G128 ? 16 : (BT >= 16 ? 2 : 4);
};

// ---------------------------------------------------------------------------
// RMSNorm prologue (one wave per token)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_rmsnorm(const float *__restrict__ x, float *__restrict__ xhat,
                                                int d, float eps)
{
    const int t = blockIdx.x, lane = threadIdx.x;
    const float *xt = x + (size_t)t * d;
    const int nch = d / 4;
    float acc = 0.0f;
    // lane p folds chunks p, p + 64, ... in increasing order; 16 loads in flight
    for (int k0 = 0; k0 * 64 < nch; k0 += 16) {
        float4 v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int c = (k0 + u) * 64 + lane;
            v[u] = c < nch ? *(const float4 *)(xt + 4 * c) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            if ((k0 + u) * 64 + lane < nch) {
                acc = __builtin_fmaf(v[u].x, v[u].x, acc);
                acc = __builtin_fmaf(v[u].y, v[u].y, acc);
                acc = __builtin_fmaf(v[u].z, v[u].z, acc);
                acc = __builtin_fmaf(v[u].w, v[u].w, acc);
            }
        }
    }
    const float ss = wave_tree_sum(acc);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    for (int c = lane; c < nch; c += 64) {
        float4 v = *(const float4 *)(xt + 4 * c);
        v.x *= r; v.y *= r; v.z *= r; v.w *= r;
        *(float4 *)(xhat + (size_t)t * d + 4 * c) = v;
    }
}

// ---------------------------------------------------------------------------
// row dot products in the fixed order: gate (+up), dense gate-up, dense down
// ---------------------------------------------------------------------------
struct RowDotArgs {
    const uint8_t *w0;
    const uint16_t *s0;
    const uint8_t *w1;
    const uint16_t *s1;
    int rows, cols, B;
    const float *x;      // [B][cols]
    float *o0;           // G / H / out, [B][rows]
    float *o1;           // U, [B][rows]
    const float *resid;  // [B][rows] or null
    int mode, act;
    float bias, theta;
    int *list_cnt, *list_idx;
    const double *wdn;   // top-k: ||W_down[:, j]||_2
    uint64_t *keys;      // top-k: fp64 score keys [B][rows] (null: not computed)
};

__device__ __forceinline__ uint64_t topk_key(float g, float u, double n);

template <int WT, int BT, int OUT>
__global__ __launch_bounds__((RdCfg<WT, BT, OUT>::NW * 64)) void k_rowdot(const RowDotArgs a)
{
    using C = Cfg<WT, BT>;
    constexpr int E = C::E, KMAX = C::KMAX, NW = RdCfg<WT, BT, OUT>::NW;
    constexpr bool TWO = (OUT == OUT_GATE_UP || OUT == OUT_DENSE_GU);
    constexpr int RPW = RdCfg<WT, BT, OUT>::RPW;
    constexpr int R = NW * RPW;
    constexpr int SL = KMAX * 64 * E;  // floats per token per slice
    __shared__ __align__(16) float xs[BT * SL];
    __shared__ int flags[R];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row_base = blockIdx.x * R;
    const int rowA = row_base + wave * RPW;
    const int nch = a.cols / E;
    const int K = (nch + 63) >> 6;
    const size_t rb = (WT == SFFN_W_F32) ? (size_t)a.cols * 4 : (WT == SFFN_W_BF16) ? (size_t)a.cols * 2 : (size_t)a.cols / 2;
    const int sst = a.cols / 128;
    const int B = a.B;

    float ag[BT][RPW], au[BT][RPW];
#pragma unroll
    for (int t = 0; t < BT; ++t)
#pragma unroll
        for (int r = 0; r < RPW; ++r) ag[t][r] = au[t][r] = 0.0f;

    for (int k0 = 0; k0 < K; k0 += KMAX) {
        const int e0 = k0 * 64 * E;
        const int ne = min(SL, a.cols - e0);
        const int n4 = ne >> 2;

        // weight loads first: they stay in flight while x is staged
        uint4 w0v[KMAX][RPW], w1v[TWO ? KMAX : 1][TWO ? RPW : 1];
        float s0v[KMAX][RPW], s1v[TWO ? KMAX : 1][TWO ? RPW : 1];
#pragma unroll
        for (int kk = 0; kk < KMAX; ++kk) {
            const int c = (k0 + kk) * 64 + lane;
            const bool ok = (k0 + kk < K) && (c < nch);
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                const int row = rowA + r;
                w0v[kk][r] = make_uint4(0, 0, 0, 0);
                s0v[kk][r] = 0.0f;
                if constexpr (TWO) { w1v[kk][r] = make_uint4(0, 0, 0, 0); s1v[kk][r] = 0.0f; }
                if (ok && row < a.rows) {
                    w0v[kk][r] = ld16_nt(a.w0 + (size_t)row * rb + (size_t)c * 16);
                    if constexpr (WT == SFFN_W_INT4_G128) s0v[kk][r] = half_bits_to_float(a.s0[(size_t)row * sst + (c >> 2)]);
                    if constexpr (TWO) {
                        w1v[kk][r] = ld16_nt(a.w1 + (size_t)row * rb + (size_t)c * 16);
                        if constexpr (WT == SFFN_W_INT4_G128) s1v[kk][r] = half_bits_to_float(a.s1[(size_t)row * sst + (c >> 2)]);
                    }
                }
            }
        }

        // x slice in LDS as [token][chunk column][E/4][lane] float4s: lane l of a
        // wave reads consecutive 16-byte words (no bank conflicts)
        __syncthreads();
        for (int i = threadIdx.x; i < B * n4; i += NW * 64) {
            const int t = i / n4, c4 = i - t * n4;
            const int q = 4 * c4, cl = q / E, e4 = (q - cl * E) >> 2;
            const int kk = cl >> 6, ln = cl & 63;
            *(float4 *)&xs[t * SL + ((kk * (E / 4) + e4) * 64 + ln) * 4] =
                *(const float4 *)&a.x[(size_t)t * a.cols + e0 + q];
        }
        __syncthreads();

#pragma unroll
        for (int kk = 0; kk < KMAX; ++kk) {
            const int c = (k0 + kk) * 64 + lane;
            if ((k0 + kk < K) && (c < nch)) {
#pragma unroll
                for (int t = 0; t < BT; ++t) {
                    if (t < B) {
                        float xv[E];
#pragma unroll
                        for (int e4 = 0; e4 < E / 4; ++e4) {
                            const float4 v = *(const float4 *)&xs[t * SL + ((kk * (E / 4) + e4) * 64 + lane) * 4];
                            xv[4 * e4 + 0] = v.x; xv[4 * e4 + 1] = v.y;
                            xv[4 * e4 + 2] = v.z; xv[4 * e4 + 3] = v.w;
                        }
#pragma unroll
                        for (int r = 0; r < RPW; ++r) {
                            ag[t][r] = chunk_dot<WT>(w0v[kk][r], s0v[kk][r], xv, ag[t][r]);
                            if constexpr (TWO) au[t][r] = chunk_dot<WT>(w1v[kk][r], s1v[kk][r], xv, au[t][r]);
                        }
                    }
                }
            }
        }
    }

#pragma unroll
    for (int t = 0; t < BT; ++t) {
        if (t < B) {
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                ag[t][r] = wave_tree_sum(ag[t][r]);
                if constexpr (TWO) au[t][r] = wave_tree_sum(au[t][r]);
            }
        }
    }

    if constexpr (OUT == OUT_GATE_UP) {
        // top-k score keys, one (row, token) per lane (every lane holds the sums)
        if (a.keys && lane < RPW * BT) {
            const int r = lane / BT, t = lane - r * BT, row = rowA + r;
            float gs = 0.0f, us = 0.0f;
#pragma unroll
            for (int rr = 0; rr < RPW; ++rr)
#pragma unroll
                for (int tt = 0; tt < BT; ++tt)
                    if (rr == r && tt == t) { gs = ag[tt][rr]; us = au[tt][rr]; }
            if (t < B && row < a.rows) a.keys[(size_t)t * a.rows + row] = topk_key(gs + a.bias, us, a.wdn[row]);
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int r = 0; r < RPW; ++r) {
            const int row = rowA + r;
            int on = 0;
            if (row < a.rows) {
#pragma unroll
                for (int t = 0; t < BT; ++t) {
                    if (t < B) {
                        const size_t o = (size_t)t * a.rows + row;
                        if constexpr (OUT == OUT_GATE || OUT == OUT_GATE_UP) {
                            const float gp = ag[t][r] + a.bias;
                            a.o0[o] = gp;
                            if constexpr (OUT == OUT_GATE_UP) a.o1[o] = au[t][r];
                            on |= gate_pred(a.mode, gp, a.theta) ? 1 : 0;
                        } else if constexpr (OUT == OUT_DENSE_GU) {
                            a.o0[o] = act_f32(a.act, ag[t][r] + a.bias) * au[t][r];
                        } else {
                            a.o0[o] = a.resid ? ag[t][r] + a.resid[o] : ag[t][r];
                        }
                    }
                }
            }
            if constexpr (OUT == OUT_GATE) flags[wave * RPW + r] = on;
        }
    }
    if constexpr (OUT == OUT_GATE) {
        // ascending compaction of this workgroup's rows: ballot + mbcnt, no atomics
        __syncthreads();
        if (wave == 0 && a.list_cnt) {
            const int on = lane < R ? flags[lane] : 0;
            const uint64_t m = __ballot(on);
            if (on) a.list_idx[(size_t)blockIdx.x * R + mbcnt64(m)] = row_base + lane;
            if (lane == 0) a.list_cnt[blockIdx.x] = __popcll(m);
        }
    }
}

// ---------------------------------------------------------------------------
// weight-aware top-k (one workgroup per token)
// ---------------------------------------------------------------------------

// fp64 exp: Cody-Waite reduction by ln2 (head/tail split) and a degree-13 Taylor
// polynomial in Horner form with fused multiply-adds, scaled by 2^n
// (W. J. Cody and W. Waite, Software Manual for the Elementary Functions).
// Written so that every step is one IEEE operation; the CPU reference
// implements the same published method independently.
__device__ double exp64(double z)
{
    if (z > 709.0) return __builtin_huge_val();
    if (z < -745.0) return 0.0;
    const double log2e = 0x1.71547652b82fep+0;
    const double ln2_hi = 0x1.62e42feep-1;
    const double ln2_lo = 0x1.a39ef35793c76p-33;
    const double c[14] = {0x1.0000000000000p+0,  0x1.0000000000000p+0,  0x1.0000000000000p-1,
                          0x1.5555555555555p-3,  0x1.5555555555555p-5,  0x1.1111111111111p-7,
                          0x1.6c16c16c16c17p-10, 0x1.a01a01a01a01ap-13, 0x1.a01a01a01a01ap-16,
                          0x1.71de3a556c734p-19, 0x1.27e4fb7789f5cp-22, 0x1.ae64567f544e4p-26,
                          0x1.1eed8eff8d898p-29, 0x1.6124613a86d09p-33};
    const double n = rint(z * log2e);
    double r = fma(-n, ln2_hi, z);
    r = fma(-n, ln2_lo, r);
    double p = c[13];
#pragma unroll
    for (int k = 12; k >= 0; --k) p = fma(p, r, c[k]);
    return ldexp(p, (int)n);
}

__device__ __forceinline__ uint64_t topk_key(float g, float u, double n)
{
    const double gd = (double)g;
    const double silu = gd / (1.0 + exp64(-gd));
    const double s = fabs(silu * (double)u) * n;  // >= 0: the bits order like the values
    return (uint64_t)__double_as_longlong(s);
}

struct TopkArgs {
    int f, k, nw32;
    const uint64_t *keys;   // [B][f] fp64 score keys (written by the gate / up kernel)
    uint32_t *bits;
};

// The exact top k of one token's f fp64 score keys (key = the bits of the
// non-negative score with bit 63 cleared, so the integer order is the value
// order), ties to the lower index, decided by the 1024 threads of a workgroup:
// thread tid holds keys j = tid + 1024 q.  Radix select from the top:
//   pass 0   the 11 exponent bits (key bits 62..52).  Scores spread over few
//            octaves, so lanes of one wave often share a digit; the histogram
//            is kept in kTopkSlots copies indexed by lane, which keeps such
//            lanes off one LDS word (their atomic adds would serialise)
//   pass 1   key bits 51..40 of the keys in the chosen exponent (high words)
//   then     12-bit digits 39..28, 27..16, 15..4 and bits 3..0.
// Each pass counts the keys that share the digits chosen so far, and a block
// scan in descending digit order finds the digit of the k-th key; keys in
// higher digits are kept.  It stops as soon as the chosen bin is kept whole,
// or holds at most kTopkCand keys: those are ranked exactly by (key desc,
// index asc), sixteen threads per candidate, and the k-th names the threshold
// (key, index) that every thread compares its keys with.  Only a bin of more
// than kTopkCand equal keys is resolved by an index-order scan.
// Returns the thread's decisions: bit q set = key q kept.
constexpr int kTopkCand = 64;    // at most this many keys left in the chosen bin: rank them exactly
constexpr int kTopkSlots = 4;    // copies of the first pass's histogram, one per lane & (kTopkSlots - 1)

struct TopkLds {
    uint32_t h0[2048 * kTopkSlots];   // pass 0: (key bits 62..52) * kTopkSlots + lane slot
    uint32_t hist[2][4096];           // later passes (12-bit digits), alternating
    int wsum[16];
    int s_digit, s_above, s_cnt, s_ncand, s_tidx;
    uint64_t s_tkey;
    uint64_t ckey[kTopkCand];
    int cidx[kTopkCand];
};

constexpr int kTopkPer = kMaxTopkNeurons / 1024;   // keys per thread

// block scan of per-thread bin counts given in descending digit order (c[0] the
// highest digit of the thread, digits hi0 - e): finds the digit holding the
// kk-th key, the keys above it and its count, in L.s_digit / s_above / s_cnt
template <int E>
__device__ __forceinline__ void topk_scan_pick(const int (&c)[E], int hi0, int kk, TopkLds &L)
{
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    int cs = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) cs += c[e];
    int incl = wave_incl_scan(cs);
    if (lane == 63) L.wsum[wave] = incl;
    __syncthreads();
#pragma unroll
    for (int w2 = 0; w2 < 16; ++w2) incl += w2 < wave ? L.wsum[w2] : 0;
    int above = incl - cs;
    if (above < kk && kk <= incl) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if (above < kk && kk <= above + c[e]) {
                L.s_digit = hi0 - e;
                L.s_above = above;
                L.s_cnt = c[e];
            }
            above += c[e];
        }
    }
    __syncthreads();
}

__device__ uint32_t topk_decide(const uint64_t (&kv)[kTopkPer], int f, int k, TopkLds &L)
{
    constexpr int PER = kTopkPer, NT = 1024;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const uint4 zero = {0u, 0u, 0u, 0u};
    for (int i = tid; i < (int)sizeof(L.h0) / 16; i += NT) ((uint4 *)L.h0)[i] = zero;
    __syncthreads();
    // pass 0, and meanwhile the later passes' counters are cleared
    const int slot = lane & (kTopkSlots - 1);
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        if (q * NT >= f) break;   // uniform
        const int j = tid + NT * q;
        if (j < f) atomicAdd(&L.h0[(int)(kv[q] >> 52) * kTopkSlots + slot], 1u);
    }
    for (int i = tid; i < (int)sizeof(L.hist) / 16; i += NT) ((uint4 *)L.hist)[i] = zero;
    if (tid == 0) L.s_ncand = 0;
    __syncthreads();
    int kk = k;
    {
        // thread tid: digits 2047 - 2 tid and 2046 - 2 tid, 2 kTopkSlots consecutive words
        const uint4 *r = (const uint4 *)&L.h0[(2046 - 2 * tid) * kTopkSlots];
        int c2[2] = {0, 0};
#pragma unroll
        for (int i = 0; i < kTopkSlots / 4; ++i) {
            const uint4 lo = r[i], hi = r[kTopkSlots / 4 + i];
            c2[1] += (int)(lo.x + lo.y + lo.z + lo.w);
            c2[0] += (int)(hi.x + hi.y + hi.z + hi.w);
        }
        topk_scan_pick<2>(c2, 2047 - 2 * tid, kk, L);
    }
    kk -= L.s_above;
    const uint32_t d0 = (uint32_t)L.s_digit;
    uint64_t prefix = (uint64_t)d0 << 52, pmask = 0xFFFull << 52;
    int mode = 3;   // 1: keep the chosen bin whole, 2: rank the candidates, 3: equal keys by index
    int cnt = L.s_cnt;
    if (cnt == kk) mode = 1;
    else if (cnt <= kTopkCand) mode = 2;
    if (mode == 3) {
        // pass 1 on the high words: exponent d0, digit = key bits 51..40
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            if (q * NT >= f) break;
            const int j = tid + NT * q;
            const uint32_t hw = (uint32_t)(kv[q] >> 32);
            if (j < f && (hw >> 20) == d0) atomicAdd(&L.hist[1][(hw >> 8) & 0xFFFu], 1u);
        }
        __syncthreads();
        {
            int c4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int dg = 4095 - (4 * tid + e);
                c4[e] = (int)L.hist[1][dg];
                L.hist[1][dg] = 0;   // clear for pass 3
            }
            topk_scan_pick<4>(c4, 4095 - 4 * tid, kk, L);
        }
        kk -= L.s_above;
        prefix |= (uint64_t)L.s_digit << 40;
        pmask |= 0xFFFull << 40;
        cnt = L.s_cnt;
        if (cnt == kk) mode = 1;
        else if (cnt <= kTopkCand) mode = 2;
    }
    for (int pass = 2; pass < 6 && mode == 3; ++pass) {
        // rare: more than kTopkCand keys share the top 24 bits
        const int width = pass < 5 ? 12 : 4;
        const int shift = pass < 5 ? 52 - 12 * pass : 0;
        const int nb = 1 << width;
        uint32_t *h = L.hist[pass & 1];
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            if (q * NT >= f) break;
            const int j = tid + NT * q;
            if (j < f && (kv[q] & pmask) == prefix) atomicAdd(&h[(int)(kv[q] >> shift) & (nb - 1)], 1u);
        }
        __syncthreads();
        // thread tid owns digits nb-1-4tid .. nb-4-4tid (descending) and clears
        // them for the pass after next
        int c4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int dg = nb - 1 - (4 * tid + e);
            c4[e] = 0;
            if (dg >= 0) {
                c4[e] = (int)h[dg];
                h[dg] = 0;
            }
        }
        topk_scan_pick<4>(c4, nb - 1 - 4 * tid, kk, L);
        kk -= L.s_above;   // still to keep from the chosen bin
        prefix |= (uint64_t)L.s_digit << shift;
        pmask |= (uint64_t)(nb - 1) << shift;
        cnt = L.s_cnt;
        if (cnt == kk) mode = 1;            // uniform
        else if (cnt <= kTopkCand) mode = 2;
    }
    uint32_t dm = 0;
    if (mode == 2) {
        // the candidates (keys of the chosen bin, at most kTopkCand) into LDS,
        // ranked by (key desc, index asc); the kk-th is the threshold (tkey, tidx)
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            if (q * NT >= f) break;
            const int j = tid + NT * q;
            const bool c = j < f && (kv[q] & pmask) == prefix;
            const uint64_t m = __ballot(c);
            if (m == 0) continue;   // uniform in the wave
            int base = 0;
            if (lane == 0) base = atomicAdd(&L.s_ncand, __popcll(m));
            base = __shfl(base, 0, 64);
            if (c) {
                const int pos = base + mbcnt64(m);
                L.ckey[pos] = kv[q];
                L.cidx[pos] = j;
            }
        }
        __syncthreads();
        {
            // sixteen threads per candidate, each a sixteenth of the comparisons
            const int nc = L.s_ncand;
            const int ci = tid >> 4, part = tid & 15;
            uint64_t my = 0;
            int mi = 0, r = 0;
            if (ci < nc) {
                my = L.ckey[ci];
                mi = L.cidx[ci];
                for (int i = part; i < nc; i += 16) {
                    const uint64_t o = L.ckey[i];
                    r += (o > my || (o == my && L.cidx[i] < mi)) ? 1 : 0;
                }
            }
            r += __shfl_xor(r, 1, 64);
            r += __shfl_xor(r, 2, 64);
            r += __shfl_xor(r, 4, 64);
            r += __shfl_xor(r, 8, 64);
            if (part == 0 && ci < nc && r == kk - 1) {
                L.s_tkey = my;
                L.s_tidx = mi;
            }
        }
        __syncthreads();
        const uint64_t tk = L.s_tkey;
        const int ti = L.s_tidx;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            if (q * NT >= f) break;   // uniform
            const int j = tid + NT * q;
            const bool on = j < f && (kv[q] > tk || (kv[q] == tk && j <= ti));
            dm |= on ? (1u << q) : 0u;
        }
        return dm;
    }
    if (mode == 1 && (uint32_t)pmask == 0u) {
        // the kept bin is a prefix of the high words
        const uint32_t ph = (uint32_t)(prefix >> 32), mh = (uint32_t)(pmask >> 32);
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            if (q * NT >= f) break;   // uniform
            const int j = tid + NT * q;
            const bool on = j < f && ((uint32_t)(kv[q] >> 32) & mh) >= ph;
            dm |= on ? (1u << q) : 0u;
        }
        return dm;
    }
    int base_rank = 0;   // equal keys before this round (index order), mode 3 only
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        if (q * NT >= f) break;   // uniform
        const int j = tid + NT * q;
        const uint64_t v = kv[q] & pmask;
        bool on;
        if (mode == 1) {
            on = j < f && v >= prefix;
        } else {
            // more than kTopkCand keys equal to the threshold: the lowest indices
            const bool tie = j < f && v == prefix;
            const uint64_t tm = __ballot(tie);
            if (lane == 0) L.wsum[wave] = __popcll(tm);
            __syncthreads();
            int off = 0, tot = 0;
            for (int w2 = 0; w2 < 16; ++w2) {
                const int c2 = L.wsum[w2];
                off += w2 < wave ? c2 : 0;
                tot += c2;
            }
            const int below = __popcll(tm & ((1ull << lane) - 1ull));
            on = j < f && (v > prefix || (tie && base_rank + off + below < kk));
            base_rank += tot;
            __syncthreads();
        }
        dm |= on ? (1u << q) : 0u;
    }
    return dm;
}

// Every load is issued before any is used (the index is clamped instead of the
// load made conditional, which would make each load wait for the previous
// one); keys past f are never counted.  Bit 63 is cleared afterwards.
__device__ __forceinline__ void load_token_keys(uint64_t (&kv)[kTopkPer], const uint64_t *keys, int f)
{
#pragma unroll
    for (int q = 0; q < kTopkPer; ++q) kv[q] = keys[min((int)threadIdx.x + 1024 * q, f - 1)];
#pragma unroll
    for (int q = 0; q < kTopkPer; ++q) kv[q] &= 0x7FFFFFFFFFFFFFFFull;
}

// One workgroup per token: the token's selection as bit words (key j in bit
// j % 64 of 64-bit word j / 64; f is a multiple of 64)
__global__ __launch_bounds__(1024) void k_topk(const TopkArgs a)
{
    __shared__ TopkLds L;
    const int t = blockIdx.x, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    uint64_t kv[kTopkPer];
    load_token_keys(kv, a.keys + (size_t)t * a.f, a.f);
    const uint32_t dm = topk_decide(kv, a.f, a.k, L);
    uint64_t *bits = (uint64_t *)(a.bits + (size_t)t * a.nw32);
#pragma unroll
    for (int q = 0; q < kTopkPer; ++q) {
        if (q * 1024 >= a.f) break;   // uniform
        const uint64_t m = __ballot((dm >> q) & 1u);
        if (lane == 0 && q * 1024 + 64 * wave < a.f) bits[16 * q + wave] = m;
    }
}

// ---------------------------------------------------------------------------
// gather: the active list in equal shares -> partial y
// ---------------------------------------------------------------------------
struct GatherArgs {
    const int *list_cnt, *list_idx;
    int nL, R;
    const float *G, *U;
    const uint32_t *bits;
    int nw32;
    const float *x;
    int B, d, f;
    const uint8_t *wu;
    const uint16_t *su;
    const uint8_t *wdt;
    const uint16_t *sdt;
    int mode, act, use_union;
    float theta;
    float *partial;  // [P][B][d]
    int32_t *idx_out, *count_out;
    int maxs;        // capacity of the share arrays
    int stage_x;     // 1: the up projection runs here (x slices in LDS)
    const int *path; // run only when *path == want (nullptr: always)
    int want;
    int share_bits;  // top-k: 1 = equal shares of the union's ascending list (from the bit words),
                     // 2 = workgroup q owns the neurons [q R, q R + R), R = ceil(f / P) <= 64
    int merge_gap;   // share 2: also read the unselected neurons of gaps of at most this many rows
    int P;           // workgroups (partitions of the share, partial sums); 0: kGatherWGs
};

// Top-k share by neuron range: wave 0 of workgroup q takes the neurons
// [q R, q R + R) in chunks of 64 (one per lane), loads each one's bit words, g'
// and u for every token (the loads of all chunks are issued before the first
// use), forms h = act(g') u for the tokens whose set holds the neuron (all
// tokens with the union rule) and compacts the neurons of the union into
// jl / hs in ascending order (ballot + mbcnt).  Returns the number of neurons
// (all threads).
template <int BT>
__device__ int share_of_range(const GatherArgs &a, int R, int *jl, float *hs, int *s_ns)
{
    constexpr int MAXC = BT == 1 ? 8 : 1;   // chunks of 64 neurons: R <= 512 at batch 1, else <= 64
    const int lane = threadIdx.x & 63;
    if (threadIdx.x < 64) {
        uint32_t wb[MAXC][BT];
        float gv[MAXC][BT], uv[MAXC][BT];
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
            const int j = blockIdx.x * R + 64 * c + lane;
            const bool in = 64 * c + lane < R && j < a.f;
            const int jc = in ? j : 0;
#pragma unroll
            for (int t = 0; t < BT; ++t) {
                const int tc = min(t, a.B - 1);
                wb[c][t] = 0u;
                gv[c][t] = 0.0f;
                uv[c][t] = 0.0f;
                if (64 * c < R) {
                    wb[c][t] = a.bits[(size_t)tc * a.nw32 + (jc >> 5)];
                    gv[c][t] = a.G[(size_t)tc * a.f + jc];
                    uv[c][t] = a.U[(size_t)tc * a.f + jc];
                }
            }
        }
        int base = 0;
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
            if (64 * c >= R) break;
            const int j = blockIdx.x * R + 64 * c + lane;
            const bool in = 64 * c + lane < R && j < a.f;
            uint32_t tb = 0;       // bit t: neuron j is in token t's set
            float h[BT];
#pragma unroll
            for (int t = 0; t < BT; ++t) {
                h[t] = 0.0f;
                if (in && t < a.B) {
                    if ((wb[c][t] >> (j & 31)) & 1u) tb |= 1u << t;
                    h[t] = act_f32(a.act, gv[c][t]) * uv[c][t];
                }
            }
            const bool on = tb != 0;
            const uint64_t sel = __ballot(on);
            // run merging: an unselected neuron whose gap between the selected
            // neighbours on either side (within its chunk) is at most merge_gap
            // rows is read as well
            bool rd = on;
            if (a.merge_gap > 0 && !on && in) {
                const uint64_t below = sel & ((1ull << lane) - 1ull), above = lane < 63 ? sel >> (lane + 1) : 0ull;
                if (below && above) {
                    const int prev = 63 - __builtin_clzll(below), next = lane + 1 + __builtin_ctzll(above);
                    rd = next - prev - 1 <= a.merge_gap;
                }
            }
            const uint64_t m = __ballot(rd);
            if (rd) {
                const int pos = base + mbcnt64(m);
                jl[pos] = j;
#pragma unroll
                for (int t = 0; t < BT; ++t)
                    if (t < a.B) hs[pos * BT + t] = (on && (a.use_union || ((tb >> t) & 1u))) ? h[t] : 0.0f;
            }
            base += __popcll(m);
        }
        if (lane == 0) *s_ns = base;
    }
    __syncthreads();
    return *s_ns;
}

// Share of the union of the tokens' top-k bit words for this workgroup: the
// selected neurons in ascending order are cut into gridDim.x equal shares;
// writes this share's neuron indices to jl (and to idx_out), returns their
// number.  pref needs nw32 + 1 ints.
__device__ int share_of_bits(const uint32_t *bits, int nw32, int B, int *pref, int *jl, int32_t *idx_out,
                             int32_t *count_out, int *tmp)
{
    const int NT = blockDim.x, tid = threadIdx.x;
    auto word = [&](int w) {
        uint32_t u = 0;
        for (int t = 0; t < B; ++t) u |= bits[(size_t)t * nw32 + w];
        return u;
    };
    const int per = (nw32 + NT - 1) / NT;
    const int w0 = min(nw32, tid * per), w1 = min(nw32, w0 + per);
    int s = 0;
    for (int w = w0; w < w1; ++w) s += __popc(word(w));
    int total;
    int run = block_exclusive_scan(s, tmp, &total);
    for (int w = w0; w < w1; ++w) {
        pref[w] = run;
        run += __popc(word(w));
    }
    if (tid == 0) pref[nw32] = total;
    __syncthreads();
    const int P = gridDim.x, q = blockIdx.x;
    const int lo = (int)((int64_t)q * total / P), hi = (int)((int64_t)(q + 1) * total / P);
    for (int p = lo + tid; p < hi; p += NT) {
        int a = 0, b = nw32 - 1;   // the last word whose prefix is <= p
        while (a < b) {
            const int mid = (a + b + 1) >> 1;
            if (pref[mid] <= p) a = mid; else b = mid - 1;
        }
        uint32_t u = word(a);
        for (int r = p - pref[a]; r > 0; --r) u &= u - 1u;   // drop the lower set bits
        const int j = 32 * a + __builtin_ctz(u);
        jl[p - lo] = j;
        if (idx_out) idx_out[p] = j;
    }
    if (q == 0 && tid == 0 && count_out) *count_out = total;
    __syncthreads();
    return hi - lo;
}

// Share of the concatenated per-block lists for this workgroup: writes the
// neuron indices to jl[0..ns) (and to idx_out), returns ns.  pref needs nL+1 ints.
__device__ int share_of_lists(const int *cnt, const int *idx, int nL, int R, int *pref, int *jl,
                              int32_t *idx_out, int32_t *count_out, int *tmp)
{
    const int NT = blockDim.x, tid = threadIdx.x;
    const int per = (nL + NT - 1) / NT;
    const int i0 = min(nL, tid * per), i1 = min(nL, i0 + per);
    int s = 0;
    for (int i = i0; i < i1; ++i) s += cnt[i];
    int total;
    int run = block_exclusive_scan(s, tmp, &total);
    for (int i = i0; i < i1; ++i) {
        pref[i] = run;
        run += cnt[i];
    }
    if (tid == 0) pref[nL] = total;
    __syncthreads();
    const int P = gridDim.x, q = blockIdx.x;
    const int lo = (int)((int64_t)q * total / P), hi = (int)((int64_t)(q + 1) * total / P);
    for (int p = lo + tid; p < hi; p += NT) {
        int a = 0, b = nL - 1;
        while (a < b) {
            const int mid = (a + b + 1) >> 1;
            if (pref[mid] <= p) a = mid; else b = mid - 1;
        }
        const int j = idx[(size_t)a * R + (p - pref[a])];
        jl[p - lo] = j;
        if (idx_out) idx_out[p] = j;
    }
    if (q == 0 && tid == 0 && count_out) *count_out = total;
    __syncthreads();
    return hi - lo;
}

// the ascending list of the selected union (select calls): from the per-block
// lists, or (bits != nullptr) from the tokens' top-k bit words
__global__ __launch_bounds__(256) void k_emit_list(const int *cnt, const int *idx, int nL, int R,
                                                   int32_t *idx_out, int32_t *count_out, int maxs,
                                                   const uint32_t *bits, int B)
{
    extern __shared__ __align__(16) int lds_e[];
    __shared__ int tmp[17];
    int *jl = lds_e, *pref = lds_e + maxs;
    if (bits)
        share_of_bits(bits, nL, B, pref, jl, idx_out, count_out, tmp);
    else
        share_of_lists(cnt, idx, nL, R, pref, jl, idx_out, count_out, tmp);
}

template <int WT, int BT>
__global__ __launch_bounds__((Cfg<WT, BT>::NW * 64)) void k_gather(const GatherArgs a)
{
    using C = Cfg<WT, BT>;
    constexpr int E = C::E, KMAX = C::KMAX, NW = C::NW, RPW = C::RPW, CPT = C::CPT, UNR = C::UNR;
    constexpr int NT = NW * 64;
    constexpr int R2 = NW * RPW;
    constexpr int SL = KMAX * 64 * E;
    extern __shared__ __align__(16) unsigned char lds[];
    float *xs = (float *)lds;
    float *hs = xs + (a.stage_x ? BT * SL : 0);
    int *jl = (int *)(hs + (size_t)a.maxs * BT);
    int *pref = jl + a.maxs;
    __shared__ int tmp[17];

    if (a.path && *a.path != a.want) return;   // uniform, before any barrier
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int B = a.B, d = a.d, f = a.f;
    __shared__ int s_ns;
    const int ns = a.share_bits == 2 ? share_of_range<BT>(a, a.R, jl, hs, &s_ns)
                   : a.share_bits ? share_of_bits(a.bits, a.nL, B, pref, jl, a.idx_out, a.count_out, tmp)
                                  : share_of_lists(a.list_cnt, a.list_idx, a.nL, a.R, pref, jl, a.idx_out, a.count_out,
                                                   tmp);

    // ---- phase A: h_tj for the share ----
    if (a.share_bits == 2) {
        // formed with the share
    } else if (a.mode == SFFN_MODE_TOPK) {
        for (int i = tid; i < ns * B; i += NT) {
            const int jj = i / B, t = i - jj * B, j = jl[jj];
            const float gp = a.G[(size_t)t * f + j];
            const bool on = a.use_union || ((a.bits[(size_t)t * a.nw32 + (j >> 5)] >> (j & 31)) & 1);
            hs[jj * BT + t] = on ? act_f32(a.act, gp) * a.U[(size_t)t * f + j] : 0.0f;
        }
    } else {
        const int nch = d / E, K = (nch + 63) >> 6;
        const size_t rb = (WT == SFFN_W_F32) ? (size_t)d * 4 : (WT == SFFN_W_BF16) ? (size_t)d * 2 : (size_t)d / 2;
        const int sst = d / 128;
        const int ngroups = (ns + R2 - 1) / R2;
        const bool single = K <= KMAX;
        for (int gi = 0; gi < ngroups; ++gi) {
            float au[BT][RPW];
#pragma unroll
            for (int t = 0; t < BT; ++t)
#pragma unroll
                for (int r = 0; r < RPW; ++r) au[t][r] = 0.0f;
            int jrow[RPW];
#pragma unroll
            for (int r = 0; r < RPW; ++r) {
                const int jj = gi * R2 + wave * RPW + r;
                jrow[r] = jj < ns ? jl[jj] : -1;
            }
            for (int k0 = 0; k0 < K; k0 += KMAX) {
                if (!single || gi == 0) {
                    const int e0 = k0 * 64 * E;
                    const int n4 = min(SL, d - e0) >> 2;
                    __syncthreads();
                    for (int i = tid; i < B * n4; i += NT) {
                        const int t = i / n4, c4 = i - t * n4;
                        *(float4 *)&xs[t * SL + 4 * c4] = *(const float4 *)&a.x[(size_t)t * d + e0 + 4 * c4];
                    }
                    __syncthreads();
                }
                uint4 wv[KMAX][RPW];
                float sv[KMAX][RPW];
#pragma unroll
                for (int kk = 0; kk < KMAX; ++kk) {
                    const int c = (k0 + kk) * 64 + lane;
                    const bool ok = (k0 + kk < K) && (c < nch);
#pragma unroll
                    for (int r = 0; r < RPW; ++r) {
                        wv[kk][r] = make_uint4(0, 0, 0, 0);
                        sv[kk][r] = 0.0f;
                        if (ok && jrow[r] >= 0) {
                            wv[kk][r] = ld16_nt(a.wu + (size_t)jrow[r] * rb + (size_t)c * 16);
                            if constexpr (WT == SFFN_W_INT4_G128) sv[kk][r] = half_bits_to_float(a.su[(size_t)jrow[r] * sst + (c >> 2)]);
                        }
                    }
                }
#pragma unroll
                for (int kk = 0; kk < KMAX; ++kk) {
                    const int c = (k0 + kk) * 64 + lane;
                    if ((k0 + kk < K) && (c < nch)) {
#pragma unroll
                        for (int t = 0; t < BT; ++t) {
                            if (t < B) {
                                float xv[E];
                                const float4 *xp = (const float4 *)&xs[t * SL + kk * 64 * E + lane * E];
#pragma unroll
                                for (int e4 = 0; e4 < E / 4; ++e4) {
                                    const float4 v = xp[e4];
                                    xv[4 * e4 + 0] = v.x; xv[4 * e4 + 1] = v.y;
                                    xv[4 * e4 + 2] = v.z; xv[4 * e4 + 3] = v.w;
                                }
#pragma unroll
                                for (int r = 0; r < RPW; ++r) au[t][r] = chunk_dot<WT>(wv[kk][r], sv[kk][r], xv, au[t][r]);
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int t = 0; t < BT; ++t)
                if (t < B)
#pragma unroll
                    for (int r = 0; r < RPW; ++r) au[t][r] = wave_tree_sum(au[t][r]);
            if (lane == 0) {
#pragma unroll
                for (int r = 0; r < RPW; ++r) {
                    if (jrow[r] < 0) continue;
                    const int jj = gi * R2 + wave * RPW + r;
#pragma unroll
                    for (int t = 0; t < BT; ++t) {
                        if (t < B) {
                            const float gp = a.G[(size_t)t * f + jrow[r]];
                            const bool on = a.use_union || gate_pred(a.mode, gp, a.theta);
                            hs[jj * BT + t] = on ? act_f32(a.act, gp) * au[t][r] : 0.0f;
                        }
                    }
                }
            }
        }
    }
    __syncthreads();

    // ---- phase B: partial y over the share's W_down^T rows ----
    float *part = a.partial + (size_t)blockIdx.x * B * d;
    for (int c0 = 0; c0 < d; c0 += NT * CPT) {
        const int col = c0 + tid * CPT;
        const bool okc = col < d;
        float acc[BT][CPT];
#pragma unroll
        for (int t = 0; t < BT; ++t)
#pragma unroll
            for (int c = 0; c < CPT; ++c) acc[t][c] = 0.0f;

        if constexpr (WT == SFFN_W_INT4_G128) {
            // y_i += h_j * (q_ji s[j/128][i]) with the exact dequantised weight
            // (a 4-bit integer times an fp16 scale is exact in fp32).  Rows come
            // in batches of UNR, two batches in flight; with each batch the
            // thread also loads the 8 scales of its columns for the groups of
            // the batch's first and last rows (one 16-byte load each), so a
            // group change never waits; a row in a third group (a union sparser
            // than 1 in 8) loads its scales itself.
            static_assert(CPT == 8, "one dword of nibbles and one 16-byte scale load per row");
            const size_t rbd = (size_t)d / 2;
            const uint8_t *wcol = a.wdt + col / 2;
            const uint16_t *scol = a.sdt + col;
            uint32_t qa[UNR], qb[UNR];
            uint4 sa0, sa1, sb0, sb1;
            int ga0 = 0, ga1 = 0, gb0 = 0, gb1 = 0;
            // rows past the share's end repeat its last row (loaded, never used)
#define SFFN_I4_LOAD(Q, S0, S1, G0, G1, jj0)                                                     \
    do {                                                                                         \
        const int last_ = min(ns, (jj0) + UNR) - 1;                                              \
        _Pragma("unroll") for (int u = 0; u < UNR; ++u)                                          \
            Q[u] = __builtin_nontemporal_load((const uint32_t *)(wcol + (size_t)jl[min((jj0) + u, last_)] * rbd)); \
        G0 = jl[(jj0)] >> 7;                                                                     \
        G1 = jl[last_] >> 7;                                                                     \
        S0 = ld16(scol + (size_t)G0 * d);                                                        \
        S1 = ld16(scol + (size_t)G1 * d);                                                        \
    } while (0)
#define SFFN_I4_RUN(Q, S0, S1, G0, G1, jj0)                                                      \
    do {                                                                                         \
        const int n_ = min(UNR, ns - (jj0));                                                     \
        _Pragma("unroll") for (int u = 0; u < UNR; ++u) {                                        \
            if (u >= n_) break;                                                                  \
            const int g = jl[(jj0) + u] >> 7;                                                    \
            uint32_t s4[4] = {g == G0 ? S0.x : S1.x, g == G0 ? S0.y : S1.y,                      \
                              g == G0 ? S0.z : S1.z, g == G0 ? S0.w : S1.w};                     \
            if (g != G0 && g != G1) {                                                            \
                const uint4 t_ = ld16(scol + (size_t)g * d);                                     \
                s4[0] = t_.x; s4[1] = t_.y; s4[2] = t_.z; s4[3] = t_.w;                          \
            }                                                                                    \
            float w[8];                                                                          \
            _Pragma("unroll") for (int c = 0; c < 8; ++c)                                        \
                w[c] = (float)nib(Q[u], c) * half_bits_to_float((uint16_t)(s4[c >> 1] >> (16 * (c & 1)))); \
            _Pragma("unroll") for (int t = 0; t < BT; ++t) {                                     \
                if (t < B) {                                                                     \
                    const float h = hs[((jj0) + u) * BT + t];                                    \
                    _Pragma("unroll") for (int c = 0; c < 8; ++c)                                \
                        acc[t][c] = __builtin_fmaf(h, w[c], acc[t][c]);                          \
                }                                                                                \
            }                                                                                    \
        }                                                                                        \
    } while (0)
            if (okc && ns > 0) {
                SFFN_I4_LOAD(qa, sa0, sa1, ga0, ga1, 0);
                for (int jj0 = 0; jj0 < ns; jj0 += 2 * UNR) {
                    if (jj0 + UNR < ns) SFFN_I4_LOAD(qb, sb0, sb1, gb0, gb1, jj0 + UNR);
                    SFFN_I4_RUN(qa, sa0, sa1, ga0, ga1, jj0);
                    if (jj0 + UNR >= ns) break;
                    if (jj0 + 2 * UNR < ns) SFFN_I4_LOAD(qa, sa0, sa1, ga0, ga1, jj0 + 2 * UNR);
                    SFFN_I4_RUN(qb, sb0, sb1, gb0, gb1, jj0 + UNR);
                }
            }
#undef SFFN_I4_LOAD
#undef SFFN_I4_RUN
        } else {
            constexpr int EB = WT == SFFN_W_F32 ? 4 : 2;
            constexpr int NV = CPT * EB / 16;  // 16-byte loads per row per thread
            const size_t rbd = (size_t)d * EB;
            for (int jj0 = 0; jj0 < ns; jj0 += UNR) {
                uint4 wv[UNR][NV];
#pragma unroll
                for (int u = 0; u < UNR; ++u) {
                    const int jj = jj0 + u;
                    const bool ok = okc && jj < ns;
                    const int j = ok ? jl[jj] : 0;
#pragma unroll
                    for (int v = 0; v < NV; ++v)
                        wv[u][v] = ok ? ld16_nt(a.wdt + (size_t)j * rbd + (size_t)col * EB + 16 * v) : make_uint4(0, 0, 0, 0);
                }
#pragma unroll
                for (int u = 0; u < UNR; ++u) {
                    if (jj0 + u >= ns) break;
                    float w[CPT];
#pragma unroll
                    for (int v = 0; v < NV; ++v) unpack<WT>(wv[u][v], w + v * (16 / EB));
#pragma unroll
                    for (int t = 0; t < BT; ++t) {
                        if (t < B) {
                            const float h = hs[(jj0 + u) * BT + t];
#pragma unroll
                            for (int c = 0; c < CPT; ++c) acc[t][c] = __builtin_fmaf(h, w[c], acc[t][c]);
                        }
                    }
                }
            }
        }
        if (okc) {
#pragma unroll
            for (int t = 0; t < BT; ++t) {
                if (t < B) {
                    float *dst = part + (size_t)t * d + col;
#pragma unroll
                    for (int c = 0; c < CPT; c += 4)
                        *(float4 *)(dst + c) = make_float4(acc[t][c], acc[t][c + 1], acc[t][c + 2], acc[t][c + 3]);
                }
            }
        }
    }
}


// ---------------------------------------------------------------------------
// batched decode (5..16 tokens, bf16 weights): up and down on MFMA.
// The gate GEMV stays in the fixed fp32 order (it decides the selection); the
// up projection and the down projection only produce values, so they run on
// v_mfma_f32_16x16x32_bf16 with their fp32 operand split into bf16 hi + lo
// (x = hi + lo to about 2^-17 relative), two MFMAs per step, fp32 accumulate.
// W_up and W_down are read from copies stored as 16 x 32 operand tiles, so
// every load of a wave is one contiguous kilobyte; the activations use the
// same lane order ([cols/32][64 lanes][8], lane = (k-group << 4) | token).
//   k_split_x   x_hat [B][d] -> X_hi, X_lo in lane order (tokens >= B are 0)
//   k_up_tiled  one wave per 16 neurons (one gate block): u for the block's
//               rows, h = act(g') u for the selected (token, neuron) pairs and
//               0 elsewhere -> H_hi, H_lo in lane order over d_ff; blocks with
//               no selected neuron skip the weight stream
//   k_down_tiled one wave per (16 output columns, d_ff split): partial y of
//               H W_down^T over its share of d_ff (H is 0 outside the selection)
//   k_down_sum  fixed-order sum over the splits, plus the residual
// ---------------------------------------------------------------------------
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

__device__ __forceinline__ uint16_t bf16_rne_bits(float v)
{
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// one thread per lane slot of 8 values: (d/32) * 64 threads
// Union size -> forward path: the row gather when |U| * 1000 < thr * f, else
// the tiles.  Every workgroup that calls it computes the same value.
__device__ int pick_path(const int *__restrict__ list_cnt, int nL, int f, int thr)
{
    __shared__ int red[256];
    int s = 0;
    for (int i = threadIdx.x; i < nL; i += 256) s += list_cnt[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if ((int)threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
        __syncthreads();
    }
    return (long long)red[0] * 1000 < (long long)thr * f ? kPathGather : kPathTiled;
}

// x_hat as bf16 hi / lo in MFMA lane order.  With path != nullptr the path is
// picked here first (workgroup 0 stores it for the later kernels) and the
// split is skipped when the gather was picked.
__global__ __launch_bounds__(256) void k_split_x(const float *__restrict__ x, int B, int d, uint16_t *__restrict__ xh,
                                                 uint16_t *__restrict__ xl, const int *__restrict__ list_cnt, int nL,
                                                 int f, int thr, int *__restrict__ path)
{
    if (path) {
        const int pk = pick_path(list_cnt, nL, f, thr);
        if (blockIdx.x == 0 && threadIdx.x == 0) *path = pk;
        if (pk != kPathTiled) return;
    }
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= (d / 32) * 64) return;
    const int s = i >> 6, l = i & 63, n = l & 15;
    const int c = s * 32 + 8 * (l >> 4);
    uint16_t h[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float v = n < B ? x[(size_t)n * d + c + e] : 0.0f;
        h[e] = bf16_rne_bits(v);
        lo[e] = bf16_rne_bits(v - bf16_lo(h[e]));
    }
    uint4 ph, pl;
    __builtin_memcpy(&ph, h, 16);
    __builtin_memcpy(&pl, lo, 16);
    *(uint4 *)(xh + (size_t)i * 8) = ph;
    *(uint4 *)(xl + (size_t)i * 8) = pl;
}

struct UpTiledArgs {
    const uint16_t *wut;             // W_up tiles [f/16][d/32][64][8]
    const uint16_t *xh, *xl;         // [d/32][64][8]
    const float *G;                  // [B][f]
    const int *list_cnt, *list_idx;  // per gate block of 16 neurons
    int d, f, B, mode, act, use_union;
    float theta;
    uint16_t *hh, *hl;               // [f/32][64][8]
    const int *path;                 // run only when *path == want (nullptr: always)
    int want;
};

// One MFMA k-step group: U k-steps of the activation operand (bf16 hi / lo,
// lane order) loaded once and applied to NB weight tiles (NB x 16 rows), two
// MFMAs per tile and step.  w[b], xh, xl are already offset by lane * 8; step
// k is 512 elements further.  live[b] false skips tile b (uniform per wave).
template <int U, int NB>
__device__ __forceinline__ void mfma_group(const uint16_t *const (&w)[NB], const bool (&live)[NB],
                                           const uint16_t *__restrict__ xh, const uint16_t *__restrict__ xl, int k,
                                           int k1, f32x4_t (&acc)[NB])
{
    bf16x8_t bh[U], bl[U], av[U][NB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const bool ok = k + u < k1;
        const size_t o = (size_t)(k + u) * 512;
        const uint4 xa = ok ? *(const uint4 *)(xh + o) : make_uint4(0, 0, 0, 0);
        const uint4 xb = ok ? *(const uint4 *)(xl + o) : make_uint4(0, 0, 0, 0);
        __builtin_memcpy(&bh[u], &xa, 16);
        __builtin_memcpy(&bl[u], &xb, 16);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const uint4 wa = (ok && live[b]) ? ld16_nt(w[b] + o) : make_uint4(0, 0, 0, 0);
            __builtin_memcpy(&av[u][b], &wa, 16);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (live[b]) {
                acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u][b], bh[u], acc[b], 0, 0, 0);
                acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u][b], bl[u], acc[b], 0, 0, 0);
            }
        }
    }
}

// Up on the W_up tiles: a workgroup owns kUpBlocks consecutive blocks of 16
// neurons; its four waves split the k range in quarters and each streams the
// activation steps once for all of the workgroup's tiles (the activation
// operand is as large as a weight tile per step, so sharing it halves the
// bytes moved); the four partial tiles are added in LDS in wave order, then
// wave b forms h for block b.  Blocks with no selected neuron skip their weights.
constexpr int kUpBlocks = 2;

__global__ __launch_bounds__(256) void k_up_tiled(const UpTiledArgs a)
{
    if (a.path && *a.path != a.want) return;
    __shared__ f32x4_t part[4][kUpBlocks][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int t0 = blockIdx.x * kUpBlocks;
    const int KS = a.d / 32;
    const int k0 = (KS * w) / 4, k1 = (KS * (w + 1)) / 4;
    bool live[kUpBlocks];
    const uint16_t *wp[kUpBlocks];
    f32x4_t acc[kUpBlocks];
#pragma unroll
    for (int b = 0; b < kUpBlocks; ++b) {
        live[b] = a.list_cnt[t0 + b] > 0;
        wp[b] = a.wut + (size_t)(t0 + b) * KS * 512 + lane * 8;
        acc[b] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    for (int k = k0; k < k1; k += 4) mfma_group<4, kUpBlocks>(wp, live, a.xh + lane * 8, a.xl + lane * 8, k, k1, acc);
#pragma unroll
    for (int b = 0; b < kUpBlocks; ++b) part[w][b][lane] = acc[b];
    __syncthreads();
    const int t = t0 + w;   // wave w finishes block w
    if (w >= kUpBlocks) return;
    const f32x4_t s4 = ((part[0][w][lane] + part[1][w][lane]) + part[2][w][lane]) + part[3][w][lane];
    const int cnt = a.list_cnt[t];
    uint32_t m = 0;
    for (int s2 = 0; s2 < cnt; ++s2) m |= 1u << (a.list_idx[t * 16 + s2] - t * 16);
    // C[neuron 4q + e][token n]
    const int n = lane & 15, q = lane >> 4;
    uint16_t hb[4], lb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int r = 4 * q + e, j = t * 16 + r;
        float h = 0.0f;
        if (n < a.B && ((m >> r) & 1u)) {
            const float gp = a.G[(size_t)n * a.f + j];
            if (a.use_union || gate_pred(a.mode, gp, a.theta)) h = act_f32(a.act, gp) * s4[e];
        }
        hb[e] = bf16_rne_bits(h);
        lb[e] = bf16_rne_bits(h - bf16_lo(hb[e]));
    }
    // lane order over d_ff: step t/2, k-group 2(t&1) + (q>>1), elements 4(q&1) .. +4
    const int g = 2 * (t & 1) + (q >> 1);
    const size_t o = ((size_t)(t >> 1) * 64 + (g << 4) + n) * 8 + 4 * (q & 1);
    uint2 ph, pl;
    __builtin_memcpy(&ph, hb, 8);
    __builtin_memcpy(&pl, lb, 8);
    *(uint2 *)(a.hh + o) = ph;
    *(uint2 *)(a.hl + o) = pl;
}

struct DownTiledArgs {
    const uint16_t *wdtl;            // W_down tiles [d/16][f/32][64][8]
    const uint16_t *hh, *hl;         // [f/32][64][8]
    int d, f, per;                   // per: k-steps per split (multiple of 4)
    float *partial;                  // [splits][16][d]
    const int *path;                 // run only when *path == want (nullptr: always)
    int want;
};

// Down on the W_down tiles: one wave per (kDownCols blocks of 16 output
// columns, d_ff split); each k-step's h operand (hi / lo) is loaded once for
// the wave's kDownCols weight tiles.
constexpr int kDownCols = 4;

__global__ __launch_bounds__(64) void k_down_tiled(const DownTiledArgs a)
{
    if (a.path && *a.path != a.want) return;
    const int tc = blockIdx.x * kDownCols, p = blockIdx.y, lane = threadIdx.x;
    const int KS = a.f / 32;
    const int k0 = min(KS, p * a.per), k1 = min(KS, k0 + a.per);
    bool live[kDownCols];
    const uint16_t *wp[kDownCols];
    f32x4_t acc[kDownCols];
#pragma unroll
    for (int b = 0; b < kDownCols; ++b) {
        live[b] = true;
        wp[b] = a.wdtl + (size_t)(tc + b) * KS * 512 + lane * 8;
        acc[b] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    for (int k = k0; k < k1; k += 4) mfma_group<4, kDownCols>(wp, live, a.hh + lane * 8, a.hl + lane * 8, k, k1, acc);
    // C[output column 16 (tc + b) + 4q + e][token n]
    const int n = lane & 15, q = lane >> 4;
#pragma unroll
    for (int b = 0; b < kDownCols; ++b)
        *(float4 *)(a.partial + ((size_t)p * 16 + n) * a.d + (tc + b) * 16 + 4 * q) =
            make_float4(acc[b][0], acc[b][1], acc[b][2], acc[b][3]);
}

// four consecutive outputs (i4 = index of the group): the split partials added
// in split order, then the residual.  All loads of a batch of 16 splits are
// issued before the adds (a split past ns reloads the last one, unused).
__device__ __forceinline__ void down_sum4(const float *__restrict__ partial, int ns, int d, int i4,
                                          const float *__restrict__ resid, float *__restrict__ out)
{
    const size_t stride = (size_t)16 * d;
    const float *src = partial + 4 * (size_t)i4;
    float y[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int p0 = 0; p0 < ns; p0 += 16) {
        f32x4_t v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = *(const f32x4_t *)(src + (size_t)min(p0 + u, ns - 1) * stride);
#pragma unroll
        for (int u = 0; u < 16; ++u)
            if (p0 + u < ns)
#pragma unroll
                for (int e = 0; e < 4; ++e) y[e] += v[u][e];
    }
    if (resid) {
        const float4 r = *(const float4 *)(resid + 4 * (size_t)i4);
        y[0] += r.x; y[1] += r.y; y[2] += r.z; y[3] += r.w;
    }
    *(float4 *)(out + 4 * (size_t)i4) = make_float4(y[0], y[1], y[2], y[3]);
}

// partial is [splits][16][d] (16 token slots); out [B][d]
__global__ __launch_bounds__(256) void k_down_sum(const float *__restrict__ partial, int ns, int B, int d,
                                                  const float *__restrict__ resid, float *__restrict__ out)
{
    const int i4 = blockIdx.x * 256 + threadIdx.x;
    if (i4 < B * d / 4) down_sum4(partial, ns, d, i4, resid, out);
}



// ---------------------------------------------------------------------------
// int4 top-k at 5..16 tokens: the down projection on MFMA over all of W_down.
// The tokens' union is most of d_ff at these batch sizes (about 3/4 of the
// neurons at 8 tokens, keep 17 %), so the whole int4 W_down [d][f] is read once,
// densely, with h = 0 outside each token's set, instead of gathering rows:
//   k_form_h_i4     h = act(g') u on the selected (token, neuron) pairs (the
//                   union rule as in the gather), as bf16 hi + lo in MFMA lane
//                   order (16 token slots)
//   k_down_i4_mfma  one wave per (4 blocks of 16 output columns, d_ff split):
//                   per group of 128 neurons (one fp16 scale per output
//                   column) the 4-bit weights, exact in bf16, times h hi and lo
//                   on v_mfma_f32_16x16x32_bf16, then the group's sum times the
//                   scale into the fp32 total; partial y per split
//   k_down_sum      the splits in order, plus the residual
// Inside a group the MFMA k order is permuted (k-step ks, lane k-group kg,
// element e <-> neuron 32 kg + 8 ks + e) so that each lane's four k-steps of
// W are one 16-byte load; h is stored in the same order.
// ---------------------------------------------------------------------------
struct FormHArgs {
    const uint32_t *bits;   // [B][f/32] top-k sets, or nullptr: G already holds h for every neuron (dense)
    const float *G, *U;     // [B][f]
    int B, f, nw32, act, use_union;
    uint16_t *hh, *hl;      // [f/128][4 k-steps][64 lanes][8]
};

// one thread per (group, k-step, lane): 8 neurons 128 g + 32 kg + 8 ks .. + 8 of token t
__global__ __launch_bounds__(256) void k_form_h_i4(const FormHArgs a)
{
    const int g = blockIdx.x, ks = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int kg = lane >> 4, t = lane & 15;
    const int j0 = 128 * g + 32 * kg + 8 * ks;
    uint32_t uni = 0xFFu, own = 0xFFu;   // bits of the 8 neurons: union over the tokens, this token's
    if (a.bits) {
        uni = 0;
        own = 0;
        for (int t2 = 0; t2 < a.B; ++t2) {
            const uint32_t w = (a.bits[(size_t)t2 * a.nw32 + (j0 >> 5)] >> (j0 & 31)) & 0xFFu;
            uni |= w;
            if (t2 == t) own = w;
        }
    }
    const int tc = min(t, a.B - 1);
    const f32x4_t g0 = *(const f32x4_t *)(a.G + (size_t)tc * a.f + j0), g1 = *(const f32x4_t *)(a.G + (size_t)tc * a.f + j0 + 4);
    const float *Ut = a.bits ? a.U : a.G;   // dense: h is read from G (u unused)
    const f32x4_t u0 = *(const f32x4_t *)(Ut + (size_t)tc * a.f + j0), u1 = *(const f32x4_t *)(Ut + (size_t)tc * a.f + j0 + 4);
    const float gv[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
    const float uv[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
    uint16_t hb[8], lb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const bool on = t < a.B && ((uni >> e) & 1u) && (a.use_union || ((own >> e) & 1u));
        const float h = !on ? 0.0f : a.bits ? act_f32(a.act, gv[e]) * uv[e] : gv[e];
        hb[e] = bf16_rne_bits(h);
        lb[e] = bf16_rne_bits(h - bf16_lo(hb[e]));
    }
    const size_t o = (((size_t)g * 4 + ks) * 64 + lane) * 8;
    uint4 ph, pl;
    __builtin_memcpy(&ph, hb, 16);
    __builtin_memcpy(&pl, lb, 16);
    *(uint4 *)(a.hh + o) = ph;
    *(uint4 *)(a.hl + o) = pl;
}

struct DownI4Args {
    const uint8_t *wd;        // W_down int4 [d][f] (element j of a row: nibble j % 2 of byte j / 2)
    const uint16_t *sdt;      // fp16 scales [f/128][d]
    const uint16_t *hh, *hl;  // h, as k_form_h_i4 writes it
    int d, f, per;            // per: groups of 128 neurons per split
    float *partial;           // [splits][16][d]
};

constexpr int kDownI4Cols = 4;     // blocks of 16 output columns per wave
constexpr int kDownI4Waves = 1024;  // waves of the launch: d_ff splits so that (d / 64) x splits reach it
constexpr int kDownI4Groups = 4;    // most groups of 128 neurons per split (all loaded at once)

// the 4-bit values of one dword as 8 bf16 (exact: small integers)
__device__ __forceinline__ bf16x8_t i4x8_to_bf16(uint32_t w)
{
    uint16_t b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) b[e] = (uint16_t)(__float_as_uint((float)nib(w, e)) >> 16);
    bf16x8_t r;
    __builtin_memcpy(&r, b, 16);
    return r;
}

__global__ __launch_bounds__(64) void k_down_i4_mfma(const DownI4Args a)
{
    const int lane = threadIdx.x, n = lane & 15, q = lane >> 4;
    const int col0 = blockIdx.x * 16 * kDownI4Cols, p = blockIdx.y;
    const int ng = a.f / 128;
    const int g0 = min(ng, p * a.per), cnt = min(ng, g0 + a.per) - g0;   // cnt <= kDownI4Groups
    const size_t rowb = (size_t)a.f / 2;
    // every load of the split first (one round trip): per group h (4 k-steps,
    // hi and lo), W (one 16-byte piece per column block) and the scales of the
    // lane's 4 output columns; groups past the split reload its last one (unused)
    uint4 hv[kDownI4Groups][4][2], wv[kDownI4Groups][kDownI4Cols];
    uint2 sv[kDownI4Groups][kDownI4Cols];
#pragma unroll
    for (int i = 0; i < kDownI4Groups; ++i) {
        const int g = g0 + min(i, max(cnt - 1, 0));
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const size_t o = (((size_t)g * 4 + ks) * 64 + lane) * 8;
            hv[i][ks][0] = *(const uint4 *)(a.hh + o);
            hv[i][ks][1] = *(const uint4 *)(a.hl + o);
        }
#pragma unroll
        for (int c = 0; c < kDownI4Cols; ++c) {
            const int col = col0 + 16 * c + n;   // A row of this lane
            wv[i][c] = ld16_nt(a.wd + (size_t)col * rowb + 64 * (size_t)g + 16 * q);
            sv[i][c] = *(const uint2 *)(a.sdt + (size_t)g * a.d + col0 + 16 * c + 4 * q);
        }
    }
    f32x4_t acc[kDownI4Cols];
#pragma unroll
    for (int c = 0; c < kDownI4Cols; ++c) acc[c] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < kDownI4Groups; ++i) {
        if (i >= cnt) break;
#pragma unroll
        for (int c = 0; c < kDownI4Cols; ++c) {
            const uint32_t wd4[4] = {wv[i][c].x, wv[i][c].y, wv[i][c].z, wv[i][c].w};
            f32x4_t s4 = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8_t wf = i4x8_to_bf16(wd4[ks]);
                bf16x8_t hf, lf;
                __builtin_memcpy(&hf, &hv[i][ks][0], 16);
                __builtin_memcpy(&lf, &hv[i][ks][1], 16);
                s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, hf, s4, 0, 0, 0);
                s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, lf, s4, 0, 0, 0);
            }
            // C[output column 4q + e][token n]: the group's sum times the column's scale
            const float sc[4] = {half_bits_to_float((uint16_t)sv[i][c].x), half_bits_to_float((uint16_t)(sv[i][c].x >> 16)),
                                 half_bits_to_float((uint16_t)sv[i][c].y), half_bits_to_float((uint16_t)(sv[i][c].y >> 16))};
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[c][e] = __builtin_fmaf(sc[e], s4[e], acc[c][e]);
        }
    }
#pragma unroll
    for (int c = 0; c < kDownI4Cols; ++c)
        *(float4 *)(a.partial + ((size_t)p * 16 + n) * a.d + col0 + 16 * c + 4 * q) =
            make_float4(acc[c][0], acc[c][1], acc[c][2], acc[c][3]);
}

// ---------------------------------------------------------------------------
// batched gate GEMV in the fixed order (5..16 tokens, bf16, BATCH layout).
// The fixed order splits a row into 64 lane accumulators (accumulator c sums
// chunks c, c + 64, ... with an fma chain per chunk) and adds them in a halving
// tree that pairs c with c ^ 32, then ^ 16, ^ 8, ^ 4, ^ 2, ^ 1.  The last two
// levels join the four classes c mod 4, so a workgroup can own one class m: it
// stages only that quarter of x (the chunks m + 4i + 64k), its lanes are the 16
// accumulators i of the class times 4 row groups, every lane keeps its x values
// for RPW rows, and the class's tree levels (c ^ 32 ... c ^ 4 = lane ^ 8 ... ^ 1)
// are shuffles inside 16 lanes.  W_gate is read from a copy laid out
// [class][k][row][i] (16 bytes each), so four consecutive rows' 256-byte pieces
// form one contiguous kilobyte per wave load.  k_gate_combine adds the classes
// (0 with 2, 1 with 3, then the two) and the bias: bit for bit the fixed order.
// ---------------------------------------------------------------------------
constexpr int kGateClsRPW = 4;                   // rows per lane
constexpr int kGateClsRows = 16 * kGateClsRPW;   // rows per workgroup (4 waves x 4 groups x RPW)

struct GateClsArgs {
    const uint16_t *wgc;   // [4][K][f][16][8]
    int d, f, B;
    float *part;           // [4][B][f]
};

// The class-split gate runs as a two-stage pipeline of asynchronous global ->
// LDS copies (global_load_lds_dwordx4): each slice k brings the workgroup's 64
// W_gate rows (16 KB, each wave its own 16 rows) and the class's x values
// (8 KB, shared) into stage k % 2, one slice ahead of the FMAs, without holding
// registers for them.
constexpr int kGateStages = 2;
constexpr int kGateXAhead = 2;   // tokens of x read ahead of the FMAs

// s_waitcnt immediate that waits until at most n vector-memory operations are
// outstanding (expcnt and lgkmcnt left at their no-wait maxima)
constexpr int waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

template <bool NT = false>
__device__ __forceinline__ void lds_copy16(const void *g, void *lds_wave_base)
{
    // lane l writes bytes [16 l, 16 l + 16) of the wave's 1 KB LDS block, whose
    // (wave-uniform) LDS address goes in M0.  Issued as inline assembly so the
    // compiler's wait insertion, which cannot tell the stages apart, does not
    // drain every copy in flight before each LDS read; the kernel waits on the
    // vector-memory counter itself.  Nothing else in these kernels uses M0.
    const uint32_t la = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)lds_wave_base);
    // NT: the streaming (non-temporal) cache policy, for weights read once per call
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g), "s"(la) : "memory");
    else
        asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(la) : "memory");
}

// LDS of one class-split gate workgroup: W stages [stage][wave][row in wave][i]
// (16 bytes each), then x stages [stage][token][half][i][4] (conflict-free reads)
typedef uint4 GateWsm[kGateStages][4][4 * kGateClsRPW][16];
typedef float GateXs[kGateStages][16][2][16][4];
constexpr int kGateSmem = (int)(sizeof(GateWsm) + sizeof(GateXs));

// one class-split gate workgroup: rows tile * kGateClsRows .. + kGateClsRows,
// accumulator class m, partial sums to a.part
template <int BT>
__device__ __forceinline__ void gate_pipe_tile(const GateClsArgs &a, const float *__restrict__ x, int tile, int m,
                                               uint8_t *smem)
{
    constexpr int RPW = kGateClsRPW, S = kGateStages;
    GateWsm &wsm = *reinterpret_cast<GateWsm *>(smem);
    GateXs &xs = *reinterpret_cast<GateXs *>(smem + sizeof(GateWsm));
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i = lane & 15, r = lane >> 4;
    const int nch = a.d / 8, K = (nch + 63) / 64, B = a.B, f = a.f;
    const int jw = tile * kGateClsRows + w * 4 * RPW;   // first row of this wave
    const size_t kstride = (size_t)f * 128;
    const uint16_t *wsrc = a.wgc + ((size_t)m * K * f + jw) * 128 + lane * 8;

    auto issue = [&](int k) {
        const int st = k % S;
        // this wave's 4 RPW rows: 4 RPW x 256 B = RPW loads of 1 KB
#pragma unroll
        for (int q = 0; q < RPW; ++q) lds_copy16<true>(wsrc + k * kstride + q * 512, &wsm[st][w][4 * q][0]);
        // x: 8 KB = 8 loads of 1 KB, two per wave; item = [t][half][i'], t < 16
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int item = (w * 2 + h) * 64 + lane;
            const int t = item >> 5, half = (item >> 4) & 1, ii = item & 15;
            const int ch = min(m + 4 * ii + 64 * k, nch - 1);   // past the row: any valid chunk (never used)
            lds_copy16(x + (size_t)min(t, B - 1) * a.d + ch * 8 + 4 * half, &xs[st][0][0][0][0] + (w * 2 + h) * 256);
        }
    };

    float acc[RPW][BT];
#pragma unroll
    for (int q = 0; q < RPW; ++q)
#pragma unroll
        for (int t = 0; t < BT; ++t) acc[q][t] = 0.0f;

    issue(0);
    for (int k = 0; k < K; ++k) {
        // slice k has landed once at most the next slice's loads are outstanding
        if (k + 1 < K) {
            issue(k + 1);
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(RPW + 2));
        } else {
            __builtin_amdgcn_s_waitcnt(waitcnt_vm(0));
        }
        // this wave's copies of slice k are in LDS; the barrier (no fence, so the
        // later slices stay in flight) waits for every wave's
        __builtin_amdgcn_s_barrier();
        const int st = k % S;
        if (m + 4 * i + 64 * k < nch) {
            uint4 wv[RPW];
#pragma unroll
            for (int q = 0; q < RPW; ++q) wv[q] = wsm[st][w][4 * q + r][i];
            // x of token t + kGateXAhead is read while token t computes (a rotating
            // register set per token in flight; the scheduling barriers keep the
            // compiler from pulling the reads back next to their use)
            constexpr int XA = kGateXAhead;
            f32x4_t xq[XA + 1][2];
#pragma unroll
            for (int t = 0; t < XA; ++t) {
                xq[t][0] = *(const f32x4_t *)&xs[st][t][0][i][0];
                xq[t][1] = *(const f32x4_t *)&xs[st][t][1][i][0];
            }
#pragma unroll
            for (int t = 0; t < BT; ++t) {
                if (t + XA < BT) {
                    xq[(t + XA) % (XA + 1)][0] = *(const f32x4_t *)&xs[st][t + XA][0][i][0];
                    xq[(t + XA) % (XA + 1)][1] = *(const f32x4_t *)&xs[st][t + XA][1][i][0];
                }
                __builtin_amdgcn_sched_barrier(0);
                const f32x4_t x0 = xq[t % (XA + 1)][0], x1 = xq[t % (XA + 1)][1];
                const float xv[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
                for (int q = 0; q < RPW; ++q) acc[q][t] = chunk_dot<SFFN_W_BF16>(wv[q], 0.0f, xv, acc[q][t]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __builtin_amdgcn_s_barrier();   // stage st is refilled by the next iteration's issue
    }
#pragma unroll
    for (int q = 0; q < RPW; ++q)
#pragma unroll
        for (int t = 0; t < BT; ++t) {
            float v = acc[q][t];
            v = v + __shfl_xor(v, 8, 64);
            v = v + __shfl_xor(v, 4, 64);
            v = v + __shfl_xor(v, 2, 64);
            v = v + __shfl_xor(v, 1, 64);
            acc[q][t] = v;
        }
    const int j0 = jw + r;
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
        float v = 0.0f;
#pragma unroll
        for (int t = 0; t < BT; ++t) v = (t == i) ? acc[q][t] : v;
        if (i < B) a.part[((size_t)m * B + i) * f + j0 + 4 * q] = v;
    }
}

template <int BT>
__global__ __launch_bounds__(256) void k_gate_pipe(const GateClsArgs a, const float *__restrict__ x)
{
    __shared__ __align__(16) uint8_t smem[kGateSmem];
    gate_pipe_tile<BT>(a, x, blockIdx.x, blockIdx.y, smem);
}

// ---------------------------------------------------------------------------
// 9..16 tokens on the tile path: the class-split gate and the MFMA up
// projection in one launch.  Up does not need the gate (h = act(g') u is
// formed afterwards), so the two run side by side: the grid interleaves two
// gate workgroups (VALU- and LDS-bound) with one up workgroup (bound by the
// W_up stream), so every CU holds both kinds and the gate's arithmetic hides
// under the up projection's weight traffic.  Both roles fit one resource
// budget (the gate's LDS, the larger register count).  u is written in fp32;
// k_combine_h adds the gate classes and the two halves of u and forms the
// selection, the lists and h.
// ---------------------------------------------------------------------------
struct UpUArgs {
    const uint16_t *wut;             // W_up tiles [f/16][d/32][64][8]
    const uint16_t *xh, *xl;         // x_hat bf16 hi / lo, lane order [d/32][64][8]
    int d, f, B;
    float *U;                        // [B][f]
};

// u over one half of d_model (hf = 0, 1) for the blocks NB ui .. NB ui + NB - 1
// of 16 neurons: the four waves split the half in quarters, each streams its
// activation steps once for all NB tiles (U steps in flight), and the partial
// tiles are added in LDS in wave order into U + hf B f
template <int NB, int U>
__device__ __forceinline__ void up_u_tiles(const UpUArgs &a, int ui, int hf, uint8_t *smem)
{
    f32x4_t(&part)[4][NB][64] = *reinterpret_cast<f32x4_t(*)[4][NB][64]>(smem);
    const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int t0 = ui * NB, KS = a.d / 32;
    const int h0 = (KS * hf) / 2, h1 = (KS * (hf + 1)) / 2;
    const int k0 = h0 + ((h1 - h0) * w) / 4, k1 = h0 + ((h1 - h0) * (w + 1)) / 4;
    bool live[NB];
    const uint16_t *wp[NB];
    f32x4_t acc[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        live[b] = true;
        wp[b] = a.wut + (size_t)(t0 + b) * KS * 512 + lane * 8;
        acc[b] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    for (int k = k0; k < k1; k += U) mfma_group<U, NB>(wp, live, a.xh + lane * 8, a.xl + lane * 8, k, k1, acc);
#pragma unroll
    for (int b = 0; b < NB; ++b) part[w][b][lane] = acc[b];
    __syncthreads();
    // C[neuron 4q + e][token n]
    const int n = lane & 15, q = lane >> 4;
    float *Uh = a.U + (size_t)hf * a.B * a.f;
    for (int b = w; b < NB; b += 4) {
        const f32x4_t s4 = ((part[0][b][lane] + part[1][b][lane]) + part[2][b][lane]) + part[3][b][lane];
        if (n < a.B)
            *(float4 *)(Uh + (size_t)n * a.f + (t0 + b) * 16 + 4 * q) = make_float4(s4[0], s4[1], s4[2], s4[3]);
    }
}

// up blocks of 16 neurons per up item and MFMA k-steps in flight per wave.
// Work items: f / 16 gate workgroups (4 classes x f / 64 tiles) and f / 16 up
// items (f / (16 kDualNB) block groups x 2 halves of d_model).  The grid
// interleaves two gate items with one first-half up item, then runs the
// second-half up items: the shorter up items come last, so the launch drains
// quickly once the gate items are done.
constexpr int kDualNB = 2, kDualU = 4;

template <int BT>
__global__ __launch_bounds__(256) void k_gate_up_dual(const GateClsArgs ga, const float *__restrict__ x,
                                                      const UpUArgs ua)
{
    __shared__ __align__(16) uint8_t smem[kGateSmem];
    const int ngu = ua.f / (16 * kDualNB);   // up block groups
    const int b = blockIdx.x;
    if (b < 3 * ngu) {
        const int per = b / 3, ph = b % 3;
        if (ph < 2) {
            const int gi = 2 * per + ph;
            gate_pipe_tile<BT>(ga, x, gi >> 2, gi & 3, smem);
        } else {
            up_u_tiles<kDualNB, kDualU>(ua, per, 0, smem);
        }
    } else {
        up_u_tiles<kDualNB, kDualU>(ua, b - 3 * ngu, 1, smem);
    }
}

// g' = ((class 0 + class 2) + (class 1 + class 3)) + b, the selection, the
// lists per block of 16 neurons and h = act(g') u on the selected (token,
// neuron) pairs (0 elsewhere) as bf16 hi / lo in lane order over d_ff.  One
// wave per 32 neurons; lane (g, n) takes neurons 8 g .. 8 g + 7 of token n
// (one 16-byte piece of the lane order: step j0 / 32, k-group g, slot n).
__global__ __launch_bounds__(64) void k_combine_h(const float *__restrict__ part, const float *__restrict__ U, int B,
                                                  int f, float bias, int mode, float theta, int act, int use_union,
                                                  float *__restrict__ G, int *__restrict__ list_cnt,
                                                  int *__restrict__ list_idx, uint16_t *__restrict__ hh,
                                                  uint16_t *__restrict__ hl)
{
    const int lane = threadIdx.x, g = lane >> 4, n = lane & 15, s = blockIdx.x;
    const int j = s * 32 + 8 * g;   // first of the lane's 8 neurons
    float gp[8];
    uint32_t on = 0;
    // u first, so that its loads share the partials' round trip (token slots >= B
    // read token B - 1's, unused)
    float u[8];
    {
        // u = (first half of d_model) + (second half)
        const size_t ou = (size_t)min(n, B - 1) * f + j, hs = (size_t)B * f;
        const f32x4_t a0 = *(const f32x4_t *)(U + ou), a1 = *(const f32x4_t *)(U + ou + 4);
        const f32x4_t b0 = *(const f32x4_t *)(U + hs + ou), b1 = *(const f32x4_t *)(U + hs + ou + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            u[e] = a0[e] + b0[e];
            u[4 + e] = a1[e] + b1[e];
        }
    }
    {
        // the class partials (unconditional loads: slots past B read token B - 1's, unused)
        const size_t cs = (size_t)B * f, o = (size_t)min(n, B - 1) * f + j;
        float p[4][8];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float4 v0 = *(const float4 *)(part + c * cs + o), v1 = *(const float4 *)(part + c * cs + o + 4);
            p[c][0] = v0.x; p[c][1] = v0.y; p[c][2] = v0.z; p[c][3] = v0.w;
            p[c][4] = v1.x; p[c][5] = v1.y; p[c][6] = v1.z; p[c][7] = v1.w;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            gp[e] = ((p[0][e] + p[2][e]) + (p[1][e] + p[3][e])) + bias;
            on |= (n < B && gate_pred(mode, gp[e], theta)) ? (1u << e) : 0u;
        }
        if (n < B) {
            *(float4 *)(G + o) = make_float4(gp[0], gp[1], gp[2], gp[3]);
            *(float4 *)(G + o + 4) = make_float4(gp[4], gp[5], gp[6], gp[7]);
        }
    }
    // union over the tokens: neuron 8 g + e is selected if any lane of group g has bit e
    uint32_t mask = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint64_t bal = __ballot((on >> e) & 1u);
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) mask |= ((bal >> (16 * gg)) & 0xFFFFull) ? (1u << (8 * gg + e)) : 0u;
    }
    if (lane < 32 && ((mask >> lane) & 1u)) {
        const int b = lane >> 4;
        const uint32_t mb = (mask >> (16 * b)) & 0xFFFFu;
        list_idx[(size_t)(2 * s + b) * 16 + __popc(mb & ((1u << (lane & 15)) - 1u))] = s * 32 + lane;
    }
    if (lane < 2) list_cnt[2 * s + lane] = __popc((mask >> (16 * lane)) & 0xFFFFu);
    uint16_t hb[8], lb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float h = 0.0f;
        if (n < B && ((mask >> (8 * g + e)) & 1u) && (use_union || ((on >> e) & 1u))) h = act_f32(act, gp[e]) * u[e];
        hb[e] = bf16_rne_bits(h);
        lb[e] = bf16_rne_bits(h - bf16_lo(hb[e]));
    }
    const size_t o = ((size_t)s * 64 + (g << 4) + n) * 8;
    uint4 ph, pl;
    __builtin_memcpy(&ph, hb, 16);
    __builtin_memcpy(&pl, lb, 16);
    *(uint4 *)(hh + o) = ph;
    *(uint4 *)(hl + o) = pl;
}

// g' = ((class 0 + class 2) + (class 1 + class 3)) + b; selection flags; ascending
// lists per block of 16 rows (ballot + mbcnt), the format of the gate kernels
__global__ __launch_bounds__(64) void k_gate_combine(const float *__restrict__ part, int B, int f, float bias,
                                                     int mode, float theta, float *__restrict__ G,
                                                     int *__restrict__ list_cnt, int *__restrict__ list_idx)
{
    const int lane = threadIdx.x, j = blockIdx.x * 64 + lane;
    int on = 0;
    for (int t = 0; t < B; ++t) {
        const size_t o = (size_t)t * f + j, cs = (size_t)B * f;
        const float g = (part[o] + part[2 * cs + o]) + (part[cs + o] + part[3 * cs + o]);
        const float gp = g + bias;
        G[o] = gp;
        on |= gate_pred(mode, gp, theta) ? 1 : 0;
    }
    const uint64_t m = __ballot(on);
    const int sb = lane >> 4;
    const uint64_t below = m & ((1ull << lane) - 1ull) & (0xFFFFull << (16 * sb));
    if (on) list_idx[(size_t)(j >> 4) * 16 + __popcll(below)] = j;
    if ((lane & 15) == 0) list_cnt[j >> 4] = __popcll(m & (0xFFFFull << (16 * sb)));
}

// RMSNorm prologue with the MFMA operand split: one wave per token slot (16
// slots); x_hat as k_rmsnorm computes it (same order, same scale), plus x_hat
// as bf16 hi / lo in lane order.  Slots >= B write zero operands only.
__global__ __launch_bounds__(64) void k_rmsnorm_split(const float *__restrict__ x, float *__restrict__ xhat,
                                                      int B, int d, float eps, uint16_t *__restrict__ xh,
                                                      uint16_t *__restrict__ xl)
{
    const int t = blockIdx.x, lane = threadIdx.x;
    float r = 0.0f;
    const float *xt = x + (size_t)min(t, B - 1) * d;
    if (d <= 4096) {
        // every chunk of the row in registers (at most 16 per lane), loaded once,
        // unconditionally; slots past B load token B - 1's and write zeros
        const int nch = d / 4;
        f32x4_t v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) v[u] = *(const f32x4_t *)(xt + 4 * min(u * 64 + lane, nch - 1));
        float acc = 0.0f;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            if (u * 64 + lane < nch) {
#pragma unroll
                for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(v[u][e], v[u][e], acc);
            }
        }
        const float ss = wave_tree_sum_dpp(acc);
        r = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int c = u * 64 + lane;
            if (c < nch) {
                f32x4_t y = v[u] * r;
                if (t < B) *(f32x4_t *)(xhat + (size_t)t * d + 4 * c) = y;
                else y = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
                const int pc = c >> 1, sstep = pc >> 2, g = pc & 3;
                uint16_t h[4], lo[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h[e] = bf16_rne_bits(y[e]);
                    lo[e] = bf16_rne_bits(y[e] - bf16_lo(h[e]));
                }
                const size_t o = ((size_t)sstep * 64 + (g << 4) + t) * 8 + 4 * (c & 1);
                uint2 ph, pl;
                __builtin_memcpy(&ph, h, 8);
                __builtin_memcpy(&pl, lo, 8);
                *(uint2 *)(xh + o) = ph;
                *(uint2 *)(xl + o) = pl;
            }
        }
        return;
    }
    if (t < B) {
        const int nch = d / 4;
        float acc = 0.0f;
        for (int k0 = 0; k0 * 64 < nch; k0 += 16) {
            float4 v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int c = (k0 + u) * 64 + lane;
                v[u] = c < nch ? *(const float4 *)(xt + 4 * c) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                if ((k0 + u) * 64 + lane < nch) {
                    acc = __builtin_fmaf(v[u].x, v[u].x, acc);
                    acc = __builtin_fmaf(v[u].y, v[u].y, acc);
                    acc = __builtin_fmaf(v[u].z, v[u].z, acc);
                    acc = __builtin_fmaf(v[u].w, v[u].w, acc);
                }
            }
        }
        const float ss = wave_tree_sum(acc);
        r = 1.0f / sqrtf(ss / (float)d + eps);
    }
    // x_hat and its split, 16 float4 chunks per lane in flight: chunk c holds
    // values 4c .. 4c + 3, half (c & 1) of the 8-value piece c / 2 = 4 s + g,
    // which sits in lane slot (g << 4) | t of step s
    const int nch = d / 4;
    for (int k0 = 0; k0 * 64 < nch; k0 += 16) {
        f32x4_t v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int c = min((k0 + u) * 64 + lane, nch - 1);
            v[u] = t < B ? *(const f32x4_t *)(xt + 4 * c) : f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int c = (k0 + u) * 64 + lane;
            if (c < nch) {
                const f32x4_t y = v[u] * r;
                if (t < B) *(f32x4_t *)(xhat + (size_t)t * d + 4 * c) = y;
                const int pc = c >> 1, sstep = pc >> 2, g = pc & 3;
                uint16_t h[4], lo[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    h[e] = bf16_rne_bits(y[e]);
                    lo[e] = bf16_rne_bits(y[e] - bf16_lo(h[e]));
                }
                const size_t o = ((size_t)sstep * 64 + (g << 4) + t) * 8 + 4 * (c & 1);
                uint2 ph, pl;
                __builtin_memcpy(&ph, h, 8);
                __builtin_memcpy(&pl, lo, 8);
                *(uint2 *)(xh + o) = ph;
                *(uint2 *)(xl + o) = pl;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// batch-1 kernels.  One 1024-thread workgroup per compute unit, every weight
// row load issued before x is staged into LDS, so each workgroup keeps its whole
// share of rows in flight at once (up to 3 rows x 8 KB per wave).
// ---------------------------------------------------------------------------


struct FusedArgs {
    const uint8_t *wg, *wu, *wdt;
    const float *x;
    float *G;          // [f] g' (for inspection)
    float *partial;    // [P][d]
    int *list_cnt, *list_idx;  // per-workgroup ascending active lists (stride RB)
    int f, RB;
    int mode, act;
    float bias, theta;
};

template <int WT, int KC>
__device__ __forceinline__ void load_row(uint4 (&w)[KC], const uint8_t *base, size_t rb, int row, int lane)
{
#pragma unroll
    for (int k = 0; k < KC; ++k) w[k] = ld16_nt(base + (size_t)row * rb + (size_t)(k * 64 + lane) * 16);
}

// fixed-order dot of one row (chunks in registers) with x in LDS
template <int WT, int KC>
__device__ __forceinline__ float dot_row_lds(const uint4 (&w)[KC], const float *xs, int lane)
{
    constexpr int E = Chunk<WT>::E;
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < KC; ++k) {
        float xv[E];
        const float4 *xp = (const float4 *)(xs + (size_t)(k * 64 + lane) * E);
#pragma unroll
        for (int e4 = 0; e4 < E / 4; ++e4) {
            const float4 v = xp[e4];
            xv[4 * e4 + 0] = v.x; xv[4 * e4 + 1] = v.y;
            xv[4 * e4 + 2] = v.z; xv[4 * e4 + 3] = v.w;
        }
        acc = chunk_dot<WT>(w[k], 0.0f, xv, acc);
    }
    return wave_tree_sum_dpp(acc);
}

__device__ __forceinline__ void stage_vec(float *xs, const float *x, int n)
{
    for (int i = threadIdx.x; i < n / 4; i += blockDim.x) ((float4 *)xs)[i] = ((const float4 *)x)[i];
}

// Fused sparse layer for one token.  Each workgroup owns RB <= 48 consecutive
// neurons and runs 8 waves.
// Phase 1: the gate stream.  Wave w walks the rows w, w + 8, ... with the next
// two rows' loads in flight (with the non-temporal loads three rows per wave
// measured 1 % faster than two; every row requested at once was slower),
// forms g' in the fixed order and the predicate, and records g' and the flag
// in LDS.
// Phase 2: the ascending list of active neurons (ballot + mbcnt).  Wave q loads
// the W_up rows of active neurons q, q + 8, ... (two in flight) and forms
// h = act(g') u.  Before the first of those products is waited for, every
// wave also requests its slice of the active neurons' W_down^T rows: wave w
// owns the chunks [w CW, (w + 1) CW) of a row (CW = 8 KC), lane (s, c) chunk c
// of the neurons s, s + S, ... (S = 64 / CW slots; one slot at d_model 4096
// bf16).  Once every h is in LDS, each lane adds h_q * W_down^T[j_q] for its
// chunk in ascending q, the slots of a chunk are summed in slot order, and the
// workgroup's partial y is written in the blocked layout [D / 16][P][16] that
// the reduce reads.  No per-wave copy of y is kept, so LDS holds only x and
// the workgroup's neuron bookkeeping.
constexpr int kFusedNW = 8;
constexpr int kFusedNT = kFusedNW * 64;
constexpr int kFusedDB = 8;  // W_down^T chunks per lane per batch (two batches in flight)

template <int WT, int KC>
__global__ __launch_bounds__(kFusedNT) void k_decode_b1(const FusedArgs a)
{
    constexpr int E = Chunk<WT>::E;
    constexpr int NW = kFusedNW;
    constexpr int EB = WT == SFFN_W_F32 ? 4 : 2;
    constexpr int D = KC * 64 * E;
    constexpr size_t RBYTES = (size_t)D * EB;
    constexpr int CW = KC * 64 / NW;       // chunks of a W_down^T row per wave
    constexpr int S = CW >= 64 ? 1 : 64 / CW;  // neuron slots per wave
    constexpr int DB = kFusedDB;
    static_assert(NW * CW == KC * 64 && CW <= 64, "column split of the down rows");
    __shared__ __align__(16) float xs[D];
    __shared__ int flags[kFusedMaxRB];
    __shared__ float gsm[kFusedMaxRB];
    __shared__ int alist[kFusedMaxRB];
    __shared__ float hs[kFusedMaxRB];
    __shared__ int s_nact;

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r0 = blockIdx.x * a.RB;
    const int nr = min(a.RB, a.f - r0);

    // phase 1: the gate stream (wave w walks rows w, w + NW, ..., the next row's
    // loads in flight), g' and the selection into LDS
    auto gate = [&](const uint4 (&cur)[KC], int i) {
        const float gp = dot_row_lds<WT, KC>(cur, xs, lane) + a.bias;
        if (lane == 0) {
            a.G[r0 + i] = gp;
            flags[i] = gate_pred(a.mode, gp, a.theta) ? 1 : 0;
            gsm[i] = gp;
        }
    };
    {
        uint4 ga[KC];
        if (wave < nr) load_row<WT, KC>(ga, a.wg, RBYTES, r0 + wave, lane);
        stage_vec(xs, a.x, D);
        __syncthreads();
        // three rows in flight per wave: ga, gb, gc in rotation
        uint4 gb[KC], gc[KC];
        if (wave + NW < nr) load_row<WT, KC>(gb, a.wg, RBYTES, r0 + wave + NW, lane);
        for (int i = wave; i < nr; i += 3 * NW) {
            if (i + 2 * NW < nr) load_row<WT, KC>(gc, a.wg, RBYTES, r0 + i + 2 * NW, lane);
            gate(ga, i);
            if (i + NW >= nr) break;
            if (i + 3 * NW < nr) load_row<WT, KC>(ga, a.wg, RBYTES, r0 + i + 3 * NW, lane);
            gate(gb, i + NW);
            if (i + 2 * NW >= nr) break;
            if (i + 4 * NW < nr) load_row<WT, KC>(gb, a.wg, RBYTES, r0 + i + 4 * NW, lane);
            gate(gc, i + 2 * NW);
        }
    }
    __syncthreads();
    // ascending list of this workgroup's active neurons (ballot + mbcnt)
    if (wave == 0) {
        const int on = lane < nr ? flags[lane] : 0;
        const uint64_t m = __ballot(on);
        if (on) {
            alist[mbcnt64(m)] = lane;
            a.list_idx[(size_t)blockIdx.x * a.RB + mbcnt64(m)] = r0 + lane;
        }
        if (lane == 0) {
            s_nact = __popcll(m);
            a.list_cnt[blockIdx.x] = __popcll(m);
        }
    }
    __syncthreads();
    const int nact = s_nact;

    // phase 2
    const int s = lane / CW, c = lane - s * CW;  // lanes with s >= S (when CW does not divide 64) idle
    const bool dl = s < S;
    const size_t coff = (size_t)(wave * CW + c) * 16;  // byte offset of this lane's chunk in a row
    constexpr int PER = S * DB;                        // neurons per batch
    auto load_down = [&](uint4 (&dst)[DB], int q0) {
#pragma unroll
        for (int t = 0; t < DB; ++t) {
            const int q = q0 + s + S * t;
            if (dl && q < nact) dst[t] = ld16_nt(a.wdt + (size_t)(r0 + alist[q]) * RBYTES + coff);
        }
    };
    float yacc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) yacc[e] = 0.0f;
    auto fma_down = [&](const uint4 (&src)[DB], int q0) {
#pragma unroll
        for (int t = 0; t < DB; ++t) {
            const int q = q0 + s + S * t;
            if (dl && q < nact) {
                const float h = hs[q];
                float w[E];
                unpack<WT>(src[t], w);
#pragma unroll
                for (int e = 0; e < E; ++e) yacc[e] = __builtin_fmaf(h, w[e], yacc[e]);
            }
        }
    };
    auto up_h = [&](const uint4 (&ur)[KC], int q) {
        const float u = dot_row_lds<WT, KC>(ur, xs, lane);
        if (lane == 0) hs[q] = act_f32(a.act, gsm[alist[q]]) * u;
    };
    uint4 da[DB], db[DB];
    {
        uint4 ua[KC], ub[KC];
        int q = wave;
        if (q < nact) load_row<WT, KC>(ua, a.wu, RBYTES, r0 + alist[q], lane);
        if (q + NW < nact) load_row<WT, KC>(ub, a.wu, RBYTES, r0 + alist[q + NW], lane);
        load_down(da, 0);
        for (; q < nact; q += 2 * NW) {
            up_h(ua, q);
            if (q + 2 * NW < nact) load_row<WT, KC>(ua, a.wu, RBYTES, r0 + alist[q + 2 * NW], lane);
            if (q + NW >= nact) break;
            up_h(ub, q + NW);
            if (q + 3 * NW < nact) load_row<WT, KC>(ub, a.wu, RBYTES, r0 + alist[q + 3 * NW], lane);
        }
    }
    __syncthreads();
    for (int q0 = 0; q0 < nact; q0 += 2 * PER) {
        if (q0 + PER < nact) load_down(db, q0 + PER);
        fma_down(da, q0);
        if (q0 + PER >= nact) break;
        if (q0 + 2 * PER < nact) load_down(da, q0 + 2 * PER);
        fma_down(db, q0 + PER);
    }
    // slots summed in slot order (lanes with s = 0 keep the result)
    float ys[E];
#pragma unroll
    for (int e = 0; e < E; ++e) ys[e] = yacc[e];
#pragma unroll
    for (int t = 1; t < S; ++t) {
#pragma unroll
        for (int e = 0; e < E; ++e) ys[e] += __shfl(yacc[e], t * CW + c, 64);
    }
    if (s == 0) {
        const int col = (wave * CW + c) * E;
        float *dst = a.partial + ((size_t)(col >> 4) * gridDim.x + blockIdx.x) * 16 + (col & 15);
#pragma unroll
        for (int e4 = 0; e4 < E / 4; ++e4)
            *(float4 *)(dst + 4 * e4) = make_float4(ys[4 * e4], ys[4 * e4 + 1], ys[4 * e4 + 2], ys[4 * e4 + 3]);
    }
}

// int4 gate + up for one token (weight-aware top-k): a persistent streaming
// GEMV.  A 16-byte int4 chunk holds 32 elements, so at d_model = 2048 KC each
// lane p owns KC chunks (p, p + 64, ...) of every row, which is the fixed
// order's accumulator p: the lane keeps its 32 KC x values in registers for
// the whole kernel (no LDS), and a wave reads a whole row with one 16-byte load
// per lane per chunk.  One workgroup per compute unit owns RB <= 48
// consecutive neurons; wave w walks the rows w, w + NW, ... with three rows
// (gate and up, with their group scales) in rotation, the next two in flight
// while one is reduced.  (Every row requested at once with 16 waves was
// measured slower, 11.1 against 9.2 us at 2048 x 11008: the fixed-order int4
// dot costs about as much VALU time as the stream takes, and the rotation
// overlaps the two.)  g' = g + b and u are stored (fixed order, bit for bit the
// values of the generic kernel); the workgroup's fp64 score keys are formed at
// the end, one neuron per thread.
struct GuI4Args {
    const uint8_t *wg, *wu;      // [f][d/2] int4
    const uint16_t *sg, *su;     // [f][d/128] fp16
    const float *x;              // [d]
    const double *wdn;           // ||W_down[:, j]||_2
    float *G, *U;                // [f]
    uint64_t *keys;              // [f], or null: no score keys
    int f, RB;
    float bias;
    int act = 0, write_h = 0;    // write_h: G receives h = act(g') u instead of g' (U unused; the dense layer)
};

template <int KC, int NW>
__global__ __launch_bounds__(NW * 64) void k_gu_i4_b1(const GuI4Args a)
{
    constexpr size_t RBYTES = (size_t)KC * 1024;   // d / 2
    constexpr int SST = KC * 16;                   // d / 128
    __shared__ float gsm[kFusedMaxRB], usm[kFusedMaxRB];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r0 = blockIdx.x * a.RB, nr = min(a.RB, a.f - r0);

    float xr[KC][32];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
        const float4 *xp = (const float4 *)(a.x + (size_t)(k * 64 + lane) * 32);
#pragma unroll
        for (int e4 = 0; e4 < 8; ++e4) {
            const float4 v = xp[e4];
            xr[k][4 * e4] = v.x; xr[k][4 * e4 + 1] = v.y; xr[k][4 * e4 + 2] = v.z; xr[k][4 * e4 + 3] = v.w;
        }
    }
    struct RowSlot {
        uint4 g[KC], u[KC];
        uint16_t sg[KC], su[KC];
    };
    auto load = [&](RowSlot &r, int i) {
        const size_t row = (size_t)(r0 + i);
#pragma unroll
        for (int k = 0; k < KC; ++k) {
            const int c = k * 64 + lane;
            r.g[k] = ld16_nt(a.wg + row * RBYTES + (size_t)c * 16);
            r.u[k] = ld16_nt(a.wu + row * RBYTES + (size_t)c * 16);
            r.sg[k] = a.sg[row * SST + (c >> 2)];
            r.su[k] = a.su[row * SST + (c >> 2)];
        }
    };
    auto reduce = [&](const RowSlot &r, int i) {
        float ag = 0.0f, au = 0.0f;
#pragma unroll
        for (int k = 0; k < KC; ++k) {
            ag = chunk_dot<SFFN_W_INT4_G128>(r.g[k], half_bits_to_float(r.sg[k]), xr[k], ag);
            au = chunk_dot<SFFN_W_INT4_G128>(r.u[k], half_bits_to_float(r.su[k]), xr[k], au);
        }
        const float g = wave_tree_sum_dpp(ag), u = wave_tree_sum_dpp(au);
        if (lane == 0) {
            const float gp = g + a.bias;
            if (a.write_h) {
                a.G[r0 + i] = act_f32(a.act, gp) * u;
            } else {
                a.G[r0 + i] = gp;
                a.U[r0 + i] = u;
            }
            gsm[i] = gp;
            usm[i] = u;
        }
    };
    {
        RowSlot ra, rb, rc;
        if (wave < nr) load(ra, wave);
        if (wave + NW < nr) load(rb, wave + NW);
        for (int i = wave; i < nr; i += 3 * NW) {
            if (i + 2 * NW < nr) load(rc, i + 2 * NW);
            reduce(ra, i);
            if (i + NW >= nr) break;
            if (i + 3 * NW < nr) load(ra, i + 3 * NW);
            reduce(rb, i + NW);
            if (i + 2 * NW >= nr) break;
            if (i + 4 * NW < nr) load(rb, i + 4 * NW);
            reduce(rc, i + 2 * NW);
        }
    }
    __syncthreads();
    if (a.keys && (int)threadIdx.x < nr)   // keys = nullptr: g' and u only (the dense layer)
        a.keys[r0 + threadIdx.x] = topk_key(gsm[threadIdx.x], usm[threadIdx.x], a.wdn[r0 + threadIdx.x]);
}

// int4 dense layer for one token, down projection: y_i = sum_j W_down[i][j] h_j
// (+ x_i) with h from the gate + up kernel.  The down projection decides
// nothing, so its order is free.  Each workgroup stages h once in LDS (every
// load issued before the first store; a pad of 4 values after every 32, so
// that the 64 lanes of a wave, each on its own 32-neuron run, spread over the
// banks) and owns kDenseDownRows rows of the natural W_down [d][f]: a wave
// takes one row at a time and requests every 16-byte chunk of it (32 weights
// of one scale group) at once.
constexpr int kDenseDownRows = 8;        // rows per workgroup, two per wave
constexpr int kDenseDownChunks = 8;      // chunks per lane and row: f <= 64 * 8 * 32 = 16384
struct DenseDownArgs {
    const uint8_t *wd;      // W_down int4 [d][f / 2] (element j of a row: nibble j % 2 of byte j / 2)
    const uint16_t *sd;     // fp16 scales [d][f / 128]
    const float *H;         // h [f]
    int d, f;
    const float *resid;     // x [d] or null
    float *out;             // y [d]
};

__device__ __forceinline__ int dense_h_pos(int j) { return j + (j >> 5) * 4; }

__global__ __launch_bounds__(256) void k_dense_down_i4_b1(const DenseDownArgs a)
{
    extern __shared__ float hs[];   // f + f / 8 values
    constexpr int RW = kDenseDownRows / 4;   // rows per wave
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nch = a.f / 32, ng = a.f / 128;
    const size_t rowb = (size_t)a.f / 2;
    // the wave's weights first (they do not wait for h), then h: one round trip
    uint4 wv[RW][kDenseDownChunks];
    uint16_t sv[RW][kDenseDownChunks];
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        const int row = min((int)blockIdx.x * kDenseDownRows + 4 * r + wave, a.d - 1);
#pragma unroll
        for (int i = 0; i < kDenseDownChunks; ++i) {
            const int c = min(lane + 64 * i, nch - 1);   // unconditional: every load in flight at once
            wv[r][i] = ld16_nt(a.wd + (size_t)row * rowb + 16 * (size_t)c);
            sv[r][i] = a.sd[(size_t)row * ng + (c >> 2)];
        }
    }
    {
        f32x4_t hv[kDenseDownChunks * 2];   // f <= 1024 * 2 kDenseDownChunks
#pragma unroll
        for (int i = 0; i < kDenseDownChunks * 2; ++i)
            hv[i] = *(const f32x4_t *)(a.H + min(4 * (int)threadIdx.x + 1024 * i, a.f - 4));
#pragma unroll
        for (int i = 0; i < kDenseDownChunks * 2; ++i) {
            const int j = 4 * (int)threadIdx.x + 1024 * i;
            if (j < a.f) *(f32x4_t *)(hs + dense_h_pos(j)) = hv[i];
        }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < RW; ++r) {
        const int row = (int)blockIdx.x * kDenseDownRows + 4 * r + wave;
        float acc = 0.0f;
#pragma unroll
        for (int i = 0; i < kDenseDownChunks; ++i) {
            const int c = lane + 64 * i;
            if (c >= nch) break;
            const uint32_t w4[4] = {wv[r][i].x, wv[r][i].y, wv[r][i].z, wv[r][i].w};
            const float *hc = hs + dense_h_pos(32 * c);
            float t = 0.0f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const f32x4_t h0 = *(const f32x4_t *)(hc + 8 * k), h1 = *(const f32x4_t *)(hc + 8 * k + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) t = __builtin_fmaf((float)nib(w4[k], e), h0[e], t);
#pragma unroll
                for (int e = 0; e < 4; ++e) t = __builtin_fmaf((float)nib(w4[k], 4 + e), h1[e], t);
            }
            acc = __builtin_fmaf(half_bits_to_float(sv[r][i]), t, acc);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, 64);
        if (lane == 0 && row < a.d) a.out[row] = a.resid ? acc + a.resid[row] : acc;
    }
}

// y = sum over the partials in a fixed order (+ residual): 16 columns per
// workgroup; thread (column, group g) sums partials g, g + 64, g + 128, ...
// with all of its loads issued before the first add, then the 64 groups are
// combined in a fixed order through LDS.
__device__ __forceinline__ void reduce16_block(const float *__restrict__ partial, int P, int BD,
                                               const float *__restrict__ resid, float *__restrict__ out)
{
    __shared__ float red[64][17];
    __shared__ float red2[16][17];
    const int l = threadIdx.x & 15, qg = threadIdx.x >> 4;
    const int col = blockIdx.x * 16 + l;
    float s = 0.0f;
    if (col < BD) {
        for (int q0 = qg; q0 < P; q0 += 64 * 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int q = q0 + 64 * u;
                v[u] = q < P ? partial[(size_t)q * BD + col] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) s += v[u];
        }
    }
    red[qg][l] = s;
    __syncthreads();
    if (qg < 16) {
        float v = 0.0f;
#pragma unroll
        for (int g = 0; g < 4; ++g) v += red[qg * 4 + g][l];
        red2[qg][l] = v;
    }
    __syncthreads();
    if (qg == 0 && col < BD) {
        float y = 0.0f;
        for (int g = 0; g < 16; ++g) y += red2[g][l];
        if (resid) y += resid[col];
        out[col] = y;
    }
}

__global__ __launch_bounds__(1024) void k_reduce16(const float *__restrict__ partial, int P, int BD,
                                                   const float *__restrict__ resid, float *__restrict__ out)
{
    reduce16_block(partial, P, BD, resid, out);
}

// The output of a batched call whose path the device picked: the tile path's
// split sums (as k_down_sum) or the gather path's partials (as k_reduce16), one
// launch for either; the branch is uniform.
__global__ __launch_bounds__(1024) void k_batched_out(const float *__restrict__ partial, int ns, int P, int B, int d,
                                                      const float *__restrict__ resid, float *__restrict__ out,
                                                      const int *__restrict__ path)
{
    if (*path == kPathTiled) {
        const int i4 = blockIdx.x * 4 + (int)threadIdx.x;
        if (threadIdx.x < 4 && i4 < B * d / 4) down_sum4(partial, ns, d, i4, resid, out);
        return;
    }
    reduce16_block(partial, P, B * d, resid, out);
}

// y = sum of the fused kernel's P partials (+ residual) from the blocked layout
// [d/16][P][16]: one workgroup per 16 columns reads its 16 P floats as one
// contiguous block; thread (column c, group g) adds partials g, g + 16, ... in
// order, then the 16 groups are added in order through LDS.
__global__ __launch_bounds__(256) void k_reduce_blk(const float *__restrict__ partial, int P, int d,
                                                    const float *__restrict__ resid, float *__restrict__ out)
{
    __shared__ float red[16][17];
    const int c = threadIdx.x & 15, g = threadIdx.x >> 4;
    const float *base = partial + (size_t)blockIdx.x * P * 16 + c;
    float s = 0.0f;
    // 16 loads in flight per thread: one round trip for P <= 256
    for (int p0 = g; p0 < P; p0 += 16 * 16) {
        float v[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int p = p0 + 16 * u;
            v[u] = p < P ? base[(size_t)p * 16] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) s += v[u];
    }
    red[g][c] = s;
    __syncthreads();
    if (g == 0) {
        float y = 0.0f;
#pragma unroll
        for (int q = 0; q < 16; ++q) y += red[q][c];
        const int col = blockIdx.x * 16 + c;
        out[col] = resid ? y + resid[col] : y;
    }
}

template <int WT>
static hipError_t run_decode_b1(const FusedArgs &a, int KC, int P, hipStream_t st, hipEvent_t evb, hipEvent_t eve)
{
    switch (KC) {
#define CASE_KC(k)                                                                                 \
    case k:                                                                                        \
        SFFN_LAUNCH((k_decode_b1<WT, k>), dim3(P), dim3(kFusedNT), 0, st, evb, eve, a);            \
        return hipGetLastError();
        CASE_KC(1) CASE_KC(2) CASE_KC(3) CASE_KC(4) CASE_KC(5) CASE_KC(6) CASE_KC(7) CASE_KC(8)
#undef CASE_KC
    }
    return hipErrorInvalidValue;
}

// rows per workgroup of the fused batch-1 kernel: one workgroup per CU when
// d_ff allows it, never more than 48 rows
int fused_rows_per_wg(int f) { return std::min(kFusedMaxRB, std::max(1, (f + 255) / 256)); }

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
template <int WT, int BT, int OUT>
static hipError_t run_rowdot(const RowDotArgs &a, hipStream_t st, hipEvent_t evb = nullptr, hipEvent_t eve = nullptr)
{
    using C = Cfg<WT, BT>;
    constexpr bool TWO = (OUT == OUT_GATE_UP || OUT == OUT_DENSE_GU);
    constexpr int RPW = RdCfg<WT, BT, OUT>::RPW;
    const int R = RdCfg<WT, BT, OUT>::NW * RPW;
    const int grid = (a.rows + R - 1) / R;
    SFFN_LAUNCH((k_rowdot<WT, BT, OUT>), dim3(grid), dim3(RdCfg<WT, BT, OUT>::NW * 64), 0, st, evb, eve, a);
    return hipGetLastError();
}

template <int WT, int BT>
static int gate_rows_per_block()
{
    return Cfg<WT, BT>::NW * Cfg<WT, BT>::RPW;
}

// Workgroups of the top-k gather (each owns a range of ceil(f / P) neurons,
// at most 512 at batch 1 and 64 above).  Every one writes a partial y of B d
// floats that the reduce reads back, but fewer partitions were measured slower
// at batch 1 (2048 / 11008 int4, keep 17-50 %: 37.9-43.0 us per step at 128,
// 39.7-54.7 at 64, 48.0-78.6 at 32, against about 36 at 256): a workgroup's
// rows come in batches, one round trip each, so the partition count stays.
static int topk_gather_wgs(int B, int f)
{
    return B <= 1 ? std::max(kGatherWGs, (f + 511) / 512) : std::max(kGatherWGs, (f + 63) / 64);
}

template <int WT, int BT>
static hipError_t run_gather(const GatherArgs &a0, hipStream_t st)
{
    using C = Cfg<WT, BT>;
    GatherArgs a = a0;
    const int P = a.P > 0 ? a.P : kGatherWGs;
    a.maxs = (a.f + P - 1) / P + 1;
    a.stage_x = a.mode != SFFN_MODE_TOPK;
    const size_t lds = (a.stage_x ? (size_t)BT * C::KMAX * 64 * C::E * 4 : 0) + (size_t)a.maxs * BT * 4 +
                       (size_t)a.maxs * 4 + (size_t)(a.nL + 1) * 4;
    // the limit is raised once to the most any call can need (the device's LDS
    // per workgroup), never to one call's request, so a later layer with a
    // larger d_ff or batch still launches
    static std::once_flag once;
    static hipError_t attr_err = hipSuccess;
    static int lds_limit = 0;
    hipError_t e = allow_full_dynamic_lds((const void *)k_gather<WT, BT>, once, attr_err, lds_limit);
    if (e != hipSuccess) return e;
    if (lds > (size_t)lds_limit) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((k_gather<WT, BT>), dim3(P), dim3(C::NW * 64), lds, st, a);
    return hipGetLastError();
}

// int4, 5..16 tokens: h in MFMA lane order (from the top-k sets, or bits ==
// nullptr: G already holds h), the down projection over all of W_down on MFMA,
// and the sum of the d_ff splits plus the residual
static hipError_t down_i4_mfma(const Layer &L, uint8_t *sc, const ScratchLayout &S, const uint32_t *bits,
                               const float *G, const float *U, int B, int act, int use_union, const float *x,
                               float *out, hipStream_t st)
{
    const sffn_layer_desc &D = L.desc;
    const int d = D.d_model, f = D.d_ff;
    hipError_t e;
    uint16_t *hh = (uint16_t *)(sc + S.hsplit), *hl = hh + (size_t)16 * f;
    FormHArgs fh{bits, G, U, B, f, f / 32, act, use_union, hh, hl};
    hipLaunchKernelGGL(k_form_h_i4, dim3(f / 128), dim3(256), 0, st, fh);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    const int ng = f / 128, T = d / (16 * kDownI4Cols);
    const int ns0 = std::max(1, std::min(std::min(ng, kMaxDownSplits), (kDownI4Waves + T - 1) / T));
    const int per = std::min((ng + ns0 - 1) / ns0, kDownI4Groups), ns = (ng + per - 1) / per;
    float *partial = (float *)(sc + S.partial);
    DownI4Args da{L.wd, L.sdt, hh, hl, d, f, per, partial};
    hipLaunchKernelGGL(k_down_i4_mfma, dim3(T, ns), dim3(64), 0, st, da);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(k_down_sum, dim3((B * d / 4 + 255) / 256), dim3(256), 0, st, (const float *)partial, ns, B, d,
                       D.residual ? x : nullptr, out);
    return hipGetLastError();
}

template <int WT, int BT>
static hipError_t decode_typed(const DecodeCall &c, bool forward)
{
    const Layer &L = *c.L;
    const sffn_layer_desc &D = L.desc;
    const int d = D.d_model, f = D.d_ff, B = c.B;
    const ScratchLayout S = scratch_layout(D);
    uint8_t *sc = c.scratch;
    hipStream_t st = c.stream;
    hipError_t e;

    // 9..16 tokens on the tile path: gate and up in one kernel (k_gu_tiles),
    // with the MFMA operand split done by the RMSNorm prologue
    bool gu_fused = false;
    if constexpr (WT == SFFN_W_BF16 && BT == 16)
        gu_fused = forward && c.mode != SFFN_MODE_TOPK && c.mode != SFFN_MODE_DENSE && L.wut &&
                   (c.batch_path ? c.batch_path == kPathTiled : gather_below_permille(B) == 0);
    uint16_t *const xsh = (uint16_t *)(sc + S.xsplit), *const xsl = xsh + (size_t)16 * d;

    const float *xin = c.x;
    if (D.rmsnorm) {
        float *xh = (float *)(sc + S.xhat);
        if (gu_fused)
            hipLaunchKernelGGL(k_rmsnorm_split, dim3(16), dim3(64), 0, st, c.x, xh, B, d, D.eps, xsh, xsl);
        else
            hipLaunchKernelGGL(k_rmsnorm, dim3(B), dim3(64), 0, st, c.x, xh, d, D.eps);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        xin = xh;
    } else if (gu_fused) {
        hipLaunchKernelGGL(k_split_x, dim3((2 * d + 255) / 256), dim3(256), 0, st, xin, B, d, xsh, xsl,
                           (const int *)nullptr, 0, f, 0, (int *)nullptr);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    float *G = (float *)(sc + S.G);
    float *U = (float *)(sc + S.U);
    int *lcnt = (int *)(sc + S.list_cnt);
    int *lidx = (int *)(sc + S.list_idx);

    RowDotArgs r{};
    r.B = B;
    r.mode = c.mode;
    r.act = D.act;
    r.bias = c.bias;
    r.theta = c.theta;

    if constexpr (BT == 1 && WT != SFFN_W_INT4_G128) {
        constexpr int E = Chunk<WT>::E;
        const int KC = d / (64 * E);
        const bool fits = d % (64 * E) == 0 && KC >= 1 && KC <= 8;
        // DENSE at batch 1 is the same streaming kernel over every neuron with
        // no selection, so the dense reference reads its 3 d_model d_ff weights
        // as fast as the sparse path reads its share
        if (c.mode != SFFN_MODE_TOPK && fits) {
            FusedArgs fa{};
            fa.wg = L.wg; fa.wu = L.wu; fa.wdt = L.wdt;
            fa.x = xin;
            fa.G = G;
            fa.partial = (float *)(sc + S.partial);
            fa.list_cnt = lcnt; fa.list_idx = lidx;
            fa.f = f;
            fa.RB = fused_rows_per_wg(f);
            fa.mode = c.mode == SFFN_MODE_DENSE ? SFFN_MODE_ALL : c.mode;
            fa.act = D.act; fa.bias = c.bias; fa.theta = c.theta;
            const int P = (f + fa.RB - 1) / fa.RB;
            hipEvent_t evb = nullptr, eve = nullptr;
            if (forward) L.timer->take(&evb, &eve);
            if ((e = run_decode_b1<WT>(fa, KC, P, st, evb, eve)) != hipSuccess) return e;
            if (c.idx_out || c.count_out) {
                const int maxs = (f + kGatherWGs - 1) / kGatherWGs + 1;
                hipLaunchKernelGGL(k_emit_list, dim3(kGatherWGs), dim3(256), (size_t)(maxs + P + 1) * 4, st,
                                   (const int *)lcnt, (const int *)lidx, P, fa.RB, c.idx_out, c.count_out, maxs,
                                   (const uint32_t *)nullptr, 0);
                if ((e = hipGetLastError()) != hipSuccess) return e;
            }
            if (!forward) return hipSuccess;
            hipLaunchKernelGGL(k_reduce_blk, dim3(d / 16), dim3(256), 0, st, (const float *)(sc + S.partial), P, d,
                               D.residual ? c.x : nullptr, c.out);
            return hipGetLastError();
        }
    }

    if (c.mode == SFFN_MODE_DENSE) {
        if constexpr (WT == SFFN_W_INT4_G128 && BT == 1) {
            // one token: the streaming gate + up kernel (g' and u), then the row-streaming down GEMV
            if (d % 2048 == 0 && d <= 4096 && f <= 64 * kDenseDownChunks * 32) {
                static std::once_flag once;
                static hipError_t err = hipSuccess;
                static int lim = 0;
                if ((e = allow_full_dynamic_lds((const void *)k_dense_down_i4_b1, once, err, lim)) != hipSuccess) return e;
                const size_t lds = (size_t)(f + f / 8) * 4;
                if (lds <= (size_t)lim) {
                    GuI4Args ga{L.wg, L.wu, L.sg, L.su, xin, L.wdn, G, U, nullptr, f, fused_rows_per_wg(f), c.bias,
                                D.act, 1};
                    const int P = (f + ga.RB - 1) / ga.RB;
                    if (d == 2048)
                        hipLaunchKernelGGL((k_gu_i4_b1<1, kGuI4Waves>), dim3(P), dim3(kGuI4Waves * 64), 0, st, ga);
                    else
                        hipLaunchKernelGGL((k_gu_i4_b1<2, kGuI4Waves>), dim3(P), dim3(kGuI4Waves * 64), 0, st, ga);
                    if ((e = hipGetLastError()) != hipSuccess) return e;
                    DenseDownArgs dd{L.wd, L.sd, G, d, f, D.residual ? c.x : nullptr, c.out};
                    hipLaunchKernelGGL(k_dense_down_i4_b1, dim3((d + kDenseDownRows - 1) / kDenseDownRows), dim3(256),
                                       lds, st, dd);
                    return hipGetLastError();
                }
            }
        }
        r.w0 = L.wg; r.s0 = L.sg; r.w1 = L.wu; r.s1 = L.su;
        r.rows = f; r.cols = d; r.x = xin; r.o0 = G;
        if ((e = run_rowdot<WT, BT, OUT_DENSE_GU>(r, st)) != hipSuccess) return e;
        if constexpr (WT == SFFN_W_INT4_G128 && BT >= 8) {
            // int4, 5..16 tokens: the dense down projection on MFMA, as the top-k path's
            if (f / 128 <= kMaxDownSplits * kDownI4Groups)
                return down_i4_mfma(L, sc, S, nullptr, G, nullptr, B, D.act, 1, c.x, c.out, st);
        }
        RowDotArgs q{};
        q.w0 = L.wd; q.s0 = L.sd; q.rows = d; q.cols = f; q.B = B; q.x = G; q.o0 = c.out;
        q.resid = D.residual ? c.x : nullptr;
        return run_rowdot<WT, BT, OUT_DENSE_DOWN>(q, st);
    }

    if constexpr (WT == SFFN_W_BF16 && BT >= 8) {
        if (c.mode != SFFN_MODE_TOPK && c.mode != SFFN_MODE_DENSE && L.wut) {
            const int R = 16;
            uint16_t *hh = (uint16_t *)(sc + S.hsplit), *hl = hh + (size_t)16 * f;
            hipEvent_t evb = nullptr, eve = nullptr;
            if (forward) L.timer->take(&evb, &eve);
            if (gu_fused) {
                // class-split gate and MFMA u side by side, then g', selection, lists and h
                GateClsArgs ga{L.wgt, d, f, B, (float *)(sc + S.gpart)};
                UpUArgs ua{L.wut, xsh, xsl, d, f, B, U};
                SFFN_LAUNCH((k_gate_up_dual<BT>), dim3(2 * (f / 16)), dim3(256), 0, st, evb, eve, ga,
                            (const float *)xin, ua);
                if ((e = hipGetLastError()) != hipSuccess) return e;
                hipLaunchKernelGGL(k_combine_h, dim3(f / 32), dim3(64), 0, st, (const float *)ga.part, (const float *)U,
                                   B, f, c.bias, c.mode, c.theta, D.act, c.use_union, G, lcnt, lidx, hh, hl);
                if ((e = hipGetLastError()) != hipSuccess) return e;
            } else {
                // class-split gate in the fixed order, lists per block of 16 rows
                GateClsArgs ga{L.wgt, d, f, B, (float *)(sc + S.gpart)};
                SFFN_LAUNCH((k_gate_pipe<BT>), dim3(f / kGateClsRows, 4), dim3(256), 0, st, evb, eve, ga,
                            (const float *)xin);
                if ((e = hipGetLastError()) != hipSuccess) return e;
                hipLaunchKernelGGL(k_gate_combine, dim3(f / 64), dim3(64), 0, st, (const float *)ga.part, B, f, c.bias,
                                   c.mode, c.theta, G, lcnt, lidx);
                if ((e = hipGetLastError()) != hipSuccess) return e;
            }
            const int nblk = (f + R - 1) / R;
            if (c.idx_out || c.count_out) {
                const int maxs = (f + kGatherWGs - 1) / kGatherWGs + 1;
                hipLaunchKernelGGL(k_emit_list, dim3(kGatherWGs), dim3(256), (size_t)(maxs + nblk + 1) * 4, st,
                                   (const int *)lcnt, (const int *)lidx, nblk, R, c.idx_out, c.count_out, maxs,
                                   (const uint32_t *)nullptr, 0);
                if ((e = hipGetLastError()) != hipSuccess) return e;
            }
            if (!forward) return hipSuccess;
            // Which forward path: forced by the caller, fixed by the batch size when the
            // gather never wins at it, or else picked on the device from the union size
            // (no host round trip) by the first tile kernel; then both paths are
            // launched, the kernels of the one not picked exit at once, and one output
            // kernel sums whichever partials were written.
            const int thr = gather_below_permille(B);
            const int fixed = c.batch_path ? c.batch_path : (thr == 0 ? (int)kPathTiled : 0);
            int *path = fixed ? nullptr : (int *)(sc + S.path);
            float *partial = (float *)(sc + S.partial);
            const float *resid = D.residual ? c.x : nullptr;
            const int KS = f / 32, T = d / (16 * kDownCols);
            // about 800 waves for the down tiles: split d_ff so that (d / 64) x splits fills the chip
            const int ns0 = std::max(1, std::min(std::min(KS / 4, kMaxDownSplits), (800 + T - 1) / T));
            const int per = ((KS + ns0 - 1) / ns0 + 3) / 4 * 4;
            const int ns = (KS + per - 1) / per;
            if (fixed != kPathGather) {
                // (1) MFMA tiles: up on every W_up block with a selected neuron, down on all of W_down
                if (!gu_fused) {
                    hipLaunchKernelGGL(k_split_x, dim3((2 * d + 255) / 256), dim3(256), 0, st, xin, B, d, xsh, xsl,
                                       (const int *)lcnt, nblk, f, thr, path);
                    if ((e = hipGetLastError()) != hipSuccess) return e;
                    UpTiledArgs ua{L.wut, xsh, xsl, G, lcnt, lidx, d, f, B, c.mode, D.act, c.use_union, c.theta, hh,
                                   hl, path, kPathTiled};
                    hipLaunchKernelGGL(k_up_tiled, dim3(f / (16 * kUpBlocks)), dim3(256), 0, st, ua);
                    if ((e = hipGetLastError()) != hipSuccess) return e;
                }
                DownTiledArgs da{L.wdtl, hh, hl, d, f, per, partial, path, kPathTiled};
                hipLaunchKernelGGL(k_down_tiled, dim3(T, ns), dim3(64), 0, st, da);
                if ((e = hipGetLastError()) != hipSuccess) return e;
                if (fixed == kPathTiled) {
                    hipLaunchKernelGGL(k_down_sum, dim3((B * d / 4 + 255) / 256), dim3(256), 0, st,
                                       (const float *)partial, ns, B, d, resid, c.out);
                    return hipGetLastError();
                }
            }
            // (2) row gather over the union's W_up and W_down^T rows
            GatherArgs g{};
            g.list_cnt = lcnt; g.list_idx = lidx; g.nL = nblk; g.R = R;
            g.G = G; g.U = U; g.bits = nullptr; g.nw32 = f / 32;
            g.x = xin; g.B = B; g.d = d; g.f = f;
            g.wu = L.wu; g.su = L.su; g.wdt = L.wdt; g.sdt = L.sdt;
            g.mode = c.mode; g.act = D.act; g.use_union = c.use_union; g.theta = c.theta;
            g.partial = partial;
            g.idx_out = nullptr; g.count_out = nullptr;
            g.path = path; g.want = kPathGather;
            if ((e = run_gather<WT, BT>(g, st)) != hipSuccess) return e;
            if (fixed == kPathGather)
                hipLaunchKernelGGL(k_reduce16, dim3((B * d + 15) / 16), dim3(1024), 0, st, (const float *)partial,
                                   kGatherWGs, B * d, resid, c.out);
            else
                hipLaunchKernelGGL(k_batched_out, dim3((B * d + 15) / 16), dim3(1024), 0, st, (const float *)partial,
                                   ns, kGatherWGs, B, d, resid, c.out, (const int *)path);
            return hipGetLastError();
        }
    }

    int nL, R;
    const int nw32 = f / 32;
    uint32_t *bits = (uint32_t *)(sc + S.bits);
    r.w0 = L.wg; r.s0 = L.sg; r.rows = f; r.cols = d; r.x = xin; r.o0 = G;
    if (c.mode == SFFN_MODE_TOPK) {
        r.w1 = L.wu; r.s1 = L.su; r.o1 = U;
        r.wdn = L.wdn;
        r.keys = (uint64_t *)(sc + S.keys);
        hipEvent_t evb = nullptr, eve = nullptr;
        if (forward) L.timer->take(&evb, &eve);
        bool done = false;
        if constexpr (WT == SFFN_W_INT4_G128 && BT == 1) {
            if (d % 2048 == 0 && d <= 4096 && f <= kMaxTopkNeurons) {
                GuI4Args ga{L.wg, L.wu, L.sg, L.su, xin, L.wdn, G, U, r.keys, f, fused_rows_per_wg(f), c.bias};
                const int P = (f + ga.RB - 1) / ga.RB;
                if (d == 2048)
                    SFFN_LAUNCH((k_gu_i4_b1<1, kGuI4Waves>), dim3(P), dim3(kGuI4Waves * 64), 0, st, evb, eve, ga);
                else
                    SFFN_LAUNCH((k_gu_i4_b1<2, kGuI4Waves>), dim3(P), dim3(kGuI4Waves * 64), 0, st, evb, eve, ga);
                if ((e = hipGetLastError()) != hipSuccess) return e;
                done = true;
            }
        }
        if (!done && (e = run_rowdot<WT, BT, OUT_GATE_UP>(r, st, evb, eve)) != hipSuccess) return e;

        TopkArgs t{f, c.topk_k, nw32, (const uint64_t *)(sc + S.keys), bits};
        hipLaunchKernelGGL(k_topk, dim3(B), dim3(1024), 0, st, t);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        // the gather takes its share of the union straight from the bit words
        nL = nw32;
        R = 32;
    } else {
        r.list_cnt = lcnt;
        r.list_idx = lidx;
        hipEvent_t evb = nullptr, eve = nullptr;
        if (forward) L.timer->take(&evb, &eve);
        if ((e = run_rowdot<WT, BT, OUT_GATE>(r, st, evb, eve)) != hipSuccess) return e;
        R = gate_rows_per_block<WT, BT>();
        nL = (f + R - 1) / R;
    }

    const bool topk = c.mode == SFFN_MODE_TOPK;
    if (!forward) {
        const int maxs = (f + kGatherWGs - 1) / kGatherWGs + 1;
        hipLaunchKernelGGL(k_emit_list, dim3(kGatherWGs), dim3(256), (size_t)(maxs + nL + 1) * 4, st,
                           (const int *)lcnt, (const int *)lidx, nL, R, c.idx_out, c.count_out, maxs,
                           topk ? (const uint32_t *)bits : nullptr, B);
        return hipGetLastError();
    }

    if constexpr (WT == SFFN_W_INT4_G128 && BT >= 8) {
        // (f <= kMaxTopkNeurons keeps the splits within kMaxDownSplits)
        if (topk && f / 128 <= kMaxDownSplits * kDownI4Groups) {
            // 5..16 tokens: the union is most of d_ff, so the down projection reads
            // all of W_down on MFMA instead of gathering rows
            if (c.idx_out || c.count_out) {
                const int maxs = (f + kGatherWGs - 1) / kGatherWGs + 1;
                hipLaunchKernelGGL(k_emit_list, dim3(kGatherWGs), dim3(256), (size_t)(maxs + nL + 1) * 4, st,
                                   (const int *)lcnt, (const int *)lidx, nL, R, c.idx_out, c.count_out, maxs,
                                   (const uint32_t *)bits, B);
                if ((e = hipGetLastError()) != hipSuccess) return e;
            }
            return down_i4_mfma(L, sc, S, bits, G, U, B, D.act, c.use_union, c.x, c.out, st);
        }
    }

    GatherArgs g{};
    g.list_cnt = lcnt; g.list_idx = lidx; g.nL = nL; g.R = R;
    g.G = G; g.U = U; g.bits = bits; g.nw32 = nw32;
    g.x = xin; g.B = B; g.d = d; g.f = f;
    g.wu = L.wu; g.su = L.su; g.wdt = L.wdt; g.sdt = L.sdt;
    g.mode = c.mode; g.act = D.act; g.use_union = c.use_union; g.theta = c.theta;
    float *partial = (float *)(sc + S.partial);
    g.partial = partial;
    g.idx_out = c.idx_out; g.count_out = c.count_out;
    g.share_bits = 0;
    if (topk) {
        // each workgroup owns a range of R neurons; the ascending list, when asked
        // for, comes from the bit words in a launch of its own
        g.share_bits = 2;
        g.merge_gap = c.merge_gap;
        g.P = topk_gather_wgs(B, f);
        g.R = (f + g.P - 1) / g.P;
        g.idx_out = nullptr;
        g.count_out = nullptr;
        if (c.idx_out || c.count_out) {
            const int maxs = (f + kGatherWGs - 1) / kGatherWGs + 1;
            hipLaunchKernelGGL(k_emit_list, dim3(kGatherWGs), dim3(256), (size_t)(maxs + nL + 1) * 4, st,
                               (const int *)lcnt, (const int *)lidx, nL, R, c.idx_out, c.count_out, maxs,
                               (const uint32_t *)bits, B);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
    }
    if ((e = run_gather<WT, BT>(g, st)) != hipSuccess) return e;

    const int BD = B * d;
    hipLaunchKernelGGL(k_reduce16, dim3((BD + 15) / 16), dim3(1024), 0, st, (const float *)partial,
                       g.P > 0 ? g.P : kGatherWGs, BD, D.residual ? c.x : nullptr, c.out);
    return hipGetLastError();
}

template <int WT>
static hipError_t decode_bt(const DecodeCall &c, bool forward)
{
    if (c.B <= 1) return decode_typed<WT, 1>(c, forward);
    if (c.B <= 4) return decode_typed<WT, 4>(c, forward);
    if (c.B <= 8) return decode_typed<WT, 8>(c, forward);
    if constexpr (WT != SFFN_W_INT4_G128) return decode_typed<WT, 16>(c, forward);
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeCall &c, bool forward)
{
    switch (c.L->desc.wtype) {
    case SFFN_W_F32: return decode_bt<SFFN_W_F32>(c, forward);
    case SFFN_W_BF16: return decode_bt<SFFN_W_BF16>(c, forward);
    default: return decode_bt<SFFN_W_INT4_G128>(c, forward);
    }
}

}  // namespace sffn
