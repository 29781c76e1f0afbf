// prefill.hip -- token-selective prefill FFN (gfx950).
//
// RedKnot article, Algorithm 1 (section on why the FFN is the hidden
// bottleneck) and the section on the token-selective sparse FFN: the FFN runs
// only on the important tokens S, Z[~S] = 0 and X_next = Y + Z.
//   t1 k_token_norms   s_i = ||A_i||_2 (attention output row), sum of squares in
//                      the fixed fp32 order (64 lane accumulators), IEEE sqrt.
//   t2 k_token_select  fp64 cumulative mass of the scores in descending order, in
//                      blocks of 256, shortest prefix reaching mass * total, plus
//                      the last recent_n tokens, plus top-ranked tokens up to
//                      min_keep; mass >= 1, total == 0 or a non-finite total
//                      keeps every token.  When every partial sum is exact in
//                      fp64, a radix select on the score bits finds the prefix
//                      with no sort (one workgroup); otherwise the (score, index)
//                      keys are sorted (chunks of 1024 in LDS, then exact merge
//                      ranks) and the blocked prefix is taken in order.  Writes
//                      the ascending keep list and its length, all on the device
//                      (no host synchronisation).
//   t3 k_gemm_big<GATE_UP> H = SiLU(Y_S W_gate^T) (.) (Y_S W_up^T), bf16 MFMA with
//                      the A rows gathered through the keep list and the gate /
//                      up columns of the same neurons in one tile (the weights
//                      are interleaved in blocks of 32 rows at creation).
//   t4 k_gemm_big<DOWN> Z = H W_down^T; epilogue X_next[S_m] = bf16(Y[S_m] + Z_m),
//                      a scatter through the keep list.
//   k_copy_unkept      X_next[i] = Y[i] for i not kept (skipped when X_next == Y).
// Tiles whose rows start past the device-side count exit at once, so the grid
// is sized for the largest count without a host round trip.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "dev_common.h"

namespace sffn {

// ---------------------------------------------------------------------------
// t1: token norms
// ---------------------------------------------------------------------------
// zero3 (or null): three words the selection kernel that follows finds zero
__global__ __launch_bounds__(256) void k_token_norms(const uint16_t *__restrict__ A, int L, int d,
                                                     float *__restrict__ s, int32_t *__restrict__ zero3)
{
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (zero3 && blockIdx.x == 0 && threadIdx.x < 3) zero3[threadIdx.x] = 0;
    if (row >= L) return;
    const int nch = d / 8;
    const uint8_t *rp = (const uint8_t *)(A + (size_t)row * d);
    float acc = 0.0f;
    constexpr int KB = 8;  // chunk-columns loaded per batch
    for (int k0 = 0; k0 * 64 < nch; k0 += KB) {
        uint4 v[KB];
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const int c = (k0 + k) * 64 + lane;
            v[k] = c < nch ? ld16_nt(rp + (size_t)c * 16) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < KB; ++k) {
            const int c = (k0 + k) * 64 + lane;
            if (c < nch) {
                float w[8];
                unpack<SFFN_W_BF16>(v[k], w);
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(w[e], w[e], acc);
            }
        }
    }
    acc = wave_tree_sum(acc);
    if (lane == 0) s[row] = sqrtf(acc);
}

// ---------------------------------------------------------------------------
// t2: token selection (one launch of ceil(L / 1024) workgroups of 1024 threads)
// ---------------------------------------------------------------------------
struct SelectArgs {
    const float *s;           // L scores; the array spans at least round_up(L, 16) floats
    int L, recent_n, min_keep;
    double mass;
    int32_t *keep, *count;
    int32_t *keep_copy, *count_copy;   // the same list and count in the scratch (for forward without a list)
    uint64_t *chunks;         // ceil(L / 1024) chunks of 1024 keys, each sorted descending
    uint64_t *sorted;         // the L keys in descending order
    // [0] the path taken (0 undecided, 1 exact mass, 2 sorted), [1] chunks
    // sorted, [2] chunks merged; zero when the selection starts
    int32_t *sync;
};

__device__ __forceinline__ uint64_t rank_key(float s, int i)
{
    // descending key order = score descending, then index ascending
    return ((uint64_t)__float_as_uint(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)i);
}

// t2, sorted path, sort in two steps.  tsort_chunk: every workgroup sorts 1024
// keys descending in LDS (padding keys are 0, below every token's key).
// tsort_merge: the keys are unique (the index is part of the key), so the
// global rank of a key is its place in its chunk plus, for every other chunk,
// the number of larger keys there (a binary search); the key is written to that
// rank.  The result is the full descending order.
// the key of lane lane ^ J (J < 64): lane swaps for 32 and 16, a rotation by
// 8 inside a row of 16 for 8, rotations by 4 and 12 for 4 (lane i ^ 4 is
// i - 4 or i + 4), quad permutations for 2 and 1; each half of the key moves
// separately.  Every lane of the wave must be active.
template <int J>
__device__ __forceinline__ uint32_t xchg32(uint32_t v)
{
    const int lane = threadIdx.x & 63;
    if constexpr (J == 32) {
        const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return lane < 32 ? p[1] : p[0];
    } else if constexpr (J == 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (lane & 16) ? p[0] : p[1];
    } else if constexpr (J == 8) {
        return __builtin_amdgcn_update_dpp(0u, v, 0x128, 0xf, 0xf, false);   // row_ror:8
    } else if constexpr (J == 4) {
        const uint32_t dn = __builtin_amdgcn_update_dpp(0u, v, 0x124, 0xf, 0xf, false);   // row_ror:4, lane i - 4
        const uint32_t up = __builtin_amdgcn_update_dpp(0u, v, 0x12C, 0xf, 0xf, false);   // row_ror:12, lane i + 4
        return (lane & 4) ? dn : up;
    } else if constexpr (J == 2) {
        return __builtin_amdgcn_update_dpp(0u, v, 0x4E, 0xf, 0xf, false);    // quad [2,3,0,1]
    } else {
        return __builtin_amdgcn_update_dpp(0u, v, 0xB1, 0xf, 0xf, false);    // quad [1,0,3,2]
    }
}

template <int J>
__device__ __forceinline__ uint64_t xchg64(uint64_t v)
{
    return ((uint64_t)xchg32<J>((uint32_t)(v >> 32)) << 32) | xchg32<J>((uint32_t)v);
}

// one compare-exchange stage of the bitonic network: positions tid and
// tid ^ J inside runs of K; the lower position keeps the larger key when its
// run descends ((tid & K) == 0), the smaller otherwise
template <int K, int J>
__device__ __forceinline__ uint64_t bitonic_step(uint64_t v, uint64_t o, int tid)
{
    const bool lower = (tid & J) == 0, desc = (tid & K) == 0;
    return (lower == desc) ? (v > o ? v : o) : (v < o ? v : o);
}

template <int K, int J>
__device__ __forceinline__ void bitonic_in_wave(uint64_t &v, int tid)
{
    if constexpr (J >= 1) {
        v = bitonic_step<K, J>(v, xchg64<J>(v), tid);
        bitonic_in_wave<K, J / 2>(v, tid);
    }
}

// Bitonic sort of the chunk's 1024 keys, descending, one key per thread.
// Partners less than 64 apart are in the same wave and are exchanged without
// LDS (lane swaps and DPP); the 10 stages with partners 64 or more apart go
// through LDS, double-buffered, one barrier each.
template <int K>
__device__ __forceinline__ void bitonic_merge_k(uint64_t &v, int tid, uint64_t (&buf)[2][1024], int &nb)
{
#pragma unroll
    for (int j = K >> 1; j >= 64; j >>= 1) {
        buf[nb][tid] = v;
        __syncthreads();
        const uint64_t o = buf[nb][tid ^ j];
        nb ^= 1;
        const bool lower = (tid & j) == 0, desc = (tid & K) == 0;
        v = (lower == desc) ? (v > o ? v : o) : (v < o ? v : o);
    }
    bitonic_in_wave<K, (K >> 1) < 32 ? (K >> 1) : 32>(v, tid);
}

__device__ __forceinline__ void tsort_chunk(const SelectArgs &a, int c, uint64_t (&buf)[2][1024])
{
    const int tid = threadIdx.x;
    const int i = c * 1024 + tid;
    uint64_t v = i < a.L ? rank_key(a.s[i], i) : 0ull;
    int nb = 0;
    bitonic_merge_k<2>(v, tid, buf, nb);
    bitonic_merge_k<4>(v, tid, buf, nb);
    bitonic_merge_k<8>(v, tid, buf, nb);
    bitonic_merge_k<16>(v, tid, buf, nb);
    bitonic_merge_k<32>(v, tid, buf, nb);
    bitonic_merge_k<64>(v, tid, buf, nb);
    bitonic_merge_k<128>(v, tid, buf, nb);
    bitonic_merge_k<256>(v, tid, buf, nb);
    bitonic_merge_k<512>(v, tid, buf, nb);
    bitonic_merge_k<1024>(v, tid, buf, nb);
    a.chunks[(size_t)c * 1024 + tid] = v;
}

// The rank search runs on two levels: every chunk's 32 splitters (the last,
// smallest key of each run of 32) say how many whole runs lie above the key,
// then a search inside the one run that straddles it.  The splitter tables
// are small, so the first five steps hit few LDS words; only the last five
// read the full chunks at scattered addresses.
__device__ __forceinline__ void tsort_merge(const SelectArgs &a, int G, int c, uint64_t *all /* [G][1024] */)
{
    const uint64_t *chunks = a.chunks;
    constexpr int GMAX = kMaxPrefillRows / 1024;
    __shared__ uint64_t spl[GMAX][32];
    {
        uint64_t kv[GMAX];
#pragma unroll
        for (int q = 0; q < GMAX; ++q) kv[q] = q < G ? chunks[q * 1024 + threadIdx.x] : 0ull;
#pragma unroll
        for (int q = 0; q < GMAX; ++q) {
            if (q < G) {
                all[q * 1024 + threadIdx.x] = kv[q];
                if ((threadIdx.x & 31) == 31) spl[q][threadIdx.x >> 5] = kv[q];
            }
        }
    }
    __syncthreads();
    const int p = threadIdx.x;
    const uint64_t key = all[c * 1024 + p];   // 0: padding, not written
    // in every other chunk, the number of keys above this key (a chunk is sorted
    // descending): branch-free binary searches of all chunks advanced together
    // (unconditional reads, so the reads of a step are in flight at once).
    // Level 1: runs whose smallest key is above the key, s in 0..32
    int run[GMAX];
#pragma unroll
    for (int c2 = 0; c2 < GMAX; ++c2) run[c2] = 0;
#pragma unroll
    for (int step = 16; step >= 1; step >>= 1) {
        uint64_t q[GMAX];
#pragma unroll
        for (int c2 = 0; c2 < GMAX; ++c2) q[c2] = spl[min(c2, G - 1)][run[c2] + step - 1];
#pragma unroll
        for (int c2 = 0; c2 < GMAX; ++c2)
            if (q[c2] > key) run[c2] += step;
    }
    // run[c2] is 0..31 here; 31 with the last splitter above too means all 32 runs
#pragma unroll
    for (int c2 = 0; c2 < GMAX; ++c2) run[c2] += (run[c2] == 31 && spl[min(c2, G - 1)][31] > key) ? 1 : 0;
    // Level 2: inside run r (when r < 32), the keys above the key
    int lo[GMAX];
#pragma unroll
    for (int c2 = 0; c2 < GMAX; ++c2) lo[c2] = 0;
#pragma unroll
    for (int step = 16; step >= 1; step >>= 1) {
        uint64_t q[GMAX];
#pragma unroll
        for (int c2 = 0; c2 < GMAX; ++c2)
            q[c2] = all[min(c2, G - 1) * 1024 + min(run[c2], 31) * 32 + lo[c2] + step - 1];
#pragma unroll
        for (int c2 = 0; c2 < GMAX; ++c2)
            if (q[c2] > key) lo[c2] += step;
    }
    int rank = p;
#pragma unroll
    for (int c2 = 0; c2 < GMAX; ++c2) {
        if (c2 < G && c2 != c) {
            // the whole table is above when run = 32; else 32 run + the keys of the run above
            // (lo = 31 with its last key above too means 32, impossible: that key is the
            // run's splitter, which is not above)
            rank += run[c2] == 32 ? 1024 : 32 * run[c2] + lo[c2];
        }
    }
    if (key != 0) a.sorted[rank] = key;
}

// Positions in ascending token order of flagged tokens, 1024 threads: bit q of
// a thread's flags is token q * 1024 + tid.  The flagged count of every (round
// q, wave) goes to LDS, one thread per round turns its row into wave offsets,
// then one thread turns the round totals into round offsets (three barriers,
// none between global stores and LDS traffic).  A flagged token of round q then
// sits at qbase[q] + wbase[q][wave] + its rank among the flagged lanes of its
// wave; qbase[16] is the number of flagged tokens.
static_assert(kMaxPrefillRows == 16 * 1024, "16 rounds of 1024 tokens");
struct OrderScan {
    int wbase[16][16];
    int qbase[17];
};

__device__ __forceinline__ void order_scan(uint32_t fb, OrderScan &os)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const uint64_t m = __ballot((fb >> q) & 1u);
        if (lane == 0) os.wbase[q][wave] = __popcll(m);
    }
    __syncthreads();
    if (tid < 16) {
        int run = 0;
        for (int w2 = 0; w2 < 16; ++w2) {
            const int c2 = os.wbase[tid][w2];
            os.wbase[tid][w2] = run;
            run += c2;
        }
        os.qbase[tid] = run;   // the round's total for now
    }
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int q = 0; q < 16; ++q) {
            const int t = os.qbase[q];
            os.qbase[q] = run;
            run += t;
        }
        os.qbase[16] = run;
    }
    __syncthreads();
}

// the position of round q's token of this thread (meaningful when it is flagged);
// every lane of the wave must call it
__device__ __forceinline__ int order_pos(uint32_t fb, int q, const OrderScan &os)
{
    const uint64_t m = __ballot((fb >> q) & 1u);
    return os.qbase[q] + os.wbase[q][threadIdx.x >> 6] + mbcnt64(m);
}

// the ascending keep list of the tokens flagged in onb, into both copies
__device__ __forceinline__ void write_keep(uint32_t onb, const OrderScan &os, int32_t *keep, int32_t *keep_copy)
{
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int pos = order_pos(onb, q, os);
        if ((onb >> q) & 1u) {
            const int i = q * 1024 + (int)threadIdx.x;
            keep[pos] = i;
            keep_copy[pos] = i;
        }
    }
}

// The sorted path's selection, by workgroup 0.  The sorted order is held in LDS as
// the fp32 scores, block by block of kMassBlock entries with one word of
// padding per block (so the 64 threads that each walk one block read
// different banks), and the 16-bit token index of every rank.  The fp64 block
// sums are taken by wave 0 (lane b adds block b in order, keeping the running
// sum after every 32 entries), the block bases by a sequential chain over the
// lanes' totals; the threshold block's scan restarts from its last checkpoint
// below the threshold.  The keep list is built in rounds of 1024 consecutive
// tokens (ballot + mbcnt, wave offsets through LDS), so every store of the list
// is coalesced.
constexpr int kMassPad = kMassBlock + 1;

__device__ __forceinline__ int mass_slot(int r) { return (r / kMassBlock) * kMassPad + (r % kMassBlock); }

__device__ __forceinline__ void select_sorted(const SelectArgs &a, unsigned char *lds_raw)
{
    constexpr int NBMAX = kMaxPrefillRows / kMassBlock;
    constexpr int NCP = kMassBlock / 32;
    const int L = a.L, tid = threadIdx.x, NT = 1024, lane = tid & 63, wave = tid >> 6;
    const int nb = (L + kMassBlock - 1) / kMassBlock;
    float *sc = (float *)lds_raw;                                        // [nb][kMassPad]
    uint16_t *tok = (uint16_t *)(sc + (size_t)nb * kMassPad);             // [L]
    unsigned char *in = (unsigned char *)(tok + ((L + 7) & ~7));          // [L] membership
    __shared__ double blk_base[NBMAX + 1];
    __shared__ double cpt[NBMAX][NCP];
    __shared__ int s_m, s_all;
    __shared__ int tmp[17];

    {
        // all loads first, then the LDS stores (L <= 16 * 1024)
        constexpr int PER = kMaxPrefillRows / 1024;
        uint64_t kv[PER];
#pragma unroll
        for (int q = 0; q < PER; ++q) kv[q] = tid + q * NT < L ? a.sorted[tid + q * NT] : 0ull;
#pragma unroll
        for (int q = 0; q < PER; ++q) {
            const int r = tid + q * NT;
            if (r < L) {
                sc[mass_slot(r)] = __uint_as_float((uint32_t)(kv[q] >> 32));
                tok[r] = (uint16_t)(0xFFFFFFFFu - (uint32_t)kv[q]);
            }
        }
    }
    for (int i = tid; i < L; i += NT) in[i] = 0;
    if (tid == 0) s_m = -1;   // no prefix unless a block finds the threshold
    __syncthreads();
    // fp64 cumulative mass in blocks of kMassBlock sorted entries: lane b of
    // wave 0 adds block b in order (32 values read ahead of the dependent adds)
    // and keeps the running sum after every 32 entries; then the block bases
    // are the sequential sums of the block totals
    if (wave == 0) {
        double run = 0.0;
        if (lane < nb) {
            const int b0 = lane * kMassBlock, b1 = min(L, b0 + kMassBlock);
            const float *sb = sc + (size_t)lane * kMassPad;
            for (int k0 = 0; k0 < b1 - b0; k0 += 32) {
                // the 32 reads are unconditional (a short last block reads padding
                // slots inside the array, masked below), so they are all in flight
                // before the dependent adds
                float v[32];
#pragma unroll
                for (int u = 0; u < 32; ++u) v[u] = sb[k0 + u];
#pragma unroll
                for (int u = 0; u < 32; ++u) v[u] = b0 + k0 + u < b1 ? v[u] : 0.0f;
                if (b0 + k0 + 32 <= b1) {
#pragma unroll
                    for (int u = 0; u < 32; ++u) run = run + (double)v[u];
                } else {
#pragma unroll
                    for (int u = 0; u < 32; ++u)
                        if (b0 + k0 + u < b1) run = run + (double)v[u];
                }
                cpt[lane][k0 >> 5] = run;   // the sum of the block's entries up to k0 + 31
            }
        }
        // block b's base = total of blocks 0 .. b-1, added in order
        double base = 0.0;
        for (int b = 0; b < nb; ++b) {
            if (lane == 0) blk_base[b] = base;
            const double tb = __longlong_as_double(
                ((long long)__builtin_amdgcn_readlane((int)(__double_as_longlong(run) >> 32), b) << 32) |
                (long long)(uint32_t)__builtin_amdgcn_readlane((int)__double_as_longlong(run), b));
            base = base + tb;
        }
        const double total = base;   // equals the last cumulative value
        if (lane == 0) {
            blk_base[nb] = total;
            // a non-finite total (a NaN or infinite score) keeps every token, like an all-zero row
            s_all = (a.mass >= 1.0 || total == 0.0 || !isfinite(total)) ? 1 : 0;
        }
    }
    __syncthreads();
    const bool all = s_all != 0;
    if (!all && a.mass > 0.0) {
        const double thr = a.mass * blk_base[nb];
        // the cumulative mass only grows, and its value at the end of block b is
        // blk_base[b + 1]: the first block whose end reaches thr holds the answer
        if (tid < nb && blk_base[tid + 1] >= thr && (tid == 0 || blk_base[tid] < thr)) {
            const double base = blk_base[tid];
            const int b0 = tid * kMassBlock, b1 = min(L, b0 + kMassBlock);
            const float *sb = sc + (size_t)tid * kMassPad;
            // the 32-entry span where the cumulative mass first reaches thr
            int j = 0;
            while (b0 + 32 * (j + 1) < b1 && base + cpt[tid][j] < thr) ++j;
            double run = j > 0 ? cpt[tid][j - 1] : 0.0;
            const int k0 = 32 * j;
            float v[32];
#pragma unroll
            for (int u = 0; u < 32; ++u) v[u] = sb[k0 + u];   // unconditional, masked below
#pragma unroll
            for (int u = 0; u < 32; ++u) v[u] = b0 + k0 + u < b1 ? v[u] : 0.0f;
            int hit = -1;
#pragma unroll
            for (int u = 0; u < 32; ++u) {
                if (hit < 0 && b0 + k0 + u < b1) {
                    run = run + (double)v[u];
                    if (base + run >= thr) hit = b0 + k0 + u;
                }
            }
            s_m = hit;
        }
        __syncthreads();
        // the shortest prefix: ranks 0..m
        for (int r = tid; r <= s_m; r += NT) in[tok[r]] = 1;
    }
    __syncthreads();
    if (all) {
        for (int i = tid; i < L; i += NT) in[i] = 1;
    } else {
        for (int i = max(0, L - a.recent_n) + tid; i < L; i += NT) in[i] = 1;
    }
    __syncthreads();
    // min_keep: add the highest-ranked tokens not yet kept.  Threads own
    // contiguous runs of ranks; a scan of their not-yet-kept counts tells each
    // thread how many of its tokens are among the first `need` ones.  Nothing
    // to do when the prefix (ranks 0..s_m) already holds min_keep tokens.
    if (a.min_keep > (all ? L : s_m + 1)) {
        int c = 0;
        for (int i = tid; i < L; i += NT) c += in[i];
        int tot;
        block_exclusive_scan(c, tmp, &tot);
        const int need = a.min_keep - tot;
        if (need > 0) {
            const int per = (L + NT - 1) / NT;
            const int r0 = min(L, tid * per), r1 = min(L, r0 + per);
            int free = 0;
            for (int r = r0; r < r1; ++r) free += in[tok[r]] ? 0 : 1;
            int ftot;
            int before = block_exclusive_scan(free, tmp, &ftot);
            for (int r = r0; r < r1 && before < need; ++r) {
                const int i = tok[r];
                if (!in[i]) {
                    in[i] = 1;
                    ++before;
                }
            }
        }
    }
    __syncthreads();
    uint32_t onb = 0;
#pragma unroll
    for (int q = 0; q < kMaxPrefillRows / 1024; ++q) {
        const int i = q * NT + tid;
        onb |= (i < L && in[i]) ? (1u << q) : 0u;
    }
    __shared__ OrderScan os;
    order_scan(onb, os);
    if (tid == 0) {
        *a.count = os.qbase[16];
        *a.count_copy = os.qbase[16];
    }
    write_keep(onb, os, a.keep, a.keep_copy);
}

// ---------------------------------------------------------------------------
// t2, exact-mass path (one workgroup of 1024 threads).
// The scores are >= 0.  Let u be the ulp of the smallest nonzero score: every
// score is an integer multiple of u, and so is every partial sum of scores.
// When the total is at most 2^53 u, every partial sum the blocked fp64 prefix
// forms (inside a block, of the block totals, and a block base plus a partial
// block) is a multiple of u no larger than 2^53 u, so it is an fp64 number:
// each addition is exact, and the prefix at rank m is the exact sum of the
// m + 1 largest scores, whatever the order of the additions.  The shortest
// prefix is then fixed by the threshold score alone, found by a radix select
// on the score bits with the mass of every digit summed as an integer in units
// of u (integer sums do not depend on the order of the atomics).  The ties at
// the threshold score are taken in ascending index order, as the sorted order
// does.  Scores outside the condition (negative, infinite or NaN, more than
// 2^26 between the largest and the smallest nonzero score -- which also keeps
// every integer sum below 2^64 -- or a total above 2^53 u), a threshold that
// underflows to zero, or a min_keep that the prefix and the recent window do
// not reach return 2 without writing anything: the sorted path then makes the
// selection.  Thread t holds the 16 consecutive tokens 16 t .. 16 t + 15.

// exclusive prefix of one int per thread over the 1024 threads (one barrier;
// wcnt[16] must not be reused before another barrier)
__device__ __forceinline__ int block1024_exclusive(int v, int *wcnt, int *total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int incl = wave_incl_scan(v);
    if (lane == 63) wcnt[wave] = incl;
    __syncthreads();
    int below = 0, tot = 0;
#pragma unroll
    for (int w2 = 0; w2 < 16; ++w2) {
        const int t = wcnt[w2];
        tot += t;
        below += w2 < wave ? t : 0;
    }
    *total = tot;
    return below + incl - v;
}

// A finite score >= 0 of bits b is sig(b) * 2^(uexp(b) - 150): the significand
// (with the implicit bit of normal numbers) and the exponent that sets its ulp
// (the exponent field, 1 for subnormals).  In units of u = 2^(emin - 150) it
// is the integer sig(b) << (uexp(b) - emin).  Every digit of the passes below
// lies inside one exponent (the first digit holds the 8 exponent bits), so a
// digit sums the bare significands and its mass in units of u is that sum
// shifted by the digit's exponent: below 2^38 << 26 = 2^64.
__device__ __forceinline__ uint32_t score_sig(uint32_t b) { return (b & 0x7FFFFFu) | (b >= 0x800000u ? 0x800000u : 0u); }
__device__ __forceinline__ int score_uexp(uint32_t b) { return max((int)(b >> 23), 1); }

// The digit (b >> SHIFT) & (NB - 1) of the candidates, the tokens whose bits
// above it equal `prefix` (the first pass: every finite nonzero score): their
// significands summed into hm (zero before).
template <int NB, int SHIFT, bool FIRST>
__device__ __forceinline__ void digit_sums(const uint32_t (&b)[16], uint32_t valid, uint32_t prefix, uint64_t *hm)
{
    constexpr int W = NB == 4096 ? 12 : NB == 1024 ? 10 : 9;
    static_assert((1 << W) == NB, "digit width");
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const bool cand = FIRST ? (b[k] - 1u < 0x7F7FFFFFu) : ((b[k] >> (SHIFT + W)) == prefix);
        if (((valid >> k) & 1u) && cand)
            atomicAdd((unsigned long long *)&hm[(b[k] >> SHIFT) & (NB - 1)], (unsigned long long)score_sig(b[k]));
    }
}

// The digits' masses in units of u, this thread's BPT consecutive digits in
// loc, scanned from the largest digit down starting at `above` (the mass of
// the tokens above every candidate): the one digit where the cumulative mass
// first reaches the threshold.  The threshold is held as the integer need, the
// fewest units of u whose mass reaches thr = mass * T * u in fp64: every
// cumulative mass is an integer m <= 2^53 and m * u is exact, so m * u >= thr
// exactly when m >= need.  FIRST: the total T comes from the same sums; returns
// -1 when T exceeds 2^53 or thr underflows to zero, and sets need.  Returns
// the digit (every thread); `above` becomes the mass above it and `bin` its
// own mass.
template <int BPT, bool FIRST>
__device__ __forceinline__ int digit_find(const uint64_t (&loc)[BPT], int nb, double mass, double u, int emin,
                                          uint64_t &need, uint64_t &above, uint64_t &bin, uint64_t *wtot, int *s_dig,
                                          uint64_t *s_res)
{
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool owns = tid * BPT < nb;
    uint64_t sum = 0;
#pragma unroll
    for (int k = 0; k < BPT; ++k) sum += loc[k];
    const uint64_t incl = wave_incl_scan_u64(sum);
    if (lane == 63) wtot[wave] = incl;
    __syncthreads();
    uint64_t total = 0, below = 0;
#pragma unroll
    for (int w2 = 0; w2 < 16; ++w2) {
        const uint64_t t = wtot[w2];
        total += t;
        below += w2 < wave ? t : 0ull;
    }
    if (FIRST) {
        if (total > (1ull << 53)) return -1;
        const double thr = mass * ((double)total * u);   // mass * total, the total exact
        if (!(thr > 0.0)) return -1;
        // thr / u scales by a power of two: exact unless it underflows, and then
        // (or when it is below 1) the fewest units is 1
        const double q = thr * __longlong_as_double((long long)(150 - emin + 1023) << 52);
        need = q <= 1.0 ? 1ull : (uint64_t)ceil(q);
    }
    uint64_t cum = above + (total - (incl + below));
#pragma unroll
    for (int k = BPT - 1; k >= 0; --k) {
        const uint64_t nxt = cum + loc[k];
        if (owns && nxt >= need && cum < need) {
            *s_dig = tid * BPT + k;
            s_res[0] = cum;
            s_res[1] = loc[k];
        }
        cum = nxt;
    }
    __syncthreads();
    above = s_res[0];
    bin = s_res[1];
    return *s_dig;
}

// returns 1 when it made the selection (keep lists and counts written), 2 when
// the sorted path must.  lds: at least max(4096 words, L ints).
__device__ __forceinline__ int mass_select(const SelectArgs &a, unsigned char *lds)
{
    uint64_t *hm = (uint64_t *)lds;
    __shared__ uint64_t wtot[16];
    __shared__ uint32_t wred[2][16];
    __shared__ int wcnt[2][16];
    __shared__ int s_dig;
    __shared__ uint64_t s_res[2];
    const int L = a.L, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // four 16-byte loads per thread, unconditional: threads past the end read
    // the last 16 floats of the padded array (masked below)
    uint32_t b[16];
    {
        const int base = min(16 * tid, ((L + 15) & ~15) - 16);
        const uint4 *p = (const uint4 *)(a.s + base);
        uint4 v[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) v[m] = p[m];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            b[4 * m] = v[m].x;
            b[4 * m + 1] = v[m].y;
            b[4 * m + 2] = v[m].z;
            b[4 * m + 3] = v[m].w;
        }
    }
    const int nv = min(max(L - 16 * tid, 0), 16);
    const uint32_t valid = nv >= 16 ? 0xFFFFu : (1u << nv) - 1u;
    for (int i = tid; i < 4096; i += 1024) hm[i] = 0ull;
    __syncthreads();   // while the loads are in flight
    // the first digit's sums, and beside them the largest score bits (above
    // 0x7F7FFFFF: negative, infinite or NaN) and the smallest exponent of a
    // nonzero score
    digit_sums<4096, 19, true>(b, valid, 0u, hm);
    uint32_t bmax = 0, emn = 255;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        if ((valid >> k) & 1u) {
            bmax = max(bmax, b[k]);
            if (b[k] - 1u < 0x7F7FFFFFu) emn = min(emn, (uint32_t)score_uexp(b[k]));
        }
    }
    bmax = wave_max_dpp(bmax);
    const uint32_t nemn = wave_max_dpp(255u - emn);
    if (lane == 0) {
        wred[0][wave] = bmax;
        wred[1][wave] = nemn;
    }
    __syncthreads();
    uint32_t gmax = 0, gne = 0;
#pragma unroll
    for (int w2 = 0; w2 < 16; ++w2) {
        gmax = max(gmax, wred[0][w2]);
        gne = max(gne, wred[1][w2]);
    }
    const int emin = 255 - (int)gne;   // 255 when every score is zero
    const int emax = max((int)(gmax >> 23), 1);
    // mass >= 1 keeps every token whatever the scores; so does a zero total
    if (a.mass >= 1.0 || gmax == 0u) {
        for (int i = tid; i < L; i += 1024) {
            a.keep[i] = i;
            a.keep_copy[i] = i;
        }
        if (tid == 0) {
            *a.count = L;
            *a.count_copy = L;
        }
        return 1;
    }
    if (gmax > 0x7F7FFFFFu || emax - emin > 26) return 2;
    bool prefix = false;
    uint32_t sb = 0;
    int j = 0, c_eq = 0;
    if (a.mass > 0.0) {
        const double u = __longlong_as_double((long long)(emin - 150 + 1023) << 52);   // 2^(emin - 150), normal in fp64
        uint64_t need = 0, above = 0, bin = 0;
        int d1;
        {
            // digit d holds exponent max(d >> 4, 1); a nonzero sum has it >= emin
            uint64_t loc[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int d = tid * 4 + k;
                const uint64_t r = hm[d];
                loc[k] = r == 0ull ? 0ull : r << (max(d >> 4, 1) - emin);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) hm[tid * 4 + k] = 0ull;   // for the next pass (after the barriers)
            d1 = digit_find<4, true>(loc, 4096, a.mass, u, emin, need, above, bin, wtot, &s_dig, s_res);
        }
        if (d1 < 0) return 2;
        const int sh = max(d1 >> 4, 1) - emin;   // the exponent of every later candidate
        digit_sums<1024, 9, false>(b, valid, (uint32_t)d1, hm);
        __syncthreads();
        int d2;
        {
            uint64_t loc[1];
            loc[0] = hm[tid] << sh;
            hm[tid] = 0ull;
            d2 = digit_find<1, false>(loc, 1024, a.mass, u, emin, need, above, bin, wtot, &s_dig, s_res);
        }
        digit_sums<512, 0, false>(b, valid, ((uint32_t)d1 << 10) | (uint32_t)d2, hm);
        __syncthreads();
        int d3;
        {
            uint64_t loc[1];
            loc[0] = tid < 512 ? hm[tid] << sh : 0ull;
            d3 = digit_find<1, false>(loc, 512, a.mass, u, emin, need, above, bin, wtot, &s_dig, s_res);
        }
        sb = ((uint32_t)d1 << 19) | ((uint32_t)d2 << 9) | (uint32_t)d3;
        // the digit holds c_eq tokens of score sb (its mass is > 0, so sb > 0);
        // the prefix takes the fewest j of them with above + j q* >= need:
        // 1 <= j <= c_eq since above < need <= above + bin
        const uint64_t qs = (uint64_t)score_sig(sb) << (score_uexp(sb) - emin);
        c_eq = (int)(bin / qs);
        j = (int)((need - above + qs - 1) / qs);
        prefix = true;
    }
    const int r0 = L - min(a.recent_n, L);
    uint32_t onb = 0, tie = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const bool hi = prefix && b[k] > sb;
        const bool eq = prefix && b[k] == sb;
        onb |= (hi || 16 * tid + k >= r0) ? (1u << k) : 0u;
        tie |= eq ? (1u << k) : 0u;
    }
    onb &= valid;
    tie &= valid;
    if (j == c_eq) {
        onb |= tie;
    } else {
        // the j lowest-indexed tokens of score sb
        int nt;
        int r = block1024_exclusive(__popc(tie), wcnt[0], &nt);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            if ((tie >> k) & 1u) {
                onb |= r < j ? (1u << k) : 0u;
                ++r;
            }
        }
    }
    int n;
    int pos = block1024_exclusive(__popc(onb), wcnt[1], &n);
    if (n < a.min_keep) return 2;
    // the list staged in LDS (the digit sums are done with), then stored coalesced
    int32_t *klist = (int32_t *)lds;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        if ((onb >> k) & 1u) klist[pos++] = 16 * tid + k;
    }
    __syncthreads();
    for (int i = tid; i < n; i += 1024) {
        const int32_t v = klist[i];
        a.keep[i] = v;
        a.keep_copy[i] = v;
    }
    if (tid == 0) {
        *a.count = n;
        *a.count_copy = n;
    }
    return 1;
}

// ---------------------------------------------------------------------------
// t2, the selection kernel: ceil(L / 1024) workgroups of 1024 threads.
// Workgroup 0 tries the exact-mass path and publishes the path taken in
// sync[0]; the others wait for it and end when it made the selection.  On the
// sorted path every workgroup sorts its chunk of 1024 keys, all wait until
// every chunk is sorted (sync[1]), each merges its chunk into the full order,
// and workgroup 0 waits for every merge (sync[2]) and makes the selection from
// the sorted order.  At most 16 workgroups, each waiting only for workgroups
// of the same launch, so all of them run at once; every wait is bounded
// (kSpinPolls polls), so every workgroup ends even if one never started, and
// then workgroup 0 writes an empty selection.
// ---------------------------------------------------------------------------
constexpr int kSpinPolls = 1 << 20;   // a few tens of ms

// the value at p once it reaches v, or what it holds after kSpinPolls polls;
// one thread.  The polls are relaxed device-scope loads: an acquire on every
// poll would invalidate the XCD's L2 each time; a caller that then reads data
// published before the word fences once after the wait.
__device__ __forceinline__ int spin_until(int32_t *p, int v)
{
    int x = 0;
    for (int it = 0; it < kSpinPolls; ++it) {
        x = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (x >= v) break;
        __builtin_amdgcn_s_sleep(2);
    }
    return x;
}

// every thread's global stores made visible at device scope, then one arrival
// at *p; when wait_for > 0, the workgroup waits until *p reaches it and returns
// whether it did (every thread), with device-scope acquire
__device__ __forceinline__ bool arrive_and_wait(int32_t *p, int wait_for, int *s_flag)
{
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        __hip_atomic_fetch_add(p, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = wait_for > 0 ? (spin_until(p, wait_for) >= wait_for ? 1 : 0) : 1;
    }
    __syncthreads();
    __threadfence();
    return *s_flag != 0;
}

__global__ __launch_bounds__(1024) void k_token_select(const SelectArgs a)
{
    extern __shared__ __align__(16) unsigned char lds[];
    __shared__ int s_flag;
    const int c = blockIdx.x, G = gridDim.x, tid = threadIdx.x;
    if (c == 0) {
        const int path = mass_select(a, lds);
        // relaxed: the other workgroups use only the word's value (the sorted path
        // reads the scores, written by the previous launch); a release here would
        // write back the XCD's L2
        if (tid == 0) __hip_atomic_store(&a.sync[0], path, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (path == 1) return;
    } else {
        if (tid == 0) s_flag = spin_until(&a.sync[0], 1);
        __syncthreads();
        if (s_flag != 2) return;
    }
    __syncthreads();   // the LDS is reused
    tsort_chunk(a, c, *reinterpret_cast<uint64_t(*)[2][1024]>(lds));
    bool ok = arrive_and_wait(&a.sync[1], G, &s_flag);
    if (ok) tsort_merge(a, G, c, (uint64_t *)lds);
    if (c != 0) {
        arrive_and_wait(&a.sync[2], 0, &s_flag);
        return;
    }
    ok = ok && arrive_and_wait(&a.sync[2], G, &s_flag);
    if (!ok) {
        if (tid == 0) {
            *a.count = 0;
            *a.count_copy = 0;
        }
        return;
    }
    select_sorted(a, lds);
}

// ---------------------------------------------------------------------------
// t3 / t4: gathered bf16 MFMA GEMM,  C[m][n] = sum_k A[m][k] B[n][k]
// ---------------------------------------------------------------------------
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

enum { EPI_GATE_UP = 0, EPI_DOWN = 1 };
// which of the down projection's launches a GemmArgs opens
enum { ROLE_SMALL = 0, ROLE_BIG = 1, ROLE_SPLIT = 2 };

struct GemmArgs {
    const uint16_t *A;      // GATE_UP: Y [L][K] gathered through keep; DOWN: H [Mmax][K]
    const uint16_t *B;      // [N][K]
    int K, N;
    const int32_t *keep;    // kept token indices
    const int32_t *count;   // device count M
    uint16_t *H;            // GATE_UP output [Mmax][N/2]; split DOWN: the partial sums go past its row M
    const uint16_t *Y;      // DOWN: residual rows
    uint16_t *X;            // DOWN: output rows (scatter)
    int ldo;                // row length of H (GATE_UP) or X/Y (DOWN)
    int gate;               // 0: always run; else the role decides from the number of 256 x 256 tiles
    int role;               // ROLE_BIG: tiles >= gate, or a k split; ROLE_SMALL: neither; ROLE_SPLIT: the split's sum
    int units;              // compute units (one workgroup each)
    int hrows;              // DOWN: rows H holds
    int rows;               // tokens of the call: the count and the kept indices are clamped to it
};

// The device-side count and kept indices, clamped to the call's rows: a list
// that did not come from a selection over these rows gives wrong rows, never
// an access outside Y, X or H.
__device__ __forceinline__ int gemm_rows(const GemmArgs &a) { return min(max(*a.count, 0), a.rows); }
__device__ __forceinline__ int kept_row(const GemmArgs &a, int m) { return min(max(a.keep[m], 0), a.rows - 1); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v)
{
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ---------------------------------------------------------------------------
// TM x 256 tiles (TM = 256, or 128 when too few 256-row tiles fill the compute
// units), eight waves of TM / 2 x 64 (blocks of v_mfma_f32_32x32x16_bf16), both
// operands copied global -> LDS asynchronously (global_load_lds_dwordx4) in
// slices of 32 along k, four stages deep (three slices in flight while one is
// consumed).  A copy writes one contiguous kilobyte (sixteen 64-byte rows of 32
// bf16), so the LDS layout is chosen through the source addresses: the 16-byte
// chunk c of row r sits at position c ^ ((r >> 2) & 3), which spreads the rows
// that one MFMA operand read touches over all banks.
// ---------------------------------------------------------------------------
constexpr int BBM = 256, BBN = 256, BBK = 32, BSTAGES = 4;
constexpr int kGemmWaves = 8;   // waves per 256 x 256 workgroup

// The down projection's k ranges when too few 256 x 256 tiles fill the compute
// units (1: no split): among S = 2..8 with K a multiple of 32 S and the S
// partial sums ([S][M][N] fp32) fitting in H's rows past M, the S with the
// fewest tile rounds per unit of work (rounds / S), the smallest on ties.
__device__ __forceinline__ int down_split(const GemmArgs &a, int M)
{
    const int tiles = ((M + BBM - 1) / BBM) * (a.N / BBN);
    int best = 1, br = 0, bs = 0;   // the best cost so far is br / bs (bs = 0: none)
    for (int S = 2; S <= 8; ++S) {
        if (a.K % (S * BBK) != 0) continue;
        if ((size_t)S * M * a.N * 4 > (size_t)(a.hrows - M) * a.K * 2) continue;
        const int r = (tiles * S + a.units - 1) / a.units;
        if (bs == 0 || r * bs < br * S) {
            best = S;
            br = r;
            bs = S;
        }
    }
    return best;
}

// The device-side row count decides between the tile sizes without a host
// round trip: with too few 256 x 256 tiles for the compute units, the k range
// is split over more 256 x 256 workgroups when the partial sums fit, else
// 128 x 256 tiles keep more units busy.
__device__ __forceinline__ bool gemm_gate_open(const GemmArgs &a, int M)
{
    if (a.gate == 0) return true;
    const int big = ((M + BBM - 1) / BBM) * (a.N / BBN);
    if (big >= a.gate) return a.role == ROLE_BIG;
    // the 256 x 256 kernel also runs the split, whose sums ROLE_SPLIT adds
    return (down_split(a, M) > 1) == (a.role != ROLE_SMALL);
}

__device__ __forceinline__ void lds_copy16_pf(const void *g, void *lds_wave_base)
{
    // lane l writes bytes [16 l, 16 l + 16) of the 1 KB LDS block whose
    // (wave-uniform) address goes in M0; inline assembly keeps the compiler's
    // wait insertion from draining every copy in flight before each LDS read
    // (the kernel waits on the vector-memory counter itself).  Nothing else in
    // this kernel uses M0.
    const uint32_t la = __builtin_amdgcn_readfirstlane(
        (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void *)lds_wave_base);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(la) : "memory");
}

constexpr int gemm_waitcnt_vm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

// TM x 256 tiles (TM = 256 or 128 rows).  NW waves per workgroup: 4 (2 x 2
// waves of 128 x 128, TM = 256) or 8 (2 x 4 waves of TM / 2 x 64, two waves per
// SIMD; waves w and w + 4 share a SIMD, and the two groups of four alternate
// between reading a slice's fragments and issuing its products, so each SIMD's
// matrix unit is fed while the other wave reads)
template <int EPI, int NW, int TM>
__global__ __launch_bounds__(NW * 64) void k_gemm_big(const GemmArgs a)
{
    static_assert((NW == 4 && TM == 256) || (NW == 8 && (TM == 256 || TM == 128)), "tile shape");
    constexpr int WNN = NW / 2;            // waves along n
    constexpr int JB = 8 / WNN;            // 32-column blocks per wave (4 or 2)
    constexpr int WM = TM / 2;             // rows per wave (128 or 64)
    constexpr int IB = WM / 32;            // 32-row blocks per wave (4 or 2)
    constexpr int QAA = TM / NW / 16;      // 16-row copies of A per wave and stage (4, 2 or 1)
    constexpr int QAB = BBN / NW / 16;     // 16-row copies of B per wave and stage (4 or 2)
    __shared__ __align__(1024) uint16_t As[BSTAGES][TM * BBK];
    __shared__ __align__(1024) uint16_t Bs[BSTAGES][BBN * BBK];
    __shared__ int rowsrc[TM];
    __shared__ int rowtok[TM];   // DOWN: the kept token of each tile row (the epilogue's scatter)

    const int M = gemm_rows(a);
    if (!gemm_gate_open(a, M)) return;
    // the down projection in 256 x 256 tiles with too few of them: S k ranges of
    // K / S each, S work items per tile, fp32 partial sums instead of the epilogue
    int S = 1;
    if constexpr (EPI == EPI_DOWN && TM == 256)
        if (a.gate != 0 && ((M + BBM - 1) / BBM) * (a.N / BBN) < a.gate) S = down_split(a, M);
    const int mt = (M + TM - 1) / TM;
    const int nt = a.N / BBN;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = w / WNN, wn = w % WNN;
    const int KT = a.K / BBK / S;
    // per wave and stage: QAA copies of A rows and QAB of B rows
    constexpr int CPS = QAA + QAB;

    // Workgroups are dealt to the 8 XCDs round-robin; renumbering them so that
    // each XCD walks a contiguous run of tiles (M-tiles fastest) keeps the
    // workgroups that share a weight tile on the same L2.
    const int G = gridDim.x;
    const int v = (G % 8 == 0) ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
    for (int tile = v; tile < mt * nt * S; tile += G) {
        const int tm = tile % mt, ts = (tile / mt) % S, tn = tile / (mt * S);
        const int m0 = tm * TM, n0 = tn * BBN;
        const int k0 = ts * (a.K / S);   // first k of the item's range
        __syncthreads();
        if (tid < TM) {
            // rows past M read a valid row; their results are not written
            const int m = min(m0 + tid, M - 1);
            rowsrc[tid] = EPI == EPI_GATE_UP ? kept_row(a, m) : m;
            if constexpr (EPI == EPI_DOWN) rowtok[tid] = kept_row(a, m);
        }
        __syncthreads();
        // this wave copies rows 16 Q w + 16 q + (lane >> 2), q < Q, of each operand
        // (Q = QAA for A, QAB for B); lane position p = lane & 3 holds logical
        // chunk p ^ ((r >> 2) & 3)
        constexpr int RWA = 16 * QAA, RWB = 16 * QAB;   // rows copied per wave
        uint32_t aoff[QAA];   // element offsets of the gathered A rows (< 2^31 for every supported shape)
#pragma unroll
        for (int q = 0; q < QAA; ++q) {
            const int r = RWA * w + 16 * q + (lane >> 2);
            aoff[q] = (uint32_t)rowsrc[r] * (uint32_t)a.K + (uint32_t)(((lane & 3) ^ ((r >> 2) & 3)) * 8);
        }
        // (r >> 2) & 3 does not depend on q (16 q only changes higher bits)
        const int rb0 = RWB * w + (lane >> 2);
        const uint16_t *bsrc = a.B + (size_t)(n0 + rb0) * a.K + k0 + (((lane & 3) ^ ((rb0 >> 2) & 3)) * 8);
        auto issue = [&](int kt) {
            const int st = kt % BSTAGES;
#pragma unroll
            for (int q = 0; q < QAA; ++q)
                lds_copy16_pf(a.A + aoff[q] + (size_t)(k0 + kt * BBK), &As[st][(RWA * w + 16 * q) * BBK]);
#pragma unroll
            for (int q = 0; q < QAB; ++q)
                lds_copy16_pf(bsrc + (size_t)q * 16 * a.K + (size_t)kt * BBK, &Bs[st][(RWB * w + 16 * q) * BBK]);
        };

        f32x16 acc[IB][JB];
#pragma unroll
        for (int i = 0; i < IB; ++i)
#pragma unroll
            for (int j = 0; j < JB; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

        // the slice's operand fragments of this wave, from LDS into registers
        bf16x8 fa[BBK / 16][IB], fb[BBK / 16][JB];
        auto read_frags = [&](int kt) {
            const uint16_t *as = As[kt % BSTAGES], *bs = Bs[kt % BSTAGES];
#pragma unroll
            for (int ks = 0; ks < BBK / 16; ++ks) {
                const int kc = 2 * ks + (lane >> 5);
#pragma unroll
                for (int i = 0; i < IB; ++i) {
                    const int r = wm * WM + i * 32 + (lane & 31);
                    fa[ks][i] = *(const bf16x8 *)&as[r * BBK + ((kc ^ ((r >> 2) & 3)) * 8)];
                }
#pragma unroll
                for (int j = 0; j < JB; ++j) {
                    const int c = wn * 32 * JB + j * 32 + (lane & 31);
                    fb[ks][j] = *(const bf16x8 *)&bs[c * BBK + ((kc ^ ((c >> 2) & 3)) * 8)];
                }
            }
        };
        auto products = [&]() {
#pragma unroll
            for (int ks = 0; ks < BBK / 16; ++ks)
#pragma unroll
                for (int i = 0; i < IB; ++i)
#pragma unroll
                    for (int j = 0; j < JB; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks][i], fb[ks][j], acc[i][j], 0, 0, 0);
        };
        // wait until this wave's copies of slice kt have landed, given the
        // slices issued after it (lgkm0: and every LDS read of this wave)
        auto wait_slice = [&](int kt, bool lgkm0) {
            const int later = min(min(KT - 1, kt + BSTAGES - 2) - kt, BSTAGES - 2);
            const int n = later >= 2 ? 2 * CPS : later == 1 ? CPS : 0;
            if (lgkm0) {
                if (n == 2 * CPS) __builtin_amdgcn_s_waitcnt(gemm_waitcnt_vm(2 * CPS) & ~(0xF << 8));
                else if (n == CPS) __builtin_amdgcn_s_waitcnt(gemm_waitcnt_vm(CPS) & ~(0xF << 8));
                else __builtin_amdgcn_s_waitcnt(gemm_waitcnt_vm(0) & ~(0xF << 8));
            } else {
                if (n == 2 * CPS) __builtin_amdgcn_s_waitcnt(gemm_waitcnt_vm(2 * CPS));
                else if (n == CPS) __builtin_amdgcn_s_waitcnt(gemm_waitcnt_vm(CPS));
                else __builtin_amdgcn_s_waitcnt(gemm_waitcnt_vm(0));
            }
        };

        for (int p = 0; p < BSTAGES - 1; ++p)
            if (p < KT) issue(p);
        if constexpr (NW == 8) {
            // Two groups of four waves, one wave of each per SIMD, one phase
            // apart: while the waves of one group issue a slice's products, the
            // other group's waves read their fragments of the slice and issue
            // their copies, so every SIMD has products to run across the
            // barriers.  Phases are separated by workgroup barriers; the lead
            // group (waves 0-3) reads slice kt in phase 2 kt - 1 and multiplies
            // in phase 2 kt, the other one phase later.  The stage of slice kt
            // is refilled (slice kt + 4) from phase 2 kt + 1 on, after the
            // second group's reads of it have completed; every wave's copies of
            // slice kt + 1 have landed by the barrier that opens phase 2 kt + 1.
            // Both groups take the same number of barriers: the second one more
            // at the start, the lead one more at the end.
            const bool lead = w < NW / 2;
            wait_slice(0, false);
            __builtin_amdgcn_s_barrier();
            if (!lead) __builtin_amdgcn_s_barrier();
            for (int kt = 0; kt < KT; ++kt) {
                __builtin_amdgcn_sched_barrier(0);
                read_frags(kt);
                if (kt + BSTAGES - 1 < KT) issue(kt + BSTAGES - 1);
                // the second group's reads must be complete before the stage can
                // be refilled; its copies of slice kt + 1 must have landed
                if (!lead) wait_slice(kt + 1, true);
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_barrier();
                __builtin_amdgcn_sched_barrier(0);
                products();
                __builtin_amdgcn_sched_barrier(0);
                if (lead) wait_slice(kt + 1, false);
                __builtin_amdgcn_s_barrier();
            }
            if (lead) __builtin_amdgcn_s_barrier();
        } else {
            for (int kt = 0; kt < KT; ++kt) {
                // every wave's copies of slice kt are in LDS, and every wave has
                // finished slice kt - 1, whose stage the next copies refill
                wait_slice(kt, false);
                __builtin_amdgcn_s_barrier();
                // every operand fragment of the slice is read from LDS before the
                // first product, so only the first two reads' latency is exposed;
                // the refill of the stage finished two slices ago goes out behind them
                read_frags(kt);
                if (kt + BSTAGES - 1 < KT) issue(kt + BSTAGES - 1);
                __builtin_amdgcn_sched_barrier(0);
                products();
            }
        }
        __builtin_amdgcn_s_barrier();   // the next tile's first copies reuse the stages

        // epilogue: lane holds col = lane & 31 and rows 8 g + 4 (lane >> 5) + e of a 32 x 32 block
        const int ccol = lane & 31;
        if constexpr (EPI == EPI_GATE_UP) {
            // wave columns: [gate | up] of neurons nb .. nb + 31 (then of nb + 32 .. nb + 63)
            const int nb = (n0 + wn * 32 * JB) / 2;
#pragma unroll
            for (int i = 0; i < IB; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    __builtin_amdgcn_sched_barrier(0);   // bound the live values of the epilogue
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int m = m0 + wm * WM + i * 32 + 8 * g + 4 * (lane >> 5) + e;
                        if (m < M) {
#pragma unroll
                            for (int hb = 0; hb < JB / 2; ++hb) {
                                const float gv = acc[i][2 * hb][4 * g + e], uv = acc[i][2 * hb + 1][4 * g + e];
                                const float h = gv / (1.0f + expf(-gv)) * uv;
                                a.H[(size_t)m * a.ldo + nb + 32 * hb + ccol] = f32_to_bf16_rne(h);
                            }
                        }
                    }
                }
        } else if (S > 1) {
            // the item's fp32 partial sums of rows m < M: [S][M][N] past H's row M
            float *part = (float *)(a.H + (size_t)M * a.K) + (size_t)ts * M * a.N;
#pragma unroll
            for (int i = 0; i < IB; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int m = m0 + wm * WM + i * 32 + 8 * g + 4 * (lane >> 5) + e;
                        if (m < M) {
#pragma unroll
                            for (int j = 0; j < JB; ++j)
                                part[(size_t)m * a.N + n0 + wn * 32 * JB + j * 32 + ccol] = acc[i][j][4 * g + e];
                        }
                    }
                }
        } else {
            // per group of 4 rows: the residual values first (rows past M read
            // their clamped row), then the guarded stores
#pragma unroll
            for (int i = 0; i < IB; ++i)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    __builtin_amdgcn_sched_barrier(0);
                    const int rl0 = wm * WM + i * 32 + 8 * g + 4 * (lane >> 5);
                    float y[4][JB];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
#pragma unroll
                        for (int j = 0; j < JB; ++j)
                            y[e][j] = bf16_lo(a.Y[(size_t)rowtok[rl0 + e] * a.ldo + n0 + wn * 32 * JB + j * 32 + ccol]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        if (m0 + rl0 + e < M) {
#pragma unroll
                            for (int j = 0; j < JB; ++j)
                                a.X[(size_t)rowtok[rl0 + e] * a.ldo + n0 + wn * 32 * JB + j * 32 + ccol] =
                                    f32_to_bf16_rne(y[e][j] + acc[i][j][4 * g + e]);
                        }
                    }
                }
        }
    }
}

// The split down projection's partial sums added in k-range order, then the
// residual and the scatter: X[keep[m]][n] = bf16(Y[keep[m]][n] + sum_s part[s][m][n]),
// four columns per thread.
__global__ __launch_bounds__(256) void k_split_reduce(const GemmArgs a)
{
    const int M = gemm_rows(a);
    if (!gemm_gate_open(a, M)) return;
    const int S = down_split(a, M);
    const float *part = (const float *)(a.H + (size_t)M * a.K);
    const int q4 = a.N / 4;
    const size_t total = (size_t)M * q4;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (size_t)gridDim.x * 256) {
        const int m = (int)(i / q4), n = (int)(i % q4) * 4;
        float4 z = *(const float4 *)(part + (size_t)m * a.N + n);
        for (int t = 1; t < S; ++t) {
            const float4 p = *(const float4 *)(part + ((size_t)t * M + m) * a.N + n);
            z.x += p.x;
            z.y += p.y;
            z.z += p.z;
            z.w += p.w;
        }
        const size_t o = (size_t)kept_row(a, m) * a.ldo + n;
        const float y0 = bf16_lo(a.Y[o]), y1 = bf16_lo(a.Y[o + 1]), y2 = bf16_lo(a.Y[o + 2]), y3 = bf16_lo(a.Y[o + 3]);
        a.X[o] = f32_to_bf16_rne(y0 + z.x);
        a.X[o + 1] = f32_to_bf16_rne(y1 + z.y);
        a.X[o + 2] = f32_to_bf16_rne(y2 + z.z);
        a.X[o + 3] = f32_to_bf16_rne(y3 + z.w);
    }
}

// flags[i] = 1 iff i is in the ascending keep list (binary search per token)
__global__ __launch_bounds__(256) void k_fill_flags(int32_t *__restrict__ flags, int L, const int32_t *__restrict__ keep,
                                                    const int32_t *__restrict__ count)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= L) return;
    const int n = min(max(*count, 0), L);
    int lo = 0, hi = n;  // search [lo, hi)
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (keep[mid] < i) lo = mid + 1; else hi = mid;
    }
    flags[i] = (lo < n && keep[lo] == i) ? 1 : 0;
}

// X_next rows of tokens that are not kept: a copy of Y
__global__ __launch_bounds__(256) void k_copy_unkept(const uint16_t *__restrict__ Y, uint16_t *__restrict__ X,
                                                     const int32_t *__restrict__ flags, int d)
{
    const int row = blockIdx.x;
    if (flags[row]) return;
    const uint4 *src = (const uint4 *)(Y + (size_t)row * d);
    uint4 *dst = (uint4 *)(X + (size_t)row * d);
    for (int i = threadIdx.x; i < d / 8; i += 256) dst[i] = src[i];
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_token_norms(const uint16_t *A, int rows, int d, float *s, hipStream_t st)
{
    hipLaunchKernelGGL(k_token_norms, dim3((rows + 3) / 4), dim3(256), 0, st, A, rows, d, s, (int32_t *)nullptr);
    return hipGetLastError();
}

hipError_t launch_prefill_select(const PrefillSelectCall &c)
{
    const Layer &L = *c.L;
    const int d = L.desc.d_model, rows = c.rows;
    const ScratchLayout S = scratch_layout(L.desc);
    float *sc_s = (float *)(c.scratch + S.tscore);
    int32_t *sync = (int32_t *)(c.scratch + S.tdone);
    hipLaunchKernelGGL(k_token_norms, dim3((rows + 3) / 4), dim3(256), 0, c.stream, c.A, rows, d, sc_s, sync);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // dynamic LDS, the largest of: the exact-mass digits (4096 words), a chunk
    // sort (2 x 1024 keys), the merge (every chunk), the sorted selection (scores
    // in padded blocks, 16-bit token indices, membership bytes)
    const int G = (rows + 1023) / 1024;   // <= kMaxPrefillRows / 1024 = 16
    const size_t lds_sel = (size_t)((rows + kMassBlock - 1) / kMassBlock) * kMassPad * 4 +
                           (size_t)((rows + 7) & ~7) * 2 + (size_t)rows;
    const size_t lds = std::max(std::max((size_t)4096 * 8, (size_t)G * 1024 * 8), lds_sel);
    static std::once_flag once_sel;
    static hipError_t err_sel = hipSuccess;
    static int lim_sel = 0;
    if ((e = allow_full_dynamic_lds((const void *)k_token_select, once_sel, err_sel, lim_sel)) != hipSuccess) return e;
    if (lds > (size_t)lim_sel) return hipErrorInvalidConfiguration;
    SelectArgs a{sc_s, rows, c.recent_n, c.min_keep, c.mass, c.idx_out, c.count_out,
                 (int32_t *)(c.scratch + S.tkeep), (int32_t *)(c.scratch + S.tkcnt),
                 (uint64_t *)(c.scratch + S.tkeys), (uint64_t *)(c.scratch + S.tsorted), sync};
    hipLaunchKernelGGL(k_token_select, dim3(G), dim3(1024), lds, c.stream, a);
    return hipGetLastError();
}

// compute units of the current device, a multiple of 8 when possible
static int gemm_grid(hipStream_t)
{
    const int n = compute_units();
    return n >= 8 ? n / 8 * 8 : n;
}

hipError_t launch_prefill_forward(const PrefillForwardCall &c)
{
    const Layer &L = *c.L;
    const int d = L.desc.d_model, f = L.desc.d_ff, rows = c.rows;
    const ScratchLayout S = scratch_layout(L.desc);
    uint16_t *H = (uint16_t *)(c.scratch + S.pH);
    int32_t *flags = (int32_t *)(c.scratch + S.tflag);
    hipError_t e;
    if (c.X != c.Y) {
        // flags come from the keep list: rebuild them here so that forward does
        // not depend on a previous select call on the same scratch
        hipLaunchKernelGGL(k_fill_flags, dim3((rows + 255) / 256), dim3(256), 0, c.stream, flags, rows, c.keep,
                           c.count);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        hipLaunchKernelGGL(k_copy_unkept, dim3(rows), dim3(256), 0, c.stream, c.Y, c.X, (const int32_t *)flags, d);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    GemmArgs g{};
    g.A = c.Y; g.B = L.wgu; g.K = d; g.N = 2 * f; g.keep = c.keep; g.count = c.count; g.H = H; g.ldo = f;
    g.rows = rows;
    const int mt_big = (c.L->desc.max_rows + BBM - 1) / BBM;
    const int tiles1 = mt_big * (2 * f / BBN);
    hipEvent_t evb = nullptr, eve = nullptr;
    L.timer->take(&evb, &eve);
    // one workgroup per compute unit (128 KB of LDS each), looping over tiles
    const int G = gemm_grid(c.stream);
    SFFN_LAUNCH((k_gemm_big<EPI_GATE_UP, kGemmWaves, 256>), dim3(std::min(tiles1, G)), dim3(kGemmWaves * 64), 0, c.stream,
                evb, eve, g);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    GemmArgs g2{};
    g2.A = H; g2.B = L.wdp; g2.K = f; g2.N = d; g2.keep = c.keep; g2.count = c.count; g2.Y = c.Y; g2.X = c.X;
    g2.ldo = d;
    g2.rows = rows;
    g2.H = H;
    g2.hrows = L.desc.max_rows;
    g2.units = G;
    // down projection: 256 x 256 tiles when they fill at least half of the compute
    // units; else the k range split over more 256 x 256 workgroups with a
    // fixed-order sum of the partial sums when they fit in H's free rows, else
    // 128 x 256 tiles (all launched; the device-side count opens one path)
    const int tiles2 = mt_big * (d / BBN);
    // measured: 220 tiles of 256 rows on 256 units beat 420 of 128 rows (2.15 against
    // 2.44 ms per FFN at 2674 rows)
    g2.gate = G / 2;
    g2.role = ROLE_BIG;
    hipLaunchKernelGGL((k_gemm_big<EPI_DOWN, kGemmWaves, 256>), dim3(std::max(1, std::min(tiles2 * 8, G))),
                       dim3(kGemmWaves * 64), 0, c.stream, g2);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    g2.role = ROLE_SPLIT;
    hipLaunchKernelGGL(k_split_reduce, dim3(4 * G), dim3(256), 0, c.stream, g2);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    g2.role = ROLE_SMALL;
    const int tiles2s = ((rows + 127) / 128) * (d / BBN);
    hipLaunchKernelGGL((k_gemm_big<EPI_DOWN, kGemmWaves, 128>), dim3(std::min(tiles2s, G)), dim3(kGemmWaves * 64), 0,
                       c.stream, g2);
    return hipGetLastError();
}

}  // namespace sffn
