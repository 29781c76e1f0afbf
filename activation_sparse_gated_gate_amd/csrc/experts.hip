// experts.hip -- adaptive expert top-K by routing-probability mass (gfx950).
//
// RedKnot article, section on adaptive expert top-K: how many experts a token
// activates follows its routing probability mass (threshold 0.50 over the
// candidate buckets 3, 4, 5, 6), so confident tokens take few experts and
// diffuse ones more; the per-depth schedule (6 / 5 / 4) caps the largest
// bucket.  One wave per token: the top experts are extracted one by one,
// ranked by probability then lowest index, and their fp32 mass is added in
// rank order until it reaches tau.  The work per round is a handful of wave
// reductions and selects per key, so the kernel is bound by instruction issue
// rather than by the probabilities it reads.
#include <hip/hip_runtime.h>

#include <climits>

#include "dev_common.h"
#include "sffn_internal.h"

namespace sffn {

// fp32 value -> signed 32-bit key in numeric order: non-negative values keep
// their bits, negative ones flip the magnitude bits; -0 is made +0 first so
// that the two compare equal (the index then decides, as for any tie)
__device__ __forceinline__ int order_key(float p)
{
    const int u = __float_as_int(p + 0.0f);
    return u ^ ((u >> 31) & 0x7FFFFFFF);
}

__device__ __forceinline__ float order_value(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF)); }

// Wave-wide maximum / minimum through DPP: within each row of 16 lanes by
// xor 1, xor 2 (quad permutes) and rotations by 4 and 8, then across rows by
// the row-15 and row-31 broadcasts; lane 63 ends with the result.
__device__ __forceinline__ int wave_max(int v)
{
    v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
    v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
    v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x124, 0xF, 0xF, false));   // row_ror 4
    v = max(v, __builtin_amdgcn_update_dpp(INT_MIN, v, 0x128, 0xF, 0xF, false));   // row_ror 8
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x142, 0xA, 0xF, false));         // row_bcast 15
    v = max(v, __builtin_amdgcn_update_dpp(v, v, 0x143, 0xC, 0xF, false));         // row_bcast 31
    return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ int wave_min(int v)
{
    v = min(v, __builtin_amdgcn_update_dpp(INT_MAX, v, 0xB1, 0xF, 0xF, false));
    v = min(v, __builtin_amdgcn_update_dpp(INT_MAX, v, 0x4E, 0xF, 0xF, false));
    v = min(v, __builtin_amdgcn_update_dpp(INT_MAX, v, 0x124, 0xF, 0xF, false));
    v = min(v, __builtin_amdgcn_update_dpp(INT_MAX, v, 0x128, 0xF, 0xF, false));
    v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x142, 0xA, 0xF, false));
    v = min(v, __builtin_amdgcn_update_dpp(v, v, 0x143, 0xC, 0xF, false));
    return __builtin_amdgcn_readlane(v, 63);
}

// The two best keys of one lane in (key desc, slot asc) order, optionally only
// among the keys that rank after (hl, ql), the last expert the lane gave up.
template <int PER>
__device__ __forceinline__ void lane_top2(const int (&key)[PER], bool after, int hl, int ql, int &h1, int &q1,
                                          int &h2, int &q2)
{
    h1 = INT_MIN;
    q1 = PER;
    h2 = INT_MIN;
    q2 = PER;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        int k = key[q];
        if (after) k = (k < hl || (k == hl && q > ql)) ? k : INT_MIN;
        // strict comparisons keep the lower slot first among equal keys
        const bool g1 = k > h1, g2 = k > h2;
        h2 = g1 ? h1 : (g2 ? k : h2);
        q2 = g1 ? q1 : (g2 ? q : q2);
        h1 = g1 ? k : h1;
        q1 = g1 ? q : q1;
    }
}

// One wave per token; lane l holds the keys of experts l, l + 64, ... (PER of
// them, PER = ceil(E / 64)) and keeps its two best.  Round r takes the
// wave-wide maximum m of the lanes' best keys (DPP); the lane holding it (the
// lowest expert index if several lanes tie: a DPP minimum of their indices)
// gives it up and promotes its second best, and only a lane that gives up a
// second expert recomputes its two best among the keys ranking after the last
// one it gave up.  The mass c of the ranked probabilities is added in rank
// order and the rounds stop at the first b >= kmin with c >= tau.  Lanes past E
// load expert E - 1 (in bounds) and hold the lowest key instead.
template <int PER>
__global__ __launch_bounds__(256) void k_expert_select(const float *__restrict__ probs, int T, int E, float tau,
                                                       int kmin, int kmax, int32_t *__restrict__ k_out,
                                                       int32_t *__restrict__ idx_out, float *__restrict__ w_out)
{
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;   // uniform per wave
    const float *p = probs + (size_t)t * E;
    float x[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) x[q] = __builtin_nontemporal_load(p + min(lane + 64 * q, E - 1));   // every load issued before any use
    int key[PER];
#pragma unroll
    for (int q = 0; q < PER; ++q) key[q] = lane + 64 * q < E ? order_key(x[q]) : INT_MIN;
    int h1, q1, h2, q2;
    lane_top2<PER>(key, false, 0, 0, h1, q1, h2, q2);
    bool have2 = true;           // h2 / q2 hold this lane's next expert
    int hl = INT_MAX, ql = -1;   // the last expert this lane gave up
    int sel_j = -1;              // lane r keeps the rank-r expert and its probability
    float sel_p = 0.0f;
    int K = kmax;
    float c = 0.0f;
    for (int r = 0; r < kmax; ++r) {
        const int m = wave_max(h1);
        const uint64_t hit = __ballot(h1 == m);   // never empty: some lane holds m
        int owner;
        if (__builtin_popcountll(hit) == 1) {
            owner = (int)__builtin_ctzll(hit);
        } else {
            const int cand = h1 == m ? lane + 64 * q1 : INT_MAX;
            owner = wave_min(cand) & 63;
        }
        // clamped: only a non-finite input could point past E - 1
        const int j = min(64 * __builtin_amdgcn_readlane(q1, owner) + owner, E - 1);
        const bool refill = __builtin_amdgcn_readlane((int)!have2, owner) != 0;
        if (lane == owner) {
            hl = h1;
            ql = q1;
            h1 = h2;
            q1 = q2;
            have2 = false;
        }
        if (refill) {   // uniform: the owner had already given up its second best
            int a1, b1, a2, b2;
            lane_top2<PER>(key, true, hl, ql, a1, b1, a2, b2);
            if (lane == owner) {
                h1 = a1;
                q1 = b1;
                h2 = a2;
                q2 = b2;
                have2 = true;
            }
        }
        const float v = order_value(m);
        if (lane == r) {
            sel_j = j;
            sel_p = v;
        }
        c = c + v;
        if (r + 1 >= kmin && c >= tau) {
            K = r + 1;
            break;
        }
    }
    if (lane < kmax) {
        idx_out[(size_t)t * kmax + lane] = lane < K ? sel_j : -1;
        // the key's value is the stored probability except for a stored -0
        w_out[(size_t)t * kmax + lane] = lane < K ? (sel_p == 0.0f ? p[sel_j] : sel_p) : 0.0f;
    }
    if (lane == 0) k_out[t] = K;
}

template <int PER>
static void launch_per(const float *probs, int T, int E, float tau, int kmin, int kmax, int32_t *k_out,
                       int32_t *idx_out, float *w_out, hipStream_t st, hipEvent_t evb, hipEvent_t eve)
{
    SFFN_LAUNCH(k_expert_select<PER>, dim3((T + 3) / 4), dim3(256), 0, st, evb, eve, probs, T, E, tau, kmin, kmax,
                k_out, idx_out, w_out);
}

hipError_t launch_expert_select(const float *probs, int T, int E, float tau, int kmin, int kmax, int32_t *k_out,
                                int32_t *idx_out, float *w_out, hipStream_t st, KernelTimer *timer)
{
    if (T == 0) return hipSuccess;
    if (E < 1 || E > kMaxExpertsAbi || kmax > kMaxExpertKAbi) return hipErrorInvalidValue;
    hipEvent_t evb = nullptr, eve = nullptr;
    if (timer) timer->take(&evb, &eve);
#define SFFN_EXPERT_CASE(n)                                                                     \
    case n:                                                                                     \
        launch_per<n>(probs, T, E, tau, kmin, kmax, k_out, idx_out, w_out, st, evb, eve);      \
        break;
    switch ((E + 63) / 64) {   // keys per lane
        SFFN_EXPERT_CASE(1) SFFN_EXPERT_CASE(2) SFFN_EXPERT_CASE(3) SFFN_EXPERT_CASE(4)
        SFFN_EXPERT_CASE(5) SFFN_EXPERT_CASE(6) SFFN_EXPERT_CASE(7) SFFN_EXPERT_CASE(8)
        SFFN_EXPERT_CASE(9) SFFN_EXPERT_CASE(10) SFFN_EXPERT_CASE(11) SFFN_EXPERT_CASE(12)
        SFFN_EXPERT_CASE(13) SFFN_EXPERT_CASE(14) SFFN_EXPERT_CASE(15)
    default:
        launch_per<16>(probs, T, E, tau, kmin, kmax, k_out, idx_out, w_out, st, evb, eve);
        break;
    }
#undef SFFN_EXPERT_CASE
    return hipGetLastError();
}

}  // namespace sffn
