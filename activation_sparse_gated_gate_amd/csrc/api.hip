// api.hip -- the C ABI of libsffn: descriptor validation, workspace layout and
// dispatch to the gfx950 kernels.  Every entry point validates its arguments
// before any launch and reports problems through the status code.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <new>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "sffn_internal.h"
#include "../../include/sffn_diag.h"

namespace sffn {

static thread_local char g_hip_err[256] = "";

static sffn_status hip_status(hipError_t e)
{
    if (e == hipSuccess) return SFFN_OK;
    snprintf(g_hip_err, sizeof g_hip_err, "%s: %s", hipGetErrorName(e), hipGetErrorString(e));
    return SFFN_ERR_HIP;
}

PersistentLayout persistent_layout(const sffn_layer_desc &D)
{
    PersistentLayout P{};
    const int d = D.d_model, f = D.d_ff, wt = D.wtype;
    const size_t mat = row_bytes(wt, d) * (size_t)f;
    const size_t scl_f = wt == SFFN_W_INT4_G128 ? (size_t)f * (d / 128) * 2 : 0;  // [f][d/128]
    const size_t scl_d = wt == SFFN_W_INT4_G128 ? (size_t)d * (f / 128) * 2 : 0;  // [d][f/128] or transposed
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align256(o + bytes);
        return at;
    };
    const bool dec = D.layouts & SFFN_LAYOUT_DECODE;
    const bool pre = D.layouts & SFFN_LAYOUT_PREFILL;
    P.wg = dec ? take(mat) : 0;
    P.sg = dec ? take(scl_f) : 0;
    P.wu = dec ? take(mat) : 0;
    P.su = dec ? take(scl_f) : 0;
    P.wdt = dec ? take(mat) : 0;
    P.sdt = dec ? take(scl_d) : 0;
    P.wdn = dec ? take((size_t)f * 8) : 0;
    P.wd = take(mat);
    P.sd = take(scl_d);
    P.wgu = pre ? take(2 * mat) : 0;
    P.wdp = P.wd;
    const bool bat = dec && (D.layouts & SFFN_LAYOUT_BATCH);
    P.wut = bat ? take(mat) : 0;
    P.wdtl = bat ? take(mat) : 0;
    // class-tiled W_gate: 4 x ceil(d / 512) x f x 256 bytes (d % 512 == 256 pads a half slice)
    P.wgt = bat ? take((size_t)4 * ((d / 8 + 63) / 64) * f * 256) : 0;
    P.total = o;
    return P;
}

ScratchLayout scratch_layout(const sffn_layer_desc &D)
{
    ScratchLayout S{};
    const int d = D.d_model, f = D.d_ff;
    const size_t B = (size_t)D.max_rows;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align256(o + bytes);
        return at;
    };
    if (D.layouts & SFFN_LAYOUT_DECODE) {
        S.xhat = take(B * d * 4);
        S.G = take(B * f * 4);
        // u; the batched tile path keeps one partial per half of d_model
        S.U = take((D.layouts & SFFN_LAYOUT_BATCH ? 2 : 1) * B * f * 4);
        S.keys = take(B * f * 8);
        S.bits = take(B * (f / 32) * 4);
        S.list_cnt = take((size_t)f * 4);
        S.list_idx = take(((size_t)f + 64) * 4);
        // partial sums: kGatherWGs per token for the batched gather; the batch-1
        // fused kernel uses ceil(f / RB) <= max(256, ceil(f / 48)) workgroups
        S.partial = take(std::max((size_t)kGatherWGs * B, (size_t)(f + 47) / 48 + 256) * d * 4);
        S.xsplit = take((size_t)2 * 16 * d * 2);   // x_hat as bf16 hi / lo, 16 token slots
        S.hsplit = take((size_t)2 * 16 * f * 2);   // h as bf16 hi / lo, 16 token slots
        // four partial gate sums per (token, neuron) of the row-per-lane gate kernel
        S.gpart = (D.layouts & SFFN_LAYOUT_BATCH) ? take((size_t)4 * B * f * 4) : 0;
        S.path = (D.layouts & SFFN_LAYOUT_BATCH) ? take(256) : 0;   // the chosen forward path
    }
    if (D.layouts & SFFN_LAYOUT_PREFILL) {
        // scores and their sorted copy; at least round_up(B, 16) floats, which the
        // exact-mass selection reads 16 at a time
        S.tscore = take(std::max(B * 4 * 2, (B + 15) / 16 * 16 * 4));
        S.tflag = take(B * 4);
        S.pH = take(B * f * 2);       // H (bf16) for up to L gathered rows
        // token sort keys: the sorted chunks of 1024 (the last one padded), then the full order
        S.tkeys = take((B + 1023) / 1024 * 1024 * 8);
        S.tsorted = take(B * 8);
        // the keep list and count of the last selection made with this scratch
        // (sffn_forward in TOKENS mode reads them when it is given no list)
        S.tkeep = take(B * 4);
        S.tkcnt = take(4);
        // the token selection's path and arrival words: [0] 1 when the exact-mass
        // path made the last selection, 2 when the sorted path did
        S.tdone = take(3 * 4);
    }
    S.total = o;
    return S;
}

static bool desc_ok(const sffn_layer_desc *D, sffn_status *why)
{
    *why = SFFN_ERR_INVALID_ARG;
    if (!D) return false;
    if (D->d_model < 256 || D->d_model > 16384 || D->d_model % 256) return false;
    if (D->d_ff < 128 || D->d_ff > 65536 || D->d_ff % 128) return false;
    if (D->wtype < SFFN_W_F32 || D->wtype > SFFN_W_INT4_G128) return false;
    if (D->act != SFFN_ACT_RELU && D->act != SFFN_ACT_SILU) return false;
    if ((D->rmsnorm != 0 && D->rmsnorm != 1) || (D->residual != 0 && D->residual != 1)) return false;
    if (D->layouts <= 0 || (D->layouts & ~(SFFN_LAYOUT_DECODE | SFFN_LAYOUT_PREFILL | SFFN_LAYOUT_BATCH))) return false;
    if (D->layouts == SFFN_LAYOUT_BATCH) return false;
    if ((D->layouts & SFFN_LAYOUT_BATCH) && (!(D->layouts & SFFN_LAYOUT_DECODE) || D->wtype != SFFN_W_BF16)) {
        *why = SFFN_ERR_UNSUPPORTED;
        return false;
    }
    if (D->rmsnorm && !(D->eps >= 0.0f)) return false;
    if (D->max_rows < 1) return false;
    if (D->layouts & SFFN_LAYOUT_DECODE) {
        if (D->max_rows > kMaxDecodeRows) return false;
        if (D->wtype == SFFN_W_INT4_G128 && D->max_rows > kMaxInt4Rows) { *why = SFFN_ERR_UNSUPPORTED; return false; }
    }
    if (D->layouts & SFFN_LAYOUT_PREFILL) {
        if (D->max_rows > kMaxPrefillRows) return false;
        if (D->wtype != SFFN_W_BF16 || D->act != SFFN_ACT_SILU || D->rmsnorm || D->residual) {
            *why = SFFN_ERR_UNSUPPORTED;
            return false;
        }
    }
    return true;
}

// compute units of the current device, cached per device (256 when the query fails)
int compute_units()
{
    static std::atomic<int> cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

hipError_t allow_full_dynamic_lds(const void *kernel, std::once_flag &once, hipError_t &err, int &limit)
{
    std::call_once(once, [&]() {
        int dev = 0, per_block = 0;
        hipFuncAttributes fa{};
        err = hipGetDevice(&dev);
        if (err == hipSuccess) err = hipDeviceGetAttribute(&per_block, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
        if (err == hipSuccess) err = hipFuncGetAttributes(&fa, kernel);
        if (err == hipSuccess) {
            limit = per_block - (int)fa.sharedSizeBytes;
            err = limit > 0 ? hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, limit)
                            : hipErrorInvalidConfiguration;
        }
    });
    return err;
}

// ---------------------------------------------------------------------------
// built-in scratch of sffn_forward_noalloc: one file-scope device array, which
// every GPU the library runs on holds (its own copy) until the process ends.
// In host code the array's name is only a host-side stand-in, never a device
// address: the address is taken once per device with hipGetSymbolAddress and
// only that pointer is passed to kernels.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocScratchBytes = (size_t)80 << 20;   // 80 MiB
constexpr int kNoAllocMaxDevices = 64;
static __device__ __align__(256) uint8_t noalloc_scratch[kNoAllocScratchBytes];

// the calling thread's current device's copy of the array (set up on the first
// call made with that device current)
static hipError_t noalloc_scratch_ptr(void **out)
{
    static std::once_flag once[kNoAllocMaxDevices];
    static hipError_t err[kNoAllocMaxDevices];
    static void *ptr[kNoAllocMaxDevices];
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kNoAllocMaxDevices) return hipErrorInvalidDevice;
    std::call_once(once[dev], [dev]() {
        void *p = nullptr;
        err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch));
        ptr[dev] = err[dev] == hipSuccess ? p : nullptr;
    });
    if (err[dev] != hipSuccess) return err[dev];
    *out = ptr[dev];
    return hipSuccess;
}

// the timer of the entry points that take no handle (sffn_expert_select, the read probe)
KernelTimer &free_timer()
{
    static KernelTimer t;
    return t;
}

}  // namespace sffn

using namespace sffn;

struct sffn_layer {
    Layer L;
    KernelTimer timer;
};

extern "C" {

const char *sffn_status_string(sffn_status s)
{
    switch (s) {
    case SFFN_OK: return "ok";
    case SFFN_ERR_INVALID_ARG: return "invalid argument";
    case SFFN_ERR_UNSUPPORTED: return "unsupported configuration";
    case SFFN_ERR_WORKSPACE: return "workspace too small";
    case SFFN_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

const char *sffn_last_hip_error(void) { return g_hip_err; }

sffn_status sffn_workspace_size(const sffn_layer_desc *desc, size_t *persistent_bytes, size_t *scratch_bytes)
{
    sffn_status why;
    if (!desc_ok(desc, &why)) return why;
    if (!persistent_bytes || !scratch_bytes) return SFFN_ERR_INVALID_ARG;
    *persistent_bytes = persistent_layout(*desc).total;
    *scratch_bytes = scratch_layout(*desc).total;
    return SFFN_OK;
}

static sffn_status create_layer(const sffn_layer_desc *desc, const void *w_gate, const void *w_up,
                               const void *w_down, const void *s_gate, const void *s_up, const void *s_down,
                               const int32_t *perm, void *persistent, size_t persistent_bytes, void *stream,
                               sffn_t *out)
{
    sffn_status why;
    if (!desc_ok(desc, &why)) return why;
    if (!out || !w_gate || !w_up || !w_down || !persistent) return SFFN_ERR_INVALID_ARG;
    const bool i4 = desc->wtype == SFFN_W_INT4_G128;
    if (i4 != (s_gate != nullptr) || i4 != (s_up != nullptr) || i4 != (s_down != nullptr)) return SFFN_ERR_INVALID_ARG;
    if ((uintptr_t)persistent & 255) return SFFN_ERR_INVALID_ARG;
    if (((uintptr_t)w_gate | (uintptr_t)w_up | (uintptr_t)w_down) & 15) return SFFN_ERR_INVALID_ARG;
    const PersistentLayout P = persistent_layout(*desc);
    if (persistent_bytes < P.total) return SFFN_ERR_WORKSPACE;

    sffn_layer *h = new (std::nothrow) sffn_layer;
    if (!h) return SFFN_ERR_INVALID_ARG;
    Layer &L = h->L;
    L.desc = *desc;
    L.timer = &h->timer;
    uint8_t *base = (uint8_t *)persistent;
    const bool dec = desc->layouts & SFFN_LAYOUT_DECODE;
    if (dec) {
        L.wg = base + P.wg;
        L.wu = base + P.wu;
        L.wdt = base + P.wdt;
        L.wdn = (const double *)(base + P.wdn);
        if (i4) {
            L.sg = (const uint16_t *)(base + P.sg);
            L.su = (const uint16_t *)(base + P.su);
            L.sdt = (const uint16_t *)(base + P.sdt);
        }
    }
    L.wd = base + P.wd;
    if (i4) L.sd = (const uint16_t *)(base + P.sd);
    if (desc->layouts & SFFN_LAYOUT_PREFILL) {
        L.wgu = (const uint16_t *)(base + P.wgu);
        L.wdp = (const uint16_t *)(base + P.wdp);
    }
    if (dec && (desc->layouts & SFFN_LAYOUT_BATCH)) {
        L.wut = (const uint16_t *)(base + P.wut);
        L.wdtl = (const uint16_t *)(base + P.wdtl);
        L.wgt = (const uint16_t *)(base + P.wgt);
    }
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    const int32_t *ilv_perm = nullptr;
    if (perm) {
        // the permuted natural copies first; every other layout is built from them
        e = launch_permute_weights(*desc, w_gate, w_up, w_down, perm, base, st);
        if (dec) {
            w_gate = base + P.wg;
            w_up = base + P.wu;
        } else {
            ilv_perm = perm;
        }
        w_down = base + P.wd;
    }
    if (e == hipSuccess) e = launch_relayout(L, w_gate, w_up, w_down, s_gate, s_up, s_down, base, st, ilv_perm);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) {
        delete h;
        return hip_status(e);
    }
    *out = h;
    return SFFN_OK;
}

sffn_status sffn_create(const sffn_layer_desc *desc, const void *w_gate, const void *w_up, const void *w_down,
                        const void *s_gate, const void *s_up, const void *s_down, void *persistent,
                        size_t persistent_bytes, void *stream, sffn_t *out)
{
    return create_layer(desc, w_gate, w_up, w_down, s_gate, s_up, s_down, nullptr, persistent, persistent_bytes,
                        stream, out);
}

sffn_status sffn_create_permuted(const sffn_layer_desc *desc, const void *w_gate, const void *w_up,
                                 const void *w_down, const int32_t *perm, void *persistent, size_t persistent_bytes,
                                 void *stream, sffn_t *out)
{
    sffn_status why;
    if (!desc_ok(desc, &why)) return why;
    if (desc->wtype == SFFN_W_INT4_G128) return SFFN_ERR_UNSUPPORTED;
    if (!perm) return SFFN_ERR_INVALID_ARG;
    // the permutation is checked on the host before any kernel indexes with it
    const int f = desc->d_ff;
    std::vector<int32_t> hp(f);
    std::vector<char> seen(f, 0);
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(hp.data(), perm, (size_t)f * 4, hipMemcpyDeviceToHost, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);
    if (e != hipSuccess) return hip_status(e);
    for (int j = 0; j < f; ++j) {
        if (hp[j] < 0 || hp[j] >= f || seen[hp[j]]) return SFFN_ERR_INVALID_ARG;
        seen[hp[j]] = 1;
    }
    return create_layer(desc, w_gate, w_up, w_down, nullptr, nullptr, nullptr, perm, persistent, persistent_bytes,
                        stream, out);
}

void sffn_destroy(sffn_t layer) { delete layer; }


sffn_status sffn_expert_select(const float *probs, int32_t tokens, int32_t experts, const sffn_expert_policy *policy,
                               int32_t *k_out, int32_t *idx_out, float *w_out, void *stream)
{
    if (!policy || tokens < 0 || experts < 1 || experts > kMaxExpertsAbi) return SFFN_ERR_INVALID_ARG;
    if (tokens > 0 && (!probs || !k_out || !idx_out || !w_out)) return SFFN_ERR_INVALID_ARG;
    const int kmin = policy->kmin, kmax = policy->kmax;
    if (kmin < 1 || kmax < kmin || kmax > experts || kmax > kMaxExpertKAbi) return SFFN_ERR_INVALID_ARG;
    if (!(policy->tau == policy->tau)) return SFFN_ERR_INVALID_ARG;   // NaN
    return hip_status(launch_expert_select(probs, tokens, experts, policy->tau, kmin, kmax, k_out, idx_out, w_out,
                                           (hipStream_t)stream, &sffn::free_timer()));
}

sffn_status sffn_set_kernel_timer(sffn_t layer, void *const *begin_events, void *const *end_events, int32_t n)
{
    if (n < 0 || (n > 0 && (!begin_events || !end_events))) return SFFN_ERR_INVALID_ARG;
    KernelTimer &t = layer ? layer->timer : sffn::free_timer();
    t.begin = begin_events;
    t.end = end_events;
    t.n = n;
    t.next = 0;
    return SFFN_OK;
}

sffn_status sffn_token_select_path(sffn_t layer, const void *scratch, size_t scratch_bytes, int32_t *path,
                                   void *stream)
{
    if (!layer || !scratch || !path) return SFFN_ERR_INVALID_ARG;
    const sffn_layer_desc &D = layer->L.desc;
    if (!(D.layouts & SFFN_LAYOUT_PREFILL)) return SFFN_ERR_INVALID_ARG;
    const ScratchLayout S = scratch_layout(D);
    if (scratch_bytes < S.total) return SFFN_ERR_WORKSPACE;
    return hip_status(hipMemcpyAsync(path, (const uint8_t *)scratch + S.tdone, 4, hipMemcpyDeviceToDevice,
                                     (hipStream_t)stream));
}

static bool decode_mode(int m)
{
    return m == SFFN_MODE_ALL || m == SFFN_MODE_EXACT || m == SFFN_MODE_THRESH || m == SFFN_MODE_TOPK;
}

static sffn_status policy_ok(const sffn_layer *h, const sffn_policy *p)
{
    if (!h || !p) return SFFN_ERR_INVALID_ARG;
    const sffn_layer_desc &D = h->L.desc;
    if (p->mode == SFFN_MODE_TOKENS) {
        if (!(D.layouts & SFFN_LAYOUT_PREFILL)) return SFFN_ERR_INVALID_ARG;
        if (!(p->mass_thresh >= 0.0) || p->recent_n < 0 || p->min_keep < 0) return SFFN_ERR_INVALID_ARG;
        return SFFN_OK;
    }
    if (!decode_mode(p->mode) && p->mode != SFFN_MODE_DENSE) return SFFN_ERR_INVALID_ARG;
    if (!(D.layouts & SFFN_LAYOUT_DECODE)) return SFFN_ERR_INVALID_ARG;
    if (p->mode == SFFN_MODE_TOPK && (p->topk_k < 1 || p->topk_k > D.d_ff)) return SFFN_ERR_INVALID_ARG;
    if (p->use_union != 0 && p->use_union != 1) return SFFN_ERR_INVALID_ARG;
    if (p->batch_path < 0 || p->batch_path > 2) return SFFN_ERR_INVALID_ARG;
    if (p->merge_gap < 0 || p->merge_gap > 64) return SFFN_ERR_INVALID_ARG;
    if (p->mode == SFFN_MODE_TOPK && D.act != SFFN_ACT_SILU) return SFFN_ERR_UNSUPPORTED;
    if (p->mode == SFFN_MODE_THRESH) {
        // THRESH stands for |act(g')| > tau, taken in the gate domain as g' > theta.
        // For SiLU the two agree only when tau exceeds SiLU's minimum depth
        // (0.27846...), i.e. theta > 0.45511541... on the positive branch:
        // 0.4551154f is the largest float below that bound.  For ReLU, theta >= 0.
        if (!(p->theta == p->theta)) return SFFN_ERR_INVALID_ARG;   // NaN
        if (D.act == SFFN_ACT_SILU ? !(p->theta > 0.4551154f) : !(p->theta >= 0.0f)) return SFFN_ERR_UNSUPPORTED;
    }
    if (p->mode == SFFN_MODE_TOPK && D.d_ff > kMaxTopkNeurons) return SFFN_ERR_UNSUPPORTED;
    return SFFN_OK;
}

sffn_status sffn_select(sffn_t layer, const sffn_policy *policy, const void *in, int32_t rows, int32_t *idx_out,
                        int32_t *count_out, void *scratch, size_t scratch_bytes, void *stream)
{
    sffn_status s = policy_ok(layer, policy);
    if (s != SFFN_OK) return s;
    if (policy->mode == SFFN_MODE_DENSE) return SFFN_ERR_INVALID_ARG;
    const sffn_layer_desc &D = layer->L.desc;
    if (!in || !idx_out || !count_out || !scratch) return SFFN_ERR_INVALID_ARG;
    if (rows < 1 || rows > D.max_rows) return SFFN_ERR_INVALID_ARG;
    if ((uintptr_t)scratch & 255) return SFFN_ERR_INVALID_ARG;
    if (scratch_bytes < scratch_layout(D).total) return SFFN_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    if (policy->mode == SFFN_MODE_TOKENS) {
        if ((uintptr_t)in & 15) return SFFN_ERR_INVALID_ARG;
        PrefillSelectCall c{&layer->L, (const uint16_t *)in, rows, policy->mass_thresh, policy->recent_n,
                            policy->min_keep, idx_out, count_out, (uint8_t *)scratch, st};
        return hip_status(launch_prefill_select(c));
    }
    if ((uintptr_t)in & 15) return SFFN_ERR_INVALID_ARG;
    DecodeCall c{&layer->L, policy->mode, policy->use_union, policy->topk_k, policy->batch_path, policy->merge_gap, policy->gate_bias, policy->theta,
                 rows, (const float *)in, nullptr, idx_out, count_out, (uint8_t *)scratch, st};
    return hip_status(launch_decode(c, false));
}

sffn_status sffn_select_blocks(sffn_t layer, const sffn_block_policy *policy, const void *A, int32_t rows,
                               const int32_t *cu_seqlens, int32_t nseq, int32_t *idx_out, int32_t *count_out,
                               void *scratch, size_t scratch_bytes, void *stream)
{
    if (!layer || !policy || !A || !cu_seqlens || !idx_out || !count_out || !scratch) return SFFN_ERR_INVALID_ARG;
    const sffn_layer_desc &D = layer->L.desc;
    if (!(D.layouts & SFFN_LAYOUT_PREFILL)) return SFFN_ERR_INVALID_ARG;
    if (rows < 1 || rows > D.max_rows || nseq < 1 || nseq > rows) return SFFN_ERR_INVALID_ARG;
    const sffn_block_policy &p = *policy;
    if (p.block < kMinTokenBlock || p.block > kMaxPrefillRows) return SFFN_ERR_INVALID_ARG;
    if (!(p.mass_thresh == p.mass_thresh)) return SFFN_ERR_INVALID_ARG;   // NaN
    if (!(p.min_full_ratio >= 0.0f && p.max_full_ratio <= 1.0f && p.min_full_ratio <= p.max_full_ratio))
        return SFFN_ERR_INVALID_ARG;
    if (p.recent_n < 0 || p.min_keep < 0) return SFFN_ERR_INVALID_ARG;
    if (((uintptr_t)scratch & 255) || ((uintptr_t)A & 15)) return SFFN_ERR_INVALID_ARG;
    if (scratch_bytes < scratch_layout(D).total) return SFFN_ERR_WORKSPACE;
    BlockSelectCall c{&layer->L, (const uint16_t *)A, rows, cu_seqlens, nseq, p.block, p.mass_thresh,
                      p.min_full_ratio, p.max_full_ratio, p.recent_n, p.min_keep, idx_out, count_out,
                      (uint8_t *)scratch, (hipStream_t)stream};
    return hip_status(launch_block_select(c));
}

double sffn_schedule_mass(int32_t layer, int32_t dense_until, int32_t deep_layer_start, double mass_thresh,
                          double mass_thresh_deep)
{
    if (layer < dense_until) return 1.0;
    if (layer < deep_layer_start) return mass_thresh;
    return mass_thresh_deep;
}

sffn_status sffn_forward(sffn_t layer, const sffn_policy *policy, const void *in, int32_t rows, void *out,
                         const int32_t *idx_in, const int32_t *count_in, int32_t *idx_out, int32_t *count_out,
                         void *scratch, size_t scratch_bytes, void *stream)
{
    sffn_status s = policy_ok(layer, policy);
    if (s != SFFN_OK) return s;
    const sffn_layer_desc &D = layer->L.desc;
    if (!in || !out || !scratch) return SFFN_ERR_INVALID_ARG;
    if (rows < 1 || rows > D.max_rows) return SFFN_ERR_INVALID_ARG;
    if ((uintptr_t)scratch & 255) return SFFN_ERR_INVALID_ARG;
    if (((uintptr_t)in | (uintptr_t)out) & 15) return SFFN_ERR_INVALID_ARG;
    if (scratch_bytes < scratch_layout(D).total) return SFFN_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    if (policy->mode == SFFN_MODE_TOKENS) {
        if ((idx_in == nullptr) != (count_in == nullptr) || idx_out || count_out) return SFFN_ERR_INVALID_ARG;
        if (!idx_in) {
            // no list given: the keep list the last selection on this scratch left there
            const ScratchLayout S = scratch_layout(D);
            idx_in = (const int32_t *)((const uint8_t *)scratch + S.tkeep);
            count_in = (const int32_t *)((const uint8_t *)scratch + S.tkcnt);
        }
        PrefillForwardCall c{&layer->L, (const uint16_t *)in, (uint16_t *)out, rows, idx_in, count_in,
                             (uint8_t *)scratch, st};
        return hip_status(launch_prefill_forward(c));
    }
    if (idx_in || count_in) return SFFN_ERR_INVALID_ARG;
    if (in == out) return SFFN_ERR_INVALID_ARG;
    if (policy->mode == SFFN_MODE_DENSE && (idx_out || count_out)) return SFFN_ERR_INVALID_ARG;
    DecodeCall c{&layer->L, policy->mode, policy->use_union, policy->topk_k, policy->batch_path, policy->merge_gap, policy->gate_bias, policy->theta,
                 rows, (const float *)in, (float *)out, idx_out, count_out, (uint8_t *)scratch, st};
    return hip_status(launch_decode(c, true));
}

sffn_status sffn_forward_noalloc(sffn_t layer, const sffn_policy *policy, const void *in, int32_t rows, void *out,
                                 const int32_t *idx_in, const int32_t *count_in, int32_t *idx_out, int32_t *count_out,
                                 void *stream)
{
    sffn_status s = policy_ok(layer, policy);
    if (s != SFFN_OK) return s;
    const size_t need = scratch_layout(layer->L.desc).total;
    if (need > kNoAllocScratchBytes) return SFFN_ERR_WORKSPACE;
    void *p = nullptr;
    hipError_t e = noalloc_scratch_ptr(&p);
    if (e != hipSuccess) return hip_status(e);
    // the same validation and kernels as sffn_forward, on the built-in array
    return sffn_forward(layer, policy, in, rows, out, idx_in, count_in, idx_out, count_out, p, need, stream);
}

size_t sffn_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

}  // extern "C"
