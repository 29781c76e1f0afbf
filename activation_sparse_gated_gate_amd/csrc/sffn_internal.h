// sffn_internal.h -- shared definitions of the gfx950 library (not part of the ABI).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "../../include/sffn.h"

namespace sffn {

// ---------------------------------------------------------------------------
// limits and launch constants
// ---------------------------------------------------------------------------
constexpr int kMaxDecodeRows = 16;
constexpr int kMaxInt4Rows = 8;
constexpr int kMaxPrefillRows = 16384;
constexpr int kMaxTopkNeurons = 16384;  // d_ff limit of the top-k mode (sort in LDS)
constexpr int kGatherWGs = 256;      // partitions of the active list (partial sums)
constexpr int kMassBlock = 256;      // sorted scores per block of the fp64 mass prefix
constexpr int kMaxDownSplits = 64;     // d_ff splits of the batched MFMA down projection
constexpr int kIlvRows = 32;         // prefill: W_gate / W_up interleave granularity

// weight bytes per row of `cols` elements
inline size_t row_bytes(int wtype, int cols)
{
    return wtype == SFFN_W_F32 ? (size_t)cols * 4 : wtype == SFFN_W_BF16 ? (size_t)cols * 2 : (size_t)cols / 2;
}

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// compute units of the current device (cached per device)
int compute_units();

// Raises a kernel's dynamic-LDS limit, once per process (thread-safe), to all
// the LDS a workgroup may hold on the current device minus the kernel's static
// LDS.  *limit receives that number of bytes; a launch asking for more must be
// refused by the caller.
hipError_t allow_full_dynamic_lds(const void *kernel, std::once_flag &once, hipError_t &err, int &limit);

// ---------------------------------------------------------------------------
// the handle
// ---------------------------------------------------------------------------
// optional per-launch timing of the main kernel (diagnostics): the next n
// launches of the path's main kernel take their start / stop events from this
// list; the events are recorded by the kernel dispatch itself
// (hipExtLaunchKernel), so they bracket the kernel and nothing else.
struct KernelTimer {
    void *const *begin = nullptr;
    void *const *end = nullptr;
    int n = 0, next = 0;
    void take(hipEvent_t *b, hipEvent_t *e)
    {
        if (next < n) {
            *b = (hipEvent_t)begin[next];
            *e = (hipEvent_t)end[next];
            ++next;
        } else {
            *b = nullptr;
            *e = nullptr;
        }
    }
};

// launch with dispatch-recorded events when given, a plain launch otherwise
#define SFFN_LAUNCH(kernel, grid, block, shmem, stream, evb, eve, ...)                                   \
    do {                                                                                                \
        if (evb)                                                                                        \
            hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, evb, eve, 0, __VA_ARGS__);         \
        else                                                                                            \
            hipLaunchKernelGGL(kernel, grid, block, shmem, stream, __VA_ARGS__);                        \
    } while (0)

// the timer of the entry points that take no handle (sffn_set_kernel_timer(NULL, ...))
KernelTimer &free_timer();

struct Layer {
    sffn_layer_desc desc;
    // decode layouts
    const uint8_t *wg = nullptr, *wu = nullptr;   // [f][d]
    const uint16_t *sg = nullptr, *su = nullptr;  // int4 scales [f][d/128]
    const uint8_t *wdt = nullptr;                 // W_down^T [f][d]
    const uint16_t *sdt = nullptr;                // int4 scales [f/128][d]
    const uint8_t *wd = nullptr;                  // W_down natural [d][f] (dense baseline)
    const uint16_t *sd = nullptr;                 // int4 scales [d][f/128]
    const double *wdn = nullptr;                  // ||W_down[:, j]||_2, [f]
    // prefill layouts (bf16)
    const uint16_t *wgu = nullptr;                // [f/32][2][32][d]: gate rows then up rows
    const uint16_t *wdp = nullptr;                // W_down natural [d][f]
    // batched-decode MFMA tiles (bf16): [rows/16][cols/32][64 lanes][8], lane = (k-group << 4) | row
    const uint16_t *wut = nullptr;                // W_up   [f][d] as tiles
    const uint16_t *wdtl = nullptr;               // W_down [d][f] as tiles
    const uint16_t *wgt = nullptr;                // W_gate [f][d] as [4][ceil(d/512)][f][16][8] (class-tiled)
    KernelTimer *timer = nullptr;                 // owned by the handle
};

// persistent-buffer layout, in creation order
struct PersistentLayout {
    size_t wg, sg, wu, su, wdt, sdt, wd, sd, wdn, wgu, wdp, wut, wdtl, wgt, total;
};
PersistentLayout persistent_layout(const sffn_layer_desc &d);

// scratch layout for one call
struct ScratchLayout {
    size_t xhat, G, U, keys, bits, list_cnt, list_idx, partial, H;       // decode
    size_t xsplit, hsplit, gpart, path;                                  // decode, batches (BATCH layout)
    size_t tscore, tflag, pH, tkeys, tsorted, tkeep, tkcnt, tdone;       // prefill
    size_t total;
    int n_lists_gate, rows_per_list_gate;
};
ScratchLayout scratch_layout(const sffn_layer_desc &d);

// ---------------------------------------------------------------------------
// kernel launchers (return hipError_t of the launch)
// ---------------------------------------------------------------------------
// batched decode with the BATCH layout: which forward path the device-side
// union size picked (or the caller forced)
enum { kPathTiled = 1, kPathGather = 2 };

struct DecodeCall {
    const Layer *L;
    int mode, use_union, topk_k;
    int batch_path;     // 0 auto, kPathTiled, kPathGather
    int merge_gap;      // top-k gather: unselected neurons read between selected ones (0 = off)
    float bias, theta;
    int B;
    const float *x;     // [B][d] caller input
    float *out;         // [B][d] caller output (forward) or nullptr (select)
    int32_t *idx_out, *count_out;
    uint8_t *scratch;
    hipStream_t stream;
};
hipError_t launch_decode(const DecodeCall &c, bool forward);

struct PrefillSelectCall {
    const Layer *L;
    const uint16_t *A;
    int rows;
    double mass;
    int recent_n, min_keep;
    int32_t *idx_out, *count_out;
    uint8_t *scratch;
    hipStream_t stream;
};
hipError_t launch_prefill_select(const PrefillSelectCall &c);
// t1 alone: s_i = ||A_i||_2 for rows bf16 rows of d_model d
hipError_t launch_token_norms(const uint16_t *A, int rows, int d, float *s, hipStream_t st);

// block-granular token selection over a batch of sequences (blocks.hip)
constexpr int kMinTokenBlock = 16;
constexpr int kMaxBlocksPerSeq = (kMaxPrefillRows + kMinTokenBlock - 1) / kMinTokenBlock;   // 1024
struct BlockSelectCall {
    const Layer *L;
    const uint16_t *A;
    int rows;
    const int32_t *cu;   // device [nseq + 1]
    int nseq;
    int block;
    double mass;
    float min_full, max_full;
    int recent_n, min_keep;
    int32_t *idx_out, *count_out;
    uint8_t *scratch;
    hipStream_t stream;
};
hipError_t launch_block_select(const BlockSelectCall &c);
// adaptive expert top-K (experts.hip)
constexpr int kMaxExpertsAbi = 1024;
constexpr int kMaxExpertKAbi = 16;
hipError_t launch_expert_select(const float *probs, int T, int E, float tau, int kmin, int kmax, int32_t *k_out,
                                int32_t *idx_out, float *w_out, hipStream_t st, KernelTimer *timer);

struct PrefillForwardCall {
    const Layer *L;
    const uint16_t *Y;
    uint16_t *X;
    int rows;
    const int32_t *keep, *count;
    uint8_t *scratch;
    hipStream_t stream;
};
hipError_t launch_prefill_forward(const PrefillForwardCall &c);

// ilv_perm (device, or null): the prefill interleave reads neuron n from row
// ilv_perm[n] of w_gate / w_up
hipError_t launch_relayout(const Layer &L, const void *w_gate, const void *w_up, const void *w_down,
                           const void *s_gate, const void *s_up, const void *s_down,
                           uint8_t *persistent, hipStream_t stream, const int32_t *ilv_perm);

// gathers the neurons in the order perm (fp32 / bf16) into the persistent
// natural-layout copies: W_down's columns always, W_gate's and W_up's rows
// when the DECODE layout holds copies of them
hipError_t launch_permute_weights(const sffn_layer_desc &D, const void *w_gate, const void *w_up,
                                  const void *w_down, const int32_t *perm, uint8_t *persistent,
                                  hipStream_t stream);

// consecutive neurons per workgroup of the batch-1 fused decode kernel
int fused_rows_per_wg(int f);

}  // namespace sffn
