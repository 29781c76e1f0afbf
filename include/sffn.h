/*
 * sffn.h -- C ABI of the activation-sparse gated FFN library (libsffn.so, gfx950).
 *
 * The library evaluates one gated FFN layer
 *
 *     y = W_down . ( m (.) act(W_gate x + b) (.) (W_up x) )
 *
 * where neuron j owns row j of W_gate, row j of W_up and column j of W_down
 * (denseflux: skipping most of a dense FFN, section 1 "why the FFN"), and the
 * mask m keeps only the neurons that matter for each token:
 *
 *   SFFN_MODE_ALL     every neuron, through the sparse kernels (100% active);
 *   SFFN_MODE_EXACT   ReLU exact gating: neurons with fl32(g + b) > 0; the skipped
 *                     neurons have an exactly zero activation, so the result
 *                     equals the dense FFN (denseflux, sections 3 and 5.1-5.3);
 *   SFFN_MODE_THRESH  a threshold on |SiLU(W_gate x)| (denseflux, section 4.1),
 *                     given in the gate domain: neurons with fl32(g + b) > theta.
 *                     This equals |SiLU(g + b)| > SiLU(theta) exactly when
 *                     SiLU(theta) exceeds SiLU's minimum depth 0.27846..., i.e.
 *                     theta > 0.45511541...: for SiLU layers a theta at or below
 *                     that bound (theta <= 0.4551154f, the largest float below
 *                     it) is SFFN_ERR_UNSUPPORTED; for ReLU layers theta must be
 *                     >= 0 (|ReLU(g)| > theta), else SFFN_ERR_UNSUPPORTED; a
 *                     NaN theta is SFFN_ERR_INVALID_ARG;
 *   SFFN_MODE_TOPK    weight-aware top-k: the topk_k neurons with the largest
 *                     score |SiLU(g + b) * u| * ||W_down[:, j]||_2, ties to the
 *                     lower index (WiSparse reproduction notes, sections 2.3 and
 *                     3.2); with use_union a batch runs over the union of its
 *                     tokens' sets (same notes, section 5, batch > 1);
 *   SFFN_MODE_DENSE   the dense FFN with no selection (the baseline): at batch 1
 *                     (fp32 / bf16) the streaming kernel of the sparse path over
 *                     every neuron, otherwise plain fixed-order GEMV kernels;
 *   SFFN_MODE_TOKENS  token-selective prefill (RedKnot article, Algorithm 1 and
 *                     the section on the token-selective sparse FFN): token
 *                     importance = L2 norm of the attention output row; keep the
 *                     shortest prefix of the tokens in descending importance whose
 *                     mass reaches mass_thresh of the total, plus the last
 *                     recent_n tokens, plus top-ranked tokens up to min_keep;
 *                     mass_thresh >= 1 or an all-zero score row keeps every
 *                     token (so does a NaN or infinite score, which makes the
 *                     total mass non-finite); X_next = Y + FFN(Y) on kept
 *                     rows, Y elsewhere.
 *
 * Conventions for every entry point:
 *  - Every pointer named *device* is HIP device memory; descriptors and
 *    policies are host memory read during the call only.
 *  - The caller owns every buffer (weights, inputs, outputs, index lists,
 *    workspaces).  The library allocates no device memory.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream); no call synchronises the host, except sffn_create, which waits
 *    for its relayout kernels before returning.  Device-side counts stay on
 *    the device; synchronise the stream before reading results.
 *  - Argument validation happens before any launch and returns a status;
 *    no exception or abort crosses the ABI.  After SFFN_ERR_HIP the outputs
 *    are undefined and the handle stays valid.
 *  - Non-finite inputs give undefined values (not detected), except that a
 *    non-finite token score keeps every token (see SFFN_MODE_TOKENS); no
 *    input makes a kernel access memory outside the buffers it was given.
 *  - Diagnostics used by benchmarks (a read-bandwidth probe, per-launch kernel
 *    timing) are declared in sffn_diag.h.
 *  - Calls on one handle from different streams need distinct scratch buffers.
 */
#ifndef SFFN_H
#define SFFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sffn_status {
    SFFN_OK = 0,
    SFFN_ERR_INVALID_ARG = 1,  /* NULL pointer, size out of range, bad enum */
    SFFN_ERR_UNSUPPORTED = 2,  /* valid request this build does not implement */
    SFFN_ERR_WORKSPACE = 3,    /* workspace smaller than sffn_workspace_size says */
    SFFN_ERR_HIP = 4           /* a HIP launch or runtime call failed */
} sffn_status;

/* weight storage formats */
enum {
    SFFN_W_F32 = 0,        /* fp32 */
    SFFN_W_BF16 = 1,       /* bf16 bit patterns (uint16) */
    SFFN_W_INT4_G128 = 2   /* int4, groups of 128 along the input dimension, fp16 scales */
};

enum { SFFN_ACT_RELU = 0, SFFN_ACT_SILU = 1 };

enum {
    SFFN_MODE_ALL = 0,
    SFFN_MODE_EXACT = 1,
    SFFN_MODE_THRESH = 2,
    SFFN_MODE_TOPK = 3,
    SFFN_MODE_TOKENS = 4,
    SFFN_MODE_DENSE = 5
};

/*
 * Which internal layouts sffn_create builds.
 *  DECODE   row-major W_gate, W_up, W_down^T and the W_down column norms (decode at every batch size)
 *  PREFILL  interleaved W_gate / W_up rows for the token-selective prefill GEMMs
 *  BATCH    with DECODE and bf16 weights only: W_gate copied once more with the rows of each block
 *           of 64 interleaved per 8-column chunk, W_up and W_down as 16 x 32 MFMA operand tiles
 *           (3 * d_model * d_ff * 2 bytes more); used by decode calls of 5..16 tokens in the
 *           ALL / EXACT / THRESH modes; without it those calls run the VALU gather path
 */
enum { SFFN_LAYOUT_DECODE = 1, SFFN_LAYOUT_PREFILL = 2, SFFN_LAYOUT_BATCH = 4 };

/*
 * Layer descriptor.
 *  d_model   multiple of 256, 256..16384
 *  d_ff      multiple of 128, 128..65536
 *  max_rows  decode: tokens per call, 1..16; prefill: sequence length, 1..16384
 *  wtype     SFFN_W_*; prefill requires SFFN_W_BF16
 *  act       SFFN_ACT_RELU (ReGLU) or SFFN_ACT_SILU (SwiGLU); prefill requires SILU
 *  rmsnorm   1: the FFN input is x * 1/sqrt(mean(x^2) + eps) (unit weight), decode only
 *  residual  1: decode output is x + y instead of y
 *  eps       RMSNorm epsilon
 *  layouts   SFFN_LAYOUT_* bit set
 */
typedef struct sffn_layer_desc {
    int32_t d_model;
    int32_t d_ff;
    int32_t max_rows;
    int32_t wtype;
    int32_t act;
    int32_t rmsnorm;
    int32_t residual;
    float eps;
    int32_t layouts;
} sffn_layer_desc;

/*
 * Per-call policy.
 *  mode         SFFN_MODE_*
 *  gate_bias    b added to the gate pre-activation (fp32 add) before the
 *               activation and every predicate
 *  theta        THRESH: gate-domain threshold
 *  topk_k       TOPK: neurons kept per token, 1..d_ff (TOPK needs d_ff <= 16384
 *               and act = SFFN_ACT_SILU, else SFFN_ERR_UNSUPPORTED)
 *  use_union    decode batches: 1 = every token of the call is computed over
 *               the union of the tokens' selected sets; 0 = each token over
 *               its own set (the gathered rows are still the union)
 *  mass_thresh  TOKENS: fraction of the total importance mass (fp64)
 *  recent_n     TOKENS: trailing tokens always kept (>= 0)
 *  min_keep     TOKENS: minimum kept tokens (>= 0)
 *  batch_path   decode calls that use the BATCH layout (5..16 tokens): 0 = the
 *               device picks, from the size of the selected union, between
 *               the MFMA tile path (every W_up block with a selected neuron
 *               and all of W_down) and the row gather (only the union's
 *               W_up and W_down^T rows) at the measured breakeven; 1 forces
 *               the tiles, 2 the gather (both give the same results within
 *               the bf16 / fp32 tolerance).  Other calls ignore it.
 *  merge_gap    TOPK forward: run merging of the W_down^T row gather (denseflux,
 *               section 5.5: adjacent reads are merged when reading the gap costs
 *               less than a new request, gap < L * B bytes).  A neuron lying
 *               between two selected neurons of a gather share, with at most
 *               merge_gap unselected neurons between them, is read as well
 *               (with h = 0, so the result is unchanged); 0 = off (the default,
 *               the measured best on MI355X), 0..64.
 */
typedef struct sffn_policy {
    int32_t mode;
    float gate_bias;
    float theta;
    int32_t topk_k;
    int32_t use_union;
    int32_t recent_n;
    int32_t min_keep;
    int32_t batch_path;
    int32_t merge_gap;
    int32_t reserved;
    double mass_thresh;
} sffn_policy;

typedef struct sffn_layer *sffn_t;

/*
 * Bytes the caller must provide: `persistent` for sffn_create (relayouted
 * weights, kept for the life of the handle) and `scratch` for every
 * sffn_select / sffn_forward call (reused between calls, contents not
 * preserved).  Both are device buffers aligned to 256 bytes.
 */
sffn_status sffn_workspace_size(const sffn_layer_desc *desc, size_t *persistent_bytes,
                                size_t *scratch_bytes);

/*
 * Builds a layer handle.  Weights are device buffers in natural layout:
 *   W_gate, W_up: [d_ff][d_model] row-major; W_down: [d_model][d_ff] row-major.
 *   int4: packed bytes [rows][cols/2] (even column in the low nibble, two's
 *   complement) with fp16 scales [rows][cols/128] in s_gate / s_up / s_down;
 *   other formats pass NULL scales.
 * The library copies what it needs into `persistent` (row-major W_gate and
 * W_up, the transposed W_down^T [d_ff][d_model] for decode with its scales
 * regrouped as [d_ff/128][d_model], the fp64 column norms ||W_down[:, j]||_2,
 * and for prefill W_gate / W_up interleaved in blocks of 32 rows plus a copy of
 * W_down), waits for the copies to finish and keeps no weight pointer.
 * On success *out receives the handle (free with sffn_destroy).
 */
sffn_status sffn_create(const sffn_layer_desc *desc, const void *w_gate, const void *w_up,
                        const void *w_down, const void *s_gate, const void *s_up,
                        const void *s_down, void *persistent, size_t persistent_bytes,
                        void *stream, sffn_t *out);

/*
 * Selection only.
 *  decode modes (ALL, EXACT, THRESH, TOPK): `in` = x, fp32 [rows][d_model];
 *    idx_out (device, capacity d_ff) receives the ascending union of the
 *    selected neuron indices and count_out (device, one int32) its length.
 *  TOKENS: `in` = A, the attention output, bf16 [rows][d_model] (rows = L);
 *    idx_out (device, capacity rows) receives the kept token indices in
 *    ascending order and count_out their number.
 */
sffn_status sffn_select(sffn_t layer, const sffn_policy *policy, const void *in, int32_t rows,
                        int32_t *idx_out, int32_t *count_out, void *scratch,
                        size_t scratch_bytes, void *stream);

/*
 * Forward.
 *  decode modes and DENSE: `in` = x fp32 [rows][d_model] (device); `out` =
 *    fp32 [rows][d_model] (device), y, or x + y with residual; out must not
 *    alias in.  idx_in / count_in must be NULL.  idx_out / count_out
 *    (optional, device) receive the ascending union list as in sffn_select.
 *  TOKENS: `in` = Y bf16 [rows][d_model]; `out` = X_next bf16 [rows][d_model];
 *    idx_in / count_in (device) = the keep list from sffn_select or
 *    sffn_select_blocks.  Both NULL: the forward runs on the selection that
 *    the last sffn_select (TOKENS) or sffn_select_blocks call made with this
 *    same scratch buffer left in it (stream-ordered; the attention output A is
 *    only ever passed to the selection call); the result is undefined if no
 *    such call preceded it on this scratch (the kernels clamp the count and
 *    the indices to [0, rows), so no access leaves the buffers).  One NULL and
 *    the other not is SFFN_ERR_INVALID_ARG.  X_next may alias Y: then only
 *    kept rows are written.  Otherwise un-kept rows are copied bit for bit.
 *    idx_out / count_out must be NULL.
 */
sffn_status sffn_forward(sffn_t layer, const sffn_policy *policy, const void *in, int32_t rows,
                         void *out, const int32_t *idx_in, const int32_t *count_in,
                         int32_t *idx_out, int32_t *count_out, void *scratch,
                         size_t scratch_bytes, void *stream);

/*
 * sffn_forward without a scratch argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).  It runs exactly sffn_forward (same arguments,
 * validation, kernels and results, bit for bit) on a scratch array built into
 * the library: sffn_noalloc_scratch_bytes() = 80 MiB, which every GPU the
 * library runs on holds until the process ends.  The call itself allocates
 * nothing.  A layer whose scratch (sffn_workspace_size) exceeds the array is
 * refused with SFFN_ERR_WORKSPACE before any launch (every decode workload
 * here fits: the largest, d_model 3584 x d_ff 18944 at 16 tokens with the
 * BATCH layout, needs 67 MB; long prefill layers do not).
 * The layer's device must be current.  All calls on one GPU share that GPU's
 * array, which keeps the last call's contents (a TOKENS forward without a keep
 * list reads the selection left there): calls that overlap on one GPU
 * (different streams or threads) race and must be serialised by the caller.
 * No kernel needs the array cleared: every call writes what it reads.
 */
sffn_status sffn_forward_noalloc(sffn_t layer, const sffn_policy *policy, const void *in, int32_t rows,
                                 void *out, const int32_t *idx_in, const int32_t *count_in,
                                 int32_t *idx_out, int32_t *count_out, void *stream);
size_t sffn_noalloc_scratch_bytes(void);

/*
 * Block-granular token selection over a batch of sequences (RedKnot article:
 * at least min_keep tokens per sequence, section on the token-selective sparse
 * FFN; bounds min_full_ratio 0.10 / max_full_ratio 0.50 on the kept fraction
 * and a fixed-budget top-K over blocks of 128 tokens so that the kept rows
 * form a few contiguous runs, computed on the GPU without host
 * synchronisation, last paragraph of the section on adaptive expert top-K).
 *  mass_thresh     fraction of each sequence's block mass (fp64); >= 1 keeps all
 *  min_full_ratio  lower bound, as a fraction of the sequence's blocks, 0..1
 *  max_full_ratio  upper bound, min_full_ratio..1
 *  block           tokens per block, 16..16384 (the pages use 128)
 *  recent_n        trailing tokens of each sequence always kept (their blocks)
 *  min_keep        minimum kept tokens per sequence
 */
typedef struct sffn_block_policy {
    double mass_thresh;
    float min_full_ratio;
    float max_full_ratio;
    int32_t block;
    int32_t recent_n;
    int32_t min_keep;
    int32_t reserved;
} sffn_block_policy;

/*
 * For each sequence q = [cu_seqlens[q], cu_seqlens[q+1]) of the rows tokens:
 * scores s_i = ||A_i||_2 as for SFFN_MODE_TOKENS; blocks of `block` tokens
 * from the sequence start (the last may be short), S_b = fp64 sum of the
 * block's scores in token order; blocks ranked by (S_b desc, b asc); c_k =
 * fp64 sum of the k top-ranked S_b in rank order.  mass >= 1 or c_nb = 0 keeps
 * the whole sequence; otherwise K = the smallest k with c_k >= mass * c_nb (0
 * when mass <= 0), then K = max(min(K, floorf(nb * max_full_ratio)),
 * ceilf(nb * min_full_ratio)) in fp32; kept: the top K blocks, the blocks
 * holding the last recent_n tokens, then further blocks in rank order until
 * min(min_keep, length) tokens are kept.
 *  A           device bf16 [rows][d_model], 16-byte aligned; the layer needs
 *              SFFN_LAYOUT_PREFILL; 1 <= rows <= max_rows
 *  cu_seqlens  device int32 [nseq + 1], 0 = cu[0] <= cu[1] <= ... <= cu[nseq] =
 *              rows; 1 <= nseq <= rows (other contents are clamped to [0, rows]
 *              and made non-decreasing, never read or written out of bounds)
 *  idx_out     device int32, capacity rows: kept token indices, ascending
 *              (sequence by sequence); count_out (device, one int32) their number
 * Asynchronous on `stream`; no host synchronisation.  Errors: INVALID_ARG for
 * a null pointer, a size or policy out of range or a layer without the prefill
 * layout; WORKSPACE for a small scratch.
 */
sffn_status sffn_select_blocks(sffn_t layer, const sffn_block_policy *policy, const void *A, int32_t rows,
                               const int32_t *cu_seqlens, int32_t nseq, int32_t *idx_out,
                               int32_t *count_out, void *scratch, size_t scratch_bytes, void *stream);

/*
 * Three-tier layer schedule (RedKnot article, section on the token-selective
 * sparse FFN): the mass for layer `layer` is 1 (dense) below dense_until,
 * mass_thresh below deep_layer_start and mass_thresh_deep from there on.
 * Host only.
 */
double sffn_schedule_mass(int32_t layer, int32_t dense_until, int32_t deep_layer_start, double mass_thresh,
                          double mass_thresh_deep);

/* Frees the host-side handle (the persistent buffer stays the caller's). */
void sffn_destroy(sffn_t layer);

/*
 * Adaptive expert top-K (RedKnot article, section on adaptive expert top-K:
 * the routing-probability mass decides how many experts a token activates,
 * threshold 0.50 over the candidate buckets 3..6; the per-depth schedule
 * 6 / 5 / 4 caps the largest bucket).
 *  tau   mass threshold (fp32 compare)
 *  kmin  smallest bucket, >= 1
 *  kmax  largest bucket, kmin..min(16, experts)
 */
typedef struct sffn_expert_policy {
    float tau;
    int32_t kmin;
    int32_t kmax;
    int32_t reserved;
} sffn_expert_policy;

/*
 * For every token t: rank the experts of probs[t][0..experts) by (probability
 * desc, index asc); c_b = the fp32 sum of the b top-ranked probabilities added
 * in rank order; K = the smallest b in [kmin, kmax] with c_b >= tau, else kmax.
 *  probs    device fp32 [tokens][experts], router probabilities, finite (NaN
 *           ranks unspecified; -0 ties with +0), 1 <= experts <= 1024
 *  k_out    device int32 [tokens]: K
 *  idx_out  device int32 [tokens][kmax]: the K experts in rank order, then -1
 *  w_out    device fp32 [tokens][kmax]: their probabilities as stored, then 0
 *  One wave per token; outputs are owned by the caller and fully written.
 * No handle and no workspace; asynchronous on `stream`; tokens = 0 is a no-op.
 * Errors: SFFN_ERR_INVALID_ARG for a null pointer, tokens < 0, experts out of
 * range or a bad policy (checked before any launch).
 */
sffn_status sffn_expert_select(const float *probs, int32_t tokens, int32_t experts,
                               const sffn_expert_policy *policy, int32_t *k_out, int32_t *idx_out,
                               float *w_out, void *stream);

/*
 * Neuron reordering by activation frequency (WiSparse reproduction notes,
 * section 5: count how often each neuron is active, sort the neurons by that
 * frequency and store the weights in that order).
 *
 * sffn_neuron_counts: counts[idx[q]] += 1 for q < min(*count, d_ff), on the
 *   device; idx / count are an active list and its length as written by
 *   sffn_select / sffn_forward (device), counts a device int32 [d_ff] the
 *   caller zero-fills once and passes for every calibration token.  Entries
 *   outside [0, d_ff) are ignored.  Asynchronous on `stream`.
 *   Errors: SFFN_ERR_INVALID_ARG (null pointer, d_ff outside 1..65536).
 *
 * sffn_frequency_order (host memory, synchronous, no GPU work): perm[j] = the
 *   original neuron placed at position j, from counts[d_ff] >= 0.
 *   SFFN_ORDER_CLUSTER: neurons by (count desc, index asc), the page's order;
 *     frequently active neurons share the 16-row tiles of the batched path.
 *   SFFN_ORDER_BALANCE: neurons in rank order dealt in a snake
 *     (0, 1, ..., G-1, G-1, ..., 0, 0, ...) over G = ceil(d_ff / block) blocks
 *     of `block` consecutive positions (the last one shorter, full blocks
 *     passed over), each block in ascending index order; with block =
 *     sffn_decode_block_rows(d_ff) every workgroup of the batch-1 kernel gets
 *     an equal share of hot and cold neurons.
 *   Errors: SFFN_ERR_INVALID_ARG (null pointer, d_ff < 1, unknown mode,
 *   block outside 1..d_ff for BALANCE, a negative count).
 *
 * sffn_decode_block_rows: consecutive neurons per workgroup of the batch-1
 *   decode kernel for this d_ff (0 for d_ff < 1).
 *
 * sffn_create_permuted: as sffn_create for fp32 / bf16 weights (no scales),
 *   with the neurons stored in the order perm (device int32 [d_ff], new neuron
 *   j = original neuron perm[j]; read once, not retained).  The layer computes
 *   the same FFN; selections, lists and g' use the new numbering (map them
 *   back through perm).  The permutation is copied to the host and checked
 *   before any kernel uses it.  Errors: as sffn_create, SFFN_ERR_UNSUPPORTED
 *   for int4 weights (W_down's scale groups run along d_ff, so moving a neuron
 *   would change its quantisation), SFFN_ERR_INVALID_ARG if perm is null or
 *   not a permutation of 0..d_ff-1.
 */
enum { SFFN_ORDER_CLUSTER = 0, SFFN_ORDER_BALANCE = 1 };

sffn_status sffn_neuron_counts(const int32_t *idx, const int32_t *count, int32_t d_ff, int32_t *counts,
                               void *stream);
sffn_status sffn_frequency_order(const int32_t *counts, int32_t d_ff, int32_t mode, int32_t block, int32_t *perm);
int32_t sffn_decode_block_rows(int32_t d_ff);
sffn_status sffn_create_permuted(const sffn_layer_desc *desc, const void *w_gate, const void *w_up,
                                 const void *w_down, const int32_t *perm, void *persistent, size_t persistent_bytes,
                                 void *stream, sffn_t *out);

/* Static text for a status code. */
const char *sffn_status_string(sffn_status status);

/* Last HIP error text recorded by this thread, or "" (diagnostics only). */
const char *sffn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SFFN_H */
