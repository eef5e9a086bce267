/*
 * hsakv.h - C ABI of the MI355X (gfx950) HSA + HKV forward library, libhsakv.so.
 *
 * One chunk-layer of WorldAttention's Hybrid Sparse Attention (HSA) over a
 * Hierarchical KV Cache (HKV) active set, as described by the pages about the
 * paper "WorldAttention: An Efficient Attention Architecture for Interactive
 * Video World Models" (arXiv 2609.34606). The technical source is the
 * ai4snews news summary of the paper (English and Chinese editions): its HKV
 * paragraph (semantic pages of Psize = 8 frames; two-stage prompt-level then
 * page-level retrieval of the top-Kp pages; Table 5), its HSA paragraph (a
 * Linformer-style low-rank global branch plus a head-adaptive block-sparse
 * branch that keeps, per head, the fewest blocks whose cumulative attention
 * mass reaches tau_h, with Binter = 128 history and Bintra = 64 in-chunk
 * blocks, fused by learned gates; Table 4) and its kernel paragraph (KV
 * reorganisation and contiguous copies dominate the cost; Tables 9-11).
 *
 * The pages print no equations; where they are silent the library takes
 * the plainest reading, stated at each entry point below.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Element type: `dims->dtype` selects the storage type of q, k/v (chunk,
 *    pool, history), E, F and out: HSAKV_F32 (IEEE float32) or HSAKV_BF16
 *    (bfloat16). Arithmetic accumulates in float32. page_kmean, w_g, b_g,
 *    o_sparse, o_linear, gate, block_mass are float32 in every mode.
 *  - Layouts are dense, row-major, no padding:
 *      q, k_intra, v_intra, out, o_sparse, o_linear : [Lq][H][d]
 *      pool_k, pool_v                               : [P][Tp][H][d], Tp = Psize*tokens_per_frame
 *      k_hist, v_hist (the active cache)            : [Kp*Tp][H][d]; slot s in rows [s*Tp, (s+1)*Tp)
 *      page_kmean                                   : [P][H][d]
 *      E, F                                         : [r][L], L = Kp*Tp + Lq; slot s owns columns
 *                                                     [s*Tp, (s+1)*Tp), the chunk owns the last Lq
 *      sel_count                                    : [H][NQB]
 *      sel_idx                                      : [H][NQB][NB_max], ascending block ids
 *      block_mass, sel_mask                         : [H][NQB][NB_max]
 *    with NQB = ceil(Lq/Bq), NBh = ceil(n_sel*Tp/Binter), NBc = ceil(Lq/Bintra),
 *    NB = NBh + NBc and NB_max = ceil(Kp*Tp/Binter) + NBc. Block ids run over
 *    history blocks first, then chunk blocks.
 *  - Pointers: "device" pointers are HIP device memory of the current
 *    device and must be 16-byte aligned; "host" pointers are ordinary host
 *    memory read before the call returns. `stream` is a hipStream_t (NULL is
 *    the null stream). The caller owns every buffer; the library allocates
 *    nothing and keeps no pointer after returning. Buffers must stay alive
 *    until the stream's work completes. Outputs must not alias inputs.
 *  - Scratch: entry points that need scratch take a device workspace `ws`
 *    of `ws_bytes` bytes, 256-byte aligned, at least
 *    hsakv_workspace_bytes(dims, entry). Its contents on entry are ignored.
 *  - Asynchrony: everything is enqueued on `stream`; no call synchronises
 *    the host or the device. n_sel and page_idx stay on the device; grids
 *    are sized for Kp pages and work past n_sel*Tp exits early.
 *  - Errors: every entry point returns HSAKV_OK (0) or a negative status.
 *    All argument checks happen on the host before anything is enqueued, so
 *    an error leaves every output untouched. A failed launch returns
 *    HSAKV_ERR_HIP and hsakv_last_hip_error() gives the hipError_t of the
 *    calling thread.
 *  - Thread safety: reentrant; calls on different streams may overlap if
 *    their output and workspace buffers are disjoint.
 */
#ifndef HSAKV_H
#define HSAKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HSAKV_VERSION 1

/* status codes */
#define HSAKV_OK                   0
#define HSAKV_ERR_NULL_ARG        -1
#define HSAKV_ERR_BAD_DIMS        -2
#define HSAKV_ERR_BAD_DTYPE       -3
#define HSAKV_ERR_BAD_TAU         -4
#define HSAKV_ERR_WORKSPACE       -5
#define HSAKV_ERR_MISALIGNED      -6
#define HSAKV_ERR_HIP             -7
#define HSAKV_ERR_UNSUPPORTED     -8

/* element types */
#define HSAKV_F32   0
#define HSAKV_BF16  1

/* entry ids for hsakv_workspace_bytes */
#define HSAKV_ENTRY_GATHER   1
#define HSAKV_ENTRY_SELECT   2
#define HSAKV_ENTRY_SPARSE   3
#define HSAKV_ENTRY_LINEAR   4
#define HSAKV_ENTRY_FORWARD  6

/* Sizes of one chunk-layer; all host integers. Supported: d in {64, 128};
 * Bq = 64; Binter and Bintra multiples of 64 up to 512; r a multiple of 32
 * up to 1024; NB_max <= 4096; 1 <= Kp <= 64; 1 <= P <= 65536; H <= 1024. */
typedef struct hsakv_dims {
    int32_t H;                /* attention heads */
    int32_t d;                /* head dimension */
    int32_t Lq;               /* current-chunk tokens: queries and in-chunk keys */
    int32_t tokens_per_frame; /* latent tokens per video frame */
    int32_t Psize;            /* frames per page (8 on the pages); Tp = Psize * tokens_per_frame */
    int32_t P;                /* pages in the HBM pool */
    int32_t Kp;               /* pages retrieved per chunk-layer (4 on the pages) */
    int32_t Binter;           /* history key-block size (128 on the pages) */
    int32_t Bintra;           /* in-chunk key-block size (64 on the pages) */
    int32_t Bq;               /* query-block size: one block set per (head, query block) */
    int32_t r;                /* Linformer rank */
    int32_t dtype;            /* HSAKV_F32 or HSAKV_BF16 */
} hsakv_dims;

/* Inputs of the fused forward; every pointer is device memory. */
typedef struct hsakv_inputs {
    const void*    q;            /* [Lq][H][d] dtype */
    const void*    k_intra;      /* [Lq][H][d] dtype: the chunk's own keys */
    const void*    v_intra;      /* [Lq][H][d] dtype */
    const void*    pool_k;       /* [P][Tp][H][d] dtype */
    const void*    pool_v;       /* [P][Tp][H][d] dtype */
    const float*   page_kmean;   /* [P][H][d] f32, from hkv_page_summary */
    const int32_t* page_prompt;  /* [P] prompt id of each page */
    const void*    E;            /* [r][L] dtype */
    const void*    F;            /* [r][L] dtype */
    const float*   w_g;          /* [H][d] f32 gate weights */
    const float*   b_g;          /* [H] f32 gate biases */
} hsakv_inputs;

/* Outputs of the fused forward. `out` is required; every other pointer is
 * optional (NULL: kept in the workspace and not returned). */
typedef struct hsakv_outputs {
    void*    out;        /* [Lq][H][d] dtype */
    int32_t* page_idx;   /* [Kp] */
    int32_t* n_sel;      /* [1] */
    void*    k_hist;     /* [Kp*Tp][H][d] dtype */
    void*    v_hist;     /* [Kp*Tp][H][d] dtype */
    int32_t* sel_count;  /* [H][NQB] */
    int32_t* sel_idx;    /* [H][NQB][NB_max] */
    float*   o_sparse;   /* [Lq][H][d] f32 */
    float*   o_linear;   /* [Lq][H][d] f32 */
    float*   gate;       /* [Lq][H] f32 */
} hsakv_outputs;

/* ---- helpers (host only; none touches the GPU) ---- */

int         hsakv_version(void);
const char* hsakv_status_str(int status);
/* hipError_t of the last failed launch on the calling thread (0 if none). */
int         hsakv_last_hip_error(void);
/* Checks dims against the supported set; HSAKV_OK or a negative status. */
int         hsakv_validate(const hsakv_dims* dims);
/* Workspace bytes `entry` needs for these dims (0 if dims are invalid). */
size_t      hsakv_workspace_bytes(const hsakv_dims* dims, int32_t entry);

/* ---- entry points ---- */

/* Page summary: page_kmean[p][h][:] = mean over the page's Tp tokens of
 * pool_k[p][:][h][:]. Commit-time metadata of each semantic page (HKV
 * paragraph: semantically indexed pages; the score that uses it is the
 * page-level retrieval stage). Reads pool_k (device), writes page_kmean
 * (device, f32 [P][H][d]). Float32 accumulation in a fixed order, so
 * identical pages give identical means. */
int hkv_page_summary(const hsakv_dims* dims, const void* pool_k, float* page_kmean, void* stream);

/* Two-stage retrieval and active-cache assembly (HKV paragraph: prompt-level
 * then page-level top-Kp; kernel paragraph: contiguous copies).
 *  1. Prompt stage: candidates are the pages with page_prompt[p] == cur_prompt
 *     (the single matching prompt: Top-1, per the open-questions paragraph).
 *  2. Page stage: s_p = sum over heads and dims of page_kmean[p] * mean-over-
 *     chunk(q), in float32. The min(Kp, #candidates) best pages are kept,
 *     equal scores to the lower page index, and stored in ascending page
 *     order: page_idx[0..n_sel) (device, int32 [Kp]; entries past n_sel are
 *     set to -1) and *n_sel (device).
 *  3. Gather: k_hist[s*Tp + t] = pool_k[page_idx[s]][t] for s < n_sel, same
 *     for v; a bit copy. Rows at or past n_sel*Tp are not written.
 * q is [Lq][H][d] (device). cur_prompt is a host value. Workspace:
 * HSAKV_ENTRY_GATHER. */
int hkv_gather(const hsakv_dims* dims, const void* pool_k, const void* pool_v,
               const float* page_kmean, const int32_t* page_prompt, int32_t cur_prompt,
               const void* q, int32_t* page_idx, int32_t* n_sel, void* k_hist, void* v_hist,
               void* ws, size_t ws_bytes, void* stream);

/* Head-adaptive block selection (HSA paragraph: per head, the fewest blocks
 * whose cumulative attention mass reaches tau_h; Binter history blocks,
 * Bintra chunk blocks).
 *  - Keys are [k_hist rows 0..n_sel*Tp) ; k_intra], tiled into blocks as in
 *    the layout notes. Queries are tiled into blocks of Bq.
 *  - Pooling: qb and kb are the means over each block's valid tokens.
 *  - Mass of row (h, i) over blocks b: softmax_b(<qb[h,i], kb[h,b]> / sqrt(d)).
 *  - Selection: rank blocks by mass (larger first, equal masses to the lower
 *    id), keep the shortest prefix whose float32 cumulative mass is >= tau[h];
 *    tau[h] >= 1 keeps every block; at least one block is kept.
 * Outputs (device): sel_count[h][i]; sel_idx[h][i][0..count) ascending ids
 * (entries past count are undefined); sel_mask[h][i][b] in {0,1} for
 * b < NB (optional, NULL to skip); block_mass[h][i][b] for b < NB (optional).
 * n_sel is device memory written by hkv_gather. tau is a host array of H
 * floats in (0, 1] (else HSAKV_ERR_BAD_TAU). Workspace: HSAKV_ENTRY_SELECT. */
int hsa_select(const hsakv_dims* dims, const void* q, const void* k_hist, const void* k_intra,
               const int32_t* n_sel, const float* tau, int32_t* sel_count, int32_t* sel_idx,
               uint8_t* sel_mask, float* block_mass, void* ws, size_t ws_bytes, void* stream);

/* Block-sparse exact attention (HSA paragraph: the sparse branch). For each
 * query t of query block i and head h:
 *   o_sparse[t][h] = sum_j softmax_j(<q[t,h], K[j,h]> / sqrt(d)) V[j,h]
 * over the tokens j of the blocks sel_idx[h][i][0..sel_count[h][i]), where
 * K, V are the key sequence [k_hist rows 0..n_sel*Tp) ; k_intra]. No mask.
 * o_sparse is f32 [Lq][H][d] (device). Workspace: HSAKV_ENTRY_SPARSE; with
 * bf16 it holds the work plan (union of the selected blocks of every four
 * query blocks of a head, tile offsets) and the softmax partials of query
 * blocks whose tiles are split between work-groups. Its contents are scratch:
 * calls that overlap in time must not share a workspace. */
int hsa_sparse_attn(const hsakv_dims* dims, const void* q, const void* k_hist, const void* v_hist,
                    const void* k_intra, const void* v_intra, const int32_t* n_sel,
                    const int32_t* sel_count, const int32_t* sel_idx, float* o_sparse,
                    void* ws, size_t ws_bytes, void* stream);

/* Linformer-style low-rank global branch (HSA paragraph; the Linformer paper
 * on the citation map). One E and one F, shared by every head:
 *   K'_h = E_act K_h, V'_h = F_act V_h            (r x d each, f32)
 *   o_linear[t][h] = softmax(<q[t,h], K'_h> / sqrt(d)) V'_h
 * where E_act, F_act are the columns of E, F facing the present keys
 * (slots s < n_sel, then the chunk). k_low, v_low (device f32 [r][H][d])
 * are optional outputs of K', V'. Workspace: HSAKV_ENTRY_LINEAR. */
int hsa_linear_branch(const hsakv_dims* dims, const void* q, const void* k_hist, const void* v_hist,
                      const void* k_intra, const void* v_intra, const int32_t* n_sel,
                      const void* E, const void* F, float* o_linear, float* k_low, float* v_low,
                      void* ws, size_t ws_bytes, void* stream);

/* Gated fusion (HSA paragraph: learned gates). Per token and head:
 *   g = sigmoid(<q[t,h], w_g[h]> + b_g[h]),  out = g*o_sparse + (1-g)*o_linear
 * out is dtype [Lq][H][d] (bf16 rounded to nearest even); gate (optional,
 * f32 [Lq][H]) receives g. All pointers are device memory. */
int hsa_fuse(const hsakv_dims* dims, const void* q, const float* w_g, const float* b_g,
             const float* o_sparse, const float* o_linear, void* out, float* gate, void* stream);

/* The whole chunk-layer: retrieval and gather, selection, linear branch,
 * sparse attention and the gate, with the gate fused into the sparse
 * attention's epilogue. Results equal the separate entry points run in that
 * order. tau (host, H floats) and cur_prompt (host) as above. Workspace:
 * HSAKV_ENTRY_FORWARD.
 * For bf16 the low-rank branch runs on a second, library-owned stream of
 * the current device (one per device, default priority), forked from
 * `stream` after the gather and joined back into it with events before the
 * attention, so all of the call's work is still ordered on `stream`. Calls
 * from several host threads on one device share that stream: they stay
 * correct but serialise their low-rank branches. */
int hsa_forward(const hsakv_dims* dims, const float* tau, int32_t cur_prompt,
                const hsakv_inputs* in, hsakv_outputs* out, void* ws, size_t ws_bytes,
                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HSAKV_H */
