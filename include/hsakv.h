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
 *    their output and workspace buffers are disjoint. The only state kept
 *    between calls is the compute-unit count of each device, looked up once
 *    and cached atomically.
 */
#ifndef HSAKV_H
#define HSAKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HSAKV_VERSION 6

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
#define HSAKV_ERR_TOO_LARGE       -9   /* scratch beyond HSAKV_STATIC_SCRATCH_BYTES */

/* Size of the fixed device scratch of hsa_sparse_attn_static (per GPU). */
#define HSAKV_STATIC_SCRATCH_BYTES (128u << 20)

/* element types */
#define HSAKV_F32   0
#define HSAKV_BF16  1

/* entry ids for hsakv_workspace_bytes */
#define HSAKV_ENTRY_GATHER   1
#define HSAKV_ENTRY_SELECT   2
#define HSAKV_ENTRY_SPARSE   3
#define HSAKV_ENTRY_LINEAR   4
#define HSAKV_ENTRY_FORWARD  6
#define HSAKV_ENTRY_SUMMARY  7
#define HSAKV_ENTRY_COMMIT   8   /* enough for a commit of up to Lq tokens */
#define HSAKV_ENTRY_BACKWARD 9
#define HSAKV_ENTRY_SPARSE_STATIC 10  /* scratch hsa_sparse_attn_static uses of its fixed array */

/* Sizes of one chunk-layer; all host integers. Supported: d in {64, 128};
 * Bq = 64; Binter and Bintra multiples of 64 up to 512; r a multiple of 32
 * up to 1024; NB_max <= 4096; 1 <= Kp <= 64; 1 <= P <= 65536; H <= 256 and
 * H * d <= 16384; r * L * (bytes per element) < 2^31 (E and F are addressed
 * with 32-bit byte offsets). Anything else returns HSAKV_ERR_UNSUPPORTED or
 * HSAKV_ERR_BAD_DIMS. */
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

/* Retrieval policies. TWO_STAGE is the method (prompt-level filter, then the
 * top-Kp pages by page score); the others are the alternatives the pages
 * compare it with under the same page budget (HKV paragraph, Table 6;
 * Table 5's sliding window of recent frames is RECENT). Each keeps Kp
 * pages (fewer if fewer are candidates), ties to the lower page, slots in
 * ascending page order:
 *   PAGE_ONLY    every page, by page score
 *   PROMPT_ONLY  the Kp most recent (highest-index) prompt-matching pages
 *   RECENT       the Kp most recent pages
 *   RANDOM       every page, by the top 24 bits of output p of SplitMix64
 *                seeded with `seed` (Steele, Lea and Flood, OOPSLA 2014)
 *   MISMATCHED   the pages of other prompts, by page score */
#define HSAKV_POLICY_TWO_STAGE    0
#define HSAKV_POLICY_PAGE_ONLY    1
#define HSAKV_POLICY_PROMPT_ONLY  2
#define HSAKV_POLICY_RECENT       3
#define HSAKV_POLICY_RANDOM       4
#define HSAKV_POLICY_MISMATCHED   5

/* Retrieval options (host struct; NULL means TWO_STAGE). A policy outside
 * 0..5 returns HSAKV_ERR_UNSUPPORTED. */
typedef struct hsakv_retrieval {
    int32_t  policy;
    int32_t  reserved;   /* set to 0 */
    uint64_t seed;       /* RANDOM only */
} hsakv_retrieval;

/* Page tiers (HKV paragraph: pages live in tiers, GPU HBM above CPU DRAM,
 * and unselected pages are demoted to the cheaper tier so that GPU memory
 * does not grow with the video's length). The pinned host store holds every
 * page, indexed by page id, as [P][Tp][H][d] (host_k, host_v: the device
 * addresses of pinned host memory, e.g. from hsakv_host_alloc); the HBM
 * pool (pool_k, pool_v of the calls below) then holds `slots` pages that
 * cache some of them. page_slot (device int32 [P]) gives, for page p, its
 * HBM slot (>= 0) or -1 when the page is only in the host store; the gather
 * then reads it from host memory over the bus (slower, same bits). NULL
 * tiers: page p is page p of the HBM pool (the whole pool in HBM).
 * hkv_tier_apply writes page_slot; the gathers read it. */
typedef struct hsakv_tiers {
    int32_t*    page_slot;
    const void* host_k;
    const void* host_v;
} hsakv_tiers;

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

/* A second stream and two events for hsa_forward, owned by the caller.
 * `stream` is a hipStream_t on the device of the call's stream; `fork` and
 * `join` are hipEvent_t (timing disabled is enough). hsa_forward records
 * `fork` on its stream after the gather, makes `stream` wait on it, runs the
 * low-rank branch there, records `join` on `stream` and makes its own stream
 * wait on `join` before the attention: all of the call's work stays ordered
 * on the call's stream. One fork serves one call at a time: calls that
 * overlap in time (several host threads) each need their own. */
typedef struct hsakv_fork {
    void* stream;
    void* fork;
    void* join;
} hsakv_fork;

/* ---- helpers (host only; none touches the GPU) ---- */

int         hsakv_version(void);
const char* hsakv_status_str(int status);
/* hipError_t of the last failed launch on the calling thread (0 if none). */
int         hsakv_last_hip_error(void);
/* Checks dims against the supported set; HSAKV_OK or a negative status. */
int         hsakv_validate(const hsakv_dims* dims);
/* Workspace bytes `entry` needs for these dims (0 if dims are invalid). */
size_t      hsakv_workspace_bytes(const hsakv_dims* dims, int32_t entry);

/* Creates the stream (non-blocking, default priority) and the two events of
 * a fork on the current device; the caller owns them and releases them with
 * hsakv_fork_destroy. These two calls are the only ones that create HIP
 * objects; they are set-up calls, made once, never on the hot path.
 * Returns HSAKV_OK, HSAKV_ERR_NULL_ARG or HSAKV_ERR_HIP (nothing is left
 * created on an error). */
int hsakv_fork_create(hsakv_fork* fork);
/* Destroys what hsakv_fork_create made (after the work that uses it is
 * done) and clears the struct. */
int hsakv_fork_destroy(hsakv_fork* fork);

/* ---- entry points ---- */

/* Page summary: page_kmean[p][h][:] = mean over the page's Tp tokens of
 * pool_k[p][:][h][:]. Commit-time metadata of each semantic page (HKV
 * paragraph: semantically indexed pages; the score that uses it is the
 * page-level retrieval stage). Reads pool_k (device), writes page_kmean
 * (device, f32 [P][H][d]). Float32 accumulation in a fixed order (each page
 * in 32 row slabs, then the slab sums in slab order), so identical pages
 * give identical means, and a page's mean is the same bits as the one
 * hkv_page_commit gives it. Workspace: HSAKV_ENTRY_SUMMARY. */
int hkv_page_summary(const hsakv_dims* dims, const void* pool_k, float* page_kmean, void* ws,
                     size_t ws_bytes, void* stream);

/* Page commit (HKV paragraph: the history's KV pairs are cut into semantic
 * pages of Psize frames, indexed for the prompt-level and page-level
 * retrieval stages; project page, second caption). The history is one token
 * sequence; page p of the pool holds its tokens [p*Tp, (p+1)*Tp), and
 * `fill` (host) tokens are already committed. The chunk's n_tokens rows of
 * k_chunk, v_chunk (device, [n_tokens][H][d] dtype) become history tokens
 * [fill, fill + n_tokens): pool rows, since pages are consecutive. Every
 * page the commit completes (fill < (p+1)*Tp <= fill + n_tokens) is
 * finalised: page_kmean[p] (device f32 [P][H][d]) is its page-mean key,
 * computed exactly as hkv_page_summary does, and page_prompt[p] (device
 * int32 [P]) is set to cur_prompt (host). Other pages' means and tags are
 * untouched. Only finalised pages should be offered to retrieval: pass
 * dims->P = (fill + n_tokens) / Tp finalised pages to hkv_gather and
 * hsa_forward. dims->P here is the pool's capacity in pages; fill +
 * n_tokens beyond P*Tp returns HSAKV_ERR_BAD_DIMS. n_tokens = 0 does
 * nothing. Workspace: HSAKV_ENTRY_COMMIT covers commits of up to dims->Lq
 * tokens; a commit completing c pages needs c * 32 * H * d * 4 bytes (none
 * when it completes no page). */
int hkv_page_commit(const hsakv_dims* dims, void* pool_k, void* pool_v, float* page_kmean,
                    int32_t* page_prompt, const void* k_chunk, const void* v_chunk, int32_t n_tokens,
                    int64_t fill, int32_t cur_prompt, void* ws, size_t ws_bytes, void* stream);

/* Two-stage retrieval and active-cache assembly (HKV paragraph: prompt-level
 * then page-level top-Kp; kernel paragraph: contiguous copies).
 *  1. Prompt stage: candidates are the pages with page_prompt[p] == cur_prompt
 *     (the single matching prompt: Top-1, per the open-questions paragraph).
 *  2. Page stage: s_p = sum over heads and dims of page_kmean[p] * mean-over-
 *     chunk(q), summed in float64 and rounded to float32, the precision the
 *     ranking is decided in (a score that is not a number ranks below every
 *     number). The min(Kp, #candidates) best pages are kept,
 *     equal scores to the lower page index, and stored in ascending page
 *     order: page_idx[0..n_sel) (device, int32 [Kp]; entries past n_sel are
 *     set to -1) and *n_sel (device).
 *  3. Gather: k_hist[s*Tp + t] = pool_k[page_idx[s]][t] for s < n_sel, same
 *     for v; a bit copy. Rows at or past n_sel*Tp are not written.
 * q is [Lq][H][d] (device). cur_prompt is a host value. `retrieval` (host,
 * nullable) selects another policy for steps 1-2 (see hsakv_retrieval).
 * `tiers` (host, nullable) reads the pages through a page table (see
 * hsakv_tiers). Workspace: HSAKV_ENTRY_GATHER. */
int hkv_gather(const hsakv_dims* dims, const void* pool_k, const void* pool_v,
               const float* page_kmean, const int32_t* page_prompt, int32_t cur_prompt,
               const hsakv_retrieval* retrieval, const hsakv_tiers* tiers, const void* q,
               int32_t* page_idx, int32_t* n_sel, void* k_hist, void* v_hist, void* ws,
               size_t ws_bytes, void* stream);

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

/* hsa_sparse_attn (bf16) in its two parts, for callers that run the plan
 * beside other work (as hsa_forward does) or time the attention alone.
 * hsa_sparse_plan reads the selection only (n_sel, sel_count, sel_idx) and
 * writes the work plan into the workspace: the rows of each head grouped
 * four at a time by selection overlap, each group's union of selected
 * blocks as 64-key tiles, and the global tile sequence. hsa_sparse_compute
 * then runs the attention over that plan and merges split groups, writing
 * o_sparse exactly as hsa_sparse_attn does. Both take the same workspace
 * (HSAKV_ENTRY_SPARSE), which must not change between the two calls;
 * compute must be ordered after plan. float32 data returns
 * HSAKV_ERR_BAD_DTYPE (its attention has no separate plan). */
int hsa_sparse_plan(const hsakv_dims* dims, const int32_t* n_sel, const int32_t* sel_count,
                    const int32_t* sel_idx, void* ws, size_t ws_bytes, void* stream);
int hsa_sparse_compute(const hsakv_dims* dims, const void* q, const void* k_hist, const void* v_hist,
                       const void* k_intra, const void* v_intra, const int32_t* n_sel, float* o_sparse,
                       void* ws, size_t ws_bytes, void* stream);

/* hsa_sparse_attn without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Arguments,
 * layouts and results are those of hsa_sparse_attn (the same kernels).
 * Scratch: a fixed array of HSAKV_STATIC_SCRATCH_BYTES in device memory,
 * one per GPU, held until the process ends; dims whose plan and partials
 * need more (hsakv_workspace_bytes(dims, HSAKV_ENTRY_SPARSE_STATIC) larger
 * than that) return HSAKV_ERR_TOO_LARGE before anything is enqueued. For
 * more than 8 heads with over 1024 key tiles per group of four query blocks
 * (over 64K history keys per head), hsa_sparse_attn gives each work-group
 * several split ranges; this entry keeps one, so that its partials fit, and
 * its output then differs from hsa_sparse_attn's by float rounding only
 * (the split points of the online softmax differ). The first
 * call on a device looks up that device's copy of the array (no
 * allocation). Every call on a GPU shares its array and leaves its contents
 * behind; nothing in it must start at zero. Calls that overlap in time on
 * one GPU (several streams or host threads) race on the array and must be
 * serialised by the caller. */
int hsa_sparse_attn_static(const hsakv_dims* dims, const void* q, const void* k_hist,
                           const void* v_hist, const void* k_intra, const void* v_intra,
                           const int32_t* n_sel, const int32_t* sel_count, const int32_t* sel_idx,
                           float* o_sparse, void* stream);

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
 * order. tau (host, H floats), cur_prompt (host), retrieval and tiers
 * (host, nullable) as above. Workspace: HSAKV_ENTRY_FORWARD.
 * `fork` (host, nullable): with a fork whose stream is set and bf16 data, the
 * low-rank branch runs on the fork's stream beside the selection (see
 * hsakv_fork); NULL, or a fork with a NULL stream, runs everything on
 * `stream`. The results are the same either way. float32 data always runs on
 * `stream`. */
int hsa_forward(const hsakv_dims* dims, const float* tau, int32_t cur_prompt,
                const hsakv_retrieval* retrieval, const hsakv_tiers* tiers,
                const hsakv_inputs* in, hsakv_outputs* out, void* ws, size_t ws_bytes,
                void* stream, const hsakv_fork* fork);

/* Backward of the learned parameters (HSA paragraph: the branches are fused
 * by learned gates, and the global branch is a Linformer-style projection
 * with parameters E, F; the Linformer paper on the citation map). For an
 * upstream gradient d_out = dLoss/dout (device, [Lq][H][d] bf16) of the
 * chunk-layer's output, writes the gradients of the gate weights d_wg
 * ([H][d] f32), biases d_bg ([H] f32) and of E and F, d_E and d_F ([r][L]
 * f32, zero at the columns of absent slots). The sparse branch has no
 * learned parameter and is held fixed. With g = sigmoid(<q, w_g[h]> +
 * b_g[h]), dx = <d_out, o_sparse - o_linear> g (1 - g): d_wg[h] = sum_t dx q
 * and d_bg[h] = sum_t dx; with dO_l = (1 - g) d_out and P = softmax(q K'^T /
 * sqrt d): dV' = P^T dO_l, dK' = (P * (dO_l V'^T - <dO_l, o_linear>))^T q /
 * sqrt d, d_E = sum_h dK'_h K_h^T and d_F = sum_h dV'_h V_h^T over the
 * active keys. Inputs are the forward's: q, k_hist, v_hist, k_intra,
 * v_intra, n_sel (device) as for hsa_linear_branch; w_g (16-byte aligned),
 * b_g; k_low, v_low
 * (K', V' from hsa_linear_branch, f32 [r][H][d]); o_sparse, o_linear (f32
 * [Lq][H][d]). bf16 only (float32 data returns HSAKV_ERR_BAD_DTYPE);
 * (Kp Tp + Lq) H d 2 bytes must stay below 2^31 (else HSAKV_ERR_UNSUPPORTED).
 * Workspace: HSAKV_ENTRY_BACKWARD. `fork` (host, nullable): with a fork
 * whose stream is set, the gate-parameter sums run on the fork's stream
 * beside the low-rank backward and dE, dF; NULL runs everything on
 * `stream`. Every reduction runs in a fixed order: the
 * results are the same bits from run to run, with or without a fork. */
int hsa_backward_params(const hsakv_dims* dims, const void* q, const void* k_hist, const void* v_hist,
                        const void* k_intra, const void* v_intra, const int32_t* n_sel, const float* w_g,
                        const float* b_g, const float* k_low, const float* v_low, const float* o_sparse,
                        const float* o_linear, const void* d_out, float* d_wg, float* d_bg, float* d_E,
                        float* d_F, void* ws, size_t ws_bytes, void* stream, const hsakv_fork* fork);

/* ---- page tiers ---- */

/* Pinned, device-mapped host memory for the host store (a set-up call, like
 * hsakv_fork_create): *host_ptr for the host's own reads and writes,
 * *device_ptr for hsakv_tiers. Freed with hsakv_host_free(host_ptr). */
int hsakv_host_alloc(size_t bytes, void** host_ptr, void** device_ptr);
int hsakv_host_free(void* host_ptr);

/* Host-only least-recently-used planner of the HBM slots; touches no GPU.
 * slot_of_page [P] (slot or -1), page_of_slot [slots] (page or -1; may be
 * NULL when slots is 0) and
 * last_use [P] are the caller's host copy of the placement, updated in
 * place. The n_want pages of `want` (e.g. the pages the last forwards
 * retrieved, then the newest pages) get last_use = now; each one not in a
 * slot takes a free slot, else the slot of the least recently used page
 * not wanted now (ties to the lower slot), which is demoted to the host
 * store (its slot is simply reused: the host store keeps every page).
 * Outputs: the promotions (promote_page[i] into promote_slot[i]; at most
 * min(n_want, slots)) and the page-table updates (upd_page[i] gets
 * upd_value[i]; at most 2 per promotion) for hkv_tier_apply. */
int hkv_tier_plan(int32_t P, int32_t slots, int32_t* slot_of_page, int32_t* page_of_slot,
                  int64_t* last_use, int64_t now, const int32_t* want, int32_t n_want,
                  int32_t* promote_page, int32_t* promote_slot, int32_t* n_promote,
                  int32_t* upd_page, int32_t* upd_value, int32_t* n_upd);

/* Enqueues the promotions (host store page -> HBM slot copies of K and V,
 * one page of Tp*H*d elements each) and then the page-table updates
 * (n_upd <= 256) on `stream`. The arrays are host memory read before the
 * call returns. Ordering: a slot must not be overwritten while a gather
 * that reads its old page is still pending, and the next gather must see
 * the new table: enqueue this after the previous forward's gather (e.g. on
 * its fork stream) and make the next forward's stream wait for it. */
int hkv_tier_apply(const hsakv_dims* dims, const hsakv_tiers* tiers, void* pool_k, void* pool_v,
                   int32_t slots, const int32_t* promote_page, const int32_t* promote_slot,
                   int32_t n_promote, const int32_t* upd_page, const int32_t* upd_value,
                   int32_t n_upd, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HSAKV_H */
