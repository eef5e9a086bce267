// Exported C ABI of libhsakv: host-side checks, workspace carving, launches.
// Declarations, argument meaning, layouts and error behaviour: include/hsakv.h.
#include "hsakv.h"

#include <math.h>
#include <string.h>

#include <mutex>

#include "common.h"
#include "launch.h"

#define HSAKV_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local int g_last_hip_error = 0;

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int elt_bytes(const hsakv_dims* d) { return d->dtype == HSAKV_BF16 ? 2 : 4; }

Geo make_geo(const hsakv_dims* d) {
    Geo g;
    g.H = d->H;
    g.d = d->d;
    g.Lq = d->Lq;
    g.Tp = d->Psize * d->tokens_per_frame;
    g.P = d->P;
    g.Kp = d->Kp;
    g.Binter = d->Binter;
    g.Bintra = d->Bintra;
    g.Bq = d->Bq;
    g.r = d->r;
    g.HD = d->H * d->d;
    g.NQB = (d->Lq + d->Bq - 1) / d->Bq;
    g.NBc = (d->Lq + d->Bintra - 1) / d->Bintra;
    g.hist_rows = (long long)d->Kp * g.Tp;
    g.NBh_max = (int)((g.hist_rows + d->Binter - 1) / d->Binter);
    g.NB_max = g.NBh_max + g.NBc;
    g.L = g.hist_rows + d->Lq;
    g.elt = d->dtype == HSAKV_BF16 ? 2 : 4;
    return g;
}

int check_dims(const hsakv_dims* d) {
    if (!d) return HSAKV_ERR_NULL_ARG;
    if (d->dtype != HSAKV_F32 && d->dtype != HSAKV_BF16) return HSAKV_ERR_BAD_DTYPE;
    if (d->H < 1 || d->Lq < 1 || d->tokens_per_frame < 1 || d->Psize < 1 || d->P < 1 ||
        d->Kp < 1 || d->r < 1 || d->d < 1 || d->Bq < 1 || d->Binter < 1 || d->Bintra < 1)
        return HSAKV_ERR_BAD_DIMS;
    if (d->d != 64 && d->d != 128) return HSAKV_ERR_UNSUPPORTED;
    if (d->Bq != 64) return HSAKV_ERR_UNSUPPORTED;
    if (d->Binter % 64 || d->Binter > 512 || d->Bintra % 64 || d->Bintra > 512)
        return HSAKV_ERR_UNSUPPORTED;
    if (d->r % 32 || d->r > 1024) return HSAKV_ERR_UNSUPPORTED;
    if (d->Kp > 64 || d->H > kMaxHeads || (long long)d->H * d->d > 16384) return HSAKV_ERR_UNSUPPORTED;
    const long long Tp = (long long)d->Psize * d->tokens_per_frame;
    if (Tp > (1LL << 30) || (long long)d->Kp * Tp + d->Lq >= (1LL << 31)) return HSAKV_ERR_BAD_DIMS;
    if (d->P > 65536) return HSAKV_ERR_UNSUPPORTED;
    Geo g = make_geo(d);
    if (g.NB_max > 4096) return HSAKV_ERR_UNSUPPORTED;
    // one-dimensional grids of (block, 256 columns) work-groups stay below 2^32 threads
    if ((long long)(g.NQB + g.NB_max) * ((g.HD + 255) / 256) * 256 >= (1LL << 32)) return HSAKV_ERR_UNSUPPORTED;
    if (retrieve_smem_bytes(g) > 65536) return HSAKV_ERR_UNSUPPORTED;
    return HSAKV_OK;
}

int check_tau(const hsakv_dims* d, const float* tau) {
    if (!tau) return HSAKV_ERR_NULL_ARG;
    for (int h = 0; h < d->H; ++h)
        if (!(tau[h] > 0.f && tau[h] <= 1.f)) return HSAKV_ERR_BAD_TAU;   // NaN fails too
    return HSAKV_OK;
}

bool aligned(const void* p, size_t a = 16) { return ((uintptr_t)p % a) == 0; }

int done() {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return HSAKV_ERR_HIP;
    }
    return HSAKV_OK;
}

// A second stream per device (default priority, created on first use and
// kept until the process ends) for work that can run beside the caller's
// stream. nullptr if it cannot be created: the caller then stays on its own
// stream.
hipStream_t side_stream() {
    static std::mutex mu;
    static hipStream_t tab[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!tab[dev] && hipStreamCreateWithFlags(&tab[dev], hipStreamNonBlocking) != hipSuccess) tab[dev] = nullptr;
    return tab[dev];
}

// ---- workspace sizes -------------------------------------------------------

size_t ws_gather(const Geo& g) { return align_up(((size_t)retrieve_slabs(g) + 1) * g.HD * 4); }

size_t ws_select(const Geo& g) {
    return align_up((size_t)g.H * g.NQB * g.d * 4) + align_up((size_t)g.H * g.NB_max * g.d * 4) +
           align_up((size_t)g.H * g.NQB * g.NB_max * 4);   // pooled q, pooled k, block logits
}

size_t ws_sparse(const Geo& g) { return g.elt == 2 ? align_up(sparse_bf16_ws_bytes(g)) : kAlign; }

size_t ws_linear(const Geo& g, int eb) {
    const size_t n = (size_t)g.r * g.HD;
    const size_t parts = align_up((size_t)lowrank_splits(g) * 2 * n * 4);
    const size_t ops = eb == 2 ? 4 * align_up(n * 2) : 2 * align_up(n * 4);
    return parts + ops;
}

size_t ws_forward(const Geo& g, int eb) {
    size_t s = ws_gather(g) + ws_select(g) + ws_sparse(g) + ws_linear(g, eb);
    s += align_up((size_t)g.Kp * 4) + align_up(4);                        // page_idx, n_sel
    s += 2 * align_up((size_t)g.hist_rows * g.HD * eb);                   // k_hist, v_hist
    s += align_up((size_t)g.H * g.NQB * 4);                                // sel_count
    s += align_up((size_t)g.H * g.NQB * g.NB_max * 4);                     // sel_idx
    s += align_up((size_t)g.Lq * g.HD * 4);                                // o_linear
    return s;
}

struct Carver {
    char* p;
    size_t left;
    bool ok = true;
    void* take(size_t n) {
        n = align_up(n);
        if (n > left) { ok = false; return nullptr; }
        void* r = p;
        p += n;
        left -= n;
        return r;
    }
};

// ---- typed bodies ------------------------------------------------------------

template <typename T>
void run_gather(const Geo& g, const void* pool_k, const void* pool_v, const float* page_kmean,
                const int32_t* page_prompt, int cur_prompt, const void* q, int32_t* page_idx,
                int32_t* n_sel, void* k_hist, void* v_hist, float* partial, float* kb, hipStream_t st) {
    launch_q_partials<T>(g, q, partial, st);
    launch_retrieve(g, partial, page_kmean, page_prompt, cur_prompt, page_idx, n_sel, st);
    if (kb)   // the history blocks of the pooled keys come with the copy
        launch_gather_pool<T>(g, pool_k, pool_v, page_idx, n_sel, k_hist, v_hist, kb, st);
    else
        launch_gather(g, (int)sizeof(T), pool_k, pool_v, page_idx, n_sel, k_hist, v_hist, st);
}

template <typename T>
void run_select(const Geo& g, const void* q, const void* k_hist, const void* k_intra,
                const int32_t* n_sel, const TauArg& tau, int32_t* sel_count, int32_t* sel_idx,
                uint8_t* sel_mask, float* block_mass, float* qb, float* kb, float* zl, bool hist_pooled,
                hipStream_t st) {
    launch_pool<T>(g, q, k_hist, k_intra, n_sel, qb, kb, hist_pooled, st);
    launch_select(g, qb, kb, zl, n_sel, tau, sel_count, sel_idx, sel_mask, block_mass, st);
}

template <typename T>
void run_linear(const Geo& g, const void* q, const void* k_hist, const void* v_hist,
                const void* k_intra, const void* v_intra, const int32_t* n_sel, const void* E,
                const void* F, float* o_linear, float* k_low, float* v_low, Carver& c,
                hipStream_t st) {
    const size_t n = (size_t)g.r * g.HD;
    float* part = (float*)c.take((size_t)lowrank_splits(g) * 2 * n * 4);
    void *khi, *vhi, *klo = nullptr, *vlo = nullptr;
    if (sizeof(T) == 2) {
        khi = c.take(n * 2); vhi = c.take(n * 2); klo = c.take(n * 2); vlo = c.take(n * 2);
    } else {
        khi = c.take(n * 4); vhi = c.take(n * 4);
    }
    launch_lowrank_proj<T>(g, E, F, k_hist, v_hist, k_intra, v_intra, n_sel, part, st);
    launch_lowrank_reduce<T>(g, part, k_low, v_low, khi, vhi, klo, vlo, st);
    Epi ep{o_linear, nullptr, nullptr, nullptr, nullptr, nullptr};
    launch_lowrank_attn<T>(g, q, khi, vhi, klo, vlo, ep, st);
}

TauArg pack_tau(const hsakv_dims* d, const float* tau) {
    TauArg t;
    memset(&t, 0, sizeof(t));
    for (int h = 0; h < d->H; ++h) t.v[h] = tau[h];
    return t;
}

}  // namespace

// ---- helpers -------------------------------------------------------------------

HSAKV_API int hsakv_version(void) { return HSAKV_VERSION; }

HSAKV_API const char* hsakv_status_str(int s) {
    switch (s) {
        case HSAKV_OK: return "ok";
        case HSAKV_ERR_NULL_ARG: return "null argument";
        case HSAKV_ERR_BAD_DIMS: return "invalid dimensions";
        case HSAKV_ERR_BAD_DTYPE: return "invalid element type";
        case HSAKV_ERR_BAD_TAU: return "tau outside (0, 1]";
        case HSAKV_ERR_WORKSPACE: return "workspace too small or misaligned";
        case HSAKV_ERR_MISALIGNED: return "device pointer not 16-byte aligned";
        case HSAKV_ERR_HIP: return "HIP launch failed";
        case HSAKV_ERR_UNSUPPORTED: return "unsupported dimensions";
        default: return "unknown status";
    }
}

HSAKV_API int hsakv_last_hip_error(void) { return g_last_hip_error; }

HSAKV_API int hsakv_validate(const hsakv_dims* dims) { return check_dims(dims); }

HSAKV_API size_t hsakv_workspace_bytes(const hsakv_dims* dims, int32_t entry) {
    if (check_dims(dims) != HSAKV_OK) return 0;
    const Geo g = make_geo(dims);
    const int eb = elt_bytes(dims);
    switch (entry) {
        case HSAKV_ENTRY_GATHER: return ws_gather(g);
        case HSAKV_ENTRY_SELECT: return ws_select(g);
        case HSAKV_ENTRY_SPARSE: return ws_sparse(g);
        case HSAKV_ENTRY_LINEAR: return ws_linear(g, eb);
        case HSAKV_ENTRY_FORWARD: return ws_forward(g, eb);
        default: return 0;
    }
}

#define HSAKV_CHECK(expr)                     \
    do {                                      \
        int _s = (expr);                      \
        if (_s != HSAKV_OK) return _s;        \
    } while (0)
#define HSAKV_REQUIRE(cond, code) \
    do {                          \
        if (!(cond)) return code; \
    } while (0)

static int check_ws(void* ws, size_t ws_bytes, size_t need) {
    if (need == 0) return HSAKV_OK;
    if (!ws || ws_bytes < need || !aligned(ws, kAlign)) return HSAKV_ERR_WORKSPACE;
    return HSAKV_OK;
}

// ---- entry points ----------------------------------------------------------------

HSAKV_API int hkv_page_summary(const hsakv_dims* dims, const void* pool_k, float* page_kmean,
                               void* stream) {
    HSAKV_CHECK(check_dims(dims));
    HSAKV_REQUIRE(pool_k && page_kmean, HSAKV_ERR_NULL_ARG);
    HSAKV_REQUIRE(aligned(pool_k) && aligned(page_kmean), HSAKV_ERR_MISALIGNED);
    const Geo g = make_geo(dims);
    hipStream_t st = (hipStream_t)stream;
    if (dims->dtype == HSAKV_BF16) launch_page_summary<bf16_t>(g, pool_k, page_kmean, st);
    else launch_page_summary<float>(g, pool_k, page_kmean, st);
    return done();
}

HSAKV_API int hkv_gather(const hsakv_dims* dims, const void* pool_k, const void* pool_v,
                         const float* page_kmean, const int32_t* page_prompt, int32_t cur_prompt,
                         const void* q, int32_t* page_idx, int32_t* n_sel, void* k_hist,
                         void* v_hist, void* ws, size_t ws_bytes, void* stream) {
    HSAKV_CHECK(check_dims(dims));
    HSAKV_REQUIRE(pool_k && pool_v && page_kmean && page_prompt && q && page_idx && n_sel &&
                      k_hist && v_hist,
                  HSAKV_ERR_NULL_ARG);
    HSAKV_REQUIRE(aligned(pool_k) && aligned(pool_v) && aligned(page_kmean) && aligned(q) &&
                      aligned(k_hist) && aligned(v_hist) && aligned(page_idx, 4) &&
                      aligned(n_sel, 4) && aligned(page_prompt, 4),
                  HSAKV_ERR_MISALIGNED);
    const Geo g = make_geo(dims);
    HSAKV_CHECK(check_ws(ws, ws_bytes, ws_gather(g)));
    hipStream_t st = (hipStream_t)stream;
    if (dims->dtype == HSAKV_BF16)
        run_gather<bf16_t>(g, pool_k, pool_v, page_kmean, page_prompt, cur_prompt, q, page_idx,
                           n_sel, k_hist, v_hist, (float*)ws, nullptr, st);
    else
        run_gather<float>(g, pool_k, pool_v, page_kmean, page_prompt, cur_prompt, q, page_idx,
                          n_sel, k_hist, v_hist, (float*)ws, nullptr, st);
    return done();
}

HSAKV_API int hsa_select(const hsakv_dims* dims, const void* q, const void* k_hist,
                         const void* k_intra, const int32_t* n_sel, const float* tau,
                         int32_t* sel_count, int32_t* sel_idx, uint8_t* sel_mask,
                         float* block_mass, void* ws, size_t ws_bytes, void* stream) {
    HSAKV_CHECK(check_dims(dims));
    HSAKV_REQUIRE(q && k_hist && k_intra && n_sel && sel_count && sel_idx, HSAKV_ERR_NULL_ARG);
    HSAKV_CHECK(check_tau(dims, tau));
    HSAKV_REQUIRE(aligned(q) && aligned(k_hist) && aligned(k_intra) && aligned(n_sel, 4) &&
                      aligned(sel_count, 4) && aligned(sel_idx, 4) && aligned(block_mass, 4),
                  HSAKV_ERR_MISALIGNED);
    const Geo g = make_geo(dims);
    HSAKV_CHECK(check_ws(ws, ws_bytes, ws_select(g)));
    Carver c{(char*)ws, ws_bytes};
    float* qb = (float*)c.take((size_t)g.H * g.NQB * g.d * 4);
    float* kb = (float*)c.take((size_t)g.H * g.NB_max * g.d * 4);
    float* zl = (float*)c.take((size_t)g.H * g.NQB * g.NB_max * 4);
    const TauArg t = pack_tau(dims, tau);
    hipStream_t st = (hipStream_t)stream;
    if (dims->dtype == HSAKV_BF16)
        run_select<bf16_t>(g, q, k_hist, k_intra, n_sel, t, sel_count, sel_idx, sel_mask,
                           block_mass, qb, kb, zl, false, st);
    else
        run_select<float>(g, q, k_hist, k_intra, n_sel, t, sel_count, sel_idx, sel_mask,
                          block_mass, qb, kb, zl, false, st);
    return done();
}

HSAKV_API int hsa_sparse_attn(const hsakv_dims* dims, const void* q, const void* k_hist,
                              const void* v_hist, const void* k_intra, const void* v_intra,
                              const int32_t* n_sel, const int32_t* sel_count,
                              const int32_t* sel_idx, float* o_sparse, void* ws, size_t ws_bytes,
                              void* stream) {
    HSAKV_CHECK(check_dims(dims));
    HSAKV_REQUIRE(q && k_hist && v_hist && k_intra && v_intra && n_sel && sel_count && sel_idx &&
                      o_sparse,
                  HSAKV_ERR_NULL_ARG);
    HSAKV_REQUIRE(aligned(q) && aligned(k_hist) && aligned(v_hist) && aligned(k_intra) &&
                      aligned(v_intra) && aligned(o_sparse) && aligned(n_sel, 4) &&
                      aligned(sel_count, 4) && aligned(sel_idx, 4),
                  HSAKV_ERR_MISALIGNED);
    const Geo g = make_geo(dims);
    HSAKV_CHECK(check_ws(ws, ws_bytes, ws_sparse(g)));
    Epi ep{o_sparse, nullptr, nullptr, nullptr, nullptr, nullptr};
    hipStream_t st = (hipStream_t)stream;
    if (dims->dtype == HSAKV_BF16)
        launch_sparse_attn<bf16_t>(g, q, k_hist, v_hist, k_intra, v_intra, n_sel, sel_count,
                                   sel_idx, ws, ep, st);
    else
        launch_sparse_attn<float>(g, q, k_hist, v_hist, k_intra, v_intra, n_sel, sel_count,
                                  sel_idx, ws, ep, st);
    return done();
}

HSAKV_API int hsa_linear_branch(const hsakv_dims* dims, const void* q, const void* k_hist,
                                const void* v_hist, const void* k_intra, const void* v_intra,
                                const int32_t* n_sel, const void* E, const void* F,
                                float* o_linear, float* k_low, float* v_low, void* ws,
                                size_t ws_bytes, void* stream) {
    HSAKV_CHECK(check_dims(dims));
    HSAKV_REQUIRE(q && k_hist && v_hist && k_intra && v_intra && n_sel && E && F && o_linear,
                  HSAKV_ERR_NULL_ARG);
    HSAKV_REQUIRE(aligned(q) && aligned(k_hist) && aligned(v_hist) && aligned(k_intra) &&
                      aligned(v_intra) && aligned(E) && aligned(F) && aligned(o_linear) &&
                      aligned(k_low) && aligned(v_low) && aligned(n_sel, 4),
                  HSAKV_ERR_MISALIGNED);
    const Geo g = make_geo(dims);
    const int eb = elt_bytes(dims);
    HSAKV_CHECK(check_ws(ws, ws_bytes, ws_linear(g, eb)));
    Carver c{(char*)ws, ws_bytes};
    hipStream_t st = (hipStream_t)stream;
    if (eb == 2)
        run_linear<bf16_t>(g, q, k_hist, v_hist, k_intra, v_intra, n_sel, E, F, o_linear, k_low,
                           v_low, c, st);
    else
        run_linear<float>(g, q, k_hist, v_hist, k_intra, v_intra, n_sel, E, F, o_linear, k_low,
                          v_low, c, st);
    return done();
}

HSAKV_API int hsa_fuse(const hsakv_dims* dims, const void* q, const float* w_g, const float* b_g,
                       const float* o_sparse, const float* o_linear, void* out, float* gate,
                       void* stream) {
    HSAKV_CHECK(check_dims(dims));
    HSAKV_REQUIRE(q && w_g && b_g && o_sparse && o_linear && out, HSAKV_ERR_NULL_ARG);
    HSAKV_REQUIRE(aligned(q) && aligned(w_g, 4) && aligned(b_g, 4) && aligned(o_sparse) &&
                      aligned(o_linear) && aligned(out) && aligned(gate, 4),
                  HSAKV_ERR_MISALIGNED);
    const Geo g = make_geo(dims);
    hipStream_t st = (hipStream_t)stream;
    if (dims->dtype == HSAKV_BF16)
        launch_fuse<bf16_t>(g, q, w_g, b_g, o_sparse, o_linear, out, gate, st);
    else
        launch_fuse<float>(g, q, w_g, b_g, o_sparse, o_linear, out, gate, st);
    return done();
}

HSAKV_API int hsa_forward(const hsakv_dims* dims, const float* tau, int32_t cur_prompt,
                          const hsakv_inputs* in, hsakv_outputs* out, void* ws, size_t ws_bytes,
                          void* stream) {
    HSAKV_CHECK(check_dims(dims));
    HSAKV_REQUIRE(in && out, HSAKV_ERR_NULL_ARG);
    HSAKV_CHECK(check_tau(dims, tau));
    HSAKV_REQUIRE(in->q && in->k_intra && in->v_intra && in->pool_k && in->pool_v &&
                      in->page_kmean && in->page_prompt && in->E && in->F && in->w_g && in->b_g &&
                      out->out,
                  HSAKV_ERR_NULL_ARG);
    HSAKV_REQUIRE(aligned(in->q) && aligned(in->k_intra) && aligned(in->v_intra) &&
                      aligned(in->pool_k) && aligned(in->pool_v) && aligned(in->page_kmean) &&
                      aligned(in->page_prompt, 4) && aligned(in->E) && aligned(in->F) &&
                      aligned(in->w_g, 4) && aligned(in->b_g, 4) && aligned(out->out) &&
                      aligned(out->page_idx, 4) && aligned(out->n_sel, 4) &&
                      aligned(out->k_hist) && aligned(out->v_hist) &&
                      aligned(out->sel_count, 4) && aligned(out->sel_idx, 4) &&
                      aligned(out->o_sparse) && aligned(out->o_linear) && aligned(out->gate, 4),
                  HSAKV_ERR_MISALIGNED);
    const Geo g = make_geo(dims);
    const int eb = elt_bytes(dims);
    HSAKV_CHECK(check_ws(ws, ws_bytes, ws_forward(g, eb)));
    Carver c{(char*)ws, ws_bytes};
    float* partial = (float*)c.take(ws_gather(g));
    float* qb = (float*)c.take((size_t)g.H * g.NQB * g.d * 4);
    float* kb = (float*)c.take((size_t)g.H * g.NB_max * g.d * 4);
    float* zl = (float*)c.take((size_t)g.H * g.NQB * g.NB_max * 4);
    void* sparse_ws = c.take(ws_sparse(g));
    int32_t* page_idx = (int32_t*)c.take((size_t)g.Kp * 4);
    int32_t* n_sel = (int32_t*)c.take(4);
    void* k_hist = c.take((size_t)g.hist_rows * g.HD * eb);
    void* v_hist = c.take((size_t)g.hist_rows * g.HD * eb);
    int32_t* sel_count = (int32_t*)c.take((size_t)g.H * g.NQB * 4);
    int32_t* sel_idx = (int32_t*)c.take((size_t)g.H * g.NQB * g.NB_max * 4);
    float* o_linear = (float*)c.take((size_t)g.Lq * g.HD * 4);
    if (out->page_idx) page_idx = out->page_idx;
    if (out->n_sel) n_sel = out->n_sel;
    if (out->k_hist) k_hist = out->k_hist;
    if (out->v_hist) v_hist = out->v_hist;
    if (out->sel_count) sel_count = out->sel_count;
    if (out->sel_idx) sel_idx = out->sel_idx;
    if (out->o_linear) o_linear = out->o_linear;
    const TauArg t = pack_tau(dims, tau);
    Epi ep{out->o_sparse, out->out, o_linear, out->gate, in->w_g, in->b_g};
    hipStream_t st = (hipStream_t)stream;
    if (eb == 2) {
        run_gather<bf16_t>(g, in->pool_k, in->pool_v, in->page_kmean, in->page_prompt, cur_prompt,
                           in->q, page_idx, n_sel, k_hist, v_hist, partial, kb, st);
        // The low-rank branch needs the gathered KV only: it runs on a side
        // stream beside the pooling, the block selection and the sparse plan
        // (small, latency-bound kernels), and the attention waits for both.
        hipStream_t side = side_stream();
        hipEvent_t fork = nullptr, join = nullptr;
        const bool split = side && side != st &&
                           hipEventCreateWithFlags(&fork, hipEventDisableTiming) == hipSuccess &&
                           hipEventCreateWithFlags(&join, hipEventDisableTiming) == hipSuccess &&
                           hipEventRecord(fork, st) == hipSuccess && hipStreamWaitEvent(side, fork, 0) == hipSuccess;
        run_linear<bf16_t>(g, in->q, k_hist, v_hist, in->k_intra, in->v_intra, n_sel, in->E,
                           in->F, o_linear, nullptr, nullptr, c, split ? side : st);
        const bool joined = split && hipEventRecord(join, side) == hipSuccess;
        run_select<bf16_t>(g, in->q, k_hist, in->k_intra, n_sel, t, sel_count, sel_idx, nullptr,
                           nullptr, qb, kb, zl, true, st);
        launch_sparse_plan_bf16(g, n_sel, sel_count, sel_idx, sparse_ws, st);
        if (joined) (void)hipStreamWaitEvent(st, join, 0);
        else if (split) (void)hipStreamSynchronize(side);   // branch enqueued but not joined: finish it
        launch_sparse_compute_bf16(g, in->q, k_hist, v_hist, in->k_intra, in->v_intra, n_sel, sparse_ws, ep,
                                   st);
        if (fork) (void)hipEventDestroy(fork);
        if (join) (void)hipEventDestroy(join);
    } else {
        run_gather<float>(g, in->pool_k, in->pool_v, in->page_kmean, in->page_prompt, cur_prompt,
                          in->q, page_idx, n_sel, k_hist, v_hist, partial, kb, st);
        run_select<float>(g, in->q, k_hist, in->k_intra, n_sel, t, sel_count, sel_idx, nullptr,
                          nullptr, qb, kb, zl, true, st);
        run_linear<float>(g, in->q, k_hist, v_hist, in->k_intra, in->v_intra, n_sel, in->E,
                          in->F, o_linear, nullptr, nullptr, c, st);
        launch_sparse_attn<float>(g, in->q, k_hist, v_hist, in->k_intra, in->v_intra, n_sel,
                                  sel_count, sel_idx, sparse_ws, ep, st);
    }
    return c.ok ? done() : HSAKV_ERR_WORKSPACE;
}
