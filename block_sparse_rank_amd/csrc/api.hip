// Exported C ABI of libhsakv: host-side checks, workspace carving, launches.
// Declarations, argument meaning, layouts and error behaviour: include/hsakv.h.
#include "hsakv.h"

#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "common.h"
#include "launch.h"

#define HSAKV_API extern "C" __attribute__((visibility("default")))

int device_cu_count() {
    static std::atomic<int> cache[64];   // zero-initialised: not looked up yet
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = -1;
    if (dev >= 0) {
        const int c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev < 0 ? 0 : dev) != hipSuccess ||
        cus < 1)
        cus = 256;
    if (dev >= 0) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

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
    g.one_range = 0;
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
    if (d->Kp > kMaxKp || d->H > kMaxHeads || (long long)d->H * d->d > 16384) return HSAKV_ERR_UNSUPPORTED;
    const long long Tp = (long long)d->Psize * d->tokens_per_frame;
    if (Tp > (1LL << 30) || (long long)d->Kp * Tp + d->Lq >= (1LL << 31)) return HSAKV_ERR_BAD_DIMS;
    if (d->P > 65536) return HSAKV_ERR_UNSUPPORTED;
    Geo g = make_geo(d);
    if (g.NB_max > 4096) return HSAKV_ERR_UNSUPPORTED;
    // one-dimensional grids of (block, 256 columns) work-groups stay below 2^32 threads
    if ((long long)(g.NQB + g.NB_max) * ((g.HD + 255) / 256) * 256 >= (1LL << 32)) return HSAKV_ERR_UNSUPPORTED;
    if (retrieve_smem_bytes(g) > 65536) return HSAKV_ERR_UNSUPPORTED;
    // the projection kernels address E and F with 32-bit byte offsets
    if ((long long)d->r * g.L * g.elt >= (1LL << 31)) return HSAKV_ERR_UNSUPPORTED;
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


// ---- workspace sizes -------------------------------------------------------

size_t ws_gather(const Geo& g) { return align_up(retrieve_ws_bytes(g)); }

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

// Retrieval policy and seed (two-stage when the caller passes none).
struct Policy {
    int policy = HSAKV_POLICY_TWO_STAGE;
    unsigned long long seed = 0;
};

Policy policy_of(const hsakv_retrieval* r) {
    Policy p;
    if (r) {
        p.policy = r->policy;
        p.seed = r->seed;
    }
    return p;
}

int check_policy(const hsakv_retrieval* r) {
    if (r && (r->policy < HSAKV_POLICY_TWO_STAGE || r->policy > HSAKV_POLICY_MISMATCHED))
        return HSAKV_ERR_UNSUPPORTED;
    return HSAKV_OK;
}

Tiers tiers_of(const hsakv_tiers* t) {
    Tiers r{nullptr, nullptr, nullptr};
    if (t) {
        r.page_slot = t->page_slot;
        r.host_k = t->host_k;
        r.host_v = t->host_v;
    }
    return r;
}

int check_tiers(const hsakv_tiers* t) {
    if (!t) return HSAKV_OK;
    if (!t->page_slot || !t->host_k || !t->host_v) return HSAKV_ERR_NULL_ARG;
    if (!aligned(t->page_slot, 4) || !aligned(t->host_k) || !aligned(t->host_v)) return HSAKV_ERR_MISALIGNED;
    return HSAKV_OK;
}

template <typename T>
void run_gather(const Geo& g, const void* pool_k, const void* pool_v, const float* page_kmean,
                const int32_t* page_prompt, int cur_prompt, const Policy& pol, const Tiers& tiers, const void* q,
                int32_t* page_idx, int32_t* n_sel, void* k_hist, void* v_hist, void* retrieve_ws, float* kb,
                hipStream_t st) {
    launch_retrieve<T>(g, q, page_kmean, page_prompt, cur_prompt, pol.policy, pol.seed, retrieve_ws, page_idx,
                       n_sel, st);
    if (kb)   // the history blocks of the pooled keys come with the copy
        launch_gather_pool<T>(g, pool_k, pool_v, page_idx, n_sel, k_hist, v_hist, kb, tiers, st);
    else
        launch_gather(g, (int)sizeof(T), pool_k, pool_v, page_idx, n_sel, k_hist, v_hist, tiers, st);
}

template <typename T>
void run_select(const Geo& g, const void* q, const void* k_hist, const void* k_intra,
                const int32_t* n_sel, const TauArg& tau, int32_t* sel_count, int32_t* sel_idx,
                uint8_t* sel_mask, float* block_mass, float* qb, float* kb, float* zl, bool hist_pooled,
                hipStream_t st) {
    launch_pool<T>(g, q, k_hist, k_intra, n_sel, qb, kb, hist_pooled, st);
    launch_select(g, qb, kb, zl, n_sel, tau, sel_count, sel_idx, sel_mask, block_mass, st);
}

// Scratch of the low-rank branch: split partials, then K' and V' (bf16 hi + lo
// pairs, or float32).
struct LinBufs {
    float* part;
    void *khi, *vhi, *klo, *vlo;
};

LinBufs carve_linear(const Geo& g, int eb, Carver& c) {
    const size_t n = (size_t)g.r * g.HD;
    LinBufs b;
    b.part = (float*)c.take((size_t)lowrank_splits(g) * 2 * n * 4);
    b.klo = b.vlo = nullptr;
    if (eb == 2) {
        b.khi = c.take(n * 2); b.vhi = c.take(n * 2); b.klo = c.take(n * 2); b.vlo = c.take(n * 2);
    } else {
        b.khi = c.take(n * 4); b.vhi = c.take(n * 4);
    }
    return b;
}

template <typename T>
void run_linear(const Geo& g, const void* q, const void* k_hist, const void* v_hist,
                const void* k_intra, const void* v_intra, const int32_t* n_sel, const void* E,
                const void* F, float* o_linear, float* k_low, float* v_low, const LinBufs& b,
                hipStream_t st) {
    launch_lowrank_proj<T>(g, E, F, k_hist, v_hist, k_intra, v_intra, n_sel, b.part, st);
    launch_lowrank_reduce<T>(g, b.part, k_low, v_low, b.khi, b.vhi, b.klo, b.vlo, st);
    Epi ep{o_linear, nullptr, nullptr, nullptr, nullptr, nullptr};
    launch_lowrank_attn<T>(g, q, b.khi, b.vhi, b.klo, b.vlo, ep, st);
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
        case HSAKV_ERR_TOO_LARGE: return "scratch needed exceeds the static scratch of the allocation-free entry point";
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
        case HSAKV_ENTRY_SUMMARY: return align_up(page_means_ws_bytes(g, g.P));
        case HSAKV_ENTRY_COMMIT: return align_up(page_means_ws_bytes(g, g.Lq / g.Tp + 1));
        case HSAKV_ENTRY_BACKWARD: return align_up(backward_ws_bytes(g));
        case HSAKV_ENTRY_SPARSE_STATIC: {
            Geo g1 = g;
            g1.one_range = 1;
            return ws_sparse(g1);
        }
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
                               void* ws, size_t ws_bytes, void* stream) {
    HSAKV_CHECK(check_dims(dims));
    HSAKV_REQUIRE(pool_k && page_kmean, HSAKV_ERR_NULL_ARG);
    HSAKV_REQUIRE(aligned(pool_k) && aligned(page_kmean), HSAKV_ERR_MISALIGNED);
    const Geo g = make_geo(dims);
    HSAKV_CHECK(check_ws(ws, ws_bytes, page_means_ws_bytes(g, g.P)));
    hipStream_t st = (hipStream_t)stream;
    if (dims->dtype == HSAKV_BF16) launch_page_summary<bf16_t>(g, pool_k, page_kmean, (float*)ws, st);
    else launch_page_summary<float>(g, pool_k, page_kmean, (float*)ws, st);
    return done();
}

HSAKV_API int hkv_page_commit(const hsakv_dims* dims, void* pool_k, void* pool_v, float* page_kmean,
                              int32_t* page_prompt, const void* k_chunk, const void* v_chunk, int32_t n_tokens,
                              int64_t fill, int32_t cur_prompt, void* ws, size_t ws_bytes, void* stream) {
    HSAKV_CHECK(check_dims(dims));
    HSAKV_REQUIRE(pool_k && pool_v && page_kmean && page_prompt && (n_tokens == 0 || (k_chunk && v_chunk)),
                  HSAKV_ERR_NULL_ARG);
    HSAKV_REQUIRE(aligned(pool_k) && aligned(pool_v) && aligned(page_kmean) && aligned(page_prompt, 4) &&
                      aligned(k_chunk) && aligned(v_chunk),
                  HSAKV_ERR_MISALIGNED);
    const Geo g = make_geo(dims);
    HSAKV_REQUIRE(n_tokens >= 0 && fill >= 0 && fill + (long long)n_tokens <= (long long)g.P * g.Tp,
                  HSAKV_ERR_BAD_DIMS);
    if (n_tokens == 0) return HSAKV_OK;
    const int completes = (int)((fill + n_tokens) / g.Tp - fill / g.Tp);
    if (completes > 0) HSAKV_CHECK(check_ws(ws, ws_bytes, page_means_ws_bytes(g, completes)));
    hipStream_t st = (hipStream_t)stream;
    if (dims->dtype == HSAKV_BF16)
        launch_page_commit<bf16_t>(g, pool_k, pool_v, page_kmean, page_prompt, k_chunk, v_chunk, n_tokens, fill,
                                   cur_prompt, (float*)ws, st);
    else
        launch_page_commit<float>(g, pool_k, pool_v, page_kmean, page_prompt, k_chunk, v_chunk, n_tokens, fill,
                                  cur_prompt, (float*)ws, st);
    return done();
}

HSAKV_API int hkv_gather(const hsakv_dims* dims, const void* pool_k, const void* pool_v,
                         const float* page_kmean, const int32_t* page_prompt, int32_t cur_prompt,
                         const hsakv_retrieval* retrieval, const hsakv_tiers* tiers, const void* q,
                         int32_t* page_idx, int32_t* n_sel, void* k_hist, void* v_hist, void* ws,
                         size_t ws_bytes, void* stream) {
    HSAKV_CHECK(check_dims(dims));
    HSAKV_CHECK(check_policy(retrieval));
    HSAKV_CHECK(check_tiers(tiers));
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
        run_gather<bf16_t>(g, pool_k, pool_v, page_kmean, page_prompt, cur_prompt, policy_of(retrieval),
                           tiers_of(tiers), q, page_idx,
                           n_sel, k_hist, v_hist, ws, nullptr, st);
    else
        run_gather<float>(g, pool_k, pool_v, page_kmean, page_prompt, cur_prompt, policy_of(retrieval),
                          tiers_of(tiers), q, page_idx,
                          n_sel, k_hist, v_hist, ws, nullptr, st);
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
    if (!c.ok) return HSAKV_ERR_WORKSPACE;
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

HSAKV_API int hsa_sparse_plan(const hsakv_dims* dims, const int32_t* n_sel, const int32_t* sel_count,
                              const int32_t* sel_idx, void* ws, size_t ws_bytes, void* stream) {
    HSAKV_CHECK(check_dims(dims));
    HSAKV_REQUIRE(dims->dtype == HSAKV_BF16, HSAKV_ERR_BAD_DTYPE);
    HSAKV_REQUIRE(n_sel && sel_count && sel_idx, HSAKV_ERR_NULL_ARG);
    HSAKV_REQUIRE(aligned(n_sel, 4) && aligned(sel_count, 4) && aligned(sel_idx, 4), HSAKV_ERR_MISALIGNED);
    const Geo g = make_geo(dims);
    HSAKV_CHECK(check_ws(ws, ws_bytes, ws_sparse(g)));
    launch_sparse_plan_bf16(g, n_sel, sel_count, sel_idx, ws, (hipStream_t)stream);
    return done();
}

HSAKV_API int hsa_sparse_compute(const hsakv_dims* dims, const void* q, const void* k_hist,
                                 const void* v_hist, const void* k_intra, const void* v_intra,
                                 const int32_t* n_sel, float* o_sparse, void* ws, size_t ws_bytes,
                                 void* stream) {
    HSAKV_CHECK(check_dims(dims));
    HSAKV_REQUIRE(dims->dtype == HSAKV_BF16, HSAKV_ERR_BAD_DTYPE);
    HSAKV_REQUIRE(q && k_hist && v_hist && k_intra && v_intra && n_sel && o_sparse, HSAKV_ERR_NULL_ARG);
    HSAKV_REQUIRE(aligned(q) && aligned(k_hist) && aligned(v_hist) && aligned(k_intra) &&
                      aligned(v_intra) && aligned(o_sparse) && aligned(n_sel, 4),
                  HSAKV_ERR_MISALIGNED);
    const Geo g = make_geo(dims);
    HSAKV_CHECK(check_ws(ws, ws_bytes, ws_sparse(g)));
    Epi ep{o_sparse, nullptr, nullptr, nullptr, nullptr, nullptr};
    launch_sparse_compute_bf16(g, q, k_hist, v_hist, k_intra, v_intra, n_sel, ws, ep, (hipStream_t)stream);
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
    const LinBufs lb = carve_linear(g, eb, c);
    if (!c.ok) return HSAKV_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    if (eb == 2)
        run_linear<bf16_t>(g, q, k_hist, v_hist, k_intra, v_intra, n_sel, E, F, o_linear, k_low,
                           v_low, lb, st);
    else
        run_linear<float>(g, q, k_hist, v_hist, k_intra, v_intra, n_sel, E, F, o_linear, k_low,
                          v_low, lb, st);
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

HSAKV_API int hsakv_fork_create(hsakv_fork* f) {
    if (!f) return HSAKV_ERR_NULL_ARG;
    hipStream_t st = nullptr;
    hipEvent_t a = nullptr, b = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&st, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&a, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&b, hipEventDisableTiming);
    if (e != hipSuccess) {
        if (b) (void)hipEventDestroy(b);
        if (a) (void)hipEventDestroy(a);
        if (st) (void)hipStreamDestroy(st);
        g_last_hip_error = (int)e;
        return HSAKV_ERR_HIP;
    }
    f->stream = st;
    f->fork = a;
    f->join = b;
    return HSAKV_OK;
}

HSAKV_API int hsakv_fork_destroy(hsakv_fork* f) {
    if (!f) return HSAKV_ERR_NULL_ARG;
    hipError_t e = hipSuccess, x;
    if (f->join && (x = hipEventDestroy((hipEvent_t)f->join)) != hipSuccess) e = x;
    if (f->fork && (x = hipEventDestroy((hipEvent_t)f->fork)) != hipSuccess) e = x;
    if (f->stream && (x = hipStreamDestroy((hipStream_t)f->stream)) != hipSuccess) e = x;
    f->stream = f->fork = f->join = nullptr;
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return HSAKV_ERR_HIP;
    }
    return HSAKV_OK;
}

HSAKV_API int hsa_forward(const hsakv_dims* dims, const float* tau, int32_t cur_prompt,
                          const hsakv_retrieval* retrieval, const hsakv_tiers* tiers,
                          const hsakv_inputs* in, hsakv_outputs* out, void* ws, size_t ws_bytes,
                          void* stream, const hsakv_fork* fork) {
    HSAKV_CHECK(check_dims(dims));
    HSAKV_CHECK(check_policy(retrieval));
    HSAKV_CHECK(check_tiers(tiers));
    const Tiers tr = tiers_of(tiers);
    const Policy pol = policy_of(retrieval);
    HSAKV_REQUIRE(in && out, HSAKV_ERR_NULL_ARG);
    HSAKV_CHECK(check_tau(dims, tau));
    HSAKV_REQUIRE(in->q && in->k_intra && in->v_intra && in->pool_k && in->pool_v &&
                      in->page_kmean && in->page_prompt && in->E && in->F && in->w_g && in->b_g &&
                      out->out,
                  HSAKV_ERR_NULL_ARG);
    const bool split = fork && fork->stream;
    HSAKV_REQUIRE(!split || (fork->fork && fork->join), HSAKV_ERR_NULL_ARG);
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
    void* part = c.take(ws_gather(g));
    float* qb = (float*)c.take((size_t)g.H * g.NQB * g.d * 4);
    float* kb = (float*)c.take((size_t)g.H * g.NB_max * g.d * 4);
    float* zl = (float*)c.take((size_t)g.H * g.NQB * g.NB_max * 4);
    void* sparse_ws = c.take(ws_sparse(g));
    const LinBufs lb = carve_linear(g, eb, c);
    int32_t* page_idx = (int32_t*)c.take((size_t)g.Kp * 4);
    int32_t* n_sel = (int32_t*)c.take(4);
    void* k_hist = c.take((size_t)g.hist_rows * g.HD * eb);
    void* v_hist = c.take((size_t)g.hist_rows * g.HD * eb);
    int32_t* sel_count = (int32_t*)c.take((size_t)g.H * g.NQB * 4);
    int32_t* sel_idx = (int32_t*)c.take((size_t)g.H * g.NQB * g.NB_max * 4);
    float* o_linear = (float*)c.take((size_t)g.Lq * g.HD * 4);
    if (!c.ok) return HSAKV_ERR_WORKSPACE;   // every check is done before the first launch
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
        run_gather<bf16_t>(g, in->pool_k, in->pool_v, in->page_kmean, in->page_prompt, cur_prompt, pol, tr,
                           in->q, page_idx, n_sel, k_hist, v_hist, part, kb, st);
        // The low-rank branch needs the gathered KV only: with a fork it runs
        // on the caller's second stream beside the pooling, the block
        // selection and the sparse plan (small, latency-bound kernels), and
        // the attention waits for both.
        hipStream_t side = split ? (hipStream_t)fork->stream : st;
        if (split) {
            hipError_t e = hipEventRecord((hipEvent_t)fork->fork, st);
            if (e == hipSuccess) e = hipStreamWaitEvent(side, (hipEvent_t)fork->fork, 0);
            if (e != hipSuccess) {
                g_last_hip_error = (int)e;
                return HSAKV_ERR_HIP;
            }
        }
        run_linear<bf16_t>(g, in->q, k_hist, v_hist, in->k_intra, in->v_intra, n_sel, in->E,
                           in->F, o_linear, nullptr, nullptr, lb, side);
        if (split) {
            hipError_t e = hipEventRecord((hipEvent_t)fork->join, side);
            if (e != hipSuccess) {
                g_last_hip_error = (int)e;
                return HSAKV_ERR_HIP;
            }
        }
        run_select<bf16_t>(g, in->q, k_hist, in->k_intra, n_sel, t, sel_count, sel_idx, nullptr,
                           nullptr, qb, kb, zl, true, st);
        launch_sparse_plan_bf16(g, n_sel, sel_count, sel_idx, sparse_ws, st);
        if (split) {
            const hipError_t e = hipStreamWaitEvent(st, (hipEvent_t)fork->join, 0);
            if (e != hipSuccess) {
                g_last_hip_error = (int)e;
                return HSAKV_ERR_HIP;
            }
        }
        launch_sparse_compute_bf16(g, in->q, k_hist, v_hist, in->k_intra, in->v_intra, n_sel, sparse_ws, ep,
                                   st);
    } else {
        run_gather<float>(g, in->pool_k, in->pool_v, in->page_kmean, in->page_prompt, cur_prompt, pol, tr,
                          in->q, page_idx, n_sel, k_hist, v_hist, part, kb, st);
        run_select<float>(g, in->q, k_hist, in->k_intra, n_sel, t, sel_count, sel_idx, nullptr,
                          nullptr, qb, kb, zl, true, st);
        run_linear<float>(g, in->q, k_hist, v_hist, in->k_intra, in->v_intra, n_sel, in->E,
                          in->F, o_linear, nullptr, nullptr, lb, st);
        launch_sparse_attn<float>(g, in->q, k_hist, v_hist, in->k_intra, in->v_intra, n_sel,
                                  sel_count, sel_idx, sparse_ws, ep, st);
    }
    return done();
}

// ---- allocation-free variant of hsa_sparse_attn ----------------------------------
//
// Its scratch (the work plan and the split-group softmax partials) lives in a
// fixed device array of HSAKV_STATIC_SCRATCH_BYTES, one copy per GPU for the
// life of the process. Host code never passes the array's name to a kernel:
// the name is a host-side stand-in; the device address of each GPU's copy is
// looked up once per device and kept.

static __device__ __align__(256) unsigned char scratch[HSAKV_STATIC_SCRATCH_BYTES];

namespace {

// Device address of this device's `scratch`, looked up on the first call on
// the device (with that device current). nullptr with the HIP error recorded
// if the lookup fails.
void* static_scratch() {
    static std::mutex mu;
    static void* addr[64] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess || dev < 0 || dev >= 64) {
        g_last_hip_error = (int)(e != hipSuccess ? e : hipErrorInvalidDevice);
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            g_last_hip_error = (int)(e != hipSuccess ? e : hipErrorInvalidSymbol);
            return nullptr;
        }
        addr[dev] = p;
    }
    return addr[dev];
}

}  // namespace

HSAKV_API int hsa_sparse_attn_static(const hsakv_dims* dims, const void* q, const void* k_hist,
                                     const void* v_hist, const void* k_intra, const void* v_intra,
                                     const int32_t* n_sel, const int32_t* sel_count,
                                     const int32_t* sel_idx, float* o_sparse, void* stream) {
    HSAKV_CHECK(check_dims(dims));
    HSAKV_REQUIRE(q && k_hist && v_hist && k_intra && v_intra && n_sel && sel_count && sel_idx &&
                      o_sparse,
                  HSAKV_ERR_NULL_ARG);
    HSAKV_REQUIRE(aligned(q) && aligned(k_hist) && aligned(v_hist) && aligned(k_intra) &&
                      aligned(v_intra) && aligned(o_sparse) && aligned(n_sel, 4) &&
                      aligned(sel_count, 4) && aligned(sel_idx, 4),
                  HSAKV_ERR_MISALIGNED);
    // one split range per work-group: the partials of the several ranges per
    // work-group that hsa_sparse_attn runs for the largest heads would not fit
    Geo g = make_geo(dims);
    g.one_range = 1;
    if (ws_sparse(g) > (size_t)HSAKV_STATIC_SCRATCH_BYTES) return HSAKV_ERR_TOO_LARGE;
    void* ws = static_scratch();
    if (!ws) return HSAKV_ERR_HIP;
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

// ---- page tiers: HBM slots caching pages of a pinned host store ----------------

HSAKV_API int hsakv_host_alloc(size_t bytes, void** host_ptr, void** device_ptr) {
    if (!host_ptr || !device_ptr) return HSAKV_ERR_NULL_ARG;
    *host_ptr = *device_ptr = nullptr;
    void* h = nullptr;
    hipError_t e = hipHostMalloc(&h, bytes ? bytes : 1, hipHostMallocMapped);
    void* d = nullptr;
    if (e == hipSuccess) e = hipHostGetDevicePointer(&d, h, 0);
    if (e != hipSuccess) {
        if (h) (void)hipHostFree(h);
        g_last_hip_error = (int)e;
        return HSAKV_ERR_HIP;
    }
    *host_ptr = h;
    *device_ptr = d;
    return HSAKV_OK;
}

HSAKV_API int hsakv_host_free(void* host_ptr) {
    if (!host_ptr) return HSAKV_OK;
    const hipError_t e = hipHostFree(host_ptr);
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return HSAKV_ERR_HIP;
    }
    return HSAKV_OK;
}

HSAKV_API int hkv_tier_plan(int32_t P, int32_t slots, int32_t* slot_of_page, int32_t* page_of_slot,
                            int64_t* last_use, int64_t now, const int32_t* want, int32_t n_want,
                            int32_t* promote_page, int32_t* promote_slot, int32_t* n_promote,
                            int32_t* upd_page, int32_t* upd_value, int32_t* n_upd) {
    // with no slots there is no page_of_slot to pass, and nothing is promoted
    if (!slot_of_page || (slots > 0 && !page_of_slot) || !last_use || (n_want > 0 && !want) || !promote_page ||
        !promote_slot || !n_promote || !upd_page || !upd_value || !n_upd)
        return HSAKV_ERR_NULL_ARG;
    if (P < 1 || slots < 0 || n_want < 0) return HSAKV_ERR_BAD_DIMS;
    for (int i = 0; i < n_want; ++i)
        if (want[i] < 0 || want[i] >= P) return HSAKV_ERR_BAD_DIMS;
    // the wanted pages are the most recently used from now on
    for (int i = 0; i < n_want; ++i) last_use[want[i]] = now;
    int np = 0, nu = 0;
    for (int i = 0; i < n_want; ++i) {
        const int p = want[i];
        if (slot_of_page[p] >= 0) continue;
        // a free slot, else the slot of the least recently used page not wanted now
        int best = -1;
        long long best_use = 0;
        for (int s = 0; s < slots; ++s) {
            const int q = page_of_slot[s];
            if (q < 0) {
                best = s;
                break;
            }
            if (last_use[q] >= now) continue;
            if (best < 0 || last_use[q] < best_use) {
                best = s;
                best_use = last_use[q];
            }
        }
        if (best < 0) break;   // every slot holds a page wanted now
        const int victim = page_of_slot[best];
        if (victim >= 0) {
            slot_of_page[victim] = -1;
            upd_page[nu] = victim;
            upd_value[nu++] = -1;
        }
        slot_of_page[p] = best;
        page_of_slot[best] = p;
        upd_page[nu] = p;
        upd_value[nu++] = best;
        promote_page[np] = p;
        promote_slot[np++] = best;
    }
    *n_promote = np;
    *n_upd = nu;
    return HSAKV_OK;
}

HSAKV_API int hkv_tier_apply(const hsakv_dims* dims, const hsakv_tiers* tiers, void* pool_k, void* pool_v,
                             int32_t slots, const int32_t* promote_page, const int32_t* promote_slot,
                             int32_t n_promote, const int32_t* upd_page, const int32_t* upd_value,
                             int32_t n_upd, void* stream) {
    HSAKV_CHECK(check_dims(dims));
    HSAKV_REQUIRE(tiers && pool_k && pool_v, HSAKV_ERR_NULL_ARG);
    HSAKV_CHECK(check_tiers(tiers));
    HSAKV_REQUIRE(aligned(pool_k) && aligned(pool_v), HSAKV_ERR_MISALIGNED);
    HSAKV_REQUIRE(n_promote >= 0 && n_upd >= 0 && n_upd <= 256 && slots >= 0, HSAKV_ERR_BAD_DIMS);
    HSAKV_REQUIRE((n_promote == 0 || (promote_page && promote_slot)) && (n_upd == 0 || (upd_page && upd_value)),
                  HSAKV_ERR_NULL_ARG);
    const Geo g = make_geo(dims);
    for (int i = 0; i < n_promote; ++i)
        if (promote_page[i] < 0 || promote_page[i] >= g.P || promote_slot[i] < 0 || promote_slot[i] >= slots)
            return HSAKV_ERR_BAD_DIMS;
    for (int i = 0; i < n_upd; ++i)
        if (upd_page[i] < 0 || upd_page[i] >= g.P || upd_value[i] < -1 || upd_value[i] >= slots)
            return HSAKV_ERR_BAD_DIMS;
    hipStream_t st = (hipStream_t)stream;
    const size_t page_bytes = (size_t)g.Tp * g.HD * g.elt;
    for (int i = 0; i < n_promote; ++i) {
        const size_t src = (size_t)promote_page[i] * page_bytes, dst = (size_t)promote_slot[i] * page_bytes;
        hipError_t e = hipMemcpyAsync((char*)pool_k + dst, (const char*)tiers->host_k + src, page_bytes,
                                      hipMemcpyDefault, st);
        if (e == hipSuccess)
            e = hipMemcpyAsync((char*)pool_v + dst, (const char*)tiers->host_v + src, page_bytes, hipMemcpyDefault,
                               st);
        if (e != hipSuccess) {
            g_last_hip_error = (int)e;
            return HSAKV_ERR_HIP;
        }
    }
    if (n_upd > 0) launch_tier_table(tiers->page_slot, n_upd, upd_page, upd_value, st);
    return done();
}

// ---- backward of the learned parameters ------------------------------------------

HSAKV_API int hsa_backward_params(const hsakv_dims* dims, const void* q, const void* k_hist,
                                  const void* v_hist, const void* k_intra, const void* v_intra,
                                  const int32_t* n_sel, const float* w_g, const float* b_g,
                                  const float* k_low, const float* v_low, const float* o_sparse,
                                  const float* o_linear, const void* d_out, float* d_wg, float* d_bg,
                                  float* d_E, float* d_F, void* ws, size_t ws_bytes, void* stream,
                                  const hsakv_fork* fork) {
    HSAKV_CHECK(check_dims(dims));
    HSAKV_REQUIRE(dims->dtype == HSAKV_BF16, HSAKV_ERR_BAD_DTYPE);
    HSAKV_REQUIRE(q && k_hist && v_hist && k_intra && v_intra && n_sel && w_g && b_g && k_low && v_low &&
                      o_sparse && o_linear && d_out && d_wg && d_bg && d_E && d_F,
                  HSAKV_ERR_NULL_ARG);
    HSAKV_REQUIRE(aligned(q) && aligned(k_hist) && aligned(v_hist) && aligned(k_intra) && aligned(v_intra) &&
                      aligned(n_sel, 4) && aligned(w_g) && aligned(b_g, 4) && aligned(k_low) &&
                      aligned(v_low) && aligned(o_sparse) && aligned(o_linear) && aligned(d_out) &&
                      aligned(d_wg, 4) && aligned(d_bg, 4) && aligned(d_E) && aligned(d_F),
                  HSAKV_ERR_MISALIGNED);
    const bool split = fork && fork->stream;
    HSAKV_REQUIRE(!split || (fork->fork && fork->join), HSAKV_ERR_NULL_ARG);
    const Geo g = make_geo(dims);
    // the dE / dF kernel reads key rows through buffer resources of < 2^31 bytes
    HSAKV_REQUIRE(g.L * g.HD * 2 < (1LL << 31), HSAKV_ERR_UNSUPPORTED);
    HSAKV_CHECK(check_ws(ws, ws_bytes, backward_ws_bytes(g)));
    hipStream_t st = (hipStream_t)stream;
    const hipError_t e = launch_backward_params(
        g, q, k_hist, v_hist, k_intra, v_intra, n_sel, w_g, b_g, k_low, v_low, o_sparse, o_linear, d_out, d_wg,
        d_bg, d_E, d_F, ws, st, split ? (hipStream_t)fork->stream : st,
        split ? (hipEvent_t)fork->fork : nullptr, split ? (hipEvent_t)fork->join : nullptr);
    if (e != hipSuccess) {
        g_last_hip_error = (int)e;
        return HSAKV_ERR_HIP;
    }
    return done();
}
