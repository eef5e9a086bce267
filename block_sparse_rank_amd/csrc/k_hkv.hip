// HKV kernels: page summary, two-stage retrieval, active-cache gather.
//
// Pages: WorldAttention news summary (ai4snews), HKV paragraph (semantic
// pages of Psize frames, prompt-level then page-level retrieval of the
// top-Kp pages) and kernel paragraph (KV reorganisation and contiguous
// copies are the dominant cost).
#include "common.h"
#include "launch.h"

// ---------------------------------------------------------------------------
// Retrieval, step 1: partial column sums of q over token slabs (k_item_colsum,
// below).

int retrieve_slabs(const Geo& g) {
    int slabs = (g.Lq + 63) / 64;
    return slabs > 64 ? 64 : slabs;
}


// ---------------------------------------------------------------------------
// Retrieval, step 2: chunk-mean query, one column per thread, slab partials
// added in slab order.

__global__ void __launch_bounds__(256)
k_qbar(const float* __restrict__ partial, int slabs, int HD, float inv_Lq, float* __restrict__ qbar) {
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= HD) return;
    float v[64];
#pragma unroll
    for (int k = 0; k < 64; ++k) v[k] = k < slabs ? partial[(size_t)k * HD + c] : 0.f;
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 64; ++k) s += v[k];
    qbar[c] = s * inv_Lq;
}

// ---------------------------------------------------------------------------
// Retrieval, step 3 (one block of 1024 threads): page scores, prompt filter,
// top-Kp with ties to the lower page, slots ascending.

constexpr int kRetrieveThreads = 1024;

__global__ void __launch_bounds__(kRetrieveThreads)
k_retrieve(const float* __restrict__ qbar_g, int HD, int P, int Kp,
           const float* __restrict__ page_kmean, const int32_t* __restrict__ page_prompt,
           int cur_prompt, int32_t* __restrict__ page_idx, int32_t* __restrict__ n_sel) {
    extern __shared__ float smem[];
    float* qbar = smem;                       // [HD]
    float* score = smem + HD;                 // [P]
    int* cand = reinterpret_cast<int*>(score + P);      // [P] 1 if the page matches
    __shared__ int n_cand;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int nwaves = kRetrieveThreads / 64;

    for (int c = tid; c < HD; c += kRetrieveThreads) qbar[c] = qbar_g[c];
    if (tid == 0) n_cand = 0;
    __syncthreads();

    // page scores, one wave per page; lanes take columns lane, lane + 64, ...
    // in a fixed order (up to 24 independent loads in flight), then a fixed tree
    for (int p = wave; p < P; p += nwaves) {
        const bool match = page_prompt[p] == cur_prompt;
        float s = 0.f;
        if (match) {
            const float* km = page_kmean + (size_t)p * HD;
            int c = lane;
            for (; c + 23 * 64 < HD; c += 24 * 64) {   // 24 loads in flight (one pass at H d = 1536)
                float k24[24];
#pragma unroll
                for (int u = 0; u < 24; ++u) k24[u] = km[c + 64 * u];
#pragma unroll
                for (int u = 0; u < 24; ++u) s = fmaf(k24[u], qbar[c + 64 * u], s);
            }
            for (; c + 7 * 64 < HD; c += 8 * 64) {
                float k8[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) k8[u] = km[c + 64 * u];
#pragma unroll
                for (int u = 0; u < 8; ++u) s = fmaf(k8[u], qbar[c + 64 * u], s);
            }
            for (; c < HD; c += 64) s = fmaf(km[c], qbar[c], s);
            s = wave_sum(s);
        }
        if (lane == 0) {
            score[p] = s;
            cand[p] = match ? 1 : 0;
            if (match) atomicAdd(&n_cand, 1);
        }
    }
    __syncthreads();

    // rank of each candidate: better score, or equal score and lower index;
    // the Kp best are marked chosen (cand = 2; still nonzero for the others'
    // candidate test)
    for (int p = tid; p < P; p += kRetrieveThreads) {
        if (!cand[p]) continue;
        const float sp = score[p];
        int rank = 0;
        for (int o = 0; o < P && rank < Kp; ++o) {
            if (!cand[o] || o == p) continue;
            const float so = score[o];
            if (so > sp || (so == sp && o < p)) ++rank;
        }
        if (rank < Kp) cand[p] = 2;
    }
    __syncthreads();

    // slots in ascending page order: a chosen page's slot is the number of
    // chosen pages below it
    const int n = n_cand < Kp ? n_cand : Kp;
    for (int p = tid; p < P; p += kRetrieveThreads) {
        if (cand[p] != 2) continue;
        int slot = 0;
        for (int o = 0; o < p; ++o) slot += cand[o] == 2 ? 1 : 0;
        page_idx[slot] = p;
    }
    for (int k = n + tid; k < Kp; k += kRetrieveThreads) page_idx[k] = -1;
    if (tid == 0) *n_sel = n;
}

size_t retrieve_smem_bytes(const Geo& g) {
    return (size_t)g.HD * 4 + (size_t)g.P * 8;
}

void launch_retrieve(const Geo& g, const float* partial, const float* page_kmean,
                     const int32_t* page_prompt, int cur_prompt, int32_t* page_idx,
                     int32_t* n_sel, hipStream_t st) {
    // the chunk mean goes right after the slab partials in the workspace
    float* qbar = const_cast<float*>(partial) + (size_t)retrieve_slabs(g) * g.HD;
    hipLaunchKernelGGL(k_qbar, dim3((g.HD + 255) / 256), dim3(256), 0, st, partial,
                       retrieve_slabs(g), g.HD, 1.0f / (float)g.Lq, qbar);
    hipLaunchKernelGGL(k_retrieve, dim3(1), dim3(kRetrieveThreads), retrieve_smem_bytes(g), st,
                       (const float*)qbar, g.HD, g.P, g.Kp, page_kmean, page_prompt, cur_prompt,
                       page_idx, n_sel);
}

// ---------------------------------------------------------------------------
// Gather: slot s of the active cache <- pool page page_idx[s], for K and V.
// A pure HBM-to-HBM copy: 16-byte vectors, kGatherUnroll loads in flight per
// thread before the stores. blockIdx.y = slot, blockIdx.z = 0 for K, 1 for V.

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 8;

__global__ void __launch_bounds__(kGatherThreads)
k_gather(const u32x4* __restrict__ pool_k, const u32x4* __restrict__ pool_v,
         const int32_t* __restrict__ page_idx, const int32_t* __restrict__ n_sel,
         u32x4* __restrict__ k_hist, u32x4* __restrict__ v_hist, long long vec_per_page) {
    const int slot = blockIdx.y;
    if (slot >= *n_sel) return;
    const long long page = page_idx[slot];
    const u32x4* src = (blockIdx.z == 0 ? pool_k : pool_v) + page * vec_per_page;
    u32x4* dst = (blockIdx.z == 0 ? k_hist : v_hist) + (long long)slot * vec_per_page;
    const long long chunk = (long long)kGatherThreads * kGatherUnroll;
    for (long long base = (long long)blockIdx.x * chunk; base < vec_per_page;
         base += (long long)gridDim.x * chunk) {
        u32x4 v[kGatherUnroll];
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
            long long i = base + u * kGatherThreads + threadIdx.x;
            if (i < vec_per_page) v[u] = __builtin_nontemporal_load(src + i);
        }
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
            long long i = base + u * kGatherThreads + threadIdx.x;
            if (i < vec_per_page) dst[i] = v[u];
        }
    }
}

// ---------------------------------------------------------------------------
// Gather with the history K pooled on the way (the forward's variant): one
// work-group per (history block of Binter rows, 256 columns, K or V), the
// column slabs of a block adjacent in launch order so that the work-groups
// running together read whole rows. Rows are
// copied bit for bit; for K each thread also sums its 8 columns over the rows
// grp, grp + 8, ... of the block in row order, and the eight row groups are
// added in group order: the same float32 operations as the pooling of a
// gathered block, so both give the same pooled key.

template <typename T> struct Row8;
template <> struct Row8<bf16_t> {
    u32x4 a;
    HSAKV_DEV void load(const bf16_t* p) { a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)); }
    HSAKV_DEV void store(bf16_t* p) const { *reinterpret_cast<u32x4*>(p) = a; }
    HSAKV_DEV void add_to(float* acc) const {
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] += __uint_as_float(w[i] << 16);
            acc[2 * i + 1] += __uint_as_float(w[i] & 0xffff0000u);
        }
    }
};
template <> struct Row8<float> {
    u32x4 a, b;
    HSAKV_DEV void load(const float* p) {
        a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
        b = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 4));
    }
    HSAKV_DEV void store(float* p) const {
        reinterpret_cast<u32x4*>(p)[0] = a;
        reinterpret_cast<u32x4*>(p)[1] = b;
    }
    HSAKV_DEV void add_to(float* acc) const {
        acc[0] += __uint_as_float(a.x); acc[1] += __uint_as_float(a.y);
        acc[2] += __uint_as_float(a.z); acc[3] += __uint_as_float(a.w);
        acc[4] += __uint_as_float(b.x); acc[5] += __uint_as_float(b.y);
        acc[6] += __uint_as_float(b.z); acc[7] += __uint_as_float(b.w);
    }
};

template <typename T>
__global__ void __launch_bounds__(256)
k_gather_pool(Geo g, const T* __restrict__ pool_k, const T* __restrict__ pool_v,
              const int32_t* __restrict__ page_idx, const int32_t* __restrict__ n_sel_p,
              T* __restrict__ k_hist, T* __restrict__ v_hist, float* __restrict__ kb) {
    constexpr int kRows = sizeof(T) == 2 ? 16 : 8;   // rows in flight per thread
    const int n_sel = *n_sel_p;
    const int nslab = (g.HD + 255) / 256;
    const int b = blockIdx.x / nslab, slab = blockIdx.x - b * nslab;
    if (b >= hist_blocks(g, n_sel)) return;
    const bool is_k = blockIdx.y == 0;
    const long long Lh = (long long)n_sel * g.Tp;
    const long long t0 = (long long)b * g.Binter;
    const long long t1 = t0 + g.Binter < Lh ? t0 + g.Binter : Lh;
    const int lane = threadIdx.x & 31, grp = threadIdx.x >> 5;
    const int col0 = (slab * 32 + lane) * 8;
    const T* src = is_k ? pool_k : pool_v;
    T* dst = is_k ? k_hist : v_hist;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    // rows t, t + 8, ... of this thread's group, kRows loads in flight; row
    // tu of the active history is row srow(tu) of the pool
    auto copy_rows = [&](auto srow) __attribute__((always_inline)) {
        for (long long t = t0 + grp; t < t1; t += 8 * kRows) {
            Row8<T> v[kRows];
#pragma unroll
            for (int u = 0; u < kRows; ++u) {
                const long long tu = t + 8 * u;
                if (tu < t1) v[u].load(src + srow(tu) * g.HD + col0);
            }
#pragma unroll
            for (int u = 0; u < kRows; ++u) {
                const long long tu = t + 8 * u;
                if (tu < t1) {
                    v[u].store(dst + tu * g.HD + col0);
                    if (is_k) v[u].add_to(acc);
                }
            }
        }
    };
    if (col0 < g.HD) {
        const int slot0 = (int)(t0 / g.Tp);
        const long long first0 = (long long)slot0 * g.Tp;
        if (g.Binter <= g.Tp) {
            // the block touches the pages of slot0 and slot0 + 1 at most: both
            // looked up once, so no row load waits for a page lookup
            const long long pa = page_idx[slot0];
            const long long pb = slot0 + 1 < n_sel ? page_idx[slot0 + 1] : pa;
            copy_rows([&](long long tu) {
                const long long rel = tu - first0;
                return rel < g.Tp ? pa * g.Tp + rel : pb * g.Tp + (rel - g.Tp);
            });
        } else {
            // short pages: several per block, each row looks its page up
            copy_rows([&](long long tu) {
                const long long slot = tu / g.Tp;
                return (long long)page_idx[slot] * g.Tp + (tu - slot * g.Tp);
            });
        }
    }
    if (!is_k) return;
    __shared__ float part[8][32 * 8 + 4];
#pragma unroll
    for (int e = 0; e < 8; ++e) part[grp][lane * 8 + e] = acc[e];
    __syncthreads();
    const int c = slab * 256 + threadIdx.x;
    if (c < g.HD) {
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < 8; ++k) s += part[k][threadIdx.x];
        const int h = c / g.d, e = c % g.d;
        kb[((size_t)h * g.NB_max + b) * g.d + e] = s / (float)(t1 - t0);
    }
}

template <typename T>
void launch_gather_pool(const Geo& g, const void* pool_k, const void* pool_v, const int32_t* page_idx,
                        const int32_t* n_sel, void* k_hist, void* v_hist, float* kb, hipStream_t st) {
    dim3 grid((unsigned)((long long)g.NBh_max * ((g.HD + 255) / 256)), 2);
    hipLaunchKernelGGL(k_gather_pool<T>, grid, dim3(256), 0, st, g, (const T*)pool_k, (const T*)pool_v,
                       page_idx, n_sel, (T*)k_hist, (T*)v_hist, kb);
}
template void launch_gather_pool<float>(const Geo&, const void*, const void*, const int32_t*, const int32_t*,
                                        void*, void*, float*, hipStream_t);
template void launch_gather_pool<bf16_t>(const Geo&, const void*, const void*, const int32_t*, const int32_t*,
                                         void*, void*, float*, hipStream_t);

void launch_gather(const Geo& g, int elt_bytes, const void* pool_k, const void* pool_v,
                   const int32_t* page_idx, const int32_t* n_sel, void* k_hist, void* v_hist,
                   hipStream_t st) {
    long long vec = (long long)g.Tp * g.HD * elt_bytes / 16;
    long long chunk = (long long)kGatherThreads * kGatherUnroll;
    long long blocks = (vec + chunk - 1) / chunk;
    if (blocks > 4096) blocks = 4096;
    dim3 grid((unsigned)blocks, g.Kp, 2);
    hipLaunchKernelGGL(k_gather, grid, dim3(kGatherThreads), 0, st, (const u32x4*)pool_k,
                       (const u32x4*)pool_v, page_idx, n_sel, (u32x4*)k_hist, (u32x4*)v_hist, vec);
}

// Column sums of items of consecutive token rows: item i is rows
// [i n, min((i + 1) n, total)) of x, its sum (times `scale`) goes to out[i].
// Used for the page summary (items = pages, scale 1/Tp) and for the slab sums
// of the chunk-mean query. One work-group of 1024 threads per (item, 256
// columns): 32 column lanes of 8 elements x 32 row groups, 16 rows (bf16; 8
// for f32) in flight per thread as raw vectors. Each thread keeps a Kahan
// sum per column over its rows (in row order); the 32 group sums are added
// in group order, again with Kahan, so identical items give identical sums.
template <typename T>
__global__ void __launch_bounds__(1024)
k_item_colsum(const T* __restrict__ x, long long rows_per_item, long long total_rows, int HD, float scale,
              float* __restrict__ out) {
    const int lane = threadIdx.x & 31, grp = threadIdx.x >> 5;
    const int col0 = (blockIdx.y * 32 + lane) * 8;
    const long long item = blockIdx.x;
    const long long r0 = item * rows_per_item;
    const long long left = total_rows - r0;
    const int rows = (int)(left < rows_per_item ? left : rows_per_item);
    const T* base = x + r0 * HD + col0;
    Kahan acc[8];
    if (col0 < HD) {
        constexpr int kRows = sizeof(T) == 2 ? 16 : 8;
        for (int t = grp; t < rows; t += 32 * kRows) {
            Row8<T> v[kRows];
#pragma unroll
            for (int u = 0; u < kRows; ++u) {
                const int tu = t + 32 * u < rows ? t + 32 * u : t;
                v[u].load(base + (long long)tu * HD);
            }
#pragma unroll
            for (int u = 0; u < kRows; ++u)
                if (t + 32 * u < rows) {
                    float xv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                    v[u].add_to(xv);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e].add(xv[e]);
                }
        }
    }
    __shared__ float part[32][32 * 8 + 4];
#pragma unroll
    for (int e = 0; e < 8; ++e) part[grp][lane * 8 + e] = acc[e].s;
    __syncthreads();
    if (threadIdx.x < 256) {
        const int c = blockIdx.y * 256 + threadIdx.x;
        if (c < HD) {
            Kahan k;
            for (int q = 0; q < 32; ++q) k.add(part[q][threadIdx.x]);
            out[item * HD + c] = k.s * scale;
        }
    }
}

template <typename T>
void launch_page_summary(const Geo& g, const void* pool_k, float* page_kmean, hipStream_t st) {
    dim3 grid(g.P, (g.HD + 255) / 256);
    hipLaunchKernelGGL(k_item_colsum<T>, grid, dim3(1024), 0, st, (const T*)pool_k, (long long)g.Tp,
                       (long long)g.P * g.Tp, g.HD, 1.0f / (float)g.Tp, page_kmean);
}
template void launch_page_summary<float>(const Geo&, const void*, float*, hipStream_t);
template void launch_page_summary<bf16_t>(const Geo&, const void*, float*, hipStream_t);

template <typename T>
void launch_q_partials(const Geo& g, const void* q, float* partial, hipStream_t st) {
    const int slabs = retrieve_slabs(g);
    const int per = (g.Lq + slabs - 1) / slabs;
    dim3 grid(slabs, (g.HD + 255) / 256);
    hipLaunchKernelGGL(k_item_colsum<T>, grid, dim3(1024), 0, st, (const T*)q, (long long)per, (long long)g.Lq,
                       g.HD, 1.0f, partial);
}
template void launch_q_partials<float>(const Geo&, const void*, float*, hipStream_t);
template void launch_q_partials<bf16_t>(const Geo&, const void*, float*, hipStream_t);
