// HKV kernels: page summary, two-stage retrieval, active-cache gather.
//
// Pages: WorldAttention news summary (ai4snews), HKV paragraph (semantic
// pages of Psize frames, prompt-level then page-level retrieval of the
// top-Kp pages) and kernel paragraph (KV reorganisation and contiguous
// copies are the dominant cost).
#include "common.h"
#include "launch.h"

// ---------------------------------------------------------------------------
// Rows of 8 elements as one 16-byte (bf16) or two (f32) vector loads.

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

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

// ---------------------------------------------------------------------------
// Retrieval, step 1 (k_slab_scores): the chunk's query sums and the terms of
// the page scores. Work-group (slab s, 256 columns g) sums those columns of q
// over the slab's rows in float64, writes the sums (colsum[s][c], kept for
// step 2's exact path) and, for every page, the float64 dot product of the
// sums with the page-mean key over the 256 columns: part[p][s G + g]. A page's
// parts add up to Lq <page-mean key, chunk-mean query>, all H d columns.

constexpr int kSlabs = 32;            // row slabs of q (and of a page, for the page means)
constexpr int kQsumGroups = 16;       // row groups per work-group

int retrieve_parts(const Geo& g) { return kSlabs * ((g.HD + 255) / 256); }

// Rows r0 + grp, r0 + grp + 16, ... of the slab in order per thread (16 rows
// in flight for bf16, 8 for f32), the 16 row groups added in group order.
// The page terms: thread (page t / 16 of a pass of 32 pages, chunk t % 16)
// takes the 16 columns of its chunk in order, and a page's 16 chunk sums are
// added in chunk order.
constexpr int kChunks = 16;                                  // 16-column chunks of the 256 columns
constexpr int kPagesPerPass = 32 * kQsumGroups / kChunks;    // 32

template <typename T>
__global__ void __launch_bounds__(32 * kQsumGroups)
k_slab_scores(const T* __restrict__ q, int Lq, int HD, int P, const float* __restrict__ page_kmean,
              double* __restrict__ colsum, double* __restrict__ part) {
    const int tid = threadIdx.x, lane = tid & 31, grp = tid >> 5;
    const int slab = blockIdx.x, cg = blockIdx.y, G = gridDim.y;
    const int col0 = (cg * 32 + lane) * 8;
    const int ncol = HD - cg * 256 < 256 ? HD - cg * 256 : 256;   // a multiple of 64 (H d is one of 64)
    const int pp = tid / kChunks, ch = tid % kChunks;
    const bool ch_ok = kChunks * ch < ncol;
    // the first pass's page means do not depend on q: loaded first (addresses
    // clamped into the array, values of absent pages or chunks unused)
    auto load_means = [&](int p, float4 (&kf)[4]) __attribute__((always_inline)) {
        const int pc = p < P ? p : P - 1;
        const float4* src =
            reinterpret_cast<const float4*>(page_kmean + (size_t)pc * HD + cg * 256 + (ch_ok ? kChunks * ch : 0));
#pragma unroll
        for (int i = 0; i < 4; ++i) kf[i] = src[i];
    };
    float4 kf[4];
    load_means(pp, kf);
    const int per = (Lq + kSlabs - 1) / kSlabs;
    const int r0 = slab * per, r1 = r0 + per < Lq ? r0 + per : Lq;
    double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (col0 < HD) {
        constexpr int kRows = sizeof(T) == 2 ? 16 : 8;
        for (int t = r0 + grp; t < r1; t += kQsumGroups * kRows) {
            Row8<T> v[kRows];
#pragma unroll
            for (int u = 0; u < kRows; ++u)
                if (t + kQsumGroups * u < r1) v[u].load(q + (size_t)(t + kQsumGroups * u) * HD + col0);
#pragma unroll
            for (int u = 0; u < kRows; ++u)
                if (t + kQsumGroups * u < r1) {
                    float x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                    v[u].add_to(x);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] += (double)x[e];
                }
        }
    }
    __shared__ double gs[kQsumGroups][256];
    __shared__ double cs[256];
    __shared__ double pd[kPagesPerPass][kChunks + 1];
#pragma unroll
    for (int e = 0; e < 8; ++e) gs[grp][lane * 8 + e] = acc[e];
    __syncthreads();
    if (tid < ncol) {
        double a = 0.0;
#pragma unroll
        for (int g2 = 0; g2 < kQsumGroups; ++g2) a += gs[g2][tid];
        cs[tid] = a;
        colsum[(size_t)slab * HD + cg * 256 + tid] = a;
    }
    __syncthreads();
    for (int p0 = 0; p0 < P; p0 += kPagesPerPass) {
        if (p0 > 0) load_means(p0 + pp, kf);
        double d = 0.0;
        if (ch_ok) {
            const double* c = cs + kChunks * ch;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                d = fma((double)kf[i].x, c[4 * i], d);
                d = fma((double)kf[i].y, c[4 * i + 1], d);
                d = fma((double)kf[i].z, c[4 * i + 2], d);
                d = fma((double)kf[i].w, c[4 * i + 3], d);
            }
        }
        pd[pp][ch] = d;
        __syncthreads();
        if (tid < kPagesPerPass && p0 + tid < P) {
            double a = 0.0;
#pragma unroll
            for (int c = 0; c < kChunks; ++c) a += pd[tid][c];
            part[(size_t)(p0 + tid) * G * kSlabs + slab * G + cg] = a;
        }
        __syncthreads();
    }
}

template <typename T>
void launch_slab_scores(const Geo& g, const void* q, const float* page_kmean, double* colsum, double* part,
                        hipStream_t st) {
    const dim3 grid(kSlabs, (g.HD + 255) / 256);
    hipLaunchKernelGGL(k_slab_scores<T>, grid, dim3(32 * kQsumGroups), 0, st, (const T*)q, g.Lq, g.HD, g.P,
                       page_kmean, colsum, part);
}
template void launch_slab_scores<float>(const Geo&, const void*, const float*, double*, double*, hipStream_t);
template void launch_slab_scores<bf16_t>(const Geo&, const void*, const float*, double*, double*, hipStream_t);

// ---------------------------------------------------------------------------
// Retrieval, step 2: scores, prompt filter, top-Kp with ties to the lower
// page, slots in ascending page order.

constexpr int kRetrieveThreads = 1024;

// Output i of SplitMix64 seeded with `seed` (Steele, Lea and Flood, OOPSLA
// 2014): the state after i + 1 steps, then the generator's output mix.
HSAKV_DEV uint64_t splitmix64_at(uint64_t seed, uint64_t i) {
    uint64_t z = seed + (i + 1) * 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Candidate test and ranking key of each policy (HSAKV_POLICY_*): the
// method's two-stage retrieval scores the prompt-matching pages; the
// alternatives the pages compare it with change the candidates and the key.
HSAKV_DEV bool policy_candidate(int policy, int prompt, int cur) {
    switch (policy) {
        case 0: case 2: return prompt == cur;   // two-stage, prompt-only
        case 5: return prompt != cur;           // mismatched
        default: return true;                   // page-only, recent, random
    }
}
HSAKV_DEV bool policy_by_score(int policy) { return policy == 0 || policy == 1 || policy == 5; }

// Step 2, one work-group (k_retrieve):
// - a page's score is its parts added in float64 (segments of kSegParts
//   parts in order, then the segments in order), divided by Lq and rounded
//   to float32, the precision the ranking is decided in. A sum that is not
//   finite means a NaN or an infinity among the page mean or the queries;
//   such a page's score is then taken from the terms kbar[c] qbar[c] of the
//   exact dot product (qbar from the slab sums), whose value is then +inf,
//   -inf or NaN whatever the order of the sum. A score that is not a number
//   ranks below every number, as -inf;
// - the other policies' keys (page index, or SplitMix64 output p >> 40) are
//   exact in float32;
// - a candidate's rank counts the candidates with a better key, or an equal
//   key and a lower index; the Kp best are chosen, and a chosen page's slot
//   is the number of chosen pages below it.
constexpr int kSegParts = 8;

__global__ void __launch_bounds__(kRetrieveThreads)
k_retrieve(const double* __restrict__ part, const double* __restrict__ colsum, const float* __restrict__ page_kmean,
           int HD, int Lq, int P, int Kp, const int32_t* __restrict__ page_prompt, int cur_prompt, int policy,
           unsigned long long seed, int32_t* __restrict__ page_idx, int32_t* __restrict__ n_sel) {
    constexpr int NT = kRetrieveThreads, NWV = NT / 64;
    extern __shared__ float smem[];   // key[P], cand[P]
    float* key = smem;
    int* cand = reinterpret_cast<int*>(smem + P);
    __shared__ double seg[NT];
    __shared__ double psum[NT];
    __shared__ int wave_cnt[2 * NWV];
    __shared__ int slot_page[kMaxKp];
    __shared__ int flags;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool by_score = policy_by_score(policy);
    // thread t adds segment t % nseg of page p0 + t / nseg (NG is a multiple
    // of 32, so segments are whole); the first chunk's loads go out first
    const int NG = kSlabs * ((HD + 255) / 256);
    const int nseg = NG / kSegParts;   // at most 256
    const int ppc = NT / nseg;
    auto load_seg = [&](int p0, double (&v)[kSegParts]) __attribute__((always_inline)) {
        const int p = p0 + tid / nseg;
        const bool ok = tid < ppc * nseg && p < P;   // else a valid address, value unused
        const double* src = part + (size_t)(ok ? p : 0) * NG + (ok ? tid % nseg : 0) * kSegParts;
#pragma unroll
        for (int i = 0; i < kSegParts; ++i) v[i] = src[i];
    };
    double v[kSegParts];
    if (by_score) load_seg(0, v);
    for (int p = tid; p < P; p += NT) {
        const bool m = policy_candidate(policy, page_prompt[p], cur_prompt);
        cand[p] = m ? 1 : 0;
        if (!by_score) key[p] = m ? (policy == 4 ? (float)(splitmix64_at(seed, p) >> 40) : (float)p) : 0.f;
    }
    if (by_score) {
        for (int p0 = 0; p0 < P; p0 += ppc) {
            if (p0 > 0) load_seg(p0, v);
            if (tid < ppc * nseg && p0 + tid / nseg < P) {
                double a = 0.0;
#pragma unroll
                for (int i = 0; i < kSegParts; ++i) a += v[i];
                seg[tid] = a;
            }
            __syncthreads();
            bool bad = false;
            if (tid < ppc && p0 + tid < P) {
                double a = 0.0;
#pragma unroll 8
                for (int s2 = 0; s2 < nseg; ++s2) a += seg[tid * nseg + s2];
                const float f = (float)(a / (double)Lq);
                key[p0 + tid] = __builtin_isnan(f) ? -INFINITY : f;
                psum[tid] = a;
                bad = !__builtin_isfinite(a);
            }
            if (!__syncthreads_or(bad)) continue;
            // the pages of this chunk whose sum is not finite, one at a time by the work-group
            for (int i = 0; i < ppc && p0 + i < P; ++i) {
                if (__builtin_isfinite(psum[i])) continue;   // uniform: every thread reads the same word
                const int pg = p0 + i;
                if (tid == 0) flags = 0;
                __syncthreads();
                int f = 0;   // bit 0: a NaN term, bit 1: +inf, bit 2: -inf
                for (int c = tid; c < HD; c += NT) {
                    double qs = 0.0;
                    for (int sl = 0; sl < kSlabs; ++sl) qs += colsum[(size_t)sl * HD + c];
                    const double t = (double)page_kmean[(size_t)pg * HD + c] * (qs / (double)Lq);
                    f |= __builtin_isnan(t) ? 1 : __builtin_isinf(t) ? (t > 0 ? 2 : 4) : 0;
                }
                if (f) atomicOr(&flags, f);
                __syncthreads();
                if (tid == 0) {
                    const int fl = flags;
                    key[pg] = (fl & 1) || (fl & 6) == 6 ? -INFINITY : (fl & 2) ? INFINITY : -INFINITY;
                }
                __syncthreads();
            }
        }
    } else {
        __syncthreads();
    }
    // rank and slot: each thread compares its page with every other, eight at
    // a time (no early exit, so a group's LDS reads are in flight together);
    // the slot is the ballot prefix within the pass plus the passes before
    int carry = 0, ncand = 0;
    for (int base = 0; base < P; base += NT) {
        const int p = base + tid;
        const bool is_c = p < P && cand[p] != 0;
        bool pick = false;
        if (is_c) {
            const float kp = key[p];
            int rank = 0;
#pragma unroll 8
            for (int o = 0; o < P; ++o) {
                const float ko = key[o];
                rank += (cand[o] != 0 && (ko > kp || (ko == kp && o < p))) ? 1 : 0;
            }
            pick = rank < Kp;
        }
        const unsigned long long bp = __builtin_amdgcn_ballot_w64(pick);
        const unsigned long long bc = __builtin_amdgcn_ballot_w64(is_c);
        if (lane == 0) {
            wave_cnt[2 * wave] = __builtin_popcountll(bp);
            wave_cnt[2 * wave + 1] = __builtin_popcountll(bc);
        }
        __syncthreads();
        int below = 0, tp = 0, tc = 0;
#pragma unroll
        for (int v = 0; v < NWV; ++v) {
            below += v < wave ? wave_cnt[2 * v] : 0;
            tp += wave_cnt[2 * v];
            tc += wave_cnt[2 * v + 1];
        }
        if (pick) slot_page[carry + below + __builtin_popcountll(bp & ((1ull << lane) - 1ull))] = p;
        carry += tp;
        ncand += tc;
        __syncthreads();   // wave_cnt is rewritten by the next pass; slot_page is complete after the last
    }
    const int n = ncand < Kp ? ncand : Kp;
    for (int k = tid; k < Kp; k += NT) page_idx[k] = k < n ? slot_page[k] : -1;
    if (tid == 0) *n_sel = n;
}

size_t retrieve_smem_bytes(const Geo& g) { return (size_t)g.P * 8; }

// part[P][retrieve_parts] then, 256-byte aligned, colsum[kSlabs][HD], both float64
size_t retrieve_part_bytes(const Geo& g) { return ((size_t)g.P * retrieve_parts(g) * 8 + 255) / 256 * 256; }
size_t retrieve_ws_bytes(const Geo& g) { return retrieve_part_bytes(g) + (size_t)kSlabs * g.HD * 8; }

template <typename T>
void launch_retrieve(const Geo& g, const void* q, const float* page_kmean, const int32_t* page_prompt,
                     int cur_prompt, int policy, unsigned long long seed, void* ws, int32_t* page_idx,
                     int32_t* n_sel, hipStream_t st) {
    double* part = (double*)ws;
    double* colsum = (double*)((char*)ws + retrieve_part_bytes(g));
    if (policy == 0 || policy == 1 || policy == 5) launch_slab_scores<T>(g, q, page_kmean, colsum, part, st);
    hipLaunchKernelGGL(k_retrieve, dim3(1), dim3(kRetrieveThreads), retrieve_smem_bytes(g), st, part, colsum,
                       page_kmean, g.HD, g.Lq, g.P, g.Kp, page_prompt, cur_prompt, policy, seed, page_idx, n_sel);
}
template void launch_retrieve<float>(const Geo&, const void*, const float*, const int32_t*, int, int,
                                     unsigned long long, void*, int32_t*, int32_t*, hipStream_t);
template void launch_retrieve<bf16_t>(const Geo&, const void*, const float*, const int32_t*, int, int,
                                      unsigned long long, void*, int32_t*, int32_t*, hipStream_t);

// ---------------------------------------------------------------------------
// Gather: slot s of the active cache <- pool page page_idx[s], for K and V.
// A pure HBM-to-HBM copy: 16-byte vectors, kGatherUnroll loads in flight per
// thread before the stores. blockIdx.y = slot, blockIdx.z = 0 for K, 1 for V.

constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 8;

// First element of page `page` (K or V) in its tier: HBM pool slot or host store.
template <typename E>
HSAKV_DEV const E* page_base(const E* pool, const Tiers& t, bool is_k, long long page, long long per_page) {
    if (!t.page_slot) return pool + page * per_page;
    const int slot = t.page_slot[page];
    if (slot >= 0) return pool + (long long)slot * per_page;
    return (const E*)(is_k ? t.host_k : t.host_v) + page * per_page;
}

__global__ void __launch_bounds__(kGatherThreads)
k_gather(const u32x4* __restrict__ pool_k, const u32x4* __restrict__ pool_v,
         const int32_t* __restrict__ page_idx, const int32_t* __restrict__ n_sel,
         u32x4* __restrict__ k_hist, u32x4* __restrict__ v_hist, long long vec_per_page, Tiers tiers) {
    const int slot = blockIdx.y;
    if (slot >= *n_sel) return;
    const long long page = page_idx[slot];
    const bool is_k = blockIdx.z == 0;
    const u32x4* src = page_base(is_k ? pool_k : pool_v, tiers, is_k, page, vec_per_page);
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

template <typename T>
__global__ void __launch_bounds__(256)
k_gather_pool(Geo g, const T* __restrict__ pool_k, const T* __restrict__ pool_v,
              const int32_t* __restrict__ page_idx, const int32_t* __restrict__ n_sel_p,
              T* __restrict__ k_hist, T* __restrict__ v_hist, float* __restrict__ kb, Tiers tiers) {
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
    // tu of the active history starts at srow(tu)
    auto copy_rows = [&](auto srow) __attribute__((always_inline)) {
        for (long long t = t0 + grp; t < t1; t += 8 * kRows) {
            Row8<T> v[kRows];
#pragma unroll
            for (int u = 0; u < kRows; ++u) {
                const long long tu = t + 8 * u;
                if (tu < t1) v[u].load(srow(tu) + col0);
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
        const long long per_page = (long long)g.Tp * g.HD;
        if (g.Binter <= g.Tp) {
            // the block touches the pages of slot0 and slot0 + 1 at most: both
            // looked up once, so no row load waits for a page lookup
            const long long pa = page_idx[slot0];
            const long long pb = slot0 + 1 < n_sel ? page_idx[slot0 + 1] : pa;
            const T* ba = page_base(src, tiers, is_k, pa, per_page);
            const T* bb = page_base(src, tiers, is_k, pb, per_page);
            copy_rows([&](long long tu) {
                const long long rel = tu - first0;
                return rel < g.Tp ? ba + rel * g.HD : bb + (rel - g.Tp) * g.HD;
            });
        } else {
            // short pages: several per block, each row looks its page up
            copy_rows([&](long long tu) {
                const long long slot = tu / g.Tp;
                return page_base(src, tiers, is_k, (long long)page_idx[slot], per_page) +
                       (tu - slot * g.Tp) * g.HD;
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
                        const int32_t* n_sel, void* k_hist, void* v_hist, float* kb, const Tiers& tiers,
                        hipStream_t st) {
    dim3 grid((unsigned)((long long)g.NBh_max * ((g.HD + 255) / 256)), 2);
    hipLaunchKernelGGL(k_gather_pool<T>, grid, dim3(256), 0, st, g, (const T*)pool_k, (const T*)pool_v,
                       page_idx, n_sel, (T*)k_hist, (T*)v_hist, kb, tiers);
}
template void launch_gather_pool<float>(const Geo&, const void*, const void*, const int32_t*, const int32_t*,
                                        void*, void*, float*, const Tiers&, hipStream_t);
template void launch_gather_pool<bf16_t>(const Geo&, const void*, const void*, const int32_t*, const int32_t*,
                                         void*, void*, float*, const Tiers&, hipStream_t);

void launch_gather(const Geo& g, int elt_bytes, const void* pool_k, const void* pool_v,
                   const int32_t* page_idx, const int32_t* n_sel, void* k_hist, void* v_hist,
                   const Tiers& tiers, hipStream_t st) {
    long long vec = (long long)g.Tp * g.HD * elt_bytes / 16;
    long long chunk = (long long)kGatherThreads * kGatherUnroll;
    long long blocks = (vec + chunk - 1) / chunk;
    if (blocks > 4096) blocks = 4096;
    dim3 grid((unsigned)blocks, g.Kp, 2);
    hipLaunchKernelGGL(k_gather, grid, dim3(kGatherThreads), 0, st, (const u32x4*)pool_k,
                       (const u32x4*)pool_v, page_idx, n_sel, (u32x4*)k_hist, (u32x4*)v_hist, vec, tiers);
}

// Page means in two deterministic passes, so a page's mean does not depend on
// which call computes it (the pool summary or the commit that completes the
// page) and a single page still spreads over many work-groups:
//  1. k_slab_colsum: item i (a page) is cut into kSlabs slabs of rows; the
//     column sums of each slab go to partial[i][slab][HD];
//  2. k_slab_mean: per item and column, the slab sums added in slab order
//     (Kahan), times 1/rows.

// Slab column sums of `items` consecutive items of item_rows rows each:
// work-group (item * kSlabs + slab, 256 columns) of 512 threads, 32 column
// lanes of 8 elements x 16 row groups, 16 rows (bf16; 8 for f32) in flight
// per thread. Each thread keeps a Kahan sum per column over its rows in row
// order; the 16 group sums are added in group order (Kahan).

template <typename T>
__global__ void __launch_bounds__(32 * kQsumGroups)
k_slab_colsum(const T* __restrict__ x, long long item_rows, int HD, float* __restrict__ partial) {
    const int lane = threadIdx.x & 31, grp = threadIdx.x >> 5;
    const int col0 = (blockIdx.y * 32 + lane) * 8;
    const long long item = blockIdx.x / kSlabs;
    const int slab = blockIdx.x % kSlabs;
    const long long per = (item_rows + kSlabs - 1) / kSlabs;
    const long long r0 = item * item_rows + slab * per;
    const long long end = (item + 1) * item_rows;
    const long long r1 = r0 + per < end ? r0 + per : end;
    Kahan acc[8];
    if (col0 < HD) {
        constexpr int kRows = sizeof(T) == 2 ? 16 : 8;
        for (long long t = r0 + grp; t < r1; t += kQsumGroups * kRows) {
            Row8<T> v[kRows];
#pragma unroll
            for (int u = 0; u < kRows; ++u)
                if (t + kQsumGroups * u < r1) v[u].load(x + (t + kQsumGroups * u) * HD + col0);
#pragma unroll
            for (int u = 0; u < kRows; ++u)
                if (t + kQsumGroups * u < r1) {
                    float xv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
                    v[u].add_to(xv);
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e].add(xv[e]);
                }
        }
    }
    __shared__ float part[kQsumGroups][32 * 8 + 4];
#pragma unroll
    for (int e = 0; e < 8; ++e) part[grp][lane * 8 + e] = acc[e].s;
    __syncthreads();
    const int c = blockIdx.y * 256 + threadIdx.x;
    if (threadIdx.x < 256 && c < HD) {
        Kahan k;
#pragma unroll
        for (int g2 = 0; g2 < kQsumGroups; ++g2) k.add(part[g2][threadIdx.x]);
        partial[(size_t)blockIdx.x * HD + c] = k.s;
    }
}

// out[item][c] = (sum over slabs, in slab order, of partial[item][slab][c]) * scale
__global__ void __launch_bounds__(256)
k_slab_mean(const float* __restrict__ partial, int HD, float scale, float* __restrict__ out) {
    const int c = blockIdx.y * 256 + threadIdx.x;
    if (c >= HD) return;
    const long long item = blockIdx.x;
    float v[kSlabs];
#pragma unroll
    for (int k = 0; k < kSlabs; ++k) v[k] = partial[(size_t)(item * kSlabs + k) * HD + c];
    Kahan s;
#pragma unroll
    for (int k = 0; k < kSlabs; ++k) s.add(v[k]);
    out[item * HD + c] = s.s * scale;
}

// Page means of `count` pages starting at `pages` into page_kmean rows
// starting at `kmean`; partial holds count * kSlabs * HD floats.
template <typename T>
void launch_page_means(const Geo& g, const T* pages, int count, float* kmean, float* partial, hipStream_t st) {
    dim3 g1((unsigned)count * kSlabs, (g.HD + 255) / 256);
    hipLaunchKernelGGL(k_slab_colsum<T>, g1, dim3(32 * kQsumGroups), 0, st, pages, (long long)g.Tp, g.HD, partial);
    dim3 g2((unsigned)count, (g.HD + 255) / 256);
    hipLaunchKernelGGL(k_slab_mean, g2, dim3(256), 0, st, (const float*)partial, g.HD, 1.0f / (float)g.Tp, kmean);
}

size_t page_means_ws_bytes(const Geo& g, int pages) { return (size_t)pages * kSlabs * g.HD * 4; }

template <typename T>
void launch_page_summary(const Geo& g, const void* pool_k, float* page_kmean, float* partial, hipStream_t st) {
    launch_page_means<T>(g, (const T*)pool_k, g.P, page_kmean, partial, st);
}
template void launch_page_summary<float>(const Geo&, const void*, float*, float*, hipStream_t);
template void launch_page_summary<bf16_t>(const Geo&, const void*, float*, float*, hipStream_t);


// ---------------------------------------------------------------------------
// Page commit: the chunk's K and V rows become history tokens [fill, fill + n)
// of the pool (pages are consecutive in the pool, so that is one contiguous
// row range), then each page the commit completes gets its page-mean key
// (the page summary kernel, per page) and the committing prompt's id.

__global__ void __launch_bounds__(kGatherThreads)
k_commit_copy(const u32x4* __restrict__ k_chunk, const u32x4* __restrict__ v_chunk, u32x4* __restrict__ pool_k,
              u32x4* __restrict__ pool_v, long long vec, long long dst_off) {
    const u32x4* src = blockIdx.y == 0 ? k_chunk : v_chunk;
    u32x4* dst = (blockIdx.y == 0 ? pool_k : pool_v) + dst_off;
    const long long chunk = (long long)kGatherThreads * kGatherUnroll;
    for (long long base = (long long)blockIdx.x * chunk; base < vec; base += (long long)gridDim.x * chunk) {
        u32x4 v[kGatherUnroll];
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
            const long long i = base + u * kGatherThreads + threadIdx.x;
            if (i < vec) v[u] = __builtin_nontemporal_load(src + i);
        }
#pragma unroll
        for (int u = 0; u < kGatherUnroll; ++u) {
            const long long i = base + u * kGatherThreads + threadIdx.x;
            if (i < vec) dst[i] = v[u];
        }
    }
}

__global__ void k_tag_pages(int32_t* __restrict__ page_prompt, int first, int count, int32_t tag) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) page_prompt[first + i] = tag;
}

template <typename T>
void launch_page_commit(const Geo& g, void* pool_k, void* pool_v, float* page_kmean, int32_t* page_prompt,
                        const void* k_chunk, const void* v_chunk, int n, long long fill, int cur_prompt,
                        float* partial, hipStream_t st) {
    const long long vec = (long long)n * g.HD * (long long)sizeof(T) / 16;
    const long long chunk = (long long)kGatherThreads * kGatherUnroll;
    long long blocks = (vec + chunk - 1) / chunk;
    if (blocks > 4096) blocks = 4096;
    if (blocks > 0)
        hipLaunchKernelGGL(k_commit_copy, dim3((unsigned)blocks, 2), dim3(kGatherThreads), 0, st,
                           (const u32x4*)k_chunk, (const u32x4*)v_chunk, (u32x4*)pool_k, (u32x4*)pool_v, vec,
                           fill * g.HD * (long long)sizeof(T) / 16);
    // pages p with fill < (p + 1) Tp <= fill + n
    const long long first = fill / g.Tp, last = (fill + n) / g.Tp;   // [first, last)
    const int count = (int)(last - first);
    if (count > 0) {
        const T* pages = (const T*)pool_k + first * (long long)g.Tp * g.HD;
        launch_page_means<T>(g, pages, count, page_kmean + first * g.HD, partial, st);
        hipLaunchKernelGGL(k_tag_pages, dim3((count + 255) / 256), dim3(256), 0, st, page_prompt, (int)first, count,
                           (int32_t)cur_prompt);
    }
}
template void launch_page_commit<float>(const Geo&, void*, void*, float*, int32_t*, const void*, const void*, int,
                                        long long, int, float*, hipStream_t);
template void launch_page_commit<bf16_t>(const Geo&, void*, void*, float*, int32_t*, const void*, const void*, int,
                                         long long, int, float*, hipStream_t);

// ---------------------------------------------------------------------------
// Tier moves: page_slot[page] = value for each (page, value) update, after
// the promotions' page copies that precede it on the stream.

constexpr int kMaxTierUpdates = 256;
struct TierUpdates {
    int n;
    int page[kMaxTierUpdates];
    int value[kMaxTierUpdates];
};

__global__ void k_tier_table(int32_t* __restrict__ page_slot, TierUpdates u) {
    const int i = threadIdx.x;
    if (i < u.n) page_slot[u.page[i]] = u.value[i];
}

void launch_tier_table(int32_t* page_slot, int n, const int32_t* pages, const int32_t* values, hipStream_t st) {
    TierUpdates u;
    u.n = n;
    for (int i = 0; i < n; ++i) {
        u.page[i] = pages[i];
        u.value[i] = values[i];
    }
    hipLaunchKernelGGL(k_tier_table, dim3(1), dim3(kMaxTierUpdates), 0, st, page_slot, u);
}
