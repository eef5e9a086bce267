// Head-adaptive block selection: block pooling, block mass, minimal set.
//
// Pages: WorldAttention news summary (ai4snews), HSA paragraph: per head, the
// fewest key blocks whose cumulative attention mass reaches tau_h, with
// Binter-token history blocks and Bintra-token chunk blocks; tau from 0.35 to
// 1.00 (Table 4).
#include "common.h"
#include "launch.h"

// ---------------------------------------------------------------------------
// Pooling: the mean over each block's valid tokens, for query blocks, history
// key blocks and chunk key blocks. One work-group per (token block, 256
// columns): 32 column lanes of 8 elements x 8 token groups, Kahan-free fixed
// order sums (blocks are at most 512 tokens).
//   blockIdx.x in [0, NQB)                 : query block i    -> qb[h][i][:]
//   blockIdx.x in [NQB, NQB + hist_grid)   : history block b  -> kb[h][b][:]
//   blockIdx.x in [NQB + hist_grid, ...)   : chunk block j    -> kb[h][NBh + j][:]
// hist_grid is NBh_max, or 0 when the gather has pooled the history blocks.
// kb rows are indexed with the present history length, so chunk blocks
// follow the last present history block directly.

template <typename T>
__global__ void __launch_bounds__(256)
k_pool(Geo g, const T* __restrict__ q, const T* __restrict__ k_hist, const T* __restrict__ k_intra,
       const int32_t* __restrict__ n_sel_p, float* __restrict__ qb, float* __restrict__ kb, int hist_grid) {
    const int n_sel = *n_sel_p;
    const int NBh = hist_blocks(g, n_sel);
    const long long Lh = (long long)n_sel * g.Tp;
    int bx = blockIdx.x;
    const T* src;
    long long t0, t1;
    float* dst;
    size_t dst_head_stride;
    if (bx < g.NQB) {
        src = q;
        t0 = (long long)bx * g.Bq;
        t1 = t0 + g.Bq < g.Lq ? t0 + g.Bq : g.Lq;
        dst = qb + (size_t)bx * g.d;
        dst_head_stride = (size_t)g.NQB * g.d;
    } else if (bx < g.NQB + hist_grid) {
        int b = bx - g.NQB;
        if (b >= NBh) return;
        src = k_hist;
        t0 = (long long)b * g.Binter;
        t1 = t0 + g.Binter < Lh ? t0 + g.Binter : Lh;
        dst = kb + (size_t)b * g.d;
        dst_head_stride = (size_t)g.NB_max * g.d;
    } else {
        int j = bx - g.NQB - hist_grid;
        src = k_intra;
        t0 = (long long)j * g.Bintra;
        t1 = t0 + g.Bintra < g.Lq ? t0 + g.Bintra : g.Lq;
        dst = kb + (size_t)(NBh + j) * g.d;
        dst_head_stride = (size_t)g.NB_max * g.d;
    }
    const int lane = threadIdx.x & 31;
    const int grp = threadIdx.x >> 5;              // 8 token groups
    const int col0 = (blockIdx.y * 32 + lane) * 8; // first of 8 columns
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (col0 < g.HD) {
        // four tokens of this group in flight at a time; the sum order is
        // still token order within the group
        for (long long t = t0 + grp; t < t1; t += 32) {
            float v[4][8];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const long long tu = t + 8 * u < t1 ? t + 8 * u : t;
                Elt<T>::load8(src + tu * g.HD + col0, v[u]);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (t + 8 * u < t1) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[e] += v[u][e];
                }
        }
    }
    __shared__ float part[8][32 * 8 + 4];
#pragma unroll
    for (int e = 0; e < 8; ++e) part[grp][lane * 8 + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < 256) {
        const int c = blockIdx.y * 256 + threadIdx.x;   // column handled in the final add
        if (c < g.HD) {
            float s = 0.f;
#pragma unroll
            for (int k = 0; k < 8; ++k) s += part[k][threadIdx.x];
            const int h = c / g.d, e = c % g.d;
            dst[(size_t)h * dst_head_stride + e] = s / (float)(t1 - t0);
        }
    }
}

template <typename T>
void launch_pool(const Geo& g, const void* q, const void* k_hist, const void* k_intra,
                 const int32_t* n_sel, float* qb, float* kb, bool hist_pooled, hipStream_t st) {
    const int hist_grid = hist_pooled ? 0 : g.NBh_max;
    dim3 grid(g.NQB + hist_grid + g.NBc, (g.HD + 255) / 256);
    hipLaunchKernelGGL(k_pool<T>, grid, dim3(256), 0, st, g, (const T*)q, (const T*)k_hist,
                       (const T*)k_intra, n_sel, qb, kb, hist_grid);
}
template void launch_pool<float>(const Geo&, const void*, const void*, const void*, const int32_t*,
                                 float*, float*, bool, hipStream_t);
template void launch_pool<bf16_t>(const Geo&, const void*, const void*, const void*,
                                  const int32_t*, float*, float*, bool, hipStream_t);

// ---------------------------------------------------------------------------
// Selection: one work-group (256 threads) per row (head h, query block i).
//  1. z_b = <qb[h,i], kb[h,b]> / sqrt(d), one wave per block in turn.
//  2. p_b = softmax_b(z) in float32 (max-subtracted, fixed-order sums).
//  3. Sort 64-bit keys (~bits(p_b) << 32 | b) ascending with a bitonic sort
//     in LDS: mass descending, equal masses by ascending id.
//  4. Inclusive float32 scan of the sorted masses (fixed tree order); k* is
//     one past the first position whose running mass reaches tau.
//  5. Flag the first k* sorted ids and compact them in ascending id order.

constexpr int kSelThreads = 256;
constexpr int kSelMaxNB = 4096;

__device__ __forceinline__ float block_reduce_max(float v, float* red) {
    v = wave_max(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return r;
}

__device__ __forceinline__ float block_reduce_sum(float v, float* red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float r = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return r;
}

__global__ void __launch_bounds__(kSelThreads)
k_select(Geo g, const float* __restrict__ qb, const float* __restrict__ kb,
         const int32_t* __restrict__ n_sel_p, TauArg tau,
         int32_t* __restrict__ sel_count, int32_t* __restrict__ sel_idx,
         uint8_t* __restrict__ sel_mask, float* __restrict__ block_mass) {
    __shared__ unsigned long long keys[kSelMaxNB];
    __shared__ float mass[kSelMaxNB];        // by block id, later reused for the scan
    __shared__ float qrow[512];
    __shared__ float red[4];
    __shared__ int first_hit;

    const int row = blockIdx.x;
    const int h = row / g.NQB;
    const int i = row % g.NQB;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n_sel = *n_sel_p;
    const int NB = hist_blocks(g, n_sel) + g.NBc;
    const float t = tau.v[h];

    for (int e = tid; e < g.d; e += kSelThreads) qrow[e] = qb[((size_t)h * g.NQB + i) * g.d + e];
    __syncthreads();

    // 1. pooled logits
    const float inv_sqrt_d = 1.0f / sqrtf((float)g.d);
    const float* kbh = kb + (size_t)h * g.NB_max * g.d;
    for (int b = wave; b < NB; b += kSelThreads / 64) {
        float s = 0.f;
        for (int e = lane; e < g.d; e += 64) s = fmaf(qrow[e], kbh[(size_t)b * g.d + e], s);
        s = wave_sum(s);
        if (lane == 0) mass[b] = s * inv_sqrt_d;
    }
    __syncthreads();

    // 2. softmax over blocks
    float m = -INFINITY;
    for (int b = tid; b < NB; b += kSelThreads) m = fmaxf(m, mass[b]);
    m = block_reduce_max(m, red);
    float part = 0.f;
    for (int b = tid; b < NB; b += kSelThreads) {
        float e = expf(mass[b] - m);
        mass[b] = e;
        part += e;
    }
    const float total = block_reduce_sum(part, red);  // also a barrier for mass[]
    const float inv_total = 1.0f / total;
    int NBp = 1;
    while (NBp < NB) NBp <<= 1;
    for (int b = tid; b < NBp; b += kSelThreads) {
        if (b < NB) {
            float p = mass[b] * inv_total;
            mass[b] = p;
            keys[b] = ((unsigned long long)(~__float_as_uint(p)) << 32) | (unsigned)b;
        } else {
            keys[b] = ~0ull;
        }
    }
    __syncthreads();
    if (block_mass) {
        float* dst = block_mass + ((size_t)h * g.NQB + i) * g.NB_max;
        for (int b = tid; b < NB; b += kSelThreads) dst[b] = mass[b];
    }
    __syncthreads();

    // 3. bitonic sort, ascending keys
    for (int k = 2; k <= NBp; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int x = tid; x < NBp; x += kSelThreads) {
                int y = x ^ j;
                if (y > x) {
                    unsigned long long a = keys[x], c = keys[y];
                    bool up = (x & k) == 0;
                    if ((a > c) == up) { keys[x] = c; keys[y] = a; }
                }
            }
            __syncthreads();
        }
    }

    // 4. inclusive scan of the sorted masses (Hillis-Steele in LDS, fixed order)
    int kstar;
    if (t >= 1.0f) {
        kstar = NB;
    } else {
        float* scan = mass;   // masses by id are no longer needed
        for (int x = tid; x < NB; x += kSelThreads)
            scan[x] = __uint_as_float(~(unsigned)(keys[x] >> 32));
        __syncthreads();
        for (int off = 1; off < NB; off <<= 1) {
            float v[kSelMaxNB / kSelThreads];
            int n = 0;
            for (int x = tid; x < NB; x += kSelThreads, ++n) v[n] = x >= off ? scan[x - off] : 0.f;
            __syncthreads();
            n = 0;
            for (int x = tid; x < NB; x += kSelThreads, ++n) scan[x] += v[n];
            __syncthreads();
        }
        if (tid == 0) first_hit = NB;
        __syncthreads();
        for (int x = tid; x < NB; x += kSelThreads)
            if (scan[x] >= t) atomicMin(&first_hit, x);
        __syncthreads();
        kstar = first_hit < NB ? first_hit + 1 : NB;
    }
    __syncthreads();

    // 5. flags by id, then ascending compaction
    int* flag = reinterpret_cast<int*>(mass);
    for (int b = tid; b < NB; b += kSelThreads) flag[b] = 0;
    __syncthreads();
    for (int x = tid; x < kstar; x += kSelThreads) flag[(int)(keys[x] & 0xffffffffu)] = 1;
    __syncthreads();
    int32_t* out = sel_idx + ((size_t)h * g.NQB + i) * g.NB_max;
    if (sel_mask) {
        uint8_t* mk = sel_mask + ((size_t)h * g.NQB + i) * g.NB_max;
        for (int b = tid; b < NB; b += kSelThreads) mk[b] = (uint8_t)flag[b];
    }
    // ascending compaction: each wave scans a contiguous range of ids
    __shared__ int wave_count[4];
    const int per = (NB + 3) / 4;
    const int lo = wave * per, hi = lo + per < NB ? lo + per : NB;
    int cnt = 0;
    for (int b0 = lo; b0 < hi; b0 += 64) {
        int b = b0 + lane;
        bool f = b < hi && flag[b];
        cnt += __popcll(__ballot(f));
    }
    if (lane == 0) wave_count[wave] = cnt;
    __syncthreads();
    int pos = 0;
    for (int w = 0; w < wave; ++w) pos += wave_count[w];
    for (int b0 = lo; b0 < hi; b0 += 64) {
        int b = b0 + lane;
        bool f = b < hi && flag[b];
        unsigned long long bal = __ballot(f);
        int before = __popcll(bal & ((1ull << lane) - 1ull));
        if (f) out[pos + before] = b;
        pos += __popcll(bal);
    }
    if (tid == 0) sel_count[(size_t)h * g.NQB + i] = kstar;
}

// ---------------------------------------------------------------------------
// Selection, one wave per row, everything in registers (NB <= 64 * NPL).
// Lane l owns blocks b = l + 64 j. After the softmax, the selected set is the
// shortest prefix of the order (mass descending, id ascending) whose mass
// reaches tau. With key(b) = (~bits(p_b), b) (ascending key = that order) it
// is {b : key(b) <= K*}, K* the smallest key with S(K) >= tau, where
// S(K) = sum over b of (key(b) <= K ? p_b : 0) taken by a fixed butterfly:
// S is monotone in K, so K* is found by binary search, first over the mass
// bits, then over the ids that tie on them. No sort and no barrier.

// Block logits for the wave path, as one small GEMM per head on float32 MFMA:
// Z[h][i][b] = <qb[h][i], kb[h][b]> / sqrt(d) (i < NQB, b < NB), one wave per
// 32 x 32 tile of (query block, key block) pairs, v_mfma_f32_32x32x2_f32 over
// d. Lane l feeds A[i = l % 32][k] and B[k][b = l % 32] for the d term its
// half (l / 32) takes in each product; any assignment of the d terms to
// products gives the same dot product.
template <int D>
__global__ void __launch_bounds__(256)
k_block_logits(Geo g, const float* __restrict__ qb, const float* __restrict__ kb,
               const int32_t* __restrict__ n_sel_p, float* __restrict__ z) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int mt = (g.NQB + 31) / 32, nt = (g.NB_max + 31) / 32;
    const int tile = blockIdx.x * 4 + wave;
    if (tile >= g.H * mt * nt) return;
    const int h = tile / (mt * nt), rem = tile % (mt * nt), ti = rem / nt, tb = rem % nt;
    const int NB = hist_blocks(g, *n_sel_p) + g.NBc;
    if (tb * 32 >= NB) return;
    const int r32 = lane & 31, g2 = lane >> 5;
    const int ia = ti * 32 + r32 < g.NQB ? ti * 32 + r32 : g.NQB - 1;
    const int ba = tb * 32 + r32 < NB ? tb * 32 + r32 : NB - 1;
    const float* qa = qb + ((size_t)h * g.NQB + ia) * D;
    const float* kr = kb + ((size_t)h * g.NB_max + ba) * D;
    f32x16_t acc = f32x16_t{};
    // 32 d-values of each operand in flight at a time
    // products 2u, 2u + 1 take d = 4u + 2 (l / 32) and the one after it
#pragma unroll
    for (int t0 = 0; t0 < D; t0 += 32) {
        float2 a[8], b[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            a[u] = *reinterpret_cast<const float2*>(qa + t0 + 4 * u + 2 * g2);
            b[u] = *reinterpret_cast<const float2*>(kr + t0 + 4 * u + 2 * g2);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[u].x, b[u].x, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[u].y, b[u].y, acc, 0, 0, 0);
        }
    }
    // element e of lane l: query block 8 (e / 4) + 4 (l / 32) + e % 4, key block l % 32
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    const int b = tb * 32 + r32;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int i = ti * 32 + 8 * (e >> 2) + 4 * g2 + (e & 3);
        if (i < g.NQB && b < NB) z[((size_t)h * g.NQB + i) * g.NB_max + b] = acc[e] * inv_sqrt_d;
    }
}

HSAKV_DEV float masked_sum(const float* p, const unsigned* mb, int NPL_, unsigned M, int I,
                           bool use_id, int lane) {
    float acc = 0.f;
    for (int j = 0; j < NPL_; ++j) {
        const int b = lane + 64 * j;
        const bool in = mb[j] < M || (mb[j] == M && (!use_id || b <= I));
        acc += in ? p[j] : 0.f;
    }
    return wave_sum(acc);
}

template <int NPL>
__global__ void __launch_bounds__(256)
k_select_wave(Geo g, const float* __restrict__ zl, const int32_t* __restrict__ n_sel_p, TauArg tau,
              int32_t* __restrict__ sel_count, int32_t* __restrict__ sel_idx, uint8_t* __restrict__ sel_mask,
              float* __restrict__ block_mass) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int row = blockIdx.x * 4 + wave;
    if (row >= g.H * g.NQB) return;
    const int h = row / g.NQB;
    const int i = row % g.NQB;
    const int n_sel = *n_sel_p;
    const int NB = hist_blocks(g, n_sel) + g.NBc;

    // the row's pooled logits (k_block_logits), one block per lane and item
    const float* zr = zl + ((size_t)h * g.NQB + i) * g.NB_max;
    float p[NPL];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const int b = lane + 64 * j;
        const float z = b < NB ? zr[b] : -INFINITY;
        p[j] = z;
        mx = fmaxf(mx, z);
    }
    mx = wave_max(mx);
    float part = 0.f;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const float e = lane + 64 * j < NB ? expf(p[j] - mx) : 0.f;
        p[j] = e;
        part += e;
    }
    const float inv_total = 1.0f / wave_sum(part);
    unsigned mb[NPL];
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const bool ok = lane + 64 * j < NB;
        p[j] = ok ? p[j] * inv_total : 0.f;
        mb[j] = ok ? ~__float_as_uint(p[j]) : 0xffffffffu;    // padding sorts last
    }
    if (block_mass) {
        float* dst = block_mass + ((size_t)h * g.NQB + i) * g.NB_max;
#pragma unroll
        for (int j = 0; j < NPL; ++j)
            if (lane + 64 * j < NB) dst[lane + 64 * j] = p[j];
    }

    // threshold key (M*, I*)
    const float t = tau.v[h];
    unsigned Mst = 0xffffffffu;
    int Ist = NB - 1;
    bool all = t >= 1.0f;
    if (!all) {
        if (masked_sum(p, mb, NPL, 0xffffffffu, 0, false, lane) < t) {
            all = true;                                  // rounding kept the total below tau
        } else {
            unsigned lo = 0, hi = 0xffffffffu;           // smallest M with S(M, all ids) >= t
            while (lo < hi) {
                const unsigned mid = lo + ((hi - lo) >> 1);
                if (masked_sum(p, mb, NPL, mid, 0, false, lane) >= t) hi = mid; else lo = mid + 1;
            }
            Mst = lo;
            int ilo = 0, ihi = NB - 1;                    // smallest id among the ties
            while (ilo < ihi) {
                const int mid = (ilo + ihi) >> 1;
                if (masked_sum(p, mb, NPL, Mst, mid, true, lane) >= t) ihi = mid; else ilo = mid + 1;
            }
            Ist = ilo;
        }
    }

    // ascending compaction of {b : key(b) <= (M*, I*)}
    int32_t* out = sel_idx + ((size_t)h * g.NQB + i) * g.NB_max;
    uint8_t* mk = sel_mask ? sel_mask + ((size_t)h * g.NQB + i) * g.NB_max : nullptr;
    int pos = 0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) {
        const int b = lane + 64 * j;
        const bool f = b < NB && (all || mb[j] < Mst || (mb[j] == Mst && b <= Ist));
        const unsigned long long bal = __ballot(f);
        if (f) out[pos + __popcll(bal & ((1ull << lane) - 1ull))] = b;
        if (mk && b < NB) mk[b] = (uint8_t)f;
        pos += __popcll(bal);
    }
    if (lane == 0) sel_count[(size_t)h * g.NQB + i] = pos;
}

void launch_select(const Geo& g, const float* qb, const float* kb, float* zl, const int32_t* n_sel,
                   const TauArg& tau_dev, int32_t* sel_count, int32_t* sel_idx, uint8_t* sel_mask,
                   float* block_mass, hipStream_t st) {
    const int rows = g.H * g.NQB;
    const int per_lane = (g.NB_max + 63) / 64;
    if ((g.d == 64 || g.d == 128) && per_lane <= 32) {
        const int tiles = g.H * ((g.NQB + 31) / 32) * ((g.NB_max + 31) / 32);
        if (g.d == 128)
            hipLaunchKernelGGL(k_block_logits<128>, dim3((tiles + 3) / 4), dim3(256), 0, st, g, qb, kb, n_sel, zl);
        else
            hipLaunchKernelGGL(k_block_logits<64>, dim3((tiles + 3) / 4), dim3(256), 0, st, g, qb, kb, n_sel, zl);
        const dim3 grid((rows + 3) / 4);
#define HSAKV_SEL(NPL)                                                                            \
    hipLaunchKernelGGL(k_select_wave<NPL>, grid, dim3(256), 0, st, g, (const float*)zl, n_sel, tau_dev, \
                       sel_count, sel_idx, sel_mask, block_mass)
        if (per_lane <= 2) HSAKV_SEL(2);
        else if (per_lane <= 8) HSAKV_SEL(8);
        else if (per_lane <= 16) HSAKV_SEL(16);
        else HSAKV_SEL(32);
#undef HSAKV_SEL
        return;
    }
    hipLaunchKernelGGL(k_select, dim3(rows), dim3(kSelThreads), 0, st, g, qb, kb, n_sel,
                       tau_dev, sel_count, sel_idx, sel_mask, block_mass);
}
