// Flash-style attention on gfx950 MFMA for the two HSA branches.
//
//  * Sparse branch (WorldAttention news summary, HSA paragraph): the 64
//    queries of query block i of head h attend, with exact softmax, to the
//    tokens of that row's selected key blocks only.
//  * Low-rank branch attention (same paragraph; Linformer projection): the
//    queries attend to the r projected keys K' with values V'. K' and V' are
//    float32; in the bf16 build they are carried as a bf16 hi + lo pair so the
//    MFMA products keep about 16 mantissa bits.
//
// Work-group: 256 threads = 4 waves, one row (64 queries) per work-group,
// wave w owns queries 16w..16w+15. Keys stream through LDS in tiles of 64:
//   Ks [64 keys][D + pad]  row-major, the A operand of S^T = K Q^T
//   Vt [D][64 keys + pad]  transposed, the A operand of O^T = V^T P^T
// Q stays in registers as the B operand. With S^T (keys x queries) in the
// 16x16 accumulator layout, lane l holds query (l & 15) and keys
// 16t + 4(l >> 4) + j; those same registers, read as a 32-key chunk whose k
// order is permuted consistently in P^T and V^T, are directly the B operand
// of O^T += V^T P^T, so P never moves between lanes. Softmax runs in float32
// with exp2 and a log2(e)/sqrt(d) prescale; the output is O / l.
#include "common.h"
#include "launch.h"

#include <type_traits>

namespace {

constexpr int KT = 64;          // keys per LDS tile
constexpr int kAttnThreads = 256;

// 8-element MFMA operand fragment of element type T.
template <typename T> struct Frag;
template <> struct Frag<bf16_t> {
    bf16x8_t v;
    HSAKV_DEV void set(int e, float x) { v[e] = (__bf16)x; }
};
template <> struct Frag<float> {
    float v[8];
    HSAKV_DEV void set(int e, float x) { v[e] = x; }
};

// acc(16x16) += A(16x32) * B(32x16) with 8-element fragments: lane l holds
// A[l & 15][8(l >> 4) + e] and B[8(l >> 4) + e][l & 15].
HSAKV_DEV void mma(f32x4_t& acc, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
// float32: eight 16x16x4 products. Product e pairs element e of every lane;
// across the four lane groups it contracts k = 8g + e, so the eight together
// contract the same 32 k as one bf16 16x16x32 product.
HSAKV_DEV void mma(f32x4_t& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

// 8 contiguous elements from LDS or global memory into a fragment.
HSAKV_DEV void load_frag(Frag<bf16_t>& f, const bf16_t* p) {
    f.v = *reinterpret_cast<const bf16x8_t*>(p);
}
HSAKV_DEV void load_frag(Frag<float>& f, const float* p) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
// 4 + 4 contiguous elements (two runs) into a fragment.
HSAKV_DEV void load_frag_split(Frag<bf16_t>& f, const bf16_t* p0, const bf16_t* p1) {
    uint2 a = *reinterpret_cast<const uint2*>(p0);
    uint2 b = *reinterpret_cast<const uint2*>(p1);
    uint4 w = {a.x, a.y, b.x, b.y};
    f.v = __builtin_bit_cast(bf16x8_t, w);
}
HSAKV_DEV void load_frag_split(Frag<float>& f, const float* p0, const float* p1) {
    float4 a = *reinterpret_cast<const float4*>(p0);
    float4 b = *reinterpret_cast<const float4*>(p1);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

// Raw 8-element chunk used to stage tiles (16 bytes for bf16, 32 for f32).
template <typename T> struct Chunk;
template <> struct Chunk<bf16_t> {
    uint4 w;
    HSAKV_DEV void load(const bf16_t* p) { w = *reinterpret_cast<const uint4*>(p); }
    HSAKV_DEV void zero() { w = {0, 0, 0, 0}; }
    HSAKV_DEV void store(bf16_t* p) const { *reinterpret_cast<uint4*>(p) = w; }
    HSAKV_DEV bf16_t at(int e) const {
        uint32_t x = e < 2 ? w.x : e < 4 ? w.y : e < 6 ? w.z : w.w;
        return (bf16_t)((e & 1) ? (x >> 16) : (x & 0xffffu));
    }
};
template <> struct Chunk<float> {
    float4 a, b;
    HSAKV_DEV void load(const float* p) {
        a = *reinterpret_cast<const float4*>(p);
        b = *reinterpret_cast<const float4*>(p + 4);
    }
    HSAKV_DEV void zero() { a = b = {0.f, 0.f, 0.f, 0.f}; }
    HSAKV_DEV void store(float* p) const {
        *reinterpret_cast<float4*>(p) = a;
        *reinterpret_cast<float4*>(p + 4) = b;
    }
    HSAKV_DEV float at(int e) const {
        switch (e) {
            case 0: return a.x; case 1: return a.y; case 2: return a.z; case 3: return a.w;
            case 4: return b.x; case 5: return b.y; case 6: return b.z; default: return b.w;
        }
    }
};

template <typename T, int D>
struct Tile {
    static constexpr int PADK = 16 / sizeof(T);   // 16 bytes per K row: conflict-free b128 reads
    static constexpr int PADV = 4;                // 4 elements per V^T row
    static constexpr int KLD = D + PADK;
    static constexpr int VLD = KT + PADV;
    T k[KT * KLD];
    T vt[D * VLD];
};

// Stage 64 key rows (K row-major, V transposed) into LDS. Row kk of the tile
// is token (t0 + kk) of `ksrc`/`vsrc` (row stride HD, this head's column
// offset already applied); rows kk >= nvalid are zero.
template <typename T, int D>
HSAKV_DEV void stage_tile(Tile<T, D>& tl, const T* __restrict__ ksrc, const T* __restrict__ vsrc,
                          long long t0, int nvalid, int HD) {
    constexpr int CPR = D / 8;                    // chunks per key row
    constexpr int ITER = KT * CPR / kAttnThreads;
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
        const int c = threadIdx.x + it * kAttnThreads;
        const int kk = c / CPR;
        const int ch = c % CPR;
        Chunk<T> kc, vc;
        if (kk < nvalid) {
            const long long off = (t0 + kk) * (long long)HD + ch * 8;
            kc.load(ksrc + off);
            vc.load(vsrc + off);
        } else {
            kc.zero();
            vc.zero();
        }
        kc.store(&tl.k[kk * Tile<T, D>::KLD + ch * 8]);
#pragma unroll
        for (int e = 0; e < 8; ++e) tl.vt[(ch * 8 + e) * Tile<T, D>::VLD + kk] = vc.at(e);
    }
}

// Online-softmax state and accumulators of one wave (16 queries).
template <typename T, int D>
struct WaveState {
    static constexpr int DS = D / 32;   // 32-wide k steps over d
    static constexpr int DT = D / 16;   // 16-row output tiles over d
    Frag<T> qf[DS];
    f32x4_t o[DT];
    float m;        // running max (log2 domain, prescaled)
    float l;        // this lane's partial row sum
};

// One 64-key tile: S^T = K Q^T, mask keys >= nvalid, online softmax, O^T += V^T P^T.
// Two K/V sources are summed when LO is set (the hi + lo split of K', V').
template <typename T, int D, bool LO>
HSAKV_DEV void tile_step(WaveState<T, D>& ws, const Tile<T, D>& th, const Tile<T, D>* tlo,
                         int nvalid, float scale_log2) {
    constexpr int DS = WaveState<T, D>::DS;
    constexpr int DT = WaveState<T, D>::DT;
    const int lane = threadIdx.x & 63;
    const int r16 = lane & 15;
    const int g = lane >> 4;

    f32x4_t s[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        s[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DS; ++ks) {
            Frag<T> a;
            load_frag(a, &th.k[(16 * t + r16) * Tile<T, D>::KLD + 32 * ks + 8 * g]);
            mma(s[t], a, ws.qf[ks]);
            if constexpr (LO) {
                load_frag(a, &tlo->k[(16 * t + r16) * Tile<T, D>::KLD + 32 * ks + 8 * g]);
                mma(s[t], a, ws.qf[ks]);
            }
        }
    }
    // scale, mask, row max over this lane's 16 keys and the 4 lane groups
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int key = 16 * t + 4 * g + j;
            float v = s[t][j] * scale_log2;
            v = key < nvalid ? v : -INFINITY;
            s[t][j] = v;
            mx = fmaxf(mx, v);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(ws.m, mx);
    const float alpha = fast_exp2(ws.m - m_new);   // m starts at -inf: exp2(-inf) = 0
    ws.m = m_new;
    float rs = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float p = fast_exp2(s[t][j] - m_new);
            s[t][j] = p;
            rs += p;
        }
    }
    ws.l = ws.l * alpha + rs;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) ws.o[dt] *= alpha;

    // O^T += V^T P^T over two 32-key chunks
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        Frag<T> pf;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            pf.set(j, s[2 * c][j]);
            pf.set(4 + j, s[2 * c + 1][j]);
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int drow = 16 * dt + r16;
            Frag<T> vf;
            load_frag_split(vf, &th.vt[drow * Tile<T, D>::VLD + 32 * c + 4 * g],
                            &th.vt[drow * Tile<T, D>::VLD + 32 * c + 16 + 4 * g]);
            mma(ws.o[dt], vf, pf);
            if constexpr (LO) {
                load_frag_split(vf, &tlo->vt[drow * Tile<T, D>::VLD + 32 * c + 4 * g],
                                &tlo->vt[drow * Tile<T, D>::VLD + 32 * c + 16 + 4 * g]);
                mma(ws.o[dt], vf, pf);
            }
        }
    }
}

template <typename T, int D>
HSAKV_DEV void load_q(WaveState<T, D>& ws, const T* __restrict__ q, int query, int Lq, int HD, int h) {
    const int g = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int ks = 0; ks < WaveState<T, D>::DS; ++ks) {
        if (query < Lq) {
            load_frag(ws.qf[ks], q + (long long)query * HD + (long long)h * D + 32 * ks + 8 * g);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) ws.qf[ks].set(e, 0.f);
        }
    }
#pragma unroll
    for (int dt = 0; dt < WaveState<T, D>::DT; ++dt) ws.o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    ws.m = -INFINITY;
    ws.l = 0.f;
}

// Write O / l for this lane's query; optionally the gated fusion with the
// low-rank branch: out = g * O + (1 - g) * o_lin, g = sigmoid(<q, w_g> + b_g).
template <typename T, int D>
HSAKV_DEV void epilogue(const WaveState<T, D>& ws, const Epi& ep, int query, int Lq, int HD, int h) {
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    float lt = ws.l;
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
    const float inv_l = 1.0f / lt;
    float gate = 0.f;
    if (ep.out) {
        float dot = 0.f;
#pragma unroll
        for (int ks = 0; ks < WaveState<T, D>::DS; ++ks) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                float qv;
                if constexpr (sizeof(T) == 2) qv = (float)ws.qf[ks].v[e];
                else qv = ws.qf[ks].v[e];
                dot = fmaf(qv, ep.w_g[h * D + 32 * ks + 8 * g + e], dot);
            }
        }
        dot += __shfl_xor(dot, 16, 64);
        dot += __shfl_xor(dot, 32, 64);
        const float x = dot + ep.b_g[h];
        // overflow-free logistic
        const float z = expf(-fabsf(x));
        gate = x >= 0.f ? 1.0f / (1.0f + z) : z / (1.0f + z);
    }
    if (query >= Lq) return;
    const long long row = (long long)query * HD + (long long)h * D;
    if (ep.gate && g == 0) ep.gate[(long long)query * (HD / D) + h] = gate;
#pragma unroll
    for (int dt = 0; dt < WaveState<T, D>::DT; ++dt) {
        const int d0 = 16 * dt + 4 * g;
        float4 o = {ws.o[dt][0] * inv_l, ws.o[dt][1] * inv_l, ws.o[dt][2] * inv_l, ws.o[dt][3] * inv_l};
        if (ep.o_main) *reinterpret_cast<float4*>(ep.o_main + row + d0) = o;
        if (ep.out) {
            const float4 lin = *reinterpret_cast<const float4*>(ep.o_lin + row + d0);
            float r[4] = {gate * o.x + (1.f - gate) * lin.x, gate * o.y + (1.f - gate) * lin.y,
                          gate * o.z + (1.f - gate) * lin.z, gate * o.w + (1.f - gate) * lin.w};
            T* dst = reinterpret_cast<T*>(ep.out) + row + d0;
#pragma unroll
            for (int j = 0; j < 4; ++j) dst[j] = Elt<T>::from_f32(r[j]);
        }
    }
}

// Key block b -> token range and source (history blocks first, then chunk blocks).
HSAKV_DEV void block_range(const Geo& g, int NBh, long long Lh, int b, bool& hist, long long& t0,
                           int& len) {
    if (b < NBh) {
        hist = true;
        t0 = (long long)b * g.Binter;
        long long e = t0 + g.Binter < Lh ? t0 + g.Binter : Lh;
        len = (int)(e - t0);
    } else {
        hist = false;
        t0 = (long long)(b - NBh) * g.Bintra;
        long long e = t0 + g.Bintra < g.Lq ? t0 + g.Bintra : g.Lq;
        len = (int)(e - t0);
    }
}

template <typename T, int D>
__global__ void __launch_bounds__(kAttnThreads)
k_sparse_attn(Geo g, const T* __restrict__ q, const T* __restrict__ k_hist,
              const T* __restrict__ v_hist, const T* __restrict__ k_intra,
              const T* __restrict__ v_intra, const int32_t* __restrict__ n_sel_p,
              const int32_t* __restrict__ sel_count, const int32_t* __restrict__ sel_idx,
              const int32_t* __restrict__ row_order, Epi ep) {
    __shared__ Tile<T, D> tl;
    const int row = row_order ? row_order[blockIdx.x] : (int)blockIdx.x;
    const int h = row / g.NQB;
    const int i = row % g.NQB;
    const int wave = threadIdx.x >> 6;
    const int query = i * g.Bq + 16 * wave + (threadIdx.x & 15);
    const int n_sel = *n_sel_p;
    const int NBh = hist_blocks(g, n_sel);
    const long long Lh = (long long)n_sel * g.Tp;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);

    WaveState<T, D> ws;
    load_q(ws, q, query, g.Lq, g.HD, h);

    const int cnt = sel_count[row];
    const int32_t* ids = sel_idx + (size_t)row * g.NB_max;
    const long long hoff = (long long)h * D;
    for (int n = 0; n < cnt; ++n) {
        bool hist;
        long long t0;
        int len;
        block_range(g, NBh, Lh, ids[n], hist, t0, len);
        const T* ks = (hist ? k_hist : k_intra) + hoff;
        const T* vs = (hist ? v_hist : v_intra) + hoff;
        for (int s0 = 0; s0 < len; s0 += KT) {
            const int nvalid = len - s0 < KT ? len - s0 : KT;
            __syncthreads();
            stage_tile<T, D>(tl, ks, vs, t0 + s0, nvalid, g.HD);
            __syncthreads();
            tile_step<T, D, false>(ws, tl, nullptr, nvalid, scale_log2);
        }
    }
    epilogue<T, D>(ws, ep, query, g.Lq, g.HD, h);
}

// Dense attention of the queries over the r projected keys (hi + lo pair in
// the bf16 build, plain float32 in the f32 build).
template <typename T, int D, bool LO>
__global__ void __launch_bounds__(kAttnThreads)
k_lowrank_attn(Geo g, const T* __restrict__ q, const T* __restrict__ k_hi,
               const T* __restrict__ v_hi, const T* __restrict__ k_lo, const T* __restrict__ v_lo,
               Epi ep) {
    struct Pair { Tile<T, D> hi, lo; };
    __shared__ typename std::conditional<LO, Pair, Tile<T, D>>::type sm;
    Tile<T, D>& th = *reinterpret_cast<Tile<T, D>*>(&sm);
    Tile<T, D>* tlo = LO ? reinterpret_cast<Tile<T, D>*>(&sm) + 1 : nullptr;
    const int row = blockIdx.x;
    const int h = row / g.NQB;
    const int i = row % g.NQB;
    const int wave = threadIdx.x >> 6;
    const int query = i * g.Bq + 16 * wave + (threadIdx.x & 15);
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    WaveState<T, D> ws;
    load_q(ws, q, query, g.Lq, g.HD, h);
    const long long hoff = (long long)h * D;
    for (int s0 = 0; s0 < g.r; s0 += KT) {
        const int nvalid = g.r - s0 < KT ? g.r - s0 : KT;
        __syncthreads();
        stage_tile<T, D>(th, k_hi + hoff, v_hi + hoff, s0, nvalid, g.HD);
        if constexpr (LO) stage_tile<T, D>(*tlo, k_lo + hoff, v_lo + hoff, s0, nvalid, g.HD);
        __syncthreads();
        tile_step<T, D, LO>(ws, th, tlo, nvalid, scale_log2);
    }
    epilogue<T, D>(ws, ep, query, g.Lq, g.HD, h);
}

}  // namespace

template <typename T>
void launch_sparse_attn(const Geo& g, const void* q, const void* k_hist, const void* v_hist,
                        const void* k_intra, const void* v_intra, const int32_t* n_sel,
                        const int32_t* sel_count, const int32_t* sel_idx,
                        void* ws, const Epi& ep, hipStream_t st) {
    if constexpr (sizeof(T) == 2) {
        // bf16: the balanced 32x32x16 MFMA kernels (k_sparse32.hip)
        launch_sparse_attn_bf16_mfma32(g, q, k_hist, v_hist, k_intra, v_intra, n_sel, sel_count,
                                       sel_idx, ws, ep, st);
        return;
    }
    const int32_t* row_order = nullptr;
    dim3 grid(g.H * g.NQB);
    if (g.d == 128)
        hipLaunchKernelGGL((k_sparse_attn<T, 128>), grid, dim3(kAttnThreads), 0, st, g, (const T*)q,
                           (const T*)k_hist, (const T*)v_hist, (const T*)k_intra,
                           (const T*)v_intra, n_sel, sel_count, sel_idx, row_order, ep);
    else
        hipLaunchKernelGGL((k_sparse_attn<T, 64>), grid, dim3(kAttnThreads), 0, st, g, (const T*)q,
                           (const T*)k_hist, (const T*)v_hist, (const T*)k_intra,
                           (const T*)v_intra, n_sel, sel_count, sel_idx, row_order, ep);
}
template void launch_sparse_attn<float>(const Geo&, const void*, const void*, const void*,
                                        const void*, const void*, const int32_t*, const int32_t*,
                                        const int32_t*, void*, const Epi&, hipStream_t);
template void launch_sparse_attn<bf16_t>(const Geo&, const void*, const void*, const void*,
                                         const void*, const void*, const int32_t*, const int32_t*,
                                         const int32_t*, void*, const Epi&, hipStream_t);

template <typename T>
void launch_lowrank_attn(const Geo& g, const void* q, const void* k_hi, const void* v_hi,
                         const void* k_lo, const void* v_lo, const Epi& ep, hipStream_t st) {
    if (sizeof(T) == 2 && !ep.out && ep.o_main && (g.d == 64 || g.d == 128)) {
        // bf16: the 32x32x16 MFMA kernel (k_lowrank32.hip)
        launch_lowrank_attn_bf16_mfma32(g, q, k_hi, v_hi, k_lo, v_lo, ep.o_main, st);
        return;
    }
    dim3 grid(g.H * g.NQB);
    constexpr bool LO = sizeof(T) == 2;
    if (g.d == 128)
        hipLaunchKernelGGL((k_lowrank_attn<T, 128, LO>), grid, dim3(kAttnThreads), 0, st, g,
                           (const T*)q, (const T*)k_hi, (const T*)v_hi, (const T*)k_lo,
                           (const T*)v_lo, ep);
    else
        hipLaunchKernelGGL((k_lowrank_attn<T, 64, LO>), grid, dim3(kAttnThreads), 0, st, g,
                           (const T*)q, (const T*)k_hi, (const T*)v_hi, (const T*)k_lo,
                           (const T*)v_lo, ep);
}
template void launch_lowrank_attn<float>(const Geo&, const void*, const void*, const void*,
                                         const void*, const void*, const Epi&, hipStream_t);
template void launch_lowrank_attn<bf16_t>(const Geo&, const void*, const void*, const void*,
                                          const void*, const void*, const Epi&, hipStream_t);
