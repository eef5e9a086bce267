// Low-rank (Linformer-style) global branch and the gated fusion.
//
// Pages: WorldAttention news summary (ai4snews), HSA paragraph: the linear
// branch projects the L keys and values to rank r (O(L r) instead of O(L^2)),
// and learned gates fuse it with the sparse branch. The projection follows
// the Linformer paper cited on the mlsanity map: K' = E K, V' = F V, one E
// and one F shared by all heads.
#include "common.h"
#include "launch.h"

namespace {

// ---------------------------------------------------------------------------
// Projection: part[z][split][m][n] = sum over the split's active key indices k
// of X_z[m][col(k)] * Y_z[row(k)][n], (X, Y) = (E, K) for z = 0, (F, V) for z = 1.
// Active key index k runs over the present history rows [0, Lh) then the
// chunk rows; col(k) is its column of E/F (slot columns, then the chunk's
// last Lq columns). A dense contraction: bf16 MFMA 16x16x32 (f32: 16x16x4).
// Tile 256 (m) x 64 (n), k-step 32; wave w owns m rows 64w..64w+63.

constexpr int PBM = 256, PBN = 64, PBK = 32;
constexpr int kProjThreads = 256;

template <typename T> struct PFrag;
template <> struct PFrag<bf16_t> { bf16x8_t v; };
template <> struct PFrag<float> { float v[8]; };

HSAKV_DEV void pmma(f32x4_t& acc, const PFrag<bf16_t>& a, const PFrag<bf16_t>& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
HSAKV_DEV void pmma(f32x4_t& acc, const PFrag<float>& a, const PFrag<float>& b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
}
HSAKV_DEV void pload(PFrag<bf16_t>& f, const bf16_t* p) { f.v = *reinterpret_cast<const bf16x8_t*>(p); }
HSAKV_DEV void pload(PFrag<float>& f, const float* p) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f.v[e] = p[e];
}

template <typename T>
struct ProjSmem {
    static constexpr int LD = PBK + 16 / sizeof(T);
    T a[PBM * LD];     // [m][k]
    T bt[PBN * LD];    // [n][k]
};

template <typename T>
__global__ void __launch_bounds__(kProjThreads)
k_lowrank_proj(Geo g, const T* __restrict__ E, const T* __restrict__ F,
               const T* __restrict__ k_hist, const T* __restrict__ v_hist,
               const T* __restrict__ k_intra, const T* __restrict__ v_intra,
               const int32_t* __restrict__ n_sel_p, int nsplit, float* __restrict__ part) {
    __shared__ ProjSmem<T> sm;
    constexpr int LD = ProjSmem<T>::LD;
    const int n0 = blockIdx.x * PBN;
    const int m0 = blockIdx.y * PBM;
    const int z = blockIdx.z & 1;
    const int split = blockIdx.z >> 1;
    const T* X = z == 0 ? E : F;
    const T* Yh = z == 0 ? k_hist : v_hist;
    const T* Yc = z == 0 ? k_intra : v_intra;
    const long long Lh = (long long)(*n_sel_p) * g.Tp;
    const long long Lact = Lh + g.Lq;
    const long long per = ((Lact + nsplit - 1) / nsplit + PBK - 1) / PBK * PBK;
    const long long kb = (long long)split * per;
    const long long ke = kb + per < Lact ? kb + per : Lact;

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, r16 = lane & 15, grp = lane >> 4;
    f32x4_t acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (long long k0 = kb; k0 < ke; k0 += PBK) {
        __syncthreads();
        // A: 256 rows x 32 k of X, 4 chunks of 8 per row
#pragma unroll
        for (int it = 0; it < PBM * (PBK / 8) / kProjThreads; ++it) {
            const int c = tid + it * kProjThreads;
            const int m = c >> 2, kc = c & 3;
            T* dst = &sm.a[m * LD + kc * 8];
            const long long k = k0 + kc * 8;
            const bool row_ok = m0 + m < g.r;
            const long long col = k < Lh ? k : g.hist_rows + (k - Lh);
            const long long colend = k + 7 < Lh ? k + 7 : g.hist_rows + (k + 7 - Lh);
            const T* src = X + (long long)(m0 + m) * g.L;
            if (row_ok && k + 8 <= ke && colend == col + 7 && ((col & 7) == 0) && ((g.L & 7) == 0)) {
                *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src + col);
                if constexpr (sizeof(T) == 4)
                    *reinterpret_cast<uint4*>(dst + 4) = *reinterpret_cast<const uint4*>(src + col + 4);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const long long kk = k + e;
                    T v = T(0);
                    if (row_ok && kk < ke) v = src[kk < Lh ? kk : g.hist_rows + (kk - Lh)];
                    dst[e] = v;
                }
            }
        }
        // B: 32 k rows x 64 n of Y, stored transposed [n][k]
        {
            const int kr = tid >> 3, nc = tid & 7;
            const long long k = k0 + kr;
            T vals[8];
            if (k < ke) {
                const T* src = (k < Lh ? Yh + k * g.HD : Yc + (k - Lh) * g.HD) + n0 + nc * 8;
                if (n0 + nc * 8 + 8 <= g.HD) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) vals[e] = src[e];
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) vals[e] = n0 + nc * 8 + e < g.HD ? src[e] : T(0);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) vals[e] = T(0);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) sm.bt[(nc * 8 + e) * LD + kr] = vals[e];
        }
        __syncthreads();
        PFrag<T> af[4], bfr[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) pload(af[a], &sm.a[(64 * wave + 16 * a + r16) * LD + 8 * grp]);
#pragma unroll
        for (int b = 0; b < 4; ++b) pload(bfr[b], &sm.bt[(16 * b + r16) * LD + 8 * grp]);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) pmma(acc[a][b], af[a], bfr[b]);
    }
    // D[m = 16a + 4grp + j][n = 16b + r16]
    float* out = part + ((size_t)(split * 2 + z) * g.r) * g.HD;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int m = m0 + 64 * wave + 16 * a + 4 * grp + j;
            if (m >= g.r) continue;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int n = n0 + 16 * b + r16;
                if (n < g.HD) out[(size_t)m * g.HD + n] = acc[a][b][j];
            }
        }
}

// Sum the split partials in split order; write K', V' (f32, optional) and
// the attention operands: bf16 hi + lo pair, or the f32 values. Four
// consecutive elements per thread (r H d is a multiple of 64), eight split
// loads in flight; the sums still run in split order.
template <typename T>
__global__ void __launch_bounds__(256)
k_lowrank_reduce(int nsplit, long long n_per_z, const float* __restrict__ part,
                 float* __restrict__ k_low, float* __restrict__ v_low, T* __restrict__ k_hi,
                 T* __restrict__ v_hi, T* __restrict__ k_lo, T* __restrict__ v_lo) {
    const long long idx = ((long long)blockIdx.x * blockDim.x + threadIdx.x) * 4;
    if (idx >= 2 * n_per_z) return;
    const int z = idx >= n_per_z;
    const long long e = idx - z * n_per_z;
    const float* src = part + (long long)z * n_per_z + e;
    const long long stride = 2 * n_per_z;   // next split, same z
    float4 s = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < nsplit; k0 += 8) {
        float4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (k0 + u < nsplit) v[u] = *reinterpret_cast<const float4*>(src + (long long)(k0 + u) * stride);
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (k0 + u < nsplit) {
                s.x += v[u].x; s.y += v[u].y; s.z += v[u].z; s.w += v[u].w;
            }
    }
    float* low = z ? v_low : k_low;
    if (low) *reinterpret_cast<float4*>(low + e) = s;
    T* hi = z ? v_hi : k_hi;
    if constexpr (sizeof(T) == 2) {
        const float sv[4] = {s.x, s.y, s.z, s.w};
        bf16_t h[4], l[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            h[c] = f32_to_bf16(sv[c]);
            l[c] = f32_to_bf16(sv[c] - bf16_to_f32(h[c]));
        }
        uint2 ph, pl;
        ph.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16); ph.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
        pl.x = (uint32_t)l[0] | ((uint32_t)l[1] << 16); pl.y = (uint32_t)l[2] | ((uint32_t)l[3] << 16);
        *reinterpret_cast<uint2*>(hi + e) = ph;
        *reinterpret_cast<uint2*>((z ? v_lo : k_lo) + e) = pl;
    } else {
        *reinterpret_cast<float4*>(hi + e) = s;
    }
}

// ---------------------------------------------------------------------------
// Gated fusion: one wave per (token, head) row.
template <typename T>
__global__ void __launch_bounds__(256)
k_fuse(Geo g, const T* __restrict__ q, const float* __restrict__ w_g, const float* __restrict__ b_g,
       const float* __restrict__ o_s, const float* __restrict__ o_l, T* __restrict__ out,
       float* __restrict__ gate_out) {
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= (long long)g.Lq * g.H) return;
    const int lane = threadIdx.x & 63;
    const int h = (int)(row % g.H);
    const long long base = row * g.d;
    float dot = 0.f;
    for (int e = lane; e < g.d; e += 64) dot = fmaf(Elt<T>::to_f32(q[base + e]), w_g[h * g.d + e], dot);
    dot = wave_sum(dot);
    const float x = dot + b_g[h];
    const float zz = expf(-fabsf(x));
    const float gt = x >= 0.f ? 1.0f / (1.0f + zz) : zz / (1.0f + zz);
    if (gate_out && lane == 0) gate_out[row] = gt;
    for (int e = lane; e < g.d; e += 64) {
        const float v = gt * o_s[base + e] + (1.f - gt) * o_l[base + e];
        out[base + e] = Elt<T>::from_f32(v);
    }
}

}  // namespace

int lowrank_splits(const Geo& g) {
    if (proj32_eligible(g)) return proj32_splits(g);
    const int tiles = ((g.HD + PBN - 1) / PBN) * ((g.r + PBM - 1) / PBM) * 2;
    int s = (512 + tiles - 1) / tiles;
    if (s < 1) s = 1;
    if (s > 32) s = 32;
    return s;
}

template <typename T>
void launch_lowrank_proj(const Geo& g, const void* E, const void* F, const void* k_hist,
                         const void* v_hist, const void* k_intra, const void* v_intra,
                         const int32_t* n_sel, float* part, hipStream_t st) {
    if (sizeof(T) == 2 && proj32_eligible(g)) {
        launch_lowrank_proj32(g, E, F, k_hist, v_hist, k_intra, v_intra, n_sel, part, st);
        return;
    }
    const int ns = lowrank_splits(g);
    dim3 grid((g.HD + PBN - 1) / PBN, (g.r + PBM - 1) / PBM, ns * 2);
    hipLaunchKernelGGL(k_lowrank_proj<T>, grid, dim3(kProjThreads), 0, st, g, (const T*)E,
                       (const T*)F, (const T*)k_hist, (const T*)v_hist, (const T*)k_intra,
                       (const T*)v_intra, n_sel, ns, part);
}

template <typename T>
void launch_lowrank_reduce(const Geo& g, const float* part, float* k_low, float* v_low, void* k_hi,
                           void* v_hi, void* k_lo, void* v_lo, hipStream_t st) {
    const long long n = (long long)g.r * g.HD;
    const long long blocks = (2 * n / 4 + 255) / 256;   // four elements per thread
    hipLaunchKernelGGL(k_lowrank_reduce<T>, dim3((unsigned)blocks), dim3(256), 0, st,
                       lowrank_splits(g), n, part, k_low, v_low, (T*)k_hi, (T*)v_hi, (T*)k_lo,
                       (T*)v_lo);
}

template <typename T>
void launch_fuse(const Geo& g, const void* q, const float* w_g, const float* b_g, const float* o_s,
                 const float* o_l, void* out, float* gate, hipStream_t st) {
    const long long rows = (long long)g.Lq * g.H;
    hipLaunchKernelGGL(k_fuse<T>, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, g,
                       (const T*)q, w_g, b_g, o_s, o_l, (T*)out, gate);
}

#define HSAKV_INST(T)                                                                              \
    template void launch_lowrank_proj<T>(const Geo&, const void*, const void*, const void*,       \
                                         const void*, const void*, const void*, const int32_t*,   \
                                         float*, hipStream_t);                                    \
    template void launch_lowrank_reduce<T>(const Geo&, const float*, float*, float*, void*, void*, \
                                           void*, void*, hipStream_t);                            \
    template void launch_fuse<T>(const Geo&, const void*, const float*, const float*,             \
                                 const float*, const float*, void*, float*, hipStream_t);
HSAKV_INST(float)
HSAKV_INST(bf16_t)
#undef HSAKV_INST
