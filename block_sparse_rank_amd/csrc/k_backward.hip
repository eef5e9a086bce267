// Backward of the learned parameters of HSA: the gates (w_g, b_g) and the
// Linformer projections E and F (pages: WorldAttention news summary, HSA
// paragraph: the two branches are fused by learned gates and the global
// branch is a Linformer-style low-rank projection; the Linformer paper on the
// citation map). The sparse branch has no learned parameter.
//
// For an upstream gradient dO of the fused output, per token t and head h:
//   g = sigmoid(<q, w_g[h]> + b_g[h]),  dx = <dO, O_s - O_l> g (1 - g)
//   dw_g[h] = sum_t dx q,  db_g[h] = sum_t dx
//   dO_l = (1 - g) dO,  D_t = <dO_l, O_l>
// and per head for the low-rank branch (P = softmax(q K'^T / sqrt d)):
//   dV' = P^T dO_l,  dK' = (P * (dO_l V'^T - D)) ^T q / sqrt d
//   dE = sum_h dK'_h K_h^T,  dF = sum_h dV'_h V_h^T
// with E and F columns of absent history slots getting zero.
//
// Kernels (bf16 storage, float32 arithmetic):
//   k_bwd_gate       one wave per (t, h): dx, dO_l, D
//   k_bwd_gate_sum   one work-group per head: dw_g, db_g over tokens in a fixed order
//   k_bwd_lse        one work-group per (head, 64 queries): log-sum-exp of each query's logits
//   k_bwd_lowrank    one work-group per (head, 32 projected keys, query slice): partial dK', dV'
//   k_bwd_lowrank_sum  partials added in slice order; dK', dV' also as bf16 hi + lo pairs
//   k_bwd_proj       dE, dF = dK' K^T, dV' V^T on 32x32x16 bf16 MFMA (hi and lo products)
#include "common.h"
#include "launch.h"

namespace {

constexpr int kSlices = 8;          // query slices of the low-rank backward
constexpr int kKeyTile = 32;        // projected keys per work-group

HSAKV_DEV float gate_of(float x) {
    const float z = expf(-fabsf(x));
    return x >= 0.f ? 1.0f / (1.0f + z) : z / (1.0f + z);
}

// One wave per (t, h); lanes take the head's columns e = lane, lane + 64.
__global__ void __launch_bounds__(256)
k_bwd_gate(Geo g, const bf16_t* __restrict__ q, const float* __restrict__ w_g, const float* __restrict__ b_g,
           const float* __restrict__ o_s, const float* __restrict__ o_l, const bf16_t* __restrict__ d_out,
           float* __restrict__ dx, float* __restrict__ dol, float* __restrict__ Dt) {
    const int lane = threadIdx.x & 63;
    const long long item = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= (long long)g.Lq * g.H) return;
    const int h = (int)(item % g.H);
    const long long base = item * g.d;            // (t * H + h) * d
    float xw = 0.f, dg = 0.f;
    for (int e = lane; e < g.d; e += 64) {
        xw = fmaf(bf16_to_f32(q[base + e]), w_g[h * g.d + e], xw);
        dg = fmaf(bf16_to_f32(d_out[base + e]), o_s[base + e] - o_l[base + e], dg);
    }
    xw = wave_sum(xw);
    dg = wave_sum(dg);
    const float gv = gate_of(xw + b_g[h]);
    float dd = 0.f;
    for (int e = lane; e < g.d; e += 64) {
        const float v = (1.0f - gv) * bf16_to_f32(d_out[base + e]);
        dol[base + e] = v;
        dd = fmaf(v, o_l[base + e], dd);
    }
    dd = wave_sum(dd);
    if (lane == 0) {
        dx[item] = dg * gv * (1.0f - gv);
        Dt[item] = dd;
    }
}

// dw_g[h][e] = sum_t dx[t][h] q[t][h][e], db_g[h] = sum_t dx[t][h]: 256
// threads, column e = tid % d, token group tid / d takes t = grp, grp + G,
// ...; the G group sums are added in group order.
__global__ void __launch_bounds__(256)
k_bwd_gate_sum(Geo g, const bf16_t* __restrict__ q, const float* __restrict__ dx, float* __restrict__ d_wg,
               float* __restrict__ d_bg) {
    __shared__ float pw[256], pb[256];
    const int h = blockIdx.x;
    const int e = threadIdx.x % g.d, grp = threadIdx.x / g.d, G = 256 / g.d;
    float sw = 0.f, sb = 0.f;
    for (int t = grp; t < g.Lq; t += G) {
        const float x = dx[(long long)t * g.H + h];
        sw = fmaf(x, bf16_to_f32(q[((long long)t * g.H + h) * g.d + e]), sw);
        sb += x;
    }
    pw[threadIdx.x] = sw;
    pb[threadIdx.x] = sb;
    __syncthreads();
    if (threadIdx.x < g.d) {
        float a = 0.f, b = 0.f;
        for (int k = 0; k < G; ++k) {
            a += pw[k * g.d + threadIdx.x];
            b += pb[k * g.d + threadIdx.x];
        }
        d_wg[h * g.d + threadIdx.x] = a;
        if (threadIdx.x == 0) d_bg[h] = b;
    }
}

// Log-sum-exp of q_t K'^T / sqrt d over the r projected keys: one
// work-group per (head, 64 queries), 4 threads per query (a quarter of the
// head's columns each, summed by lane shuffles), online max and sum.
template <int D>
__global__ void __launch_bounds__(256)
k_bwd_lse(Geo g, const bf16_t* __restrict__ q, const float* __restrict__ k_low, float* __restrict__ lse) {
    const int h = blockIdx.y;
    const int qi = threadIdx.x >> 2, quarter = threadIdx.x & 3;
    const int t = blockIdx.x * 64 + qi;
    constexpr int dq = D / 4;
    const bool ok = t < g.Lq;
    float qv[dq];
#pragma unroll
    for (int k = 0; k < dq; ++k)
        qv[k] = ok ? bf16_to_f32(q[((long long)t * g.H + h) * g.d + quarter * dq + k]) : 0.f;
    const float scale = 1.0f / sqrtf((float)D);
    float m = -INFINITY, l = 0.f;
    for (int j = 0; j < g.r; ++j) {
        const float* kr = k_low + ((long long)j * g.H + h) * g.d + quarter * dq;
        float s = 0.f;
#pragma unroll
        for (int k = 0; k < dq; ++k) s = fmaf(qv[k], kr[k], s);
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        s *= scale;
        const float mn = fmaxf(m, s);
        l = l * expf(m - mn) + expf(s - mn);
        m = mn;
    }
    if (ok && quarter == 0) lse[(long long)t * g.H + h] = m + logf(l);
}

// Partial dK', dV' of 32 projected keys over one query slice: 256 threads =
// 32 keys x 8 column groups (d / 8 columns each); per query the two dots are
// summed over the 8 threads of a key by lane shuffles, in a fixed order.
template <int D>
__global__ void __launch_bounds__(256)
k_bwd_lowrank(Geo g, const bf16_t* __restrict__ q, const float* __restrict__ k_low,
              const float* __restrict__ v_low, const float* __restrict__ dol, const float* __restrict__ lse,
              const float* __restrict__ Dt, float* __restrict__ pk, float* __restrict__ pv) {
    const int h = blockIdx.y, slice = blockIdx.z;
    const int jl = threadIdx.x >> 3, cg = threadIdx.x & 7;
    const int j = blockIdx.x * kKeyTile + jl;
    constexpr int dc = D / 8;
    const bool ok = j < g.r;
    const long long kro = ((long long)(ok ? j : 0) * g.H + h) * D + cg * dc;
    float kj[dc], vj[dc], ak[dc], av[dc];
#pragma unroll
    for (int k = 0; k < dc; ++k) {
        kj[k] = k_low[kro + k];
        vj[k] = v_low[kro + k];
        ak[k] = 0.f;
        av[k] = 0.f;
    }
    const float scale = 1.0f / sqrtf((float)D);
    const int per = (g.Lq + kSlices - 1) / kSlices;
    const int t0 = slice * per, t1 = t0 + per < g.Lq ? t0 + per : g.Lq;
    for (int t = t0; t < t1; ++t) {
        const long long ro = ((long long)t * g.H + h) * D + cg * dc;
        float qv[dc], dv[dc];
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int k = 0; k < dc; ++k) {
            qv[k] = bf16_to_f32(q[ro + k]);
            dv[k] = dol[ro + k];
            s = fmaf(qv[k], kj[k], s);
            dp = fmaf(dv[k], vj[k], dp);
        }
        s += __shfl_xor(s, 1, 64);
        s += __shfl_xor(s, 2, 64);
        s += __shfl_xor(s, 4, 64);
        dp += __shfl_xor(dp, 1, 64);
        dp += __shfl_xor(dp, 2, 64);
        dp += __shfl_xor(dp, 4, 64);
        const long long th = (long long)t * g.H + h;
        const float p = expf(s * scale - lse[th]);
        const float ds = p * (dp - Dt[th]) * scale;
#pragma unroll
        for (int k = 0; k < dc; ++k) {
            av[k] = fmaf(p, dv[k], av[k]);
            ak[k] = fmaf(ds, qv[k], ak[k]);
        }
    }
    if (!ok) return;
    const long long o = (((long long)slice * g.r + j) * g.H + h) * D + cg * dc;
#pragma unroll
    for (int k = 0; k < dc; ++k) {
        pk[o + k] = ak[k];
        pv[o + k] = av[k];
    }
}

// dK', dV' = sum of the slice partials in slice order; also stored as bf16
// hi + lo pairs (hi = the rounded value, lo = the rounded remainder) for the
// projection products.
__global__ void __launch_bounds__(256)
k_bwd_lowrank_sum(long long n, const float* __restrict__ pk, const float* __restrict__ pv,
                  float* __restrict__ dk, float* __restrict__ dv, bf16_t* __restrict__ khi, bf16_t* __restrict__ klo,
                  bf16_t* __restrict__ vhi, bf16_t* __restrict__ vlo) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int s = 0; s < kSlices; ++s) {
        a += pk[s * n + i];
        b += pv[s * n + i];
    }
    if (dk) dk[i] = a;
    if (dv) dv[i] = b;
    const bf16_t ah = f32_to_bf16(a), bh = f32_to_bf16(b);
    khi[i] = ah;
    klo[i] = f32_to_bf16(a - bf16_to_f32(ah));
    vhi[i] = bh;
    vlo[i] = f32_to_bf16(b - bf16_to_f32(bh));
}

// dE (z = 0) or dF (z = 1) = dK' K_act^T (dV' V_act^T), written at the E/F
// columns of the active keys, zeros at the columns of absent slots. One
// work-group of 4 waves per (64 columns, 256 rows of r); wave w owns rows
// 64 w .. 64 w + 63 of its row tile as 2 x 2 tiles of 32 x 32. The
// contraction runs over the H d columns of the key rows, 16 at a time,
// with the hi and lo parts of dK' as two products into one accumulator.
// Operands are read straight from memory: A (dK' hi, lo rows) and B (key
// rows, 16 bytes per lane) are 16-byte loads.
__global__ void __launch_bounds__(256)
k_bwd_proj(Geo g, const bf16_t* __restrict__ k_hist, const bf16_t* __restrict__ v_hist,
           const bf16_t* __restrict__ k_intra, const bf16_t* __restrict__ v_intra, const int32_t* __restrict__ n_sel_p,
           const bf16_t* __restrict__ khi, const bf16_t* __restrict__ klo, const bf16_t* __restrict__ vhi,
           const bf16_t* __restrict__ vlo, float* __restrict__ dE, float* __restrict__ dF) {
    const int z = blockIdx.z;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int l32 = lane & 31, g2 = lane >> 5;
    int ns = *n_sel_p;
    ns = ns < 0 ? 0 : (ns > g.Kp ? g.Kp : ns);
    const long long Lh = (long long)ns * g.Tp;
    const bf16_t* hist = z ? v_hist : k_hist;
    const bf16_t* intra = z ? v_intra : k_intra;
    const bf16_t* ahi = z ? vhi : khi;
    const bf16_t* alo = z ? vlo : klo;
    float* out = z ? dF : dE;
    const long long c0 = (long long)blockIdx.x * 64;
    const int m0 = blockIdx.y * 256 + wave * 64;
    // B rows: columns c0 + 32 nt + l32 of E/F -> a key row, or none
    const bf16_t* brow[2];
    bool bok[2];
    for (int nt = 0; nt < 2; ++nt) {
        const long long c = c0 + 32 * nt + l32;
        bok[nt] = true;
        if (c < Lh) brow[nt] = hist + c * g.HD;
        else if (c >= g.hist_rows && c < g.L) brow[nt] = intra + (c - g.hist_rows) * g.HD;
        else {
            brow[nt] = hist;
            bok[nt] = false;
        }
    }
    const bf16_t* arow_hi[2];
    const bf16_t* arow_lo[2];
    for (int mt = 0; mt < 2; ++mt) {
        const int m = m0 + 32 * mt + l32;
        const int mc = m < g.r ? m : g.r - 1;
        arow_hi[mt] = ahi + (long long)mc * g.HD;
        arow_lo[mt] = alo + (long long)mc * g.HD;
    }
    f32x16_t acc[2][2];
    for (int mt = 0; mt < 2; ++mt)
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x16_t{};
    const bf16x8_t zero8 = {};
#pragma unroll 4
    for (int k0 = 0; k0 < g.HD; k0 += 16) {
        const int ko = k0 + 8 * g2;
        bf16x8_t a_hi[2], a_lo[2], b[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
            a_hi[mt] = *reinterpret_cast<const bf16x8_t*>(arow_hi[mt] + ko);
            a_lo[mt] = *reinterpret_cast<const bf16x8_t*>(arow_lo[mt] + ko);
        }
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) b[nt] = bok[nt] ? *reinterpret_cast<const bf16x8_t*>(brow[nt] + ko) : zero8;
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt) {
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_hi[mt], b[nt], acc[mt][nt], 0, 0, 0);
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_lo[mt], b[nt], acc[mt][nt], 0, 0, 0);
            }
    }
    // element i of a 32 x 32 tile: row 8 (i / 4) + 4 g2 + i % 4, column l32
    for (int mt = 0; mt < 2; ++mt)
        for (int nt = 0; nt < 2; ++nt) {
            const long long c = c0 + 32 * nt + l32;
            if (c >= g.L) continue;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = m0 + 32 * mt + 8 * (i >> 2) + 4 * g2 + (i & 3);
                if (m < g.r) out[(long long)m * g.L + c] = acc[mt][nt][i];
            }
        }
}

}  // namespace

size_t backward_ws_bytes(const Geo& g) {
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t th = (size_t)g.Lq * g.H, rhd = (size_t)g.r * g.HD;
    return al(th * 4) * 3 + al(th * g.d * 4) + 2 * al(kSlices * rhd * 4) + 2 * al(rhd * 4) + 4 * al(rhd * 2);
}

void launch_backward_params(const Geo& g, const void* q, const void* k_hist, const void* v_hist,
                            const void* k_intra, const void* v_intra, const int32_t* n_sel, const float* w_g,
                            const float* b_g, const float* k_low, const float* v_low, const float* o_s,
                            const float* o_l, const void* d_out, float* d_wg, float* d_bg, float* d_E, float* d_F,
                            void* ws, hipStream_t st) {
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t th = (size_t)g.Lq * g.H, rhd = (size_t)g.r * g.HD;
    char* p = (char*)ws;
    float* dx = (float*)p; p += al(th * 4);
    float* Dt = (float*)p; p += al(th * 4);
    float* lse = (float*)p; p += al(th * 4);
    float* dol = (float*)p; p += al(th * g.d * 4);
    float* pk = (float*)p; p += al(kSlices * rhd * 4);
    float* pv = (float*)p; p += al(kSlices * rhd * 4);
    float* dk = (float*)p; p += al(rhd * 4);
    float* dv = (float*)p; p += al(rhd * 4);
    bf16_t* khi = (bf16_t*)p; p += al(rhd * 2);
    bf16_t* klo = (bf16_t*)p; p += al(rhd * 2);
    bf16_t* vhi = (bf16_t*)p; p += al(rhd * 2);
    bf16_t* vlo = (bf16_t*)p;
    const bf16_t* qb = (const bf16_t*)q;
    hipLaunchKernelGGL(k_bwd_gate, dim3((unsigned)((th + 3) / 4)), dim3(256), 0, st, g, qb, w_g, b_g, o_s, o_l,
                       (const bf16_t*)d_out, dx, dol, Dt);
    hipLaunchKernelGGL(k_bwd_gate_sum, dim3(g.H), dim3(256), 0, st, g, qb, (const float*)dx, d_wg, d_bg);
    const dim3 lse_grid((g.Lq + 63) / 64, g.H), low_grid((g.r + kKeyTile - 1) / kKeyTile, g.H, kSlices);
    if (g.d == 128) {
        hipLaunchKernelGGL(k_bwd_lse<128>, lse_grid, dim3(256), 0, st, g, qb, k_low, lse);
        hipLaunchKernelGGL(k_bwd_lowrank<128>, low_grid, dim3(256), 0, st, g, qb, k_low, v_low, (const float*)dol,
                           (const float*)lse, (const float*)Dt, pk, pv);
    } else {
        hipLaunchKernelGGL(k_bwd_lse<64>, lse_grid, dim3(256), 0, st, g, qb, k_low, lse);
        hipLaunchKernelGGL(k_bwd_lowrank<64>, low_grid, dim3(256), 0, st, g, qb, k_low, v_low, (const float*)dol,
                           (const float*)lse, (const float*)Dt, pk, pv);
    }
    hipLaunchKernelGGL(k_bwd_lowrank_sum, dim3((unsigned)((rhd + 255) / 256)), dim3(256), 0, st, (long long)rhd,
                       (const float*)pk, (const float*)pv, dk, dv, khi, klo, vhi, vlo);
    hipLaunchKernelGGL(k_bwd_proj, dim3((unsigned)((g.L + 63) / 64), (g.r + 255) / 256, 2), dim3(256), 0, st, g,
                       (const bf16_t*)k_hist, (const bf16_t*)v_hist, (const bf16_t*)k_intra,
                       (const bf16_t*)v_intra, n_sel, (const bf16_t*)khi, (const bf16_t*)klo,
                       (const bf16_t*)vhi, (const bf16_t*)vlo, d_E, d_F);
}
