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
// Every float32 operand of a bf16 MFMA product is split into hi = bf16(x)
// and lo = bf16(x - hi), which keeps about 16 mantissa bits; q and the keys
// and values are bf16 already. Every sum runs in a fixed order, so results
// are the same bits from run to run.
//
// Kernels:
//   k_bwd_gate        d / 8 lanes per (t, h): dx, D_t, dO_l as a hi + lo pair
//   k_bwd_gate_part   per (head, token slice): partial dw_g, db_g
//   k_bwd_gate_fin    per head: the slice partials in slice order
//   k_bwd_split       K', V' -> hi + lo pairs
//   k_bwd_lse         per (head, 256 queries): log2-sum-exp2 of each query's
//                     scaled logits over the r projected keys (MFMA)
//   k_bwd_lowrank     per (128 projected keys, head, query slice): partial
//                     dK', dV' on MFMA, queries streamed through LDS
//   k_bwd_lowrank_sum the slice partials in slice order -> dK', dV' hi + lo
//   k_bwd_proj        dE, dF = dK' K^T, dV' V^T: 256-row tiles of 448 columns, the
//                     contraction over H d through a 3-stage LDS DMA ring
#include "common.h"
#include "launch.h"

namespace {

typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr int kGateSlices = 64;     // token slices of the gate-parameter sums
constexpr int kKeyGroup = 128;      // projected keys per low-rank work-group (4 waves x 32)
constexpr float kLog2e = 1.4426950408889634f;

HSAKV_DEV float gate_of(float x) {
    const float z = expf(-fabsf(x));
    return x >= 0.f ? 1.0f / (1.0f + z) : z / (1.0f + z);
}

HSAKV_DEV void split_bf16(float x, bf16_t& hi, bf16_t& lo) {
    hi = f32_to_bf16(x);
    lo = f32_to_bf16(x - bf16_to_f32(hi));
}

HSAKV_DEV bf16x8_t ld8(const bf16_t* p) { return *reinterpret_cast<const bf16x8_t*>(p); }
HSAKV_DEV bf16x8_t ld8(const char* p) { return *reinterpret_cast<const bf16x8_t*>(p); }

HSAKV_DEV f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ---- gate terms -------------------------------------------------------------

// D / 8 lanes per (t, h), 8 columns each (16-byte loads); the dot products
// are summed over those lanes by a fixed xor tree.
template <int D>
__global__ void __launch_bounds__(256)
k_bwd_gate(Geo g, const bf16_t* __restrict__ q, const float* __restrict__ w_g, const float* __restrict__ b_g,
           const float* __restrict__ o_s, const float* __restrict__ o_l, const bf16_t* __restrict__ d_out,
           float* __restrict__ dx, bf16_t* __restrict__ dohi, bf16_t* __restrict__ dolo, float* __restrict__ Dt) {
    constexpr int LP = D / 8, IPB = 256 / LP;     // lanes per item, items per work-group
    const int sub = threadIdx.x % LP;
    const long long n = (long long)g.Lq * g.H;
    long long item = (long long)blockIdx.x * IPB + threadIdx.x / LP;
    const bool ok = item < n;
    item = ok ? item : n - 1;                     // every lane takes part in the shuffles
    const int h = (int)(item % g.H);
    const long long base = item * D + 8 * sub;    // (t * H + h) * d + 8 sub
    float qv[8], dv[8], os[8], ol[8], wv[8];
    Elt<bf16_t>::load8(q + base, qv);
    Elt<bf16_t>::load8(d_out + base, dv);
    Elt<float>::load8(o_s + base, os);
    Elt<float>::load8(o_l + base, ol);
    Elt<float>::load8(w_g + h * D + 8 * sub, wv);
    float xw = 0.f, dg = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        xw = fmaf(qv[e], wv[e], xw);
        dg = fmaf(dv[e], os[e] - ol[e], dg);
    }
#pragma unroll
    for (int o = LP / 2; o >= 1; o >>= 1) {
        xw += __shfl_xor(xw, o, 64);
        dg += __shfl_xor(dg, o, 64);
    }
    const float gv = gate_of(xw + b_g[h]);
    float dd = 0.f;
    bf16_t hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float v = (1.0f - gv) * dv[e];
        split_bf16(v, hi[e], lo[e]);
        dd = fmaf(v, ol[e], dd);
    }
#pragma unroll
    for (int o = LP / 2; o >= 1; o >>= 1) dd += __shfl_xor(dd, o, 64);
    if (!ok) return;
    auto pack = [](const bf16_t* x) {
        return uint4{x[0] | (uint32_t)x[1] << 16, x[2] | (uint32_t)x[3] << 16, x[4] | (uint32_t)x[5] << 16,
                     x[6] | (uint32_t)x[7] << 16};
    };
    *reinterpret_cast<uint4*>(dohi + base) = pack(hi);
    *reinterpret_cast<uint4*>(dolo + base) = pack(lo);
    if (sub == 0) {
        dx[item] = dg * gv * (1.0f - gv);
        Dt[item] = dd;
    }
}

// Partial sums of dw_g[h][e] = sum_t dx[t][h] q[t][h][e] and db_g[h] over
// the tokens of one slice: column e = tid % d, token group tid / d takes
// every (256 / d)-th token of the slice; the groups are added in order.
__global__ void __launch_bounds__(256)
k_bwd_gate_part(Geo g, const bf16_t* __restrict__ q, const float* __restrict__ dx, float* __restrict__ pw,
                float* __restrict__ pb) {
    __shared__ float sw_[256], sb_[256];
    const int h = blockIdx.x, slice = blockIdx.y;
    const int e = threadIdx.x % g.d, grp = threadIdx.x / g.d, G = 256 / g.d;
    const int per = (g.Lq + kGateSlices - 1) / kGateSlices;
    const int t0 = slice * per, t1 = t0 + per < g.Lq ? t0 + per : g.Lq;
    float sw = 0.f, sb = 0.f;
    for (int t = t0 + grp; t < t1; t += G) {
        const float x = dx[(long long)t * g.H + h];
        sw = fmaf(x, bf16_to_f32(q[((long long)t * g.H + h) * g.d + e]), sw);
        sb += x;
    }
    sw_[threadIdx.x] = sw;
    sb_[threadIdx.x] = sb;
    __syncthreads();
    if (threadIdx.x < g.d) {
        float a = 0.f, b = 0.f;
        for (int k = 0; k < G; ++k) {
            a += sw_[k * g.d + threadIdx.x];
            b += sb_[k * g.d + threadIdx.x];
        }
        pw[((long long)slice * g.H + h) * g.d + threadIdx.x] = a;
        if (threadIdx.x == 0) pb[slice * g.H + h] = b;
    }
}

__global__ void __launch_bounds__(128)
k_bwd_gate_fin(Geo g, const float* __restrict__ pw, const float* __restrict__ pb, float* __restrict__ d_wg,
               float* __restrict__ d_bg) {
    const int h = blockIdx.x, e = threadIdx.x;
    if (e >= g.d) return;
    float a = 0.f, b = 0.f;
#pragma unroll 16
    for (int s = 0; s < kGateSlices; ++s) {
        a += pw[((long long)s * g.H + h) * g.d + e];
        b += pb[s * g.H + h];
    }
    d_wg[h * g.d + e] = a;
    if (e == 0) d_bg[h] = b;
}

// ---- low-rank branch ----------------------------------------------------------

// K', V' (float32 [r][H][d]) -> hi + lo bf16 pairs, same layout.
__global__ void __launch_bounds__(256)
k_bwd_split(long long n, const float* __restrict__ kl, const float* __restrict__ vl, bf16_t* __restrict__ khi,
            bf16_t* __restrict__ klo, bf16_t* __restrict__ vhi, bf16_t* __restrict__ vlo) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    split_bf16(kl[i], khi[i], klo[i]);
    split_bf16(vl[i], vhi[i], vlo[i]);
}

// lse2[t][h] = log2 sum_j 2^(c s_j), c = log2(e) / sqrt(d), s_j = <q_t, K'_j>.
// Work-group = 4 waves x 64 queries of one head (two 32-query tiles per
// wave, so each K' fragment load serves two products). S^T = K' Q^T per
// 32-key tile (A = K' hi, lo rows; B = the wave's queries, held in
// registers); in the accumulator lane l holds query l % 32 of its tile and 16
// of the tile's keys, lane l + 32 the other 16. Online max and sum per lane
// pair.
template <int D>
__global__ void __launch_bounds__(256)
k_bwd_lse(Geo g, const bf16_t* __restrict__ q, const bf16_t* __restrict__ khi, const bf16_t* __restrict__ klo,
          float* __restrict__ lse2) {
    constexpr int KS = D / 16;
    const int h = blockIdx.y;
    const int lane = threadIdx.x & 63, l32 = lane & 31, g2 = lane >> 5;
    const int qbase = blockIdx.x * 256 + (threadIdx.x >> 6) * 64 + l32;
    bf16x8_t qf[2][KS];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int query = qbase + 32 * u;
        const bool ok = query < g.Lq;
        const bf16_t* qp = q + (long long)(ok ? query : 0) * g.HD + h * D + 8 * g2;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[u][ks] = ok ? ld8(qp + 16 * ks) : bf16x8_t{};
    }
    const float c = kLog2e / sqrtf((float)D);
    float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
    for (int j0 = 0; j0 < g.r; j0 += 32) {
        const long long ko = (long long)(j0 + l32) * g.HD + h * D + 8 * g2;
        f32x16_t s[2] = {f32x16_t{}, f32x16_t{}};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8_t kh = ld8(khi + ko + 16 * ks), kl = ld8(klo + ko + 16 * ks);
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                s[u] = mfma(kh, qf[u][ks], s[u]);
                s[u] = mfma(kl, qf[u][ks], s[u]);
            }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            float mx = s[u][0];
#pragma unroll
            for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[u][i]);
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c;
            const float mn = fmaxf(m[u], mx);
            float acc = l[u] * fast_exp2(m[u] - mn);
#pragma unroll
            for (int i = 0; i < 16; ++i) acc += fast_exp2(fmaf(s[u][i], c, -mn));
            l[u] = acc;
            m[u] = mn;
        }
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const float lt = l[u] + __shfl_xor(l[u], 32, 64);
        const int query = qbase + 32 * u;
        if (query < g.Lq && g2 == 0) lse2[(long long)query * g.H + h] = m[u] + __log2f(lt);
    }
}

// LDS tile of 32 queries: Q, dO_l hi, dO_l lo rows (bf16, padded rows for the
// transpose reads), then lse2 and D_t of the 32 queries.
template <int D>
struct BLay {
    static constexpr int CPR = D / 8;                 // 16-byte chunks per row
    static constexpr int PITCH = 16 * (CPR + 4);      // bytes per LDS row
    static constexpr int MAT = 32 * PITCH;
    static constexpr int OFF_LSE = 3 * MAT, OFF_DT = 3 * MAT + 128;
    static constexpr int BUF = 3 * MAT + 256;
    static constexpr int KS = D / 16, DT = D / 32;
    static constexpr int PER = 3 * 32 * CPR / 256;    // 16-byte chunks per thread and tile
    static_assert(32 * CPR % 256 == 0, "each tile splits evenly over the 256 threads");
};

// Partial dK', dV' of 128 projected keys (4 waves x 32) of one head over one
// slice of 32-query blocks. Per block, per wave:
//   S  = Q K'^T, dP = dO_l V'^T             (A = query rows from LDS, B = key rows in registers)
//   P  = 2^(c S - lse2), dS = P (dP - D) / sqrt d
//   dV' += P^T dO_l,  dK' += dS^T Q          (A = P, dS from their own lanes, B by transpose reads)
// In the S accumulator lane l holds key l % 32 and queries 8a + 4(l/32) + b
// (a, b = 0..3); a 16-query chunk c of those registers is the A operand with
// k order e < 4: query 16c + 4(l/32) + e, e >= 4: query 16c + 8 + 4(l/32) + e - 4,
// and ds_read_b64_tr_b16 of the row-major Q and dO_l tiles gives the B
// operand in the same query order. The next block's rows are loaded into
// registers while the current one is computed, then written to the other
// LDS buffer: one barrier per block.
template <int D>
__global__ void __launch_bounds__(256)
k_bwd_lowrank(Geo g, int nslices, const bf16_t* __restrict__ q, const bf16_t* __restrict__ dohi,
              const bf16_t* __restrict__ dolo, const float* __restrict__ lse2, const float* __restrict__ Dt,
              const bf16_t* __restrict__ khi, const bf16_t* __restrict__ klo, const bf16_t* __restrict__ vhi,
              const bf16_t* __restrict__ vlo, float* __restrict__ pk, float* __restrict__ pv) {
    using LY = BLay<D>;
    __shared__ __attribute__((aligned(16))) char lds[2 * LY::BUF];
    const int h = blockIdx.y, slice = blockIdx.z;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g2 = lane >> 5;
    const int G = lane >> 4, j = lane & 15;
    const int key0 = blockIdx.x * kKeyGroup + 32 * wave;
    const bool active = key0 < g.r;                   // whole wave: r is a multiple of 32
    const int nqb = (g.Lq + 31) / 32;
    const int per = (nqb + nslices - 1) / nslices;
    const int b0 = slice * per, b1 = b0 + per < nqb ? b0 + per : nqb;

    bf16x8_t kh[LY::KS], kl[LY::KS], vh[LY::KS], vl[LY::KS];
    {
        const long long ko = (long long)(active ? key0 + l32 : 0) * g.HD + h * D + 8 * g2;
#pragma unroll
        for (int ks = 0; ks < LY::KS; ++ks) {
            kh[ks] = ld8(khi + ko + 16 * ks);
            kl[ks] = ld8(klo + ko + 16 * ks);
            vh[ks] = ld8(vhi + ko + 16 * ks);
            vl[ks] = ld8(vlo + ko + 16 * ks);
        }
    }
    f32x16_t dk[LY::DT], dv[LY::DT];
#pragma unroll
    for (int dt = 0; dt < LY::DT; ++dt) {
        dk[dt] = f32x16_t{};
        dv[dt] = f32x16_t{};
    }

    // staged chunks: matrix m (Q, dO_l hi, dO_l lo), row / chunk from tid + 256 v
    constexpr int PM3 = LY::PER / 3;
    const int Lq = g.Lq, HD = g.HD, H = g.H;
    const bf16_t* const mats[3] = {q + h * D, dohi + h * D, dolo + h * D};
    uint4 st[3][PM3];
    float stl = 0.f;
    auto gload = [&](int b) {
        const int t0 = 32 * b;
#pragma unroll
        for (int m = 0; m < 3; ++m)
#pragma unroll
            for (int v = 0; v < PM3; ++v) {
                const int cidx = tid + 256 * v;
                const int t = t0 + cidx / LY::CPR, ch = cidx % LY::CPR;
                st[m][v] = t < Lq ? *reinterpret_cast<const uint4*>(mats[m] + (long long)t * HD + 8 * ch)
                                  : uint4{0, 0, 0, 0};
            }
        if (tid < 64) {
            const int t = t0 + (tid & 31);
            // a query past Lq gets weight 2^-huge = 0 and D = 0
            const float* src = tid < 32 ? lse2 : Dt;
            stl = t < Lq ? src[(long long)t * H + h] : (tid < 32 ? 3.0e38f : 0.f);
        }
    };
    auto swrite = [&](char* buf) {
#pragma unroll
        for (int m = 0; m < 3; ++m)
#pragma unroll
            for (int v = 0; v < PM3; ++v) {
                const int cidx = tid + 256 * v;
                *reinterpret_cast<uint4*>(buf + m * LY::MAT + (cidx / LY::CPR) * LY::PITCH + 16 * (cidx % LY::CPR)) =
                    st[m][v];
            }
        if (tid < 64) reinterpret_cast<float*>(buf + LY::OFF_LSE)[tid] = stl;
    };

    const float c = kLog2e / sqrtf((float)D);
    const float inv_sqrt_d = 1.0f / sqrtf((float)D);
    auto compute = [&](const char* buf) {
        f32x16_t s = {}, dp = {};
        const char* arow = buf + l32 * LY::PITCH + 16 * g2;
#pragma unroll
        for (int ks = 0; ks < LY::KS; ++ks) {
            const bf16x8_t a = ld8(arow + 32 * ks);
            s = mfma(a, kh[ks], s);
            s = mfma(a, kl[ks], s);
            const bf16x8_t ah = ld8(arow + LY::MAT + 32 * ks);
            const bf16x8_t al = ld8(arow + 2 * LY::MAT + 32 * ks);
            dp = mfma(ah, vh[ks], dp);
            dp = mfma(al, vh[ks], dp);
            dp = mfma(ah, vl[ks], dp);
        }
        const float* ls = reinterpret_cast<const float*>(buf + LY::OFF_LSE);
        const float* dd = reinterpret_cast<const float*>(buf + LY::OFF_DT);
        bf16x8_t ph[2], pl[2], sh[2], sl[2];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int qi = 8 * (i >> 2) + 4 * g2 + (i & 3);
            const float p = fast_exp2(fmaf(s[i], c, -ls[qi]));
            const float ds = p * (dp[i] - dd[qi]) * inv_sqrt_d;
            const __bf16 p_hi = (__bf16)p, s_hi = (__bf16)ds;
            ph[i >> 3][i & 7] = p_hi;
            pl[i >> 3][i & 7] = (__bf16)(p - (float)p_hi);
            sh[i >> 3][i & 7] = s_hi;
            sl[i >> 3][i & 7] = (__bf16)(ds - (float)s_hi);
        }
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
            const int krow = 16 * cc + 4 * (G >> 1) + (j >> 2);
#pragma unroll
            for (int dt = 0; dt < LY::DT; ++dt) {
                const int off = krow * LY::PITCH + 2 * (32 * dt + 16 * (G & 1) + 4 * (j & 3));
                bf16x8_t b[3];
#pragma unroll
                for (int m = 0; m < 3; ++m) {
                    const char* p = buf + m * LY::MAT + off;
                    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p);
                    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p + 8 * LY::PITCH));
                    b[m] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                }
                dv[dt] = mfma(ph[cc], b[1], dv[dt]);
                dv[dt] = mfma(pl[cc], b[1], dv[dt]);
                dv[dt] = mfma(ph[cc], b[2], dv[dt]);
                dk[dt] = mfma(sh[cc], b[0], dk[dt]);
                dk[dt] = mfma(sl[cc], b[0], dk[dt]);
            }
        }
    };

    if (b0 < b1) {
        gload(b0);
        swrite(lds);
    }
    __syncthreads();
    for (int b = b0; b < b1; ++b) {
        const int k = b - b0;
        if (b + 1 < b1) gload(b + 1);
        if (active) compute(lds + (k & 1) * LY::BUF);
        if (b + 1 < b1) swrite(lds + ((k + 1) & 1) * LY::BUF);
        __syncthreads();
    }
    if (!active) return;
    // accumulator element i: key key0 + 8 (i / 4) + 4 g2 + i % 4, column 32 dt + l32
#pragma unroll
    for (int dt = 0; dt < LY::DT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int key = key0 + 8 * (i >> 2) + 4 * g2 + (i & 3);
            const long long o = (((long long)slice * g.r + key) * g.H + h) * D + 32 * dt + l32;
            pk[o] = dk[dt][i];
            pv[o] = dv[dt][i];
        }
}

// dK', dV' = sum of the slice partials in slice order, as hi + lo pairs.
__global__ void __launch_bounds__(256)
k_bwd_lowrank_sum(long long n, int nslices, const float* __restrict__ pk, const float* __restrict__ pv,
                  bf16_t* __restrict__ khi, bf16_t* __restrict__ klo, bf16_t* __restrict__ vhi,
                  bf16_t* __restrict__ vlo) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float a = 0.f, b = 0.f;
    for (int s = 0; s < nslices; ++s) {
        a += pk[s * n + i];
        b += pv[s * n + i];
    }
    split_bf16(a, khi[i], klo[i]);
    split_bf16(b, vhi[i], vlo[i]);
}

// ---- dE, dF --------------------------------------------------------------------

constexpr int QM = 256, QN = 256, QK = 32;   // tile rows (of r), key rows per step (columns of L), contraction step
constexpr int Q_ROW = QK * 2;                // bytes per LDS row: 4 chunks of 16, XOR-swizzled
constexpr int Q_AHI = 0, Q_ALO = QM * Q_ROW, Q_B = 2 * QM * Q_ROW;
constexpr int Q_STAGE = 2 * QM * Q_ROW + QN * Q_ROW;   // 48 KiB: 48 DMA instructions of 1 KiB
constexpr int Q_STAGES = 3;
constexpr int Q_WAVES = 8;
constexpr int Q_PER = Q_STAGE / 1024 / Q_WAVES;        // DMA instructions per wave and step
static_assert(Q_PER * Q_WAVES * 1024 == Q_STAGE && Q_AHI + 16 * 1024 == Q_ALO && Q_ALO + 16 * 1024 == Q_B,
              "instruction j of a step fills LDS bytes [1024 j, 1024 j + 1024) of its stage");

// chunk ch of row m sits at slot ch ^ ((m >> 2) & 3): the 8 lanes of one
// 128-byte LDS access (8 rows, one chunk each) hit distinct banks
HSAKV_DEV int pslot(int m, int ch) { return m * Q_ROW + 16 * (ch ^ ((m >> 2) & 3)); }

// Raw buffer resource over `bytes` from p (bytes < 2^31): loads past it read 0.
HSAKV_DEV __amdgpu_buffer_rsrc_t q_rsrc(const bf16_t* p, long long bytes) {
    const int n = bytes < 0 ? 0 : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(p), 0, n, 0x00020000);
}

// The LDS target of a DMA as a wave-uniform address the compiler cannot
// trace to the ring (the kernel orders each DMA before the reads of its step
// itself: a vmcnt wait, then the barrier).
HSAKV_DEV __attribute__((address_space(3))) void* q_dst(char* p) {
    const uint32_t v = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)p;
    return (__attribute__((address_space(3))) void*)(uintptr_t)__builtin_amdgcn_readfirstlane(v);
}

template <int N>
HSAKV_DEV void q_wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

// LDS-only work-group barrier (DMA in flight stays in flight).
HSAKV_DEV void q_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// dE (z = 0) or dF (z = 1) = dK' K_act^T (dV' V_act^T), written at the E/F
// columns of the active keys, zeros at the columns of absent slots.
// Work-group = 8 waves over QR = 448 columns of one part (history [0, Kp Tp)
// or chunk [Kp Tp, L)), taken as a 256-column chunk and then a 192-column
// one, so that the 2 x ceil(L / 448) work-groups of the 1.3B and 14B shapes
// run in a single round on 256 CUs (256-column tiles alone would need two,
// the second two-thirds full). In a chunk of 32 NTN columns per wave (NTN = 4
// or 3), wave w takes rows 64 (w % 4) and columns 32 NTN (w / 4), 2 x NTN MFMA
// tiles. A history chunk starting at or past the present rows n_sel Tp is all
// zero. The contraction over the H d columns of the key rows runs in
// 32-column steps through a 3-stage LDS ring filled by buffer-to-LDS DMA
// (dK' hi, dK' lo, 256 key rows; rows past r or past the chunk's present keys
// read as zero, and their products are zero), two steps in flight. The hi and
// lo parts of dK' are two products into one accumulator.
constexpr int QR = 448;   // columns per work-group: a 256-column chunk, then a 192-column one

template <int NTN>
HSAKV_DEV void bwd_proj_chunk(const Geo& g, char* ring, int z, int m0, long long c0, long long c_end, long long Lh,
                              bool hist, const bf16_t* __restrict__ k_hist, const bf16_t* __restrict__ v_hist,
                              const bf16_t* __restrict__ k_intra, const bf16_t* __restrict__ v_intra,
                              const bf16_t* __restrict__ khi, const bf16_t* __restrict__ klo,
                              const bf16_t* __restrict__ vhi, const bf16_t* __restrict__ vlo,
                              float* __restrict__ out) {
    const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, g2 = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave & 3, wn = wave >> 2;
    constexpr int CW = 64 * NTN;   // chunk columns
    if (hist && c0 >= Lh) {
        for (int i = tid; i < QM * CW; i += 512) {
            const int m = m0 + i / CW;
            const long long c = c0 + i % CW;
            if (m < g.r && c < c_end) out[(long long)m * g.L + c] = 0.f;
        }
        return;
    }
    const bf16_t* keys = hist ? (z ? v_hist : k_hist) + c0 * g.HD : (z ? v_intra : k_intra) + (c0 - g.hist_rows) * g.HD;
    const long long key_rows = (hist ? (Lh < c_end ? Lh : c_end) : c_end) - c0;
    const long long row_bytes = 2LL * g.HD;
    const __amdgpu_buffer_rsrc_t rb = q_rsrc(keys, key_rows * row_bytes);
    const __amdgpu_buffer_rsrc_t rh = q_rsrc((z ? vhi : khi) + (long long)m0 * g.HD, (g.r - m0) * row_bytes);
    const __amdgpu_buffer_rsrc_t rl = q_rsrc((z ? vlo : klo) + (long long)m0 * g.HD, (g.r - m0) * row_bytes);

    // Byte offsets of this wave's DMA instructions j = wave + 8 q: instruction
    // j fills LDS rows 16 (j % 16) .. + 15 of matrix j / 16 (dK' hi, lo, keys);
    // lane l fills slot l % 4 of row 16 (j % 16) + l / 4 with the chunk the
    // swizzle puts there.
    uint32_t off[Q_PER];
#pragma unroll
    for (int q = 0; q < Q_PER; ++q) {
        const int j = wave + Q_WAVES * q;
        const int row = 16 * (j & 15) + (lane >> 2);
        const int ch = (lane & 3) ^ ((row >> 2) & 3);
        off[q] = (uint32_t)(row * row_bytes + 16 * ch);
    }
    const int nk = g.HD / QK;
    auto send = [&](int st) __attribute__((always_inline)) {
        if (st >= nk) return;
        char* buf = ring + (st % Q_STAGES) * Q_STAGE;
        const uint32_t koff = (uint32_t)st * QK * 2;
#pragma unroll
        for (int q = 0; q < Q_PER; ++q) {
            const int j = wave + Q_WAVES * q;
            const __amdgpu_buffer_rsrc_t rs = q < 2 ? rh : q < 4 ? rl : rb;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, q_dst(buf + j * 1024), 16, off[q] + koff, 0, 0, 0);
        }
    };

    f32x16_t acc[2][NTN];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt) acc[mt][nt] = f32x16_t{};
    send(0);
    send(1);
#pragma unroll 1
    for (int k = 0; k < nk; ++k) {
        // step k has landed once only the step sent after it is outstanding
        if (k + 1 < nk)
            q_wait_vm<Q_PER>();
        else
            q_wait_vm<0>();
        q_barrier();
        send(k + 2);
        const char* buf = ring + (k % Q_STAGES) * Q_STAGE;
#pragma unroll
        for (int ks = 0; ks < QK / 16; ++ks) {
            const int ch = 2 * ks + g2;
            bf16x8_t ah[2], al[2], b[NTN];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const int row = 64 * wm + 32 * mt + l32;
                ah[mt] = ld8(buf + Q_AHI + pslot(row, ch));
                al[mt] = ld8(buf + Q_ALO + pslot(row, ch));
            }
#pragma unroll
            for (int nt = 0; nt < NTN; ++nt) b[nt] = ld8(buf + Q_B + pslot(32 * NTN * wn + 32 * nt + l32, ch));
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int nt = 0; nt < NTN; ++nt) {
                    acc[mt][nt] = mfma(ah[mt], b[nt], acc[mt][nt]);
                    acc[mt][nt] = mfma(al[mt], b[nt], acc[mt][nt]);
                }
        }
    }
    // every wave is done with the ring before a next chunk refills it
    q_barrier();

    // accumulator element i: row 8 (i / 4) + 4 g2 + i % 4, column l32 of its tile
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTN; ++nt) {
            const long long c = c0 + 32 * NTN * wn + 32 * nt + l32;
            if (c >= c_end) continue;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = m0 + 64 * wm + 32 * mt + 8 * (i >> 2) + 4 * g2 + (i & 3);
                if (m < g.r) out[(long long)m * g.L + c] = acc[mt][nt][i];
            }
        }
}

__global__ void __launch_bounds__(512, 1)
k_bwd_proj(Geo g, const bf16_t* __restrict__ k_hist, const bf16_t* __restrict__ v_hist,
           const bf16_t* __restrict__ k_intra, const bf16_t* __restrict__ v_intra, const int32_t* __restrict__ n_sel_p,
           const bf16_t* __restrict__ khi, const bf16_t* __restrict__ klo, const bf16_t* __restrict__ vhi,
           const bf16_t* __restrict__ vlo, float* __restrict__ dE, float* __restrict__ dF) {
    __shared__ __attribute__((aligned(16))) char ring[Q_STAGES * Q_STAGE];
    const int z = blockIdx.z;
    int ns = *n_sel_p;
    ns = ns < 0 ? 0 : (ns > g.Kp ? g.Kp : ns);
    const long long Lh = (long long)ns * g.Tp;
    float* out = z ? dF : dE;
    const int nhr = (int)((g.hist_rows + QR - 1) / QR);
    const bool hist = (int)blockIdx.x < nhr;
    const long long r0 = hist ? (long long)blockIdx.x * QR : g.hist_rows + (long long)(blockIdx.x - nhr) * QR;
    const long long part_end = hist ? g.hist_rows : g.L;
    const long long r1 = r0 + QR < part_end ? r0 + QR : part_end;
    const int m0 = blockIdx.y * QM;
    const long long e0 = r0 + 256 < r1 ? r0 + 256 : r1;
    bwd_proj_chunk<4>(g, ring, z, m0, r0, e0, Lh, hist, k_hist, v_hist, k_intra, v_intra, khi, klo, vhi, vlo, out);
    if (e0 < r1)
        bwd_proj_chunk<3>(g, ring, z, m0, e0, r1, Lh, hist, k_hist, v_hist, k_intra, v_intra, khi, klo, vhi, vlo,
                          out);
}

// Query slices of the low-rank backward: about one work-group per CU of a
// 256-CU part in total, a function of the sizes alone (so the summation
// order, and the result bits, do not depend on the device).
int lowrank_slices(const Geo& g) {
    const int groups = (g.r + kKeyGroup - 1) / kKeyGroup * g.H;
    const int nqb = (g.Lq + 31) / 32;
    int s = 256 / groups;
    s = s < 1 ? 1 : s;
    return s < nqb ? s : nqb;
}

struct BwdWs {
    float *dx, *Dt, *lse, *pw, *pb, *pk, *pv;
    bf16_t *dohi, *dolo, *khf, *klf, *vhf, *vlf, *dkhi, *dklo, *dvhi, *dvlo;
    size_t bytes;
};

// Workspace layout (each part 256-byte aligned); base null only sizes it.
BwdWs carve(const Geo& g, void* base) {
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t th = (size_t)g.Lq * g.H, rhd = (size_t)g.r * g.HD;
    const int ns = lowrank_slices(g);
    char* p = (char*)base;
    size_t off = 0;
    auto take = [&](size_t n) {
        char* r = p ? p + off : nullptr;
        off += al(n);
        return r;
    };
    BwdWs w;
    w.dx = (float*)take(th * 4);
    w.Dt = (float*)take(th * 4);
    w.lse = (float*)take(th * 4);
    w.pw = (float*)take((size_t)kGateSlices * g.H * g.d * 4);
    w.pb = (float*)take((size_t)kGateSlices * g.H * 4);
    w.dohi = (bf16_t*)take(th * g.d * 2);
    w.dolo = (bf16_t*)take(th * g.d * 2);
    w.khf = (bf16_t*)take(rhd * 2);
    w.klf = (bf16_t*)take(rhd * 2);
    w.vhf = (bf16_t*)take(rhd * 2);
    w.vlf = (bf16_t*)take(rhd * 2);
    w.pk = (float*)take((size_t)ns * rhd * 4);
    w.pv = (float*)take((size_t)ns * rhd * 4);
    w.dkhi = (bf16_t*)take(rhd * 2);
    w.dklo = (bf16_t*)take(rhd * 2);
    w.dvhi = (bf16_t*)take(rhd * 2);
    w.dvlo = (bf16_t*)take(rhd * 2);
    w.bytes = off;
    return w;
}

}  // namespace

size_t backward_ws_bytes(const Geo& g) { return carve(g, nullptr).bytes; }

hipError_t launch_backward_params(const Geo& g, const void* q, const void* k_hist, const void* v_hist,
                                  const void* k_intra, const void* v_intra, const int32_t* n_sel, const float* w_g,
                                  const float* b_g, const float* k_low, const float* v_low, const float* o_s,
                                  const float* o_l, const void* d_out, float* d_wg, float* d_bg, float* d_E,
                                  float* d_F, void* ws, hipStream_t st, hipStream_t side, hipEvent_t ev_fork,
                                  hipEvent_t ev_join) {
    const BwdWs w = carve(g, ws);
    const size_t th = (size_t)g.Lq * g.H, rhd = (size_t)g.r * g.HD;
    const bf16_t* qb = (const bf16_t*)q;
    const int ns = lowrank_slices(g);
    const bool split = side != st;
    hipError_t e = hipSuccess;

    // main: the K', V' split, the log-sum-exp and the gate terms, one after
    // another (on two streams they slowed each other down, and the low-rank
    // backward needs all three)
    hipLaunchKernelGGL(k_bwd_split, dim3((unsigned)((rhd + 255) / 256)), dim3(256), 0, st, (long long)rhd, k_low,
                       v_low, w.khf, w.klf, w.vhf, w.vlf);
    const dim3 lse_grid((g.Lq + 255) / 256, g.H), low_grid((g.r + kKeyGroup - 1) / kKeyGroup, g.H, ns);
    if (g.d == 128)
        hipLaunchKernelGGL(k_bwd_lse<128>, lse_grid, dim3(256), 0, st, g, qb, (const bf16_t*)w.khf,
                           (const bf16_t*)w.klf, w.lse);
    else
        hipLaunchKernelGGL(k_bwd_lse<64>, lse_grid, dim3(256), 0, st, g, qb, (const bf16_t*)w.khf,
                           (const bf16_t*)w.klf, w.lse);
    if (g.d == 128)
        hipLaunchKernelGGL(k_bwd_gate<128>, dim3((unsigned)((th + 15) / 16)), dim3(256), 0, st, g, qb, w_g, b_g, o_s,
                           o_l, (const bf16_t*)d_out, w.dx, w.dohi, w.dolo, w.Dt);
    else
        hipLaunchKernelGGL(k_bwd_gate<64>, dim3((unsigned)((th + 31) / 32)), dim3(256), 0, st, g, qb, w_g, b_g, o_s,
                           o_l, (const bf16_t*)d_out, w.dx, w.dohi, w.dolo, w.Dt);
    // side: the gate-parameter sums, once dx is there, beside the low-rank
    // backward and dE, dF (nothing after them on the main stream needs them)
    if (split && (e = hipEventRecord(ev_fork, st)) == hipSuccess) e = hipStreamWaitEvent(side, ev_fork, 0);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_bwd_gate_part, dim3(g.H, kGateSlices), dim3(256), 0, side, g, qb, (const float*)w.dx, w.pw,
                       w.pb);
    hipLaunchKernelGGL(k_bwd_gate_fin, dim3(g.H), dim3(128), 0, side, g, (const float*)w.pw, (const float*)w.pb,
                       d_wg, d_bg);
    if (split && (e = hipEventRecord(ev_join, side)) != hipSuccess) return e;

    // main: the low-rank backward, its slice sum, then dE and dF; the call's
    // stream waits for the sums at the end
    if (g.d == 128)
        hipLaunchKernelGGL(k_bwd_lowrank<128>, low_grid, dim3(256), 0, st, g, ns, qb, (const bf16_t*)w.dohi,
                           (const bf16_t*)w.dolo, (const float*)w.lse, (const float*)w.Dt, (const bf16_t*)w.khf,
                           (const bf16_t*)w.klf, (const bf16_t*)w.vhf, (const bf16_t*)w.vlf, w.pk, w.pv);
    else
        hipLaunchKernelGGL(k_bwd_lowrank<64>, low_grid, dim3(256), 0, st, g, ns, qb, (const bf16_t*)w.dohi,
                           (const bf16_t*)w.dolo, (const float*)w.lse, (const float*)w.Dt, (const bf16_t*)w.khf,
                           (const bf16_t*)w.klf, (const bf16_t*)w.vhf, (const bf16_t*)w.vlf, w.pk, w.pv);
    hipLaunchKernelGGL(k_bwd_lowrank_sum, dim3((unsigned)((rhd + 255) / 256)), dim3(256), 0, st, (long long)rhd, ns,
                       (const float*)w.pk, (const float*)w.pv, w.dkhi, w.dklo, w.dvhi, w.dvlo);
    const unsigned ranges = (unsigned)((g.hist_rows + QR - 1) / QR + (g.Lq + QR - 1) / QR);
    hipLaunchKernelGGL(k_bwd_proj, dim3(ranges, (g.r + QM - 1) / QM, 2), dim3(512), 0, st, g, (const bf16_t*)k_hist,
                       (const bf16_t*)v_hist, (const bf16_t*)k_intra, (const bf16_t*)v_intra, n_sel,
                       (const bf16_t*)w.dkhi, (const bf16_t*)w.dklo, (const bf16_t*)w.dvhi, (const bf16_t*)w.dvlo, d_E,
                       d_F);
    if (split) e = hipStreamWaitEvent(st, ev_join, 0);
    return e;
}
