// Low-rank branch attention, bf16, on gfx950 32x32x16 MFMA.
//
// Pages: WorldAttention news summary (ai4snews), HSA paragraph (a
// Linformer-style low-rank global branch, O(L r)); the projection is the
// Linformer paper's (cited on the mlsanity map). Every query attends, with
// exact softmax, to the r projected keys K' = E K_act with the projected
// values V' = F V_act of its head.
//
// K' and V' come as bf16 hi + lo pairs (hi = bf16(x), lo = bf16(x - hi)), so
// a product with them keeps about 16 mantissa bits:
//   S^T = K'_hi Q^T + K'_lo Q^T,   O^T += V'_hi^T P^T + V'_lo^T P^T.
//
// Work-group = 8 waves, 32 queries each: 256 consecutive queries of one head.
// The r keys stream through LDS in 64-key tiles (K'_hi, K'_lo, V'_hi, V'_lo),
// two buffers, the next tile's DMA in flight while the current one is
// computed. Rows are padded for conflict-free operand reads with plain base +
// immediate addresses: a K row holds its D/8 16-byte chunks and one pad slot,
// a V row its chunks and four pad slots (a DMA pad lane loads the row's first
// chunk again, into the pad). The DMA uses buffer loads whose resource ends at
// the tile's last valid key row, so rows past r read as zero; their scores
// are masked to -inf before the softmax.
//
// In the 32x32 accumulator layout lane l holds query l%32 and keys
// 8a + 4(l/32) + b (a, b = 0..3) of a 32-key half. A 16-key chunk c of those
// registers is the P^T operand with k order
//   e < 4: key 16c + 4(l/32) + e,   e >= 4: key 16c + 8 + 4(l/32) + e - 4
// and the V^T operand comes in the same key order from ds_read_b64_tr_b16
// transpose reads of the row-major V tile, so P never leaves its lane. Each
// 64-key tile is one online-softmax step (float32, exp2 with the log2(e)/
// sqrt(d) scale folded into the exponent's FMA; the running max raised only
// when a score passes it by more than 8 in log2 units, so O is rarely
// rescaled); the row sum is taken on the bf16 weights the MFMA consumes.
#include "common.h"
#include "launch.h"

namespace {

constexpr int LT = 64;        // keys per tile
constexpr int LW = 8;         // waves per work-group
constexpr int LQ = 32 * LW;   // queries per work-group

typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(8))) short i16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

template <int D>
struct LLay {
    static constexpr int CPR = D / 8;                     // 16-byte chunks per row
    static constexpr int KSL = CPR + 1, VSL = CPR + 4;    // LDS slots per K / V row
    static constexpr int KP = 16 * KSL, VP = 16 * VSL;    // LDS row pitches (bytes)
    static constexpr int KMAT = LT * KP, VMAT = LT * VP;
    // buffer: K'_hi, K'_lo, V'_hi, V'_lo
    static constexpr int KLO = KMAT, VHI = 2 * KMAT, VLO = 2 * KMAT + VMAT, BUF = 2 * KMAT + 2 * VMAT;
    static constexpr int NI = 2 * KSL + 2 * VSL;          // DMA instructions per tile (64 rows each)
    static constexpr int PER_WAVE = (NI + LW - 1) / LW;   // per wave, the last ones idle
    static constexpr int KS = D / 16, DT = D / 32;
};

template <int D>
struct LWave {
    bf16x8_t qf[LLay<D>::KS];
    f32x16_t o[LLay<D>::DT];
    float m, l;   // running max (log2 units), this lane's share of the row sum
};

// This wave's DMA instructions j = wave + LW q: matrix mat (0 K'_hi, 1 K'_lo,
// 2 V'_hi, 3 V'_lo, 4 idle), LDS offset of the instruction within the buffer,
// and per lane the source byte offset within the tile (row r, chunk c).
template <int D>
struct LDma {
    int off[LLay<D>::PER_WAVE];
};

template <int D>
HSAKV_DEV int dma_mat(int j) {
    using LY = LLay<D>;
    return j < LY::KSL ? 0 : j < 2 * LY::KSL ? 1 : j < 2 * LY::KSL + LY::VSL ? 2 : j < LY::NI ? 3 : 4;
}

template <int D>
HSAKV_DEV void ldma_lanes(LDma<D>& dl, int wave, int row_bytes) {
    using LY = LLay<D>;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < LY::PER_WAVE; ++q) {
        const int j = wave + LW * q;
        const int mat = dma_mat<D>(j);
        const int j0 = mat == 0 ? 0 : mat == 1 ? LY::KSL : mat == 2 ? 2 * LY::KSL : 2 * LY::KSL + LY::VSL;
        const int sl_n = mat < 2 ? LY::KSL : LY::VSL;
        const int L = (j - j0) * 64 + lane;
        const int r = L / sl_n, sl = L % sl_n;
        dl.off[q] = mat < 4 ? r * row_bytes + (sl < LY::CPR ? 16 * sl : 0) : 0;
    }
}

HSAKV_DEV uint32_t lds_addr(char* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)p);
}

// DMA the tile of keys [t0, t0 + nvalid) into the buffer at LDS address buf.
// Each source resource ends at the tile's last valid row, so rows past it are
// out of range and land as zeros; idle instructions have an empty resource
// and land in `spare`.
template <int D>
HSAKV_DEV void ldma_tile(uint32_t buf, uint32_t spare, const bf16_t* const (&src)[4], long long t0, int nvalid,
                         int HD, const LDma<D>& dl, int wave) {
    using LY = LLay<D>;
    const int bytes = ((nvalid - 1) * HD + D) * 2;
    __amdgpu_buffer_rsrc_t rs[5];
#pragma unroll
    for (int m = 0; m < 4; ++m)
        rs[m] = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(src[m] + t0 * HD), 0, bytes, 0x00020000);
    rs[4] = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(src[0]), 0, 0, 0x00020000);
#pragma unroll
    for (int q = 0; q < LY::PER_WAVE; ++q) {
        const int j = wave + LW * q;
        const int mat = dma_mat<D>(j);
        const uint32_t dst = mat < 4 ? buf + 1024u * j : spare;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs[mat], (lds_void_t*)(uintptr_t)dst, 16, dl.off[q], 0, 0, 0);
    }
}

template <int N>
HSAKV_DEV void lwait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

HSAKV_DEV void llds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

constexpr float kLazyMaxL = 8.0f;   // margin (log2 units) before the running max is raised
constexpr int kSchedMfmaL = 0x008, kSchedDsReadL = 0x100;

typedef __attribute__((ext_vector_type(2))) float lf32x2_t;

// O^T += V^T P^T over one 32-key half for both V parts, P^T from the half's
// weights (bf16, as the MFMA takes them), which are also added to this lane's
// share of the row sum. The V^T operands are read four reads ahead of their
// MFMAs.
template <int D>
HSAKV_DEV void lpv_half(LWave<D>& w, const f32x16_t& s, const char* buf, int sub) {
    using LY = LLay<D>;
    constexpr int DT = LY::DT;
    const int lane = threadIdx.x & 63;
    const int G = lane >> 4, j = lane & 15;
    bf16x2_t pp[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) pp[i] = __builtin_convertvector((lf32x2_t){s[2 * i], s[2 * i + 1]}, bf16x2_t);
    bf16x8_t pf[2];
#pragma unroll
    for (int c = 0; c < 2; ++c)
        pf[c] = __builtin_shufflevector(__builtin_shufflevector(pp[4 * c], pp[4 * c + 1], 0, 1, 2, 3),
                                        __builtin_shufflevector(pp[4 * c + 2], pp[4 * c + 3], 0, 1, 2, 3),
                                        0, 1, 2, 3, 4, 5, 6, 7);
    const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
    float rs = w.l;
#pragma unroll
    for (int i = 0; i < 8; ++i) rs = __builtin_amdgcn_fdot2_f32_bf16(pp[i], ones, rs, false);
    w.l = rs;
    i16x4_t lo[2][DT][2], hi[2][DT][2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int krow = 32 * sub + 16 * c + 4 * (G >> 1) + (j >> 2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int off = krow * LY::VP + 2 * (32 * dt + 16 * (G & 1) + 4 * (j & 3));
#pragma unroll
            for (int part = 0; part < 2; ++part) {
                const char* vt = buf + (part ? LY::VLO : LY::VHI);
                lo[c][dt][part] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vt + off));
                hi[c][dt][part] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vt + off + 8 * LY::VP));
            }
        }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int part = 0; part < 2; ++part) {
                const i16x8_t vv = __builtin_shufflevector(lo[c][dt][part], hi[c][dt][part], 0, 1, 2, 3, 4, 5, 6, 7);
                w.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vv), pf[c], w.o[dt],
                                                                  0, 0, 0);
            }
    // 4 reads ahead, then one MFMA per two reads, then the last two MFMAs
    __builtin_amdgcn_sched_group_barrier(kSchedDsReadL, 4, 0);
#pragma unroll
    for (int m = 0; m < 4 * DT - 2; ++m) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfmaL, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsReadL, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfmaL, 2, 0);
}

// One 64-key tile: S^T = K'_hi Q^T + K'_lo Q^T for both 32-key halves (K
// operands read four MFMAs ahead), one online-softmax step over the 64 keys
// (keys past nvalid masked; the running max is raised only when a score
// passes it by more than kLazyMaxL, so O is rarely rescaled and the weights
// stay below 2^kLazyMaxL), then P V of both halves. A half with no valid key
// has no products.
template <int D>
HSAKV_DEV void ltile(LWave<D>& w, const char* buf, int nvalid, float scale_log2) {
    using LY = LLay<D>;
    constexpr int KS = LY::KS;
    const int lane = threadIdx.x & 63;
    const int r32 = lane & 31, g2 = lane >> 5;
    bf16x8_t ah[2][KS], al[2][KS];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
        const char* kr = buf + (32 * sub + r32) * LY::KP + 16 * g2;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            ah[sub][ks] = *reinterpret_cast<const bf16x8_t*>(kr + 32 * ks);
            al[sub][ks] = *reinterpret_cast<const bf16x8_t*>(kr + LY::KLO + 32 * ks);
        }
    }
    f32x16_t s[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
        s[sub] = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah[sub][ks], w.qf[ks], s[sub], 0, 0, 0);
            s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al[sub][ks], w.qf[ks], s[sub], 0, 0, 0);
        }
    }
    __builtin_amdgcn_sched_group_barrier(kSchedDsReadL, 4, 0);
#pragma unroll
    for (int m = 0; m < 4 * KS - 4; ++m) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfmaL, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsReadL, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfmaL, 4, 0);
    if (nvalid < 64) {
        // element i of half sub holds key 32 sub + 4 g2 + 8 (i / 4) + i % 4: valid below t
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int t = nvalid - 32 * sub - 4 * g2;
#pragma unroll
            for (int i = 0; i < 16; ++i) s[sub][i] = 8 * (i >> 2) + (i & 3) < t ? s[sub][i] : -INFINITY;
        }
    }
    // raw scores: the max is taken before scaling (scale > 0); NaN-propagating
    // three-input maxima (a NaN score makes its row NaN either way)
    float mx = __builtin_elementwise_maximum(s[0][0], s[1][0]);
#pragma unroll
    for (int i = 1; i < 16; ++i)
        mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(s[0][i], s[1][i]));
    // lanes l and l + 32 hold the two key quarters of the same query
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    const float mt = mx * scale_log2;
    const bool moved = mt > w.m + kLazyMaxL;
    const float m_old = w.m;
    const float m_new = moved ? mt : m_old;
    w.m = m_new;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[sub][i] = fast_exp2(fmaf(s[sub][i], scale_log2, -m_new));
    // the row sum and O are rescaled only when some running max of the wave
    // was raised (the factor is 1 in every other lane; 0 on the first tile)
    if (__builtin_amdgcn_ballot_w64(moved)) {
        const float alpha = moved ? fast_exp2(m_old - m_new) : 1.0f;
        w.l *= alpha;
#pragma unroll
        for (int dt = 0; dt < LY::DT; ++dt) w.o[dt] *= alpha;
    }
    lpv_half<D>(w, s[0], buf, 0);
    if (nvalid > 32) lpv_half<D>(w, s[1], buf, 1);
}

template <int D>
__global__ void __launch_bounds__(64 * LW)
k_lowrank_attn32(Geo g, const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_hi,
                 const bf16_t* __restrict__ v_hi, const bf16_t* __restrict__ k_lo,
                 const bf16_t* __restrict__ v_lo, float* __restrict__ out) {
    using LY = LLay<D>;
    __shared__ __attribute__((aligned(16))) char buf0[LY::BUF];
    __shared__ __attribute__((aligned(16))) char buf1[LY::BUF];
    __shared__ __attribute__((aligned(16))) char spare[1024];
    const int nqb = (g.Lq + LQ - 1) / LQ;
    const int h = blockIdx.x / nqb, qb = blockIdx.x % nqb;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int query = qb * LQ + 32 * wave + (lane & 31);
    const bool ok = query < g.Lq;
    const long long hoff = (long long)h * D;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);

    LWave<D> w;
    const bf16_t* qp = q + (long long)(ok ? query : 0) * g.HD + hoff + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < LY::KS; ++ks) w.qf[ks] = ok ? *reinterpret_cast<const bf16x8_t*>(qp + 16 * ks) : bf16x8_t{};
#pragma unroll
    for (int dt = 0; dt < LY::DT; ++dt) w.o[dt] = f32x16_t{};
    w.m = -INFINITY;
    w.l = 0.f;

    LDma<D> dl;
    ldma_lanes<D>(dl, wave, 2 * g.HD);
    const bf16_t* const src[4] = {k_hi + hoff, k_lo + hoff, v_hi + hoff, v_lo + hoff};
    const uint32_t a0 = lds_addr(buf0), a1 = lds_addr(buf1), asp = lds_addr(spare);
    const int nt = (g.r + LT - 1) / LT;
    auto nval = [&](int t) { return g.r - t * LT < LT ? g.r - t * LT : LT; };
    ldma_tile<D>(a0, asp, src, 0, nval(0), g.HD, dl, wave);
    for (int t = 0; t < nt; t += 2) {
        lwait_vmcnt<0>();
        llds_barrier();
        if (t + 1 < nt) ldma_tile<D>(a1, asp, src, (long long)(t + 1) * LT, nval(t + 1), g.HD, dl, wave);
        ltile<D>(w, buf0, nval(t), scale_log2);
        if (t + 1 >= nt) break;
        lwait_vmcnt<0>();
        llds_barrier();
        if (t + 2 < nt) ldma_tile<D>(a0, asp, src, (long long)(t + 2) * LT, nval(t + 2), g.HD, dl, wave);
        ltile<D>(w, buf1, nval(t + 1), scale_log2);
    }

    // O / l for this lane's query: lanes l and l + 32 hold halves of the row sum
    const float lt = w.l + __shfl_xor(w.l, 32, 64);
    const float inv_l = lt > 0.f ? 1.0f / lt : 0.f;
    if (!ok) return;
    float* dst = out + (long long)query * g.HD + hoff;
    const int g2 = lane >> 5;
#pragma unroll
    for (int dt = 0; dt < LY::DT; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a)
            *reinterpret_cast<float4*>(dst + 32 * dt + 8 * a + 4 * g2) =
                float4{w.o[dt][4 * a] * inv_l, w.o[dt][4 * a + 1] * inv_l, w.o[dt][4 * a + 2] * inv_l,
                       w.o[dt][4 * a + 3] * inv_l};
}

}  // namespace

// bf16 low-rank attention (hi + lo K', V'), d = 64 or 128, output float32.
void launch_lowrank_attn_bf16_mfma32(const Geo& g, const void* q, const void* k_hi, const void* v_hi,
                                     const void* k_lo, const void* v_lo, float* out, hipStream_t st) {
    const int nqb = (g.Lq + LQ - 1) / LQ;
    const dim3 grid(g.H * nqb);
    if (g.d == 128)
        hipLaunchKernelGGL(k_lowrank_attn32<128>, grid, dim3(64 * LW), 0, st, g, (const bf16_t*)q,
                           (const bf16_t*)k_hi, (const bf16_t*)v_hi, (const bf16_t*)k_lo, (const bf16_t*)v_lo, out);
    else
        hipLaunchKernelGGL(k_lowrank_attn32<64>, grid, dim3(64 * LW), 0, st, g, (const bf16_t*)q,
                           (const bf16_t*)k_hi, (const bf16_t*)v_hi, (const bf16_t*)k_lo, (const bf16_t*)v_lo, out);
}
