// Block-sparse attention, bf16, on gfx950 32x32x16 MFMA (HSA sparse branch).
//
// Pages: WorldAttention news summary (ai4snews), HSA paragraph: each query
// block of a head attends, with exact softmax, to the tokens of its own
// selected key blocks only (Binter-token history blocks, Bintra-token chunk
// blocks).
//
// Work-group = 4 waves = two rows (query blocks 2p and 2p+1 of one head,
// 64 queries each); each wave owns 32 queries. The work-group walks the
// union of the two rows' selected blocks in ascending order, 64 keys per
// tile; a tile is loaded once and each wave computes it only if its own row
// selected it. K and V tiles stay row-major in LDS:
//   S^T = K Q^T        A = K rows (ds_read_b128), B = Q^T held in registers
//   O^T += V^T P^T     A = V^T via ds_read_b64_tr_b16 transpose reads,
//                      B = P^T straight from the S^T accumulators
// In the 32x32 accumulator layout lane l holds query l%32 and keys
// 8a + 4(l/32) + b (a, b = 0..3) of a 32-key subtile. A 16-key chunk c of
// those registers is read as the P^T operand with k order
//   e < 4: key 16c + 4(l/32) + e,   e >= 4: key 16c + 8 + 4(l/32) + e - 4
// and the V^T operand is loaded in the same key order, so P never leaves its
// lane. The transpose read returns, to lane i of each 16-lane group, column
// d0 + i of the four rows K0..K0+3 when lane j of the group addresses row
// K0 + j/4, columns d0 + 4(j%4)..+3.
//
// Tiles arrive by global -> LDS DMA into two LDS buffers: the next tile's
// DMA is issued before the current tile is computed, so HBM/L2 latency
// overlaps the MFMA work and no registers hold the data in flight. Work-groups
// are mapped XCD-aware: work-group b runs on XCD b % 8 and takes row pair
// (b % 8) * pairs_per_xcd + b / 8, so the rows of one head stay on one XCD
// and share its L2.
#include "common.h"
#include "launch.h"

namespace {

constexpr int KT = 64;               // keys per tile

typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(8))) short i16x8_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;   // native 16-byte vector

// LDS tiles are filled by global_load_lds_dwordx4 (global -> LDS DMA, no
// registers): one wave instruction writes 64 lanes x 16 bytes contiguously,
// lane l at base + 16 l. Rows are D bf16 (no padding); the 16-byte slots of
// row r are XOR-swizzled so the MFMA operand reads hit distinct banks:
//   K: slot s of row r holds chunk s ^ (r mod CPR)        (16 rows, one chunk)
//   V: slot s of row r holds chunk s ^ (2r mod CPR)       (4 rows, two chunks)
template <int D>
struct Lay {
    static constexpr int ROWB = D * 2;        // bytes per key row
    static constexpr int CPR = D / 8;         // 16-byte chunks per row
    static constexpr int MAT = KT * ROWB;     // bytes of one K or V tile
    static constexpr int BUF = 2 * MAT;       // K tile then V tile
    HSAKV_DEV static int swz_k(int r) { return r & (CPR - 1); }
    HSAKV_DEV static int swz_v(int r) { return (2 * r) & (CPR - 1); }
};

typedef __attribute__((address_space(3))) void lds_void_t;

// DMA one tile (64 key rows of K and V) into an LDS buffer. Each of the NW
// waves issues its share of the 1 KB wave instructions. Rows past `nvalid`
// (the ragged end of a block) load the last valid row: their scores are
// masked to -inf, so P = 0 multiplies finite values.
template <int D, int NW>
HSAKV_DEV void dma_tile(char* buf, const bf16_t* __restrict__ ks, const bf16_t* __restrict__ vs,
                        long long t0, int nvalid, int HD) {
    using LY = Lay<D>;
    constexpr int INSTR = KT * LY::CPR / 64;       // wave instructions per matrix
    constexpr int PER_WAVE = INSTR / NW;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const bf16_t* kb = ks + t0 * (long long)HD;
    const bf16_t* vb = vs + t0 * (long long)HD;
#pragma unroll
    for (int j = 0; j < PER_WAVE; ++j) {
        const int slot0 = (wave * PER_WAVE + j) * 64;
        const int L = slot0 + lane;
        const int r = L / LY::CPR, sl = L % LY::CPR;
        const int rg = r < nvalid ? r : nvalid - 1;
        const int offk = rg * HD + ((sl ^ LY::swz_k(r)) << 3);
        const int offv = rg * HD + ((sl ^ LY::swz_v(r)) << 3);
        __builtin_amdgcn_global_load_lds(kb + offk, (lds_void_t*)(buf + slot0 * 16), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vb + offv, (lds_void_t*)(buf + LY::MAT + slot0 * 16), 16, 0, 0);
    }
}

// s_waitcnt vmcnt(0) with the other counters unconstrained (gfx9 encoding).
HSAKV_DEV void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0f70); }

template <int D>
struct Wave {
    static constexpr int KS = D / 16;   // 16-wide k steps of S^T = K Q^T
    static constexpr int DT = D / 32;   // 32-row tiles of O^T
    bf16x8_t qf[KS];
    f32x16_t o[DT];
    float m, l;
};

template <int D>
HSAKV_DEV void tile_step(Wave<D>& w, const char* kt, const char* vt, int nvalid, float scale_log2) {
    using LY = Lay<D>;
    const int lane = threadIdx.x & 63;
    const int r32 = lane & 31, g2 = lane >> 5;
    f32x16_t s[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
        s[sub] = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < Wave<D>::KS; ++ks) {
            const int row = 32 * sub + r32;
            const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
                kt + row * LY::ROWB + (((2 * ks + g2) ^ LY::swz_k(row)) << 4));
            s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w.qf[ks], s[sub], 0, 0, 0);
        }
    }
    // raw scores: the row max is taken before scaling (scale > 0), and the
    // scale folds into the exponent's FMA
    float mx = -INFINITY;
    if (nvalid < KT) {
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = 32 * sub + 8 * (i >> 2) + 4 * g2 + (i & 3);
                if (key >= nvalid) s[sub][i] = -INFINITY;
            }
    }
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[sub][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(w.m, mx * scale_log2);
    const bool moved = m_new > w.m;
    const float alpha = fast_exp2(w.m - m_new);   // 1 when the max did not move
    w.m = m_new;
    float rs = 0.f;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float p = fast_exp2(fmaf(s[sub][i], scale_log2, -m_new));
            s[sub][i] = p;
            rs += p;
        }
    w.l = w.l * alpha + rs;
    // rescale O only when some row max of the wave moved
    if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
        for (int dt = 0; dt < Wave<D>::DT; ++dt) w.o[dt] *= alpha;
    }

    const int G = lane >> 4, j = lane & 15;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            bf16x8_t pf;
#pragma unroll
            for (int e = 0; e < 8; ++e) pf[e] = (__bf16)s[sub][8 * c + e];
            const int krow = 32 * sub + 16 * c + 4 * (G >> 1) + (j >> 2);
#pragma unroll
            for (int dt = 0; dt < Wave<D>::DT; ++dt) {
                const int dcol = 32 * dt + 16 * (G & 1) + 4 * (j & 3);
                const int lo_off = krow * LY::ROWB + (((dcol >> 3) ^ LY::swz_v(krow)) << 4) + ((dcol & 7) << 1);
                const int hi_off = (krow + 8) * LY::ROWB + (((dcol >> 3) ^ LY::swz_v(krow + 8)) << 4) +
                                   ((dcol & 7) << 1);
                const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vt + lo_off));
                const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vt + hi_off));
                const i16x8_t vv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                w.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vv), pf,
                                                                  w.o[dt], 0, 0, 0);
            }
        }
    }
}

// Key block b -> token range and source (history blocks first, then chunk blocks).
struct Cursor {
    int n;          // position in the row's selected-block list
    int s0;         // offset of the tile inside the block
    long long t0;   // first token of the block
    int len;        // valid tokens of the block
    bool hist;
};

HSAKV_DEV void open_block(const Geo& g, int NBh, long long Lh, int b, Cursor& c) {
    c.s0 = 0;
    if (b < NBh) {
        c.hist = true;
        c.t0 = (long long)b * g.Binter;
        const long long e = c.t0 + g.Binter < Lh ? c.t0 + g.Binter : Lh;
        c.len = (int)(e - c.t0);
    } else {
        c.hist = false;
        c.t0 = (long long)(b - NBh) * g.Bintra;
        const long long e = c.t0 + g.Bintra < g.Lq ? c.t0 + g.Bintra : g.Lq;
        c.len = (int)(e - c.t0);
    }
}

// The union of R rows' sorted block lists, walked tile by tile. All threads
// of the work-group hold the same cursor.
template <int R>
struct Union {
    int pos[R];     // next unread position in each row's list
    int head[R];    // id at pos (INT_MAX when the list is exhausted)
    int blk;        // current block
    unsigned in;    // rows that selected the current block
};

template <int R>
HSAKV_DEV void union_next(Union<R>& u, const int32_t* const ids[R], const int cnt[R]) {
    int b = 0x7fffffff;
#pragma unroll
    for (int r = 0; r < R; ++r) b = u.head[r] < b ? u.head[r] : b;
    u.blk = b;
    u.in = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (u.head[r] == b && b != 0x7fffffff) {
            u.in |= 1u << r;
            ++u.pos[r];
            u.head[r] = u.pos[r] < cnt[r] ? ids[r][u.pos[r]] : 0x7fffffff;
        }
    }
}

// R rows (query blocks 2p, 2p+1, ... of one head) per work-group, 2 waves per
// row. The work-group stages the union of the rows' selected tiles once;
// each wave computes only the tiles its own row selected.
template <int D, int R>
__global__ void __launch_bounds__(128 * R, 2)
k_sparse_attn32(Geo g, const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_hist,
                const bf16_t* __restrict__ v_hist, const bf16_t* __restrict__ k_intra,
                const bf16_t* __restrict__ v_intra, const int32_t* __restrict__ n_sel_p,
                const int32_t* __restrict__ sel_count, const int32_t* __restrict__ sel_idx,
                int groups_per_xcd, Epi ep) {
    constexpr int NW = 2 * R;
    // two distinct LDS objects with fixed roles per step: the compiler can then
    // tell the next tile's DMA from this tile's reads and inserts no wait
    __shared__ __attribute__((aligned(16))) char buf0[Lay<D>::BUF];
    __shared__ __attribute__((aligned(16))) char buf1[Lay<D>::BUF];
    const int b = blockIdx.x;
    const int grp = (b & 7) * groups_per_xcd + (b >> 3);
    const int gph = (g.NQB + R - 1) / R;            // groups per head
    if (grp >= g.H * gph) return;
    const int h = grp / gph;
    const int i0 = (grp % gph) * R;                  // first query block of the group
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int myr = wave >> 1;                       // this wave's row in the group
    const int g2 = lane >> 5;
    const int i = i0 + myr;
    const int query = i * g.Bq + 32 * (wave & 1) + (lane & 31);
    const int n_sel = *n_sel_p;
    const int NBh = hist_blocks(g, n_sel);
    const long long Lh = (long long)n_sel * g.Tp;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    const long long hoff = (long long)h * D;

    Wave<D> w;
#pragma unroll
    for (int ks = 0; ks < Wave<D>::KS; ++ks) {
        if (i < g.NQB && query < g.Lq)
            w.qf[ks] = *reinterpret_cast<const bf16x8_t*>(q + (long long)query * g.HD + hoff + 16 * ks + 8 * g2);
        else
            w.qf[ks] = bf16x8_t{};
    }
#pragma unroll
    for (int dt = 0; dt < Wave<D>::DT; ++dt) w.o[dt] = f32x16_t{};
    w.m = -INFINITY;
    w.l = 0.f;

    const int32_t* ids[R];
    int cnt[R];
    Union<R> u;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int ir = i0 + r;
        const int row = h * g.NQB + ir;
        cnt[r] = ir < g.NQB ? sel_count[row] : 0;
        ids[r] = sel_idx + (size_t)row * g.NB_max;
        u.pos[r] = 0;
        u.head[r] = cnt[r] > 0 ? ids[r][0] : 0x7fffffff;
    }
    union_next<R>(u, ids, cnt);

    Cursor cur;
    int nvalid = 0;
    unsigned in_next = u.in;
    bool have = u.blk != 0x7fffffff;
    if (have) {
        open_block(g, NBh, Lh, u.blk, cur);
        nvalid = cur.len < KT ? cur.len : KT;
        dma_tile<D, NW>(buf0, (cur.hist ? k_hist : k_intra) + hoff, (cur.hist ? v_hist : v_intra) + hoff,
                        cur.t0, nvalid, g.HD);
    }
    // One pipeline step: the current tile sits in `now`, the next one is sent to `nxt`.
    auto step = [&](const char* now, char* nxt) __attribute__((always_inline)) {
        // this wave's DMA of the current tile has landed; the barrier makes every
        // wave's part visible and retires every read of `nxt` by the last step
        wait_vmcnt0();
        __syncthreads();
        const int nvalid_now = nvalid;
        const unsigned in_now = in_next;
        cur.s0 += KT;
        if (cur.s0 >= cur.len) {
            union_next<R>(u, ids, cnt);
            have = u.blk != 0x7fffffff;
            if (have) {
                open_block(g, NBh, Lh, u.blk, cur);
                in_next = u.in;
            }
        }
        if (have) {
            nvalid = cur.len - cur.s0 < KT ? cur.len - cur.s0 : KT;
            dma_tile<D, NW>(nxt, (cur.hist ? k_hist : k_intra) + hoff, (cur.hist ? v_hist : v_intra) + hoff,
                            cur.t0 + cur.s0, nvalid, g.HD);
        }
        if ((in_now >> myr) & 1u) tile_step<D>(w, now, now + Lay<D>::MAT, nvalid_now, scale_log2);
    };
    while (have) {
        step(buf0, buf1);
        if (!have) break;
        step(buf1, buf0);
    }
    if (i >= g.NQB) return;

    // epilogue: O / l, optional gated fusion with the low-rank branch
    float lt = w.l + __shfl_xor(w.l, 32, 64);
    const float inv_l = lt > 0.f ? 1.0f / lt : 0.f;
    float gate = 0.f;
    if (ep.out) {
        float dot = 0.f;
#pragma unroll
        for (int ks = 0; ks < Wave<D>::KS; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                dot = fmaf((float)w.qf[ks][e], ep.w_g[h * D + 16 * ks + 8 * g2 + e], dot);
        dot += __shfl_xor(dot, 32, 64);
        const float x = dot + ep.b_g[h];
        const float z = expf(-fabsf(x));
        gate = x >= 0.f ? 1.0f / (1.0f + z) : z / (1.0f + z);
    }
    if (query >= g.Lq) return;
    const long long base = (long long)query * g.HD + hoff;
    if (ep.gate && g2 == 0) ep.gate[(long long)query * g.H + h] = gate;
#pragma unroll
    for (int dt = 0; dt < Wave<D>::DT; ++dt) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int d0 = 32 * dt + 8 * a + 4 * g2;
            const float4 o = {w.o[dt][4 * a] * inv_l, w.o[dt][4 * a + 1] * inv_l,
                              w.o[dt][4 * a + 2] * inv_l, w.o[dt][4 * a + 3] * inv_l};
            if (ep.o_main) *reinterpret_cast<float4*>(ep.o_main + base + d0) = o;
            if (ep.out) {
                const float4 lin = *reinterpret_cast<const float4*>(ep.o_lin + base + d0);
                const float r0 = gate * o.x + (1.f - gate) * lin.x;
                const float r1 = gate * o.y + (1.f - gate) * lin.y;
                const float r2 = gate * o.z + (1.f - gate) * lin.z;
                const float r3 = gate * o.w + (1.f - gate) * lin.w;
                uint2 pk;
                pk.x = (uint32_t)f32_to_bf16(r0) | ((uint32_t)f32_to_bf16(r1) << 16);
                pk.y = (uint32_t)f32_to_bf16(r2) | ((uint32_t)f32_to_bf16(r3) << 16);
                *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(ep.out) + base + d0) = pk;
            }
        }
    }
}

}  // namespace

template <int D, int R>
static void launch_r(const Geo& g, const void* q, const void* k_hist, const void* v_hist,
                     const void* k_intra, const void* v_intra, const int32_t* n_sel,
                     const int32_t* sel_count, const int32_t* sel_idx, const Epi& ep,
                     hipStream_t st) {
    const int groups = g.H * ((g.NQB + R - 1) / R);
    const int per_xcd = (groups + 7) / 8;
    hipLaunchKernelGGL((k_sparse_attn32<D, R>), dim3(8 * per_xcd), dim3(128 * R), 0, st, g,
                       (const bf16_t*)q, (const bf16_t*)k_hist, (const bf16_t*)v_hist,
                       (const bf16_t*)k_intra, (const bf16_t*)v_intra, n_sel, sel_count, sel_idx,
                       per_xcd, ep);
}

void launch_sparse_attn_bf16_mfma32(const Geo& g, const void* q, const void* k_hist,
                                    const void* v_hist, const void* k_intra, const void* v_intra,
                                    const int32_t* n_sel, const int32_t* sel_count,
                                    const int32_t* sel_idx, const Epi& ep, hipStream_t st) {
    // two query blocks (rows) of one head per work-group
    if (g.d == 128)
        launch_r<128, 2>(g, q, k_hist, v_hist, k_intra, v_intra, n_sel, sel_count, sel_idx, ep, st);
    else
        launch_r<64, 2>(g, q, k_hist, v_hist, k_intra, v_intra, n_sel, sel_count, sel_idx, ep, st);
}
