// Low-rank projection K' = E K_act, V' = F V_act in bf16 on gfx950 32x32x16 MFMA.
//
// Pages: WorldAttention news summary (ai4snews), HSA paragraph (a
// Linformer-style low-rank global branch, O(L r)); the projection is the
// Linformer paper's (cited on the mlsanity map): one E and one F of shape
// [r][L] shared by every head, applied to the keys and values of the active
// cache followed by the chunk.
//
// As a GEMM: C[m][n] = sum_k X[m][col(k)] Y[k][n] with X = E or F (rows of r,
// k-contiguous), Y = the active keys or values as [L_act][H*d] (n-contiguous)
// and k running over the present history rows then the chunk rows. It is a
// long-K contraction (K = 54600 at the 1.3B 480p shape) with a small output
// (r x H*d), so it is split along k; each split writes an f32 partial and a
// separate pass adds the partials in split order.
//
// Two tile shapes. For r >= 128 and H*d a multiple of 256: 256 x 256 tiles
// (k_lowrank_proj256, below). Otherwise:
// Work-group = 4 waves, tile 128 (m) x 128 (n), k-step 64. Wave w computes
// rows 64(w%2).. and columns 64(w/2).. with four 32x32 accumulators. Tiles
// are brought into LDS by global -> LDS DMA (two buffers, the next k-step in
// flight during the MFMA work); the tile is small enough that two
// work-groups share a CU, doubling the DMA in flight of this latency-bound
// stream. DMA writes 64 lanes x 16 bytes contiguously,
// so the padded row pitch that keeps the operand reads free of bank conflicts
// is made by "pad lanes": the X tile has 9 slots per row (8 data + 1 pad,
// 144 B pitch), the Y tile 18 (16 + 2, 288 B pitch); a pad lane loads any
// valid address and lands in the pad. X fragments are ds_read_b128 rows; Y
// fragments come from ds_read_b64_tr_b16 transpose reads of the row-major
// tile (lane i of a 16-lane group receives column c0 + i of four rows).
#include "common.h"
#include "launch.h"

namespace {

constexpr int BM = 128, BN = 128, BK = 64, NT = 256, NWV = 4;
constexpr int A_SLOTS = BK / 8 + 1;           // 9
constexpr int B_SLOTS = BN / 8 + 2;           // 18
constexpr int A_ROWB = A_SLOTS * 16;          // 144
constexpr int B_ROWB = B_SLOTS * 16;          // 288
constexpr int A_BYTES = BM * A_ROWB;          // 18432
constexpr int B_BYTES = BK * B_ROWB;          // 18432
constexpr int STAGE = A_BYTES + B_BYTES;      // 36864; two stages: 73728 bytes (two work-groups per CU)
constexpr int A_INSTR = BM * A_SLOTS / 64;    // 18
constexpr int B_INSTR = BK * B_SLOTS / 64;    // 18
static_assert(BM * A_SLOTS % 64 == 0 && BK * B_SLOTS % 64 == 0, "whole wave instructions");

typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(8))) short i16x8_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

HSAKV_DEV void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0f70); }

struct ProjArgs {
    const bf16_t* X;      // E or F
    const bf16_t* Yh;     // k_hist or v_hist
    const bf16_t* Yc;     // k_intra or v_intra
    long long Lh;         // present history rows
    long long Lact;       // Lh + Lq
};

// Per-lane DMA offsets that do not change from one k-step to the next: the
// X row (clamped to r) and k slot, the Y row and n slot of each of this wave's
// instructions (at most A_PER / B_PER of them).
constexpr int A_PER = (A_INSTR + NWV - 1) / NWV;
constexpr int B_PER = (B_INSTR + NWV - 1) / NWV;
struct DmaLanes {
    int a_off[A_PER];    // m * L + 8 * slot (slot 0 for the pad lane)
    int b_row[B_PER];    // k row inside the stage
    int b_col[B_PER];    // n0 + 8 * slot
};

HSAKV_DEV void dma_lanes(DmaLanes& dl, const Geo& g, int m0, int n0) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < A_PER; ++q) {
        const int L = (wave + NWV * q) * 64 + lane;
        const int row = L / A_SLOTS, sl = L % A_SLOTS;
        int m = m0 + row;
        m = m < g.r ? m : g.r - 1;
        dl.a_off[q] = m * (int)g.L + (sl < BK / 8 ? sl : 0) * 8;
    }
#pragma unroll
    for (int q = 0; q < B_PER; ++q) {
        const int L = (wave + NWV * q) * 64 + lane;
        const int row = L / B_SLOTS, sl = L % B_SLOTS;
        dl.b_row[q] = row;
        dl.b_col[q] = n0 + (sl < BN / 8 ? sl : 0) * 8;
    }
}

// DMA one k-step (X: 256 rows x 64 k; Y: 64 k rows x 128 n) into `buf`.
// Fast path: the step lies on one side of the history/chunk seam and inside
// the split, so every address is a uniform base plus a fixed lane offset.
// Otherwise each lane maps its own k: k past the valid range reads a clamped
// (valid) address, and the Y rows past the split's end are zeroed before use.
HSAKV_DEV void dma_stage(char* buf, const Geo& g, const ProjArgs& a, const DmaLanes& dl, long long k0,
                         long long ke) {
    const int wave = threadIdx.x >> 6;
    const bool fast = k0 + BK <= ke && (k0 + BK <= a.Lh || k0 >= a.Lh);
    if (fast) {
        const bool hist = k0 < a.Lh;
        const bf16_t* xb = a.X + (hist ? k0 : g.hist_rows + (k0 - a.Lh));
        const bf16_t* yb = hist ? a.Yh + k0 * g.HD : a.Yc + (k0 - a.Lh) * g.HD;
#pragma unroll
        for (int q = 0; q < A_PER; ++q) {
            const int j = wave + NWV * q;
            if (j < A_INSTR)
                __builtin_amdgcn_global_load_lds(xb + dl.a_off[q], (lds_void_t*)(buf + j * 1024), 16, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < B_PER; ++q) {
            const int j = wave + NWV * q;
            if (j < B_INSTR)
                __builtin_amdgcn_global_load_lds(yb + dl.b_row[q] * g.HD + dl.b_col[q],
                                                 (lds_void_t*)(buf + A_BYTES + j * 1024), 16, 0, 0);
        }
        return;
    }
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < A_PER; ++q) {
        const int j = wave + NWV * q;
        if (j >= A_INSTR) continue;
        const int L = j * 64 + lane;
        const int sl = L % A_SLOTS;
        long long k = k0 + (sl < BK / 8 ? sl : 0) * 8;
        k = k + 8 <= a.Lact ? k : a.Lact - 8;
        const long long col = k < a.Lh ? k : g.hist_rows + (k - a.Lh);
        const int mrow = dl.a_off[q] / (int)g.L;
        __builtin_amdgcn_global_load_lds(a.X + (long long)mrow * g.L + col, (lds_void_t*)(buf + j * 1024), 16, 0, 0);
    }
#pragma unroll
    for (int q = 0; q < B_PER; ++q) {
        const int j = wave + NWV * q;
        if (j >= B_INSTR) continue;
        long long k = k0 + dl.b_row[q];
        k = k < a.Lact ? k : a.Lact - 1;
        const bf16_t* src = (k < a.Lh ? a.Yh + k * g.HD : a.Yc + (k - a.Lh) * g.HD) + dl.b_col[q];
        __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(buf + A_BYTES + j * 1024), 16, 0, 0);
    }
}

// Zero the Y rows [first, BK) of a stage (the k past the split's end).
HSAKV_DEV void zero_tail(char* buf, int first) {
    for (int idx = threadIdx.x; idx < (BK - first) * (BN / 8); idx += NT) {
        const int row = first + idx / (BN / 8), c = idx % (BN / 8);
        *reinterpret_cast<uint4*>(buf + A_BYTES + row * B_ROWB + c * 16) = uint4{0, 0, 0, 0};
    }
}

HSAKV_DEV void compute_stage(const char* buf, f32x16_t (&acc)[2][2]) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int mw = wave & 1, nw = wave >> 1;
    const int r32 = lane & 31, g2 = lane >> 5, G = lane >> 4, j = lane & 15;
    const char* A = buf;
    const char* B = buf + A_BYTES;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
        bf16x8_t af[2], bfr[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
            af[mt] = *reinterpret_cast<const bf16x8_t*>(A + (64 * mw + 32 * mt + r32) * A_ROWB + (16 * ks + 8 * g2) * 2);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
            const int krow = 16 * ks + 8 * (G >> 1) + (j >> 2);
            const int col = 64 * nw + 32 * nt + 16 * (G & 1) + 4 * (j & 3);
            const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(B + krow * B_ROWB + col * 2));
            const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(B + (krow + 4) * B_ROWB + col * 2));
            bfr[nt] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int nt = 0; nt < 2; ++nt)
                acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mt], bfr[nt], acc[mt][nt], 0, 0, 0);
    }
}

__global__ void __launch_bounds__(NT, 2)
k_lowrank_proj32(Geo g, const bf16_t* __restrict__ E, const bf16_t* __restrict__ F,
                 const bf16_t* __restrict__ k_hist, const bf16_t* __restrict__ v_hist,
                 const bf16_t* __restrict__ k_intra, const bf16_t* __restrict__ v_intra,
                 const int32_t* __restrict__ n_sel_p, int nsplit, int per_xcd, float* __restrict__ part) {
    // two distinct LDS objects with fixed roles per step, so the compiler can
    // tell the next step's DMA from this step's reads
    __shared__ __attribute__((aligned(16))) char buf0[STAGE];
    __shared__ __attribute__((aligned(16))) char buf1[STAGE];
    const int MT = (g.r + BM - 1) / BM, NTL = g.HD / BN;
    const int total = nsplit * 2 * MT * NTL;
    const int lin = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (lin >= total) return;
    const int nt_i = lin % NTL;
    const int mt_i = (lin / NTL) % MT;
    const int z = (lin / (NTL * MT)) & 1;
    const int split = lin / (NTL * MT * 2);
    const int m0 = mt_i * BM, n0 = nt_i * BN;
    ProjArgs a;
    a.X = z ? F : E;
    a.Yh = z ? v_hist : k_hist;
    a.Yc = z ? v_intra : k_intra;
    a.Lh = (long long)(*n_sel_p) * g.Tp;
    a.Lact = a.Lh + g.Lq;
    const long long per = ((g.L + nsplit - 1) / nsplit + BK - 1) / BK * BK;
    const long long kb = (long long)split * per;
    const long long ke = kb + per < a.Lact ? kb + per : a.Lact;
    DmaLanes dl;
    dma_lanes(dl, g, m0, n0);

    f32x16_t acc[2][2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x16_t{};

    long long k0 = kb;
    if (k0 < ke) dma_stage(buf0, g, a, dl, k0, ke);
    auto step = [&](char* now, char* nxt) __attribute__((always_inline)) {
        wait_vmcnt0();
        __syncthreads();
        if (k0 + BK > ke) {                  // last, partial k-step of the split
            zero_tail(now, (int)(ke - k0));
            __syncthreads();
        }
        if (k0 + BK < ke) dma_stage(nxt, g, a, dl, k0 + BK, ke);
        compute_stage(now, acc);
        k0 += BK;
    };
    while (k0 < ke) {
        step(buf0, buf1);
        if (k0 >= ke) break;
        step(buf1, buf0);
    }

    // D[m = 8(i/4) + 4(l/32) + i%4][n = l%32] of each 32x32 accumulator
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int mw = wave & 1, nw = wave >> 1, g2 = lane >> 5;
    float* out = part + (size_t)(split * 2 + z) * g.r * g.HD;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = m0 + 64 * mw + 32 * mt + 8 * (i >> 2) + 4 * g2 + (i & 3);
                const int n = n0 + 64 * nw + 32 * nt + (lane & 31);
                if (m < g.r) out[(size_t)m * g.HD + n] = acc[mt][nt][i];
            }
}

// ---- 256 x 256 tiles ---------------------------------------------------------
//
// For r >= 128 and H*d a multiple of 256 the output tile is 256 (m) x 256 (n)
// with 64-wide k-steps: a k-step reads E's slice once per 256 columns of keys
// and each key slice once per 256 rows of E (half and a quarter of the L2
// reads of 128 x 128 tiles), and each of the 256 E rows of a step is one
// whole 128-byte line. 8 waves (wave w: rows 128 (w % 2), columns 64 (w / 2),
// eight 32x32 accumulators) and one work-group per CU. The LDS is a ring of
// five 32 KB half-stages, each the X (E or F) tile or the Y (keys or values)
// tile of one k-step, sent in the order X0 Y0 X1 Y1 X2 ...: a half-stage is
// refilled as soon as the step that used it is done, so during the MFMA work
// of step i the halves X(i+1), Y(i+1) and X(i+2) are in flight (1.5 steps,
// where two 64 KB stages hold one; the 160 KB of LDS do not fit three). The
// 16-byte chunks
// of a row are XOR-swizzled in LDS for conflict-free operand reads, with rows
// unpadded so every DMA lane loads data and each row's bytes stay contiguous:
// X (128-byte rows) slot s of row r holds chunk s ^ (r / 2 mod 8), so the 16
// rows of one b128 read phase fall on distinct banks; Y (512-byte rows) slot s
// of row r holds chunk s ^ 4 (r mod 4), so the 4 rows x 4 chunks of a
// transpose read's 32 lanes do.
//
// The k-steps of a split run over its history part, then its chunk part, each
// ending in a partial step, so no step straddles the seam. The DMA goes
// through buffer loads whose resource covers exactly the valid bytes: a Y row
// past the part's end, or an X column past the end of E, is out of range and
// not read; its LDS row is zeroed before use.
constexpr int WM = 256, WN = 256, WK = 64, WT = 512, WWV = 8;
constexpr int WA_SLOTS = WK / 8;               // 8 chunks per X row
constexpr int WB_SLOTS = WN / 8;               // 32 chunks per Y row
constexpr int WA_ROWB = WA_SLOTS * 16;         // 128
constexpr int WB_ROWB = WB_SLOTS * 16;         // 512
constexpr int WA_BYTES = WM * WA_ROWB;         // 32768
constexpr int WB_BYTES = WK * WB_ROWB;         // 32768
constexpr int WHALF = 32768;                   // one half-stage: an X or a Y tile
constexpr int WRING = 5;                       // half-stages in the ring (160 KB)
constexpr int WA_INSTR = WM * WA_SLOTS / 64;   // 32
constexpr int WB_INSTR = WK * WB_SLOTS / 64;   // 32
constexpr int W_PER = 8;                       // DMA instructions per wave and k-step
static_assert(WM * WA_SLOTS % 64 == 0 && WK * WB_SLOTS % 64 == 0, "whole wave instructions");
static_assert(WA_BYTES == WHALF && WB_BYTES == WHALF, "X and Y tiles fill one half-stage each");
static_assert(WA_BYTES == WA_INSTR * 1024, "Y follows X in instruction order");
static_assert(WA_INSTR + WB_INSTR == WWV * W_PER, "every wave sends the same count");
static_assert(WA_INSTR == 4 * WWV && WB_INSTR == 4 * WWV, "four DMA instructions per wave and half-stage");
HSAKV_DEV int xswz(int row) { return (row >> 1) & 7; }   // X chunk swizzle
HSAKV_DEV int yswz(int row) { return 4 * (row & 3); }    // Y chunk swizzle

// Raw buffer resource: base p, `bytes` in range, 32-bit untyped data.
HSAKV_DEV __amdgpu_buffer_rsrc_t w_rsrc(const bf16_t* p, long long bytes) {
    const int n = bytes > 0x7fffffffLL ? 0x7fffffff : (int)(bytes < 0 ? 0 : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(p), 0, n, 0x00020000);
}

// The LDS destination of a DMA as an address the compiler cannot trace to the
// ring: the kernel orders each DMA before the reads of its stage (a vmcnt
// wait, then the barrier), and the compiler's own tracking of LDS DMA targets
// would add waits that drain the prefetch too.
HSAKV_DEV lds_void_t* w_dst(char* p) {
    const uint32_t v = (uint32_t)(uintptr_t)(lds_void_t*)p;
    return (lds_void_t*)(uintptr_t)__builtin_amdgcn_readfirstlane(v);
}

// s_waitcnt vmcnt(N) with the other counters unconstrained.
template <int N>
HSAKV_DEV void wait_vm() {
    static_assert(N >= 0 && N < 16, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(0x0f70 | N);
}

// LDS-only work-group barrier (DMA in flight stays in flight).
HSAKV_DEV void w_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Byte offsets of this wave's DMA instructions j = wave + 8 q (fixed over
// the k-steps): X (j < 32) m * L + 8 chunk from the step's first column,
// Y (j >= 32) row * HD + n0 + 8 chunk from the step's first row, the chunk a
// lane's LDS slot holds under the swizzle.
HSAKV_DEV void w_lanes(uint32_t (&off)[W_PER], const Geo& g, int wave, int m0, int n0) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int q = 0; q < W_PER; ++q) {
        const int j = wave + WWV * q;
        const int La = j * 64 + lane, Lb = (j - WA_INSTR) * 64 + lane;
        const int ra = La / WA_SLOTS, sa = La % WA_SLOTS, rb = Lb / WB_SLOTS, sb = Lb % WB_SLOTS;
        const int m = m0 + ra < g.r ? m0 + ra : g.r - 1;
        const uint32_t oa = 2u * (uint32_t)(m * (int)g.L + (sa ^ xswz(ra)) * 8);
        const uint32_t ob = 2u * (uint32_t)(rb * g.HD + n0 + (sb ^ yswz(rb)) * 8);
        off[q] = j < WA_INSTR ? oa : ob;
    }
}

// Zero the rows [first, WK) of a Y tile.
HSAKV_DEV void w_zero_tail(char* yb, int first) {
    for (int idx = threadIdx.x; idx < (WK - first) * (WN / 8); idx += WT) {
        const int row = first + idx / (WN / 8), c = idx % (WN / 8);
        *reinterpret_cast<uint4*>(yb + row * WB_ROWB + c * 16) = uint4{0, 0, 0, 0};
    }
}

typedef __attribute__((ext_vector_type(2))) unsigned w_u32x2_t;

// Keys 32 h .. 32 h + 31 of a k-step (two 16-wide MFMA steps). The eight
// transpose reads of Y sit in one asm block that waits for them itself:
// issued as builtins, they would make the compiler wait for every DMA in
// flight first (the next step's included).
HSAKV_DEV void w_compute(const char* xb, const char* yb, f32x16_t (&acc)[4][2], int wave, int h) {
    const int lane = threadIdx.x & 63;
    const int mw = wave & 1, nw = wave >> 1;
    const int r32 = lane & 31, g2 = lane >> 5, G = lane >> 4, j = lane & 15;
    // X row 128 mw + 32 mt + r32 has swizzle xswz(r32); chunk 4 h + 2 kk + g2 sits in slot chunk ^ xswz
    const char* Arow = xb + (128 * mw + r32) * WA_ROWB;
    const char* A0 = Arow + 16 * ((4 * h + g2) ^ xswz(r32));
    const char* A1 = Arow + 16 * ((4 * h + 2 + g2) ^ xswz(r32));
    // Y rows 32 h + 16 kk + 4 e + 8 (G / 2) + j / 4 have swizzle yswz(j / 4); the 8 columns of
    // chunk 8 nw + 4 nt + 2 (G & 1) + (j & 3) / 2 sit in slot chunk ^ yswz, at byte 8 (j & 1)
    const int cy = 8 * nw + 2 * (G & 1) + ((j & 3) >> 1);
    const char* Brow = yb + (32 * h + 8 * (G >> 1) + (j >> 2)) * WB_ROWB + 8 * (j & 1);
    const uint32_t bb0 = (uint32_t)(uintptr_t)(const lds_i16x4_t*)(Brow + 16 * (cy ^ yswz(j >> 2)));
    const uint32_t bb1 = (uint32_t)(uintptr_t)(const lds_i16x4_t*)(Brow + 16 * ((cy + 4) ^ yswz(j >> 2)));
    // r[4 kk + 2 nt + e]: k rows 16 kk + 4 e (+ 8 (G / 2) + j / 4), columns 32 nt + ...
    constexpr int H = 4 * WB_ROWB, K1 = 16 * WB_ROWB;
    bf16x8_t a0[4], a1[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) a0[mt] = *reinterpret_cast<const bf16x8_t*>(A0 + 32 * mt * WA_ROWB);
    w_u32x2_t r[8];
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:%10\n\t"
        "ds_read_b64_tr_b16 %2, %9\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:%10\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:%11\n\t"
        "ds_read_b64_tr_b16 %5, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %6, %9 offset:%11\n\t"
        "ds_read_b64_tr_b16 %7, %9 offset:%12\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(bb0), "v"(bb1), "i"(H), "i"(K1), "i"(K1 + H)
        : "memory");
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) a1[mt] = *reinterpret_cast<const bf16x8_t*>(A1 + 32 * mt * WA_ROWB);
    bf16x8_t b[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
            b[kk][nt] = __builtin_bit_cast(
                bf16x8_t, __builtin_shufflevector(r[4 * kk + 2 * nt], r[4 * kk + 2 * nt + 1], 0, 1, 2, 3));
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[mt], b[0][nt], acc[mt][nt], 0, 0, 0);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[mt], b[1][nt], acc[mt][nt], 0, 0, 0);
}

__global__ void __launch_bounds__(WT, 1)
k_lowrank_proj256(Geo g, const bf16_t* __restrict__ E, const bf16_t* __restrict__ F,
                  const bf16_t* __restrict__ k_hist, const bf16_t* __restrict__ v_hist,
                  const bf16_t* __restrict__ k_intra, const bf16_t* __restrict__ v_intra,
                  const int32_t* __restrict__ n_sel_p, int nsplit, int per_xcd, float* __restrict__ part) {
    __shared__ __attribute__((aligned(16))) char ring[WRING * WHALF];
    const int MT = (g.r + WM - 1) / WM, NTL = g.HD / WN;
    const int total = nsplit * 2 * MT * NTL;
    const int lin = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (lin >= total) return;
    const int nt_i = lin % NTL;
    const int mt_i = (lin / NTL) % MT;
    const int z = (lin / (NTL * MT)) & 1;
    const int split = lin / (NTL * MT * 2);
    const int m0 = mt_i * WM, n0 = nt_i * WN;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const bf16_t* X = z ? F : E;
    const bf16_t* Yh = z ? v_hist : k_hist;
    const bf16_t* Yc = z ? v_intra : k_intra;

    // The split's k-steps: nh over its history part [kb, he), then the rest
    // over its chunk part [cb, ke) (k counted over the active rows).
    const long long Lh = (long long)(*n_sel_p) * g.Tp;
    const long long Lact = Lh + g.Lq;
    const long long per = ((g.L + nsplit - 1) / nsplit + WK - 1) / WK * WK;
    const long long kb = (long long)split * per;
    const long long ke = kb + per < Lact ? kb + per : Lact;
    const long long he = ke < Lh ? ke : Lh;
    const long long cb = kb > Lh ? kb : Lh;
    const int nh = kb < he ? (int)((he - kb + WK - 1) / WK) : 0;
    const int n = nh + (cb < ke ? (int)((ke - cb + WK - 1) / WK) : 0);

    uint32_t off[W_PER];
    w_lanes(off, g, wave, m0, n0);
    const long long xbytes = 2LL * g.r * g.L;

    // Send half-stage hh (X of k-step hh / 2 when hh is even, Y when odd)
    // into ring slot hh % WRING: four DMA instructions per wave, each with a
    // uniform resource and LDS target.
    auto send = [&](int hh) __attribute__((always_inline)) {
        const int s = hh >> 1;
        const bool hist = s < nh;
        const long long k = hist ? kb + (long long)s * WK : cb + (long long)(s - nh) * WK;
        char* buf = ring + (hh % WRING) * WHALF;
        if ((hh & 1) == 0) {
            const long long col = hist ? k : g.hist_rows + (k - Lh);
            const __amdgpu_buffer_rsrc_t rx = w_rsrc(X + col, xbytes - 2 * col);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int j = wave + WWV * q;   // X instruction j < WA_INSTR
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, w_dst(buf + j * 1024), 16, off[q], 0, 0, 0);
            }
        } else {
            const long long end = hist ? he : ke;
            const bf16_t* yb = hist ? Yh + k * g.HD : Yc + (k - Lh) * g.HD;
            const int rows = end - k < WK ? (int)(end - k) : WK;
            const __amdgpu_buffer_rsrc_t ry = w_rsrc(yb, 2LL * rows * g.HD);
#pragma unroll
            for (int q = 4; q < W_PER; ++q) {
                const int j = wave + WWV * q - WA_INSTR;   // Y instruction j
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ry, w_dst(buf + j * 1024), 16, off[q], 0, 0, 0);
            }
        }
    };

    f32x16_t acc[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x16_t{};

    const int halves = 2 * n;
    int sent = halves < WRING ? halves : WRING;
    for (int hh = 0; hh < sent; ++hh) send(hh);
#pragma unroll 1
    for (int i = 0; i < n; ++i) {
        // halves 2i and 2i + 1 have landed once at most the halves sent after
        // them are outstanding (four DMA instructions per wave each); the
        // barrier makes every wave's part visible and retires every read of
        // step i - 1, whose two slots are then refilled
        const int later = sent - (2 * i + 2);
        if (later >= 3)
            wait_vm<12>();
        else if (later == 2)
            wait_vm<8>();
        else if (later == 1)
            wait_vm<4>();
        else
            wait_vm<0>();
        w_barrier();
        const char* xb = ring + ((2 * i) % WRING) * WHALF;
        char* yb = ring + ((2 * i + 1) % WRING) * WHALF;
        const bool hist = i < nh;
        const long long k = hist ? kb + (long long)i * WK : cb + (long long)(i - nh) * WK;
        const long long end = hist ? he : ke;
        if (end - k < WK) {   // the last, partial step of a part
            w_zero_tail(yb, (int)(end - k));
            w_barrier();
        }
        // a half may be sent once the half WRING before it is consumed
        while (sent < halves && sent < 2 * i + WRING) send(sent++);
        w_compute(xb, yb, acc, wave, 0);
        w_compute(xb, yb, acc, wave, 1);
    }

    const int lane = threadIdx.x & 63;
    const int mw = wave & 1, nw = wave >> 1, g2 = lane >> 5;
    float* out = part + (size_t)(split * 2 + z) * g.r * g.HD;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = m0 + 128 * mw + 32 * mt + 8 * (e >> 2) + 4 * g2 + (e & 3);
                const int nn = n0 + 64 * nw + 32 * nt + (lane & 31);
                if (m < g.r) out[(size_t)m * g.HD + nn] = acc[mt][nt][e];
            }
}


bool big_tiles(const Geo& g) { return g.r >= 128 && g.HD % WN == 0; }

}  // namespace

// The MFMA projection needs 16-byte aligned 8-element runs of E's columns
// and of the key rows on both sides of the history/chunk seam.
bool proj32_eligible(const Geo& g) {
    return g.elt == 2 && g.Tp % 8 == 0 && g.Lq % 8 == 0 && g.L % 8 == 0 && g.HD % BN == 0;
}

// Splits per tile: as many work-groups as are resident at once (two per CU
// with 128 x 128 tiles, one with 256 x 256) and no more, so no work-group
// waits for a second round.
int proj32_splits(const Geo& g) {
    const int cus = device_cu_count();
    int s;
    if (big_tiles(g)) {
        const int tiles = 2 * ((g.r + WM - 1) / WM) * (g.HD / WN);
        s = cus / tiles;
    } else {
        const int tiles = 2 * ((g.r + BM - 1) / BM) * (g.HD / BN);
        s = 2 * cus / tiles;
    }
    return s < 1 ? 1 : (s > 32 ? 32 : s);
}

void launch_lowrank_proj32(const Geo& g, const void* E, const void* F, const void* k_hist,
                           const void* v_hist, const void* k_intra, const void* v_intra,
                           const int32_t* n_sel, float* part, hipStream_t st) {
    const int ns = proj32_splits(g);
    if (big_tiles(g)) {
        const int total = ns * 2 * ((g.r + WM - 1) / WM) * (g.HD / WN);
        const int per_xcd = (total + 7) / 8;
        hipLaunchKernelGGL(k_lowrank_proj256, dim3(8 * per_xcd), dim3(WT), 0, st, g, (const bf16_t*)E,
                           (const bf16_t*)F, (const bf16_t*)k_hist, (const bf16_t*)v_hist,
                           (const bf16_t*)k_intra, (const bf16_t*)v_intra, n_sel, ns, per_xcd, part);
        return;
    }
    const int total = ns * 2 * ((g.r + BM - 1) / BM) * (g.HD / BN);
    const int per_xcd = (total + 7) / 8;
    hipLaunchKernelGGL(k_lowrank_proj32, dim3(8 * per_xcd), dim3(NT), 0, st, g, (const bf16_t*)E,
                       (const bf16_t*)F, (const bf16_t*)k_hist, (const bf16_t*)v_hist,
                       (const bf16_t*)k_intra, (const bf16_t*)v_intra, n_sel, ns, per_xcd, part);
}
