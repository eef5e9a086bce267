// Block-sparse attention, bf16, on gfx950 32x32x16 MFMA (HSA sparse branch).
//
// Pages: WorldAttention news summary (ai4snews), HSA paragraph: each query
// block of a head attends, with exact softmax, to the tokens of its own
// selected key blocks only (Binter-token history blocks, Bintra-token chunk
// blocks).
//
// Work decomposition. Query blocks (rows) are taken four at a time: a group
// is four rows of one head, chosen by a plan kernel so that their selections
// overlap (greedy, see k_plan_rows), and its work is the union of the four
// rows' selected blocks, cut into 64-key tiles. A plan kernel writes each group's
// union in ascending block order as one descriptor per tile, and the group
// tile totals are scanned into one global tile sequence. The attention
// kernel then gives work-group k the tiles [kT/G, (k+1)T/G) of that sequence
// (T tiles, G work-groups, one per CU), so every CU gets the same number of
// tiles whatever the rows' selection sizes. A group whose tiles are split
// between work-groups leaves per-segment softmax partials (running max, row
// sum, unnormalised output) that a combine kernel merges in a fixed order.
//
// Work-group = 8 waves = the 4 rows of the current group, 32 queries per wave.
// A tile is loaded once into LDS and each wave computes it only if its own row
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
// Tiles arrive by global -> LDS DMA into a ring of four LDS buffers, sent
// three tiles ahead of the one being computed, so the L2/HBM latency of a
// tile is covered by three tiles of MFMA work and no registers hold data in
// flight. Work-group b runs on XCD b % 8 and takes range (b % 8) * G/8 + b / 8,
// so neighbouring ranges (groups of one head, which select many of the same
// blocks) share an XCD's L2; within a range the tiles are taken in ascending
// block order (see the attention kernel), so those ranges also read nearby
// blocks at the same time. G is one range per CU, or a few per CU for the
// largest heads (ranges_per_wg): an XCD then runs its ranges in launch order,
// one CU's worth at a time.
#include "common.h"
#include "launch.h"

namespace {

constexpr int KT = 64;            // keys per tile
constexpr int R = 4;              // rows (query blocks) per group
constexpr int NW = 2 * R;         // waves per work-group, 32 queries each
static_assert(R <= 8, "a tile descriptor holds the row mask in bits 7..14");
constexpr float kLazyMax = 8.0f;  // margin (log2 units) before the running max is raised
constexpr int kPlanThreads = 256;
constexpr int kSparseMaxWg = 256; // attention work-groups per range pass at most (partials are sized for it)
constexpr int kMaxRangesPerWg = 8;

typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((ext_vector_type(8))) short i16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// LDS tiles are filled by global_load_lds_dwordx4 (global -> LDS DMA, no
// registers): one wave instruction writes 64 lanes x 16 bytes contiguously,
// lane l at base + 16 l. Rows are D bf16 (no padding); the 16-byte slots of
// row r are XOR-swizzled so the MFMA operand reads hit distinct banks:
//   K: slot s of row r holds chunk s ^ (r mod CPR)        (16 rows, one chunk)
//   V: slot s of row r holds chunk s ^ 4 (r mod 4) for D = 128 (a transpose
//      read's 4 rows x 4 chunks per 32 lanes on 16 distinct slots), else
//      chunk s ^ (2r mod CPR)
template <int D>
struct Lay {
    static constexpr int ROWB = D * 2;                    // bytes per key row
    static constexpr int CPR = D / 8;                     // 16-byte chunks per row
    static constexpr int MAT = KT * ROWB;                 // bytes of one K or V tile
    static constexpr int BUF = 2 * MAT;                   // K tile then V tile
    static constexpr int INSTR = KT * CPR / 64;           // wave instructions per matrix
    static constexpr int PER_WAVE = INSTR / NW;           // per wave and matrix
    static constexpr int VM_PER_TILE = 2 * PER_WAVE;      // vector-memory ops per wave and tile
    static_assert(INSTR % NW == 0, "DMA instructions split evenly over the waves");
    HSAKV_DEV static int swz_k(int r) { return r & (CPR - 1); }
    HSAKV_DEV static int swz_v(int r) { return CPR == 16 ? 4 * (r & 3) : (2 * r) & (CPR - 1); }
};

// This wave's DMA lanes, fixed over the tiles: instruction j covers slots
// (wave PER_WAVE + j) 64 + lane, i.e. key row r and, after the swizzle, the
// 16-byte chunk ck (K) / cv (V) of that row (byte offsets within the row).
template <int D>
struct DmaLanes {
    int r[Lay<D>::PER_WAVE], ck[Lay<D>::PER_WAVE], cv[Lay<D>::PER_WAVE];
};

template <int D>
HSAKV_DEV void dma_lanes(DmaLanes<D>& dl, int wave) {
    using LY = Lay<D>;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < LY::PER_WAVE; ++j) {
        const int L = (wave * LY::PER_WAVE + j) * 64 + lane;
        const int r = L / LY::CPR, sl = L % LY::CPR;
        dl.r[j] = r;
        dl.ck[j] = (sl ^ LY::swz_k(r)) << 4;
        dl.cv[j] = (sl ^ LY::swz_v(r)) << 4;
    }
}

// The LDS byte address of a ring buffer as a value the compiler cannot trace
// back to the buffer, for the tile DMA. The kernel orders every DMA before the
// reads of its buffer itself (a vmcnt wait on the tiles sent, then the
// work-group barrier); the compiler's own tracking of LDS DMA targets, which
// merges the paths of a partly filled ring, would add waits that drain the
// tiles in flight too.
HSAKV_DEV uint32_t dma_base(char* p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_t*)p);
}

// DMA one tile (64 key rows of K and V) into an LDS buffer. Rows past `nvalid`
// (the ragged end of a block) load the last valid row: their scores are
// masked to -inf, so P = 0 multiplies finite values. The DMA goes through
// buffer loads (raw buffer, base = the tile's first row): the compiler counts
// those as vector memory only, so the LDS operand reads that follow keep
// exact lgkmcnt waits and can be issued ahead of their MFMAs (a pending
// global_load_lds makes every LDS read wait for all earlier ones).
template <int D>
HSAKV_DEV void dma_tile(uint32_t buf, const bf16_t* kb, const bf16_t* vb, int nvalid, int row_bytes,
                        const DmaLanes<D>& dl, int wave) {
    using LY = Lay<D>;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(kb), 0, -1, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(vb), 0, -1, 0x00020000);
#pragma unroll
    for (int j = 0; j < LY::PER_WAVE; ++j) {
        const int slot0 = (wave * LY::PER_WAVE + j) * 64;
        const int rg = dl.r[j] < nvalid ? dl.r[j] : nvalid - 1;
        const int ro = (int)__umul24((unsigned)rg, (unsigned)row_bytes);   // rg < 64, row_bytes < 2^24
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(uintptr_t)(buf + slot0 * 16), 16, ro + dl.ck[j], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(uintptr_t)(buf + LY::MAT + slot0 * 16), 16,
                                                 ro + dl.cv[j], 0, 0, 0);
    }
}

// s_waitcnt vmcnt(N) with the other counters unconstrained (gfx9 encoding:
// vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8]).
template <int N>
HSAKV_DEV void wait_vmcnt() {
    static_assert(N >= 0 && N < 16, "vmcnt immediate");
    __builtin_amdgcn_s_waitcnt(0x0f70 | N);
}

// Work-group barrier that orders LDS only: this wave's LDS accesses are
// complete, while its global loads and LDS DMA still in flight stay in flight
// (a full __syncthreads would wait for them). The memory clobber keeps the
// compiler from moving memory accesses across it.
HSAKV_DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int D>
struct Wave {
    static constexpr int KS = D / 16;   // 16-wide k steps of S^T = K Q^T
    static constexpr int DT = D / 32;   // 32-row tiles of O^T
    bf16x8_t qf[KS];
    f32x16_t o[DT];
    float m, l;                         // running max (log2 units), this lane's share of the row sum
};

// Online softmax over a whole 64-key tile, both 32-key halves at once: mask
// the keys past `nvalid`, update the running max once per tile (raised only
// when a score passes it by more than kLazyMax, so O is rarely rescaled;
// weights stay below 2^kLazyMax) and turn the scores into weights. One
// update per tile rather than per half saves a cross-lane max, a threshold
// test and their hazard waits per tile.
template <int D>
HSAKV_DEV void softmax_tile(Wave<D>& w, f32x16_t (&s)[2], int nvalid, float scale_log2) {
    const int g2 = (threadIdx.x & 63) >> 5;
    if (nvalid < 64) {
        // element i of half sub holds key 32 sub + 4 g2 + 8 (i / 4) + i % 4: valid below t
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
            const int t = nvalid - 32 * sub - 4 * g2;
#pragma unroll
            for (int i = 0; i < 16; ++i) s[sub][i] = 8 * (i >> 2) + (i & 3) < t ? s[sub][i] : -INFINITY;
        }
    }
    // raw scores: the max is taken before scaling (scale > 0), and the scale
    // folds into the exponent's FMA. The NaN-propagating maximum maps to a
    // chain of three-input max instructions with no operand quieting (a NaN
    // score makes its row NaN either way, through its own weight)
    float mx = __builtin_elementwise_maximum(s[0][0], s[1][0]);
#pragma unroll
    for (int i = 1; i < 16; ++i)
        mx = __builtin_elementwise_maximum(mx, __builtin_elementwise_maximum(s[0][i], s[1][i]));
    // lanes l and l + 32 hold the two key quarters of the same query
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = __builtin_elementwise_maximum(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    const float mt = mx * scale_log2;
    const bool moved = mt > w.m + kLazyMax;
    const float m_old = w.m;
    const float m_new = moved ? mt : m_old;
    w.m = m_new;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[sub][i] = fast_exp2(fmaf(s[sub][i], scale_log2, -m_new));
    // the weights are added to the row sum by pv_half, as rounded for the
    // MFMA; the row sum and O are rescaled only when some running max of the
    // wave was raised (the factor is 1 in every other lane)
    if (__builtin_amdgcn_ballot_w64(moved)) {
        const float alpha = moved ? fast_exp2(m_old - m_new) : 1.0f;
        w.l *= alpha;
#pragma unroll
        for (int dt = 0; dt < Wave<D>::DT; ++dt) w.o[dt] *= alpha;
    }
}

// Scheduling groups (instruction classes of __builtin_amdgcn_sched_group_barrier).
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100;

// O^T += V^T P^T over one 32-key half of the tile, and the half's weights
// (bf16, as the MFMA takes them) added to this lane's share of the row sum by
// dot products with ones. The V^T operands are read two MFMAs ahead of their
// use, so the LDS latency hides behind the matrix work.
template <int D>
HSAKV_DEV void pv_half(Wave<D>& w, const f32x16_t& s, const char* vt, int sub) {
    using LY = Lay<D>;
    constexpr int DT = Wave<D>::DT;
    const int lane = threadIdx.x & 63;
    const int G = lane >> 4, j = lane & 15;
    // the weights as bf16 pairs, one packed conversion each; the row sum is
    // taken on the same pairs
    bf16x2_t pp[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) pp[i] = __builtin_convertvector((f32x2_t){s[2 * i], s[2 * i + 1]}, bf16x2_t);
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
    i16x4_t lo[2][DT], hi[2][DT];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int krow = 32 * sub + 16 * c + 4 * (G >> 1) + (j >> 2);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const int dcol = 32 * dt + 16 * (G & 1) + 4 * (j & 3);
            const int lo_off = krow * LY::ROWB + (((dcol >> 3) ^ LY::swz_v(krow)) << 4) + ((dcol & 7) << 1);
            const int hi_off = (krow + 8) * LY::ROWB + (((dcol >> 3) ^ LY::swz_v(krow + 8)) << 4) +
                               ((dcol & 7) << 1);
            lo[c][dt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vt + lo_off));
            hi[c][dt] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(vt + hi_off));
        }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            const i16x8_t vv = __builtin_shufflevector(lo[c][dt], hi[c][dt], 0, 1, 2, 3, 4, 5, 6, 7);
            w.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, vv), pf[c], w.o[dt], 0, 0, 0);
        }
    // 4 reads ahead, then one MFMA per two reads, then the last two MFMAs
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
    for (int m = 0; m < 2 * DT - 2; ++m) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
}

// One 64-key tile: S of both 32-key halves, one online-softmax step over the
// 64 keys, then P V of both halves. The VALU block of one wave runs beside
// the matrix work of the other wave on its SIMD.
template <int D>
HSAKV_DEV void tile_step(Wave<D>& w, const char* kt, const char* vt, int nvalid, float scale_log2) {
    using LY = Lay<D>;
    const int lane = threadIdx.x & 63;
    const int r32 = lane & 31, g2 = lane >> 5;
    constexpr int KS = Wave<D>::KS;
    // K operands read four MFMAs ahead of their use
    bf16x8_t a[2][KS];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int row = 32 * sub + r32;
            a[sub][ks] = *reinterpret_cast<const bf16x8_t*>(kt + row * LY::ROWB + (((2 * ks + g2) ^ LY::swz_k(row)) << 4));
        }
    f32x16_t s[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
        s[sub] = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s[sub] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[sub][ks], w.qf[ks], s[sub], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 0);
#pragma unroll
    for (int m = 0; m < 2 * KS - 4; ++m) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 0);
    softmax_tile<D>(w, s, nvalid, scale_log2);
    pv_half<D>(w, s[0], vt, 0);
    pv_half<D>(w, s[1], vt, 1);
}

// Key block b -> token range and source (history blocks first, then chunk blocks).
struct Cursor {
    long long t0;   // first token of the block
    int len;        // valid tokens of the block
    bool hist;
};

HSAKV_DEV Cursor open_block(const Geo& g, int NBh, long long Lh, int b) {
    Cursor c;
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
    return c;
}

HSAKV_DEV int groups_per_head(const Geo& g) { return (g.NQB + R - 1) / R; }

// Largest index i in [0, n) with a[i] <= x, for nondecreasing a with
// a[0] <= x: a 64-way search by one wave (uniform result).
HSAKV_DEV int last_le(const int32_t* __restrict__ a, int n, int x) {
    const int lane = threadIdx.x & 63;
    int lo = 0, hi = n;
    while (hi - lo > 1) {
        const int step = (hi - lo + 63) / 64;
        const int idx = lo + lane * step;
        const bool ok = idx < hi && a[idx] <= x;
        const unsigned long long m = __builtin_amdgcn_ballot_w64(ok);
        const int jl = 63 - __builtin_clzll(m);   // lane 0 always qualifies
        lo += jl * step;
        hi = lo + step < hi ? lo + step : hi;
    }
    return lo;
}

// Exclusive scan of one int per thread over a work-group of NT threads;
// *tot receives the sum over the work-group.
template <int NT>
HSAKV_DEV int block_excl_scan(int v, int* tot, int* wsum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int s = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(s, o, 64);
        if (lane >= o) s += t;
    }
    if (lane == 63) wsum[wave] = s;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
        const int x = wsum[w];
        before += w < wave ? x : 0;
        all += x;
    }
    __syncthreads();
    *tot = all;
    return before + s - v;
}

// ---- plan ------------------------------------------------------------------

// Rows of each head are grouped R at a time so that a group's rows select
// mostly the same blocks: the union walk then spends few steps on blocks only
// some rows selected. Greedy, per head: a group starts from the lowest row
// not yet grouped and takes, R - 1 times, the remaining row whose selection
// shares the most tiles with the group's union less the tiles it would add.
// grows[grp * R + r] = row (NQB past the head's rows). The row bitmasks take
// W words (W = 32: at most 1024 tiles per head; 64: at most 2048) and a lane
// holds RPL rows (2: at most 128 rows per head; 4: at most 256); heads past
// the largest of these keep consecutive rows. The grouping only orders the
// work: each row's result is the same.

// Tiles of the head's key blocks, history blocks first: block b < NBh covers
// tiles [th b, th (b + 1)), chunk block NBh + c covers th NBh + tc c onwards.
HSAKV_DEV int tiles_of_head(const Geo& g, int NBh, int& th, int& tc) {
    th = (g.Binter + KT - 1) / KT;
    tc = (g.Bintra + KT - 1) / KT;
    return th * NBh + tc * g.NBc;
}

// Selection of one row as a tile bitmask: work-group (h, i) writes
// tbits[(h NQB + i) W + w], bit t % 32 of word t / 32 set when the row
// selected the block of tile t.
template <int W>
__global__ void __launch_bounds__(64)
k_plan_bits(Geo g, const int32_t* __restrict__ n_sel_p, const int32_t* __restrict__ sel_count,
            const int32_t* __restrict__ sel_idx, uint32_t* __restrict__ tbits) {
    static_assert(W <= 64, "one word per lane");
    __shared__ uint32_t words[W];
    const int row = blockIdx.x, lane = threadIdx.x;
    const int n_sel = *n_sel_p;
    const int NBh = hist_blocks(g, n_sel);
    const int NB = NBh + g.NBc;
    int th, tc;
    if (tiles_of_head(g, NBh, th, tc) > 32 * W) return;
    if (lane < W) words[lane] = 0u;
    __syncthreads();
    const int c = sel_count[row];
    const int32_t* ids = sel_idx + (size_t)row * g.NB_max;
    for (int j = lane; j < c; j += 64) {
        const int b = ids[j];
        if (b < 0 || b >= NB) continue;
        const int t0 = b < NBh ? th * b : th * NBh + tc * (b - NBh);
        const int nt = b < NBh ? th : tc;
        for (int t = t0; t < t0 + nt; ++t) atomicOr(&words[t >> 5], 1u << (t & 31));
    }
    __syncthreads();
    if (lane < W) tbits[(size_t)row * W + lane] = words[lane];
}

// Largest value over the wave, in every lane: DPP rotations within each row
// of 16 lanes, then the row pairs (lanes l, l ^ 16) and halves (l, l ^ 32)
// through the gfx950 lane swaps.
HSAKV_DEV uint32_t wave_max_u32(uint32_t v) {
    auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, false));   // row_ror:8
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, false));   // row_ror:4
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xf, 0xf, false));   // row_ror:2
    v = mx(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xf, 0xf, false));   // row_ror:1
    const auto s16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = mx(s16[0], s16[1]);
    const auto s32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return mx(s32[0], s32[1]);
}

// One work-group per head, kGroupWaves waves: lane l of every wave holds rows
// l, l + 64, ... (RPL of them), wave v holds words [W/4 v, W/4 (v + 1)) of
// their bitmasks. The waves sum their partial overlaps through LDS; every
// wave then takes the same pick.
constexpr int kGroupWaves = 4;

template <int W, int RPL>
__global__ void __launch_bounds__(64 * kGroupWaves)
k_plan_rows(Geo g, const int32_t* __restrict__ n_sel_p, const uint32_t* __restrict__ tbits,
            int32_t* __restrict__ grows) {
    constexpr int kWordsPerWave = W / kGroupWaves;
    constexpr int kGroupRowsPerLane = RPL;
    static_assert(RPL <= 4, "row ids of a head fit the 8-bit field of the pick key");
    __shared__ int part[2][kGroupWaves][64 * kGroupRowsPerLane];
    const int h = blockIdx.x, lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int gph = groups_per_head(g);
    const int n_sel = *n_sel_p;
    const int NBh = hist_blocks(g, n_sel);
    int th, tc;
    const int NT = tiles_of_head(g, NBh, th, tc);
    int32_t* out = grows + (size_t)h * gph * R;
    if (NT > 32 * W || g.NQB > 64 * kGroupRowsPerLane) {
        for (int e = threadIdx.x; e < gph * R; e += 64 * kGroupWaves) out[e] = e < g.NQB ? e : g.NQB;
        return;
    }
    const int Wn = (NT + 31) >> 5;   // words in use
    uint32_t bits[kGroupRowsPerLane][kWordsPerWave];
    bool left[kGroupRowsPerLane];
#pragma unroll
    for (int k = 0; k < kGroupRowsPerLane; ++k) {
        const int row = lane + 64 * k;
        left[k] = row < g.NQB;
        const uint32_t* src = tbits + (size_t)(h * g.NQB + (left[k] ? row : 0)) * W;
        int cnt = 0;
#pragma unroll
        for (int x = 0; x < kWordsPerWave; ++x) {
            const int w = kWordsPerWave * wv + x;
            bits[k][x] = left[k] && w < Wn ? src[w] : 0u;
            cnt += __builtin_popcount(bits[k][x]);
        }
        part[1][wv][row] = cnt;
    }
    __syncthreads();
    int own[kGroupRowsPerLane];
#pragma unroll
    for (int k = 0; k < kGroupRowsPerLane; ++k) {
        own[k] = 0;
#pragma unroll
        for (int v = 0; v < kGroupWaves; ++v) own[k] += part[1][v][lane + 64 * k];
    }
    uint32_t uni[kWordsPerWave];
#pragma unroll
    for (int x = 0; x < kWordsPerWave; ++x) uni[x] = 0u;
    int buf = 0;
    for (int j = 0; j < gph; ++j) {
        for (int r = 0; r < R; ++r) {
            // partial overlaps of this wave's words with the group's union
            if (r > 0) {
#pragma unroll
                for (int k = 0; k < kGroupRowsPerLane; ++k) {
                    int ov = 0;
#pragma unroll
                    for (int x = 0; x < kWordsPerWave; ++x) ov += __builtin_popcount(bits[k][x] & uni[x]);
                    part[buf][wv][lane + 64 * k] = ov;
                }
                __syncthreads();
            }
            // key: score (shared tiles less added tiles) above the lowest row
            uint32_t key = 0;
#pragma unroll
            for (int k = 0; k < kGroupRowsPerLane; ++k) {
                if (!left[k]) continue;
                int score = 0;
                if (r > 0) {
                    int ov = 0;
#pragma unroll
                    for (int v = 0; v < kGroupWaves; ++v) ov += part[buf][v][lane + 64 * k];
                    score = 2 * ov - own[k];
                }
                const uint32_t kk = ((uint32_t)(score + 4096) << 8) | (uint32_t)(255 - (lane + 64 * k));
                key = kk > key ? kk : key;
            }
            key = wave_max_u32(key);
            if (r > 0) buf ^= 1;
            const int pick = key ? 255 - (int)(key & 255u) : g.NQB;
            if (threadIdx.x == 0) out[j * R + r] = pick;
            if (!key) continue;
            const int pl_ = pick & 63, pk = pick >> 6;
#pragma unroll
            for (int x = 0; x < kWordsPerWave; ++x) {
                uint32_t v = bits[0][x];
#pragma unroll
                for (int k = 1; k < kGroupRowsPerLane; ++k) v = pk == k ? bits[k][x] : v;   // fixed indices
                const uint32_t bw = (uint32_t)__builtin_amdgcn_readlane((int)v, pl_);
                uni[x] = r == 0 ? bw : (uni[x] | bw);
            }
#pragma unroll
            for (int k = 0; k < kGroupRowsPerLane; ++k)
                if (k == pk && lane == pl_) left[k] = false;   // fixed indices: `left` stays in registers
        }
    }
}

// Union of the selected blocks of one group's rows, in ascending block order,
// as one descriptor per 64-key tile: tdesc[grp * tpg + t] = (first token row
// of the tile in its source, valid keys | row mask << 7 | 1 << 15 for a
// history tile).
__global__ void __launch_bounds__(kPlanThreads)
k_plan_groups(Geo g, const int32_t* __restrict__ n_sel_p, const int32_t* __restrict__ sel_count,
              const int32_t* __restrict__ sel_idx, const int32_t* __restrict__ grows, int2* __restrict__ tdesc,
              int tpg, int32_t* __restrict__ gcount, int32_t* __restrict__ gtiles) {
    __shared__ int mask[4096];
    __shared__ int wsum[2][kPlanThreads / 64];
    const int grp = blockIdx.x, tid = threadIdx.x;
    const int gph = groups_per_head(g);
    const int h = grp / gph;
    const int n_sel = *n_sel_p;
    const int NBh = hist_blocks(g, n_sel);
    const int NB = NBh + g.NBc;
    const long long Lh = (long long)n_sel * g.Tp;
    for (int b = tid; b < NB; b += kPlanThreads) mask[b] = 0;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = grows[grp * R + r];
        if (i >= g.NQB) continue;
        const int row = h * g.NQB + i;
        const int c = sel_count[row];
        const int32_t* ids = sel_idx + (size_t)row * g.NB_max;
        for (int j = tid; j < c; j += kPlanThreads) {
            const int b = ids[j];
            if (b >= 0 && b < NB) atomicOr(&mask[b], 1 << r);
        }
    }
    __syncthreads();
    const int per = (NB + kPlanThreads - 1) / kPlanThreads;
    const int b0 = tid * per, b1 = b0 + per < NB ? b0 + per : NB;
    int ne = 0, nt = 0;
    for (int b = b0; b < b1; ++b)
        if (mask[b]) {
            ++ne;
            nt += (open_block(g, NBh, Lh, b).len + KT - 1) / KT;
        }
    int ce_tot, ct_tot;
    block_excl_scan<kPlanThreads>(ne, &ce_tot, wsum[0]);
    int ct = block_excl_scan<kPlanThreads>(nt, &ct_tot, wsum[1]);
    int2* td = tdesc + (size_t)grp * tpg;
    for (int b = b0; b < b1; ++b) {
        const int mk = mask[b];
        if (mk) {
            const Cursor c = open_block(g, NBh, Lh, b);
            for (int t = 0; t * KT < c.len; ++t) {
                const int nvalid = c.len - t * KT < KT ? c.len - t * KT : KT;
                td[ct++] = int2{(int)(c.t0 + (long long)t * KT), nvalid | (mk << 7) | (c.hist ? 1 << 15 : 0)};
            }
        }
    }
    if (tid == 0) {
        gcount[grp] = ce_tot;
        gtiles[grp] = ct_tot;
    }
}

// gstart[p] = tiles of the groups before p; gstart[NG] = all tiles.
__global__ void __launch_bounds__(1024) k_plan_scan(int NG, const int32_t* __restrict__ gtiles,
                                                    int32_t* __restrict__ gstart) {
    __shared__ int wsum[16];
    int carry = 0;
    for (int base = 0; base < NG; base += 1024) {
        const int p = base + threadIdx.x;
        const int v = p < NG ? gtiles[p] : 0;
        int tot;
        const int ex = block_excl_scan<1024>(v, &tot, wsum);
        if (p < NG) gstart[p] = carry + ex;
        carry += tot;
    }
    if (threadIdx.x == 0) gstart[NG] = carry;
}

// ---- attention ---------------------------------------------------------------

struct PlanArgs {
    float* part_o;          // [G][2][NW][DT][64 lanes][16]: unnormalised O of split groups
    float2* part_ml;        // [G][2][NW][64 lanes]: (running max, lane's row-sum share)
    const int32_t* grows;   // [NG][R]: rows of each group (NQB past the head's rows)
    int NG, G;
};

HSAKV_DEV int range_start(long long k, int T, int G) { return (int)(k * T / G); }

// Loads the 32 queries of this wave (zeros past the chunk) and clears the state.
template <int D>
HSAKV_DEV void start_rows(const Geo& g, const bf16_t* __restrict__ q, int h, int i, Wave<D>& w) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int query = i * g.Bq + 32 * (wave & 1) + (lane & 31);
    const bool ok = i < g.NQB && query < g.Lq;
    const bf16_t* qp = q + (long long)(ok ? query : 0) * g.HD + (long long)h * D + 8 * (lane >> 5);
#pragma unroll
    for (int ks = 0; ks < Wave<D>::KS; ++ks)
        w.qf[ks] = ok ? *reinterpret_cast<const bf16x8_t*>(qp + 16 * ks) : bf16x8_t{};
#pragma unroll
    for (int dt = 0; dt < Wave<D>::DT; ++dt) w.o[dt] = f32x16_t{};
    w.m = -INFINITY;
    w.l = 0.f;
}

// O / l and the optional gated fusion with the low-rank branch.
template <int D>
HSAKV_DEV void finish_rows(const Geo& g, const Epi& ep, int h, int i, const Wave<D>& w) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g2 = lane >> 5;
    const int query = i * g.Bq + 32 * (wave & 1) + (lane & 31);
    const float lt = w.l + __shfl_xor(w.l, 32, 64);
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
    if (i >= g.NQB || query >= g.Lq) return;
    const long long base = (long long)query * g.HD + (long long)h * D;
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

template <int D>
HSAKV_DEV size_t part_index(int slot, int wave, int dt, int lane) {
    return ((((size_t)slot * NW + wave) * Wave<D>::DT + dt) * 64 + lane) * 16;
}

// Work-group k computes tiles [kT/G, (k+1)T/G) of the global tile sequence.
template <int D>
__global__ void __launch_bounds__(64 * NW)
k_sparse_attn32(Geo g, const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_hist,
                const bf16_t* __restrict__ v_hist, const bf16_t* __restrict__ k_intra,
                const bf16_t* __restrict__ v_intra, const int32_t* __restrict__ n_sel_p,
                const int2* __restrict__ tdesc, int tpg,
                const int32_t* __restrict__ gcount, const int32_t* __restrict__ gtiles,
                const int32_t* __restrict__ gstart, PlanArgs pl, int per_xcd, Epi ep) {
    using LY = Lay<D>;
    // four distinct LDS objects with fixed roles per unrolled step: the
    // compiler can tell the tiles' DMA from the reads and inserts no wait
    __shared__ __attribute__((aligned(16))) char lds0[LY::BUF];
    __shared__ __attribute__((aligned(16))) char lds1[LY::BUF];
    __shared__ __attribute__((aligned(16))) char lds2[LY::BUF];
    __shared__ __attribute__((aligned(16))) char lds3[LY::BUF];
    const int b = blockIdx.x;
    const int k = (b & 7) * per_xcd + (b >> 3);
    if (k >= pl.G) return;
    const int T = gstart[pl.NG];
    const int a0 = range_start(k, T, pl.G), a1 = range_start(k + 1, T, pl.G);
    const int total = a1 - a0;
    if (total <= 0) return;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int myr = wave >> 1;
    const float scale_log2 = 1.4426950408889634f / sqrtf((float)D);
    const int gph = groups_per_head(g);
    DmaLanes<D> dl;
    dma_lanes<D>(dl, wave);
    const uint32_t b0 = dma_base(lds0), b1 = dma_base(lds1), b2 = dma_base(lds2), b3 = dma_base(lds3);

    // The range holds pieces of consecutive groups: the tail of the first
    // (its highest blocks) when the range starts inside it, whole groups, and
    // the head of the last (its lowest blocks). A range that starts inside a
    // group and runs past it takes the later groups first and that first
    // tail last, so it sweeps the blocks from low to high indices, in step
    // with the other ranges: the work-groups of an XCD then read nearby
    // blocks at the same time and share them in L2.
    const int g0 = last_le(gstart, pl.NG, a0);
    const bool wrap = a0 > gstart[g0] && gstart[g0] + gtiles[g0] < a1;
    auto next_group = [&](int p) __attribute__((always_inline)) -> int {
        do {
            ++p;
        } while (p < pl.NG && gcount[p] == 0);
        return p;
    };
    int pg = wrap ? next_group(g0) : g0;

    Wave<D> w;
    int done = 0;     // tiles of the range computed
    while (true) {
        // one group per pass: its tiles [lo, hi) of this range, with the ring
        // refilled from the first buffer (a pipeline drain per group change)
        const int grp = pg;
        const int h = grp / gph, i = pl.grows[grp * R + myr];
        const int S = gstart[grp], Tg = gtiles[grp];
        const int lo = S > a0 ? S : a0, hi = S + Tg < a1 ? S + Tg : a1;
        const int end = hi - lo;
        // the piece's tile descriptors; the next one to send is loaded at the
        // end of the step before, so its latency hides under that step's MFMAs
        const int2* td = tdesc + (size_t)grp * tpg + (lo - S);
        int2 dnext = td[0];
        int n = 0;        // tiles of the piece computed
        int issued = 0;   // tiles of the piece sent
        const long long hoff = (long long)h * D;
        start_rows<D>(g, q, h, i, w);
        // tile info for the consumer: row mask << 7 | valid keys
        int info0 = 0, info1 = 0, info2 = 0, info3 = 0;
        auto issue = [&](uint32_t dst) __attribute__((always_inline)) -> int {
            const int2 d = dnext;
            ++issued;
            const long long roff = hoff + (long long)d.x * g.HD;
            const bool hist = (d.y >> 15) & 1;
            dma_tile<D>(dst, (hist ? k_hist : k_intra) + roff, (hist ? v_hist : v_intra) + roff, d.y & 127,
                        2 * g.HD, dl, wave);
            return d.y & 0x7fff;   // row mask << 7 | valid keys
        };
        info0 = issue(b0);
        if (issued < end) {
            dnext = td[issued];
            info1 = issue(b1);
        }
        if (issued < end) {
            dnext = td[issued];
            info2 = issue(b2);
        }
        if (issued < end) dnext = td[issued];
        auto step = [&](const char* now, uint32_t nxt, int inf, int& inf_nxt) __attribute__((always_inline)) {
            // this wave's DMA of tile n has landed once at most the tiles sent
            // after it are outstanding; the barrier makes every wave's part
            // visible and retires every read of `nxt` (tile n - 1)
            const int later = issued - n - 1;
            if (later >= 2)
                wait_vmcnt<2 * LY::VM_PER_TILE>();
            else if (later == 1)
                wait_vmcnt<LY::VM_PER_TILE>();
            else
                wait_vmcnt<0>();
            lds_barrier();
            if (issued < end) inf_nxt = issue(nxt);
            if ((inf >> (7 + myr)) & 1) tile_step<D>(w, now, now + LY::MAT, inf & 127, scale_log2);
            if (issued < end) dnext = td[issued];
        };
        while (true) {
            step(lds0, b3, info0, info3);
            if (++n == end) break;
            step(lds1, b0, info1, info0);
            if (++n == end) break;
            step(lds2, b1, info2, info1);
            if (++n == end) break;
            step(lds3, b2, info3, info2);
            if (++n == end) break;
        }
        if (S >= a0 && S + Tg <= a1) {
            finish_rows<D>(g, ep, h, i, w);
        } else {
            const int slot = 2 * k + (grp == g0 ? 0 : 1);
            const int lane = threadIdx.x & 63;
#pragma unroll
            for (int dt = 0; dt < Wave<D>::DT; ++dt) {
                float4* po = reinterpret_cast<float4*>(pl.part_o + part_index<D>(slot, wave, dt, lane));
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    po[c] = float4{w.o[dt][4 * c], w.o[dt][4 * c + 1], w.o[dt][4 * c + 2], w.o[dt][4 * c + 3]};
            }
            pl.part_ml[((size_t)slot * NW + wave) * 64 + lane] = float2{w.m, w.l};
        }
        done += end;
        if (done == total) break;
        // next piece; every wave is done with the ring before it refills
        pg = next_group(pg);
        if (wrap && (pg >= pl.NG || gstart[pg] >= a1)) pg = g0;
        lds_barrier();
    }
}

// Groups split between work-groups: merge the segment partials in range order,
// then the same epilogue. Groups without tiles get O = 0. One work-group per
// (group, row wave) and one wave per 32-row tile of O^T: a thread holds 16
// outputs, so many waves keep their partial loads in flight at once. The
// gate's dot product is split over the waves (two 16-wide column steps each)
// and added in wave order through LDS.
template <int D>
__global__ void __launch_bounds__(64 * Wave<D>::DT)
k_sparse_combine(Geo g, const bf16_t* __restrict__ q, const int32_t* __restrict__ gtiles,
                 const int32_t* __restrict__ gstart, PlanArgs pl, Epi ep) {
    constexpr int DT = Wave<D>::DT;
    const int grp = blockIdx.x, wave = blockIdx.y;
    const int dt = threadIdx.x >> 6, lane = threadIdx.x & 63, g2 = lane >> 5;
    const int T = gstart[pl.NG];
    const int S = gstart[grp], Tg = gtiles[grp];
    const int G = pl.G;
    int k0 = 0;
    if (Tg > 0) {
        // the range holding the group's first tile: largest k with start <= S
        k0 = (int)((long long)S * G / T);
        while (k0 + 1 < G && range_start(k0 + 1, T, G) <= S) ++k0;
        while (k0 > 0 && range_start(k0, T, G) > S) --k0;
        if (range_start(k0 + 1, T, G) >= S + Tg) return;   // one range holds the whole group
    }
    const int gph = groups_per_head(g);
    const int h = grp / gph, i = pl.grows[grp * R + (wave >> 1)];
    const int query = i * g.Bq + 32 * (wave & 1) + (lane & 31);
    const bool ok = i < g.NQB && query < g.Lq;
    __shared__ float gpart[DT][64];
    // the low-rank output this thread blends, loaded first so that its
    // latency overlaps that of the partials
    float4 lin[4] = {};
    if (ep.out && ok) {
        const float* lp = ep.o_lin + (long long)query * g.HD + (long long)h * D + 32 * dt + 4 * g2;
#pragma unroll
        for (int a = 0; a < 4; ++a) lin[a] = *reinterpret_cast<const float4*>(lp + 8 * a);
    }
    if (ep.out) {
        float dot = 0.f;
        if (ok) {
            const bf16_t* qp = q + (long long)query * g.HD + (long long)h * D + 8 * g2;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int ks = 2 * dt + u;
                const bf16x8_t qv = *reinterpret_cast<const bf16x8_t*>(qp + 16 * ks);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    dot = fmaf((float)qv[e], ep.w_g[h * D + 16 * ks + 8 * g2 + e], dot);
            }
        }
        gpart[dt][lane] = dot;
    }
    float o[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = 0.f;
    float m = -INFINITY, l = 0.f;
    if (Tg > 0) {
        for (int kk = k0; kk < G; ++kk) {
            const int s0 = range_start(kk, T, G);
            if (s0 >= S + Tg) break;
            if (range_start(kk + 1, T, G) == s0) continue;   // empty range
            const int slot = 2 * kk + (s0 < S ? 1 : 0);
            const float2 ml = pl.part_ml[((size_t)slot * NW + wave) * 64 + lane];
            const float4* po = reinterpret_cast<const float4*>(pl.part_o + part_index<D>(slot, wave, dt, lane));
            float4 v[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) v[c] = po[c];
            const float m_new = fmaxf(m, ml.x);
            const float a_old = m == -INFINITY ? 0.f : exp2f(m - m_new);
            const float a_seg = ml.x == -INFINITY ? 0.f : exp2f(ml.x - m_new);
            m = m_new;
            l = l * a_old + ml.y * a_seg;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                o[4 * c] = o[4 * c] * a_old + v[c].x * a_seg;
                o[4 * c + 1] = o[4 * c + 1] * a_old + v[c].y * a_seg;
                o[4 * c + 2] = o[4 * c + 2] * a_old + v[c].z * a_seg;
                o[4 * c + 3] = o[4 * c + 3] * a_old + v[c].w * a_seg;
            }
        }
    }
    float gate = 0.f;
    if (ep.out) {
        __syncthreads();
        float dot = gpart[0][lane];
#pragma unroll
        for (int k = 1; k < DT; ++k) dot += gpart[k][lane];
        dot += __shfl_xor(dot, 32, 64);
        const float x = dot + ep.b_g[h];
        const float z = expf(-fabsf(x));
        gate = x >= 0.f ? 1.0f / (1.0f + z) : z / (1.0f + z);
    }
    const float lt = l + __shfl_xor(l, 32, 64);
    const float inv_l = lt > 0.f ? 1.0f / lt : 0.f;
    if (!ok) return;
    const long long base = (long long)query * g.HD + (long long)h * D;
    if (ep.gate && g2 == 0 && dt == 0) ep.gate[(long long)query * g.H + h] = gate;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int d0 = 32 * dt + 8 * a + 4 * g2;
        const float4 r = {o[4 * a] * inv_l, o[4 * a + 1] * inv_l, o[4 * a + 2] * inv_l, o[4 * a + 3] * inv_l};
        if (ep.o_main) *reinterpret_cast<float4*>(ep.o_main + base + d0) = r;
        if (ep.out) {
            const float r0 = gate * r.x + (1.f - gate) * lin[a].x;
            const float r1 = gate * r.y + (1.f - gate) * lin[a].y;
            const float r2 = gate * r.z + (1.f - gate) * lin[a].z;
            const float r3 = gate * r.w + (1.f - gate) * lin[a].w;
            uint2 pk;
            pk.x = (uint32_t)f32_to_bf16(r0) | ((uint32_t)f32_to_bf16(r1) << 16);
            pk.y = (uint32_t)f32_to_bf16(r2) | ((uint32_t)f32_to_bf16(r3) << 16);
            *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(ep.out) + base + d0) = pk;
        }
    }
}

// Attention work-groups running at once on the current device: one per CU, at
// most kSparseMaxWg.
int sparse_wgs() {
    const int cus = device_cu_count();
    return cus < kSparseMaxWg ? cus : kSparseMaxWg;
}

size_t al256(size_t x) { return (x + 255) / 256 * 256; }

struct SparseWs {
    uint32_t* tbits;
    int32_t* grows;
    int2* tdesc;
    int32_t *gcount, *gtiles, *gstart;
    float* part_o;
    float2* part_ml;
};

int n_groups(const Geo& g) { return g.H * ((g.NQB + R - 1) / R); }
// Bitmask words per row of the row grouping: 32 up to 1024 tiles per head
// (every history slot present), 64 up to 2048; past that the grouping keeps
// consecutive rows and the bitmasks go unused.
int plan_words(const Geo& g) {
    const int tiles = ((g.Binter + KT - 1) / KT) * g.NBh_max + ((g.Bintra + KT - 1) / KT) * g.NBc;
    return tiles <= 1024 ? 32 : 64;
}
// Tiles of a group's union at most (every block of the head selected).
int tiles_per_group(const Geo& g) {
    return ((g.Binter + KT - 1) / KT) * g.NBh_max + ((g.Bintra + KT - 1) / KT) * g.NBc;
}
// Split ranges per attention work-group. Past 1024 tiles per group a head's
// K and V outgrow what the work-groups of an XCD reuse from L2 while they
// sweep several heads at once. With M = ceil(H / 8) ranges per work-group the
// grid holds M times as many work-groups as CUs; XCD x runs its ranges
// x * 32 M + j in launch order (j = 0, 1, ...), so the 32 it runs at a time
// cover about one head's tiles. Measured on the attention entry: 18.5 against
// 19.6 ms at 14B 720p over 90 s (M = 5); at 14B 480p no change; at 1.3B 480p
// 3% slower with two ranges, the extra split partials costing more there.
int ranges_per_wg(const Geo& g) {
    if (g.one_range || tiles_per_group(g) <= 1024) return 1;
    const int m = (g.H + 7) / 8;
    return m < kMaxRangesPerWg ? m : kMaxRangesPerWg;
}
// partials: two slots (a range's first and last group) per range
size_t part_o_bytes(const Geo& g) {
    return al256((size_t)kSparseMaxWg * ranges_per_wg(g) * 2 * NW * 64 * 16 * 4 * (g.d / 32));
}
size_t part_ml_bytes(const Geo& g) { return al256((size_t)kSparseMaxWg * ranges_per_wg(g) * 2 * NW * 64 * 8); }

SparseWs carve(const Geo& g, void* ws) {
    const int NG = n_groups(g);
    char* p = (char*)ws;
    SparseWs s;
    s.tbits = (uint32_t*)p;  p += al256((size_t)g.H * g.NQB * plan_words(g) * 4);
    s.grows = (int32_t*)p;   p += al256((size_t)NG * R * 4);
    s.tdesc = (int2*)p;      p += al256((size_t)NG * tiles_per_group(g) * 8);
    s.gcount = (int32_t*)p;  p += al256((size_t)NG * 4);
    s.gtiles = (int32_t*)p;  p += al256((size_t)NG * 4);
    s.gstart = (int32_t*)p;  p += al256((size_t)(NG + 1) * 4);
    s.part_o = (float*)p;    p += part_o_bytes(g);
    s.part_ml = (float2*)p;
    return s;
}

}  // namespace

size_t sparse_bf16_ws_bytes(const Geo& g) {
    const int NG = n_groups(g);
    return al256((size_t)g.H * g.NQB * plan_words(g) * 4) + al256((size_t)NG * R * 4) +
           al256((size_t)NG * tiles_per_group(g) * 8) + 2 * al256((size_t)NG * 4) +
           al256((size_t)(NG + 1) * 4) + part_o_bytes(g) + part_ml_bytes(g);
}

// The plan: it depends on the selection only, so a caller may run it beside
// other work and order the compute part after it.
void launch_sparse_plan_bf16(const Geo& g, const int32_t* n_sel, const int32_t* sel_count,
                             const int32_t* sel_idx, void* ws, hipStream_t st) {
    const int NG = n_groups(g);
    const SparseWs s = carve(g, ws);
    const int W = plan_words(g);
    const bool wide_rows = g.NQB > 128;   // 4 rows per lane (up to 256 per head), else 2
    if (W == 32) {
        hipLaunchKernelGGL(k_plan_bits<32>, dim3(g.H * g.NQB), dim3(64), 0, st, g, n_sel, sel_count, sel_idx,
                           s.tbits);
        if (wide_rows)
            hipLaunchKernelGGL((k_plan_rows<32, 4>), dim3(g.H), dim3(64 * kGroupWaves), 0, st, g, n_sel,
                               (const uint32_t*)s.tbits, s.grows);
        else
            hipLaunchKernelGGL((k_plan_rows<32, 2>), dim3(g.H), dim3(64 * kGroupWaves), 0, st, g, n_sel,
                               (const uint32_t*)s.tbits, s.grows);
    } else {
        hipLaunchKernelGGL(k_plan_bits<64>, dim3(g.H * g.NQB), dim3(64), 0, st, g, n_sel, sel_count, sel_idx,
                           s.tbits);
        if (wide_rows)
            hipLaunchKernelGGL((k_plan_rows<64, 4>), dim3(g.H), dim3(64 * kGroupWaves), 0, st, g, n_sel,
                               (const uint32_t*)s.tbits, s.grows);
        else
            hipLaunchKernelGGL((k_plan_rows<64, 2>), dim3(g.H), dim3(64 * kGroupWaves), 0, st, g, n_sel,
                               (const uint32_t*)s.tbits, s.grows);
    }
    hipLaunchKernelGGL(k_plan_groups, dim3(NG), dim3(kPlanThreads), 0, st, g, n_sel, sel_count, sel_idx,
                       (const int32_t*)s.grows, s.tdesc, tiles_per_group(g), s.gcount, s.gtiles);
    hipLaunchKernelGGL(k_plan_scan, dim3(1), dim3(1024), 0, st, NG, (const int32_t*)s.gtiles, s.gstart);
}

namespace {

template <int D>
void launch_compute_d(const Geo& g, const void* q, const void* k_hist, const void* v_hist, const void* k_intra,
                      const void* v_intra, const int32_t* n_sel, void* ws, const Epi& ep, hipStream_t st) {
    const int NG = n_groups(g);
    const SparseWs s = carve(g, ws);
    PlanArgs pl{s.part_o, s.part_ml, s.grows, NG, sparse_wgs() * ranges_per_wg(g)};
    const int per_xcd = (pl.G + 7) / 8;
    hipLaunchKernelGGL((k_sparse_attn32<D>), dim3(8 * per_xcd), dim3(64 * NW), 0, st, g, (const bf16_t*)q,
                       (const bf16_t*)k_hist, (const bf16_t*)v_hist, (const bf16_t*)k_intra,
                       (const bf16_t*)v_intra, n_sel, (const int2*)s.tdesc, tiles_per_group(g),
                       (const int32_t*)s.gcount, (const int32_t*)s.gtiles, (const int32_t*)s.gstart, pl,
                       per_xcd, ep);
    hipLaunchKernelGGL((k_sparse_combine<D>), dim3(NG, NW), dim3(64 * Wave<D>::DT), 0, st, g, (const bf16_t*)q,
                       (const int32_t*)s.gtiles, (const int32_t*)s.gstart, pl, ep);
}

}  // namespace

// Attention and combine over a plan already in ws (launch_sparse_plan_bf16).
void launch_sparse_compute_bf16(const Geo& g, const void* q, const void* k_hist, const void* v_hist,
                                const void* k_intra, const void* v_intra, const int32_t* n_sel, void* ws,
                                const Epi& ep, hipStream_t st) {
    if (g.d == 128)
        launch_compute_d<128>(g, q, k_hist, v_hist, k_intra, v_intra, n_sel, ws, ep, st);
    else
        launch_compute_d<64>(g, q, k_hist, v_hist, k_intra, v_intra, n_sel, ws, ep, st);
}

void launch_sparse_attn_bf16_mfma32(const Geo& g, const void* q, const void* k_hist,
                                    const void* v_hist, const void* k_intra, const void* v_intra,
                                    const int32_t* n_sel, const int32_t* sel_count,
                                    const int32_t* sel_idx, void* ws, const Epi& ep, hipStream_t st) {
    launch_sparse_plan_bf16(g, n_sel, sel_count, sel_idx, ws, st);
    launch_sparse_compute_bf16(g, q, k_hist, v_hist, k_intra, v_intra, n_sel, ws, ep, st);
}
