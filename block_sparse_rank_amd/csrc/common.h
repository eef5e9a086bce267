// Device helpers shared by the gfx950 kernels of libhsakv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

typedef uint16_t bf16_t;                                       // bfloat16 storage bits
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;   // MFMA bf16 operand
typedef __attribute__((ext_vector_type(4))) float f32x4_t;     // 16x16 MFMA accumulator
typedef __attribute__((ext_vector_type(16))) float f32x16_t;   // 32x32 MFMA accumulator

#define HSAKV_DEV __device__ __forceinline__

// Sizes of one chunk-layer, derived once on the host and passed by value.
struct Geo {
    int H, d, Lq, Tp, P, Kp, Binter, Bintra, Bq, r;
    int HD;        // H * d: elements in one token row
    int NQB;       // query blocks
    int NBc;       // chunk key blocks
    int NBh_max;   // history key blocks when every slot is present
    int NB_max;    // NBh_max + NBc
    long long hist_rows;  // Kp * Tp
    long long L;          // Kp * Tp + Lq: columns of E and F
    int elt;              // bytes per element of the storage type (2 bf16, 4 f32)
    int one_range;        // nonzero: the bf16 sparse attention runs one split range per work-group
};

// Where a page's rows are read from. Without a page table (page_slot null)
// page p is page p of the HBM pool. With one, page_slot[p] >= 0 is the HBM
// pool slot caching the page, and page_slot[p] < 0 means the page is only in
// the pinned host store (host_k / host_v, indexed by page id), which the
// kernels read directly over the bus.
struct Tiers {
    const int32_t* page_slot;
    const void* host_k;
    const void* host_v;
};

// Per-head thresholds passed by value in the kernel arguments, so no host to
// device copy is needed (and the call stays capturable).
constexpr int kMaxHeads = 256;
struct TauArg { float v[kMaxHeads]; };

// Number of history blocks for the slots actually present.
HSAKV_DEV int hist_blocks(const Geo& g, int n_sel) {
    long long Lh = (long long)n_sel * g.Tp;
    return (int)((Lh + g.Binter - 1) / g.Binter);
}

HSAKV_DEV float bf16_to_f32(bf16_t u) { return __uint_as_float((uint32_t)u << 16); }

// float32 -> bf16 bits, round to nearest even (the hardware conversion).
HSAKV_DEV bf16_t f32_to_bf16(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(bf16_t, b);
}

// Element-type traits: loads of 8 consecutive elements as float, and stores.
template <typename T> struct Elt;

template <> struct Elt<float> {
    static constexpr int bytes = 4;
    HSAKV_DEV static void load8(const float* p, float* out) {
        float4 a = *reinterpret_cast<const float4*>(p);
        float4 b = *reinterpret_cast<const float4*>(p + 4);
        out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
        out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
    }
    HSAKV_DEV static float to_f32(float v) { return v; }
    HSAKV_DEV static float from_f32(float v) { return v; }
};

template <> struct Elt<bf16_t> {
    static constexpr int bytes = 2;
    HSAKV_DEV static void load8(const bf16_t* p, float* out) {
        uint4 a = *reinterpret_cast<const uint4*>(p);
        uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            out[2 * i] = __uint_as_float(w[i] << 16);
            out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
        }
    }
    HSAKV_DEV static float to_f32(bf16_t v) { return bf16_to_f32(v); }
    HSAKV_DEV static bf16_t from_f32(float v) { return f32_to_bf16(v); }
};

// 2^x with the hardware v_exp_f32 alone. Results below 2^-126 flush to zero
// instead of going through the denormal fix-up: softmax weights that small
// vanish against the row sum, so the probabilities are unchanged.
HSAKV_DEV float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wave-level helpers (64 lanes).
HSAKV_DEV float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
HSAKV_DEV float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Kahan-compensated float32 accumulator: the error of a long sum stays a few
// ulps of the result whatever its length.
struct Kahan {
    float s = 0.f, c = 0.f;
    HSAKV_DEV void add(float x) {
        float y = x - c;
        float t = s + y;
        c = (t - s) - y;
        s = t;
    }
};
