// Internal launchers of libhsakv (not exported). Each enqueues on `st` and
// returns immediately; the caller checks hipGetLastError.
#pragma once

#include "common.h"

// Compute units of the current device, looked up once per device (a
// lock-free cache: concurrent first calls store the same value atomically).
int device_cu_count();

// Epilogue of the attention kernels.
//  o_main : f32 [Lq][H][d] receives O (NULL: not written)
//  out    : dtype [Lq][H][d] receives the gated fusion g*O + (1-g)*o_lin (NULL: no fusion)
//  o_lin  : f32 [Lq][H][d] the low-rank branch, read when `out` is set
//  gate   : f32 [Lq][H] receives g (NULL: not written); only with `out`
//  w_g, b_g : gate parameters, read when `out` is set
struct Epi {
    float* o_main;
    void* out;
    const float* o_lin;
    float* gate;
    const float* w_g;
    const float* b_g;
};

// Page means: partial holds page_means_ws_bytes(g, pages) bytes of scratch.
size_t page_means_ws_bytes(const Geo&, int pages);
template <typename T>
void launch_page_summary(const Geo&, const void* pool_k, float* page_kmean, float* partial, hipStream_t);
// Page commit: chunk rows -> pool rows [fill, fill + n); page means and tags of the pages completed.
template <typename T>
void launch_page_commit(const Geo&, void* pool_k, void* pool_v, float* page_kmean, int32_t* page_prompt,
                        const void* k_chunk, const void* v_chunk, int n, long long fill, int cur_prompt,
                        float* partial, hipStream_t);
constexpr int kMaxKp = 64;   // active-cache slots at most

// Retrieval (two kernels; the first for the score policies only): the
// workspace holds retrieve_ws_bytes bytes of float64 partial sums.
size_t retrieve_smem_bytes(const Geo&);
size_t retrieve_ws_bytes(const Geo&);
template <typename T>
void launch_retrieve(const Geo&, const void* q, const float* page_kmean, const int32_t* page_prompt, int cur_prompt,
                     int policy, unsigned long long seed, void* ws, int32_t* page_idx, int32_t* n_sel, hipStream_t);
void launch_gather(const Geo&, int elt_bytes, const void* pool_k, const void* pool_v, const int32_t* page_idx,
                   const int32_t* n_sel, void* k_hist, void* v_hist, const Tiers& tiers, hipStream_t);
// The gather with the history blocks of the pooled keys kb written on the way.
template <typename T>
void launch_gather_pool(const Geo&, const void* pool_k, const void* pool_v, const int32_t* page_idx,
                        const int32_t* n_sel, void* k_hist, void* v_hist, float* kb, const Tiers& tiers,
                        hipStream_t);
// Page-table updates page_slot[pages[i]] = values[i], i < n <= 256.
void launch_tier_table(int32_t* page_slot, int n, const int32_t* pages, const int32_t* values, hipStream_t);

// hist_pooled: the history blocks of kb are already written (launch_gather_pool)
template <typename T>
void launch_pool(const Geo&, const void* q, const void* k_hist, const void* k_intra, const int32_t* n_sel,
                 float* qb, float* kb, bool hist_pooled, hipStream_t);
void launch_select(const Geo&, const float* qb, const float* kb, float* zl, const int32_t* n_sel, const TauArg& tau,
                   int32_t* sel_count, int32_t* sel_idx, uint8_t* sel_mask, float* block_mass, hipStream_t);

template <typename T>
void launch_sparse_attn(const Geo&, const void* q, const void* k_hist, const void* v_hist, const void* k_intra,
                        const void* v_intra, const int32_t* n_sel, const int32_t* sel_count,
                        const int32_t* sel_idx, void* ws, const Epi& ep, hipStream_t);
// bf16 path: ws holds sparse_bf16_ws_bytes(g) bytes (plan and split partials)
size_t sparse_bf16_ws_bytes(const Geo&);
void launch_sparse_attn_bf16_mfma32(const Geo&, const void* q, const void* k_hist, const void* v_hist,
                                    const void* k_intra, const void* v_intra, const int32_t* n_sel,
                                    const int32_t* sel_count, const int32_t* sel_idx, void* ws,
                                    const Epi& ep, hipStream_t);
// the same in two parts: the plan (selection only) and, ordered after it,
// the attention and combine
void launch_sparse_plan_bf16(const Geo&, const int32_t* n_sel, const int32_t* sel_count, const int32_t* sel_idx,
                             void* ws, hipStream_t);
void launch_sparse_compute_bf16(const Geo&, const void* q, const void* k_hist, const void* v_hist,
                                const void* k_intra, const void* v_intra, const int32_t* n_sel, void* ws,
                                const Epi& ep, hipStream_t);
template <typename T>
void launch_lowrank_attn(const Geo&, const void* q, const void* k_hi, const void* v_hi, const void* k_lo,
                         const void* v_lo, const Epi& ep, hipStream_t);
// bf16 K', V' (hi + lo pairs), d = 64 or 128: the 32x32x16 MFMA kernel; writes O (float32) to out.
void launch_lowrank_attn_bf16_mfma32(const Geo&, const void* q, const void* k_hi, const void* v_hi,
                                     const void* k_lo, const void* v_lo, float* out, hipStream_t);

int lowrank_splits(const Geo&);
bool proj32_eligible(const Geo&);
int proj32_splits(const Geo&);
void launch_lowrank_proj32(const Geo&, const void* E, const void* F, const void* k_hist, const void* v_hist,
                           const void* k_intra, const void* v_intra, const int32_t* n_sel, float* part,
                           hipStream_t);
template <typename T>
void launch_lowrank_proj(const Geo&, const void* E, const void* F, const void* k_hist, const void* v_hist,
                         const void* k_intra, const void* v_intra, const int32_t* n_sel, float* part,
                         hipStream_t);
template <typename T>
void launch_lowrank_reduce(const Geo&, const float* part, float* k_low, float* v_low, void* k_hi, void* v_hi,
                           void* k_lo, void* v_lo, hipStream_t);
template <typename T>
void launch_fuse(const Geo&, const void* q, const float* w_g, const float* b_g, const float* o_s,
                 const float* o_l, void* out, float* gate, hipStream_t);

// Backward of the learned parameters (bf16): workspace of backward_ws_bytes(g)
// bytes. With side != st part of the work runs on `side`, ordered by the two
// events; returns the first failing event call's error (hipSuccess otherwise).
size_t backward_ws_bytes(const Geo&);
hipError_t launch_backward_params(const Geo&, const void* q, const void* k_hist, const void* v_hist,
                                  const void* k_intra, const void* v_intra, const int32_t* n_sel, const float* w_g,
                                  const float* b_g, const float* k_low, const float* v_low, const float* o_s,
                                  const float* o_l, const void* d_out, float* d_wg, float* d_bg, float* d_E,
                                  float* d_F, void* ws, hipStream_t st, hipStream_t side, hipEvent_t ev_fork,
                                  hipEvent_t ev_join);
