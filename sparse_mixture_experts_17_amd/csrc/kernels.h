// Host-side launchers of the gfx950 MoE kernels (internal to the library).
// Every launcher enqueues on `stream` and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Tokens per router block; also the chunk size of the dispatch counting sort.
constexpr int kRouteTokens = 16;

inline int route_blocks(int T) { return (T + kRouteTokens - 1) / kRouteTokens; }

// Router: fp32 logits via MFMA, softmax or sigmoid scores, top-k (optionally limited to the
// best topk_group of n_group expert groups; lowest index on ties), gates, per-block partial
// sums of p (or s) and per-block expert histograms.
hipError_t launch_router(int dtype, const void* x, const void* w_r, const float* b_r, int T, int d,
                         int E, int k, int renorm, int scoring, int n_group, int topk_group, int32_t* idx,
                         float* gate, float* p_part, int32_t* hist, hipStream_t stream);

// Per-chunk expert histograms of an index array (dispatch without the router).
hipError_t launch_hist(const int32_t* idx, int T, int k, int E, int32_t* hist, hipStream_t stream);

// One block: counts, capacity, offsets, per-chunk bases, grouped-GEMM tile starts,
// and (when p_part != NULL) f, P, aux.
hipError_t launch_scan(const int32_t* hist, const float* p_part, int nb, int T, int k, int E, int cap,
                       int32_t* counts, int32_t* kept, int32_t* offsets, int32_t* chunk_base,
                       float* f, float* P, float* aux, int bm1, int32_t* tstart1, int bm2,
                       int32_t* tstart2, hipStream_t stream);

// Grouped-GEMM tile starts from row offsets alone.
hipError_t launch_tile_sched(const int32_t* offsets, int E, int bm1, int32_t* tstart1, int bm2,
                             int32_t* tstart2, hipStream_t stream);

// Stable ranks within each expert, capacity, row_of / row_token, and the gather
// x_perm[row] = x[token] (skipped when x_perm is NULL).
hipError_t launch_rank_gather(int dtype, const void* x, const int32_t* idx, int T, int d, int k, int E,
                              int cap, const int32_t* chunk_base, const int32_t* offsets,
                              int32_t* row_token, int32_t* row_of, void* x_perm, hipStream_t stream);

// y[t] = shared[t] (or 0) + sum_j gate[t,j] * o[row_of[t,j]] over kept slots, where a row of o
// is the sum of nsplit partials o + p * split_stride (floats; a multiple of 4), p = 0 .. nsplit-1.
hipError_t launch_combine(const float* o, const int32_t* row_of, const float* gate, const float* shared,
                          float* y, int T, int d, int k, int nsplit, size_t split_stride, hipStream_t stream);

// Grouped GEMM tile configurations (one kernel template; see grouped_gemm.hip).
enum GemmKind { kGemmLarge = 0, kGemmStream = 1, kGemmDecode = 2 };
// Tile rows of the kernel that `kind` selects for the gate/up (gated) or down product.
int gemm_block_m(GemmKind kind, int dtype, bool gated, int wfmt);

// Gate/up product with the SiLU(a) * b epilogue:  h[r, n] = SiLU(A_r W_g[e]^T) * (A_r W_u[e]^T).
// A_r is row r of A, or row a_rows[r] of A when a_rows != NULL (the dispatch gather done by
// the loads; the byte offset a_rows[r] * K * elem must stay below 2^32).
// offsets == NULL means one group of `dense_rows` rows.  tstart = per-group tile starts.
// wfmt 1: Wg, Wu hold E4M3 codes and Sg, Su [G, N] their row scales (bf16 activations).
hipError_t launch_gemm_gateup(GemmKind kind, int dtype, int wfmt, const void* A, const int32_t* a_rows,
                              const void* Wg, const void* Wu, const float* Sg, const float* Su,
                              const int32_t* offsets, const int32_t* tstart, int G, int dense_rows, int max_tiles_m,
                              int N, int K, void* H, hipStream_t stream);

// Down projection:  o[r, n] = H_e W_d[e]^T, fp32 out (times Sd[e, n] for FP8 weights).
hipError_t launch_gemm_down(GemmKind kind, int dtype, int wfmt, const void* H, const void* Wd, const float* Sd,
                            const int32_t* offsets, const int32_t* tstart, int G, int dense_rows, int max_tiles_m,
                            int N, int K, float* O, int ksplit, size_t split_stride, hipStream_t stream);

}  // namespace moe
