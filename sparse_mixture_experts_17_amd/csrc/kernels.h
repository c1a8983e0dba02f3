// Host-side launchers of the gfx950 MoE kernels (internal to the library).
// Every launcher enqueues on `stream` and returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Tokens per router block; also the chunk size of the dispatch counting sort.
constexpr int kRouteTokens = 16;
// Work counters of a dynamically scheduled grouped GEMM: one per XCD.
constexpr int kTileCtrInts = 8;

inline int route_blocks(int T) { return (T + kRouteTokens - 1) / kRouteTokens; }

// Router: fp32 logits via MFMA, softmax or sigmoid scores, top-k (optionally limited to the
// best topk_group of n_group expert groups; lowest index on ties), gates, per-block partial
// sums of p (or s) and per-block expert histograms.  When router_logits_by_gemm(E), the logits
// come from a dense GEMM into `logits` (router_gemm_ksplit(d) partial [T, E] fp32 arrays) first;
// otherwise `logits` is unused.
hipError_t launch_router(int dtype, const void* x, const void* w_r, const float* b_r, int T, int d,
                         int E, int k, int renorm, int scoring, int n_group, int topk_group, int32_t* idx,
                         float* gate, float* p_part, int32_t* hist, float* logits, hipStream_t stream);

// 64 or more experts (a whole number of 64-wide tiles): a 16-token router block would stream all
// of W_r, so a tiled GEMM computes the logits instead, its contraction cut into router_gemm_ksplit
// chunks for parallelism.  The forward and the backward both read these logits, summing the
// chunks in order, so both see the same bits.
inline bool router_logits_by_gemm(int E) { return E >= 64 && E % 64 == 0; }
inline int router_gemm_ksplit(int d) {
  const int steps = d / 64;                               // 64-element K steps
  return steps % 4 == 0 ? 4 : (steps % 2 == 0 ? 2 : 1);
}
inline size_t router_logits_bytes(int T, int d, int E) {
  return router_logits_by_gemm(E) ? (size_t)router_gemm_ksplit(d) * (size_t)T * (size_t)E * sizeof(float) : 0;
}

// Dense partial logits: chunk c of router_gemm_ksplit(d) writes logits + c T E = x [T, d] W_r^T over
// its K range, in fp32 (tiles of 64 tokens x 64 experts).
hipError_t launch_gemm_router(int dtype, const void* x, const void* w_r, int T, int d, int E, float* logits,
                              hipStream_t stream);

// Routing and dispatch of a batch that is one router block (decode: at most 16 tokens, at most
// 16 experts) in one launch: the router block also runs the scan's expert pass and the ranks.
// The outputs equal launch_router + launch_scan + launch_rank_gather (without x_perm) bit for bit.
struct SmallDispatch {
  int cap = -1;
  int32_t* counts = nullptr;       // may be NULL
  int32_t* kept = nullptr;
  int32_t* offsets = nullptr;
  float* f = nullptr;
  float* P = nullptr;
  float* aux = nullptr;
  int bm1 = 1, bm2 = 1;
  int32_t* tstart1 = nullptr;
  int32_t* tstart2 = nullptr;
  int32_t* row_token = nullptr;
  int32_t* row_of = nullptr;
};
inline bool route_small_ok(int T, int E) { return T >= 1 && T <= kRouteTokens && E <= 16; }
hipError_t launch_route_small(int dtype, const void* x, const void* w_r, const float* b_r, int T, int d, int E, int k,
                              int renorm, int scoring, int n_group, int topk_group, int32_t* idx, float* gate,
                              const SmallDispatch& sd, hipStream_t stream);

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
// tile_ctr: kTileCtrInts ints of workspace for dynamic tile scheduling (zeroed by this call, on
// `stream`), or NULL; only the large bf16 tiles use it.
hipError_t launch_gemm_down(GemmKind kind, int dtype, int wfmt, const void* H, const void* Wd, const float* Sd,
                            const int32_t* offsets, const int32_t* tstart, int G, int dense_rows, int max_tiles_m,
                            int N, int K, float* O, int ksplit, size_t split_stride, hipStream_t stream,
                            int32_t* tile_ctr = nullptr);

// ---- FP8 products with MXFP8 activations (grouped_gemm_mx.hip)
// OCP MXFP8 of the rows of x [rows, K] (bf16): codes [rows, K] E4M3, scales [rows, K/32] E8M0,
// block scale 2^(floor(log2 max|v|) - 8), elements rounded to nearest even, saturated at 448.
hipError_t launch_mxfp8_quantize(const void* x, int rows, int K, uint8_t* codes, uint8_t* scales,
                                 hipStream_t stream);
// Rows per tile of the MXFP8 products for `kind`.
int gemm_block_m_mx(GemmKind kind);
// Gate/up product on the scaled MFMA: A = MXFP8 rows (codes [*, K] and scales [*, K/32], row
// a_rows[r] when a_rows != NULL), weights wfmt 1 (E4M3 with row scales Sg, Su [G, N]) or 2
// (MXFP4 with E8M0 [G, K/32, N]).  h = SiLU(a) * b is written as MXFP8: Hq [rows, N] codes,
// Hs [rows, N/32] scales.
hipError_t launch_gemm_gateup_mx(GemmKind kind, int wfmt, const uint8_t* A, const uint8_t* As, const int32_t* a_rows,
                                 const void* Wg, const void* Wu, const void* Sg, const void* Su,
                                 const int32_t* offsets, const int32_t* tstart, int G, int dense_rows,
                                 int max_tiles_m, int N, int K, uint8_t* Hq, uint8_t* Hs, hipStream_t stream);
// Down product on the scaled MFMA: o [rows, N] fp32 = Hq W_d^T (times Sd [G, N] for wfmt 1).
hipError_t launch_gemm_down_mx(GemmKind kind, int wfmt, const uint8_t* Hq, const uint8_t* Hs, const void* Wd,
                               const void* Sd, const int32_t* offsets, const int32_t* tstart, int G, int dense_rows,
                               int max_tiles_m, int N, int K, float* O, hipStream_t stream);

// ---- backward products (grouped_gemm_bwd.hip)
// Gate/up product again with the gate/up tiles of `kind`: a_out, b_out [rows, N] fp32 (the
// pre-activations) and hT [N, ldt] = h^T in dtype, row r of group g at column
// poff[g] + r - offsets[g] (poff == NULL: column r).
hipError_t launch_gemm_save_ab(GemmKind kind, int dtype, const void* A, const int32_t* a_rows, const void* Wg,
                               const void* Wu, const int32_t* offsets, const int32_t* tstart, int G, int dense_rows,
                               int max_tiles_m, int N, int K, float* a_out, float* b_out, void* hT,
                               const int32_t* poff, int ldt, hipStream_t stream);
// u = A_r WdT[e]^T (N = d_e, K = d; WdT = W_d transposed, [G, d_e, d]) with the SwiGLU
// backward in the epilogue: dAB [rows, 2N] and dABT [2N, ldt] (dA then dB, dtype), and
// part [rows, N / gemm_dgrad_part_cols] the partial dots sum_n h u (part may be NULL).
// g_row [rows] scales u (NULL: 1).  Tile heights are the gate/up ones of `kind`.
hipError_t launch_gemm_dgrad(GemmKind kind, int dtype, const void* A, const int32_t* a_rows, const void* WdT,
                             const int32_t* offsets, const int32_t* tstart, int G, int dense_rows, int max_tiles_m,
                             int N, int K, const float* a_in, const float* b_in, const float* g_row, void* dAB,
                             void* dABT, const int32_t* poff, int ldt, float* part, hipStream_t stream);
int gemm_dgrad_part_cols(GemmKind kind, int N);
// C[g] = A[:, K_g] B[:, K_g]^T for groups g < G, K_g = [koffsets[g], koffsets[g+1]) (multiples
// of 64 in bf16, 32 in fp32); A [M, ld], B [N, ld] in dtype; C [G, M, N] fp32.
hipError_t launch_gemm_kgrouped(int dtype, const void* A, const void* B, const int32_t* koffsets, int G, int M,
                                int N, int ld, float* C, hipStream_t stream);

// ---- backward, non-GEMM kernels (backward.hip)
// poff [E+1]: padded column of each expert's first row (whole 64-column steps); g_row [R]:
// gate of each kept row; koff_dense {0, dense_pad} when not NULL.
hipError_t launch_bwd_layout(const int32_t* offsets, int E, const int32_t* row_of, const float* gate, int R,
                             int32_t* poff, float* g_row, int dense_pad, int32_t* koff_dense, hipStream_t stream);
// dst[b][c][coff + r] = src[b][r][c]  (src [B, Rn, C], dst [B, C, ldd]; Rn, C multiples of 64)
hipError_t launch_transpose(int dtype, const void* src, int B, int Rn, int C, void* dst, int ldd, int coff,
                            size_t dst_batch, hipStream_t stream);
// dst [C, ldt] (dst_dtype): column p of expert e = source row rows[r] (or r) times scale[r]
// (or 1) for r = offsets[e] + p - poff[e] < offsets[e+1], else 0; offsets == NULL: one group
// of n_dense rows.  Columns [0, p_bound) are visited (p_bound <= ldt, multiples of 64).
hipError_t launch_gather_t(int src_dtype, int dst_dtype, const void* src, int C, const int32_t* rows,
                           const float* scale, const int32_t* offsets, const int32_t* poff, int E, int n_dense,
                           int p_bound, void* dst, int ldt, hipStream_t stream);
// zero columns [poff[e] + kept_e, poff[e+1]) (dense: [n_dense, pad_dense)) of dst [nrows, ldt]
hipError_t launch_zero_gaps(int dtype, void* dst, int nrows, int ldt, const int32_t* offsets, const int32_t* poff,
                            int E, int n_dense, int pad_dense, hipStream_t stream);
hipError_t launch_to_bf16(const float* src, size_t n, void* dst, hipStream_t stream);
// dr [T, E] = dL/dlogits; dgate [T, k] (may be NULL) = sum of each kept row's partial dots.
// `logits`: scratch of router_logits_bytes(T, d, E) bytes (the logits GEMM's output), or unused.
hipError_t launch_router_bwd(int dtype, const void* x, const void* w_r, const float* b_r, int T, int d, int E, int k,
                             int renorm, int scoring, const int32_t* idx, const float* gate, const int32_t* row_of,
                             const int32_t* counts, const float* part, int npart, float d_aux, float* dr,
                             float* dgate, float* logits, hipStream_t stream);
// dw_r [E, d] = dr^T x; db_r [E] = sum_t dr (zeros when zero_bias), skipped when NULL;
// part: scratch of dwr_workspace_bytes(T, d, E)
size_t dwr_workspace_bytes(int T, int d, int E);
hipError_t launch_dwr(int dtype, const float* dr, const void* x, int T, int d, int E, float* dw_r, float* db_r,
                      int zero_bias, float* part, hipStream_t stream);
// dx [T, d] = dr W_r + sum_j dX[row_of[t, j]] + dXs[t] (dXs may be NULL)
hipError_t launch_dx(int dtype, const float* dr, const void* w_r, int T, int d, int E, int k, const float* dX,
                     const int32_t* row_of, const float* dXs, float* dx, hipStream_t stream);

}  // namespace moe
