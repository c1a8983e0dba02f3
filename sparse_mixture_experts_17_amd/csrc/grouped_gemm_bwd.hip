// Launch configurations of the grouped GEMMs of the backward pass (kernel template in
// grouped_gemm_kernel.h, epilogues in gemm_common.h).
//
// The backward of an expert o = (SiLU(X W_g^T) * (X W_u^T)) W_d^T (Zero to Frontier §13.1
// "Why MoE", section "The MoE layer") needs, besides plain products:
//   * the gate/up product again, keeping a and b (recomputing instead of storing in the
//     forward pass, the trade of the FlashAttention backward in AI Engineering Illustrated's
//     FlashAttention issue, "The trick that makes tiling legal");
//   * u = dy W_d with the SwiGLU derivative applied in the epilogue;
//   * K-grouped products for the weight gradients, whose contraction runs over each
//     expert's rows.
#include "grouped_gemm_kernel.h"

namespace moe {

template <typename T, int BM, int BN, int WM, int WN, bool GATED, int STAGES, int BSTAGES, int EPI>
static hipError_t launch_bwd(const GemmArgs& a, int max_tiles_m, hipStream_t stream) {
  return launch_kernel<GemmTile<T, BM, BN, WM, WN, GATED, STAGES, BSTAGES, 0, EPI>,
                       grouped_gemm_kernel<T, BM, BN, WM, WN, GATED, STAGES, BSTAGES, 0, EPI, 1>>(a, max_tiles_m,
                                                                                                   stream);
}

// The gate/up recompute uses the forward's gate/up tiles (same rows per tile, so the same
// tile starts, and the same accumulation order: a and b equal the forward's bit for bit).
template <typename T>
static hipError_t save_ab_kind(GemmKind kind, const GemmArgs& a, int max_tiles_m, hipStream_t s) {
  switch (kind) {
    case kGemmLarge: return launch_bwd<T, 256, 128, 4, 2, true, 2, 3, 1>(a, max_tiles_m, s);
    case kGemmStream: return launch_bwd<T, 160, 128, 2, 4, true, 3, 3, 1>(a, max_tiles_m, s);
    default: return launch_bwd<T, 16, 64, 1, 4, true, 4, 4, 1>(a, max_tiles_m, s);
  }
}

// The down-product backward has the gate/up tile heights, so it shares their tile starts.
template <typename T>
static hipError_t dgrad_kind(GemmKind kind, const GemmArgs& a, int max_tiles_m, hipStream_t s) {
  switch (kind) {
    case kGemmLarge:
      if (a.N % 256 == 0) return launch_bwd<T, 256, 256, 4, 2, false, 2, 3, 2>(a, max_tiles_m, s);
      return launch_bwd<T, 256, 128, 4, 2, false, 2, 3, 2>(a, max_tiles_m, s);
    case kGemmStream: return launch_bwd<T, 160, 128, 2, 4, false, 3, 3, 2>(a, max_tiles_m, s);
    default: return launch_bwd<T, 16, 32, 1, 2, false, 4, 4, 2>(a, max_tiles_m, s);
  }
}

// columns per partial dot of the down-product backward (the wave tile width BN / WN)
int gemm_dgrad_part_cols(GemmKind kind, int N) {
  switch (kind) {
    case kGemmLarge: return N % 256 == 0 ? 128 : 64;
    case kGemmStream: return 32;
    default: return 16;
  }
}

hipError_t launch_gemm_save_ab(GemmKind kind, int dtype, const void* A, const int32_t* a_rows, const void* Wg,
                               const void* Wu, const int32_t* offsets, const int32_t* tstart, int G, int dense_rows,
                               int max_tiles_m, int N, int K, float* a_out, float* b_out, void* hT,
                               const int32_t* poff, int ldt, hipStream_t stream) {
  GemmArgs a{A, a_rows, Wg, Wu, nullptr, nullptr, offsets, tstart, G, dense_rows, N, K, nullptr};
  a.ep_a = a_out;
  a.ep_b = b_out;
  a.ep_t = hT;
  a.ep_poff = poff;
  a.ep_ldt = ldt;
  if (dtype == 1) return save_ab_kind<uint16_t>(kind, a, max_tiles_m, stream);
  return save_ab_kind<float>(kind, a, max_tiles_m, stream);
}

hipError_t launch_gemm_dgrad(GemmKind kind, int dtype, const void* A, const int32_t* a_rows, const void* WdT,
                             const int32_t* offsets, const int32_t* tstart, int G, int dense_rows, int max_tiles_m,
                             int N, int K, const float* a_in, const float* b_in, const float* g_row, void* dAB,
                             void* dABT, const int32_t* poff, int ldt, float* part, hipStream_t stream) {
  GemmArgs a{A, a_rows, WdT, nullptr, nullptr, nullptr, offsets, tstart, G, dense_rows, N, K, dAB};
  a.ep_a = const_cast<float*>(a_in);
  a.ep_b = const_cast<float*>(b_in);
  a.ep_g = g_row;
  a.ep_t = dABT;
  a.ep_part = part;
  a.ep_poff = poff;
  a.ep_ldt = ldt;
  a.ep_npart = N / gemm_dgrad_part_cols(kind, N);
  if (dtype == 1) return dgrad_kind<uint16_t>(kind, a, max_tiles_m, stream);
  return dgrad_kind<float>(kind, a, max_tiles_m, stream);
}

hipError_t launch_gemm_kgrouped(int dtype, const void* A, const void* B, const int32_t* koffsets, int G, int M,
                                int N, int ld, float* C, hipStream_t stream) {
  if (M < 1 || N % 128 != 0 || ld % 64 != 0) return hipErrorInvalidValue;
  GemmArgs a{A, nullptr, B, nullptr, nullptr, nullptr, nullptr, nullptr, G, M, N, ld, C};
  a.koffsets = koffsets;
  const int mt = (M + 255) / 256;
  if (dtype == 1) {
    if (N % 256 == 0) return launch_bwd<uint16_t, 256, 256, 4, 2, false, 2, 3, 3>(a, G * mt, stream);
    return launch_bwd<uint16_t, 256, 128, 4, 2, false, 2, 3, 3>(a, G * mt, stream);
  }
  if (N % 256 == 0) return launch_bwd<float, 256, 256, 4, 2, false, 2, 3, 3>(a, G * mt, stream);
  return launch_bwd<float, 256, 128, 4, 2, false, 2, 3, 3>(a, G * mt, stream);
}

}  // namespace moe
