// Launch configurations of the forward grouped GEMMs (kernel template in grouped_gemm_kernel.h).
#include "grouped_gemm_kernel.h"

namespace moe {

// ------------------------------------------------------------------------------ launch

template <typename T, int BM, int BN, int WM, int WN, bool GATED, int STAGES, int BSTAGES = STAGES,
          int WF = 0, int KSUB = 1>
static hipError_t launch_cfg(const GemmArgs& a, int max_tiles_m, hipStream_t stream) {
  return launch_kernel<GemmTile<T, BM, BN, WM, WN, GATED, STAGES, BSTAGES, WF, 0, KSUB>,
                       grouped_gemm_kernel<T, BM, BN, WM, WN, GATED, STAGES, BSTAGES, WF, 0, KSUB>>(a, max_tiles_m,
                                                                                                  stream);
}

// Zeroes the per-XCD work counters of a dynamically scheduled product (one block, before it).
__global__ void zero_tile_ctr_kernel(int32_t* ctr) {
  static_assert(kTileCtrInts >= kNumXcd, "one counter per XCD");
  if (threadIdx.x < kNumXcd) ctr[threadIdx.x] = 0;
}

int gemm_block_m(GemmKind kind, int dtype, bool gated, int wfmt) {
  if (kind == kGemmLarge) return dtype == 1 && !gated && wfmt == 0 ? kLargeBf16BlockM : 256;
  return kind == kGemmStream ? 160 : 16;
}

// Decode tiles with quantised weights take KSUB 64-element sub-steps per LDS stage, so that a
// weight row gives 128 contiguous bytes per stage (FP8: 2 x 64 bytes, MXFP4: 4 x 32 bytes).
template <int WF>
constexpr int kDecodeKsub = WF == 1 ? 2 : (WF == 2 ? 4 : 1);
// LDS ring depth of the decode tiles.  With 4-bit weights more blocks per CU beat a deeper
// ring (measured: 2 stages, 3 blocks per CU, best).
template <int WF>
constexpr int kDecodeStages = WF == 0 ? 4 : (WF == 2 ? 2 : 3);
// weight rows per decode tile (gate/up: per matrix).  The 4-bit down product takes 64: with its
// two K chunks that gives as many blocks as fit, each streaming twice the bytes per stage
// (measured at the Mixtral decode shape: 32 rows 75 us, 64 rows 54 us, 128 rows 68 us).
template <int WF, bool GATED>
constexpr int kDecodeBN = GATED ? 64 : (WF == 2 ? 64 : 32);

template <typename T, bool GATED, int WF>
static hipError_t dispatch_kind(GemmKind kind, GemmArgs a, int max_tiles_m, hipStream_t s) {
  int32_t* const ctr = a.tile_ctr;
  a.tile_ctr = nullptr;   // dynamic scheduling only where it was measured to pay (below)
  switch (kind) {
    case kGemmLarge:
      // 8 waves; activations in a 2-deep ring, weights (the HBM stream) in a 3-deep one
      if constexpr (GATED) {
        return launch_cfg<T, 256, 128, 4, 2, GATED, 2, 3, WF>(a, max_tiles_m, s);   // 64x(64+64) per wave
      } else if constexpr (sizeof(T) == 2 && WF == 0) {
        // bf16 down: 192-row tiles (48 x 128 per wave).  At the Mixtral prefill shape they make
        // 2.94 rounds of the grid where 256-row tiles make 2.25 (measured 0.90-0.94 against
        // 0.99-1.02 ms).  Scheduled dynamically when given counters: each expert's last m-tile
        // is partly empty and cheap, and static round-robin leaves some blocks a third full
        // tile (Mixtral prefill down 2-3 % faster, bit-identical)
        if (ctr) {
          hipLaunchKernelGGL(zero_tile_ctr_kernel, dim3(1), dim3(64), 0, s, ctr);
          a.tile_ctr = ctr;
        }
        if (a.N % 256 == 0) return launch_cfg<T, kLargeBf16BlockM, 256, 4, 2, GATED, 2, 3, WF>(a, max_tiles_m, s);
        return launch_cfg<T, kLargeBf16BlockM, 128, 4, 2, GATED, 2, 3, WF>(a, max_tiles_m, s);
      } else {
        if (a.N % 256 == 0) return launch_cfg<T, 256, 256, 4, 2, GATED, 2, 3, WF>(a, max_tiles_m, s);
        return launch_cfg<T, 256, 128, 4, 2, GATED, 2, 3, WF>(a, max_tiles_m, s);
      }
    case kGemmStream:
      // weight streaming with ~100-250 rows per expert: wide weight tiles, 3-deep ring so
      // two K steps of weights are in flight per CU
      if constexpr (GATED) {
        return launch_cfg<T, 160, 128, 2, 4, GATED, 3, 3, WF>(a, max_tiles_m, s);   // 80x(32+32) per wave
      } else {
        if (a.N % 256 == 0) return launch_cfg<T, 160, 256, 2, 4, GATED, 3, 3, WF>(a, max_tiles_m, s);
        return launch_cfg<T, 160, 128, 2, 4, GATED, 3, 3, WF>(a, max_tiles_m, s);
      }
    default:
      // decode: a few rows per expert, 4-deep ring; the down product has half the weight
      // rows of gate/up, so narrower tiles give it as many blocks streaming in parallel
      // (sub-steps need K, per K chunk, to be a whole number of stages; else one per stage)
      if (a.K % (64 * kDecodeKsub<WF> * a.ksplit) != 0) {
        if constexpr (GATED)
          return launch_cfg<T, 16, kDecodeBN<WF, true>, 1, 4, GATED, 4, 4, WF, 1>(a, max_tiles_m, s);
        else
          return launch_cfg<T, 16, kDecodeBN<WF, false>, 1, 2, GATED, 4, 4, WF, 1>(a, max_tiles_m, s);
      }
      if constexpr (GATED)
        return launch_cfg<T, 16, kDecodeBN<WF, true>, 1, 4, GATED, kDecodeStages<WF>, kDecodeStages<WF>, WF,
                          kDecodeKsub<WF>>(a, max_tiles_m, s);
      else
        return launch_cfg<T, 16, kDecodeBN<WF, false>, 1, 2, GATED, kDecodeStages<WF>, kDecodeStages<WF>, WF,
                          kDecodeKsub<WF>>(a, max_tiles_m, s);
  }
}

hipError_t launch_gemm_gateup(GemmKind kind, int dtype, int wfmt, const void* A, const int32_t* a_rows,
                              const void* Wg, const void* Wu, const float* Sg, const float* Su,
                              const int32_t* offsets, const int32_t* tstart, int G, int dense_rows, int max_tiles_m,
                              int N, int K, void* H, hipStream_t stream) {
  GemmArgs a{A, a_rows, Wg, Wu, Sg, Su, offsets, tstart, G, dense_rows, N, K, H};
  if (dtype == 1) {
    if (wfmt == 1) return dispatch_kind<uint16_t, true, 1>(kind, a, max_tiles_m, stream);
    if (wfmt == 2) return dispatch_kind<uint16_t, true, 2>(kind, a, max_tiles_m, stream);
    return dispatch_kind<uint16_t, true, 0>(kind, a, max_tiles_m, stream);
  }
  return dispatch_kind<float, true, 0>(kind, a, max_tiles_m, stream);
}

hipError_t launch_gemm_down(GemmKind kind, int dtype, int wfmt, const void* H, const void* Wd, const float* Sd,
                            const int32_t* offsets, const int32_t* tstart, int G, int dense_rows, int max_tiles_m,
                            int N, int K, float* O, int ksplit, size_t split_stride, hipStream_t stream,
                            int32_t* tile_ctr) {
  GemmArgs a{H, nullptr, Wd, nullptr, Sd, nullptr, offsets, tstart, G, dense_rows, N, K, O, ksplit, split_stride};
  a.tile_ctr = tile_ctr;
  // K chunks: decode tiles only, each chunk a whole number of K steps (64 elements; 32 in fp32)
  if (ksplit < 1 || (ksplit > 1 && (kind != kGemmDecode || K % (ksplit * (dtype == 1 ? 64 : 32)) != 0)))
    return hipErrorInvalidValue;
  if (dtype == 1) {
    if (wfmt == 1) return dispatch_kind<uint16_t, false, 1>(kind, a, max_tiles_m, stream);
    if (wfmt == 2) return dispatch_kind<uint16_t, false, 2>(kind, a, max_tiles_m, stream);
    return dispatch_kind<uint16_t, false, 0>(kind, a, max_tiles_m, stream);
  }
  return dispatch_kind<float, false, 0>(kind, a, max_tiles_m, stream);
}

hipError_t launch_gemm_router(int dtype, const void* x, const void* w_r, int T, int d, int E, float* logits,
                              hipStream_t stream) {
  if (!router_logits_by_gemm(E) || d % 64 != 0) return hipErrorInvalidValue;
  GemmArgs a{x, nullptr, w_r, nullptr, nullptr, nullptr, nullptr, nullptr, 1, T, E, d, logits};
  a.dense_n_minor = 1;   // an XCD's tiles share their token rows; W_r (E x d) stays in its L2
  a.ksplit = router_gemm_ksplit(d);
  a.split_stride = (size_t)T * E;
  // 64 x 64 tiles, times the K chunks: 1,024 work items at 4096 tokens x 256 experts
  const int tiles_m = (T + 63) / 64;
  if (dtype == 1) return launch_cfg<uint16_t, 64, 64, 2, 2, false, 4, 4>(a, tiles_m, stream);
  return launch_cfg<float, 64, 64, 2, 2, false, 4, 4>(a, tiles_m, stream);
}

}  // namespace moe
