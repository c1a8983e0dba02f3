// Grouped expert GEMMs for gfx950 on MFMA (16x16 tiles, fp32 accumulate).
//
// The experts are SwiGLU networks (Zero to Frontier §13.1 "Why MoE", section "The MoE
// layer"): h = SiLU(X W_g) * (X W_u), then o = h W_d.  After dispatch the rows of each
// expert are contiguous, so each product is a grouped GEMM ("replace the loop itself
// with a grouped matrix multiply", the same page's "In PyTorch" section).  Weights are
// stored [out, in], so both operands are read along the contraction dimension.
//
// One kernel template, three tile configurations:
//   large   BM=128 BN=128, 2x2 waves  -- many rows per expert (MFMA-bound)
//   stream  BM=192 BN=64,  1x4 waves  -- ~100-190 rows per expert: one block holds all
//                                         of an expert's rows, so each weight tile is read once
//   decode  BM=16  BN=64,  1x4 waves  -- a few rows per expert (weight streaming)
// The gate/up variant holds two accumulators per output tile (gate and up rows of the
// same n-tile share the A fragments) and applies SiLU(a) * b in registers; the down
// variant writes fp32.
//
// Memory path per K step (128 bytes of each row): global -> registers (16 B per thread
// per piece, coalesced along K) -> LDS (XOR-swizzled 16-byte pieces) -> MFMA operands,
// with the next step's global loads in flight during the current step's MFMAs
// (two LDS stages, one barrier per step).
//
// Scheduling: a persistent grid of (#CUs x occupancy) blocks; tiles are numbered
// L = 0 .. live-1 and each XCD (blocks b with b % 8 == x) walks its own contiguous
// eighth of L, so tiles that share operands run on the same L2.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

struct GemmArgs {
  const void* A;            // [rows, K] activations in expert order
  const void* B0;           // [G, N, K] gate (gated) or down weights
  const void* B1;           // [G, N, K] up weights (gated only)
  const int32_t* offsets;   // [G+1] or NULL (dense: one group of dense_rows)
  const int32_t* tstart;    // [G+1] first m-tile of each group (unused when dense)
  int G, dense_rows, N, K;
  void* C;                  // [rows, N]  (dtype for gated, fp32 for down)
  int m_fast;               // tile order: 1 = m-tiles fastest, 0 = n-tiles fastest
};

template <typename T, int BM, int BN, int WM, int WN, bool GATED>
struct GemmTile {
  static constexpr int NT = WM * WN * kWave;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / 16, TN = WTN / 16;
  static constexpr int NB = GATED ? 2 : 1;
  static constexpr int BROWS = BN * NB;
  static constexpr int ROWB = 128;                                  // bytes of K per row per stage
  static constexpr int EPP = Mfma<T>::kElemsPerPiece;               // elements per 16-byte piece
  static constexpr int BKE = 8 * EPP;                               // elements of K per stage
  static constexpr int A_IT = (BM * 8 + NT - 1) / NT;
  static constexpr int B_IT = (BROWS * 8 + NT - 1) / NT;
  static constexpr int STAGE = (BM + BROWS) * ROWB;
  static constexpr int LDS = 2 * STAGE;
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be whole 16x16 MFMA tiles");
};

__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

template <typename T, int BM, int BN, int WM, int WN, bool GATED>
__global__ __launch_bounds__(WM* WN * 64) void grouped_gemm_kernel(GemmArgs args) {
  using Cfg = GemmTile<T, BM, BN, WM, WN, GATED>;
  constexpr int NT = Cfg::NT, TM = Cfg::TM, TN = Cfg::TN, NB = Cfg::NB, BROWS = Cfg::BROWS;
  constexpr int A_IT = Cfg::A_IT, B_IT = Cfg::B_IT, EPP = Cfg::EPP, BKE = Cfg::BKE, STAGE = Cfg::STAGE;
  extern __shared__ __align__(16) char lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int N = args.N, K = args.K, G = args.G;
  const int ntn = N / BN;
  const int32_t* __restrict__ offsets = args.offsets;
  const int32_t* __restrict__ tstart = args.tstart;
  const int mt_live = offsets ? tstart[G] : (args.dense_rows + BM - 1) / BM;
  const int live = mt_live * ntn;
  const int xcd = blockIdx.x % kNumXcd, j0 = blockIdx.x / kNumXcd, bpx = gridDim.x / kNumXcd;
  const int lo = (int)((long long)live * xcd / kNumXcd);
  const int hi = (int)((long long)live * (xcd + 1) / kNumXcd);
  const int nks = K / BKE;
  const size_t row_stride = (size_t)K * sizeof(T);   // bytes per row of A and of every weight

  for (int L = lo + j0; L < hi; L += bpx) {
    int mt, nt;
    if (args.m_fast) { mt = L % mt_live; nt = L / mt_live; }
    else { nt = L % ntn; mt = L / ntn; }
    int g = 0, row0, rows;
    if (offsets) {
      int a = 0, b = G - 1;                            // largest g with tstart[g] <= mt
      while (a < b) {
        int mid = (a + b + 1) >> 1;
        if (tstart[mid] <= mt) a = mid; else b = mid - 1;
      }
      g = a;
      row0 = offsets[g] + (mt - tstart[g]) * BM;
      rows = min(BM, offsets[g + 1] - row0);
    } else {
      row0 = mt * BM;
      rows = min(BM, args.dense_rows - row0);
    }
    const char* Ab = (const char*)args.A + (size_t)row0 * row_stride;
    const char* B0b = (const char*)args.B0 + ((size_t)g * N + (size_t)nt * BN) * row_stride;
    const char* B1b = GATED ? (const char*)args.B1 + ((size_t)g * N + (size_t)nt * BN) * row_stride : nullptr;

    f32x4_t acc0[TM][TN], acc1[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        acc0[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        acc1[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }

    u32x4_t ra[A_IT], rb[B_IT];
    auto load_global = [&](int ks) {
      const size_t kb = (size_t)ks * 128;
#pragma unroll
      for (int it = 0; it < A_IT; ++it) {
        const int p = tid + it * NT;
        const int r = p >> 3, c = p & 7;
        if (p < BM * 8 && r < rows)
          ra[it] = *(const u32x4_t*)(Ab + (size_t)r * row_stride + kb + c * 16);
        else
          ra[it] = u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int it = 0; it < B_IT; ++it) {
        const int p = tid + it * NT;
        const int r = p >> 3, c = p & 7;
        if (p < BROWS * 8) {
          const char* src = (!GATED || r < BN) ? B0b + (size_t)r * row_stride : B1b + (size_t)(r - BN) * row_stride;
          rb[it] = *(const u32x4_t*)(src + kb + c * 16);
        }
      }
    };
    auto store_lds = [&](int s) {
      char* As = lds + s * STAGE;
      char* Bs = As + BM * 128;
#pragma unroll
      for (int it = 0; it < A_IT; ++it) {
        const int p = tid + it * NT;
        if (p < BM * 8) *(u32x4_t*)(As + swz(p >> 3, p & 7)) = ra[it];
      }
#pragma unroll
      for (int it = 0; it < B_IT; ++it) {
        const int p = tid + it * NT;
        if (p < BROWS * 8) *(u32x4_t*)(Bs + swz(p >> 3, p & 7)) = rb[it];
      }
    };
    auto compute = [&](int s) {
      const char* As = lds + s * STAGE;
      const char* Bs = As + BM * 128;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const int c = kc * 4 + (lane >> 4);
        u32x4_t bfr[TN * NB];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int r = wn * Cfg::WTN + j * 16 + (lane & 15);
          bfr[j] = *(const u32x4_t*)(Bs + swz(r, c));
          if constexpr (GATED) bfr[TN + j] = *(const u32x4_t*)(Bs + swz(BN + r, c));
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if (wm * Cfg::WTM + i * 16 < rows) {          // wave-uniform: skip all-padding subtiles
            const int r = wm * Cfg::WTM + i * 16 + (lane & 15);
            const u32x4_t af = *(const u32x4_t*)(As + swz(r, c));
#pragma unroll
            for (int j = 0; j < TN; ++j) {
              Mfma<T>::step(acc0[i][j], af, bfr[j]);
              if constexpr (GATED) Mfma<T>::step(acc1[i][j], af, bfr[TN + j]);
            }
          }
        }
      }
    };

    load_global(0);
    store_lds(0);
    __syncthreads();
    for (int ks = 0; ks < nks; ++ks) {
      if (ks + 1 < nks) load_global(ks + 1);
      compute(ks & 1);
      if (ks + 1 < nks) store_lds((ks + 1) & 1);
      __syncthreads();
    }

    // epilogue: lane holds rows 4*(lane/16)+q of each 16x16 tile, column lane%16
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = wm * Cfg::WTM + i * 16 + (lane >> 4) * 4 + q;
          const int col = nt * BN + wn * Cfg::WTN + j * 16 + (lane & 15);
          if (r < rows) {
            const size_t o = (size_t)(row0 + r) * N + col;
            if constexpr (GATED) {
              const float a = acc0[i][j][q], b = acc1[i][j][q];
              const float h = a / (1.f + expf(-a)) * b;     // SiLU(a) * b
              ((T*)args.C)[o] = ElemOut<T>::from_f32(h);
            } else {
              ((float*)args.C)[o] = acc0[i][j][q];
            }
          }
        }
  }
}

// ------------------------------------------------------------------------------ launch

template <typename T, int BM, int BN, int WM, int WN, bool GATED>
static hipError_t launch_cfg(const GemmArgs& a, int max_tiles_m, hipStream_t stream) {
  using Cfg = GemmTile<T, BM, BN, WM, WN, GATED>;
  auto kern = grouped_gemm_kernel<T, BM, BN, WM, WN, GATED>;
  static const int occ = [&] {
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS);
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, Cfg::NT, Cfg::LDS) != hipSuccess || n < 1) n = 1;
    return n;
  }();
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return hipErrorInvalidDevice;
  const long long max_live = (long long)max_tiles_m * (a.N / BN);
  long long grid = std::min<long long>(max_live, (long long)cus * occ);
  grid = ((grid + kNumXcd - 1) / kNumXcd) * kNumXcd;
  if (grid < kNumXcd) grid = kNumXcd;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(Cfg::NT), Cfg::LDS, stream, a);
  return hipGetLastError();
}

int gemm_block_m(GemmKind kind) { return kind == kGemmLarge ? 128 : (kind == kGemmStream ? 192 : 16); }

template <typename T, bool GATED>
static hipError_t dispatch_kind(GemmKind kind, GemmArgs a, int max_tiles_m, hipStream_t s) {
  switch (kind) {
    case kGemmLarge: a.m_fast = 1; return launch_cfg<T, 128, 128, 2, 2, GATED>(a, max_tiles_m, s);
    case kGemmStream: a.m_fast = 0; return launch_cfg<T, 192, 64, 1, 4, GATED>(a, max_tiles_m, s);
    default: a.m_fast = 0; return launch_cfg<T, 16, 64, 1, 4, GATED>(a, max_tiles_m, s);
  }
}

hipError_t launch_gemm_gateup(GemmKind kind, int dtype, const void* A, const void* Wg, const void* Wu,
                              const int32_t* offsets, const int32_t* tstart, int G, int dense_rows, int max_tiles_m,
                              int N, int K, void* H, hipStream_t stream) {
  GemmArgs a{A, Wg, Wu, offsets, tstart, G, dense_rows, N, K, H, 0};
  return dtype == 1 ? dispatch_kind<uint16_t, true>(kind, a, max_tiles_m, stream)
                    : dispatch_kind<float, true>(kind, a, max_tiles_m, stream);
}

hipError_t launch_gemm_down(GemmKind kind, int dtype, const void* H, const void* Wd, const int32_t* offsets,
                            const int32_t* tstart, int G, int dense_rows, int max_tiles_m, int N, int K, float* O,
                            hipStream_t stream) {
  GemmArgs a{H, Wd, nullptr, offsets, tstart, G, dense_rows, N, K, O, 0};
  return dtype == 1 ? dispatch_kind<uint16_t, false>(kind, a, max_tiles_m, stream)
                    : dispatch_kind<float, false>(kind, a, max_tiles_m, stream);
}

}  // namespace moe
