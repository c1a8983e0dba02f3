// Router logits of one block of tokens (shared by the forward router and its backward,
// so both see the same fp32 logits bit for bit).
#pragma once

#include "common.h"
#include "kernels.h"

namespace moe {

// Contraction split of the router for E experts: 4 waves share the work.
__host__ __device__ inline int router_ksplit(int E) {
  const int groups = ((E + 15) / 16 + 3) / 4;
  return groups == 1 ? 4 : (groups == 2 ? 2 : 1);
}

// Partial logits of NTL consecutive expert tiles over chunks [c0, c1) of 64 bytes.  With one
// or two expert tiles the loads of U = 16 or 8 chunks are issued before their MFMAs (the
// accumulation order over chunks is unchanged), so that many chunks' memory latency overlaps
// (one tile: 16 rather than 8 took the Mixtral-shape router from 18.2 to 17.2 us); with more
// tiles each chunk already has NTL + 1 loads in flight (measured: batching them too is slower
// at 256 experts).
template <typename T, int NTL>
__device__ __forceinline__ void router_tiles(const char* xrow, const char* const* wrow, int c0, int c1,
                                             f32x4_t* acc) {
  constexpr int U = NTL >= 3 ? 1 : (NTL == 1 ? 16 : 8);
  int c = c0;
  for (; U > 1 && c + U <= c1; c += U) {
    u32x4_t a[U], b[U][NTL];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      a[u] = *(const u32x4_t*)(xrow + (size_t)(c + u) * 64);
#pragma unroll
      for (int j = 0; j < NTL; ++j) b[u][j] = *(const u32x4_t*)(wrow[j] + (size_t)(c + u) * 64);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < NTL; ++j) Mfma<T>::step(acc[j], a[u], b[u][j]);
  }
  for (; c < c1; ++c) {
    const u32x4_t a = *(const u32x4_t*)(xrow + (size_t)c * 64);
#pragma unroll
    for (int j = 0; j < NTL; ++j) {
      const u32x4_t b = *(const u32x4_t*)(wrow[j] + (size_t)c * 64);
      Mfma<T>::step(acc[j], a, b);
    }
  }
}

// Logits [kRouteTokens][E] of tokens t0 .. t0+15 into LDS (`logits` holds router_ksplit(E)
// partial copies), bias added last when b_r != NULL; ends with a block barrier.
// 16x16 MFMA tiles (A = 16 token rows, B = 16 router rows), operands read straight from
// global memory (16 B per lane).  Expert tiles are dealt to waves in groups of up to 4;
// with fewer than 4 groups the contraction is split across waves instead, and the partial
// logits are summed in LDS in a fixed order.
template <typename T>
__device__ __forceinline__ void router_block_logits(const T* __restrict__ x, const T* __restrict__ w_r,
                                                    const float* __restrict__ b_r, int T_, int d, int E, int t0,
                                                    float* logits, int wave, int lane, int tid) {
  constexpr int TB = kRouteTokens;
  const int ksplit = router_ksplit(E);
  const int r16 = lane & 15, grp = lane >> 4;
  const int tok = min(t0 + r16, T_ - 1);            // rows past T repeat row T-1; never used
  const size_t row_bytes = (size_t)d * sizeof(T);
  const char* xrow = (const char*)x + (size_t)tok * row_bytes + grp * 16;
  const int nchunks = (int)(row_bytes / 64);
  const int n_et = (E + 15) / 16;
  const int kpart = wave % ksplit;
  const int c0 = kpart * nchunks / ksplit, c1 = (kpart + 1) * nchunks / ksplit;
  float* part = logits + kpart * TB * E;
  for (int tb = (wave / ksplit) * 4; tb < n_et; tb += 4 * (4 / ksplit)) {
    const int ntl = min(4, n_et - tb);
    const char* wrow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int e = min((tb + j) * 16 + r16, E - 1);
      wrow[j] = (const char*)w_r + (size_t)e * row_bytes + grp * 16;
    }
    f32x4_t acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    switch (ntl) {
      case 4: router_tiles<T, 4>(xrow, wrow, c0, c1, acc); break;
      case 3: router_tiles<T, 3>(xrow, wrow, c0, c1, acc); break;
      case 2: router_tiles<T, 2>(xrow, wrow, c0, c1, acc); break;
      default: router_tiles<T, 1>(xrow, wrow, c0, c1, acc); break;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int e = (tb + j) * 16 + r16;
      if (j < ntl && e < E) {
#pragma unroll
        for (int i = 0; i < 4; ++i) part[(grp * 4 + i) * E + e] = acc[j][i];
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < TB * E; i += 256) {          // fixed-order sum of the K parts, then bias
    float v = logits[i];
    for (int p = 1; p < ksplit; ++p) v += logits[p * TB * E + i];
    logits[i] = v + (b_r ? b_r[i % E] : 0.f);
  }
  __syncthreads();
}

// The same [kRouteTokens][E] LDS logits from the router GEMM's output: ksp partial [T, E] arrays
// summed in chunk order, then the bias when b_r != NULL; ends with a block barrier.
__device__ __forceinline__ void router_block_logits_from(const float* __restrict__ lg, int ksp, int T_, int E,
                                                         int t0, const float* __restrict__ b_r, float* logits,
                                                         int tid, int nthreads) {
  const size_t chunk = (size_t)T_ * E;
  for (int i = tid; i < kRouteTokens * E; i += nthreads) {
    const int tl = i / E, e = i - tl * E;
    const int t = min(t0 + tl, T_ - 1);                   // rows past T repeat row T-1; never used
    const float* src = lg + (size_t)t * E + e;
    float v = src[0];
    for (int c = 1; c < ksp; ++c) v += src[c * chunk];
    logits[i] = v + (b_r ? b_r[e] : 0.f);
  }
  __syncthreads();
}

}  // namespace moe
