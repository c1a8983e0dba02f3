// Backward pass of the MoE layer, everything but the grouped GEMMs: padded layouts for the
// weight-gradient products, transposes, the router backward, dW_r and the assembly of dx.
//
// The routing is held fixed: the top-k choice is a hard selection with no gradient, and the
// router learns only through the weights of the chosen experts (Moatlab AI-064,
// "Inside the Router"); aux = E sum_e f_e P_e adds its P_e term (f_e are counts).
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "router_logits.h"

namespace moe {

// ------------------------------------------------------------------------------ layouts

// poff[e] = sum_{e' < e} roundup(kept_e', 64) (e = 0..E): each expert's rows start on a whole
// K step in the transposed operands of the weight-gradient products.  Also writes
// koff_dense = {0, dense_pad} (the one group of a dense product) when it is not NULL.
__global__ __launch_bounds__(1024) void pad_offsets_kernel(const int32_t* __restrict__ offsets, int E,
                                                           int32_t* __restrict__ poff, int dense_pad,
                                                           int32_t* __restrict__ koff_dense) {
  __shared__ int s[1024];
  const int e = threadIdx.x;
  s[e] = e < E ? ((offsets[e + 1] - offsets[e] + 63) & ~63) : 0;
  __syncthreads();
  for (int o = 1; o < 1024; o <<= 1) {
    const int t = e >= o ? s[e - o] : 0;
    __syncthreads();
    s[e] += t;
    __syncthreads();
  }
  if (e < E) poff[e + 1] = s[e];
  if (e == 0) {
    poff[0] = 0;
    if (koff_dense) {
      koff_dense[0] = 0;
      koff_dense[1] = dense_pad;
    }
  }
}

// g_row[row_of[a]] = gate[a] for every kept assignment a = t*k + j.
__global__ __launch_bounds__(256) void row_gate_kernel(const int32_t* __restrict__ row_of,
                                                       const float* __restrict__ gate, int R,
                                                       float* __restrict__ g_row) {
  const int a = blockIdx.x * 256 + threadIdx.x;
  if (a < R) {
    const int row = row_of[a];
    if (row >= 0) g_row[row] = gate[a];
  }
}

hipError_t launch_bwd_layout(const int32_t* offsets, int E, const int32_t* row_of, const float* gate, int R,
                             int32_t* poff, float* g_row, int dense_pad, int32_t* koff_dense, hipStream_t stream) {
  if (E > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(pad_offsets_kernel, dim3(1), dim3(1024), 0, stream, offsets, E, poff, dense_pad, koff_dense);
  if (R > 0) hipLaunchKernelGGL(row_gate_kernel, dim3((R + 255) / 256), dim3(256), 0, stream, row_of, gate, R, g_row);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ transposes

template <typename T> struct Elem4;
template <> struct Elem4<uint16_t> {
  typedef uint2 V;
  __device__ static void to_f32(V v, float* f) {
    f[0] = bf16_bits_to_f32(v.x & 0xffffu); f[1] = bf16_bits_to_f32(v.x >> 16);
    f[2] = bf16_bits_to_f32(v.y & 0xffffu); f[3] = bf16_bits_to_f32(v.y >> 16);
  }
  __device__ static V from_f32(const float* f) {
    return V{f32x2_to_bf16x2_bits(f[0], f[1]), f32x2_to_bf16x2_bits(f[2], f[3])};
  }
};
template <> struct Elem4<float> {
  typedef float4 V;
  __device__ static void to_f32(V v, float* f) { f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w; }
  __device__ static V from_f32(const float* f) { return V{f[0], f[1], f[2], f[3]}; }
};

// One 64 x 64 tile: dst[c][p] (leading dimension ldd) from source rows src_row(p) (a row
// index, or -1 for a zero column) times scale(p).  Rows and columns come in whole groups of 4.
template <typename TI, typename TO>
__device__ __forceinline__ void transpose_tile(const TI* __restrict__ src, size_t lds, int C, const int* srow,
                                               const float* sscale, TO* __restrict__ dst, size_t ldd, int c0,
                                               int p0, float (*tile)[65]) {
  const int tid = threadIdx.x;
  // load: thread -> tile row (p) tid / 16 + 16 i, columns 4 (tid % 16) .. +3
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int pp = tid / 16 + 16 * i, cc = 4 * (tid % 16);
    float f[4] = {0.f, 0.f, 0.f, 0.f};
    const int r = srow[pp];
    if (r >= 0 && c0 + cc < C) {
      Elem4<TI>::to_f32(*(const typename Elem4<TI>::V*)(src + (size_t)r * lds + c0 + cc), f);
      const float sc = sscale[pp];
#pragma unroll
      for (int q = 0; q < 4; ++q) f[q] *= sc;
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) tile[pp][cc + q] = f[q];
  }
  __syncthreads();
  // store: thread -> dst row (c) tid / 16 + 16 i, columns (p) 4 (tid % 16) .. +3
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int cc = tid / 16 + 16 * i, pp = 4 * (tid % 16);
    if (c0 + cc < C) {
      float f[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) f[q] = tile[pp + q][cc];
      *(typename Elem4<TO>::V*)(dst + (size_t)(c0 + cc) * ldd + p0 + pp) = Elem4<TO>::from_f32(f);
    }
  }
}

// dst[b][c][coff + r] = src[b][r][c]: src [B, Rn, C], dst [B, C, ldd].  Grid (C/64, Rn/64 * B).
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src, int Rn, int C, T* __restrict__ dst,
                                                        int ldd, int coff, size_t dst_batch) {
  __shared__ float tile[64][65];
  __shared__ int srow[64];
  __shared__ float sscale[64];
  const int rtiles = Rn / 64;
  const int b = blockIdx.y / rtiles, r0 = (blockIdx.y % rtiles) * 64, c0 = blockIdx.x * 64;
  if (threadIdx.x < 64) {
    srow[threadIdx.x] = r0 + threadIdx.x;
    sscale[threadIdx.x] = 1.f;
  }
  __syncthreads();
  transpose_tile<T, T>(src + (size_t)b * Rn * C, (size_t)C, C, srow, sscale, dst + (size_t)b * dst_batch, (size_t)ldd,
                       c0, coff + r0, tile);
}

hipError_t launch_transpose(int dtype, const void* src, int B, int Rn, int C, void* dst, int ldd, int coff,
                            size_t dst_batch, hipStream_t stream) {
  if (Rn % 64 || C % 64 || ldd % 4 || coff % 4) return hipErrorInvalidValue;
  if (B == 0 || Rn == 0) return hipSuccess;
  dim3 grid(C / 64, (Rn / 64) * B);
  if (dtype == 1)
    hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, dim3(256), 0, stream, (const uint16_t*)src, Rn, C,
                       (uint16_t*)dst, ldd, coff, dst_batch);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, stream, (const float*)src, Rn, C, (float*)dst,
                       ldd, coff, dst_batch);
  return hipGetLastError();
}

// dst [C, ldt]: column p of group e holds source row src_of(r) of expert-ordered row
// r = offsets[e] + p - poff[e] (times scale[r]) while r < offsets[e+1], else zeros.  With
// offsets == NULL there is one group of n_dense rows (p = r).  src_of(r) = rows[r], or r.
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void gather_t_kernel(const TI* __restrict__ src, int C,
                                                       const int32_t* __restrict__ rows,
                                                       const float* __restrict__ scale,
                                                       const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ poff, int E, int n_dense,
                                                       TO* __restrict__ dst, int ldt) {
  __shared__ float tile[64][65];
  __shared__ int srow[64];
  __shared__ float sscale[64];
  const int p0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
  int lo = 0, hi = n_dense, pbase = 0;
  if (offsets) {
    if (p0 >= poff[E]) return;                           // past the last group (block-uniform)
    int a = 0, b = E - 1;                                // last e with poff[e] <= p0
    while (a < b) {
      const int mid = (a + b + 1) >> 1;
      if (poff[mid] <= p0) a = mid; else b = mid - 1;
    }
    lo = offsets[a];
    hi = offsets[a + 1];
    pbase = poff[a];
  }
  if (threadIdx.x < 64) {
    const int r = lo + p0 + (int)threadIdx.x - pbase;
    const bool ok = r < hi;
    srow[threadIdx.x] = ok ? (rows ? rows[r] : r) : -1;
    sscale[threadIdx.x] = ok && scale ? scale[r] : 1.f;
  }
  __syncthreads();
  transpose_tile<TI, TO>(src, (size_t)C, C, srow, sscale, dst, (size_t)ldt, c0, p0, tile);
}

hipError_t launch_gather_t(int src_dtype, int dst_dtype, const void* src, int C, const int32_t* rows,
                           const float* scale, const int32_t* offsets, const int32_t* poff, int E, int n_dense,
                           int p_bound, void* dst, int ldt, hipStream_t stream) {
  if (C % 64 || ldt % 64 || p_bound % 64 || p_bound > ldt) return hipErrorInvalidValue;
  if (p_bound == 0) return hipSuccess;
  dim3 grid(p_bound / 64, C / 64);
  if (src_dtype == 0 && dst_dtype == 1)
    hipLaunchKernelGGL((gather_t_kernel<float, uint16_t>), grid, dim3(256), 0, stream, (const float*)src, C, rows,
                       scale, offsets, poff, E, n_dense, (uint16_t*)dst, ldt);
  else if (src_dtype == 1 && dst_dtype == 1)
    hipLaunchKernelGGL((gather_t_kernel<uint16_t, uint16_t>), grid, dim3(256), 0, stream, (const uint16_t*)src, C,
                       rows, scale, offsets, poff, E, n_dense, (uint16_t*)dst, ldt);
  else if (src_dtype == 0 && dst_dtype == 0)
    hipLaunchKernelGGL((gather_t_kernel<float, float>), grid, dim3(256), 0, stream, (const float*)src, C, rows, scale,
                       offsets, poff, E, n_dense, (float*)dst, ldt);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// Zero the gap columns [poff[e] + kept_e, poff[e+1]) of rows [0, nrows) of dst [nrows, ldt]
// (one group [n_dense, pad_dense) when offsets == NULL).  Grid (nrows / 16, groups).
template <typename T>
__global__ __launch_bounds__(256) void zero_gaps_kernel(T* __restrict__ dst, int nrows, int ldt,
                                                        const int32_t* __restrict__ offsets,
                                                        const int32_t* __restrict__ poff, int n_dense,
                                                        int pad_dense) {
  const int e = blockIdx.y;
  const int c0 = offsets ? poff[e] + (offsets[e + 1] - offsets[e]) : n_dense;
  const int c1 = offsets ? poff[e + 1] : pad_dense;
  const int row = blockIdx.x * 16 + threadIdx.x / 16;
  if (row >= nrows) return;
  for (int c = c0 + (int)(threadIdx.x % 16); c < c1; c += 16) dst[(size_t)row * ldt + c] = T(0);
}

hipError_t launch_zero_gaps(int dtype, void* dst, int nrows, int ldt, const int32_t* offsets, const int32_t* poff,
                            int E, int n_dense, int pad_dense, hipStream_t stream) {
  if (nrows == 0) return hipSuccess;
  dim3 grid((nrows + 15) / 16, offsets ? E : 1);
  if (dtype == 1)
    hipLaunchKernelGGL(zero_gaps_kernel<uint16_t>, grid, dim3(256), 0, stream, (uint16_t*)dst, nrows, ldt, offsets,
                       poff, n_dense, pad_dense);
  else
    hipLaunchKernelGGL(zero_gaps_kernel<float>, grid, dim3(256), 0, stream, (float*)dst, nrows, ldt, offsets, poff,
                       n_dense, pad_dense);
  return hipGetLastError();
}

// fp32 -> bf16 (round to nearest even), n a multiple of 4.
__global__ __launch_bounds__(256) void to_bf16_kernel(const float4* __restrict__ src, uint2* __restrict__ dst,
                                                      size_t n4) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
    const float4 v = src[i];
    const float f[4] = {v.x, v.y, v.z, v.w};
    dst[i] = Elem4<uint16_t>::from_f32(f);
  }
}

hipError_t launch_to_bf16(const float* src, size_t n, void* dst, hipStream_t stream) {
  if (n % 4) return hipErrorInvalidValue;
  if (n == 0) return hipSuccess;
  const size_t n4 = n / 4;
  const unsigned blocks = (unsigned)std::min<size_t>((n4 + 255) / 256, 8192);
  hipLaunchKernelGGL(to_bf16_kernel, dim3(blocks), dim3(256), 0, stream, (const float4*)src, (uint2*)dst, n4);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ router

// dL/dr [T, E] per token, from the recomputed probabilities (same logits code as the
// forward), the slot gradients dg = sum of the row's partial dots (0 for a dropped slot)
// and the aux term:
//   renormalised gates g_j = p_{K_j} / S:  dp_{K_i} = (dg_i - sum_j dg_j g_j) / S,
//   raw gates:                             dp_{K_i} = dg_i,
//   aux:                                   dp_e += d_aux * E * f_e / T,  f_e = counts_e / (T k),
//   softmax: dr = p (dp - sum_e p_e dp_e);  sigmoid (p = sigma(r)): dr = dp p (1 - p).
// One block = 16 tokens, one wave per token at a time; lane l holds experts 64 q + l.
template <typename T, int NQ>   // NQ: 64-expert chunks per lane (E <= 64 NQ)
__global__ __launch_bounds__(256) void router_bwd_kernel(const T* __restrict__ x, const T* __restrict__ w_r,
                                                         const float* __restrict__ b_r, int T_, int d, int E, int k,
                                                         int renorm, int scoring, const int32_t* __restrict__ idx,
                                                         const float* __restrict__ gate,
                                                         const int32_t* __restrict__ row_of,
                                                         const int32_t* __restrict__ counts,
                                                         const float* __restrict__ part, int npart, float d_aux,
                                                         float* __restrict__ dr, float* __restrict__ dgate,
                                                         const float* __restrict__ logits_in, int lsplit) {
  constexpr int TB = kRouteTokens;
  const bool sigm = scoring == 1;
  extern __shared__ float smem[];
  float* logits = smem;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * TB;
  if (logits_in)     // the forward read the router GEMM's logits too
    router_block_logits_from(logits_in, lsplit, T_, E, t0, sigm ? nullptr : b_r, logits, tid, 256);
  else
    router_block_logits<T>(x, w_r, sigm ? nullptr : b_r, T_, d, E, t0, logits, wave, lane, tid);

  const int nq = (E + 63) / 64;
  const float aux_scale = T_ > 0 ? d_aux * (float)E / ((float)T_ * (float)T_ * (float)k) : 0.f;
  for (int tt = 0; tt < 4; ++tt) {
    const int tl = wave * 4 + tt;
    const int t = t0 + tl;
    if (t >= T_) break;
    float v[NQ], p[NQ];
    float m = -INFINITY, inv = 1.f;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = q * 64 + lane;
      v[q] = (q < nq && e < E) ? logits[tl * E + e] : -INFINITY;
      m = fmaxf(m, v[q]);
    }
    if (!sigm) {
      m = wave_max(m);
      float s = 0.f;
      if (E <= 16) {
        // the forward router for up to 16 experts sums the softmax terms in expert order
        for (int e = 0; e < E; ++e) {
          const float ve = logits[tl * E + e];
          s += (ve == -INFINITY) ? 0.f : expf(ve - m);
        }
      } else {
#pragma unroll
        for (int q = 0; q < NQ; ++q) s += (v[q] == -INFINITY) ? 0.f : expf(v[q] - m);
        s = wave_sum(s);
      }
      inv = 1.f / s;
#pragma unroll
      for (int q = 0; q < NQ; ++q) p[q] = (v[q] == -INFINITY) ? 0.f : expf(v[q] - m) * inv;
    } else {
#pragma unroll
      for (int q = 0; q < NQ; ++q) p[q] = (v[q] == -INFINITY) ? 0.f : 1.f / (1.f + expf(-v[q]));
    }
    // slot gradients (wave-uniform), S and sum_j dg_j g_j in slot order
    float dgs[16];
    float S = 0.f, G = 0.f;
    for (int j = 0; j < k; ++j) {
      const int row = row_of[(size_t)t * k + j];
      float acc = 0.f;
      if (row >= 0)
        for (int s = lane; s < npart; s += kWave) acc += part[(size_t)row * npart + s];
      const float dg = row >= 0 ? wave_sum(acc) : 0.f;
      dgs[j] = dg;
      const float lg = logits[tl * E + idx[(size_t)t * k + j]];
      const float pj = sigm ? 1.f / (1.f + expf(-lg)) : expf(lg - m) * inv;
      S += pj;
      G = fmaf(dg, gate[(size_t)t * k + j], G);
      if (dgate && lane == 0) dgate[(size_t)t * k + j] = dg;
    }
    float dp[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = q * 64 + lane;
      dp[q] = (q < nq && e < E) ? aux_scale * (float)counts[e] : 0.f;
    }
    for (int j = 0; j < k; ++j) {
      const int e = idx[(size_t)t * k + j];
      const float dpk = renorm ? (dgs[j] - G) / S : dgs[j];
#pragma unroll
      for (int q = 0; q < NQ; ++q)
        if (e == q * 64 + lane) dp[q] += dpk;
    }
    float c = 0.f;
    if (!sigm) {
#pragma unroll
      for (int q = 0; q < NQ; ++q) c = fmaf(p[q], dp[q], c);
      c = wave_sum(c);
    }
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int e = q * 64 + lane;
      if (q < nq && e < E) dr[(size_t)t * E + e] = sigm ? dp[q] * p[q] * (1.f - p[q]) : p[q] * (dp[q] - c);
    }
  }
}

template <typename T, int NQ>
static void router_bwd_launch(int nb, size_t lds, hipStream_t stream, const void* x, const void* w_r,
                              const float* b_r, int T_, int d, int E, int k, int renorm, int scoring,
                              const int32_t* idx, const float* gate, const int32_t* row_of, const int32_t* counts,
                              const float* part, int npart, float d_aux, float* dr, float* dgate,
                              const float* logits_in, int lsplit) {
  auto kern = router_bwd_kernel<T, NQ>;
  (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL(kern, dim3(nb), dim3(256), lds, stream, (const T*)x, (const T*)w_r, b_r, T_, d, E, k, renorm,
                     scoring, idx, gate, row_of, counts, part, npart, d_aux, dr, dgate, logits_in, lsplit);
}

template <typename T>
static void router_bwd_launch_nq(int nb, size_t lds, hipStream_t stream, const void* x, const void* w_r,
                                 const float* b_r, int T_, int d, int E, int k, int renorm, int scoring,
                                 const int32_t* idx, const float* gate, const int32_t* row_of,
                                 const int32_t* counts, const float* part, int npart, float d_aux, float* dr,
                                 float* dgate, const float* logits_in, int lsplit) {
  if (E <= 64)
    router_bwd_launch<T, 1>(nb, lds, stream, x, w_r, b_r, T_, d, E, k, renorm, scoring, idx, gate, row_of, counts,
                            part, npart, d_aux, dr, dgate, logits_in, lsplit);
  else if (E <= 256)
    router_bwd_launch<T, 4>(nb, lds, stream, x, w_r, b_r, T_, d, E, k, renorm, scoring, idx, gate, row_of, counts,
                            part, npart, d_aux, dr, dgate, logits_in, lsplit);
  else
    router_bwd_launch<T, 16>(nb, lds, stream, x, w_r, b_r, T_, d, E, k, renorm, scoring, idx, gate, row_of, counts,
                             part, npart, d_aux, dr, dgate, logits_in, lsplit);
}

hipError_t launch_router_bwd(int dtype, const void* x, const void* w_r, const float* b_r, int T, int d, int E, int k,
                             int renorm, int scoring, const int32_t* idx, const float* gate, const int32_t* row_of,
                             const int32_t* counts, const float* part, int npart, float d_aux, float* dr,
                             float* dgate, float* logits, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  const float* logits_in = nullptr;
  if (router_logits_by_gemm(E)) {   // the forward's logits path, recomputed the same way
    if (!logits) return hipErrorInvalidValue;
    const hipError_t e = launch_gemm_router(dtype, x, w_r, T, d, E, logits, stream);
    if (e != hipSuccess) return e;
    logits_in = logits;
  }
  const int lsplit = router_gemm_ksplit(d);
  const size_t lds = (size_t)router_ksplit(E) * kRouteTokens * E * sizeof(float);
  if (dtype == 1)
    router_bwd_launch_nq<uint16_t>(route_blocks(T), lds, stream, x, w_r, b_r, T, d, E, k, renorm, scoring, idx, gate,
                                   row_of, counts, part, npart, d_aux, dr, dgate, logits_in, lsplit);
  else
    router_bwd_launch_nq<float>(route_blocks(T), lds, stream, x, w_r, b_r, T, d, E, k, renorm, scoring, idx, gate,
                                row_of, counts, part, npart, d_aux, dr, dgate, logits_in, lsplit);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ dW_r, dx

// dW_r [E, d] = dr^T x and db_r[e] = sum_t dr[t, e] (fp32).  Tokens come in chunks of
// kDwrChunk: block (c-tile, e-tile, chunk) sums its chunk's tokens in ascending order into
// part [chunks, E, d] (and bpart [chunks, E]); dwr_reduce_kernel adds the chunks in order.
// 64 x 64 output tile per block, 16 tokens per LDS step, 4 x 4 outputs per thread.
constexpr int kDwrChunk = 256;

template <typename T>
__global__ __launch_bounds__(256) void dwr_kernel(const float* __restrict__ dr, const T* __restrict__ x, int T_, int d,
                                                  int E, float* __restrict__ part, float* __restrict__ bpart) {
  __shared__ float sA[16][64], sB[16][64];
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  const int c0 = blockIdx.x * 64, e0 = blockIdx.y * 64, ch = blockIdx.z;
  const int tbeg = ch * kDwrChunk, tend = min(T_, tbeg + kDwrChunk);
  float acc[4][4] = {};
  float bsum[4] = {0.f, 0.f, 0.f, 0.f};
  for (int t0 = tbeg; t0 < tend; t0 += 16) {
    {
      const int kk = tid / 16, cc = 4 * (tid % 16), t = t0 + kk;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = e0 + cc + q;
        sA[kk][cc + q] = (t < tend && e < E) ? dr[(size_t)t * E + e] : 0.f;
      }
      float f[4] = {0.f, 0.f, 0.f, 0.f};
      if (t < tend && c0 + cc < d) Elem4<T>::to_f32(*(const typename Elem4<T>::V*)(x + (size_t)t * d + c0 + cc), f);
#pragma unroll
      for (int q = 0; q < 4; ++q) sB[kk][cc + q] = f[q];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = sA[kk][ty * 4 + i];
        bsum[i] += a;
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a, sB[kk][tx * 4 + j], acc[i][j]);
      }
    }
    __syncthreads();
  }
  float* out = part + (size_t)ch * E * d;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = e0 + ty * 4 + i;
    if (e >= E) continue;
    const int c = c0 + tx * 4;
    if (c < d) *(float4*)(out + (size_t)e * d + c) = float4{acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
    if (blockIdx.x == 0 && tx == 0) bpart[(size_t)ch * E + e] = bsum[i];
  }
}

// dw_r[i] = sum over chunks of part[ch][i] (i < E*d), db_r[e] likewise (zeros when zero_bias).
__global__ __launch_bounds__(256) void dwr_reduce_kernel(const float* __restrict__ part,
                                                         const float* __restrict__ bpart, int nch, size_t n, int E,
                                                         float* __restrict__ dw_r, float* __restrict__ db_r,
                                                         int zero_bias) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n + (size_t)E; i += (size_t)gridDim.x * 256) {
    if (i < n) {
      float v = 0.f;
      for (int ch = 0; ch < nch; ++ch) v += part[(size_t)ch * n + i];
      dw_r[i] = v;
    } else if (db_r) {
      const size_t e = i - n;
      float v = 0.f;
      for (int ch = 0; ch < nch; ++ch) v += bpart[(size_t)ch * E + e];
      db_r[e] = zero_bias ? 0.f : v;
    }
  }
}

size_t dwr_workspace_bytes(int T, int d, int E) {
  const size_t nch = (size_t)(T + kDwrChunk - 1) / kDwrChunk;
  return nch * (size_t)E * ((size_t)d + 1) * sizeof(float);
}

hipError_t launch_dwr(int dtype, const float* dr, const void* x, int T, int d, int E, float* dw_r, float* db_r,
                      int zero_bias, float* part, hipStream_t stream) {
  const int nch = (T + kDwrChunk - 1) / kDwrChunk;
  float* bpart = part + (size_t)nch * E * d;
  if (nch > 0) {
    dim3 grid((d + 63) / 64, (E + 63) / 64, nch);
    if (dtype == 1)
      hipLaunchKernelGGL(dwr_kernel<uint16_t>, grid, dim3(256), 0, stream, dr, (const uint16_t*)x, T, d, E, part,
                         bpart);
    else
      hipLaunchKernelGGL(dwr_kernel<float>, grid, dim3(256), 0, stream, dr, (const float*)x, T, d, E, part, bpart);
  }
  const size_t n = (size_t)E * d;
  const unsigned blocks = (unsigned)std::min<size_t>((n + E + 255) / 256, 4096);
  hipLaunchKernelGGL(dwr_reduce_kernel, dim3(blocks), dim3(256), 0, stream, part, bpart, nch, n, E, dw_r, db_r,
                     zero_bias);
  return hipGetLastError();
}

// dx[t] = sum_e dr[t, e] W_r[e] (experts in ascending order), then + dX[row_of[t, j]] for the
// kept slots j = 0 .. k-1 in order, then + dXs[t] (the shared expert) when present.
// 64 tokens x 64 columns per block, 16 experts per LDS step.
template <typename T>
__global__ __launch_bounds__(256) void dx_kernel(const float* __restrict__ dr, const T* __restrict__ w_r, int T_,
                                                 int d, int E, int k, const float* __restrict__ dX,
                                                 const int32_t* __restrict__ row_of, const float* __restrict__ dXs,
                                                 float* __restrict__ dx) {
  __shared__ float sA[16][64], sB[16][64];
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  const int c0 = blockIdx.x * 64, t0 = blockIdx.y * 64;
  float acc[4][4] = {};
  for (int e0 = 0; e0 < E; e0 += 16) {
    {
      const int kk = tid % 16, tt = 4 * (tid / 16);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int t = t0 + tt + q;
        sA[kk][tt + q] = (t < T_ && e0 + kk < E) ? dr[(size_t)t * E + e0 + kk] : 0.f;
      }
      const int ke = tid / 16, cc = 4 * (tid % 16);
      float f[4] = {0.f, 0.f, 0.f, 0.f};
      if (e0 + ke < E && c0 + cc < d)
        Elem4<T>::to_f32(*(const typename Elem4<T>::V*)(w_r + (size_t)(e0 + ke) * d + c0 + cc), f);
#pragma unroll
      for (int q = 0; q < 4; ++q) sB[ke][cc + q] = f[q];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = sA[kk][ty * 4 + i];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a, sB[kk][tx * 4 + j], acc[i][j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + ty * 4 + i;
    if (t >= T_) continue;
    const int c = c0 + tx * 4;
    if (c >= d) continue;
    float v[4] = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
    for (int j = 0; j < k; ++j) {
      const int row = row_of[(size_t)t * k + j];
      if (row >= 0) {
        const float4 w = *(const float4*)(dX + (size_t)row * d + c);
        v[0] += w.x; v[1] += w.y; v[2] += w.z; v[3] += w.w;
      }
    }
    if (dXs) {
      const float4 w = *(const float4*)(dXs + (size_t)t * d + c);
      v[0] += w.x; v[1] += w.y; v[2] += w.z; v[3] += w.w;
    }
    *(float4*)(dx + (size_t)t * d + c) = float4{v[0], v[1], v[2], v[3]};
  }
}

hipError_t launch_dx(int dtype, const float* dr, const void* w_r, int T, int d, int E, int k, const float* dX,
                     const int32_t* row_of, const float* dXs, float* dx, hipStream_t stream) {
  if (T == 0) return hipSuccess;
  dim3 grid((d + 63) / 64, (T + 63) / 64);
  if (dtype == 1)
    hipLaunchKernelGGL(dx_kernel<uint16_t>, grid, dim3(256), 0, stream, dr, (const uint16_t*)w_r, T, d, E, k, dX, row_of,
                       dXs, dx);
  else
    hipLaunchKernelGGL(dx_kernel<float>, grid, dim3(256), 0, stream, dr, (const float*)w_r, T, d, E, k, dX, row_of,
                       dXs, dx);
  return hipGetLastError();
}

}  // namespace moe
