// Router, dispatch (counting sort + capacity + gather) and combine kernels for gfx950.
//
// Router: the linear router, softmax and top-k of the layer (Zero to Frontier §13.1
// "Why MoE", section "The MoE layer"; the routing paragraph of the kevinluzbetak.com
// "Mixture-Of-Experts" page), with logits, softmax and selection in fp32 (the Switch
// router precision remark of AI Engineering Illustrated, "The router is small but it
// decides everything").
//
// Dispatch: the per-expert token lists of the layer as one expert-contiguous list, built
// by a stable counting sort (histogram per chunk of tokens, scan, rank in arrival order),
// with the capacity limit of AI Engineering Illustrated, "The safety valve is a capacity
// limit": an expert keeps its first `cap` assignments in arrival order t*k + j.
#include <algorithm>

#include "common.h"
#include "kernels.h"
#include "router_logits.h"

namespace moe {

// ------------------------------------------------------------------------------ wave scans

__device__ __forceinline__ int wave_excl_scan(int v, int* total) {
  int x = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int y = __shfl_up(x, o, kWave);
    if ((int)(threadIdx.x & 63) >= o) x += y;
  }
  *total = __shfl(x, kWave - 1, kWave);
  return x - v;
}

// The expert-level part of the scan for E <= 64, in one wave (lane e = expert e, cnt and pe
// its totals, zero for e >= E): kept, offsets, tile starts, f, P and aux; returns expert e's
// first row.  aux is summed by the same halving tree as the 1024-wide version, so both give
// the same bits.
__device__ __forceinline__ int scan_finish_wave(int e, int cnt, float pe, bool with_p, int T, int k, int E, int cap,
                                                int32_t* counts, int32_t* kept, int32_t* offsets, float* f,
                                                float* P, float* aux, int bm1, int32_t* tstart1, int bm2,
                                                int32_t* tstart2) {
  const int kp = e < E ? (cap < 0 ? cnt : min(cnt, cap)) : 0;
  int tot, tot1, tot2;
  const int off = wave_excl_scan(kp, &tot);
  const int ts1 = wave_excl_scan((kp + bm1 - 1) / bm1, &tot1);
  const int ts2 = wave_excl_scan((kp + bm2 - 1) / bm2, &tot2);
  if (e < E) {
    if (counts) counts[e] = cnt;
    kept[e] = kp;
    offsets[e] = off;
    tstart1[e] = ts1;
    tstart2[e] = ts2;
  }
  if (e == 0) {
    offsets[E] = tot;
    tstart1[E] = tot1;
    tstart2[E] = tot2;
  }
  if (with_p) {
    const long long R = (long long)T * k;
    const float fe = (e < E && R > 0) ? (float)((double)cnt / (double)R) : 0.f;
    const float Pe = (e < E && T > 0) ? pe / (float)T : 0.f;
    if (e < E) {
      f[e] = fe;
      P[e] = Pe;
    }
    float v = fe * Pe;
#pragma unroll
    for (int h = 32; h > 0; h >>= 1) v += __shfl_down(v, h, kWave);
    if (e == 0) aux[0] = (float)E * v;
  }
  return off;
}

// ------------------------------------------------------------------------------ router
//
// One block = 16 tokens x all E experts, 4 waves.
// Phase 1: logits[16][E] via 16x16 MFMA tiles (A = 16 token rows, B = 16 router rows),
//          operands read straight from global memory (16 B per lane).  Expert tiles are
//          dealt to waves in groups of up to 4; when there are fewer than 4 groups the
//          contraction is split across waves instead, and the partial logits are summed
//          in LDS in a fixed order (bias added last).
// Phase 2: each wave takes 4 tokens: softmax over E (lane l holds experts l + 64 q),
//          k rounds of wave arg-max (ties -> lower index), gates, LDS histogram.
// Phase 3: per-block partial sums of p (fixed order over waves) and histogram to global.

// NQ: 64-expert chunks per lane (E <= 64 NQ), so small expert counts skip empty chunks.
// WAVES = 4: the block computes its logits (phase 1 above).  WAVES = 8 or 16: the logits come
// from the router GEMM's lsplit partial [T, E] arrays (logits_in), and more waves share the 16
// tokens, so each wave's chain of shuffles covers fewer tokens.
template <typename T, int NQ, int WAVES = 4>
__global__ __launch_bounds__(WAVES * 64) void router_kernel(const T* __restrict__ x, const T* __restrict__ w_r,
                                                     const float* __restrict__ b_r, int T_, int d, int E,
                                                     int k, int renorm, int scoring, int n_group,
                                                     int topk_group, int32_t* __restrict__ idx,
                                                     float* __restrict__ gate, float* __restrict__ p_part,
                                                     int32_t* __restrict__ hist,
                                                     const float* __restrict__ logits_in, int lsplit) {
  constexpr int TB = kRouteTokens, NT = WAVES * 64, TPW = TB / WAVES;   // tokens per wave
  static_assert(WAVES == 4 || WAVES == 8 || WAVES == 16, "16 tokens over the waves");
  const int slots = WAVES == 4 ? router_ksplit(E) : 1;
  const bool sigm = scoring == 1;
  extern __shared__ float smem[];
  float* logits = smem;                          // [TB][E]  (partials: [slots][TB][E])
  float* psum = smem + slots * TB * E;           // [WAVES][E]
  float* selrow = psum + WAVES * E;              // [WAVES][E]  selection scores of a wave's token
  int* lhist = (int*)(selrow + WAVES * E);       // [E]

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * TB;
  for (int i = tid; i < E; i += NT) lhist[i] = 0;

  // ---- phase 1: logits (computed here, or read from the GEMM's [T, E] output; the bias is added
  // the same way in both)
  if constexpr (WAVES == 4) {
    router_block_logits<T>(x, w_r, sigm ? nullptr : b_r, T_, d, E, t0, logits, wave, lane, tid);
  } else {
    router_block_logits_from(logits_in, lsplit, T_, E, t0, sigm ? nullptr : b_r, logits, tid, NT);
  }

  // ---- phase 2: scores and top-k, one token per wave at a time
  // Lane l holds experts e = 64 q + l.  sel = the selection score (logit for softmax, affinity
  // plus bias for sigmoid); num = the gate numerator (exp(r - max) or the affinity).
  const int nq = (E + 63) / 64;   // <= NQ
  const int gsz = E / n_group;
  float* srow = selrow + wave * E;
  float pacc[NQ];
#pragma unroll
  for (int q = 0; q < NQ; ++q) pacc[q] = 0.f;
  for (int tt = 0; tt < TPW; ++tt) {
    const int tl = wave * TPW + tt;
    const int t = t0 + tl;
    if (t >= T_) break;
    float v[NQ];
    float m = -INFINITY;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      int e = q * 64 + lane;
      v[q] = (q < nq && e < E) ? logits[tl * E + e] : -INFINITY;
      m = fmaxf(m, v[q]);
    }
    float inv = 1.f;
    float sel[NQ];
    if (!sigm) {
      m = wave_max(m);
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < NQ; ++q) s += (v[q] == -INFINITY) ? 0.f : expf(v[q] - m);
      s = wave_sum(s);
      inv = 1.f / s;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        pacc[q] += (v[q] == -INFINITY) ? 0.f : expf(v[q] - m) * inv;
        sel[q] = v[q] == v[q] ? v[q] : -INFINITY;   // a NaN logit (non-finite input) ranks last
      }
    } else {
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int e = q * 64 + lane;
        const bool ok = v[q] != -INFINITY;
        const float a = ok ? 1.f / (1.f + expf(-v[q])) : 0.f;
        pacc[q] += a;
        const float sv = a + (b_r ? b_r[e] : 0.f);
        sel[q] = ok && sv == sv ? sv : -INFINITY;
      }
    }
    if (n_group > 1) {
      // best selection score per group (lanes < n_group), then the topk_group best groups
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int e = q * 64 + lane;
        if (q < nq && e < E) srow[e] = sel[q];
      }
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      float gbest = -INFINITY;
      if (lane < n_group)
        for (int i = 0; i < gsz; ++i) gbest = fmaxf(gbest, srow[lane * gsz + i]);
      uint64_t allowed = 0;
      for (int r = 0; r < topk_group; ++r) {
        float bv = (lane < n_group && !((allowed >> lane) & 1ull)) ? gbest : -INFINITY;
        int bg = lane < n_group ? lane : 0x7fffffff;
        if ((allowed >> lane) & 1ull) bg = 0x7fffffff;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
          float ov = __shfl_xor(bv, o, kWave);
          int og = __shfl_xor(bg, o, kWave);
          if (ov > bv || (ov == bv && og < bg)) { bv = ov; bg = og; }
        }
        allowed |= 1ull << bg;
      }
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int e = q * 64 + lane;
        if (q < nq && e < E && !((allowed >> (e / gsz)) & 1ull)) sel[q] = -INFINITY;
      }
      __builtin_amdgcn_wave_barrier();       // srow is reused by this wave's next token
    }

    uint32_t taken = 0;
    int my_e = 0;
    float my_num = 0.f, numsum = 0.f;
    for (int j = 0; j < k; ++j) {
      // Each lane's candidate is its best untaken expert, at least its lowest untaken one (so a
      // token whose scores are all -inf still gets a valid index); the reduction ranks by score,
      // then lower index, and the 0x7fffffff of a lane with no untaken expert loses every tie.
      float bv = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int q = 0; q < NQ; ++q) {     // ascending expert index within the lane: '>' keeps the lowest
        int e = q * 64 + lane;
        if (q < nq && e < E && !((taken >> q) & 1u) && (be == 0x7fffffff || sel[q] > bv)) { bv = sel[q]; be = e; }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        float ov = __shfl_xor(bv, o, kWave);
        int oe = __shfl_xor(be, o, kWave);
        if (ov > bv || (ov == bv && oe < be)) { bv = ov; be = oe; }
      }
      if ((be & 63) == lane) taken |= 1u << (be >> 6);
      const float lg = logits[tl * E + be];                       // the chosen expert's logit
      const float num = sigm ? 1.f / (1.f + expf(-lg)) : expf(lg - m);
      numsum += num;
      if (lane == j) { my_e = be; my_num = num; }
    }
    if (lane < k) {
      idx[(size_t)t * k + lane] = my_e;
      gate[(size_t)t * k + lane] = renorm ? my_num / numsum : (sigm ? my_num : my_num * inv);
      atomicAdd(&lhist[my_e], 1);
    }
  }

  // ---- phase 3: block partials
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    int e = q * 64 + lane;
    if (q < nq && e < E) psum[wave * E + e] = pacc[q];
  }
  __syncthreads();
  for (int e = tid; e < E; e += NT) {
    float ps = psum[e];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) ps += psum[w * E + e];   // waves in order
    p_part[(size_t)blockIdx.x * E + e] = ps;
    hist[(size_t)blockIdx.x * E + e] = lhist[e];
  }
}

// Router for E <= EB <= 16 experts (measured: at 64 experts the serial per-thread work costs
// more than router_kernel's wave per token).  Phase 1 as above.  Phase 2 gives each of the block's 16
// tokens one thread, which holds the token's E logits in registers: max, softmax sum (in
// expert order), group limit and the k arg-max passes need no cross-lane exchange.  The
// selection rule is router_kernel's: highest score, ties to the lower index (groups too).
// LDS: the four K-partial slots of the logits, reused after the sum as slot 0 = logits,
// slot 1 = p, slot 2 = selection scores (group limit only), slot 3 = chosen experts.
template <typename T, int EB, bool FUSE>
__global__ __launch_bounds__(256) void router_tpt_kernel(const T* __restrict__ x, const T* __restrict__ w_r,
                                                         const float* __restrict__ b_r, int T_, int d, int E,
                                                         int k, int renorm, int scoring, int n_group,
                                                         int topk_group, int32_t* __restrict__ idx,
                                                         float* __restrict__ gate, float* __restrict__ p_part,
                                                         int32_t* __restrict__ hist, SmallDispatch sd) {
  static_assert(EB <= 64, "E <= 64 keeps router_ksplit(E) == 4, so four logit slots exist");
  constexpr int TB = kRouteTokens;
  const bool sigm = scoring == 1;
  extern __shared__ float smem[];
  float* logits = smem;                                  // [TB][E]
  float* pbuf = smem + TB * E;                           // [TB][E]
  float* sbuf = smem + 2 * TB * E;                       // [TB][E]
  int* cbuf = (int*)(smem + 3 * TB * E);                 // [TB][k]
  int* lhist = (int*)(smem + 4 * TB * E);                // [E]
  int* s_off = lhist + E;                                // [E] (FUSE: each expert's first row)

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * TB;
  const int ntok = min(TB, T_ - t0);
  for (int i = tid; i < E; i += 256) lhist[i] = 0;

  router_block_logits<T>(x, w_r, sigm ? nullptr : b_r, T_, d, E, t0, logits, wave, lane, tid);

  if (tid < ntok) {
    const int t = t0 + tid;
    const float* lrow = logits + tid * E;
    float* prow = pbuf + tid * E;
    float v[EB], sel[EB];
    float m = -INFINITY;
#pragma unroll
    for (int e = 0; e < EB; ++e) {
      v[e] = e < E ? lrow[e] : -INFINITY;
      m = fmaxf(m, v[e]);
    }
    float inv = 1.f;
    if (!sigm) {
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < EB; ++e) s += (v[e] == -INFINITY) ? 0.f : expf(v[e] - m);
      inv = 1.f / s;
#pragma unroll
      for (int e = 0; e < EB; ++e) {
        if (e < E) prow[e] = (v[e] == -INFINITY) ? 0.f : expf(v[e] - m) * inv;
        sel[e] = v[e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < EB; ++e) {
        const bool ok = v[e] != -INFINITY;
        const float a = ok ? 1.f / (1.f + expf(-v[e])) : 0.f;
        if (e < E) prow[e] = a;
        sel[e] = ok ? a + (b_r ? b_r[e] : 0.f) : -INFINITY;
      }
    }
    if (n_group > 1) {
      // best score per group, then the topk_group best groups; the others are masked out
      const int gsz = E / n_group;
      float* srow = sbuf + tid * E;
#pragma unroll
      for (int e = 0; e < EB; ++e)
        if (e < E) srow[e] = sel[e];
      uint64_t allowed = 0;
      for (int r = 0; r < topk_group; ++r) {
        float bv = -INFINITY;
        int bg = -1;
        for (int g = 0; g < n_group; ++g) {
          if ((allowed >> g) & 1ull) continue;
          float gb = -INFINITY;
          for (int i = 0; i < gsz; ++i) gb = fmaxf(gb, srow[g * gsz + i]);
          if (bg < 0 || gb > bv) { bv = gb; bg = g; }
        }
        allowed |= 1ull << bg;
      }
      int g = 0, gi = 0;
#pragma unroll
      for (int e = 0; e < EB; ++e) {
        if (e < E && !((allowed >> g) & 1ull)) sel[e] = -INFINITY;
        if (++gi == gsz) { gi = 0; ++g; }
      }
    }
    // k passes of arg-max over the untaken experts; '>' in ascending order keeps the lowest index
    int* crow = cbuf + tid * k;
    uint64_t taken = 0;
    float numsum = 0.f;
    for (int j = 0; j < k; ++j) {
      float bv = -INFINITY;
      int be = -1;
#pragma unroll
      for (int e = 0; e < EB; ++e)
        if (e < E && !((taken >> e) & 1ull) && (be < 0 || sel[e] > bv)) { bv = sel[e]; be = e; }
      taken |= 1ull << be;
      const float lg = lrow[be];
      numsum += sigm ? 1.f / (1.f + expf(-lg)) : expf(lg - m);
      crow[j] = be;
    }
    for (int j = 0; j < k; ++j) {
      const int be = crow[j];
      const float lg = lrow[be];
      const float num = sigm ? 1.f / (1.f + expf(-lg)) : expf(lg - m);
      idx[(size_t)t * k + j] = be;
      gate[(size_t)t * k + j] = renorm ? num / numsum : (sigm ? num : num * inv);
      atomicAdd(&lhist[be], 1);
    }
  }
  __syncthreads();
  if constexpr (!FUSE) {
    for (int e = tid; e < E; e += 256) {                 // block partial of p, tokens in order
      float ps = 0.f;
      for (int tl = 0; tl < ntok; ++tl) ps += pbuf[tl * E + e];
      p_part[(size_t)blockIdx.x * E + e] = ps;
      hist[(size_t)blockIdx.x * E + e] = lhist[e];
    }
  } else {
    // The whole batch is this block (one chunk of the counting sort, so every chunk base is 0):
    // wave 0 runs the scan's expert pass on the block totals (p summed over tokens in order, as
    // the block partial would be), then each assignment takes its rank among the earlier
    // assignments to the same expert, in arrival order, and its row.
    if (wave == 0) {
      const int e = lane;
      float ps = 0.f;
      if (e < E)
        for (int tl = 0; tl < ntok; ++tl) ps += pbuf[tl * E + e];
      const int off = scan_finish_wave(e, e < E ? lhist[e] : 0, ps, true, T_, k, E, sd.cap, sd.counts, sd.kept,
                                       sd.offsets, sd.f, sd.P, sd.aux, sd.bm1, sd.tstart1, sd.bm2, sd.tstart2);
      if (e < E) s_off[e] = off;
    }
    __syncthreads();
    if (tid < ntok * k) {
      const int e = cbuf[tid];                           // slot tid = token tid / k, choice tid % k
      int r = 0;
      for (int j = 0; j < tid; ++j) r += (cbuf[j] == e);
      const int row = (sd.cap < 0 || r < sd.cap) ? s_off[e] + r : -1;
      sd.row_of[tid] = row;
      if (row >= 0) sd.row_token[row] = tid / k;
    }
  }
}

template <typename T, int EB, bool FUSE = false>
static void router_tpt_launch(int nb, size_t lds, hipStream_t stream, const void* x, const void* w_r,
                              const float* b_r, int T_, int d, int E, int k, int renorm, int scoring, int n_group,
                              int topk_group, int32_t* idx, float* gate, float* p_part, int32_t* hist,
                              const SmallDispatch& sd = SmallDispatch{}) {
  auto kern = router_tpt_kernel<T, EB, FUSE>;
  (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL(kern, dim3(nb), dim3(256), lds, stream, (const T*)x, (const T*)w_r, b_r, T_, d, E, k, renorm,
                     scoring, n_group, topk_group, idx, gate, p_part, hist, sd);
}

hipError_t launch_route_small(int dtype, const void* x, const void* w_r, const float* b_r, int T, int d, int E, int k,
                              int renorm, int scoring, int n_group, int topk_group, int32_t* idx, float* gate,
                              const SmallDispatch& sd, hipStream_t stream) {
  if (!route_small_ok(T, E)) return hipErrorInvalidValue;
  const size_t lds = (size_t)(router_ksplit(E) * kRouteTokens * E + 8 * E) * sizeof(float) + (size_t)E * sizeof(int);
  if (dtype == 1)
    router_tpt_launch<uint16_t, 16, true>(1, lds, stream, x, w_r, b_r, T, d, E, k, renorm, scoring, n_group,
                                          topk_group, idx, gate, nullptr, nullptr, sd);
  else
    router_tpt_launch<float, 16, true>(1, lds, stream, x, w_r, b_r, T, d, E, k, renorm, scoring, n_group, topk_group,
                                       idx, gate, nullptr, nullptr, sd);
  return hipGetLastError();
}

template <typename T, int NQ, int WAVES = 4>
static void router_launch(int nb, hipStream_t stream, const void* x, const void* w_r, const float* b_r,
                          int T_, int d, int E, int k, int renorm, int scoring, int n_group, int topk_group,
                          int32_t* idx, float* gate, float* p_part, int32_t* hist, const float* logits_in,
                          int lsplit) {
  const int slots = WAVES == 4 ? router_ksplit(E) : 1;
  const size_t lds = (size_t)(slots * kRouteTokens * E + 2 * WAVES * E) * sizeof(float) + (size_t)E * sizeof(int);
  auto kern = router_kernel<T, NQ, WAVES>;
  (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL(kern, dim3(nb), dim3(WAVES * 64), lds, stream, (const T*)x, (const T*)w_r, b_r, T_, d, E, k,
                     renorm, scoring, n_group, topk_group, idx, gate, p_part, hist, logits_in, lsplit);
}

template <typename T>
static void router_launch_nq(int nb, hipStream_t stream, const void* x, const void* w_r, const float* b_r, int T_,
                             int d, int E, int k, int renorm, int scoring, int n_group, int topk_group, int32_t* idx,
                             float* gate, float* p_part, int32_t* hist, const float* logits_in, int lsplit) {
  if (logits_in) {              // logits from the GEMM (64 or more experts)
    if (E <= 64)
      router_launch<T, 1, 16>(nb, stream, x, w_r, b_r, T_, d, E, k, renorm, scoring, n_group, topk_group, idx, gate,
                              p_part, hist, logits_in, lsplit);
    else if (E <= 256)
      router_launch<T, 4, 16>(nb, stream, x, w_r, b_r, T_, d, E, k, renorm, scoring, n_group, topk_group, idx, gate,
                              p_part, hist, logits_in, lsplit);
    else if (E <= 512)
      router_launch<T, 16, 16>(nb, stream, x, w_r, b_r, T_, d, E, k, renorm, scoring, n_group, topk_group, idx, gate,
                               p_part, hist, logits_in, lsplit);
    else                        // 8 waves keep the per-wave LDS rows within 160 KB
      router_launch<T, 16, 8>(nb, stream, x, w_r, b_r, T_, d, E, k, renorm, scoring, n_group, topk_group, idx, gate,
                              p_part, hist, logits_in, lsplit);
  } else if (E <= 16) {
    const size_t lds = (size_t)(router_ksplit(E) * kRouteTokens * E + 8 * E) * sizeof(float) + (size_t)E * sizeof(int);
    router_tpt_launch<T, 16>(nb, lds, stream, x, w_r, b_r, T_, d, E, k, renorm, scoring, n_group, topk_group, idx,
                             gate, p_part, hist);
  } else if (E <= 64) {
    router_launch<T, 1>(nb, stream, x, w_r, b_r, T_, d, E, k, renorm, scoring, n_group, topk_group, idx, gate, p_part,
                        hist, nullptr, 1);
  } else if (E <= 256) {
    router_launch<T, 4>(nb, stream, x, w_r, b_r, T_, d, E, k, renorm, scoring, n_group, topk_group, idx, gate, p_part,
                        hist, nullptr, 1);
  } else {
    router_launch<T, 16>(nb, stream, x, w_r, b_r, T_, d, E, k, renorm, scoring, n_group, topk_group, idx, gate, p_part,
                         hist, nullptr, 1);
  }
}

hipError_t launch_router(int dtype, const void* x, const void* w_r, const float* b_r, int T, int d, int E,
                         int k, int renorm, int scoring, int n_group, int topk_group, int32_t* idx, float* gate,
                         float* p_part, int32_t* hist, float* logits, hipStream_t stream) {
  const int nb = route_blocks(T);
  const float* logits_in = nullptr;
  if (router_logits_by_gemm(E)) {
    if (!logits) return hipErrorInvalidValue;
    const hipError_t e = launch_gemm_router(dtype, x, w_r, T, d, E, logits, stream);
    if (e != hipSuccess) return e;
    logits_in = logits;
  }
  const int lsplit = router_gemm_ksplit(d);
  if (dtype == 1)
    router_launch_nq<uint16_t>(nb, stream, x, w_r, b_r, T, d, E, k, renorm, scoring, n_group, topk_group, idx, gate,
                               p_part, hist, logits_in, lsplit);
  else
    router_launch_nq<float>(nb, stream, x, w_r, b_r, T, d, E, k, renorm, scoring, n_group, topk_group, idx, gate,
                            p_part, hist, logits_in, lsplit);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ histogram

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ idx, int T, int k, int E,
                                                   int32_t* __restrict__ hist) {
  extern __shared__ int lh[];
  for (int i = threadIdx.x; i < E; i += 256) lh[i] = 0;
  __syncthreads();
  const int t0 = blockIdx.x * kRouteTokens;
  const int n = min(kRouteTokens, T - t0) * k;
  for (int i = threadIdx.x; i < n; i += 256) atomicAdd(&lh[idx[(size_t)t0 * k + i]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) hist[(size_t)blockIdx.x * E + e] = lh[e];
}

hipError_t launch_hist(const int32_t* idx, int T, int k, int E, int32_t* hist, hipStream_t stream) {
  hipLaunchKernelGGL(hist_kernel, dim3(route_blocks(T)), dim3(256), (size_t)E * sizeof(int), stream, idx, T,
                     k, E, hist);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ scan (1 block)
//
// Per-chunk bases by expert: chunk_base[b][e] = assignments to e in chunks < b;
// counts[e] = all of them.  The chunks are cut into G <= 1024 / E contiguous groups of
// about kScanBatch chunks, so most threads work and each reads its group in one batch of
// loads: thread (g, e) sums its group's chunks, a serial pass over the G group sums per
// expert turns them into group bases, and each thread then writes its chunks' bases.
// kept = min(counts, cap); offsets and tile starts are exclusive scans over experts.
// f, P, aux use fixed-order sums.
constexpr int kScanBatch = 16;

__global__ __launch_bounds__(1024) void scan_kernel(const int32_t* __restrict__ hist,
                                                    const float* __restrict__ p_part, int nb, int T, int k,
                                                    int E, int cap, int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ kept, int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ chunk_base, float* __restrict__ f,
                                                    float* __restrict__ P, float* __restrict__ aux, int bm1,
                                                    int32_t* __restrict__ tstart1, int bm2,
                                                    int32_t* __restrict__ tstart2) {
  __shared__ int s_scan[1024];
  __shared__ int s_part[1024];
  __shared__ float s_red[1024];
  const int tid = threadIdx.x;
  const int G = max(1, min(1024 / E, (nb + kScanBatch - 1) / kScanBatch));
  const int ge = tid / E, ee = tid - ge * E;              // group and expert of this thread
  const bool act = ge < G;
  const int b0 = act ? (int)((long long)ge * nb / G) : 0, b1 = act ? (int)((long long)(ge + 1) * nb / G) : 0;
  // group sums, loads batched so kScanBatch of them are in flight; p summed in chunk order
  int c = 0;
  float ps = 0.f;
  for (int bb = b0; bb < b1; bb += kScanBatch) {
    int h[kScanBatch];
    float q[kScanBatch];
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      const bool ok = bb + u < b1;
      h[u] = ok ? hist[(size_t)(bb + u) * E + ee] : 0;
      q[u] = (ok && p_part) ? p_part[(size_t)(bb + u) * E + ee] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kScanBatch; ++u) {
      c += h[u];
      if (bb + u < b1) ps += q[u];
    }
  }
  s_part[tid] = c;
  s_red[tid] = ps;
  __syncthreads();
  int cnt = 0;
  float pe = 0.f;
  if (tid < E) {                                          // group bases and totals per expert
    for (int g = 0; g < G; ++g) {
      const int v = s_part[g * E + tid];
      s_part[g * E + tid] = cnt;
      cnt += v;
      pe += s_red[g * E + tid];
    }
  }
  __syncthreads();
  if (act) {
    int run = s_part[tid];
    for (int bb = b0; bb < b1; bb += kScanBatch) {
      int h[kScanBatch];
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u) h[u] = bb + u < b1 ? hist[(size_t)(bb + u) * E + ee] : 0;
#pragma unroll
      for (int u = 0; u < kScanBatch; ++u)
        if (bb + u < b1) {
          chunk_base[(size_t)(bb + u) * E + ee] = run;
          run += h[u];
        }
    }
  }
  if (E <= kWave) {                                       // block-uniform
    if (tid < kWave)
      scan_finish_wave(tid, cnt, pe, p_part != nullptr, T, k, E, cap, counts, kept, offsets, f, P, aux, bm1,
                       tstart1, bm2, tstart2);
    return;
  }
  const int e = tid;
  const int kp = e < E ? (cap < 0 ? cnt : min(cnt, cap)) : 0;
  int tot;
  const int off = block1024_exclusive_scan(kp, s_scan, &tot);
  const int nt1 = (kp + bm1 - 1) / bm1, nt2 = (kp + bm2 - 1) / bm2;
  int tot1, tot2;
  const int ts1 = block1024_exclusive_scan(nt1, s_scan, &tot1);
  const int ts2 = block1024_exclusive_scan(nt2, s_scan, &tot2);
  if (e < E) {
    if (counts) counts[e] = cnt;
    kept[e] = kp;
    offsets[e] = off;
    tstart1[e] = ts1;
    tstart2[e] = ts2;
  }
  if (e == 0) {
    offsets[E] = tot;
    tstart1[E] = tot1;
    tstart2[E] = tot2;
  }
  if (p_part) {
    const long long R = (long long)T * k;
    float fe = (e < E && R > 0) ? (float)((double)cnt / (double)R) : 0.f;
    float Pe = (e < E && T > 0) ? pe / (float)T : 0.f;
    if (e < E) {
      f[e] = fe;
      P[e] = Pe;
    }
    __syncthreads();
    s_red[e] = fe * Pe;
    __syncthreads();
    for (int h = 512; h > 0; h >>= 1) {
      if (e < h) s_red[e] += s_red[e + h];
      __syncthreads();
    }
    if (e == 0) aux[0] = (float)E * s_red[0];
  }
}

// The same scan for few experts and few chunks (decode): one wave, lane e = expert e, chunks
// summed in order.  With nb <= kScanBatch scan_kernel has a single group and sums in the
// same order, so both give the same bits.
__global__ __launch_bounds__(64) void scan_small_kernel(const int32_t* __restrict__ hist,
                                                        const float* __restrict__ p_part, int nb, int T, int k,
                                                        int E, int cap, int32_t* __restrict__ counts,
                                                        int32_t* __restrict__ kept, int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ chunk_base, float* __restrict__ f,
                                                        float* __restrict__ P, float* __restrict__ aux, int bm1,
                                                        int32_t* __restrict__ tstart1, int bm2,
                                                        int32_t* __restrict__ tstart2) {
  const int e = threadIdx.x;
  int cnt = 0;
  float pe = 0.f;
  if (e < E) {
    for (int b = 0; b < nb; ++b) {
      chunk_base[(size_t)b * E + e] = cnt;
      cnt += hist[(size_t)b * E + e];
      if (p_part) pe += p_part[(size_t)b * E + e];
    }
  }
  scan_finish_wave(e, cnt, pe, p_part != nullptr, T, k, E, cap, counts, kept, offsets, f, P, aux, bm1, tstart1, bm2,
                   tstart2);
}

hipError_t launch_scan(const int32_t* hist, const float* p_part, int nb, int T, int k, int E, int cap,
                       int32_t* counts, int32_t* kept, int32_t* offsets, int32_t* chunk_base, float* f,
                       float* P, float* aux, int bm1, int32_t* tstart1, int bm2, int32_t* tstart2,
                       hipStream_t stream) {
  if (E <= kWave && nb <= kScanBatch)
    hipLaunchKernelGGL(scan_small_kernel, dim3(1), dim3(kWave), 0, stream, hist, p_part, nb, T, k, E, cap, counts,
                       kept, offsets, chunk_base, f, P, aux, bm1, tstart1, bm2, tstart2);
  else
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, stream, hist, p_part, nb, T, k, E, cap, counts, kept,
                       offsets, chunk_base, f, P, aux, bm1, tstart1, bm2, tstart2);
  return hipGetLastError();
}

__global__ __launch_bounds__(1024) void tile_sched_kernel(const int32_t* __restrict__ offsets, int E, int bm1,
                                                          int32_t* __restrict__ tstart1, int bm2,
                                                          int32_t* __restrict__ tstart2) {
  __shared__ int s_scan[1024];
  const int e = threadIdx.x;
  const int rows = e < E ? offsets[e + 1] - offsets[e] : 0;
  int tot1, tot2;
  const int ts1 = block1024_exclusive_scan((rows + bm1 - 1) / bm1, s_scan, &tot1);
  const int ts2 = block1024_exclusive_scan((rows + bm2 - 1) / bm2, s_scan, &tot2);
  if (e < E) {
    tstart1[e] = ts1;
    tstart2[e] = ts2;
  }
  if (e == 0) {
    tstart1[E] = tot1;
    tstart2[E] = tot2;
  }
}

hipError_t launch_tile_sched(const int32_t* offsets, int E, int bm1, int32_t* tstart1, int bm2, int32_t* tstart2,
                             hipStream_t stream) {
  hipLaunchKernelGGL(tile_sched_kernel, dim3(1), dim3(1024), 0, stream, offsets, E, bm1, tstart1, bm2, tstart2);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ rank + gather
//
// One block per chunk of 16 tokens (<= 256 assignments).  The rank of assignment i
// within its expert is the chunk's base for that expert plus the number of earlier
// assignments in the chunk with the same expert (stable, arrival order).  Kept
// assignments then copy their token row into x_perm with 16-byte loads and stores.
template <typename T, bool COPY>
__global__ __launch_bounds__(256) void rank_gather_kernel(const T* __restrict__ x, const int32_t* __restrict__ idx,
                                                          int T_, int d, int k, int E, int cap,
                                                          const int32_t* __restrict__ chunk_base,
                                                          const int32_t* __restrict__ offsets,
                                                          int32_t* __restrict__ row_token,
                                                          int32_t* __restrict__ row_of, T* __restrict__ x_perm) {
  __shared__ int s_e[256];
  __shared__ int s_row[256];
  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * kRouteTokens;
  const int n = min(kRouteTokens, T_ - t0) * k;
  if (tid < n) s_e[tid] = idx[(size_t)t0 * k + tid];   // the other splits redo this small rank
  __syncthreads();
  if (tid < n) {
    const int e = s_e[tid];
    int r = 0;
    for (int j = 0; j < tid; ++j) r += (s_e[j] == e);
    const int g = chunk_base[(size_t)blockIdx.x * E + e] + r;
    const int row = (cap < 0 || g < cap) ? offsets[e] + g : -1;
    s_row[tid] = row;
    if (blockIdx.y == 0) {                       // one split writes the index outputs
      row_of[(size_t)t0 * k + tid] = row;
      if (row >= 0) row_token[row] = t0 + tid / k;
    }
  }
  if constexpr (!COPY) return;                 // indices only; the GEMM gathers rows itself
  __syncthreads();
  const int P = (int)((size_t)d * sizeof(T) / 16);   // 16-byte pieces per row
  // the copy of this chunk is shared by gridDim.y blocks (more blocks for small batches)
  const int total_all = n * P;
  const int lo = (int)((long long)total_all * blockIdx.y / gridDim.y);
  const int total = (int)((long long)total_all * (blockIdx.y + 1) / gridDim.y);
  // The U loads of an iteration are unconditional, so they are all in flight together (a load
  // under a condition waits for the ones before it): a piece past the end re-reads the last
  // one, and a dropped token's piece is read too, and neither is stored.
  constexpr int U = 4;
  if (total <= lo) return;
  for (int base = lo + tid; base < total; base += 256 * U) {
    u32x4_t v[U];
    long long dst[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int it = min(base + u * 256, total - 1);
      const int item = it / P, piece = it - item * P;
      const int t = t0 + item / k;
      v[u] = *((const u32x4_t*)((const char*)x + (size_t)t * d * sizeof(T)) + piece);
      const int row = s_row[item];
      dst[u] = base + u * 256 < total && row >= 0 ? (long long)row * P + piece : -1;   // 16-byte units
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (dst[u] >= 0) ((u32x4_t*)x_perm)[dst[u]] = v[u];
  }
}

hipError_t launch_rank_gather(int dtype, const void* x, const int32_t* idx, int T, int d, int k, int E, int cap,
                              const int32_t* chunk_base, const int32_t* offsets, int32_t* row_token,
                              int32_t* row_of, void* x_perm, hipStream_t stream) {
  const int nb = route_blocks(T);
  const int splits = x_perm ? std::max(1, std::min(16, 512 / nb)) : 1;
  const dim3 grid(nb, splits);
  auto launch = [&](auto kern, auto* xt) {
    using E_ = std::remove_const_t<std::remove_pointer_t<decltype(xt)>>;
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, xt, idx, T, d, k, E, cap, chunk_base, offsets, row_token,
                       row_of, (E_*)x_perm);
  };
  if (dtype == 1) {
    if (x_perm) launch(rank_gather_kernel<uint16_t, true>, (const uint16_t*)x);
    else launch(rank_gather_kernel<uint16_t, false>, (const uint16_t*)x);
  } else {
    if (x_perm) launch(rank_gather_kernel<float, true>, (const float*)x);
    else launch(rank_gather_kernel<float, false>, (const float*)x);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ combine
//
// The layer's gate-weighted sum back in token order (Zero to Frontier §13.1, "The MoE
// layer" equation), accumulated as: shared (or 0), then slot 0, 1, ..., k-1 with one
// fused multiply-add each.  A dropped slot (row -1) adds nothing.  When the down product
// ran in nsplit K chunks, a row's output is the sum of its partials, taken in chunk order
// (fixed, so the result does not depend on scheduling).
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o, const int32_t* __restrict__ row_of,
                                                      const float* __restrict__ gate,
                                                      const float* __restrict__ shared, float* __restrict__ y,
                                                      int T, int d, int k, int nsplit, size_t split_stride) {
  __shared__ int s_row[16];
  __shared__ float s_g[16];
  const int d4 = d / 4, nch = (d4 + 255) / 256;   // blocks per token: 1024 columns each
  const int t = blockIdx.x / nch;
  if (threadIdx.x < k) {
    s_row[threadIdx.x] = row_of[(size_t)t * k + threadIdx.x];
    s_g[threadIdx.x] = gate[(size_t)t * k + threadIdx.x];
  }
  __syncthreads();
  const size_t ss4 = split_stride / 4;
  const int c = (blockIdx.x % nch) * 256 + threadIdx.x;
  if (c < d4) {
    f32x4_t acc = shared ? ((const f32x4_t*)shared)[(size_t)t * d4 + c] : f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
      const int row = s_row[j];
      if (row >= 0) {
        const f32x4_t* src = (const f32x4_t*)o + (size_t)row * d4 + c;
        f32x4_t v = src[0];
        for (int p = 1; p < nsplit; ++p) {
          const f32x4_t w = src[p * ss4];
          v[0] += w[0];
          v[1] += w[1];
          v[2] += w[2];
          v[3] += w[3];
        }
        const float g = s_g[j];
        acc[0] = fmaf(g, v[0], acc[0]);
        acc[1] = fmaf(g, v[1], acc[1]);
        acc[2] = fmaf(g, v[2], acc[2]);
        acc[3] = fmaf(g, v[3], acc[3]);
      }
    }
    ((f32x4_t*)y)[(size_t)t * d4 + c] = acc;
  }
}

hipError_t launch_combine(const float* o, const int32_t* row_of, const float* gate, const float* shared, float* y,
                          int T, int d, int k, int nsplit, size_t split_stride, hipStream_t stream) {
  if (nsplit < 1 || (nsplit > 1 && split_stride % 4 != 0)) return hipErrorInvalidValue;
  const long long blocks = (long long)T * ((d / 4 + 255) / 256);
  if (blocks >= (1LL << 31)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, o, row_of, gate, shared, y, T, d,
                     k, nsplit, split_stride);
  return hipGetLastError();
}

}  // namespace moe
