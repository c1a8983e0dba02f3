// Pieces shared by the grouped-GEMM kernels (internal to the library).
#pragma once

#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace moe {

struct GemmArgs {
  const void* A;            // [rows, K] activations in expert order, or token rows (a_rows)
  const int32_t* a_rows;    // NULL, or row of A for each expert-ordered row (gather in the load)
  const void* B0;           // [G, N, K] gate (gated) or down weights
  const void* B1;           // [G, N, K] up weights (gated only)
  const float* S0;          // scales of B0: FP8 [G, N] fp32 per row; MXFP4 [G, K/32, N] E8M0 bytes
  const float* S1;          // scales of B1 (gated), same layout
  const int32_t* offsets;   // [G+1] or NULL (dense: one group of dense_rows)
  const int32_t* tstart;    // [G+1] first m-tile of each group (unused when dense)
  int G, dense_rows, N, K;
  void* C;                  // [rows, N]  (dtype for gated, fp32 for down)
  int ksplit = 1;           // K chunks (plain product only): chunk c covers K steps
                            // [c K/ksplit, (c+1) K/ksplit) and writes C + c * split_stride
  size_t split_stride = 0;  // floats between the partial outputs of consecutive chunks
  // K-grouped products: group g covers K columns [koffsets[g], koffsets[g+1]) of A
  // [dense_rows, K] and B0 [N, K] and writes C + g * dense_rows * N
  const int32_t* koffsets = nullptr;
  // backward epilogues (see store_save_ab / store_dgrad)
  float* ep_a = nullptr;             // [rows, N] fp32 gate pre-activations (written, or read)
  float* ep_b = nullptr;             // [rows, N] fp32 up pre-activations
  const float* ep_g = nullptr;       // [rows] gate of each row (NULL: 1)
  void* ep_t = nullptr;              // transposed output, leading dimension ep_ldt
  float* ep_part = nullptr;          // [rows, ep_npart] partial row dots (or NULL)
  const int32_t* ep_poff = nullptr;  // [G+1] column of each group's first row in ep_t (NULL: row)
  int ep_ldt = 0, ep_npart = 0;
  // dense products only: number tiles n-tile-minor (all n-tiles of an m-tile consecutive, so one
  // XCD reads each activation row once; for few n-tiles and B small enough to stay in L2)
  int dense_n_minor = 0;
  // MXFP8 activations (grouped_gemm_mx.hip): E8M0 scales of A [rows of A, K/32] (gathered through
  // a_rows like A), and of the gated product's MXFP8 output h [rows, N/32] (C then holds E4M3 codes)
  const uint8_t* a_scales = nullptr;
  uint8_t* c_scales = nullptr;
  // Work counters of a dynamically scheduled product (kNumXcd ints, zero at launch), or NULL for
  // the static walk.  Dynamic: a block's first tile is its static one; after that each block
  // takes the next tile of its XCD's range from its XCD's counter, so blocks that drew cheap
  // tiles (an expert's last, partly empty m-tile) take more of them.
  int32_t* tile_ctr = nullptr;
};

// Word 3 of a raw buffer resource on gfx9-family parts (32-bit data format, no swizzle).
constexpr int kBufFlags = 0x00020000;
// Range of every buffer resource: the whole unsigned 32-bit offset space.  The offsets are
// 32-bit byte offsets from the resource base (a gathered token row of x sits at up to
// T*d*elem bytes past it, which the host keeps below 2^32); a smaller range would turn loads
// past it into zeros without an error.
constexpr int kBufRange = static_cast<int>(0xFFFFFFFFu);

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for the LDS ring.  __syncthreads() would also wait for every
// outstanding global load (its release fence), which would drain the ring; here each
// wave has already waited for the loads it needs (vmcnt) and for its own LDS reads
// (lgkmcnt), so a bare s_barrier is enough.  The empty asm statements keep the
// compiler from moving memory operations across it.
__device__ __forceinline__ void block_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 64-byte LDS rows: 4 pieces of 16 bytes, XOR-swizzled by row pair (conflict-free
// 16-byte reads of one piece by 16 consecutive rows).
__device__ __forceinline__ int swz64(int r, int c) { return r * 64 + ((c ^ ((r >> 1) & 3)) << 4); }

// Largest g in [0, G) with tstart[g] <= mq, for nondecreasing tstart with tstart[0] = 0 <= mq
// (empty groups repeat their successor's start, so g is the group holding m-tile mq).  A
// 64-way search: each round every lane reads one candidate and a ballot picks the last one
// not past mq, so up to 64 groups take one round of dependent loads and up to 4,096 two (a
// binary search takes log2 G).  Every lane of the wave must be active.
__device__ __forceinline__ int find_group(const int32_t* __restrict__ tstart, int G, int mq) {
  const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  int base = 0, span = G;                              // the answer lies in [base, base + span)
  while (span > 1) {
    const int step = (span + kWave - 1) / kWave;       // candidates base, base + step, ...
    const int idx = base + lane * step;
    const bool ok = idx < base + span && tstart[idx] <= mq;
    const unsigned long long m = __ballot(ok);         // a prefix of the lanes; lane 0 is set
    const int end = base + span;
    base += (63 - __builtin_clzll(m)) * step;
    span = min(step, end - base);
  }
  return base;
}

struct TileCoord {
  int g, nt, row0, rows;   // group (expert), n-tile, first row, valid rows (<= BM)
};

// Tile order: group by group (expert), and inside a group in super-tiles of all its
// m-tiles x GN n-tiles, GN chosen so one super-tile is about one XCD's worth of
// concurrent blocks.  Blocks that run together then share their weight tile (same
// n-tile, all m-tiles of the group: weights leave HBM once) and their activation
// rows (same m-tile, neighbouring n-tiles) in the XCD's L2.
__device__ __forceinline__ TileCoord tile_coord(const GemmArgs& args, int L, int ntn, int mt_live, int bpx, int BM) {
  const int32_t* __restrict__ offsets = args.offsets;
  const int32_t* __restrict__ tstart = args.tstart;
  if (!offsets && args.dense_n_minor) {
    TileCoord tc;
    tc.g = 0;
    tc.nt = L % ntn;
    tc.row0 = (L / ntn) * BM;
    tc.rows = min(BM, args.dense_rows - tc.row0);
    return tc;
  }
  const int mq = L / ntn;                              // any m-tile index in L's group range
  int g = 0, t0g = 0, t1g = mt_live;
  if (offsets) {
    g = find_group(tstart, args.G, mq);
    t0g = tstart[g];
    t1g = tstart[g + 1];
  }
  const int Me = t1g - t0g;                            // m-tiles of this group
  const int l = L - t0g * ntn;
  const int GN = max(1, bpx / Me);
  const int full = ntn / GN;
  int m, nt;
  if (l < full * Me * GN) {
    const int sb = l / (Me * GN), w = l - sb * (Me * GN);
    m = w % Me;
    nt = sb * GN + w / Me;
  } else {
    const int w = l - full * Me * GN;
    m = w % Me;
    nt = full * GN + w / Me;
  }
  TileCoord tc;
  tc.g = g;
  tc.nt = nt;
  if (offsets) {
    tc.row0 = offsets[g] + m * BM;
    tc.rows = min(BM, offsets[g + 1] - tc.row0);
  } else {
    tc.row0 = m * BM;
    tc.rows = min(BM, args.dense_rows - tc.row0);
  }
  return tc;
}

// Epilogue: lane holds rows 4*(lane/16)+q of each 16x16 tile, column lane%16.  The gated
// product stores SiLU(a) * b in the activation type, the plain one fp32.  Row addresses are
// formed once per (subtile row, q); the row test is per row, not per element.
template <typename Cfg, typename Acc>
__device__ __forceinline__ void store_tile(const GemmArgs& args, const Acc& acc0, const Acc& acc1, int wm, int wn,
                                           int lane, int g, int nt, int row0, int rows, size_t c_off = 0) {
  using T = typename Cfg::Elem;
  const int N = args.N;
  const int c0 = nt * Cfg::BN_ + wn * Cfg::WTN + (lane & 15);
  // FP8 row scales of the lane's columns, loaded once: interleaved with the stores below, each
  // load would wait for the one before (the compiler cannot tell them apart from the stores)
  float s0[Cfg::WF_ == 1 ? Cfg::TN : 1], s1[Cfg::WF_ == 1 && Cfg::NB == 2 ? Cfg::TN : 1];
  if constexpr (Cfg::WF_ == 1) {
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) {
      s0[j] = args.S0[(size_t)g * N + c0 + j * 16];
      if constexpr (Cfg::NB == 2) s1[j] = args.S1[(size_t)g * N + c0 + j * 16];
    }
  }
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = wm * Cfg::WTM + i * 16 + (lane >> 4) * 4 + q;
      if (r >= rows) continue;
      const size_t o = (size_t)(row0 + r) * N + c0;
#pragma unroll
      for (int j = 0; j < Cfg::TN; ++j) {
        if constexpr (Cfg::WF_ == 1) {                   // row scales of FP8 weights
          if constexpr (Cfg::NB == 2) {
            const float h = silu_mul(acc0[i][j][q] * s0[j], acc1[i][j][q] * s1[j]);
            ((T*)args.C)[o + j * 16] = ElemOut<T>::from_f32(h);
          } else {
            ((float*)args.C)[c_off + o + j * 16] = acc0[i][j][q] * s0[j];
          }
        } else if constexpr (Cfg::NB == 2) {
          ((T*)args.C)[o + j * 16] = ElemOut<T>::from_f32(silu_mul(acc0[i][j][q], acc1[i][j][q]));
        } else {
          ((float*)args.C)[c_off + o + j * 16] = acc0[i][j][q];
        }
      }
    }
}

// Four consecutive values of T as one 8-byte (bf16) or 16-byte (fp32) store.
template <typename T>
__device__ __forceinline__ void store4(T* p, const float* v) {
  if constexpr (sizeof(T) == 2) {
    *(uint2*)p = uint2{f32x2_to_bf16x2_bits(v[0], v[1]), f32x2_to_bf16x2_bits(v[2], v[3])};
  } else {
    *(float4*)p = float4{v[0], v[1], v[2], v[3]};
  }
}

// Column of row `row` (of group g) in a transposed backward operand: groups start on
// 64-aligned columns so each group's K range is whole K steps; the gaps hold zeros.
__device__ __forceinline__ int tcol(const GemmArgs& args, int g, int row) {
  return args.ep_poff ? args.ep_poff[g] + (row - args.offsets[g]) : row;
}

// Backward recompute of the gate/up product: stores the pre-activations a, b (fp32,
// row-major) and h = SiLU(a) * b -- rounded exactly as the forward rounds it -- transposed
// into ep_t [N, ldt].  A lane's 4 rows are 4 consecutive columns of ep_t (one store; the
// first is a multiple of 4 because tiles and groups start on multiples of 4 rows).
template <typename Cfg, typename Acc>
__device__ __forceinline__ void store_save_ab(const GemmArgs& args, const Acc& acc0, const Acc& acc1, int wm,
                                              int wn, int lane, int g, int nt, int row0, int rows) {
  using T = typename Cfg::Elem;
  const int N = args.N;
  const size_t ldt = (size_t)args.ep_ldt;
#pragma unroll
  for (int i = 0; i < Cfg::TM; ++i) {
    const int rl = wm * Cfg::WTM + i * 16 + (lane >> 4) * 4;     // first of the lane's 4 rows
    if (rl >= rows) continue;
    const int p0 = tcol(args, g, row0 + rl);
#pragma unroll
    for (int j = 0; j < Cfg::TN; ++j) {
      const int col = nt * Cfg::BN_ + wn * Cfg::WTN + j * 16 + (lane & 15);
      T* ht = (T*)args.ep_t + (size_t)col * ldt + p0;
      float h[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float a = acc0[i][j][q], b = acc1[i][j][q];
        h[q] = silu_mul(a, b);
        if (rl + q < rows) {
          const size_t o = (size_t)(row0 + rl + q) * N + col;
          args.ep_a[o] = a;
          args.ep_b[o] = b;
        }
      }
      if (rl + 3 < rows) {
        store4<T>(ht, h);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (rl + q < rows) ht[q] = ElemOut<T>::from_f32(h[q]);
      }
    }
  }
}

// Backward of the down product, per element of u = dy_row W_d (the accumulator): with the
// row's gate gr, dh = gr u; h = SiLU(a) b as the forward rounded it; s = sigmoid(a);
// dA = dh b s (1 + a (1 - s)), dB = dh SiLU(a).  dA, dB go to C [rows, 2N] (dA in columns
// [0, N), dB in [N, 2N)) and transposed to ep_t [2N, ldt]; the row dot sum_n h u over the
// wave's columns goes to ep_part (dL/dg of the row is the sum over the row's parts).
template <typename Cfg, typename Acc>
__device__ __forceinline__ void store_dgrad(const GemmArgs& args, const Acc& acc0, int wm, int wn, int lane, int g,
                                            int nt, int row0, int rows) {
  using T = typename Cfg::Elem;
  const int N = args.N;
  const size_t ldt = (size_t)args.ep_ldt;
  T* dab = (T*)args.C;
  T* dabt = (T*)args.ep_t;
  static_for<0, Cfg::TM>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    const int rl = wm * Cfg::WTM + i * 16 + (lane >> 4) * 4;
    float part[4] = {0.f, 0.f, 0.f, 0.f};
    if (rl < rows) {
      const int p0 = tcol(args, g, row0 + rl);
      float gr[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) gr[q] = rl + q < rows && args.ep_g ? args.ep_g[row0 + rl + q] : 1.f;
      // Every a and b of the subtile row is loaded before the first store: the compiler cannot
      // tell the stores below from these loads, and interleaved it waits for each load in turn.
      float av[Cfg::TN][4], bv[Cfg::TN][4];
      static_for<0, Cfg::TN>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        const int col = nt * Cfg::BN_ + wn * Cfg::WTN + j * 16 + (lane & 15);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const size_t o = (size_t)(row0 + rl + q) * N + col;
          av[j][q] = rl + q < rows ? args.ep_a[o] : 0.f;
          bv[j][q] = rl + q < rows ? args.ep_b[o] : 0.f;
        }
      });
      static_for<0, Cfg::TN>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        const int col = nt * Cfg::BN_ + wn * Cfg::WTN + j * 16 + (lane & 15);
        float da[4] = {0.f, 0.f, 0.f, 0.f}, db[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (rl + q < rows) {
            const int row = row0 + rl + q;
            const float a = av[j][q], b = bv[j][q], u = acc0[i][j][q];
            const float sg = sigmoid_fast(a);
            const float silu = a * sg;
            const float h = ElemOut<T>::to_f32(ElemOut<T>::from_f32(silu_mul(a, b)));
            part[q] = fmaf(h, u, part[q]);
            const float dh = gr[q] * u;
            da[q] = dh * b * sg * (1.f + a * (1.f - sg));
            db[q] = dh * silu;
            dab[(size_t)row * 2 * N + col] = ElemOut<T>::from_f32(da[q]);
            dab[(size_t)row * 2 * N + N + col] = ElemOut<T>::from_f32(db[q]);
          }
        }
        T* ta = dabt + (size_t)col * ldt + p0;
        T* tb = dabt + (size_t)(N + col) * ldt + p0;
        if (rl + 3 < rows) {
          store4<T>(ta, da);
          store4<T>(tb, db);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (rl + q < rows) {
              ta[q] = ElemOut<T>::from_f32(da[q]);
              tb[q] = ElemOut<T>::from_f32(db[q]);
            }
        }
      });
    }
    if (args.ep_part) {
      // sum over the 16 columns held by one lane group (the group's 16 lanes share rl, so
      // they are active or inactive together)
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) part[q] += __shfl_xor(part[q], o, kWave);
      if ((lane & 15) == 0) {
        const int slot = (nt * Cfg::BN_ + wn * Cfg::WTN) / Cfg::WTN;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (rl + q < rows) args.ep_part[(size_t)(row0 + rl + q) * args.ep_npart + slot] = part[q];
      }
    }
  });
}

// Persistent grid: #CUs x occupancy blocks (at most one per tile), a multiple of the XCD count.
template <typename Cfg, void (*KERN)(GemmArgs)>
static hipError_t launch_kernel(const GemmArgs& a, int max_tiles_m, hipStream_t stream) {
  static const int occ = [] {
    (void)hipFuncSetAttribute((const void*)KERN, hipFuncAttributeMaxDynamicSharedMemorySize, Cfg::LDS_ALLOC);
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, KERN, Cfg::NT, Cfg::LDS_ALLOC) != hipSuccess || n < 1) n = 1;
    return n;
  }();
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    return hipErrorInvalidDevice;
  const long long max_live = (long long)max_tiles_m * (a.N / Cfg::BN_) * std::max(1, a.ksplit);
  long long grid = std::min<long long>(max_live, (long long)cus * occ);
  grid = ((grid + kNumXcd - 1) / kNumXcd) * kNumXcd;
  if (grid < kNumXcd) grid = kNumXcd;
  hipLaunchKernelGGL(KERN, dim3((unsigned)grid), dim3(Cfg::NT), Cfg::LDS_ALLOC, stream, a);
  return hipGetLastError();
}

// Rows per tile of the bf16 down projection with many rows per expert (the other large
// tiles take 256).
constexpr int kLargeBf16BlockM = 192;

}  // namespace moe
