// bf16 down projection for many rows per expert (the MFMA-bound regime).
//
// 192-row tiles x 256 weight rows (128 when N is not a multiple of 256), 4 waves of
// 96 x 128, K in 64-byte steps through a ring of 4 LDS slots.  LDS read bandwidth (128
// bytes per clock per CU) bounds the 8-wave template in grouped_gemm.hip, whose 64 x 128
// wave tile reads 0.375 KB of LDS per MFMA; the 96 x 128 wave tile reads 0.29 KB.  With
// one wave per SIMD the latency hiding is explicit: step s's operands sit in registers
// while step s+1's are read from LDS, and global -> LDS loads run PF steps ahead.
// Accumulators live in VGPRs and operands in AGPRs (this file is compiled with MFMA
// VGPR form), which keeps every MFMA accumulating in place.  The gated product keeps the
// 8-wave kernel: its shorter K and two-output epilogue favour eight waves.
#include "gemm_common.h"

namespace moe {


template <typename T, int BN, bool GATED>
struct LargeTile {
  using Elem = T;
  static constexpr int WF_ = 0;
  static constexpr int NT = 256, WM = 2, WN = 2;
  static constexpr int BM_ = kLargeBf16BlockM, BN_ = BN, NB = GATED ? 2 : 1, BROWS = BN * NB;
  static constexpr int WTM = BM_ / WM, WTN = BN / WN;
  static constexpr int TM = WTM / 16, TN = WTN / 16, TNB = TN * NB;
  static constexpr int A_SLOT = BM_ * 64, B_SLOT = BROWS * 64, SLOT = A_SLOT + B_SLOT;
  static constexpr int NSLOT = 4, PF = 4;                // ring slots; loads run PF steps ahead
  static_assert(PF <= NSLOT && PF >= 2, "step s+PF reuses the slot of step s");
  static constexpr int LDS = NSLOT * SLOT;
  static constexpr int A_IT = BM_ * 4 / NT, B_IT = BROWS * 4 / NT;
  static constexpr int LPS = A_IT + B_IT;                // loads per step, every wave
  static_assert(BM_ % 64 == 0 && A_IT * NT == BM_ * 4 && B_IT * NT == BROWS * 4, "whole loads per wave");
  static_assert(BN_ % (NT / 4) == 0, "gate/up split on a load boundary");
  static_assert(LDS <= 160 * 1024, "LDS per workgroup");
};

template <typename Cfg>
__device__ __forceinline__ void large_issue(char* slot, uint32_t kb, __amdgpu_buffer_rsrc_t rsA,
                                            __amdgpu_buffer_rsrc_t rsB0, __amdgpu_buffer_rsrc_t rsB1,
                                            const uint32_t* voffA, const uint32_t* voffB, int wave) {
  constexpr int NT = Cfg::NT, RPI = NT / 4;             // rows covered by one load of every wave
#pragma unroll
  for (int it = 0; it < Cfg::A_IT; ++it)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsA, (__attribute__((address_space(3))) void*)(slot + (it * NT + wave * kWave) * 16), 16, voffA[it], kb, 0, 0);
#pragma unroll
  for (int it = 0; it < Cfg::B_IT; ++it) {
    auto* dst = (__attribute__((address_space(3))) void*)(slot + Cfg::A_SLOT + (it * NT + wave * kWave) * 16);
    if (Cfg::NB == 2 && it * RPI >= Cfg::BN_)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB1, dst, 16, voffB[it], kb, 0, 0);
    else
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB0, dst, 16, voffB[it], kb, 0, 0);
  }
}

template <typename T, int BN, bool GATED>
__global__ __launch_bounds__(256) void grouped_gemm_large_kernel(GemmArgs args) {
  using Cfg = LargeTile<T, BN, GATED>;
  constexpr int NT = Cfg::NT, TM = Cfg::TM, TN = Cfg::TN, TNB = Cfg::TNB, PF = Cfg::PF, LPS = Cfg::LPS;
  extern __shared__ __align__(16) char lds[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / Cfg::WN, wn = wave % Cfg::WN;
  const int N = args.N, K = args.K;
  const int ntn = N / BN;
  const int mt_live = args.offsets ? args.tstart[args.G] : (args.dense_rows + Cfg::BM_ - 1) / Cfg::BM_;
  const int live = mt_live * ntn;
  const int xcd = blockIdx.x % kNumXcd, j0 = blockIdx.x / kNumXcd, bpx = gridDim.x / kNumXcd;
  const int lo = (int)((long long)live * xcd / kNumXcd);
  const int hi = (int)((long long)live * (xcd + 1) / kNumXcd);
  const int nks = K / 32;                               // 64-byte K steps
  const size_t row_stride = (size_t)K * sizeof(T);
  // fragment read offsets inside a slot: row (lane & 15) of each 16-row subtile, piece lane >> 4
  const int offA = swz64(wm * Cfg::WTM + (lane & 15), lane >> 4);
  const int offB = Cfg::A_SLOT + swz64(wn * Cfg::WTN + (lane & 15), lane >> 4);

  for (int L = lo + j0; L < hi; L += bpx) {
    const TileCoord tc = tile_coord(args, L, ntn, mt_live, bpx, Cfg::BM_);
    const int g = tc.g, nt = tc.nt, row0 = tc.row0, rows = tc.rows;
    const char* Ab = (const char*)args.A + (args.a_rows ? 0 : (size_t)row0 * row_stride);
    const char* B0b = (const char*)args.B0 + ((size_t)g * N + (size_t)nt * BN) * row_stride;
    const char* B1b = GATED ? (const char*)args.B1 + ((size_t)g * N + (size_t)nt * BN) * row_stride : B0b;
    const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc((void*)Ab, 0, kBufRange, kBufFlags);
    const __amdgpu_buffer_rsrc_t rsB0 = __builtin_amdgcn_make_buffer_rsrc((void*)B0b, 0, kBufRange, kBufFlags);
    const __amdgpu_buffer_rsrc_t rsB1 = __builtin_amdgcn_make_buffer_rsrc((void*)B1b, 0, kBufRange, kBufFlags);

    // lane -> (row, swizzled piece) of each 16-byte load; rows past `rows` repeat the last
    uint32_t voffA[Cfg::A_IT], voffB[Cfg::B_IT];
#pragma unroll
    for (int it = 0; it < Cfg::A_IT; ++it) {
      const int q = it * NT + wave * kWave + lane, r = q >> 2;
      const int pc = (q & 3) ^ ((r >> 1) & 3);
      const int rr = min(r, rows - 1);
      const size_t arow = args.a_rows ? (size_t)args.a_rows[row0 + rr] : (size_t)rr;
      voffA[it] = (uint32_t)(arow * row_stride + pc * 16);
    }
#pragma unroll
    for (int it = 0; it < Cfg::B_IT; ++it) {
      const int q = it * NT + wave * kWave + lane, r = q >> 2;
      const int pc = (q & 3) ^ ((r >> 1) & 3);
      voffB[it] = (uint32_t)((GATED && r >= BN ? r - BN : r) * row_stride + pc * 16);
    }
    // step s of the ring; past the last step the loads repeat the last one into a slot
    // nobody reads again, which keeps every step's instruction stream the same
    auto issue = [&](int s) {
      large_issue<Cfg>(lds + (s % Cfg::NSLOT) * Cfg::SLOT, (uint32_t)min(s, nks - 1) * 64, rsA, rsB0, rsB1,
                       voffA, voffB, wave);
    };

    f32x4_t acc0[TM][TN], acc1[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        acc0[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        acc1[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    u32x4_t fa0[TM], fb0[TNB], fa1[TM], fb1[TNB];

    auto read = [&](int s, u32x4_t* fa, u32x4_t* fb) {
      const char* sl = lds + (s % Cfg::NSLOT) * Cfg::SLOT;
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[i] = *(const u32x4_t*)(sl + offA + i * 16 * 64);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        fb[j] = *(const u32x4_t*)(sl + offB + j * 16 * 64);
        if constexpr (GATED) fb[TN + j] = *(const u32x4_t*)(sl + offB + (BN + j * 16) * 64);
      }
    };
    // one K step: wait for step s+1's loads, barrier, start step s+PF's loads, then the
    // MFMAs of step s (operands in cur) alongside the LDS reads of step s+1 (nxt)
    auto step = [&](int s, const u32x4_t* fa, const u32x4_t* fb, u32x4_t* na, u32x4_t* nb) {
      wait_vmcnt<(PF - 2) * LPS>();
      block_barrier();
      issue(s + PF);
      read(s + 1, na, nb);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          Mfma<T>::step(acc0[i][j], fa[i], fb[j]);
          if constexpr (GATED) Mfma<T>::step(acc1[i][j], fa[i], fb[TN + j]);
        }
    };

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");       // previous tile's stores drained
#pragma unroll
    for (int p = 0; p < PF; ++p) issue(p);
    wait_vmcnt<(PF - 1) * LPS>();                          // own loads of step 0 landed
    block_barrier();
    read(0, fa0, fb0);
    int ks = 0;
#pragma clang loop unroll(disable)
    for (; ks + 1 < nks; ks += 2) {
      step(ks, fa0, fb0, fa1, fb1);
      step(ks + 1, fa1, fb1, fa0, fb0);
    }
    if (ks < nks) step(ks, fa0, fb0, fa1, fb1);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();                                    // LDS free for the next tile

    store_tile<Cfg>(args, acc0, acc1, wm, wn, lane, g, nt, row0, rows);
  }
}

template <typename T, int BN, bool GATED>
static hipError_t launch_large(const GemmArgs& a, int max_tiles_m, hipStream_t stream) {
  return launch_kernel<LargeTile<T, BN, GATED>, grouped_gemm_large_kernel<T, BN, GATED>>(a, max_tiles_m, stream);
}

hipError_t launch_gemm_large_bf16(const GemmArgs& a, int max_tiles_m, hipStream_t stream) {
  if (a.N % 256 == 0) return launch_large<uint16_t, 256, false>(a, max_tiles_m, stream);
  return launch_large<uint16_t, 128, false>(a, max_tiles_m, stream);
}

}  // namespace moe
