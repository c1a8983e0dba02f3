// Grouped expert GEMMs for gfx950 on MFMA (16x16 tiles, fp32 accumulate).
//
// The experts are SwiGLU networks (Zero to Frontier §13.1 "Why MoE", section "The MoE
// layer"): h = SiLU(X W_g) * (X W_u), then o = h W_d.  After dispatch the rows of each
// expert are contiguous, so each product is a grouped GEMM ("replace the loop itself
// with a grouped matrix multiply", the same page's "In PyTorch" section).  Weights are
// stored [out, in], so both operands are read along the contraction dimension.
//
// One kernel template, three tile configurations:
//   large   BM=256, BN=128 (gate/up) or 256 (down; bf16 BM=192), 4x2 waves, activations
//           2 LDS stages and weights 3 -- many rows per expert (MFMA-bound)
//   stream  BM=160, BN=128 (gate/up) or 256 (down), 2x4 waves, 3 LDS stages -- ~100-250
//           rows per expert (weight streaming; an expert's m-tiles run side by side so
//           its weight tile leaves HBM once)
//   decode  BM=16, BN=64 (gate/up, 1x4 waves) or 32 (down, 1x2 waves), 4 LDS stages --
//           a few rows per expert (weight streaming)
// The gate/up variant holds two accumulators per output tile (gate and up rows of the
// same n-tile share the A fragments) and applies SiLU(a) * b in registers; the down
// variant writes fp32.
//
// Memory path per K step (128 bytes of each row): global -> LDS directly (16-byte
// pieces, XOR-swizzled so MFMA operand reads are bank-conflict free) -> MFMA operands,
// with the next steps' loads in flight during the current step's MFMAs (a ring of
// 2-4 LDS stages, one barrier per step).
//
// Scheduling: a persistent grid of (#CUs x occupancy) blocks; tiles are numbered
// L = 0 .. live-1 and each XCD (blocks b with b % 8 == x) walks its own contiguous
// eighth of L, so tiles that share operands run on the same L2 (see the tile order
// in the kernel).
#pragma once

#include "gemm_common.h"

namespace moe {

// Epilogue / schedule of an instance (EPI):
//   0  forward: SiLU(a) * b in the activation type (gated) or fp32 (plain)
//   1  gated, backward recompute: a and b in fp32 and h = SiLU(a) * b transposed (gemm_bwd.h)
//   2  plain, backward of the down product: dA, dB from a, b and per-row partial dots (gemm_bwd.h)
//   3  plain, K-grouped: group g contracts K columns [koffsets[g], koffsets[g+1]) of one A and
//      one B into its own fp32 output (the weight gradients)
// KSUB: 64-element K sub-steps per LDS stage.  Quantised decode tiles take several, so that
// each weight row contributes 128 contiguous bytes per stage (a 64-element step of 4-bit
// codes is only 32 bytes; the memory system serves few enough requests per second that
// 32-byte requests cannot stream weights at HBM speed).
template <typename T, int BM, int BN, int WM, int WN, bool GATED, int STAGES, int BSTAGES = STAGES,
          int WF = 0, int EPI = 0, int KSUB = 1>
struct GemmTile {
  using Elem = T;
  // weight format: 0 native (dtype), 1 FP8 E4M3 with row scales, 2 MXFP4 (E2M1, E8M0 per 32)
  static constexpr int WF_ = WF;
  static constexpr int EPI_ = EPI;
  static constexpr int KSUB_ = KSUB;
  static constexpr int NT = WM * WN * kWave;
  static constexpr int BM_ = BM, BN_ = BN;
  static constexpr int WTM = BM / WM, WTN = BN / WN;
  static constexpr int TM = WTM / 16, TN = WTN / 16;
  static constexpr int NB = GATED ? 2 : 1;
  static constexpr int BROWS = BN * NB;
  static constexpr int ROWB = 128;                                  // bytes of K per row per stage
  static constexpr int EPP = Mfma<T>::kElemsPerPiece;               // elements per 16-byte piece
  static constexpr int BKE = 8 * EPP;                               // elements of K per stage
  // 16-byte weight pieces per row per stage
  static constexpr int PPR_B = (WF == 1 ? 4 : (WF == 2 ? 2 : 8)) * KSUB;
  static constexpr int ROWB_B = PPR_B * 16;
  // LDS: a ring of STAGES activation stages (KSUB slots of one 64-element sub-step each), then a
  // ring of BSTAGES weight slots.  MXFP4: the stage's 2 KSUB E8M0 scale bytes per weight row
  // follow the codes in the weight slot, [matrix][block][row of the matrix]
  static constexpr int S_BYTES = WF == 2 ? 2 * KSUB * BROWS : 0;
  static constexpr int A_SLOT = BM * ROWB, A_STAGE = KSUB * A_SLOT, B_SLOT = BROWS * ROWB_B + S_BYTES;
  static constexpr int B_BASE = STAGES * A_STAGE;
  static constexpr int LDS = STAGES * A_STAGE + BSTAGES * B_SLOT;
  // Forward tiles with 16 bytes of LDS to spare can be scheduled dynamically (GemmArgs::tile_ctr):
  // the block's next tile index passes from its first thread to the others there.
  static constexpr bool DYN = EPI == 0 && LDS + 16 <= 160 * 1024;
  static constexpr int LDS_ALLOC = LDS + (DYN ? 16 : 0);
  static constexpr int NW = WM * WN;
  // 16-byte global -> LDS pieces per K step: activations, weights, MXFP4 scales.  Each wave
  // loads a contiguous equal share of every kind (PW_* pieces, IT_* instructions of up to 64
  // lanes), so every wave issues exactly LPS loads per step and "at most LPS * n outstanding"
  // leaves exactly n newer steps in flight for every wave.
  static constexpr int P_A = BM * 8 * KSUB, P_B = BROWS * PPR_B, P_S = S_BYTES / 16;
  static constexpr int PW_A = P_A / NW, PW_B = P_B / NW, PW_S = P_S / NW;
  static constexpr int IT_A = (PW_A + kWave - 1) / kWave, IT_B = (PW_B + kWave - 1) / kWave;
  static constexpr int IT_S = P_S ? 1 : 0;
  static constexpr int LPS_B = IT_B + IT_S;
  static constexpr int LPS = IT_A + LPS_B;
  static constexpr int A_IT = IT_A, B_IT = IT_B;
  static_assert(P_A % NW == 0 && P_B % NW == 0 && P_S % NW == 0, "equal shares per wave");
  static_assert(NW % 2 == 0, "gate and up halves of the weight pieces split on a wave boundary");
  static_assert(P_S == 0 || (PW_S <= kWave && (2 * KSUB * (BN / 16)) % PW_S == 0),
                "a wave's scale share is one matrix");
  static_assert(KSUB == 1 || (WF != 0 && ROWB_B == 128 && EPI == 0), "sub-steps: 128-byte weight rows");
  static_assert(LPS * (STAGES - 2) <= 63, "vmcnt range");
  static_assert(BSTAGES == STAGES || (STAGES == 2 && BSTAGES == 3), "weight ring: same depth, or 3 with 2");
  static_assert(LDS <= 160 * 1024, "LDS per workgroup");
  // Skip MFMAs of 16-row subtiles that hold no rows.  Worth a branch only where most
  // subtiles can be empty (the stream and decode tiles); the large tile keeps a
  // branch-free inner loop.
  static constexpr bool SKIP_ROWS = BM != 256;
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be whole 16x16 MFMA tiles");
  static_assert(WF == 0 || sizeof(T) == 2, "quantised weights go with bf16 activations");
  static_assert(EPI == 0 || (WF == 0 && (EPI == 1) == GATED), "backward epilogues: native weights");

};

__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ ((r >> 1) & 7)) << 4); }

// Wait until the oldest in-flight K step has landed, leaving `ahead` newer ones in flight.
template <int LPS, int STAGES>
__device__ __forceinline__ void wait_stage(int ahead) {
  if constexpr (STAGES <= 2) {
    wait_vmcnt<0>();
  } else {
    static_assert(STAGES <= 12, "deeper rings need more cases");
    switch (ahead) {      // ahead <= STAGES - 2; each case's count is only used when reachable
      case 0: wait_vmcnt<0>(); break;
      case 1: wait_vmcnt<LPS>(); break;
      case 2: wait_vmcnt<2 * LPS>(); break;
      case 3: wait_vmcnt<(STAGES > 4 ? 3 : 0) * LPS>(); break;
      case 4: wait_vmcnt<(STAGES > 5 ? 4 : 0) * LPS>(); break;
      case 5: wait_vmcnt<(STAGES > 6 ? 5 : 0) * LPS>(); break;
      case 6: wait_vmcnt<(STAGES > 7 ? 6 : 0) * LPS>(); break;
      case 7: wait_vmcnt<(STAGES > 8 ? 7 : 0) * LPS>(); break;
      case 8: wait_vmcnt<(STAGES > 9 ? 8 : 0) * LPS>(); break;
      case 9: wait_vmcnt<(STAGES > 10 ? 9 : 0) * LPS>(); break;
      default: wait_vmcnt<(STAGES > 11 ? 10 : 0) * LPS>(); break;
    }
  }
}

// Enqueue one K step of the A (activation) or B (weight) tile into an LDS slot
// (asynchronous; completion is tracked by vmcnt).  Wave w loads pieces [w PW, (w+1) PW) of
// each kind, 64 per instruction (lane L writes LDS bytes 16 L .. 16 L + 15 past the
// instruction's base); lanes past the share are masked off.
template <typename Cfg>
__device__ __forceinline__ void issue_a(char* As, uint32_t kb, __amdgpu_buffer_rsrc_t rsA, const uint32_t* voffA,
                                        int wave, int lane) {
#pragma unroll
  for (int it = 0; it < Cfg::IT_A; ++it) {
    const int q0 = wave * Cfg::PW_A + it * kWave;
    if (Cfg::PW_A % kWave == 0 || it * kWave + lane < Cfg::PW_A)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (__attribute__((address_space(3))) void*)(As + q0 * 16), 16,
                                               voffA[it], kb, 0, 0);
  }
}

template <typename Cfg>
__device__ __forceinline__ void issue_b(char* Bs, uint32_t kb, __amdgpu_buffer_rsrc_t rsB0,
                                        __amdgpu_buffer_rsrc_t rsB1, const uint32_t* voffB, int wave, int lane) {
  // the up rows of the gated product are the second half of the pieces: whole waves
  const bool up = Cfg::NB == 2 && wave >= Cfg::NW / 2;
#pragma unroll
  for (int it = 0; it < Cfg::IT_B; ++it) {
    const int q0 = wave * Cfg::PW_B + it * kWave;
    auto* dst = (__attribute__((address_space(3))) void*)(Bs + q0 * 16);
    if (Cfg::PW_B % kWave == 0 || it * kWave + lane < Cfg::PW_B) {
      if (up)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB1, dst, 16, voffB[it], kb, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB0, dst, 16, voffB[it], kb, 0, 0);
    }
  }
}

// MXFP4 scale bytes of one stage (2 KSUB blocks of 32) for the tile's weight rows, matrix
// by matrix: the share of wave w lies inside one matrix.
template <typename Cfg>
__device__ __forceinline__ void issue_s(char* Ss, uint32_t kbs, __amdgpu_buffer_rsrc_t rsS0,
                                        __amdgpu_buffer_rsrc_t rsS1, uint32_t voffS, int wave, int lane) {
  if constexpr (Cfg::WF_ == 2) {
    constexpr int PPMS = 2 * Cfg::KSUB_ * (Cfg::BN_ / 16);         // pieces per matrix per stage
    const int q0 = wave * Cfg::PW_S;
    const bool up = Cfg::NB == 2 && q0 >= PPMS;
    auto* dst = (__attribute__((address_space(3))) void*)(Ss + q0 * 16);
    if (lane < Cfg::PW_S) {
      if (up)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsS1, dst, 16, voffS, kbs, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsS0, dst, 16, voffS, kbs, 0, 0);
    }
  }
}

// LDS byte offset of 16-byte piece `c` of weight row r in a weight slot (rows of PPR_B pieces,
// swizzled as tile_offsets places them).
template <typename Cfg>
__device__ __forceinline__ int b_piece(int r, int c) {
  if constexpr (Cfg::PPR_B == 8) return swz(r, c);
  else if constexpr (Cfg::PPR_B == 4) return swz64(r, c);
  else return r * 32 + ((c ^ ((r >> 2) & 1)) << 4);
}

// Per-lane 32-bit buffer offsets of one tile's global -> LDS pieces.  Lane L of a wave's
// buffer_load_dwordx4 ... lds writes LDS bytes [base + 16 L, base + 16 L + 16), so each
// lane loads the global piece that belongs at that swizzled LDS position.  Rows past
// `rows` repeat the last valid row: their results are never stored.
template <typename Cfg>
__device__ __forceinline__ void tile_offsets(const GemmArgs& args, int wave, int lane, int row0, int rows,
                                             size_t row_stride, size_t row_stride_b, uint32_t* voffA,
                                             uint32_t* voffB) {
#pragma unroll
  for (int it = 0; it < Cfg::A_IT; ++it) {
    const int q = min(wave * Cfg::PW_A + it * kWave + lane, Cfg::P_A - 1);
    const int u = q / (Cfg::BM_ * 8), qa = q - u * (Cfg::BM_ * 8), r = qa >> 3;   // sub-step, row
    const int cl = (qa & 7) ^ ((r >> 1) & 7);
    const int rr = min(r, rows - 1);
    const size_t arow = args.a_rows ? (size_t)args.a_rows[row0 + rr] : (size_t)rr;
    voffA[it] = (uint32_t)(arow * row_stride + u * 128 + cl * 16);
  }
#pragma unroll
  for (int it = 0; it < Cfg::B_IT; ++it) {
    const int q = min(wave * Cfg::PW_B + it * kWave + lane, Cfg::P_B - 1);
    const int r = q / Cfg::PPR_B;
    const int cl = Cfg::PPR_B == 8 ? (q & 7) ^ ((r >> 1) & 7)
                                   : (Cfg::PPR_B == 4 ? (q & 3) ^ ((r >> 1) & 3) : (q & 1) ^ ((r >> 2) & 1));
    voffB[it] = (uint32_t)((Cfg::NB == 2 && r >= Cfg::BN_ ? r - Cfg::BN_ : r) * row_stride_b + cl * 16);
  }
}

// Eight E2M1 codes (one dword, low nibble first) times a power-of-two block scale, as eight
// bf16 values, exactly.
__device__ __forceinline__ u32x4_t e2m1x8_to_bf16(uint32_t v, float scale) {
  return u32x4_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 0)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 1)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 2)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 3))};
}

// An E8M0 scale byte as a float: 2^(s - 127) (s = 0 is the subnormal 2^-127), 255 = NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return __uint_as_float(s == 0 ? 0x00400000u : (s == 255 ? 0x7FC00000u : s << 23));
}

// Eight E4M3 codes (two dwords) as eight bf16 values, exactly (every E4M3 value is a bf16).
__device__ __forceinline__ u32x4_t e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  return u32x4_t{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true))};
}

template <typename T, int BM, int BN, int WM, int WN, bool GATED, int STAGES, int BSTAGES, int WF, int EPI,
          int KSUB>
__global__ __launch_bounds__(WM* WN * 64) void grouped_gemm_kernel(GemmArgs args) {
  using Cfg = GemmTile<T, BM, BN, WM, WN, GATED, STAGES, BSTAGES, WF, EPI, KSUB>;
  constexpr bool KGRP = EPI == 3;
  constexpr int TM = Cfg::TM, TN = Cfg::TN, NB = Cfg::NB;
  constexpr int A_IT = Cfg::A_IT, B_IT = Cfg::B_IT, BKE = Cfg::BKE;
  extern __shared__ __align__(16) char lds[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in a scalar register
  const int wm = wave / WN, wn = wave % WN;
  const int N = args.N, K = args.K;
  const int ntn = N / BN;
  const int mt_live = !KGRP && args.offsets ? args.tstart[args.G] : (args.dense_rows + BM - 1) / BM;
  const int ksp = GATED || EPI != 0 ? 1 : args.ksplit;   // K chunks per output tile
  const int live = mt_live * ntn * ksp * (KGRP ? args.G : 1);
  const int xcd = blockIdx.x % kNumXcd, j0 = blockIdx.x / kNumXcd, bpx = gridDim.x / kNumXcd;
  const int lo = (int)((long long)live * xcd / kNumXcd);
  const int hi = (int)((long long)live * (xcd + 1) / kNumXcd);
  const int nks = K / (BKE * KSUB) / ksp;             // LDS stages (K steps of BKE * KSUB) per chunk
  const size_t row_stride = (size_t)K * sizeof(T);   // bytes per row of A
  const size_t row_stride_b = WF == 1 ? (size_t)K : (WF == 2 ? (size_t)K / 2 : row_stride);   // per weight row
  constexpr uint32_t KB_B = Cfg::ROWB_B;              // weight bytes per row per stage
  constexpr uint32_t KB_A = 128 * KSUB;               // activation bytes per row per stage

  // Dynamic scheduling: the ticket for the block's next tile is drawn after the K loop and
  // read once the epilogue's stores are issued; each tile waits for its predecessor's stores
  // to drain anyway, so the atomic's round trip hides behind them.
  const bool dyn = Cfg::DYN && args.tile_ctr != nullptr;
  int* ticket = (int*)(lds + Cfg::LDS);
  for (int L = lo + j0, Lnext = 0; L < hi; L = Lnext) {
    // consecutive work items are the K chunks of one output tile
    const int chunk = ksp > 1 ? L % ksp : 0;
    int g, nt, row0, rows, nk = nks;
    size_t ks0 = (size_t)chunk * nks;                   // first stage of the chunk
    size_t c_off = (size_t)chunk * args.split_stride;   // output offset (elements)
    if constexpr (KGRP) {
      // group-major; inside a group n-tile-major, so consecutive tiles share the B tile
      const int per = mt_live * ntn;
      g = L / per;
      const int rem = L - g * per;
      nt = rem / mt_live;
      row0 = (rem - nt * mt_live) * BM;
      rows = min(BM, args.dense_rows - row0);
      const int k0 = args.koffsets[g], k1 = args.koffsets[g + 1];
      nk = (k1 - k0) / BKE;
      ks0 = (size_t)(k0 / BKE);
      c_off = (size_t)g * args.dense_rows * N;
    } else {
      const TileCoord tc = tile_coord(args, ksp > 1 ? L / ksp : L, ntn, mt_live, max(1, bpx / ksp), BM);
      g = tc.g;
      nt = tc.nt;
      row0 = tc.row0;
      rows = tc.rows;
    }
    // Buffer resources over this tile's A rows and B rows (from the chunk's first K step);
    // per-lane 32-bit offsets are fixed for the tile and the K step rides in the scalar offset.
    // (K-grouped: one B for every group.)
    const size_t brow0 = (KGRP ? 0 : (size_t)g * N) + (size_t)nt * BN;
    const char* Ab = (const char*)args.A + (args.a_rows ? 0 : (size_t)row0 * row_stride) + ks0 * KB_A;
    const char* B0b = (const char*)args.B0 + brow0 * row_stride_b + ks0 * KB_B;
    const char* B1b = GATED ? (const char*)args.B1 + brow0 * row_stride_b + ks0 * KB_B : B0b;
    const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc((void*)Ab, 0, kBufRange, kBufFlags);
    const __amdgpu_buffer_rsrc_t rsB0 = __builtin_amdgcn_make_buffer_rsrc((void*)B0b, 0, kBufRange, kBufFlags);
    const __amdgpu_buffer_rsrc_t rsB1 = __builtin_amdgcn_make_buffer_rsrc((void*)B1b, 0, kBufRange, kBufFlags);

    uint32_t voffA[A_IT], voffB[B_IT];
    tile_offsets<Cfg>(args, wave, lane, row0, rows, row_stride, row_stride_b, voffA, voffB);
    auto a_slot = [&](int s) { return lds + s * Cfg::A_STAGE; };
    auto b_slot = [&](int s) { return lds + Cfg::B_BASE + s * Cfg::B_SLOT; };
    // MXFP4 block scales: [G, K/32, N] bytes per matrix; each lane loads 16 rows of one block
    // of one matrix (see issue_s), each stage advancing 2 KSUB blocks
    __amdgpu_buffer_rsrc_t rsS0 = rsB0, rsS1 = rsB1;
    uint32_t voffS = 0;
    if constexpr (WF == 2) {
      const size_t gs = (size_t)g * (K / 32) * N + ks0 * 2 * KSUB * N;
      rsS0 = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)args.S0 + gs), 0, kBufRange, kBufFlags);
      rsS1 = GATED ? __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)args.S1 + gs), 0, kBufRange, kBufFlags)
                   : rsS0;
      constexpr int PPM = BN / 16, PPMS = 2 * KSUB * PPM;
      const int qs = wave * Cfg::PW_S + min(lane, Cfg::PW_S - 1);   // [matrix][block c][piece p]
      const int c = (qs % PPMS) / PPM, p = qs % PPM;
      voffS = (uint32_t)(c * N + nt * BN + 16 * p);
    }
    // one stage of weights (codes, and MXFP4 scales) into weight slot s
    auto issue_w = [&](int s, int ks) {
      issue_b<Cfg>(b_slot(s), (uint32_t)ks * KB_B, rsB0, rsB1, voffB, wave, lane);
      issue_s<Cfg>(b_slot(s) + Cfg::BROWS * Cfg::ROWB_B, (uint32_t)ks * 2 * KSUB * N, rsS0, rsS1, voffS, wave,
                   lane);
    };

    f32x4_t acc0[TM][TN], acc1[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        acc0[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        acc1[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }

    // One K step from LDS stage s: 2 chunks of 64 bytes.  The A fragment of the next
    // subtile (and at the chunk boundary the next chunk's B fragments) is read before
    // the current subtile's MFMAs are issued, so LDS latency hides behind MFMA work.
    // issue(0) and issue(1) start the global -> LDS loads of later steps (activations, then
    // weights), each once per step and in that order; the native-weight path places them
    // between its MFMAs (see the K loop).
    auto compute = [&](const char* As, const char* Bs, auto&& issue) {
      const int ra = wm * Cfg::WTM + (lane & 15);
      const int rb = wn * Cfg::WTN + (lane & 15);
      if constexpr (WF == 2) {
        issue(0);
        issue(1);
        // MXFP4 weights: per 64-element sub-step u, an 8-byte LDS read per weight subtile gives
        // lane group q = lane >> 4 the codes of K elements 16q .. 16q+15 of the sub-step
        // (32 bytes of a row: pieces 2u and 2u+1), and one byte the scale of their block
        // (2u + (q >> 1)); the same K permutation as FP8 pairs them with A pieces 2q + h.
        const int q = lane >> 4;
        const char* Ss = Bs + Cfg::BROWS * Cfg::ROWB_B;
#pragma unroll
        for (int u = 0; u < KSUB; ++u) {
          const char* Au = As + u * Cfg::A_SLOT;
          uint32_t raw[TN * NB][2];
          float sc[TN * NB];
#pragma unroll
          for (int j = 0; j < TN * NB; ++j) {
            const int m = j < TN ? 0 : 1, rm = rb + (j - m * TN) * 16;   // matrix, row in it
            const int r = m * BN + rm;
            const uint2 v = *(const uint2*)(Bs + b_piece<Cfg>(r, 2 * u + (q >> 1)) + ((q & 1) << 3));
            raw[j][0] = v.x;
            raw[j][1] = v.y;
            sc[j] = e8m0_to_f32(*(const uint8_t*)(Ss + (m * 2 * KSUB + 2 * u + (q >> 1)) * BN + rm));
          }
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            u32x4_t b[TN * NB];
#pragma unroll
            for (int j = 0; j < TN * NB; ++j) b[j] = e2m1x8_to_bf16(raw[j][h], sc[j]);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
              if (!Cfg::SKIP_ROWS || wm * Cfg::WTM + i * 16 < rows) {
                const u32x4_t a = *(const u32x4_t*)(Au + swz(ra + i * 16, 2 * (lane >> 4) + h));
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                  Mfma<T>::step(acc0[i][j], a, b[j]);
                  if constexpr (GATED) Mfma<T>::step(acc1[i][j], a, b[TN + j]);
                }
              }
            }
          }
        }
        return;
      } else if constexpr (WF == 1) {
        issue(0);
        issue(1);
        // FP8 weights: per 64-element sub-step u, one 16-byte LDS read per weight subtile gives
        // lane group q = lane >> 4 the codes of K elements 16q .. 16q+15 of the sub-step (piece
        // 4u + q of the row); the MFMA of half h takes 16q + 8h .. 16q + 8h + 7 from both
        // operands (the same permutation of the contraction index on A and B leaves every dot
        // product unchanged), so the A fragment of half h is 16-byte piece 2q + h of the
        // sub-step's activation row.
#pragma unroll
        for (int u = 0; u < KSUB; ++u) {
          const char* Au = As + u * Cfg::A_SLOT;
          u32x4_t raw[TN * NB];
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            raw[j] = *(const u32x4_t*)(Bs + b_piece<Cfg>(rb + j * 16, 4 * u + (lane >> 4)));
            if constexpr (GATED)
              raw[TN + j] = *(const u32x4_t*)(Bs + b_piece<Cfg>(BN + rb + j * 16, 4 * u + (lane >> 4)));
          }
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            u32x4_t b[TN * NB];
#pragma unroll
            for (int j = 0; j < TN * NB; ++j) b[j] = e4m3x8_to_bf16(raw[j][2 * h], raw[j][2 * h + 1]);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
              if (!Cfg::SKIP_ROWS || wm * Cfg::WTM + i * 16 < rows) {
                const u32x4_t a = *(const u32x4_t*)(Au + swz(ra + i * 16, 2 * (lane >> 4) + h));
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                  Mfma<T>::step(acc0[i][j], a, b[j]);
                  if constexpr (GATED) Mfma<T>::step(acc1[i][j], a, b[TN + j]);
                }
              }
            }
          }
        }
        return;
      }
      auto rdA = [&](int i, int kc) {
        const int r = ra + i * 16;
        return *(const u32x4_t*)(As + swz(r, kc * 4 + (lane >> 4)));
      };
      auto rdB = [&](u32x4_t* b, int kc) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int r = rb + j * 16;
          b[j] = *(const u32x4_t*)(Bs + swz(r, kc * 4 + (lane >> 4)));
          if constexpr (GATED) b[TN + j] = *(const u32x4_t*)(Bs + swz(BN + r, kc * 4 + (lane >> 4)));
        }
      };
      u32x4_t b0[TN * NB], b1[TN * NB];
      rdB(b0, 0);
      u32x4_t a_cur = rdA(0, 0), a_nxt;
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if (i + 1 < TM) a_nxt = rdA(i + 1, kc);
          else if (kc == 0) { rdB(b1, 1); a_nxt = rdA(0, 1); }
          const u32x4_t* b = kc == 0 ? b0 : b1;
          if (!Cfg::SKIP_ROWS || wm * Cfg::WTM + i * 16 < rows) {   // wave-uniform: skip padding subtiles
#pragma unroll
            for (int j = 0; j < TN; ++j) {
              Mfma<T>::step(acc0[i][j], a_cur, b[j]);
              if constexpr (GATED) Mfma<T>::step(acc1[i][j], a_cur, b[TN + j]);
            }
          }
          a_cur = a_nxt;
          if (kc == 0 && i == 0) issue(0);
          if (kc == 0 && i == TM - 1) issue(1);
        }
      }
    };

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");       // previous tile's stores drained
    if constexpr (BSTAGES == STAGES) {
      // STAGES-deep ring: up to STAGES-1 K steps in flight while one is consumed.
#pragma unroll
      for (int p = 0; p < STAGES - 1; ++p)
        if (p < nk) {
          issue_a<Cfg>(a_slot(p), (uint32_t)p * KB_A, rsA, voffA, wave, lane);
          issue_w(p, p);
        }
      // The stream tiles start the step's loads between its MFMAs as the 2+3 ring below does
      // (DeepSeek-V3 shape gate/up 2.69 -> 2.62 ms, Switch shape down 102 -> 96 us); the
      // decode tiles, a few MFMAs per step, issue them straight after the barrier.
      int slot = 0;
      for (int ks = 0; ks < nk; ++ks) {
        wait_stage<Cfg::LPS, STAGES>(min(STAGES - 2, nk - 1 - ks));   // step ks has landed
        block_barrier();                                // ... for every wave; slot ks-1 is free
        const int fs = slot == 0 ? STAGES - 1 : slot - 1;
        const bool more = ks + STAGES - 1 < nk;
        if constexpr (BM >= 64) {
          compute(a_slot(slot), b_slot(slot), [&](int part) {
            if (!more) return;
            if (part == 0) issue_a<Cfg>(a_slot(fs), (uint32_t)(ks + STAGES - 1) * KB_A, rsA, voffA, wave, lane);
            else issue_w(fs, ks + STAGES - 1);
          });
        } else {
          if (more) {
            issue_a<Cfg>(a_slot(fs), (uint32_t)(ks + STAGES - 1) * KB_A, rsA, voffA, wave, lane);
            issue_w(fs, ks + STAGES - 1);
          }
          compute(a_slot(slot), b_slot(slot), [](int) {});
        }
        slot = slot + 1 == STAGES ? 0 : slot + 1;
      }
    } else {
      // Weights two K steps ahead, activations one.  Issue order A(0) B(0) B(1), then per
      // step A(ks+1) B(ks+2): when step ks is consumed the only newer loads than A(ks) are
      // those of B(ks+1), so waiting until at most LPS_B are outstanding lands A(ks), B(ks).
      // Both slots were freed by the barrier at the top of step ks.  The loads start after
      // the step's first MFMAs rather than straight after the barrier: all waves leave the
      // barrier together, and a burst of global -> LDS loads there delays the LDS operand
      // reads that the first MFMAs wait for (measured at the Mixtral prefill shape: activations
      // after the first subtile row and weights after the first half, 1.56 ms against
      // 1.70 ms for the gate/up product).
      if (nk > 0) {
        issue_a<Cfg>(a_slot(0), 0, rsA, voffA, wave, lane);
        issue_w(0, 0);
      }
      if (nk > 1) issue_w(1, 1);
      int bs = 0;                                       // weight slot of step ks
      if constexpr (WF == 0 && EPI == 0 && sizeof(T) == 2) {
        // Forward bf16 products with native weights: the barrier that makes step ks+1 visible is
        // taken before step ks's last subtile row, and step ks+1's first fragments are read
        // while that row's MFMAs run, so no step starts by waiting on LDS.  Every read of step
        // ks is issued before that barrier (and completed by it), so the slots refilled at
        // step ks+1 are free as in the loop below; the vmcnt accounting is the same.  (The
        // backward epilogues keep the loop below: measured slower in this form; fp32 tiles
        // too: they would spill registers in it.)
        const int ra = wm * Cfg::WTM + (lane & 15);
        const int rb = wn * Cfg::WTN + (lane & 15);
        // swz(r + 16 i, c) = swz(r, c) + 2048 i: one lane offset per operand and chunk
        const int oA0 = swz(ra, lane >> 4), oA1 = swz(ra, 4 + (lane >> 4));
        const int oB0 = swz(rb, lane >> 4), oB1 = swz(rb, 4 + (lane >> 4));
        auto rdA = [&](const char* As, int i, int kc) {
          return *(const u32x4_t*)(As + (kc ? oA1 : oA0) + i * 2048);
        };
        // Gated: only the gate half of a step's first B fragments is read ahead (at the
        // previous step's tail) and the up half at the top of the step's first subtile row;
        // reading both ahead needs more than the 256 registers a wave has at 8 waves per CU.
        auto rdBg = [&](const char* Bs, u32x4_t* b) {
#pragma unroll
          for (int j = 0; j < TN; ++j) b[j] = *(const u32x4_t*)(Bs + oB0 + j * 2048);
        };
        auto rdBu = [&](const char* Bs, u32x4_t* b) {
#pragma unroll
          for (int j = 0; j < TN; ++j) b[TN + j] = *(const u32x4_t*)(Bs + oB0 + BN * 128 + j * 2048);
        };
        auto rdB = [&](const char* Bs, u32x4_t* b, int kc) {
          const char* p = Bs + (kc ? oB1 : oB0);
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            b[j] = *(const u32x4_t*)(p + j * 2048);
            if constexpr (GATED) b[TN + j] = *(const u32x4_t*)(p + BN * 128 + j * 2048);
          }
        };
        if (nk > 1) wait_vmcnt<Cfg::LPS_B>();
        else wait_vmcnt<0>();
        block_barrier();
        u32x4_t b0[TN * NB], b1[TN * NB], a_cur, a_nxt;
        if constexpr (GATED) rdBg(b_slot(0), b0);
        else rdB(b_slot(0), b0, 0);
        a_cur = rdA(a_slot(0), 0, 0);
        for (int ks = 0; ks < nk; ++ks) {
          const char* As = a_slot(ks & 1);
          const char* Bs = b_slot(bs);
          const int bsn = bs == 2 ? 0 : bs + 1;
#pragma unroll
          for (int kc = 0; kc < 2; ++kc) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
              if (GATED && kc == 0 && i == 0) rdBu(Bs, b0);
              if (i + 1 < TM) {
                a_nxt = rdA(As, i + 1, kc);
              } else if (kc == 0) {
                rdB(Bs, b1, 1);
                a_nxt = rdA(As, 0, 1);
              } else if (ks + 1 < nk) {
                // every LDS read of step ks is issued: make step ks+1 visible and start reading it
                // while the last subtile row's MFMAs run
                if (ks + 2 < nk) wait_vmcnt<Cfg::LPS_B>();
                else wait_vmcnt<0>();
                block_barrier();
                if constexpr (GATED) rdBg(b_slot(bsn), b0);
                else rdB(b_slot(bsn), b0, 0);
                a_nxt = rdA(a_slot((ks + 1) & 1), 0, 0);
                __builtin_amdgcn_sched_barrier(0);
              }
              const u32x4_t* b = kc == 0 ? b0 : b1;
              if (!Cfg::SKIP_ROWS || wm * Cfg::WTM + i * 16 < rows) {
#pragma unroll
                for (int j = 0; j < TN; ++j) Mfma<T>::step(acc0[i][j], a_cur, b[j]);
                if constexpr (GATED) {
#pragma unroll
                  for (int j = 0; j < TN; ++j) Mfma<T>::step(acc1[i][j], a_cur, b[TN + j]);
                }
              }
              a_cur = a_nxt;
              if (kc == 0 && i == 0 && ks + 1 < nk)
                issue_a<Cfg>(a_slot((ks + 1) & 1), (uint32_t)(ks + 1) * KB_A, rsA, voffA, wave, lane);
              if (kc == 0 && i == TM - 1 && ks + 2 < nk) issue_w(bs == 0 ? 2 : bs - 1, ks + 2);
            }
          }
          bs = bsn;
        }
      } else {
        for (int ks = 0; ks < nk; ++ks) {
          if (ks + 1 < nk) wait_vmcnt<Cfg::LPS_B>();
          else wait_vmcnt<0>();
          block_barrier();                              // step ks visible; slots of ks-1 free
          compute(a_slot(ks & 1), b_slot(bs), [&](int part) {
            if (part == 0) {
              if (ks + 1 < nk) issue_a<Cfg>(a_slot((ks + 1) & 1), (uint32_t)(ks + 1) * KB_A, rsA, voffA, wave, lane);
            } else if (ks + 2 < nk) {
              issue_w(bs == 0 ? 2 : bs - 1, ks + 2);
            }
          });
          bs = bs == 2 ? 0 : bs + 1;
        }
      }
    }
    __syncthreads();                                    // LDS free for the next tile
    int nxt = 0;
    if (dyn && tid == 0) nxt = atomicAdd(args.tile_ctr + xcd, 1);

    if constexpr (EPI == 1)
      store_save_ab<Cfg>(args, acc0, acc1, wm, wn, lane, g, nt, row0, rows);
    else if constexpr (EPI == 2)
      store_dgrad<Cfg>(args, acc0, wm, wn, lane, g, nt, row0, rows);
    else
      store_tile<Cfg>(args, acc0, acc1, wm, wn, lane, g, nt, row0, rows, c_off);
    if (dyn) {
      // tiles [lo, lo + bpx) are the blocks' first ones; tickets number the rest in order
      if (tid == 0) *ticket = nxt;
      __syncthreads();
      Lnext = lo + bpx + *ticket;
    } else {
      Lnext = L + bpx;
    }
  }
}

}  // namespace moe
