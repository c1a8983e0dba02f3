// FP8 expert products on gfx950's scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4).
//
// The pages keep expert weights in one byte per parameter (jacopoparretti.dev, "Memory": the
// DeepSeek-V3 weights ship in FP8) or in MXFP4 (AI Engineering Illustrated, "Total parameters
// and active parameters are different budgets").  In this mode the activations that meet them
// are OCP MXFP8 as well -- E4M3 elements, one E8M0 scale per 32 consecutive elements along the
// contraction -- so both operands of every product are 8-bit (or 4-bit) and the products run on
// the scaled MFMA, which applies the per-32 scales of both operands itself: twice the bf16 rate
// for FP8 x FP8 and half the operand bytes per product.
//
// Operand layout of the 16x16x128 instruction (checked on the hardware): lane 16 g + r holds row
// r of A (column r of B); an 8-bit operand's bytes 0-15 are K = 16 g .. 16 g + 15 and bytes
// 16-31 are K = 64 + 16 g .. 64 + 16 g + 15; a 4-bit operand's 16 bytes are K = 32 g .. 32 g + 31
// (low nibble first); byte 0 of the scale register of lane 16 b + r is the E8M0 scale of K block
// b (K = 32 b .. 32 b + 31) of that row (column).  An LDS row of 128 activation bytes (one K step)
// therefore feeds lane group g with its 16-byte pieces g and 4 + g.
//
// Kernel structure as grouped_gemm_kernel.h: persistent XCD-aware tile order, global -> LDS by
// buffer loads straight into a ring of LDS stages (one MFMA K of 128 per stage), equal load
// shares per wave so vmcnt waits keep a fixed number of stages in flight.  Each stage holds the
// activation codes, their scales (4 bytes per row), the weight codes and, for MXFP4 weights,
// their scales.  The gate/up epilogue forms h = SiLU(a) * b and writes it as MXFP8: the block
// maximum over 32 columns comes from a 16-lane max (DPP rotations) across the lanes holding the
// block, then the scale code and the saturated E4M3 codes.
#include "grouped_gemm_kernel.h"

namespace moe {

typedef int32_t i32x8_t __attribute__((ext_vector_type(8)));

// ------------------------------------------------------------------------------ MXFP8 helpers

// E8M0 code of an MX block whose largest magnitude is m: floor(log2 m) - 8 + 127 from the
// biased fp32 exponent, clamped at 0 (zero, fp32-subnormal and very small blocks get 2^-127).
__device__ __forceinline__ uint32_t mx_scale_code(float m) {
  const int ef = (int)((__float_as_uint(m) >> 23) & 0xffu);
  return (uint32_t)max(0, ef - 8);
}

// 2^(127 - code), the factor that takes the block to E4M3 range (exact for codes 0 .. 253).
__device__ __forceinline__ float mx_inv_scale(uint32_t code) { return __uint_as_float((254u - code) << 23); }

// Two values as E4M3 codes (nearest even), saturated at +-448, in bits 0-7 and 8-15.
__device__ __forceinline__ uint32_t e4m3x2_sat(float a, float b) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// Largest value over the 16 lanes of a DPP row (lanes 16 q .. 16 q + 15), in every lane.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x121, 0xf, 0xf, false)));  // ror 1
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x122, 0xf, 0xf, false)));  // ror 2
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x124, 0xf, 0xf, false)));  // ror 4
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false)));  // ror 8
  return v;
}

// One thread per block of 32 consecutive elements of the flat array x [rows, K] (K a multiple
// of 32, so a block never crosses a row): codes and the block's scale byte.
__global__ __launch_bounds__(256) void mxfp8_quantize_kernel(const uint16_t* __restrict__ x, long long nblk,
                                                             uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const long long b = (long long)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblk) return;
  const uint4* src = (const uint4*)(x + b * 32);
  float v[32];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint4 w = src[p];
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      v[8 * p + 2 * h] = bf16_bits_to_f32(u[h] & 0xffffu);
      v[8 * p + 2 * h + 1] = bf16_bits_to_f32(u[h] >> 16);
    }
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(v[i]));
  const uint32_t c = mx_scale_code(m);
  const float inv = mx_inv_scale(c);
  uint32_t w[8];
#pragma unroll
  for (int q = 0; q < 8; ++q)
    w[q] = e4m3x2_sat(v[4 * q] * inv, v[4 * q + 1] * inv) | (e4m3x2_sat(v[4 * q + 2] * inv, v[4 * q + 3] * inv) << 16);
  uint4* dst = (uint4*)(codes + b * 32);
  dst[0] = uint4{w[0], w[1], w[2], w[3]};
  dst[1] = uint4{w[4], w[5], w[6], w[7]};
  scales[b] = (uint8_t)c;
}

hipError_t launch_mxfp8_quantize(const void* x, int rows, int K, uint8_t* codes, uint8_t* scales,
                                 hipStream_t stream) {
  if (K % 32 != 0 || rows < 0) return hipErrorInvalidValue;
  const long long nblk = (long long)rows * (K / 32);
  if (nblk == 0) return hipSuccess;
  hipLaunchKernelGGL(mxfp8_quantize_kernel, dim3((unsigned)((nblk + 255) / 256)), dim3(256), 0, stream,
                     (const uint16_t*)x, nblk, codes, scales);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------ tile configuration

// WF: weight format, 1 = E4M3 with fp32 row scales (the MFMA's weight scale is 1; the row
// scale multiplies the accumulator), 2 = MXFP4 (the MFMA applies the E8M0 block scales).
template <int BM, int BN, int WM, int WN, bool GATED, int STAGES, int WF>
struct MxTile {
  using Elem = uint8_t;
  static constexpr int WF_ = WF;
  static constexpr int NW = WM * WN, NT = NW * kWave;
  static constexpr int BM_ = BM, BN_ = BN;
  static constexpr int WTM = BM / WM, WTN = BN / WN, TM = WTM / 16, TN = WTN / 16;
  static constexpr int NB = GATED ? 2 : 1, BROWS = BN * NB;
  static constexpr int KS = 128;                               // contraction elements per stage
  static constexpr int PPR_B = WF == 2 ? 4 : 8;                // 16-byte weight pieces per row per stage
  static constexpr int KB_B = PPR_B * 16;                      // weight bytes per row per stage
  static constexpr int A_BYTES = BM * 128, AS_BYTES = BM * 4;
  static constexpr int B_BYTES = BROWS * KB_B, BS_BYTES = WF == 2 ? 4 * BROWS : 0;
  static constexpr int SLOT = A_BYTES + AS_BYTES + B_BYTES + BS_BYTES;
  static constexpr int LDS = STAGES * SLOT;
  static constexpr int LDS_ALLOC = LDS;
  // global -> LDS pieces per stage: activation codes (16 B), activation scales (4 B per row),
  // weight codes (16 B), MXFP4 weight scales (16 B = one block's scales of 16 rows)
  static constexpr int P_A = BM * 8, P_AS = BM, P_B = BROWS * PPR_B, P_BS = BS_BYTES / 16;
  static constexpr int PW_A = P_A / NW, PW_AS = P_AS / NW, PW_B = P_B / NW, PW_BS = P_BS / NW;
  static constexpr int IT_A = (PW_A + kWave - 1) / kWave, IT_AS = (PW_AS + kWave - 1) / kWave;
  static constexpr int IT_B = (PW_B + kWave - 1) / kWave, IT_BS = P_BS ? (PW_BS + kWave - 1) / kWave : 0;
  static constexpr int LPS = IT_A + IT_AS + IT_B + IT_BS;
  static_assert(P_A % NW == 0 && P_AS % NW == 0 && P_B % NW == 0 && P_BS % NW == 0, "equal shares per wave");
  static_assert(NW % 2 == 0 || !GATED, "gate and up halves of the weight pieces split on a wave boundary");
  static_assert(P_BS == 0 || (4 * BN / 16) % PW_BS == 0, "a wave's weight-scale share lies in one matrix");
  static_assert(!GATED || WTN % 32 == 0, "an MX block of h (32 columns) lies inside one wave");
  static_assert(WTM % 16 == 0 && WTN % 16 == 0, "whole 16x16 MFMA tiles");
  static_assert(SLOT % 16 == 0 && LDS <= 160 * 1024, "LDS per workgroup");
  static_assert(LPS * (STAGES - 2) <= 63, "vmcnt range");
  static constexpr bool SKIP_ROWS = BM != 256;
};

// Enqueue `IT` load instructions of `size`-byte pieces: wave w loads pieces [w PW, (w+1) PW) of
// the kind (lane L of an instruction writes LDS bytes base + size L .. + size).
template <int IT, int PW, int SIZE>
__device__ __forceinline__ void mx_issue(char* dst, uint32_t kb, __amdgpu_buffer_rsrc_t rs, const uint32_t* voff,
                                         int wave, int lane) {
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int q0 = wave * PW + it * kWave;
    if (PW % kWave == 0 || it * kWave + lane < PW) {
      auto* d = (__attribute__((address_space(3))) void*)(dst + q0 * SIZE);
      if constexpr (SIZE == 4)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 4, voff[it], kb, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, d, 16, voff[it], kb, 0, 0);
    }
  }
}

template <int BM, int BN, int WM, int WN, bool GATED, int STAGES, int WF>
__global__ __launch_bounds__(WM* WN * 64) void grouped_gemm_mx_kernel(GemmArgs args) {
  using Cfg = MxTile<BM, BN, WM, WN, GATED, STAGES, WF>;
  constexpr int TM = Cfg::TM, TN = Cfg::TN, NB = Cfg::NB;
  extern __shared__ __align__(16) char lds[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int N = args.N, K = args.K;
  const int ntn = N / BN;
  const int mt_live = args.offsets ? args.tstart[args.G] : (args.dense_rows + BM - 1) / BM;
  const int live = mt_live * ntn;
  const int xcd = blockIdx.x % kNumXcd, j0 = blockIdx.x / kNumXcd, bpx = gridDim.x / kNumXcd;
  const int lo = (int)((long long)live * xcd / kNumXcd);
  const int hi = (int)((long long)live * (xcd + 1) / kNumXcd);
  const int nk = K / Cfg::KS;
  const size_t rowb_a = (size_t)K;                             // activation code bytes per row
  const size_t rows_a = (size_t)K / 32;                        // activation scale bytes per row
  const size_t rowb_b = WF == 2 ? (size_t)K / 2 : (size_t)K;   // weight code bytes per row
  const int g4 = lane >> 4, r16 = lane & 15;

  for (int L = lo + j0; L < hi; L += bpx) {
    const TileCoord tc = tile_coord(args, L, ntn, mt_live, bpx, BM);
    const int g = tc.g, nt = tc.nt, row0 = tc.row0, rows = tc.rows;
    const size_t brow0 = (size_t)g * N + (size_t)nt * BN;
    const char* Ab = (const char*)args.A + (args.a_rows ? 0 : (size_t)row0 * rowb_a);
    const char* ASb = (const char*)args.a_scales + (args.a_rows ? 0 : (size_t)row0 * rows_a);
    const char* B0b = (const char*)args.B0 + brow0 * rowb_b;
    const char* B1b = GATED ? (const char*)args.B1 + brow0 * rowb_b : B0b;
    const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc((void*)Ab, 0, kBufRange, kBufFlags);
    const __amdgpu_buffer_rsrc_t rsAS = __builtin_amdgcn_make_buffer_rsrc((void*)ASb, 0, kBufRange, kBufFlags);
    const __amdgpu_buffer_rsrc_t rsB0 = __builtin_amdgcn_make_buffer_rsrc((void*)B0b, 0, kBufRange, kBufFlags);
    const __amdgpu_buffer_rsrc_t rsB1 = __builtin_amdgcn_make_buffer_rsrc((void*)B1b, 0, kBufRange, kBufFlags);
    __amdgpu_buffer_rsrc_t rsS0 = rsB0, rsS1 = rsB1;
    if constexpr (WF == 2) {                                   // E8M0 [G, K/32, N]: base at block 0, column nt BN
      const size_t sb = (size_t)g * (K / 32) * N + (size_t)nt * BN;
      rsS0 = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)args.S0 + sb), 0, kBufRange, kBufFlags);
      rsS1 = GATED ? __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)args.S1 + sb), 0, kBufRange, kBufFlags)
                   : rsS0;
    }
    // per-lane offsets of this tile's pieces; rows past `rows` repeat the last valid row
    uint32_t voffA[Cfg::IT_A], voffAS[Cfg::IT_AS > 0 ? Cfg::IT_AS : 1], voffB[Cfg::IT_B];
    uint32_t voffBS[Cfg::IT_BS > 0 ? Cfg::IT_BS : 1];
#pragma unroll
    for (int it = 0; it < Cfg::IT_A; ++it) {
      const int q = min(wave * Cfg::PW_A + it * kWave + lane, Cfg::P_A - 1);
      const int r = q >> 3, cl = (q & 7) ^ ((r >> 1) & 7);
      const int rr = min(r, rows - 1);
      const size_t arow = args.a_rows ? (size_t)args.a_rows[row0 + rr] : (size_t)rr;
      voffA[it] = (uint32_t)(arow * rowb_a + cl * 16);
    }
#pragma unroll
    for (int it = 0; it < Cfg::IT_AS; ++it) {
      const int r = min(wave * Cfg::PW_AS + it * kWave + lane, Cfg::P_AS - 1);
      const int rr = min(r, rows - 1);
      const size_t arow = args.a_rows ? (size_t)args.a_rows[row0 + rr] : (size_t)rr;
      voffAS[it] = (uint32_t)(arow * rows_a);
    }
#pragma unroll
    for (int it = 0; it < Cfg::IT_B; ++it) {
      const int q = min(wave * Cfg::PW_B + it * kWave + lane, Cfg::P_B - 1);
      const int r = q / Cfg::PPR_B, p = q % Cfg::PPR_B;
      const int cl = Cfg::PPR_B == 8 ? p ^ ((r >> 1) & 7) : p ^ ((r >> 1) & 3);
      voffB[it] = (uint32_t)((NB == 2 && r >= BN ? r - BN : r) * rowb_b + cl * 16);
    }
    if constexpr (Cfg::IT_BS > 0) {
      constexpr int PPM = 4 * BN / 16;                          // scale pieces per matrix per stage
#pragma unroll
      for (int it = 0; it < Cfg::IT_BS; ++it) {
        const int q = min(wave * Cfg::PW_BS + it * kWave + lane, Cfg::P_BS - 1);
        const int qm = q % PPM, b = qm / (BN / 16), p16 = qm % (BN / 16);
        voffBS[it] = (uint32_t)(b * N + p16 * 16);
      }
    }
    const bool up_w = NB == 2 && wave >= Cfg::NW / 2;           // this wave's weight share is W_u's
    const bool up_s = NB == 2 && wave * Cfg::PW_BS >= 4 * BN / 16;
    auto slot = [&](int s) { return lds + s * Cfg::SLOT; };
    // part 0: the activations and their scales, part 1: the weights and theirs, 2: both
    auto issue = [&](int s, int ks, int part) {
      char* sl = slot(s);
      if (part != 1) {
        mx_issue<Cfg::IT_A, Cfg::PW_A, 16>(sl, (uint32_t)ks * 128, rsA, voffA, wave, lane);
        mx_issue<Cfg::IT_AS, Cfg::PW_AS, 4>(sl + Cfg::A_BYTES, (uint32_t)ks * 4, rsAS, voffAS, wave, lane);
      }
      if (part == 0) return;
      mx_issue<Cfg::IT_B, Cfg::PW_B, 16>(sl + Cfg::A_BYTES + Cfg::AS_BYTES, (uint32_t)ks * Cfg::KB_B,
                                         up_w ? rsB1 : rsB0, voffB, wave, lane);
      if constexpr (Cfg::IT_BS > 0)
        mx_issue<Cfg::IT_BS, Cfg::PW_BS, 16>(sl + Cfg::A_BYTES + Cfg::AS_BYTES + Cfg::B_BYTES,
                                             (uint32_t)ks * 4 * (uint32_t)N, up_s ? rsS1 : rsS0, voffBS, wave, lane);
    };

    f32x4_t acc0[TM][TN], acc1[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        acc0[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        acc1[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }

    // One stage = one 128-element K step: A fragments (two 16-byte pieces per lane) and their
    // scale words once, then per weight subtile its fragment and scale and the MFMAs.
    // hook(0) and hook(1) run once each, in that order: after the first weight subtile's MFMAs
    // and after the first half of them.
    auto compute = [&](const char* sl, auto&& hook) {
      const char* As = sl;
      const char* ASs = sl + Cfg::A_BYTES;
      const char* Bs = sl + Cfg::A_BYTES + Cfg::AS_BYTES;
      const char* BSs = Bs + Cfg::B_BYTES;
      i32x8_t a[TM];
      int sa[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int r = wm * Cfg::WTM + i * 16 + r16;
        const u32x4_t lo4 = *(const u32x4_t*)(As + swz(r, g4));
        const u32x4_t hi4 = *(const u32x4_t*)(As + swz(r, 4 + g4));
        a[i] = i32x8_t{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3], (int)hi4[0], (int)hi4[1], (int)hi4[2],
                       (int)hi4[3]};
        sa[i] = (int)(*(const uint32_t*)(ASs + r * 4) >> (8 * g4));   // byte 0: block g4 of row r
      }
#pragma unroll
      for (int m = 0; m < NB; ++m)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int rm = wn * Cfg::WTN + j * 16 + r16;         // weight row in its matrix
          const int rb = m * BN + rm;
          i32x8_t b;
          int sb;
          if constexpr (WF == 2) {
            const u32x4_t v = *(const u32x4_t*)(Bs + rb * 64 + ((g4 ^ ((rb >> 1) & 3)) << 4));
            b = i32x8_t{(int)v[0], (int)v[1], (int)v[2], (int)v[3], 0, 0, 0, 0};
            sb = (int)*(const uint8_t*)(BSs + (m * 4 + g4) * BN + rm);
          } else {
            const u32x4_t lo4 = *(const u32x4_t*)(Bs + swz(rb, g4));
            const u32x4_t hi4 = *(const u32x4_t*)(Bs + swz(rb, 4 + g4));
            b = i32x8_t{(int)lo4[0], (int)lo4[1], (int)lo4[2], (int)lo4[3], (int)hi4[0], (int)hi4[1], (int)hi4[2],
                        (int)hi4[3]};
            sb = 127;                                          // 2^0: the row scale comes in the epilogue
          }
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            if (!Cfg::SKIP_ROWS || wm * Cfg::WTM + i * 16 < rows) {
              if (m == 0)
                acc0[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i], b, acc0[i][j], 0, WF == 2 ? 4 : 0,
                                                                              0, sa[i], 0, sb);
              else
                acc1[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[i], b, acc1[i][j], 0, WF == 2 ? 4 : 0,
                                                                              0, sa[i], 0, sb);
            }
          }
          if (m == 0 && j == 0) hook(0);
          if (m * TN + j == (NB * TN / 2 > 1 ? NB * TN / 2 - 1 : 0)) hook(1);
        }
    };

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");           // previous tile's stores drained
#pragma unroll
    for (int p = 0; p < STAGES - 1; ++p)
      if (p < nk) issue(p, p, 2);
    int sl = 0;
    for (int ks = 0; ks < nk; ++ks) {
      wait_stage<Cfg::LPS, STAGES>(min(STAGES - 2, nk - 1 - ks));   // step ks has landed
      block_barrier();                                          // ... for every wave; slot ks-1 is free
      // With a ring of 3 or more the step's loads start between its MFMAs, activations first
      // (MXFP4 prefill gate/up 0.975 -> 0.945 ms); a 2-slot ring needs them straight after the
      // barrier to land within one step (FP8: 1.04 against 1.08 ms when spread).
      const bool more = ks + STAGES - 1 < nk;
      const int fs = sl == 0 ? STAGES - 1 : sl - 1;
      if constexpr (STAGES >= 3) {
        compute(slot(sl), [&](int part) {
          if (more) issue(fs, ks + STAGES - 1, part);
        });
      } else {
        if (more) issue(fs, ks + STAGES - 1, 2);
        compute(slot(sl), [](int) {});
      }
      sl = sl + 1 == STAGES ? 0 : sl + 1;
    }
    __syncthreads();                                            // LDS free for the next tile

    if constexpr (GATED) {
      // h = SiLU(a) * b as MXFP8: per row, the 32 columns of subtiles 2p and 2p+1 form one block
      uint8_t* Hq = (uint8_t*)args.C;
      const int cw = nt * BN + wn * Cfg::WTN;                   // first column of this wave
      // FP8 row scales of the lane's columns, loaded once (interleaved with the stores, each
      // load would wait for the one before)
      float sg[WF == 1 ? TN : 1], su[WF == 1 ? TN : 1];
      if constexpr (WF == 1) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const size_t sc = (size_t)g * N + cw + j * 16 + r16;
          sg[j] = ((const float*)args.S0)[sc];
          su[j] = ((const float*)args.S1)[sc];
        }
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = wm * Cfg::WTM + i * 16 + g4 * 4 + q;
          const bool valid = r < rows;
          const size_t ro = (size_t)(row0 + (valid ? r : 0));
#pragma unroll
          for (int p = 0; p < TN / 2; ++p) {
            float h[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int j = 2 * p + e;
              float av = acc0[i][j][q], bv = acc1[i][j][q];
              if constexpr (WF == 1) {
                av *= sg[j];
                bv *= su[j];
              }
              h[e] = silu_mul(av, bv);
            }
            const float mb = row16_max(fmaxf(fabsf(h[0]), fabsf(h[1])));
            const uint32_t c = mx_scale_code(mb);
            const float inv = mx_inv_scale(c);
            const uint32_t q2 = e4m3x2_sat(h[0] * inv, h[1] * inv);
            if (valid) {
              uint8_t* dst = Hq + ro * N + cw + 32 * p + r16;
              dst[0] = (uint8_t)(q2 & 0xffu);
              dst[16] = (uint8_t)(q2 >> 8);
              if (r16 == 0) args.c_scales[ro * (size_t)(N / 32) + (cw >> 5) + p] = (uint8_t)c;
            }
          }
        }
    } else {
      store_tile<Cfg>(args, acc0, acc1, wm, wn, lane, g, nt, row0, rows);
    }
  }
}

// ------------------------------------------------------------------------------ launch

int gemm_block_m_mx(GemmKind kind) { return kind == kGemmLarge ? 256 : (kind == kGemmStream ? 128 : 16); }

template <int BM, int BN, int WM, int WN, bool GATED, int STAGES, int WF>
static hipError_t launch_mx(const GemmArgs& a, int max_tiles_m, hipStream_t stream) {
  return launch_kernel<MxTile<BM, BN, WM, WN, GATED, STAGES, WF>,
                       grouped_gemm_mx_kernel<BM, BN, WM, WN, GATED, STAGES, WF>>(a, max_tiles_m, stream);
}

// Tile configurations: large (many rows per expert) 256 x 128 (gate/up) or 256 x 256, 8 waves;
// stream 128 x 128 / 128 x 256, 8 waves; decode 16 x 64 / 16 x 32, 2 waves.  MXFP4 weights take
// half the LDS, so their large tiles keep three stages.
template <bool GATED, int WF>
static hipError_t dispatch_mx(GemmKind kind, const GemmArgs& a, int max_tiles_m, hipStream_t s) {
  constexpr int LS = WF == 2 ? 3 : 2;
  switch (kind) {
    case kGemmLarge:
      if constexpr (GATED) return launch_mx<256, 128, 4, 2, true, LS, WF>(a, max_tiles_m, s);
      else if (a.N % 256 == 0) return launch_mx<256, 256, 4, 2, false, LS, WF>(a, max_tiles_m, s);
      else return launch_mx<256, 128, 4, 2, false, LS, WF>(a, max_tiles_m, s);
    case kGemmStream:
      if constexpr (GATED) return launch_mx<128, 128, 2, 4, true, 3, WF>(a, max_tiles_m, s);
      else if (a.N % 256 == 0) return launch_mx<128, 256, 2, 4, false, 3, WF>(a, max_tiles_m, s);
      else return launch_mx<128, 128, 2, 4, false, 3, WF>(a, max_tiles_m, s);
    default:
      if constexpr (GATED) return launch_mx<16, 64, 1, 2, true, 4, WF>(a, max_tiles_m, s);
      else return launch_mx<16, 32, 1, 2, false, 4, WF>(a, max_tiles_m, s);
  }
}

hipError_t launch_gemm_gateup_mx(GemmKind kind, int wfmt, const uint8_t* A, const uint8_t* As, const int32_t* a_rows,
                                 const void* Wg, const void* Wu, const void* Sg, const void* Su,
                                 const int32_t* offsets, const int32_t* tstart, int G, int dense_rows,
                                 int max_tiles_m, int N, int K, uint8_t* Hq, uint8_t* Hs, hipStream_t stream) {
  if (K % 128 != 0 || N % 128 != 0) return hipErrorInvalidValue;
  GemmArgs a{A, a_rows, Wg, Wu, (const float*)Sg, (const float*)Su, offsets, tstart, G, dense_rows, N, K, Hq};
  a.a_scales = As;
  a.c_scales = Hs;
  if (wfmt == 1) return dispatch_mx<true, 1>(kind, a, max_tiles_m, stream);
  if (wfmt == 2) return dispatch_mx<true, 2>(kind, a, max_tiles_m, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_down_mx(GemmKind kind, int wfmt, const uint8_t* Hq, const uint8_t* Hs, const void* Wd,
                               const void* Sd, const int32_t* offsets, const int32_t* tstart, int G, int dense_rows,
                               int max_tiles_m, int N, int K, float* O, hipStream_t stream) {
  if (K % 128 != 0 || N % 128 != 0) return hipErrorInvalidValue;
  GemmArgs a{Hq, nullptr, Wd, nullptr, (const float*)Sd, nullptr, offsets, tstart, G, dense_rows, N, K, O};
  a.a_scales = Hs;
  if (wfmt == 1) return dispatch_mx<false, 1>(kind, a, max_tiles_m, stream);
  if (wfmt == 2) return dispatch_mx<false, 2>(kind, a, max_tiles_m, stream);
  return hipErrorInvalidValue;
}

}  // namespace moe
