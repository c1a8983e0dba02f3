// Shared device helpers for the gfx950 MoE kernels: element types, bf16 rounding,
// the 16x16 MFMA step on 16-byte operand pieces, and wavefront reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;      // CDNA wavefront width
constexpr int kNumXcd = 8;     // MI355X: 8 accelerator complex dies, one L2 each

// bf16 is stored as raw 16-bit patterns (uint16_t); fp32 as float.
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// Round to nearest even (gfx950's v_cvt_pk_bf16_f32); NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two floats rounded to bf16 (nearest even) in one instruction: lo in bits 0-15, hi in 16-31.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2_bits(float lo, float hi) {
  typedef float f2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 b2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2_t{lo, hi}), b2_t));
}

// sigmoid(a) = 1 / (1 + e^-a) from the hardware's exp2 and reciprocal (about 1 ulp each; the
// products round their results to bf16 or keep fp32 partials, so this is far below the
// rounding that follows).
__device__ __forceinline__ float sigmoid_fast(float a) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(a * -1.4426950408889634f));
}

// h = SiLU(a) * b = a * b * sigmoid(a).  Every kernel that forms h (the forward's gate/up
// epilogue and the backward's recompute and down-product epilogues) calls this one function,
// so they all round the same h.
__device__ __forceinline__ float silu_mul(float a, float b) { return (a * b) * sigmoid_fast(a); }

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1.  Used where an
// accumulator array is indexed inside a loop body too large for the unroller: a loop left
// rolled would index the array with a run-time value and move it to scratch memory.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

template <typename T> struct ElemOut;
template <> struct ElemOut<uint16_t> {
  __device__ __forceinline__ static uint16_t from_f32(float v) { return (uint16_t)f32_to_bf16_bits(v); }
  __device__ __forceinline__ static float to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
};
template <> struct ElemOut<float> {
  __device__ __forceinline__ static float from_f32(float v) { return v; }
  __device__ __forceinline__ static float to_f32(float v) { return v; }
};

// One 16x16 output tile step over 64 bytes of the contraction dimension.
// Operand layout: lane l supplies 16 contiguous bytes of A row (l % 16) and of
// B column (l % 16), taken from 16-byte piece (l / 16) of the 64-byte K chunk.
// A and B use the same lane -> k mapping, so the tile gets sum over all 64 bytes'
// worth of k of A[row][k] * B[k][col] whatever order the unit sums them in.
// Result layout (both element types): lane l holds D[4 * (l / 16) + i][l % 16].
template <typename T> struct Mfma;
template <> struct Mfma<uint16_t> {           // bf16: one 16x16x32 instruction
  static constexpr int kElemsPerPiece = 8;
  __device__ __forceinline__ static void step(f32x4_t& acc, const u32x4_t& a, const u32x4_t& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
};
template <> struct Mfma<float> {              // fp32: four 16x16x4 instructions
  static constexpr int kElemsPerPiece = 4;
  __device__ __forceinline__ static void step(f32x4_t& acc, const u32x4_t& a, const u32x4_t& b) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[i]), __uint_as_float(b[i]), acc, 0, 0, 0);
  }
};

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Butterfly sum: every lane ends with the same value, and the association order is
// fixed, so the result is reproducible run to run.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Exclusive prefix sum over a block of exactly 1024 threads (Hillis-Steele in LDS).
// `scratch` holds 1024 ints.  Returns the exclusive prefix; *total gets the sum.
__device__ __forceinline__ int block1024_exclusive_scan(int v, int* scratch, int* total) {
  const int tid = threadIdx.x;
  scratch[tid] = v;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int add = tid >= off ? scratch[tid - off] : 0;
    __syncthreads();
    scratch[tid] += add;
    __syncthreads();
  }
  int incl = scratch[tid];
  *total = scratch[1023];
  __syncthreads();
  return incl - v;
}

}  // namespace moe
