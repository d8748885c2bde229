// attn_device.hpp -- device-side building blocks shared by the attention kernels (gfx950).
//
// Matrix-core conventions used throughout.  A wave (64 lanes) owns one 32x32 fp32 tile held in
// the accumulator layout of the 32x32 MFMA family: lane l = col + 32 * half holds column `col`
// and, in register v (0..15), row acc_row(v, half) = 8 * (v / 4) + 4 * half + v % 4.  For the
// fp32 MFMA 32x32x2 the A operand of lane l is A[row = col][k = half] and the B operand is
// B[k = half][column = col].
//
// Because every tile a wave owns keeps one query (or one key) per column, per-row softmax
// statistics are per-lane scalars, and the probability tile can feed the next MFMA's B operand
// straight from the accumulator registers: step v of a contraction over the tile's rows uses
// register v, whose row index is acc_row(v, half).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ne {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
// Finite stand-in for -inf as the initial running maximum: exp2 of (this - finite) is 0 and
// (this - this) is 0, so no NaN appears before the first visible key.
constexpr float kNegBig = -1.0e30f;

__device__ __forceinline__ int acc_row(int v, int half) { return 8 * (v >> 2) + 4 * half + (v & 3); }

__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// exp2 on the transcendental unit; exact 0 for -inf.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of lane (l ^ 32): exchanges the two halves of the wave.
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32, 64); }

__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ void st4(float *p, f32x4 v) { *reinterpret_cast<f32x4 *>(p) = v; }

}  // namespace ne
