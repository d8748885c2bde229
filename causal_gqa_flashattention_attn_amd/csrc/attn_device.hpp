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

#include <type_traits>

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

// f(std::integral_constant<int, I>) for I = 0 .. N-1, each with I a compile-time constant.
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

__device__ __forceinline__ f32x4 ld4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }
__device__ __forceinline__ void st4(float *p, f32x4 v) { *reinterpret_cast<f32x4 *>(p) = v; }

}  // namespace ne

// ---------------------------------------------------------------------------------------------
// bfloat16 building blocks (v_mfma_f32_32x32x16_bf16).  A operand of lane l: A[row = l % 32]
// [k = 8 * (l / 32) .. + 7]; B operand: B[k = 8 * (l / 32) .. + 7][column = l % 32]; the f32
// accumulator has the same layout as the fp32 32x32 family above.
namespace ne {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mfma32_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row-major bf16 tiles in LDS, rows of D elements, 16-byte chunks permuted within each row.
// The LDS serves 256 bytes (64 banks) per cycle and a 16-byte read 16 lanes per cycle, so a
// pattern is conflict-free when the 16 lanes of each group hit 16 distinct 16-byte slots modulo
// 256 bytes.  The permutations below make three patterns conflict-free (measured with the LDS
// bank-conflict counter for D = 32, 64): 16-byte reads of one chunk from 16 consecutive rows,
// the transposed read below (32 lanes: 4 consecutive rows x 64 contiguous bytes), and staging
// writes where 16 lanes fill one (D = 128), two (D = 64) or four (D = 32) whole rows.
//   D = 128 (256-byte rows): chunk c of row r is stored at c ^ (4 (r & 3) + ((r >> 2) & 3)):
//          16 consecutive rows take 16 distinct values, and the 4 rows of a transposed read
//          land in 4 distinct groups of 4 chunks.
//   D = 64 (128-byte rows): chunk c of row r is stored at c ^ f(r),
//          f(r) = 2 * (((r & 3) + ((r >> 2) & 3)) & 3) + ((r >> 3) & 1).
//   D = 32 (64-byte rows):  chunk c of row r is stored at c ^ ((r >> 2) & 3).
// Every permutation repeats every 16 rows.
template <int D>
__host__ __device__ __forceinline__ constexpr int chunk_swizzle(int row, int ch) {
    if constexpr (D == 128) return ch ^ (4 * (row & 3) + ((row >> 2) & 3));
    else if constexpr (D == 64) return ch ^ (2 * (((row & 3) + ((row >> 2) & 3)) & 3) + ((row >> 3) & 1));
    else return ch ^ ((row >> 2) & 3);
}

// Copies that fill a tile 1024 bytes at a time cover rows [p R, p R + R) with piece p, R = 1024 /
// (2 D).  The chunk permutation of row p R + r is that of row r XOR'd with a constant that only
// depends on p; swizzle_piece_xor gives it (D = 128: p & 3; D = 64: 5 for odd p; D = 32: 0).
template <int D>
__host__ __device__ constexpr int swizzle_piece_xor(int p) {
    return D == 128 ? (p & 3) : D == 64 ? 5 * (p & 1) : 0;
}
template <int D>
constexpr bool swizzle_piece_xor_holds() {
    constexpr int R = 1024 / (2 * D);
    for (int p = 0; p < 32; ++p)
        for (int r = 0; r < R; ++r)
            for (int c = 0; c < D / 8; ++c)
                if (chunk_swizzle<D>(p * R + r, c) != (chunk_swizzle<D>(r, c) ^ swizzle_piece_xor<D>(p)))
                    return false;
    return true;
}
// Each row's permutation is a bijection of its chunks.
template <int D>
constexpr bool swizzle_is_permutation() {
    for (int r = 0; r < 16; ++r) {
        unsigned seen = 0;
        for (int c = 0; c < D / 8; ++c) seen |= 1u << chunk_swizzle<D>(r, c);
        if (seen != (D / 8 == 32 ? 0xffffffffu : (1u << (D / 8)) - 1)) return false;
    }
    return true;
}
static_assert(swizzle_piece_xor_holds<128>() && swizzle_piece_xor_holds<64>() &&
                  swizzle_piece_xor_holds<32>(),
              "piece permutation depends on more than swizzle_piece_xor gives");
static_assert(swizzle_is_permutation<128>() && swizzle_is_permutation<64>() &&
                  swizzle_is_permutation<32>(),
              "chunk swizzle is not a permutation");

// Byte offset of element (row, col) in a swizzled tile; col must be a multiple of 4.
template <int D>
__device__ __forceinline__ int tile_off(int row, int col) {
    return row * (2 * D) + 16 * chunk_swizzle<D>(row, col >> 3) + 2 * (col & 7);
}

// The 8 consecutive elements (row, col .. col+7) of a swizzled tile; col a multiple of 8.
template <int D>
__device__ __forceinline__ bf16x8 tile_read8(const unsigned char *t, int row, int col) {
    return *reinterpret_cast<const bf16x8 *>(t + tile_off<D>(row, col));
}

// Transposed read (ds_read_b64_tr_b16) at LDS byte address addr + OFF (OFF < 65536, an
// immediate of the instruction), for addresses precomputed by tr4_lane_addr: lane l receives
// M[k0 + 4 * (l / 32) + j][c0 + l % 32] for j = 0..3 (within each group of 16 lanes, lane i
// takes element i % 4 of the 8-byte pieces addressed by lanes i / 4 + 4 j).  It is issued as
// inline assembly: for tiles that LDS copies (dma16) fill, the compiler would make the intrinsic
// wait for every copy in flight, since it cannot rule out that they alias; it knows nothing of
// this form, so the caller must pass the result through lds_wait_n before using it.
template <int OFF>
__device__ __forceinline__ bf16x4 lds_read_tr4(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "LDS immediate offset out of range");
    bf16x4 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
    return r;
}

// LDS byte address of this lane's transposed read of rows k0 .. k0 + 3 (k0 a multiple of 4 below
// 16), columns c0 .. of the swizzled tile at `t`.  The chunk permutation repeats every 16 rows,
// so rows k0 + 16 j are read at this address plus 16 j rows.
template <int D>
__device__ __forceinline__ uint32_t tr4_lane_addr(const unsigned char *t, int k0, int c0, int lane) {
    const int row = k0 + 4 * (lane >> 5) + ((lane & 15) >> 2);
    const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    typedef __attribute__((address_space(3))) const unsigned char lds_u8;
    return (uint32_t)(uintptr_t)(lds_u8 *)(t + tile_off<D>(row, col));
}

// s_waitcnt lgkmcnt(N): waits until at most N of this wave's LDS operations are outstanding.
// They complete in order, so a read followed by N or more later LDS operations of the wave
// has landed.  a and b pass through the wait, so nothing that uses them moves above it.  The
// counter field holds at most 15; a larger N waits for 15, which still covers the read.
template <int N>
__device__ __forceinline__ void lds_wait_n(bf16x4 &a, bf16x4 &b) {
    static_assert(N >= 0, "negative wait count");
    asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "n"(N < 15 ? N : 15));
}

__device__ __forceinline__ bf16x8 join8(const bf16x4 &lo, const bf16x4 &hi) {
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Reductions over the two halves of the wave (lanes l and l ^ 32), result in every lane.
// v_permlane32_swap(a, b) returns {[a_lo, b_lo], [a_hi, b_hi]} (32-lane halves), so with a = b = x
// the two results hold x_lo and x_hi in every lane; both halves combine them in the same order.
__device__ __forceinline__ float max_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16 bytes per lane copied from global memory straight into LDS (global_load_lds_dwordx4): lane
// l writes bytes [16 l, 16 l + 16) of the wave-uniform destination `lds`, from its own address
// `src`.  No registers are involved; completion is tracked by the vector memory counter.
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void gbl_void_t;
__device__ __forceinline__ void dma16(const void *src, void *lds) {
    __builtin_amdgcn_global_load_lds((gbl_void_t *)src, (lds_void_t *)lds, 16, 0, 0);
}

// The same copy through a buffer resource: lane l reads `bytes` bytes at byte offset
// soff + voff (soff wave-uniform) past the resource's base.  The address arithmetic is done by
// the memory unit, so a copy costs one instruction besides the uniform operands.
typedef __amdgpu_buffer_rsrc_t buf_rsrc_t;
__device__ __forceinline__ buf_rsrc_t raw_rsrc(const void *base, unsigned bytes) {
    // Raw (unstructured) buffer: stride 0, 32-bit dwords, bounds = `bytes`.
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void dma16_buf(buf_rsrc_t r, unsigned voff, unsigned soff, void *lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds, 16, voff, soff, 0, 0);
}
// The destination as a 32-bit LDS byte address.
__device__ __forceinline__ void dma16_buf_at(buf_rsrc_t r, unsigned voff, unsigned soff, uint32_t lds) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(uintptr_t)lds, 16, voff, soff, 0, 0);
}
// With an instruction offset IMM, added to both the memory offset and the LDS destination.
template <int IMM>
__device__ __forceinline__ void dma16_buf_imm(buf_rsrc_t r, unsigned voff, unsigned soff, void *lds) {
    static_assert(IMM >= 0 && IMM < 4096, "buffer instruction offset out of range");
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)lds, 16, voff, soff, IMM, 0);
}
template <int IMM>
__device__ __forceinline__ void dma16_buf_imm_at(buf_rsrc_t r, unsigned voff, unsigned soff, uint32_t lds) {
    static_assert(IMM >= 0 && IMM < 4096, "buffer instruction offset out of range");
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t *)(uintptr_t)lds, 16, voff, soff, IMM, 0);
}

// The LDS byte address of `p`, hidden from the optimiser: values derived from it are formed
// where they are used instead of being hoisted out of loops (scalar registers are scarce).
__device__ __forceinline__ uint32_t opaque_lds_addr(const void *p) {
    typedef __attribute__((address_space(3))) const unsigned char lds_u8c;
    uint32_t a = (uint32_t)(uintptr_t)(lds_u8c *)p;
    asm volatile("" : "+s"(a));
    return a;
}

// 4 bytes per lane, global -> LDS: lane l writes bytes [4 l, 4 l + 4) of `lds`.
__device__ __forceinline__ void dma4(const void *src, void *lds) {
    __builtin_amdgcn_global_load_lds((gbl_void_t *)src, (lds_void_t *)lds, 4, 0, 0);
}

// s_waitcnt vmcnt(n) lgkmcnt(0) for a wave-uniform n: waits until at most n of this wave's
// vector memory operations are outstanding (n above 15 waits as for 15) and its LDS operations
// have completed.
__device__ __forceinline__ void wait_vm_lgkm0(int n) {
#define NE_VM(N) __builtin_amdgcn_s_waitcnt((N) | (7 << 4))  // expcnt: no wait, lgkmcnt(0)
    if (n <= 0) NE_VM(0);
    else if (n == 1) NE_VM(1);
    else if (n == 2) NE_VM(2);
    else if (n == 3) NE_VM(3);
    else if (n == 4) NE_VM(4);
    else if (n == 5) NE_VM(5);
    else if (n == 6) NE_VM(6);
    else if (n == 7) NE_VM(7);
    else if (n == 8) NE_VM(8);
    else if (n == 9) NE_VM(9);
    else if (n == 10) NE_VM(10);
    else if (n == 11) NE_VM(11);
    else if (n == 12) NE_VM(12);
    else if (n == 13) NE_VM(13);
    else if (n == 14) NE_VM(14);
    else NE_VM(15);
#undef NE_VM
}

// Registers 8 s .. 8 s + 7 of an accumulator tile, rounded to bf16, as an MFMA operand.
__device__ __forceinline__ bf16x8 pack8(const f32x16 &x, int s) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = (__bf16)x[8 * s + i];
    return r;
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// acc + the sum of the eight bf16 values of v (four v_dot2c_f32_bf16 against ones, in order).
__device__ __forceinline__ float sum8_bf16(const bf16x8 &v, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
    return acc;
}

}  // namespace ne
