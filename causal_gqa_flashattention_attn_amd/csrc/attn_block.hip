// attn_block.hip -- the attention sub-block around the kernel, float32: the pre-norm residual
// branch of a NanoEuler block, x + attn(rmsnorm(x)) ("NanoEuler -- Show HN" Japanese README
// translation, section "Architecture": RMSNorm pre-normalisation without bias, RoPE on queries
// and keys, grouped-query attention, each block computes x = x + attn(rmsnorm(x))).
//
//   r = 1 / sqrt(mean_c x^2 + eps),  xn = x r gamma          (rows of C = Hq D)
//   [q | k | v] = xn Wqkv    (Wqkv [C][(Hq + 2 Hkv) D]; heads in that order, D columns each)
//   o = attention(q, k, v)    (the library's causal GQA forward, RoPE in the kernel)
//   y = x + o Wo              (o as rows [B T][Hq D], Wo [Hq D][C])
//
// The products are plain GEMMs and go to rocBLAS; the row-wise RMSNorm and the attention are the
// library's own kernels, the attention reading q, k, v from the projection rows and writing o
// (and the gradients) as rows in place, through its strided layouts.  All matrices are
// row-major.
#include <hip/hip_runtime.h>
#include <rocblas/rocblas.h>

#include <mutex>

#include "attn_device.hpp"
#include "attn_kernels.hpp"

namespace ne {
namespace {

// One wave per row: sum of squares over 64 lanes (4 columns each per step), then xn and r.
__global__ void __launch_bounds__(256) rmsnorm_fwd_f32(const float *x, const float *gamma,
                                                       float *xn, float *rstd, long long rows,
                                                       int C, float eps) {
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const float *xr = x + row * C;
    float ss = 0.f;
    for (int c = 4 * lane; c < C; c += 256) {
        const f32x4 u = ld4(xr + c);
        ss += (u[0] * u[0] + u[1] * u[1]) + (u[2] * u[2] + u[3] * u[3]);
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) ss += __shfl_xor(ss, m, 64);
    const float r = 1.0f / sqrtf(ss / (float)C + eps);
    for (int c = 4 * lane; c < C; c += 256) {
        const f32x4 u = ld4(xr + c), g = ld4(gamma + c);
        st4(xn + row * C + c, f32x4{u[0] * r * g[0], u[1] * r * g[1], u[2] * r * g[2], u[3] * r * g[3]});
    }
    if (lane == 0) rstd[row] = r;
}

// dx = dy + r gamma dxn - x r^3 (sum_c x gamma dxn) / C, one wave per row; the row's share of
// dgamma (dxn x r) goes to part[block][C] for a deterministic column sum afterwards.
__global__ void __launch_bounds__(256) rmsnorm_bwd_f32(const float *x, const float *gamma,
                                                       const float *rstd, const float *dxn,
                                                       const float *dy, float *dx, float *part,
                                                       long long rows, int C, int rows_per_block) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const long long r0 = (long long)blockIdx.x * rows_per_block;
    float *pb = part + (size_t)blockIdx.x * C;
    // This wave's column slice of the block's dgamma partial sum: columns 4 lane + 256 j, for
    // its rows; the four waves' slices are added through LDS at the end.
    extern __shared__ float red[];  // [4][C]
    for (int c = 4 * lane; c < C; c += 256) st4(red + w * C + c, f32x4{0.f, 0.f, 0.f, 0.f});
    for (long long row = r0 + w; row < r0 + rows_per_block && row < rows; row += 4) {
        const float *xr = x + row * C, *gr = dxn + row * C;
        const float r = rstd[row];
        float s = 0.f;
        for (int c = 4 * lane; c < C; c += 256) {
            const f32x4 u = ld4(xr + c), g = ld4(gamma + c), d = ld4(gr + c);
            s += (u[0] * g[0] * d[0] + u[1] * g[1] * d[1]) + (u[2] * g[2] * d[2] + u[3] * g[3] * d[3]);
        }
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) s += __shfl_xor(s, m, 64);
        const float k3 = r * r * r * s / (float)C;
        for (int c = 4 * lane; c < C; c += 256) {
            const f32x4 u = ld4(xr + c), g = ld4(gamma + c), d = ld4(gr + c), e = ld4(dy + row * C + c);
            st4(dx + row * C + c, f32x4{e[0] + r * g[0] * d[0] - u[0] * k3, e[1] + r * g[1] * d[1] - u[1] * k3,
                                        e[2] + r * g[2] * d[2] - u[2] * k3, e[3] + r * g[3] * d[3] - u[3] * k3});
            f32x4 acc = ld4(red + w * C + c);
            acc += f32x4{d[0] * u[0] * r, d[1] * u[1] * r, d[2] * u[2] * r, d[3] * u[3] * r};
            st4(red + w * C + c, acc);
        }
    }
    __syncthreads();
    for (int c = threadIdx.x; c < C; c += 256)
        pb[c] = (red[c] + red[C + c]) + (red[2 * C + c] + red[3 * C + c]);
}

// dgamma[c] = sum over blocks of part[block][c]: 32 columns per work-group, eight groups of
// partial rows (g, g + 8, ...) summed in order, then the eight group sums added in order, so
// the result does not depend on scheduling.
__global__ void __launch_bounds__(256) colsum_f32(const float *part, float *out, int nblk, int C) {
    __shared__ float red[8][32];
    const int cg = threadIdx.x & 31, g = threadIdx.x >> 5;
    const int c = blockIdx.x * 32 + cg;
    float s = 0.f;
    if (c < C)
        for (int b = g; b < nblk; b += 8) s += part[(size_t)b * C + c];
    red[g][cg] = s;
    __syncthreads();
    if (g == 0 && c < C) {
        float t = red[0][cg];
#pragma unroll
        for (int k = 1; k < 8; ++k) t += red[k][cg];
        out[c] = t;
    }
}

}  // namespace

namespace {
// Guards the handles: their creation, and the stream and workspace a handle is bound to between
// binding them and enqueueing a product on it (host threads share a device's handle).
std::mutex blas_mu;
}  // namespace

// rocBLAS handle per device, created on first use and kept for the life of the process.  The
// caller holds blas_mu.
rocblas_handle blas_handle() {
    static rocblas_handle h[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    if (!h[dev] && rocblas_create_handle(&h[dev]) != rocblas_status_success) h[dev] = nullptr;
    return h[dev];
}

// Row-major C[M][N] = alpha op(A) op(B) + beta C with op(A) [M][K], op(B) [K][N]; ta / tb: the
// stored matrix is the transpose ([K][M] / [N][K]).  rocBLAS is column-major, so it computes
// C^T = op(B)^T op(A)^T.  The product runs on `st` with `ws` (ws_bytes, owned by the caller) as
// its rocBLAS workspace: a launch takes its workspace address when it is enqueued, so products
// of calls with distinct workspaces never share scratch memory, whatever their streams.
hipError_t gemm_rm(hipStream_t st, void *ws, size_t ws_bytes, bool ta, bool tb, int M, int N,
                   int K, const float *A, const float *Bm, float *Cm, float beta) {
    std::lock_guard<std::mutex> lock(blas_mu);  // binding + sgemm only enqueue: held briefly
    rocblas_handle h = blas_handle();
    if (!h || rocblas_set_stream(h, st) != rocblas_status_success ||
        rocblas_set_workspace(h, ws, ws_bytes) != rocblas_status_success)
        return hipErrorUnknown;
    const float alpha = 1.f;
    const rocblas_status s = rocblas_sgemm(
        h, tb ? rocblas_operation_transpose : rocblas_operation_none,
        ta ? rocblas_operation_transpose : rocblas_operation_none, N, M, K, &alpha, Bm,
        tb ? K : N, A, ta ? M : K, &beta, Cm, N);
    return s == rocblas_status_success ? hipSuccess : hipErrorUnknown;
}

hipError_t launch_rmsnorm_fwd(const float *x, const float *gamma, float *xn, float *rstd,
                              long long rows, int C, float eps, hipStream_t st) {
    void *p[] = {&x, &gamma, &xn, &rstd, &rows, &C, &eps};
    return hipLaunchKernel((const void *)rmsnorm_fwd_f32, dim3((unsigned)((rows + 3) / 4)),
                           dim3(256), p, 0, st);
}

// Rows per rmsnorm_bwd work-group: four per wave, enough work-groups to stream the rows.
constexpr int kNormRows = 16;

int rmsnorm_bwd_blocks(long long rows) { return (int)((rows + kNormRows - 1) / kNormRows); }

hipError_t launch_rmsnorm_bwd(const float *x, const float *gamma, const float *rstd,
                              const float *dxn, const float *dy, float *dx, float *part,
                              float *dgamma, long long rows, int C, hipStream_t st) {
    int rpb = kNormRows;
    const int nblk = rmsnorm_bwd_blocks(rows);
    void *p[] = {&x, &gamma, &rstd, &dxn, &dy, &dx, &part, &rows, &C, &rpb};
    hipError_t e = hipLaunchKernel((const void *)rmsnorm_bwd_f32, dim3((unsigned)nblk), dim3(256),
                                   p, (size_t)4 * C * sizeof(float), st);
    if (e != hipSuccess) return e;
    int nb = nblk;
    void *q[] = {&part, &dgamma, &nb, &C};
    return hipLaunchKernel((const void *)colsum_f32, dim3((unsigned)((C + 31) / 32)), dim3(256),
                           q, 0, st);
}

}  // namespace ne
