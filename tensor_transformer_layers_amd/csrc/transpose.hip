// transpose.hip -- layout helpers of the MLP shard's backward pass on gfx950.
//
// The backward products contract over the token dimension (dA = X^T dP, dB = Y^T dZ) or use
// a weight in the other orientation (dY = dZ B_r^T, dX = dP A_r^T); the MFMA GEMM takes both
// operands contiguous along the reduced dimension, so those operands are first transposed:
//   transpose_bf16   out[c][r] = f(in[r][c]),  f = identity or GeLU (Y = GeLU(P) on the fly)
//                    out has leading dimension ld_out >= rows; columns [rows, ld_out) of
//                    out are written as zeros (zero padding of a reduced dimension)
//   row_sum_bf16     out[r] = sum_c in[r][c] in fp32 (the bias gradient, from dP^T rows)
// Both are HBM streaming kernels. The transpose moves 64 x 64 tiles through LDS: 16-byte
// row-contiguous loads, a padded LDS tile (row pitch 66 elements, so the column reads of
// the store phase fall on distinct banks), 16-byte row-contiguous stores.
#include <algorithm>

#include "device_common.hpp"
#include "kernels.hpp"

namespace tps {
namespace {

constexpr int kTile = 64;
constexpr int kPitch = kTile + 2;
constexpr int kThreads = 256;

template <bool GELU>
__global__ __launch_bounds__(kThreads) void transpose_kernel(const bf16* __restrict__ in, int rows,
                                                             int cols, int64_t ld_in,
                                                             bf16* __restrict__ out,
                                                             int64_t ld_out)
{
    __shared__ bf16 tile[kTile][kPitch];
    const int c0 = blockIdx.x * kTile;
    const int tid = threadIdx.x;
    // row tiles (of ld_out, padding included) strided over the grid's y extent, which is
    // capped at 65535
    const int64_t n_rt = (ld_out + kTile - 1) / kTile;
    for (int64_t rt = blockIdx.y; rt < n_rt; rt += gridDim.y) {
        const int r0 = (int)(rt * kTile);
        if (rt != blockIdx.y) __syncthreads();   // the previous tile's LDS reads are done
        // load: 64 rows x 8 chunks of 8 elements; thread -> (row, chunk), 2 passes
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int idx = tid + pass * kThreads;
            const int rr = idx >> 3, ch = idx & 7;
            const int r = r0 + rr, c = c0 + ch * 8;
            bf16x8 v;
            if (r < rows && c < cols) {   // cols is a multiple of 8: a chunk is all in or all out
                v = *reinterpret_cast<const bf16x8*>(in + (int64_t)r * ld_in + c);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = bf16(0.f);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                if constexpr (GELU) {
                    tile[rr][ch * 8 + e] = to_bf16(gelu_erf(static_cast<float>(v[e])));
                } else {
                    tile[rr][ch * 8 + e] = v[e];
                }
            }
        }
        __syncthreads();
        // store: out row c (64 of them) x 8 chunks of 8 input rows each
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int idx = tid + pass * kThreads;
            const int cc = idx >> 3, ch = idx & 7;
            const int c = c0 + cc, r = r0 + ch * 8;
            if (c >= cols || r >= ld_out) continue;
            bf16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = tile[ch * 8 + e][cc];   // rows >= rows were zeroed
            if (r + 8 <= ld_out) {
                *reinterpret_cast<bf16x8*>(out + (int64_t)c * ld_out + r) = v;
            } else {
                for (int e = 0; e < 8 && r + e < ld_out; ++e) out[(int64_t)c * ld_out + r + e] = v[e];
            }
        }
    }
}

// out[r] = sum over the row's cols bf16 values, fp32, fixed order: per-lane strided partial
// sums then a butterfly across the wave and a fixed combination of the waves.
__global__ __launch_bounds__(kThreads) void row_sum_kernel(const bf16* __restrict__ in, int cols,
                                                           int64_t ld, float* __restrict__ out)
{
    __shared__ float red[4];
    const int r = blockIdx.x;
    const bf16* row = in + (int64_t)r * ld;
    float s = 0.f;
    if (ld % 8 == 0 && (reinterpret_cast<uintptr_t>(in) & 15) == 0) {
        // 16-byte rows: 8 values per load (2-byte loads left the kernel at 2.4 TB/s)
        const int c8 = cols / 8 * 8;
        for (int c = threadIdx.x * 8; c < c8; c += kThreads * 8) {
            const bf16x8 v = *reinterpret_cast<const bf16x8*>(row + c);
#pragma unroll
            for (int e = 0; e < 8; ++e) s += static_cast<float>(v[e]);
        }
        for (int c = c8 + threadIdx.x; c < cols; c += kThreads) s += static_cast<float>(row[c]);
    } else {
        for (int c = threadIdx.x; c < cols; c += kThreads) s += static_cast<float>(row[c]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) out[r] = (red[0] + red[1]) + (red[2] + red[3]);
}

}  // namespace

hipError_t transpose_bf16(const void* in, int rows, int cols, int64_t ld_in, void* out,
                          int64_t ld_out, bool gelu, hipStream_t s)
{
    if (rows < 1 || cols < 1 || cols % 8 != 0 || ld_out < rows || ld_out % 8 != 0)
        return hipErrorInvalidValue;
    const int64_t tr = (ld_out + kTile - 1) / kTile;   // cover the zero padding too
    dim3 grid((unsigned)((cols + kTile - 1) / kTile), (unsigned)std::min<int64_t>(tr, 65535)),
        block(kThreads);
    const bf16* i = reinterpret_cast<const bf16*>(in);
    bf16* o = reinterpret_cast<bf16*>(out);
    if (gelu)
        hipLaunchKernelGGL(transpose_kernel<true>, grid, block, 0, s, i, rows, cols, ld_in, o, ld_out);
    else
        hipLaunchKernelGGL(transpose_kernel<false>, grid, block, 0, s, i, rows, cols, ld_in, o, ld_out);
    return hipGetLastError();
}

hipError_t row_sum_bf16(const void* in, int rows, int cols, int64_t ld, float* out, hipStream_t s)
{
    if (rows < 1 || cols < 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(row_sum_kernel, dim3((unsigned)rows), dim3(kThreads), 0, s,
                       reinterpret_cast<const bf16*>(in), cols, ld, out);
    return hipGetLastError();
}

}  // namespace tps
