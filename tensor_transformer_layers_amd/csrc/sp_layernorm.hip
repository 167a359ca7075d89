// sp_layernorm.hip -- the sequence-parallel block boundary of one rank on gfx950.
//
// With sequence parallelism (llms.blog, "Sequence Parallelism") the all-reduce after a
// row-parallel layer becomes a reduce-scatter: the N partials are summed but each rank keeps
// only its s/N slice of every sequence, and the work between blocks (residual addition and
// LayerNorm, element-wise along the hidden dimension and independent across tokens) runs on
// that slice. Before the next column-parallel layer an all-gather restores the full sequence.
// On one device the N partials are resident, so:
//   reduce-scatter       H_r[i] = sum_q Z_q[t(i)]                       (rank r's slice rows)
//   boundary (fused)     H_r[i] = sum_q Z_q[t(i)] + R_r[i],  Y_r[i] = LayerNorm(H_r[i])
//   all-gather           X[t] = slice_{r(t)}[i(t)]
// with t(i) = b * seq + r * seq/N + s' for slice row i = b * seq/N + s'.
//
// All three are HBM streaming kernels. The boundary kernel gives each slice row to one
// workgroup: the partial rows are read once (16-byte non-temporal loads, summed in the fixed
// order 0 .. N-1 in fp32), the row of H is kept in LDS, and the LayerNorm statistics are two
// passes over that LDS copy (mean, then the mean of squared deviations), reduced across the
// workgroup's waves.
#include "device_common.hpp"
#include "kernels.hpp"

namespace tps {
namespace {

constexpr int kThreads = 256;      // all-gather workgroup
constexpr int kRowThreads = 1024;  // boundary workgroup: one slice row, two vectors per lane at
                                   // hidden 8192 (256 lanes left 8 dependent rounds per lane)
constexpr int kMaxParts = 64;

struct Parts {
    const float* p[kMaxParts];
};

template <bool BF16>
__device__ __forceinline__ f32x4 load4(const void* base, int64_t i4)
{
    if constexpr (BF16)
        return bf16x4_to_f32(reinterpret_cast<const bf16x4*>(base)[i4]);
    else
        return reinterpret_cast<const f32x4*>(base)[i4];
}

template <bool BF16>
__device__ __forceinline__ void store4(void* base, int64_t i4, f32x4 v)
{
    if constexpr (BF16)
        reinterpret_cast<bf16x4*>(base)[i4] = to_bf16x4(v);
    else
        reinterpret_cast<f32x4*>(base)[i4] = v;
}

// Sum of v over the boundary workgroup (kRowThreads lanes); every lane receives the result,
// the waves' partial sums added in a fixed order.
__device__ __forceinline__ float block_sum(float v, float* red)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    const int wave = threadIdx.x >> 6;
    __syncthreads();   // red may still be read by the previous call
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kRowThreads / 64; ++w) s += red[w];
    return s;
}

// NP > 0: compile-time partial count; NP == 0: runtime n.
template <int NP, bool BF16, bool LN>
__global__ __launch_bounds__(kRowThreads) void sp_boundary_kernel(Parts parts, int n,
                                                               const void* resid,
                                                               const float* gamma,
                                                               const float* beta, float eps,
                                                               void* hout, void* yout, int seq,
                                                               int seq_r, int rank, int hidden)
{
    extern __shared__ __attribute__((aligned(16))) float row[];   // [hidden] when LN
    __shared__ float red[kRowThreads / 64];
    const int np = NP > 0 ? NP : n;
    const int i = blockIdx.x;                  // slice row
    const int b = i / seq_r, sp = i - b * seq_r;
    const int64_t t = (int64_t)b * seq + (int64_t)rank * seq_r + sp;
    const int h4 = hidden / 4;
    const int64_t src4 = t * h4, dst4 = (int64_t)i * h4;
    float sum = 0.f;
    for (int v = threadIdx.x; v < h4; v += kRowThreads) {
        f32x4 acc = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(parts.p[0]) + src4 + v);
        if constexpr (NP > 0) {
#pragma unroll
            for (int q = 1; q < NP; ++q)
                acc += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(parts.p[q]) + src4 + v);
        } else {
            for (int q = 1; q < np; ++q)
                acc += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(parts.p[q]) + src4 + v);
        }
        if (resid) acc += load4<BF16>(resid, dst4 + v);
        store4<BF16>(hout, dst4 + v, acc);
        if constexpr (LN) {
            *reinterpret_cast<f32x4*>(row + 4 * v) = acc;
            sum += (acc[0] + acc[1]) + (acc[2] + acc[3]);
        }
    }
    if constexpr (LN) {
        const float mean = block_sum(sum, red) / (float)hidden;   // block_sum syncs the row too
        float sq = 0.f;
        for (int v = threadIdx.x; v < h4; v += kRowThreads) {
            const f32x4 d = *reinterpret_cast<const f32x4*>(row + 4 * v) - mean;
            sq += (d[0] * d[0] + d[1] * d[1]) + (d[2] * d[2] + d[3] * d[3]);
        }
        const float var = block_sum(sq, red) / (float)hidden;
        const float inv = 1.0f / __builtin_sqrtf(var + eps);
        for (int v = threadIdx.x; v < h4; v += kRowThreads) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(row + 4 * v);
            const f32x4 g = reinterpret_cast<const f32x4*>(gamma)[v];
            const f32x4 be = reinterpret_cast<const f32x4*>(beta)[v];
            store4<BF16>(yout, dst4 + v, (x - mean) * inv * g + be);
        }
    }
}

// out row t = b * seq + r * seq_r + s' takes slice r's row b * seq_r + s' (row_bytes each).
__global__ __launch_bounds__(kThreads) void all_gather_rows_kernel(Parts slices, int seq,
                                                                   int seq_r, int64_t row16,
                                                                   void* out)
{
    const int t = blockIdx.x;
    const int b = t / seq, s = t - b * seq;
    const int r = s / seq_r, sp = s - r * seq_r;
    const u32x4* src = reinterpret_cast<const u32x4*>(slices.p[r]) + ((int64_t)b * seq_r + sp) * row16;
    u32x4* dst = reinterpret_cast<u32x4*>(out) + (int64_t)t * row16;
    // four vectors per round, all loads before the stores (so they are in flight together)
    for (int64_t v0 = threadIdx.x; v0 < row16; v0 += 4 * kThreads) {
        u32x4 x[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (v0 + u * kThreads < row16) x[u] = __builtin_nontemporal_load(src + v0 + u * kThreads);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (v0 + u * kThreads < row16) __builtin_nontemporal_store(x[u], dst + v0 + u * kThreads);
    }
}

template <int NP, bool BF16>
void launch_np(const Parts& pp, int n, const SpProblem& p, hipStream_t s)
{
    const dim3 grid((unsigned)((int64_t)p.batch * (p.seq / n))), block(kRowThreads);
    const int seq_r = p.seq / n;
    if (p.gamma) {
        const size_t lds = (size_t)p.hidden * sizeof(float);
        hipLaunchKernelGGL((sp_boundary_kernel<NP, BF16, true>), grid, block, lds, s, pp, n,
                           p.resid, p.gamma, p.beta, p.eps, p.hout, p.yout, p.seq, seq_r,
                           p.rank, p.hidden);
    } else {
        hipLaunchKernelGGL((sp_boundary_kernel<NP, BF16, false>), grid, block, 0, s, pp, n,
                           p.resid, p.gamma, p.beta, p.eps, p.hout, p.yout, p.seq, seq_r,
                           p.rank, p.hidden);
    }
}

template <bool BF16>
void launch_dt(const Parts& pp, int n, const SpProblem& p, hipStream_t s)
{
    switch (n) {
        case 1: launch_np<1, BF16>(pp, n, p, s); break;
        case 2: launch_np<2, BF16>(pp, n, p, s); break;
        case 4: launch_np<4, BF16>(pp, n, p, s); break;
        case 8: launch_np<8, BF16>(pp, n, p, s); break;
        default: launch_np<0, BF16>(pp, n, p, s);
    }
}

}  // namespace

hipError_t sp_boundary(const SpProblem& p, hipStream_t s)
{
    const int n = p.n_parts;
    if (n < 1 || n > kMaxParts || p.seq % n != 0) return hipErrorInvalidValue;
    Parts pp{};
    for (int q = 0; q < n; ++q) pp.p[q] = p.parts[q];
    if (p.bf16) launch_dt<true>(pp, n, p, s);
    else launch_dt<false>(pp, n, p, s);
    return hipGetLastError();
}

hipError_t all_gather_rows(const void* const* slices, int n, int batch, int seq, int64_t row_bytes,
                           void* out, hipStream_t s)
{
    if (n < 1 || n > kMaxParts || seq % n != 0 || row_bytes % 16 != 0) return hipErrorInvalidValue;
    Parts pp{};
    for (int q = 0; q < n; ++q) pp.p[q] = reinterpret_cast<const float*>(slices[q]);
    hipLaunchKernelGGL(all_gather_rows_kernel, dim3((unsigned)((int64_t)batch * seq)), dim3(kThreads),
                       0, s, pp, seq, seq / n, row_bytes / 16, out);
    return hipGetLastError();
}

}  // namespace tps
