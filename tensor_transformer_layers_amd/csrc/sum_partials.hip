// sum_partials.hip -- Z = Z_0 + ... + Z_{N-1}: the single-device stand-in for the
// tensor-parallel all-reduce (llms.blog, Row-Parallel Linear Layer: the true output is the
// sum of the N partial products, formed by an all-reduce sum).
//
// Pure HBM streaming: each element is read once from every partial and written once, so the
// kernel is bound by (N + 1) x numel x 4 bytes of traffic. Each lane handles 16-byte float4
// vectors, grid-strided; all N loads of a vector are issued before the adds so that N
// requests per lane are in flight. The adds run in the fixed order 0, 1, ..., N-1, so the
// result is bitwise reproducible. Reads and writes are non-temporal: every byte is touched
// exactly once.
#include "device_common.hpp"
#include "kernels.hpp"

namespace tps {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxParts = 64;

struct Parts {
    const float* p[kMaxParts];
};

template <bool BF16>
__device__ __forceinline__ void put4(void* out, int64_t i4, f32x4 v)
{
    if constexpr (BF16) {
        bf16x4* o = reinterpret_cast<bf16x4*>(out) + i4;
        __builtin_nontemporal_store(to_bf16x4(v), o);
    } else {
        f32x4* o = reinterpret_cast<f32x4*>(out) + i4;
        __builtin_nontemporal_store(v, o);
    }
}

// NP > 0: compile-time part count (fully unrolled); NP == 0: runtime count n. Each lane
// handles U consecutive-by-stride float4 vectors per iteration, so N * U loads are in flight.
template <int NP, int U, bool BF16>
__global__ __launch_bounds__(kThreads) void sum_kernel(Parts parts, int n, int64_t n4, void* out)
{
    const int np = NP > 0 ? NP : n;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t i0 = (int64_t)blockIdx.x * kThreads + threadIdx.x; i0 < n4; i0 += stride * U) {
        if constexpr (NP > 0) {
            f32x4 v[U][NP];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = i0 + u * stride;
                if (i < n4) {
#pragma unroll
                    for (int r = 0; r < NP; ++r)
                        v[u][r] = __builtin_nontemporal_load(
                            reinterpret_cast<const f32x4*>(parts.p[r]) + i);
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t i = i0 + u * stride;
                if (i < n4) {
                    f32x4 acc = v[u][0];
#pragma unroll
                    for (int r = 1; r < NP; ++r) acc += v[u][r];
                    put4<BF16>(out, i, acc);
                }
            }
        } else {
            for (int u = 0; u < U; ++u) {
                const int64_t i = i0 + u * stride;
                if (i >= n4) break;
                f32x4 acc = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(parts.p[0]) + i);
                for (int r = 1; r < np; ++r)
                    acc += __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(parts.p[r]) + i);
                put4<BF16>(out, i, acc);
            }
        }
    }
}

// The numel % 4 trailing elements.
template <bool BF16>
__global__ void sum_tail_kernel(Parts parts, int n, int64_t start, int64_t numel, void* out)
{
    const int64_t i = start + threadIdx.x;
    if (i >= numel) return;
    float acc = parts.p[0][i];
    for (int r = 1; r < n; ++r) acc += parts.p[r][i];
    if constexpr (BF16)
        reinterpret_cast<bf16*>(out)[i] = to_bf16(acc);
    else
        reinterpret_cast<float*>(out)[i] = acc;
}

// Launch shape. Default: one lane per float4 vector (grid = vectors / 256, so the grid-stride
// loop runs once) with the U = 4 instantiation, whose register footprint keeps two waves per
// SIMD resident; measured on the 8 x 32 Mi-element sum this streams at about 6.4 TB/s, above a
// plain copy kernel, while more resident waves (U = 1) or a capped grid reach 5.2 to 5.8 TB/s.
// The test overrides "sum_grid=<workgroups>" and "sum_unroll=1|2|4" replace the defaults, so
// that the tests run every launch shape.

template <int U, bool BF16>
void launch_u(const Parts& parts, int n, int64_t n4, void* out, unsigned grid, hipStream_t s)
{
    switch (n) {
#define TPS_CASE(K)                                                                              \
    case K:                                                                                      \
        hipLaunchKernelGGL((sum_kernel<K, U, BF16>), dim3(grid), dim3(kThreads), 0, s, parts, n, \
                           n4, out);                                                             \
        break;
        TPS_CASE(1) TPS_CASE(2) TPS_CASE(3) TPS_CASE(4)
        TPS_CASE(5) TPS_CASE(6) TPS_CASE(7) TPS_CASE(8)
#undef TPS_CASE
        default:
            hipLaunchKernelGGL((sum_kernel<0, U, BF16>), dim3(grid), dim3(kThreads), 0, s, parts, n,
                               n4, out);
    }
}

template <bool BF16>
hipError_t launch(const Parts& parts, int n, int64_t numel, void* out, hipStream_t s)
{
    const int64_t n4 = numel / 4;
    if (n4 > 0) {
        const Tuning tu = tuning();
        const int unroll = tu.sum_unroll ? tu.sum_unroll : 4;
        int64_t grid64 = (n4 + kThreads - 1) / kThreads;
        const int64_t cap = tu.sum_grid;
        if (cap > 0 && grid64 > cap) grid64 = cap;
        if (grid64 > 0x7fffffff) grid64 = 0x7fffffff;   // the loop is grid-stride
        const unsigned grid = (unsigned)grid64;
        if (unroll >= 4)
            launch_u<4, BF16>(parts, n, n4, out, grid, s);
        else if (unroll == 2)
            launch_u<2, BF16>(parts, n, n4, out, grid, s);
        else
            launch_u<1, BF16>(parts, n, n4, out, grid, s);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (numel % 4) {
        hipLaunchKernelGGL((sum_tail_kernel<BF16>), dim3(1), dim3(4), 0, s, parts, n, n4 * 4, numel,
                           out);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace

hipError_t sum_partials(const float* const* parts, int n_parts, int64_t numel, void* out,
                        bool out_bf16, hipStream_t s)
{
    if (n_parts < 1 || n_parts > kMaxParts) return hipErrorInvalidValue;
    Parts pp{};
    for (int r = 0; r < n_parts; ++r) pp.p[r] = parts[r];
    return out_bf16 ? launch<true>(pp, n_parts, numel, out, s)
                    : launch<false>(pp, n_parts, numel, out, s);
}

}  // namespace tps
