// attention.hip -- head-local softmax attention of one tensor-parallel rank on gfx950.
//
// For each sequence b and local head j:  O = softmax(Q K^T / sqrt(d) + M) V
// (llms.blog, "Partitioning Multi-Head and Grouped-Query Attention", step 2: each rank
// evaluates scaled dot-product attention for its own heads with no cross-head exchange).
// M is the causal mask (key k visible to query s iff k <= s) or zero.
//
// The softmax is evaluated in one pass over the keys with the running-maximum rescaling of
// FlashAttention (Dao et al., 2022, cited by the llms.blog page): for each query the kernel
// keeps the running maximum m and denominator l of the scaled scores and an unnormalised
// output; a new key tile with maximum m' rescales both by exp(m - m'). This gives exactly
// the softmax result (up to rounding) without materialising the seq x seq score matrix.
//
// Work decomposition: one workgroup = 4 waves = BQ = 128 queries of one (sequence, head);
// each wave owns 32 queries (two 16-query MFMA columns). Keys stream through LDS in tiles
// of 64 (K tile [64][d], V^T tile [d][64], double-buffered, loaded from global memory
// directly into LDS during the previous tile's work). Per tile, a wave computes
//   S^T = K Q^T      (MFMA "M" = keys, "N" = queries, K = d)
//   O^T += V^T P^T   (MFMA "M" = d,    "N" = queries, K = keys)
// With keys on the MFMA's row side, each lane's accumulator values of S^T all belong to ONE
// query (lane & 15), so the row max/sum need only a 4-lane exchange, the probabilities P are
// already in the lane layout the second MFMA takes as its B operand, and the O^T rows a lane
// accumulates belong to the same query whose statistics it holds. Masks are applied only on
// tiles that cross a wave's diagonal or the end of the sequence; the scale is folded into the
// exponent's FMA; the output is rescaled only when some running maximum grew. Queries are
// dispatched longest-first (highest query tile first) to shorten the causal tail.
#include "device_common.hpp"
#include "kernels.hpp"

namespace tps {
namespace {

constexpr int kThreads = 256;
constexpr int BQ = 128;     // queries per workgroup
constexpr int BKV = 64;     // keys per tile
constexpr int QPW = 32;     // queries per wave
constexpr uint32_t kOutOfRange = 0x80000000u;

typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const void* base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff),
                                             0x00020000);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(AttnProblem p)
{
    constexpr int KS = D / 32;            // MFMA K-steps of the S product
    constexpr int DB = D / 16;            // 16-row blocks of O^T
    constexpr int KROW = D * 2;           // bytes per K-tile row
    constexpr int KRPI = 1024 / KROW;     // K rows per 1 KB load instruction (4 or 8)
    constexpr int KI = BKV / KRPI / 4;    // K load instructions per wave per tile
    constexpr int VI = D / 8 / 4;         // V^T load instructions per wave per tile (8 rows each)

    __shared__ __attribute__((aligned(16))) bf16 sK[2][BKV * D];
    __shared__ __attribute__((aligned(16))) bf16 sV[2][D * BKV];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int fr = lane & 15;
    const int fg = lane >> 4;
    // 16-byte chunk swizzle of a tile row: the 16 rows of one MFMA operand read (same logical
    // chunk) land on 16 distinct 16-byte groups of the LDS's 64 banks. 256-byte rows (K, d =
    // 128) fill the 256 bytes the banks serve per pass on their own; 128-byte rows (K for
    // d = 64, V^T) share it with their neighbour row.
    auto kswz = [](int row) { return D == 128 ? (row & 15) : ((row >> 1) & 7); };
    auto vswz = [](int row) { return (row >> 1) & 7; };

    // Longest-first: block 0 takes the last query tile of every (sequence, head) first.
    const int n_qt = (p.seq + BQ - 1) / BQ;
    const int n_bh = p.batch * p.heads_local;
    const int qt = n_qt - 1 - (int)(blockIdx.x / n_bh);
    const int bh = (int)(blockIdx.x % n_bh);
    const int q0 = qt * BQ;
    const int qw0 = q0 + wave * QPW;      // this wave's first query

    const int64_t head_rows = (int64_t)bh * p.seq;
    const bf16* __restrict__ gQ = reinterpret_cast<const bf16*>(p.q) + head_rows * D;
    // K rows past seq and V^T columns past the buffer read as zero (range-checked loads);
    // V^T columns in [seq, ld_vt) are zeroed before this kernel runs.
    const __amdgpu_buffer_rsrc_t rK =
        span_rsrc(reinterpret_cast<const bf16*>(p.k) + head_rows * D, (int64_t)p.seq * D * 2);
    const __amdgpu_buffer_rsrc_t rV = span_rsrc(
        reinterpret_cast<const bf16*>(p.vt) + (int64_t)bh * D * p.ld_vt, (int64_t)D * p.ld_vt * 2);

    // Q fragments stay in registers: lane holds query qw0 + 16*qb + fr, d chunk 4*ks + fg.
    bf16x8 qf[2][KS];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        const int q = qw0 + qb * 16 + fr;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 v = q < p.seq ? ld16(gQ + (int64_t)q * D + (ks * 4 + fg) * 8) : zero16();
            qf[qb][ks] = __builtin_bit_cast(bf16x8, v);
        }
    }

    const int kv_end = CAUSAL ? min(p.seq, q0 + BQ) : p.seq;
    const int n_kv = (kv_end + BKV - 1) / BKV;

    // Tiles go from global memory straight into LDS: a 1 KB load instruction writes lane l's
    // 16 bytes at byte 16 l of its destination, so the lane fetches the logical chunk that the
    // swizzle places there. K tile: wave w loads rows KRPI (w + 4 i) + ...; V^T tile: rows
    // (d) 8 (w + 4 i) + (l >> 3).
    auto fetch = [&](int k0, int buf) {
#pragma unroll
        for (int i = 0; i < KI; ++i) {
            const int rbase = KRPI * (wave + 4 * i);
            const int row = rbase + lane / (KROW / 16);
            const int phys = lane % (KROW / 16);
            const int c = phys ^ kswz(row);
            const uint32_t off = (uint32_t)((k0 + row) * KROW + c * 16);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rK, (lds_ptr)(&sK[buf][rbase * D]), 16, k0 + row < p.seq ? off : kOutOfRange, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < VI; ++i) {
            const int rbase = 8 * (wave + 4 * i);
            const int row = rbase + (lane >> 3);
            const int c = (lane & 7) ^ vswz(row);
            const uint32_t off = (uint32_t)(((int64_t)row * p.ld_vt + k0 + c * 8) * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rV, (lds_ptr)(&sV[buf][rbase * BKV]), 16, off,
                                                     0, 0, 0);
        }
    };

    f32x4 acc[DB][2];
#pragma unroll
    for (int i = 0; i < DB; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY};   // running max of the raw scores
    float l_run[2] = {0.f, 0.f};               // this lane's share of the denominator
    const float sl2 = p.scale_log2;

    fetch(0, 0);
    __syncthreads();

    for (int t = 0; t < n_kv; ++t) {
        const int cur = t & 1;
        const int k0 = t * BKV;
        if (t + 1 < n_kv) fetch(k0 + BKV, cur ^ 1);

        // A wave whose queries all precede this key tile has nothing to add (causal).
        const bool active = !CAUSAL || k0 <= qw0 + QPW - 1;
        if (active) {
            // ---- S^T = K Q^T : s[kb][qb][i] = score(key k0+16kb+4fg+i, query qw0+16qb+fr)
            f32x4 s[4][2];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                s[kb][0] = s[kb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
                const int row = kb * 16 + fr;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const int c = ks * 4 + fg;
                    const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
                        &sK[cur][row * D + ((c ^ kswz(row)) << 3)]);
                    s[kb][0] = mfma16x16x32(kf, qf[0][ks], s[kb][0]);
                    s[kb][1] = mfma16x16x32(kf, qf[1][ks], s[kb][1]);
                }
            }
            // ---- mask (only tiles crossing this wave's diagonal or the end of the sequence)
            const bool partial = k0 + BKV > p.seq || (CAUSAL && k0 + BKV - 1 > qw0);
            if (partial) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    const int q = qw0 + qb * 16 + fr;
                    const int lim = CAUSAL ? min(q, p.seq - 1) : p.seq - 1;   // last visible key
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (k0 + kb * 16 + 4 * fg + i > lim) s[kb][qb][i] = -INFINITY;
                }
            }
            // ---- running max (raw scores; the positive scale preserves order)
            float mx[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                float m = s[0][qb][0];
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) m = fmaxf(m, s[kb][qb][i]);
                m = fmaxf(m, __shfl_xor(m, 16));
                m = fmaxf(m, __shfl_xor(m, 32));
                mx[qb] = fmaxf(m_run[qb], m);
            }
            // ---- rescale only if some lane's maximum moved (then alpha < 1 for that query)
            const bool grew = (mx[0] > m_run[0]) || (mx[1] > m_run[1]);
            if (__any(grew)) {
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    const float alpha = m_run[qb] == -INFINITY
                                            ? 0.f
                                            : __builtin_amdgcn_exp2f((m_run[qb] - mx[qb]) * sl2);
                    l_run[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < DB; ++db) acc[db][qb] *= alpha;
                }
            }
            // ---- P = exp2((s - m) scale log2 e), packed as bf16 B-operands
            bf16x8 pf[2][2];   // [qb][j]: keys k0+32j+{4fg..4fg+3, 16+4fg..16+4fg+3}
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                m_run[qb] = mx[qb];
                const float mo = mx[qb] == -INFINITY ? 0.f : -mx[qb] * sl2;
                float ls = 0.f;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][qb][i], sl2, mo));
                        s[kb][qb][i] = e;
                        ls += e;
                    }
                l_run[qb] += ls;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        pf[qb][j][i] = to_bf16(s[2 * j][qb][i]);
                        pf[qb][j][4 + i] = to_bf16(s[2 * j + 1][qb][i]);
                    }
                }
            }
            // ---- O^T += V^T P^T
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const int row = db * 16 + fr;
                const int x = vswz(row);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    // keys 32j + 4fg + (0..3): 8-byte slot 8j + fg; keys + 16: slot 8j + 4 + fg
                    const int s0 = 8 * j + fg, s1 = 8 * j + 4 + fg;
                    const int a0 = row * BKV + ((((s0 >> 1) ^ x) << 1) + (s0 & 1)) * 4;
                    const int a1 = row * BKV + ((((s1 >> 1) ^ x) << 1) + (s1 & 1)) * 4;
                    const u32x2 lo = *reinterpret_cast<const u32x2*>(&sV[cur][a0]);
                    const u32x2 hi = *reinterpret_cast<const u32x2*>(&sV[cur][a1]);
                    const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
                    acc[db][0] = mfma16x16x32(vf, pf[0][j], acc[db][0]);
                    acc[db][1] = mfma16x16x32(vf, pf[1][j], acc[db][1]);
                }
            }
        }
        __syncthreads();   // the next tile has landed (the compiler waits for the loads first)
    }

    // ---- normalise and store O[token][head*D + d], 4 consecutive d per lane
    const int b = bh / p.heads_local;
    const int head = bh - b * p.heads_local;
    const int64_t ldo = (int64_t)p.heads_local * D;
    bf16* __restrict__ gO = reinterpret_cast<bf16*>(p.o);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        float l = l_run[qb];
        l += __shfl_xor(l, 16);
        l += __shfl_xor(l, 32);
        const float inv = 1.0f / l;
        const int q = qw0 + qb * 16 + fr;
        if (q >= p.seq) continue;
        bf16* dst = gO + ((int64_t)b * p.seq + q) * ldo + head * D + 4 * fg;
#pragma unroll
        for (int db = 0; db < DB; ++db)
            *reinterpret_cast<bf16x4*>(dst + db * 16) = to_bf16x4(acc[db][qb] * inv);
    }
}

// Zero the V^T columns [seq, ld_vt) of every (sequence, head, d) row (present when seq is not
// a multiple of 8) so that the last key tile reads zeros there.
__global__ void zero_vt_pad_kernel(bf16* vt, int64_t rows, int seq, int64_t ld_vt)
{
    const int64_t pad = ld_vt - seq;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= rows * pad) return;
    const int64_t r = i / pad, c = seq + i % pad;
    vt[r * ld_vt + c] = bf16(0.f);
}

template <int D>
hipError_t launch(const AttnProblem& p, hipStream_t s)
{
    if (p.ld_vt > p.seq) {
        const int64_t rows = (int64_t)p.batch * p.heads_local * D;
        const int64_t n = rows * (p.ld_vt - p.seq);
        hipLaunchKernelGGL(zero_vt_pad_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                           const_cast<bf16*>(reinterpret_cast<const bf16*>(p.vt)), rows, p.seq, p.ld_vt);
    }
    const int n_qt = (p.seq + BQ - 1) / BQ;
    dim3 grid((unsigned)(n_qt * p.batch * p.heads_local)), block(kThreads);
    if (p.causal)
        hipLaunchKernelGGL((attn_fwd_kernel<D, true>), grid, block, 0, s, p);
    else
        hipLaunchKernelGGL((attn_fwd_kernel<D, false>), grid, block, 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t attention_fwd(const AttnProblem& p, hipStream_t s)
{
    if (p.head_dim == 128) return launch<128>(p, s);
    if (p.head_dim == 64) return launch<64>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace tps
