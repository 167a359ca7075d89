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
// of 64 (K tile [64][d], V^T tile [d][64], double-buffered, fetched into registers during
// the MFMAs of the previous tile). Per tile, a wave computes
//   S^T = K Q^T      (MFMA "M" = keys, "N" = queries, K = d)
//   O^T += V^T P^T   (MFMA "M" = d,    "N" = queries, K = keys)
// With keys on the MFMA's row side, each lane's accumulator values of S^T all belong to ONE
// query (lane & 15), so the row max/sum need only a 4-lane exchange, the probabilities P are
// already in the lane layout the second MFMA takes as its B operand, and the O^T rows a lane
// accumulates belong to the same query whose statistics it holds. Queries are dispatched
// longest-first (highest query tile first) to shorten the causal tail.
#include "device_common.hpp"
#include "kernels.hpp"

namespace tps {
namespace {

constexpr int kThreads = 256;
constexpr int BQ = 128;     // queries per workgroup
constexpr int BKV = 64;     // keys per tile
constexpr int QPW = 32;     // queries per wave

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void attn_fwd_kernel(AttnProblem p)
{
    constexpr int DCH = D / 8;            // 16-byte chunks per K row
    constexpr int KS = D / 32;            // MFMA K-steps of the S product
    constexpr int DB = D / 16;            // 16-row blocks of O^T
    constexpr int KCH = BKV * DCH / kThreads;   // K-tile chunks per lane
    constexpr int VCH = D * (BKV / 8) / kThreads;
    static_assert(KCH >= 1 && VCH >= 1, "tile");

    __shared__ __attribute__((aligned(16))) bf16 sK[2][BKV * D];
    __shared__ __attribute__((aligned(16))) bf16 sV[2][D * BKV];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int fr = lane & 15;
    const int fg = lane >> 4;

    // Longest-first: block 0 takes the last query tile of every (sequence, head) first.
    const int n_qt = (p.seq + BQ - 1) / BQ;
    const int n_bh = p.batch * p.heads_local;
    const int qt = n_qt - 1 - (int)(blockIdx.x / n_bh);
    const int bh = (int)(blockIdx.x % n_bh);
    const int q0 = qt * BQ;
    const int qw0 = q0 + wave * QPW;      // this wave's first query

    const int64_t head_rows = (int64_t)bh * p.seq;
    const bf16* __restrict__ gQ = reinterpret_cast<const bf16*>(p.q) + head_rows * D;
    const bf16* __restrict__ gK = reinterpret_cast<const bf16*>(p.k) + head_rows * D;
    const bf16* __restrict__ gV = reinterpret_cast<const bf16*>(p.vt) + (int64_t)bh * D * p.ld_vt;

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

    u32x4 rk[KCH], rv[VCH];
    auto fetch = [&](int k0) {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int ci = tid + kThreads * i;
            const int row = ci / DCH, c = ci % DCH;
            const int key = k0 + row;
            rk[i] = key < p.seq ? ld16(gK + (int64_t)key * D + c * 8) : zero16();
        }
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            const int ci = tid + kThreads * i;
            const int row = ci >> 3, c = ci & 7;
            const int key = k0 + c * 8;
            u32x4 v = zero16();
            if (key < p.seq) {
                // ld_vt is a multiple of 8, so the chunk is in bounds; clear keys >= seq.
                v = ld16(gV + (int64_t)row * p.ld_vt + key);
                const int valid = p.seq - key;
                if (valid < 8) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int lo = 2 * e, hi = 2 * e + 1;
                        uint32_t w = v[e];
                        if (lo >= valid) w &= 0xFFFF0000u;
                        if (hi >= valid) w &= 0x0000FFFFu;
                        v[e] = w;
                    }
                }
            }
            rv[i] = v;
        }
    };
    // K tile: row = key (DCH chunks), chunk c stored at c ^ (key & 7).
    // V^T tile: row = d (8 chunks of 8 keys), addressed in 8-byte slots: slot s of row r is
    // stored at s ^ (r & 15), so a 16-byte chunk keeps its pair of slots (swapped if r is odd).
    auto stash = [&](int buf) {
#pragma unroll
        for (int i = 0; i < KCH; ++i) {
            const int ci = tid + kThreads * i;
            const int row = ci / DCH, c = ci % DCH;
            st16(&sK[buf][row * D + ((c ^ (row & 7)) << 3)], rk[i]);
        }
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
            const int ci = tid + kThreads * i;
            const int row = ci >> 3, c = ci & 7;
            const int x = row & 15;
            const int slot = (2 * c) ^ x;            // physical slot of the chunk's first half
            u32x4 v = rv[i];
            if (x & 1) v = u32x4{v[2], v[3], v[0], v[1]};
            st16(&sV[buf][row * BKV + ((slot & ~1) << 2)], v);
        }
    };

    f32x4 acc[DB][2];
#pragma unroll
    for (int i = 0; i < DB; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};           // this lane's share of the denominator

    fetch(0);
    stash(0);
    __syncthreads();

    for (int t = 0; t < n_kv; ++t) {
        const int cur = t & 1;
        const int k0 = t * BKV;
        if (t + 1 < n_kv) fetch(k0 + BKV);

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
                        &sK[cur][row * D + ((c ^ (row & 7)) << 3)]);
                    s[kb][0] = mfma16x16x32(kf, qf[0][ks], s[kb][0]);
                    s[kb][1] = mfma16x16x32(kf, qf[1][ks], s[kb][1]);
                }
            }
            // ---- scale (to log2 units), mask, running max
            float mx[2];
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int q = qw0 + qb * 16 + fr;
                float m = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int key = k0 + kb * 16 + 4 * fg + i;
                        float v = s[kb][qb][i] * p.scale_log2;
                        const bool vis = key < p.seq && (!CAUSAL || key <= q);
                        v = vis ? v : -INFINITY;
                        s[kb][qb][i] = v;
                        m = fmaxf(m, v);
                    }
                m = fmaxf(m, __shfl_xor(m, 16));
                m = fmaxf(m, __shfl_xor(m, 32));
                mx[qb] = m;
            }
            // ---- rescale running state, exponentiate, pack P as bf16 B-operands
            bf16x8 pf[2][2];   // [qb][j]: keys k0+32j+{4fg..4fg+3, 16+4fg..16+4fg+3}
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const float m_new = fmaxf(m_run[qb], mx[qb]);
                const float m_use = m_new == -INFINITY ? 0.f : m_new;
                const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_use);
                m_run[qb] = m_new;
                l_run[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) acc[db][qb] *= alpha;
                float ls = 0.f;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float e = __builtin_amdgcn_exp2f(s[kb][qb][i] - m_use);
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
                const int x = row & 15;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    // keys 32j + 4fg + (0..3) -> slot 8j + fg; keys +16 -> slot 8j + 4 + fg
                    const int s0 = (8 * j + fg) ^ x;
                    const int s1 = (8 * j + 4 + fg) ^ x;
                    const u32x2 lo = *reinterpret_cast<const u32x2*>(&sV[cur][row * BKV + s0 * 4]);
                    const u32x2 hi = *reinterpret_cast<const u32x2*>(&sV[cur][row * BKV + s1 * 4]);
                    const bf16x8 vf = __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
                    acc[db][0] = mfma16x16x32(vf, pf[0][j], acc[db][0]);
                    acc[db][1] = mfma16x16x32(vf, pf[1][j], acc[db][1]);
                }
            }
        }
        if (t + 1 < n_kv) stash(cur ^ 1);
        __syncthreads();
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

template <int D>
hipError_t launch(const AttnProblem& p, hipStream_t s)
{
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
