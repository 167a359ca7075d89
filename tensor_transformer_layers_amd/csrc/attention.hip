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
// Work decomposition: one workgroup = BQ = 128 queries of one (sequence, head), run by one
// or two sets of 4 waves; in a set a wave owns 32 queries (two 16-query MFMA columns). Key
// tiles are 64 keys (K tile [64][d], V^T tile [d][64]), streamed through each set's own
// double-buffered LDS ring (loaded from global memory directly into LDS during the previous
// tile's work).
//  * Two sets (unsplit launches): the sets take alternate key tiles (set 0 the even ones), so
//    every SIMD runs two independent waves, and their partial results (running max,
//    denominator, unnormalised output) are merged through LDS with the same rescaling.
//  * One set (with the key-range split, below): 64 KB of LDS, two workgroups per compute unit.
//  * Paired causal layout (causal, fewer than 512 query tiles): a workgroup owns the 64-query
//    tiles i and n64 - 1 - i of one (sequence, head), whose causal key ranges add up to the
//    same length for every i, so every workgroup has the same work and no partials leave it.
//  * Key-range split (available for long causal sequences, forced by a test override): each
//    query tile's keys are halved between two workgroups, which write fp32 partials;
//    attn_merge_kernel combines them.
// Per tile, a wave computes
//   S^T = K Q^T - m  (MFMA "M" = keys, "N" = queries, K = d; the running max m enters as the
//                     accumulator input, and Q arrives pre-multiplied by log2(e)/sqrt(d))
//   O^T += V^T P^T   (MFMA "M" = d,    "N" = queries, K = keys), and the denominators with an
//                     all-ones operand in place of V^T
// as a two-stage pipeline: the scores of the next tile are computed while the current tile's
// probabilities (exp2) are formed, so a wave's exponentials overlap its own matrix products.
// With keys on the MFMA's row side, each lane's accumulator values of S^T all belong to ONE
// query (lane & 15), so the row max needs only a 4-lane exchange, the probabilities P are
// already in the lane layout the second MFMA takes as its B operand, and the O^T rows a lane
// accumulates belong to the same query whose statistics it holds. Masks are applied only on
// tiles that cross a wave's diagonal or the end of the sequence; the output is rescaled only
// when some running maximum grew by more than 2^8. Queries are dispatched longest-first
// (highest query tile first) to shorten the causal tail.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace tps {
namespace {

constexpr int BQ = 128;     // queries per workgroup (per set)
constexpr int BKV = 64;     // keys per tile
constexpr int QPW = 32;     // queries per wave
constexpr uint32_t kOutOfRange = 0x80000000u;

typedef __attribute__((address_space(3))) void* lds_ptr;

// max(v, v of lane ^ X) for X = 16 or 32, in the VALU: a permlane swap of v with itself gives
// each lane the pair (its own v, its partner's v) in some order. Keeps the softmax's row
// maximum off the LDS crossbar that a shuffle uses, on every key tile's dependency chain.
template <int X>
__device__ __forceinline__ float max_xor(float v, std::integral_constant<int, X>)
{
    static_assert(X == 16 || X == 32, "partner distance");
    const unsigned u = __float_as_uint(v);
    const auto r = X == 16 ? __builtin_amdgcn_permlane16_swap(u, u, false, false)
                           : __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t span_rsrc(const void* base, int64_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                             (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff),
                                             0x00020000);
}

template <int D, bool CAUSAL, int NSETS, bool PAIRED>
__global__ __launch_bounds__(256 * NSETS, NSETS == 1 ? 2 : 1) void attn_fwd_kernel(AttnProblem p)
{
    static_assert(!PAIRED || (CAUSAL && NSETS == 2), "pairs are causal, two sets");
    constexpr int KS = D / 32;            // MFMA K-steps of the S product
    constexpr int DB = D / 16;            // 16-row blocks of O^T
    constexpr int KROW = D * 2;           // bytes per K-tile row
    constexpr int KRPI = 1024 / KROW;     // K rows per 1 KB load instruction (4 or 8)
    constexpr int KI = BKV / KRPI / 4;    // K load instructions per wave per tile
    constexpr int VI = D / 8 / 4;         // V^T load instructions per wave per tile (8 rows each)

    // [set][buffer][K tile | V^T tile]; reused for the merge of the two sets' partials.
    __shared__ __attribute__((aligned(16))) bf16 lds[NSETS * 2 * 2 * BKV * D];
    auto tileK = [&](int set, int buf) { return lds + ((set * 2 + buf) * 2) * BKV * D; };
    auto tileV = [&](int set, int buf) { return lds + ((set * 2 + buf) * 2 + 1) * BKV * D; };

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int set = NSETS == 2 ? __builtin_amdgcn_readfirstlane(tid >> 8) : 0;   // key-tile parity
    // query group within the set; scalar, so that the per-tile causal tests below (whole tile
    // visible, tile crossing this wave's diagonal) are wave-uniform branches
    const int wave = __builtin_amdgcn_readfirstlane((tid >> 6) & 3);
    const int fr = lane & 15;
    const int fg = lane >> 4;
    // 16-byte chunk swizzle of a tile row: the 16 rows of one MFMA operand read (same logical
    // chunk) land on 16 distinct 16-byte groups of the LDS's 64 banks. 256-byte rows (K, d =
    // 128) fill the 256 bytes the banks serve per pass on their own; 128-byte rows (K for
    // d = 64, V^T) share it with their neighbour row.
    // MFMA row r of S^T block kb holds key krow(kb, r) of the tile: blocks 2j and 2j + 1 cover
    // keys 32j .. 32j + 31 such that the probabilities a lane ends up holding for one P V^T
    // operand (rows 4fg .. 4fg + 3 of both blocks) are the 8 consecutive keys 32j + 8fg + 0..7,
    // i.e. one 16-byte V^T chunk. Rows read together (fixed kb, r = 0..15) are
    // 32j + 4h + 8a + b (a, b = 0..3), which the K swizzles below keep on distinct bank groups.
    auto krow = [](int kb, int r) { return 32 * (kb >> 1) + 8 * (r >> 2) + 4 * (kb & 1) + (r & 3); };
    auto kswz = [](int row) {
        return D == 128 ? ((row & 3) | (((row >> 3) & 3) << 2))
                        : (((row >> 1) & 1) | (((row >> 3) & 3) << 1));
    };
    auto vswz = [](int row) { return (row >> 1) & 7; };

    // Longest-first: block 0 takes the last query tile of every (sequence, head) first.
    // (sequence, head) varies fastest, then the key-range half: consecutive blocks go to the
    // 8 XCDs in turn, so with 8 | batch * heads every block of one head (both halves of its
    // query tiles included) runs on one XCD and that head's K and V^T stay in one L2.
    const int halves = p.kv_split;
    const int n_qt = (p.seq + BQ - 1) / BQ;
    const int n_bh = p.batch * p.heads_local;
    // With one set (two workgroups per compute unit), blocks past the first 256 take the
    // query tiles in the reverse order, so that a unit pairs a long causal tile with a short one.
    int bidx = (int)blockIdx.x;
    if (NSETS == 1 && (int)gridDim.x > 256) {
        const int r = bidx - 256, per = n_bh * halves, groups = ((int)gridDim.x - 256) / per;
        if (r >= 0 && 256 % per == 0 && (int)gridDim.x % per == 0)
            bidx = 256 + (groups - 1 - r / per) * per + r % per;
    }
    const int qt = n_qt - 1 - bidx / (n_bh * halves);
    const int rem_b = bidx % (n_bh * halves);
    const int half = rem_b / n_bh;
    const int bh = rem_b - half * n_bh;
    const int q0 = qt * BQ;
    int qw0 = q0 + wave * QPW;            // this wave's first query
    // Paired causal layout: block (pair i, sequence-head) owns the 64-query tiles A = i and
    // B = n64 - 1 - i, whose causal key ranges add up to the same length for every i. Each
    // 64-query tile is taken by two waves of each set (32 queries each); set 0 puts A on its
    // waves 0-1 and B on 2-3, set 1 the other way round, so that the two waves sharing a SIMD
    // (same wave index in both sets) have one A and one B range between them. With an odd
    // tile count the middle pair has A = B, and the waves meant for B idle.
    bool idle = false;
    int pair_kv = 0;                      // key tiles of the pair (B's causal range)
    if constexpr (PAIRED) {
        const int n64 = (p.seq + 2 * QPW - 1) / (2 * QPW);
        const int pi = (int)blockIdx.x / n_bh;
        const int ta = pi, tb = n64 - 1 - pi;
        const bool on_a = (wave < 2) != (set == 1);
        idle = !on_a && tb == ta;
        qw0 = idle ? p.seq : (on_a ? ta : tb) * (2 * QPW) + (wave & 1) * QPW;
        pair_kv = min(p.seq, (tb + 1) * 2 * QPW);
        pair_kv = (pair_kv + BKV - 1) / BKV;
    }

    const int64_t head_rows = (int64_t)bh * p.seq;
    const bf16* __restrict__ gQ = reinterpret_cast<const bf16*>(p.q) + head_rows * D;
    // Key/value head of this query head (grouped-query attention shares one among
    // Hl / KVl query heads; KVl = Hl is multi-head attention).
    const int b_of = bh / p.heads_local;
    const int64_t kvh = (int64_t)b_of * p.kv_heads_local +
                        (bh - b_of * p.heads_local) / (p.heads_local / p.kv_heads_local);
    // K rows past seq and V^T columns past the buffer read as zero (range-checked loads);
    // V^T columns in [seq, ld_vt) are zeroed before this kernel runs.
    const __amdgpu_buffer_rsrc_t rK = span_rsrc(
        reinterpret_cast<const bf16*>(p.k) + kvh * p.seq * D, (int64_t)p.seq * D * 2);
    const __amdgpu_buffer_rsrc_t rV = span_rsrc(
        reinterpret_cast<const bf16*>(p.vt) + kvh * D * p.ld_vt, (int64_t)D * p.ld_vt * 2);

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
    const int n_kv = PAIRED ? pair_kv : (kv_end + BKV - 1) / BKV;
    // this workgroup's key tiles [t_lo, t_hi): all of them, or one half
    const int n_first = (n_kv + halves - 1) / halves;
    const int t_lo = half == 0 ? 0 : n_first;
    const int t_hi = half == 0 ? n_first : n_kv;

    // Tiles go from global memory straight into LDS: a 1 KB load instruction writes lane l's
    // 16 bytes at byte 16 l of its destination, so the lane fetches the logical chunk that the
    // swizzle places there. K tile: wave w loads rows KRPI (w + 4 i) + ...; V^T tile: rows
    // (d) 8 (w + 4 i) + (l >> 3).
    auto fetchK = [&](int k0, int buf) {
        bf16* sK = tileK(set, buf);
#pragma unroll
        for (int i = 0; i < KI; ++i) {
            const int rbase = KRPI * (wave + 4 * i);
            const int row = rbase + lane / (KROW / 16);
            const int phys = lane % (KROW / 16);
            const int c = phys ^ kswz(row);
            const uint32_t off = (uint32_t)((k0 + row) * KROW + c * 16);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rK, (lds_ptr)(sK + rbase * D), 16, k0 + row < p.seq ? off : kOutOfRange, 0, 0, 0);
        }
    };
    auto fetchV = [&](int k0, int buf) {
        bf16* sV = tileV(set, buf);
#pragma unroll
        for (int i = 0; i < VI; ++i) {
            const int rbase = 8 * (wave + 4 * i);
            const int row = rbase + (lane >> 3);
            const int c = (lane & 7) ^ vswz(row);
            const uint32_t off = (uint32_t)(((int64_t)row * p.ld_vt + k0 + c * 8) * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rV, (lds_ptr)(sV + rbase * BKV), 16, off,
                                                     0, 0, 0);
        }
    };

    f32x4 acc[DB][2];
    // Denominators: the P V^T products' companion with an all-ones A operand sums each
    // query's probabilities over the tile's keys into every element of lsum[qb].
    f32x4 lsum[2];
#pragma unroll
    for (int i = 0; i < DB; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    lsum[0] = lsum[1] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Running max of the scores. Q arrives multiplied by log2(e) / sqrt(d), so a score is
    // already the exponent of base 2 and a probability is exp2(score - max).
    float m_run[2] = {-INFINITY, -INFINITY};
    bf16x8 ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones[e] = bf16(1.0f);

    // The running maximum is raised only when a tile's maximum exceeds it by more than
    // 2^kLazy in probability (FlashAttention's result does not depend on which maximum is
    // subtracted, as long as numerator and denominator use the same one); in between, the
    // probabilities stay below 2^kLazy and the rescale of the output is skipped.
    constexpr float kLazy = 8.0f;

    // ---- the phases of one key tile
    // S^T = K Q^T - m: s[kb][qb][i] = score(key k0 + krow(kb, 4fg + i), query qw0 + 16qb + fr)
    // minus that query's running max, which enters as the products' accumulator input (0
    // while the query has none); masked (keys past the query or past the end of the sequence)
    // when MASKED.
    auto scores = [&](const bf16* sKc, int k0, auto masked_c, f32x4 (&s)[4][2]) {
        constexpr bool MASKED = decltype(masked_c)::value;
        f32x4 c0[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const float mo = m_run[qb] == -INFINITY ? 0.f : -m_run[qb];
            c0[qb] = f32x4{mo, mo, mo, mo};
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int row = krow(kb, fr);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int c = ks * 4 + fg;
                const bf16x8 kf =
                    *reinterpret_cast<const bf16x8*>(&sKc[row * D + ((c ^ kswz(row)) << 3)]);
                s[kb][0] = mfma16x16x32(kf, qf[0][ks], ks == 0 ? c0[0] : s[kb][0]);
                s[kb][1] = mfma16x16x32(kf, qf[1][ks], ks == 0 ? c0[1] : s[kb][1]);
            }
        }
        if constexpr (MASKED) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int q = qw0 + qb * 16 + fr;
                const int lim = CAUSAL ? min(q, p.seq - 1) : p.seq - 1;   // last visible key
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (k0 + krow(kb, 4 * fg + i) > lim) s[kb][qb][i] = -INFINITY;
            }
        }
    };
    // Tile maximum relative to the running one; when some query's exceeds kLazy (or the query
    // had no maximum yet), raise that query's maximum by it, rescale its output and
    // denominator by exp2(-shift), and shift the tile's scores to the new maximum.
    auto update_max = [&](f32x4 (&s)[4][2]) {
        float mx[2];
        bool grew = false;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            float m = s[0][qb][0];
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) m = fmaxf(m, s[kb][qb][i]);
            m = max_xor(m, std::integral_constant<int, 16>{});
            m = max_xor(m, std::integral_constant<int, 32>{});
            mx[qb] = m;
            grew = grew || (m_run[qb] == -INFINITY ? m != -INFINITY : m > kLazy);
        }
        if (__any(grew)) {
            // (a scheduling fence keeps this a real branch: the rescale is rare, and
            // speculating it would put 64 multiplies on every tile)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const bool none = m_run[qb] == -INFINITY;
                const float shift = none ? (mx[qb] == -INFINITY ? 0.f : mx[qb]) : fmaxf(mx[qb], 0.f);
                const float alpha = none ? 0.f : __builtin_amdgcn_exp2f(-shift);
                m_run[qb] = none ? (mx[qb] == -INFINITY ? -INFINITY : mx[qb]) : m_run[qb] + shift;
                lsum[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < DB; ++db) acc[db][qb] *= alpha;
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) s[kb][qb] -= shift;
            }
        }
    };
    // P = exp2(s) <= 2^kLazy packed as bf16 B operands: pf[qb][j] = keys 32j + 8fg + 0..7.
    auto probs = [&](const f32x4 (&s)[4][2], bf16x8 (&pf)[2][2]) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pf[qb][j][i] = to_bf16(__builtin_amdgcn_exp2f(s[2 * j][qb][i]));
                    pf[qb][j][4 + i] = to_bf16(__builtin_amdgcn_exp2f(s[2 * j + 1][qb][i]));
                }
    };
    // O^T += V^T P^T, and the denominators
    auto pv = [&](const bf16* sVc, const bf16x8 (&pf)[2][2]) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const int row = db * 16 + fr;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const bf16x8 vf = *reinterpret_cast<const bf16x8*>(
                    &sVc[row * BKV + (((4 * j + fg) ^ vswz(row)) << 3)]);
                acc[db][0] = mfma16x16x32(vf, pf[0][j], acc[db][0]);
                acc[db][1] = mfma16x16x32(vf, pf[1][j], acc[db][1]);
            }
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            lsum[0] = mfma16x16x32(ones, pf[0][j], lsum[0]);
            lsum[1] = mfma16x16x32(ones, pf[1][j], lsum[1]);
        }
    };
    // A tile is needed by a wave unless all the wave's queries precede it (causal).
    auto needed = [&](int t) {
        return !idle && t < t_hi && (!CAUSAL || t * BKV <= qw0 + QPW - 1);
    };

    // Set s takes key tiles t0 = t_lo + s, t0 + 2, ... and runs them as a two-stage pipeline:
    // in iteration it it turns the scores of tile t = t0 + 2 it into probabilities and
    // accumulates P V over it while the matrix cores compute the scores of tile t + 2, so one
    // wave's exponentials overlap its own matrix products. K thus runs one tile ahead of V in
    // the set's double-buffered LDS ring: iteration it reads K(t + 2) and V(t) and loads
    // K(t + 4) into K(t)'s buffer and V(t + 2) into V(t - 2)'s. The iterations begin with the
    // shared workgroup barrier; set 1 idles in the last one when the range is odd.
    const int t0 = t_lo + set;
    const int n_it = (t_hi - t_lo + NSETS - 1) / NSETS;
    if (t0 < t_hi) {
        fetchK(t0 * BKV, 0);
        fetchV(t0 * BKV, 0);
    }
    if (t0 + NSETS < t_hi) fetchK((t0 + NSETS) * BKV, 1);
    __syncthreads();   // (the compiler waits for the loads first)
    f32x4 sA[4][2], sB[4][2];
    if (needed(t0)) {
        scores(tileK(set, 0), t0 * BKV, std::true_type{}, sA);
        update_max(sA);
    }

    auto window = [&](int it, auto masked_c, f32x4 (&s)[4][2], f32x4 (&sn)[4][2]) {
        constexpr bool MASKED = decltype(masked_c)::value;
        const int t = t0 + NSETS * it, tn = t + NSETS;
        const int kb_cur = it & 1;
        __syncthreads();   // K(tn) and V(t) have landed; K(t) and V(t - NSETS) are free
        if (tn + NSETS < t_hi) fetchK((tn + NSETS) * BKV, kb_cur);
        if (tn < t_hi) fetchV(tn * BKV, kb_cur ^ 1);
        bf16x8 pf[2][2];
        if constexpr (!MASKED) {
            // every query of the workgroup sees tiles t and t + 2 in full: one block, so the
            // scheduler can interleave the two tiles' work
            scores(tileK(set, kb_cur ^ 1), tn * BKV, std::false_type{}, sn);
            probs(s, pf);
            pv(tileV(set, kb_cur), pf);
            update_max(sn);
        } else {
            if (needed(tn)) scores(tileK(set, kb_cur ^ 1), tn * BKV, std::true_type{}, sn);
            if (needed(t)) {
                probs(s, pf);
                pv(tileV(set, kb_cur), pf);
            }
            if (needed(tn)) update_max(sn);
        }
    };
    // Windows whose next tile (t + 2, for both sets) lies inside the sequence and wholly
    // before the workgroup's first query (causal) need no mask (tile t then does not either);
    // the rest (the diagonal, a ragged end) do. Tiles must also lie in [t_lo, t_hi). In the
    // paired layout the count is the wave's own (its queries' first), so waves change loops
    // at different windows; every wave still runs n_it windows, one barrier each.
    const int full_tiles = min(min(CAUSAL ? (PAIRED ? (idle ? 0 : qw0 + 1) : q0) / BKV : n_kv,
                                   p.seq / BKV), t_hi);
    const int n_full_it = min(max(full_tiles - t_lo - NSETS, 0) / NSETS, n_it);
    int it = 0;
    {
        for (; it + 2 <= n_full_it; it += 2) {
            window(it, std::false_type{}, sA, sB);
            window(it + 1, std::false_type{}, sB, sA);
        }
        if (it < n_full_it) {
            window(it, std::false_type{}, sA, sB);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) sA[kb][0] = sB[kb][0], sA[kb][1] = sB[kb][1];
            ++it;
        }
        for (; it + 2 <= n_it; it += 2) {
            window(it, std::true_type{}, sA, sB);
            window(it + 1, std::true_type{}, sB, sA);
        }
        if (it < n_it) window(it, std::true_type{}, sA, sB);
    }

    // ---- merge the two sets' partials: set 1 publishes (output, max, denominator) of each of
    // its lanes; the set-0 wave with the same queries (same lane) combines them, rescaling
    // each side by exp2(m_side - m) with m the larger maximum.
    constexpr int NF = DB * 2 * 4 + 4;   // floats per lane: output, 2 maxima, 2 denominators
    static_assert(NSETS == 1 || 4 * NF * 64 * 4 <= (int)sizeof(lds), "merge area");
    // [slot][field][lane]: set 1's wave w publishes in the slot of the set-0 wave with the same
    // queries (w itself, or w + 2 mod 4 in the paired layout)
    const int slot = PAIRED && set == 1 ? (wave + 2) & 3 : wave;
    float* xch = reinterpret_cast<float*>(lds) + slot * NF * 64 + lane;
    if constexpr (NSETS == 2) __syncthreads();   // every wave is done with the tiles in the LDS
    if (NSETS == 2 && set == 1) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int i = 0; i < 4; ++i) xch[((db * 2 + qb) * 4 + i) * 64] = acc[db][qb][i];
        xch[(NF - 4) * 64] = m_run[0];
        xch[(NF - 3) * 64] = m_run[1];
        xch[(NF - 2) * 64] = lsum[0][0];
        xch[(NF - 1) * 64] = lsum[1][0];
    }
    if constexpr (NSETS == 2) {
        __syncthreads();
        if (set == 1) return;
    }

    // ---- combine; then normalise and store O[token][head*D + d] (4 consecutive d per lane),
    // or, with the key-range split, store this half's unnormalised output, max and denominator.
    // A side that saw no key of a query (its maximum is still -inf) carries weight 0; when
    // the whole range is split, one half may hold no visible key for a query at all.
    const int b = bh / p.heads_local;
    const int head = bh - b * p.heads_local;
    const int64_t ldo = (int64_t)p.heads_local * D;
    bf16* __restrict__ gO = reinterpret_cast<bf16*>(p.o);
    const int64_t item = ((int64_t)bh * n_qt + qt) * halves + half;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
        // (one set: there is no second partial)
        const float m1 = NSETS == 2 ? xch[(NF - 4 + qb) * 64] : -INFINITY;
        const float l1 = NSETS == 2 ? xch[(NF - 2 + qb) * 64] : 0.f;
        const float m0 = m_run[qb];
        const float m = fmaxf(m0, m1);
        const float a0 = m0 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m0 - m);
        const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - m);
        const float l = lsum[qb][0] * a0 + l1 * a1;
        const int q = qw0 + qb * 16 + fr;
        if (q >= p.seq) continue;
        if (halves == 1) {
            const float inv = 1.0f / l;
            bf16* dst = gO + ((int64_t)b * p.seq + q) * ldo + head * D + 4 * fg;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                f32x4 o1;
#pragma unroll
                for (int i = 0; i < 4; ++i) o1[i] = NSETS == 2 ? xch[((db * 2 + qb) * 4 + i) * 64] : 0.f;
                *reinterpret_cast<bf16x4*>(dst + db * 16) = to_bf16x4((acc[db][qb] * a0 + o1 * a1) * inv);
            }
        } else {
            const int r = q - q0;
            float* po = p.part_o + (item * BQ + r) * D + 4 * fg;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                f32x4 o1;
#pragma unroll
                for (int i = 0; i < 4; ++i) o1[i] = NSETS == 2 ? xch[((db * 2 + qb) * 4 + i) * 64] : 0.f;
                *reinterpret_cast<f32x4*>(po + db * 16) = acc[db][qb] * a0 + o1 * a1;
            }
            if (fg == 0) {
                float* pm = p.part_ml + (item * BQ + r) * 2;
                pm[0] = m;
                pm[1] = l;
            }
        }
    }
}

// Merge of the two key-range halves of every query tile: with m = max(m_0, m_1) (maxima of
// the base-2 exponents) and a_h = exp2(m_h - m) (0 for a half that saw no key), O = (O_0 a_0 + O_1 a_1) /
// (l_0 a_0 + l_1 a_1), the same rescaling as the online softmax. One workgroup per 16 rows
// of a (sequence, head, query tile); lanes take 4-wide vectors of those rows.
constexpr int kMergeRows = 16;
template <int D>
__global__ __launch_bounds__(256) void attn_merge_kernel(AttnProblem p)
{
    constexpr int RB = BQ / kMergeRows;
    const int n_qt = (p.seq + BQ - 1) / BQ;
    const int tile = blockIdx.x / RB, rb = blockIdx.x - tile * RB;
    const int bh = tile / n_qt, qt = tile - bh * n_qt;
    const int q0 = qt * BQ, r0 = rb * kMergeRows;
    const int rows = min(kMergeRows, p.seq - q0 - r0);
    if (rows <= 0) return;
    const int b = bh / p.heads_local, head = bh - b * p.heads_local;
    const int64_t item0 = ((int64_t)bh * n_qt + qt) * 2;
    const int64_t ldo = (int64_t)p.heads_local * D;
    bf16* __restrict__ gO = reinterpret_cast<bf16*>(p.o);
    // two vectors per lane and round, all loads before the stores
    constexpr int U = 2;
    const int n_e = rows * (D / 4);
    for (int e0 = threadIdx.x; e0 < n_e; e0 += U * 256) {
        float2 ml0[U], ml1[U];
        f32x4 o0[U], o1[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = e0 + u * 256;
            if (e < n_e) {
                const int r = r0 + e / (D / 4), c4 = e % (D / 4);
                ml0[u] = *reinterpret_cast<const float2*>(p.part_ml + (item0 * BQ + r) * 2);
                ml1[u] = *reinterpret_cast<const float2*>(p.part_ml + ((item0 + 1) * BQ + r) * 2);
                o0[u] = *reinterpret_cast<const f32x4*>(p.part_o + (item0 * BQ + r) * D + 4 * c4);
                o1[u] = *reinterpret_cast<const f32x4*>(p.part_o + ((item0 + 1) * BQ + r) * D + 4 * c4);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = e0 + u * 256;
            if (e < n_e) {
                const int r = r0 + e / (D / 4), c4 = e % (D / 4);
                const float m = fmaxf(ml0[u].x, ml1[u].x);
                const float a0 = ml0[u].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml0[u].x - m);
                const float a1 = ml1[u].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ml1[u].x - m);
                const float inv = 1.0f / (ml0[u].y * a0 + ml1[u].y * a1);
                *reinterpret_cast<bf16x4*>(gO + ((int64_t)b * p.seq + q0 + r) * ldo + head * D +
                                           4 * c4) = to_bf16x4((o0[u] * a0 + o1[u] * a1) * inv);
            }
        }
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

// Paired causal layout (a block owns 64-query tiles i and n64 - 1 - i): the default for
// causal attention with fewer than 512 query tiles of 128 (at most 256 pair workgroups, one
// round on the chip), in place of the key-range split. Measured (one box): 4 sequences of
// 2048 with 4 local heads 33.1 against 37-38 us for the split and its merge; 4096 tokens with
// 8 local heads 57-59 against 58-59 us; with 512 tiles (8 x 2048) the pairs' two rounds lose
// (55.5 against 45.5 us for one-set workgroups, two per compute unit). The test override
// "attn_pair=1" turns it off, "attn_pair=2" forces it; forcing one set per workgroup
// ("attn_sets=1") or the split turns it off too.
bool use_pairs(bool causal, int kv_split, int64_t n_tiles)
{
    const Tuning t = tuning();
    if (!causal || kv_split != 1 || t.attn_pair == 1 || t.attn_sets == 1) return false;
    return t.attn_pair == 2 || n_tiles < 2 * 256;
}

template <int D>
hipError_t launch(const AttnProblem& p, hipStream_t s)
{
    if (p.kv_heads_local < 1 || p.heads_local % p.kv_heads_local != 0) return hipErrorInvalidValue;
    if (p.ld_vt > p.seq) {
        const int64_t rows = (int64_t)p.batch * p.kv_heads_local * D;
        const int64_t n = rows * (p.ld_vt - p.seq);
        hipLaunchKernelGGL(zero_vt_pad_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                           const_cast<bf16*>(reinterpret_cast<const bf16*>(p.vt)), rows, p.seq, p.ld_vt);
    }
    if (p.kv_split != 1 && (p.kv_split != 2 || !p.part_o || !p.part_ml)) return hipErrorInvalidValue;
    const int n_qt = (p.seq + BQ - 1) / BQ;
    const int n_tiles = n_qt * p.batch * p.heads_local;
    dim3 grid((unsigned)(n_tiles * p.kv_split));
    // Sets per workgroup: with at least 512 workgroups (two per compute unit), one-set
    // workgroups (64 KB of LDS) overlap one workgroup's prologue and epilogue with the other's
    // key loop: 2.5 us faster on the 4096-token layer step (split), 57.7 against 61.0 us on
    // 8 sequences of 2048 tokens with 4 local heads (unsplit, 512 query tiles). With fewer
    // workgroups, two sets keep eight waves on every unit. The test override "attn_sets=1|2"
    // replaces the choice.
    int nsets = grid.x >= 2 * 256 ? 1 : 2;
    if (const int v = tuning().attn_sets) nsets = v;
    if (use_pairs(p.causal != 0, p.kv_split, n_tiles)) {
        // one block per (pair of 64-query tiles, sequence-head): equal causal work per block
        const int n64 = (p.seq + 2 * QPW - 1) / (2 * QPW);
        const dim3 pgrid((unsigned)(((n64 + 1) / 2) * p.batch * p.heads_local));
        hipLaunchKernelGGL((attn_fwd_kernel<D, true, 2, true>), pgrid, dim3(512), 0, s, p);
    } else if (nsets == 1) {
        if (p.causal)
            hipLaunchKernelGGL((attn_fwd_kernel<D, true, 1, false>), grid, dim3(256), 0, s, p);
        else
            hipLaunchKernelGGL((attn_fwd_kernel<D, false, 1, false>), grid, dim3(256), 0, s, p);
    } else {
        if (p.causal)
            hipLaunchKernelGGL((attn_fwd_kernel<D, true, 2, false>), grid, dim3(512), 0, s, p);
        else
            hipLaunchKernelGGL((attn_fwd_kernel<D, false, 2, false>), grid, dim3(512), 0, s, p);
    }
    if (p.kv_split == 2)
        hipLaunchKernelGGL(attn_merge_kernel<D>, dim3((unsigned)(n_tiles * (BQ / kMergeRows))),
                           dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace

// The key-range split pays when the query tiles alone give fewer than two workgroups per
// compute unit (256 on MI355X) and the causal tail is long: the longest query tiles then run
// alone for a large share of the kernel. Measured at 256 query tiles, attention plus merge:
// with 32 query tiles per sequence (4096 tokens) 74 us split against 88 us unsplit; with 16
// (2048 tokens) 42.9 against 44.0 us once split workgroups run two per compute unit. The
// paired layout balances the same shapes without partials and is the default there; the
// split remains the choice when pairing is turned off (causal, under 512 query tiles, at
// least 16 query tiles per sequence). The partials are reserved whenever there are under
// 512 query tiles (the workspace size depends on the shapes only, not on the mask or the
// overrides). The test override "attn_split=1" turns the split off, "attn_split=2" forces it
// wherever the partials are reserved.
size_t attention_partial_bytes(int batch, int heads_local, int seq, int head_dim, bool causal,
                               int* kv_split)
{
    const int n_qt = (seq + BQ - 1) / BQ;
    const int64_t n_tiles = (int64_t)n_qt * batch * heads_local;
    const int split = n_tiles < 2 * 256 ? 2 : 1;
    if (kv_split) {
        const int force = tuning().attn_split;
        if (force == 1)
            *kv_split = 1;
        else if (force == 2)
            *kv_split = split;
        else if (use_pairs(causal, 1, n_tiles))
            *kv_split = 1;   // the pairs balance the causal work without partials
        else
            *kv_split = causal && n_qt >= 16 ? split : 1;
    }
    if (split == 1) return 0;
    // two halves per query tile: output [128][d] and (max, denominator) [128][2], fp32
    return (size_t)n_tiles * 2 * BQ * ((size_t)head_dim + 2) * sizeof(float);
}

hipError_t attention_fwd(const AttnProblem& p, hipStream_t s)
{
    if (p.head_dim == 128) return launch<128>(p, s);
    if (p.head_dim == 64) return launch<64>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace tps
