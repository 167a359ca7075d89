// gemm.hip -- tensor-core (MFMA) GEMMs of the column- and row-parallel linear layers on gfx950.
//
//   C[m, n] = sum_k A[m, k] * B[n, k]      A = activations [M, K], B = weight [N, K] ([out, in])
//
// Both operands are K-contiguous, which is the layout an MFMA lane consumes: one 16-byte
// chunk of 8 bf16 (or 4 fp32) consecutive K values per lane. The output stage is fused:
//   BiasGelu  Y_i = GeLU(X A_i + a_i)                   column-parallel MLP layer (optionally
//             also P = X A_i + a_i, rounded once, for the backward)
//   F32       Z_i = Y_i B_i  (fp32 partial)             row-parallel layers (MLP, W_O)
//   Bias      Y = X W_i + b_i                           column-parallel, no activation
//   Qkv       [Q | K | V] = X W_qkv,i + b, scattered    column-parallel QKV projection
//             per head, V written transposed for the attention kernel's P V product, Q
//             multiplied by q_scale (the softmax's scale) before it is rounded.
//   SumF32    Z = sum_q Z_q with Z_rank = X_i W_i       row-parallel layer with the partial sum
//   SumBf16   (the all-reduce's sum) fused: the other ranks' fp32 partials are read in the
//             epilogue and added in the fixed order q = 0 .. N-1, the rank's own product in
//             its place, so the rank's partial is never written; fp32 or bf16 output.
//   SwiGlu    A_i = SiLU(X W_gate,i) * (X W_up,i)       gated column-parallel MLP layer: the
//             block's B slab interleaves gate and up rows in 32-row blocks (loaded from the
//             two weights), so each wave's pairs of 32-column MFMA blocks hold the gate and
//             up products of the same features and the gate is applied in registers.
//
// Block = 8 waves (512 lanes, two per SIMD) in a WM x WN grid (4 waves in 2 x 2 for the fp32
// kernel and as a tuning option), each wave owning a (BM/WM) x (BN/WN) output tile of
// 32 x 32 MFMA blocks (16 x 16 for the fp32 kernel). The K loop streams BK-wide slabs of A and B through a
// double-buffered LDS ring: the next slab is loaded from global memory directly into the
// other LDS buffer while the MFMAs run on the current one; one barrier per slab; the MFMA
// operand fragments are double-buffered in registers so LDS reads overlap the MFMAs. LDS rows are
// 128 bytes (8 chunks of 16 B). The LDS serves a 16-byte-per-lane read 16 lanes at a time
// from 64 four-byte banks (256 bytes), i.e. two consecutive 128-byte rows; chunk c of row r
// is stored at chunk c ^ ((r >> 1) & 7), so the 16 rows of one MFMA operand read (same
// logical chunk) land on 16 distinct 16-byte bank groups. (The fp32 kernel, which is not on
// the bf16 path, keeps c ^ (r & 7).)
//
// The MFMA is issued as D = B_frag * A_frag (weight rows as the "M" side), so each lane's
// four accumulator values are four consecutive output COLUMNS of one row: epilogue stores
// are 16-byte (fp32) or 8-byte (bf16) vectors, and the bias is one vector load.
#include <algorithm>
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace tps {
namespace {

constexpr int kThreads = 256;

// Map the linear block index to an output tile. Blocks are dealt round-robin to the 8 XCDs
// (block b runs on XCD b % 8); the remap gives each XCD a contiguous run of logical tiles,
// and logical tiles are ordered in bands of kGroupM tile-rows so that blocks running at the
// same time on one XCD share A rows and B columns in that XCD's L2.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& tm, int& tn,
                                            int bid = (int)blockIdx.x)
{
    constexpr int kXcd = 8, kGroupM = 4;
    const int nb = tiles_m * tiles_n;
    if (nb % kXcd == 0) bid = (bid % kXcd) * (nb / kXcd) + bid / kXcd;
    const int per_group = kGroupM * tiles_n;
    const int group = bid / per_group;
    const int first_m = group * kGroupM;
    const int gsz = min(tiles_m - first_m, kGroupM);
    const int in_group = bid - group * per_group;
    tm = first_m + in_group % gsz;
    tn = in_group / gsz;
}

// ---- output stage ------------------------------------------------------------------------
// v holds C[m, n .. n+3]; n is a multiple of 4 and N a multiple of 8, so all four are valid.
template <Epi EPI, typename T>
__device__ __forceinline__ void store_out(const GemmProblem& p, int m, int n, f32x4 v)
{
    if constexpr (EPI == Epi::F32) {
        float* c = reinterpret_cast<float*>(p.C) + (int64_t)m * p.ldc + n;
        *reinterpret_cast<f32x4*>(c) = v;
    } else {
        if (p.bias) {
            if constexpr (sizeof(T) == 2) {
                v += bf16x4_to_f32(*reinterpret_cast<const bf16x4*>(
                    reinterpret_cast<const bf16*>(p.bias) + n));
            } else {
                v += *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(p.bias) + n);
            }
        }
        if constexpr (EPI == Epi::GeluGrad) {   // dP = dY * GeLU'(P), bf16 only
            const f32x4 pre = bf16x4_to_f32(*reinterpret_cast<const bf16x4*>(
                reinterpret_cast<const bf16*>(p.aux) + (int64_t)m * p.ldaux + n));
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] *= gelu_erf_grad(pre[i]);
            bf16* c = reinterpret_cast<bf16*>(p.C) + (int64_t)m * p.ldc + n;
            *reinterpret_cast<bf16x4*>(c) = to_bf16x4(v);
        } else if constexpr (EPI == Epi::BiasGelu || EPI == Epi::Bias) {
            if constexpr (EPI == Epi::BiasGelu && sizeof(T) == 2) {
                if (p.pre)
                    *reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(p.pre) +
                                               (int64_t)m * p.ldc + n) = to_bf16x4(v);
            }
            if constexpr (EPI == Epi::BiasGelu) {
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = gelu_erf(v[i]);
            }
            if constexpr (sizeof(T) == 2) {
                bf16* c = reinterpret_cast<bf16*>(p.C) + (int64_t)m * p.ldc + n;
                *reinterpret_cast<bf16x4*>(c) = to_bf16x4(v);
            } else {
                float* c = reinterpret_cast<float*>(p.C) + (int64_t)m * p.ldc + n;
                *reinterpret_cast<f32x4*>(c) = v;
            }
        }
    }
}

__device__ __forceinline__ float silu(float x) { return x / (1.0f + __expf(-x)); }

// SwiGlu: the wave's 32-column blocks alternate gate (even) and up (odd) for the same 32
// features; combine each pair in place into the gated activation.
template <int FN, int FM>
__device__ __forceinline__ void swiglu_combine(f32x16 (&acc)[FN][FM], f32x16 (&out)[FN / 2][FM])
{
#pragma unroll
    for (int k = 0; k < FN / 2; ++k)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) out[k][j][v] = silu(acc[2 * k][j][v]) * acc[2 * k + 1][j][v];
}

// ---- bf16 GEMM ---------------------------------------------------------------------------
// Operand tiles are fetched with buffer loads: the descriptor's range ends at the last valid
// row of the tile, and a chunk past K is given an offset beyond the range, so out-of-range
// chunks read as zero with no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, int64_t row0,
                                                            int rows_valid, int64_t ld, int esz)
{
    const char* p = reinterpret_cast<const char*>(base) + row0 * ld * esz;
    const int64_t bytes = rows_valid > 0 ? (int64_t)rows_valid * ld * esz : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), (short)0,
                                             (int)(bytes < 0x7fffffff ? bytes : 0x7fffffff),
                                             0x00020000);
}

constexpr uint32_t kOutOfRange = 0x80000000u;

// s_waitcnt immediate for vmcnt(vm) expcnt(7) lgkmcnt(lgkm); vmcnt's two high bits sit at
// [15:14], so vm may reach 63 (63: no wait on vector memory).
constexpr int waitcnt_imm(int vm, int lgkm)
{
    return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8);
}

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>), in that order.
template <int N, typename F>
__device__ __forceinline__ void unroll_c(F&& f)
{
    if constexpr (N > 0) {
        unroll_c<N - 1>(f);
        f(std::integral_constant<int, N - 1>{});
    }
}

// Ring form of the fused partial sum: slabs a streamed vector's loads have to land (the K
// loop of a ring launch spans a multiple of this many slabs).
constexpr int kRingDepth = 4;

// Scheduling groups of one pipeline phase: after MFMA I come up to three fragment reads
// (front-loaded, so that the last read of the phase still has most of the phase's MFMAs to
// land before the next phase waits on it) and NV (I+1)/NM - NV I/NM slab loads (spread evenly
// between the phase's NM MFMAs). Masks: 0x8 MFMA, 0x100 LDS read, 0x20 global read.
template <int I, int NM, int NR, int NV>
struct InterleaveGroups {
    __device__ __forceinline__ static void emit()
    {
        if constexpr (I < NM) {
            constexpr int nr = NR - 3 * I < 0 ? 0 : (NR - 3 * I > 3 ? 3 : NR - 3 * I);
            constexpr int nv = NV * (I + 1) / NM - NV * I / NM;
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);
            if constexpr (nv > 0) __builtin_amdgcn_sched_group_barrier(0x020, nv, 0);
            InterleaveGroups<I + 1, NM, NR, NV>::emit();
        }
    }
};

// Scheduling groups of a phase whose fragment reads and slab loads are already interleaved
// in program order (the compiler keeps LDS reads and LDS-DMA loads in that order, since it
// cannot prove them disjoint): after MFMA I come NO (I+1)/NM - NO I/NM of the phase's NO
// memory operations, of either kind. Mask 0x120: LDS read or global read.
template <int I, int NM, int NO>
struct MixedOps {
    __device__ __forceinline__ static void emit()
    {
        if constexpr (I < NM) {
            constexpr int no = NO * (I + 1) / NM - NO * I / NM;
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            if constexpr (no > 0) __builtin_amdgcn_sched_group_barrier(0x120, no, 0);
            MixedOps<I + 1, NM, NO>::emit();
        }
    }
};

// ---- bf16 kernels' output stage -----------------------------------------------------------
// acc[i][j][4 q + v] of a wave holds C[r0 + 32 j + fr][c0 + 32 i + 8 q + 4 fg + v] (fr = lane & 31,
// fg = lane >> 5). Stored as it lies, one 16-byte vector per lane would put the 32 lanes of an
// instruction in 32 different rows. Instead each wave stages its tile through its own slice of
// the (now idle) operand LDS, FM / R block-rows at a time, and reads it back row-contiguously:
// consecutive lanes take consecutive 4-column vectors of one row, so every store instruction
// writes whole row segments. The staging rows are padded by 16 bytes, which puts the 16 rows
// written by one 16-lane pass on 16 distinct bank groups. The Qkv scatter reads the staged
// tile back in 8-element chunks along rows (queries, keys) or columns (values, transposed).
// Fewest rounds R (a divisor of the FM block-rows) whose FM / R block-rows of every wave fit
// in the LDS at once; bytes_per_block_row covers all the waves.
constexpr int staging_rounds(int fm, int bytes_per_block_row, int lds_bytes)
{
    for (int r = 1; r <= fm; ++r)
        if (fm % r == 0 && (fm / r) * bytes_per_block_row <= lds_bytes) return r;
    return fm + 1;   // does not fit even one block-row at a time: caught by the static_assert
}

// The Qkv scatter of one staged round: RR rows x WTN columns of fp32 at byte pitch PITCH, the
// round's origin at output row m0 and column c0. Query and key columns leave as 8-column row
// chunks (one 16-byte store into a head's [seq, d] row: consecutive lanes write consecutive
// chunks of a row); value columns as 8-token column chunks (one 16-byte store into the V^T row
// of that feature) when the sequence length is a multiple of 8, else token by token. The query
// columns are multiplied by q_scale after the bias. A chunk never straddles two heads (head
// widths are multiples of 8 and so are the chunks' first columns).
template <int WTN, int RR, int PITCH>
__device__ __forceinline__ void qkv_write(const GemmProblem& p, const char* region, int m0,
                                          int c0, int lane)
{
    const int d = p.head_dim;
    const int wq = p.heads_local * d;
    const int vlo = wq + p.kv_heads_local * d;   // first value column
    const bf16* bias = reinterpret_cast<const bf16*>(p.bias);
    if (c0 < vlo) {
        constexpr int C8 = WTN / 8, ITEMS = RR * C8;
#pragma unroll
        for (int t0 = 0; t0 < ITEMS; t0 += 64) {
            const int t = t0 + lane;
            const int row = t / C8, c8 = t - row * C8;
            const int m = m0 + row, n = c0 + 8 * c8;
            if (t >= ITEMS || m >= p.M || n >= vlo) continue;
            const f32x4 a = *reinterpret_cast<const f32x4*>(region + row * PITCH + c8 * 32);
            const f32x4 b = *reinterpret_cast<const f32x4*>(region + row * PITCH + c8 * 32 + 16);
            float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
            if (bias) {
                const bf16x8 bb = *reinterpret_cast<const bf16x8*>(bias + n);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] += static_cast<float>(bb[e]);
            }
            const bool isq = n < wq;
            const float sc = isq ? p.q_scale : 1.0f;
            const int rem = isq ? n : n - wq;
            const int head = rem / d, jj = rem - head * d;
            const int bb_ = m / p.seq, sq = m - bb_ * p.seq;
            const int64_t bh = (int64_t)bb_ * (isq ? p.heads_local : p.kv_heads_local) + head;
            bf16x8 o;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = to_bf16(v[e] * sc);
            bf16* dst = reinterpret_cast<bf16*>(isq ? p.q : p.k) + (bh * p.seq + sq) * d + jj;
            *reinterpret_cast<bf16x8*>(dst) = o;
        }
    }
    if (c0 + WTN > vlo) {
        constexpr int R8 = RR / 8, ITEMS = R8 * WTN;
        const bool vec = p.seq % 8 == 0;
#pragma unroll
        for (int t0 = 0; t0 < ITEMS; t0 += 64) {
            const int t = t0 + lane;
            const int rc = t / WTN, col = t - rc * WTN;
            const int n = c0 + col, mb = m0 + 8 * rc;
            if (t >= ITEMS || n < vlo || n >= p.N || mb >= p.M) continue;
            const float bv = bias ? static_cast<float>(bias[n]) : 0.0f;
            const int rem = n - vlo;
            const int head = rem / d, jj = rem - head * d;
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                v[e] = *reinterpret_cast<const float*>(region + (8 * rc + e) * PITCH + col * 4) + bv;
            bf16* vt = reinterpret_cast<bf16*>(p.vt);
            if (vec) {
                // seq % 8 == 0: the 8 tokens lie in one sequence, starting at a multiple of 8
                const int bb_ = mb / p.seq, sq = mb - bb_ * p.seq;
                bf16x8 o;
#pragma unroll
                for (int e = 0; e < 8; ++e) o[e] = to_bf16(v[e]);
                *reinterpret_cast<bf16x8*>(
                    vt + (((int64_t)bb_ * p.kv_heads_local + head) * d + jj) * p.ld_vt + sq) = o;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int m = mb + e;
                    if (m >= p.M) break;
                    const int bb_ = m / p.seq, sq = m - bb_ * p.seq;
                    vt[(((int64_t)bb_ * p.kv_heads_local + head) * d + jj) * p.ld_vt + sq] =
                        to_bf16(v[e]);
                }
            }
        }
    }
}

// ---- epilogue: every output type goes through LDS ---------------------------------------
// Each wave stages its accumulators (fp32) in its own region of the idle operand LDS, FM / R
// block-rows per round, then reads them back row-contiguously (the Qkv scatter: see qkv_write).
template <Epi EPI, int WTM, int WTN, int NW, int LDS_BYTES>
__device__ __forceinline__ void store_tile(const GemmProblem& p, f32x16 (&acc)[WTN / 32][WTM / 32],
                                           char* lds, int r0, int c0, int wave, int lane)
{
    constexpr int FM = WTM / 32, FN = WTN / 32;
    const int fr = lane & 31, fg = lane >> 5;
    constexpr int PITCH = WTN * 4 + 16;                 // bytes per staged row
    constexpr int R = staging_rounds(FM, NW * 32 * PITCH, LDS_BYTES);   // rounds
    constexpr int FMR = FM / R, RR = FMR * 32;          // block-rows and rows per round
    static_assert(NW * RR * PITCH <= LDS_BYTES, "staging does not fit");
    constexpr int V4 = WTN / 4;                         // 4-column vectors per row
    constexpr int PER_LANE = RR * V4 / 64;
    char* region = lds + wave * RR * PITCH;
    // Every wave is past its last operand read, and this wave's slab loads (including the
    // unused one past the end of K) have landed, before the operand LDS is overwritten.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
#pragma unroll
        for (int jj = 0; jj < FMR; ++jj)
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int j = rr * FMR + jj;
                    *reinterpret_cast<f32x4*>(region + (jj * 32 + fr) * PITCH +
                                              (i * 32 + 8 * q + 4 * fg) * 4) =
                        f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                              acc[i][j][4 * q + 3]};
                }
        __syncthreads();
        if constexpr (EPI == Epi::Qkv) {
            qkv_write<WTN, RR, PITCH>(p, region, r0 + rr * RR, c0, lane);
        } else if constexpr (EPI == Epi::SumF32 || EPI == Epi::SumBf16) {
            // SU vectors per pass (four with four waves, two with eight: the same bytes in
            // flight per compute unit): the other partials' loads of all of them are issued
            // before any add (streamed once: non-temporal), then each vector is summed in the
            // order q = 0 .. n_parts-1 with this product at q = part_rank -- the same fp32
            // adds, in the same order, as the partial-sum kernel.
            constexpr int SU = NW == 4 ? 4 : 2;
            static_assert(PER_LANE % SU == 0, "passes");
#pragma unroll
            for (int t = 0; t < PER_LANE; t += SU) {
                f32x4 own[SU], v[SU][kMaxSumParts];
                int64_t off[SU];
                bool ok[SU];
#pragma unroll
                for (int u = 0; u < SU; ++u) {
                    const int idx = lane + 64 * (t + u);
                    const int row = idx / V4, v4 = idx - row * V4;
                    const int m = r0 + rr * RR + row, n = c0 + v4 * 4;
                    ok[u] = m < p.M && n < p.N;
                    own[u] = *reinterpret_cast<const f32x4*>(region + row * PITCH + v4 * 16);
                    off[u] = (int64_t)m * p.ldc + n;
#pragma unroll
                    for (int q = 0; q < kMaxSumParts; ++q)
                        if (ok[u] && q < p.n_parts && q != p.part_rank)
                            v[u][q] = __builtin_nontemporal_load(
                                reinterpret_cast<const f32x4*>(p.part[q] + off[u]));
                }
#pragma unroll
                for (int u = 0; u < SU; ++u) {
                    if (!ok[u]) continue;
                    f32x4 acc = p.part_rank == 0 ? own[u] : v[u][0];
#pragma unroll
                    for (int q = 1; q < kMaxSumParts; ++q)
                        if (q < p.n_parts) acc += q == p.part_rank ? own[u] : v[u][q];
                    if constexpr (EPI == Epi::SumF32)
                        __builtin_nontemporal_store(
                            acc, reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.C) + off[u]));
                    else
                        __builtin_nontemporal_store(
                            to_bf16x4(acc), reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(p.C) + off[u]));
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < PER_LANE; ++t) {
                const int idx = lane + 64 * t;
                const int row = idx / V4, v4 = idx - row * V4;
                const f32x4 v = *reinterpret_cast<const f32x4*>(region + row * PITCH + v4 * 16);
                const int m = r0 + rr * RR + row, n = c0 + v4 * 4;
                if (m < p.M && n < p.N) store_out<EPI, bf16>(p, m, n, v);
            }
        }
        if (rr + 1 < R) __syncthreads();
    }
}

template <int BM, int BN, int WM, int WN, Epi EPI>
__global__ __launch_bounds__(64 * WM * WN) void gemm_bf16_kernel(GemmProblem p)
{
    constexpr int NW = WM * WN;             // waves per workgroup
    constexpr int BK = 64;                  // K per LDS slab: 128-byte rows, four MFMA K-steps
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;   // 32 x 32 MFMA blocks per wave
    constexpr int ACH = BM / 8 / NW;        // 8-row groups of the A slab per wave
    constexpr int BCH = BN / 8 / NW;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0 && FM >= 1 && FN >= 1, "tile");
    static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0 && NW % 2 == 0, "slab split");

    // two slab buffers, then a 256-byte sink for the weight prefetch below
    __shared__ __attribute__((aligned(16))) bf16 smem[2 * (BM + BN) * BK + 128];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    // SwiGlu: the B tile's BN rows are BN / 2 gate rows and the same BN / 2 up rows.
    constexpr bool GLU = EPI == Epi::SwiGlu;
    static_assert(!GLU || FN % 2 == 0, "SwiGlu pairs the wave's 32-column blocks");
    const int tiles_m = (p.M + BM - 1) / BM;
    const int tiles_n = ((GLU ? 2 * p.N : p.N) + BN - 1) / BN;
    // The fused partial sum in deferred form (p.defer): the workgroup takes two tiles, blocks
    // b and b + gridDim.x. The first tile's own product goes to C as an fp32 partial, and its
    // sum (the partials of every rank, in the fixed order) is streamed by the waves that load
    // no slabs while the second tile's K loop runs: the first tile is complete on every rank
    // by then. The second tile ends in the ordinary fused epilogue. PHASE: 0 the workgroup's
    // only tile, 1 the first of two, 2 the second of two, 3 a ring tile before the last (ring
    // form below), 4 the ring's last tile.
    constexpr bool DEFER = EPI == Epi::SumF32 && NW == 8;
    int dm0 = 0, dn0 = 0;        // origin of the tile whose sum is being streamed
    // Ring form (p.defer == 2; 128 x 128 tiles, eight waves): the workgroup takes the tiles
    // b, b + G, ..., b + (T - 1) G (G workgroups, T = p.ring_tiles). After each K loop but the
    // last, the tile's own product is staged in LDS (own_lds: fp32 rows padded by 16 bytes),
    // and during the next tile's K loop the waves that load no slabs stream its sum: at every
    // slab a lane finishes the vector whose loads it issued RD slabs before (the adds in the
    // fixed order, then one store) and issues the loads of its next vector, whose own part it
    // takes from LDS at once. A vector in flight carries its own part and its output offset in
    // registers, so the stream runs on across tile boundaries and own_lds is free again when
    // a K loop ends. The last tile ends in the ordinary fused epilogue. Each vector thus has RD
    // slabs to land, with RD x 7 loads of 16 bytes per streaming lane in flight (the peers'
    // partials; slots past n_parts re-read a peer's vector and their sum drops it, so the code
    // has no branch per slot). Vectors outside the tile (and the first tile's stream, which
    // has nothing to add) read offset 0 and store nothing. The K loop is exactly the 16 slabs
    // over which the 256 streaming lanes take the 4096 vectors of a tile, one per slab.
    constexpr bool RING = (EPI == Epi::SumF32 || EPI == Epi::SumBf16) && NW == 8 && BM == 128 &&
                          BN == 128;
    constexpr int RD = kRingDepth;
    constexpr int OWN_PITCH = BN + 4;         // floats per staged row
    // dynamic LDS, requested by ring launches only (BM x OWN_PITCH floats), so that the other
    // launches of this kernel keep two workgroups per compute unit
    extern __shared__ __attribute__((aligned(16))) float own_lds[];
    f32x4 rv[RING ? RD : 1][kMaxSumParts - 1];   // peers' partials of the vectors in flight
    f32x4 ro[RING ? RD : 1];                  // their own parts
    uint32_t roff[RING ? RD : 1];             // their element offsets in C
    bool rok[RING ? RD : 1];                  // a vector of the tile (else nothing is stored)
    int sm0 = p.M, sn0 = 0;                   // origin of the tile in own_lds (none: rows past M)
    const float* rP[kMaxSumParts - 1];   // slot j: partial j + (j >= part_rank), if any
    auto tile = [&](auto phase_c, const int bid, auto role_c) {
    constexpr int PHASE = decltype(phase_c)::value;
    // 0: the wave's role (slab loads or not) is decided here; 1 / 2: the caller runs the
    // loading (1) or the other (2) waves' code only (the ring form, whose stream state then
    // stays out of the loading waves' registers)
    constexpr int ROLE = decltype(role_c)::value;
    int tm, tn;
    if (EPI == Epi::F32 && p.k_splits > 1) {
        // group of blocks -> part of K: A, B and C move to the part, K to its length (a part
        // past the end has length <= 0 and writes zeros)
        const int tiles = tiles_m * tiles_n;
        const int split = bid / tiles;
        const int kc = ((p.K + p.k_splits - 1) / p.k_splits + BK - 1) / BK * BK;
        const int kb = split * kc;
        p.A = reinterpret_cast<const bf16*>(p.A) + kb;
        p.B = reinterpret_cast<const bf16*>(p.B) + kb;
        p.C = reinterpret_cast<float*>(p.C) + split * p.split_stride;
        p.K = max(min(p.K - kb, kc), 0);
        tile_coords(tiles_m, tiles_n, tm, tn, bid - split * tiles);
    } else {
        tile_coords(tiles_m, tiles_n, tm, tn, bid);
    }
    const int m0 = tm * BM, n0 = tn * BN;
    const int f0 = GLU ? n0 / 2 : n0;       // first B row (output feature) of the tile

    const __amdgpu_buffer_rsrc_t rA = tile_rsrc(p.A, m0, min(BM, p.M - m0), p.lda, 2);
    const __amdgpu_buffer_rsrc_t rB =
        tile_rsrc(p.B, f0, min(GLU ? BN / 2 : BN, p.N - f0), p.ldb, 2);
    const __amdgpu_buffer_rsrc_t rB2 =
        tile_rsrc(GLU ? p.B2 : p.B, f0, min(GLU ? BN / 2 : BN, p.N - f0), p.ldb, 2);

    // Slabs go from global memory straight into LDS (buffer_load ... lds): one instruction
    // moves 8 rows x 128 bytes, lane l writing the 16 bytes at byte 16 l of its wave's
    // destination, i.e. row (l >> 3), physical chunk (l & 7). The lane therefore fetches the
    // logical chunk that the XOR swizzle stores there: (l & 7) ^ ((row >> 1) & 7). Wave w
    // moves the 8-row groups w, w + NW, ... of each operand.
    const int grp_row = lane >> 3;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);   // scalar copy (descriptor choice)
    // row = 8 (wave + NW i) + grp_row with NW even, so (row >> 1) & 7 = 4 (wave & 1) + (lane >> 4)
    const int lchunk = (lane & 7) ^ (((wave & 1) << 2) + (lane >> 4));
    const uint32_t offA = (uint32_t)((wave * 8 + grp_row) * p.lda + lchunk * 8) * 2u;
    const uint32_t offB = (uint32_t)((wave * 8 + grp_row) * p.ldb + lchunk * 8) * 2u;
    const uint32_t stepA = (uint32_t)(8 * NW * p.lda) * 2u;
    const uint32_t stepB = (uint32_t)(8 * NW * p.ldb) * 2u;
    typedef __attribute__((address_space(3))) void* lds_ptr;

    // fetch_vw(vw, ...) issues the slab loads of wave slot vw (8-row groups vw, vw + NW, ...).
    // fetch(k0 >= K) moves no memory (every offset is out of range) and zero-fills the
    // buffer: the loop issues it unconditionally so that the loads stay in the same basic
    // block as the MFMAs they are scheduled between.
    auto fetch_vw_a = [&](int vw, int k0, int buf) {
        const bool kin = k0 + lchunk * 8 < p.K;
        const uint32_t kb = (uint32_t)k0 * 2u;
        const uint32_t dA = (uint32_t)((vw - wave) * 8 * p.lda) * 2u;
        bf16* sA = smem + buf * (BM + BN) * BK + vw * 8 * BK;
#pragma unroll
        for (int i = 0; i < ACH; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rA, (lds_ptr)(sA + i * 8 * NW * BK), 16,
                kin ? offA + dA + i * stepA + kb : kOutOfRange, 0, 0, 0);
    };
    auto fetch_vw_b = [&](int vw, int k0, int buf) {
        const bool kin = k0 + lchunk * 8 < p.K;
        const uint32_t kb = (uint32_t)k0 * 2u;
        const uint32_t dB = (uint32_t)((vw - wave) * 8 * p.ldb) * 2u;
        bf16* sB = smem + buf * (BM + BN) * BK + BM * BK + vw * 8 * BK;
#pragma unroll
        for (int i = 0; i < BCH; ++i) {
            if constexpr (GLU) {
                // LDS row group gi = vw + i NW lies in 32-row block gi / 4: even blocks hold
                // gate rows, odd ones the up rows of the same features.
                const int gi = vw + i * NW;
                const int blk = gi >> 2;
                const uint32_t off =
                    (uint32_t)((((blk >> 1) * 32 + (gi & 3) * 8 + grp_row) * p.ldb + lchunk * 8) * 2);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    (blk & 1) ? rB2 : rB, (lds_ptr)(sB + i * 8 * NW * BK), 16,
                    kin ? off + kb : kOutOfRange, 0, 0, 0);
            } else {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rB, (lds_ptr)(sB + i * 8 * NW * BK), 16,
                    kin ? offB + dB + i * stepB + kb : kOutOfRange, 0, 0, 0);
            }
        }
    };
    auto fetch_vw = [&](int vw, int k0, int buf) {
        fetch_vw_a(vw, k0, buf);
        fetch_vw_b(vw, k0, buf);
    };
    // With 8 waves, the waves of the first half (one per SIMD) issue the slab loads of both
    // halves and the other four issue none: a wave whose load cannot enter the full address
    // queue stalls its own later instructions, so keeping loads out of half of the waves
    // leaves each SIMD one wave that never waits on the queue. Wave slots w and w + NW/2 have
    // the same parity, so they share the lane's swizzled chunk.
    constexpr bool SPLIT_LOADS = NW == 8;
    auto fetch = [&](int k0, int buf, auto loader) {
        if constexpr (!SPLIT_LOADS) {
            fetch_vw(wave_u, k0, buf);
        } else if constexpr (decltype(loader)::value) {
            fetch_vw(wave_u, k0, buf);
            fetch_vw(wave_u + NW / 2, k0, buf);
        }
    };

    const int fr = lane & 31;   // operand row within a 32-row block
    const int fg = lane >> 5;   // which 8-wide half of the 16-wide MFMA K-step
    // Fragments of K-step ks (K = 16 ks ... 16 ks + 15 of the slab): chunk 2 ks + fg.
    auto read_frags = [&](int buf, int ks, bf16x8* fa, bf16x8* fb) {
        const bf16* sA = smem + buf * (BM + BN) * BK;
        const bf16* sB = sA + BM * BK;
        const int ch = ks * 2 + fg;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int r = wm * WTM + i * 32 + fr;
            fa[i] = *reinterpret_cast<const bf16x8*>(sA + r * BK + ((ch ^ ((r >> 1) & 7)) << 3));
        }
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            const int r = wn * WTN + i * 32 + fr;
            fb[i] = *reinterpret_cast<const bf16x8*>(sB + r * BK + ((ch ^ ((r >> 1) & 7)) << 3));
        }
    };

    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
    auto mma = [&](const bf16x8* fa, const bf16x8* fb) {
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j) acc[i][j] = mfma32x32x16(fb[i], fa[j], acc[i][j]);
    };

    // Software pipeline over slabs of four K-steps. Entering iteration kt, slab kt sits in
    // LDS buffer kt & 1 and the fragments of its K-step 0 are in set 0:
    //   start loading slab kt+1 into the other buffer (last read before the previous
    //   barrier) | read step 1 | MFMAs step 0 | read step 2 | MFMAs step 1 | read step 3 |
    //   MFMAs step 2 | wait for the slab, barrier | read slab kt+1 step 0 | MFMAs step 3.
    // Within each phase the fragment reads (and, in the first, the slab loads) are threaded
    // one by one between the MFMAs (sched_group_barrier), so the matrix core never waits for
    // a burst of memory instructions to issue; sched_barrier(0) fences the phases.
    constexpr int NM = FM * FN;          // MFMAs per K-step
    constexpr int NR = FM + FN;          // fragment reads per K-step
    constexpr int NV = ACH + BCH;        // slab load instructions per wave slot
    bf16x8 fa[2][FM], fb[2][FN];
    const int KT = (p.K + BK - 1) / BK;
    // The K loop, instantiated for waves that load (loader) and waves that do not.
    // Weight prefetch into the L2. The weight operand B is read once per layer step, so its
    // slabs arrive from HBM; the two-buffer LDS ring hides one slab of that latency. The
    // loading waves therefore also touch every 128-byte row segment of the B slab two slabs
    // ahead with a 4-byte LDS-DMA load into a 256-byte sink (no register destination, so
    // nothing ever waits on it early). Vector-memory loads complete in order, so the wait
    // before each barrier allows exactly these NPFT loads to stay in flight. The activations
    // (A) of the row-parallel GEMMs come from the kernel just before and are not prefetched
    // (that measured slower). The Q/K/V projection's A is the layer input, which the block's
    // other kernels have pushed out of the caches by then, and the MLP column GEMM's is the
    // attention block's sum, mostly evicted by the sum's own 1 GB of partials: both prefetch
    // their A slab rows as well. Layer step: the attention shard 350 -> 338 us, the column
    // GEMM 242 -> 238 us.
    constexpr int PFI = (BN + 255) / 256;   // weight prefetch instructions per loading wave
    constexpr int PFA = (EPI == Epi::Qkv || EPI == Epi::BiasGelu) ? (BM + 255) / 256 : 0;
    constexpr int NPFT = PFI + PFA;
    constexpr int kPrefetchAhead = 2;       // slabs
    // One workgroup per panel touches it: the workgroups of an XCD run its tiles in step, in
    // bands of 4 tile-rows by (for the usual shapes) 8 tile-columns (tile_coords), so the B
    // column panel of a band is shared by its 4 rows and the A row panel by 8 columns; the
    // first row (column) of each touches the panel for all. The others issue the same
    // instructions with out-of-range offsets (no memory access), which keeps every wave's
    // count of loads in flight the same. Layer step 1096 -> 1072 us (one box, alternating):
    // four and eight times fewer prefetch requests to the L2.
    const bool pf_b = tm % 4 == 0 || (tiles_m * tiles_n) % 8 != 0;
    const bool pf_a = tn % 8 == 0 || tiles_n % 8 != 0 || (tiles_m * tiles_n) % 8 != 0;
    auto prefetch = [&](int k0) {
        bf16* sink = smem + 2 * (BM + BN) * BK;
#pragma unroll
        for (int t = 0; t < PFA; ++t) {
            const int r = (t * 4 + (wave_u & 3)) * 64 + lane;   // a row of the A slab
            const uint32_t off =
                pf_a && k0 < p.K && r < BM ? (uint32_t)(r * p.lda + k0) * 2u : kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_ptr)sink, 4, off, 0, 0, 0);
        }
#pragma unroll
        for (int t = 0; t < PFI; ++t) {
            const int r0 = (t * 4 + (wave_u & 3)) * 64;   // a 64-row group of the B slab (scalar)
            const int r = r0 + lane;
            // SwiGlu: B rows [0, BN/2) of the gate, then the same features of the up weight
            const bool up = GLU && r0 >= BN / 2;
            const int rr = up ? r - BN / 2 : r;
            const uint32_t off =
                pf_b && k0 < p.K && r < BN ? (uint32_t)(rr * p.ldb + k0) * 2u : kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(up ? rB2 : rB, (lds_ptr)sink, 4, off, 0, 0, 0);
        }
    };
    // Streaming of the deferred tile's sum by the waves that load no slabs (NW / 2 x 64 lanes):
    // at slab kt each lane sums the vector whose loads it issued at slab kt - 1 (the partials of
    // every rank, the own one read back from C, added in the order 0 .. n_parts-1) and stores
    // it, then issues the loads of vector kt x lanes + its index. A tile of BM x BN / 4 vectors
    // needs BM x BN / 4 / lanes slabs (the launcher defers only when the K loop is that long,
    // and when C's byte offsets fit 31 bits). The code is branch-free: every slot is loaded
    // (slots past n_parts and lanes past the tile re-read C at a valid offset), and a slot
    // past n_parts is dropped by a select rather than added.
    constexpr int SLANES = NW / 2 * 64;
    constexpr int TVEC = BM * BN / 4;
    f32x4 sv[kMaxSumParts];
    uint32_t s_off = 0;
    bool s_ok = false;
    auto stream_base = [&](int q) {
        return reinterpret_cast<const char*>(
            q < p.n_parts && q != p.part_rank ? p.part[q] : reinterpret_cast<const float*>(p.C));
    };
    auto stream_finish = [&]() {
        f32x4 a = sv[0];
#pragma unroll
        for (int q = 1; q < kMaxSumParts; ++q) {
            const f32x4 t = a + sv[q];
            a = q < p.n_parts ? t : a;
        }
        if (s_ok)
            __builtin_nontemporal_store(
                a, reinterpret_cast<f32x4*>(reinterpret_cast<char*>(p.C) + s_off));
    };
    auto stream_step = [&](int kt) {
        if (kt > 0) {
            __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0): the previous slab's loads
            stream_finish();
        }
        const int v = kt * SLANES + (wave_u - NW / 2) * 64 + lane;
        const int row = v / (BN / 4), c4 = v - row * (BN / 4);
        const int m = dm0 + row, n = dn0 + 4 * c4;
        s_ok = v < TVEC && m < p.M && n < p.N;
        s_off = s_ok ? (uint32_t)(m * (int)p.ldc + n) * 4u : 0u;
#pragma unroll
        for (int q = 0; q < kMaxSumParts; ++q)
            sv[q] = __builtin_nontemporal_load(
                reinterpret_cast<const f32x4*>(stream_base(q) + s_off));
    };
    // Ring: issue vector kt x lanes + this lane's index of the tile in own_lds into slot U.
    auto ring_issue = [&](auto u_c, int kt) __attribute__((always_inline)) {
        constexpr int U = decltype(u_c)::value;
        const int v = kt * SLANES + (wave_u - NW / 2) * 64 + lane;
        const int row = v / (BN / 4), c4 = v - row * (BN / 4);
        const int m = sm0 + row, n = sn0 + 4 * c4;
        const bool ok = v < TVEC && m < p.M && n < p.N;
        rok[U] = ok;
        roff[U] = ok ? (uint32_t)(m * (int)p.ldc + n) : 0u;
        ro[U] = *reinterpret_cast<const f32x4*>(own_lds + (v < TVEC ? row : 0) * OWN_PITCH + 4 * c4);
        // global (not flat) loads: a flat load would also count against the LDS counter that
        // the fragment reads wait on
#pragma unroll
        for (int j = 0; j < kMaxSumParts - 1; ++j)
            rv[U][j] = __builtin_nontemporal_load(
                (__attribute__((address_space(1))) const f32x4*)(rP[j] + roff[U]));
    };
    // Ring: the sum of slot U's vector, q = 0 .. n_parts-1 with the own part at part_rank (the
    // adds of the in-epilogue form and of the partial-sum kernel), stored non-temporally.
    auto ring_finish = [&](auto u_c) __attribute__((always_inline)) {
        constexpr int U = decltype(u_c)::value;
        // position q holds slot q below the own rank, the own part at it, slot q - 1 above
        // (selects on uniform conditions: branches here were if-converted into more selects)
        f32x4 a = p.part_rank == 0 ? ro[U] : rv[U][0];
#pragma unroll
        for (int q = 1; q < kMaxSumParts; ++q) {
            const f32x4 x = q < p.part_rank ? rv[U][q < kMaxSumParts - 1 ? q : 0]
                                            : (q == p.part_rank ? ro[U] : rv[U][q - 1]);
            const f32x4 t = a + x;
            a = q < p.n_parts ? t : a;
        }
        if (rok[U]) {
            if constexpr (EPI == Epi::SumF32)
                __builtin_nontemporal_store(
                    a, reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.C) + roff[U]));
            else
                __builtin_nontemporal_store(
                    to_bf16x4(a), reinterpret_cast<bf16x4*>(reinterpret_cast<bf16*>(p.C) + roff[U]));
        }
    };
    // Ring, at slab kt: slot U's loads (issued RD slabs ago) have landed once at most the
    // 7 (RD - 1) loads issued since are in flight (vector-memory operations complete in order;
    // the stores in between only make the wait stricter).
    auto ring_step = [&](auto u_c, int kt) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(waitcnt_imm((kMaxSumParts - 1) * (RD - 1), 15));
        ring_finish(u_c);
        ring_issue(u_c, kt);
    };
    auto k_loop = [&](auto loader) {
        constexpr bool LD = !SPLIT_LOADS || decltype(loader)::value;   // this wave loads
        constexpr int NVW = !SPLIT_LOADS ? NV : (decltype(loader)::value ? 2 * NV : 0);
        constexpr bool RS = RING && PHASE >= 3 && !LD;                   // streams the ring
        // pre-barrier wait: loading waves let their prefetches stay in flight; streaming waves
        // their streamed loads and stores (the barrier only guards the slabs in LDS)
        constexpr int NPF = LD ? NPFT : (PHASE == 2 ? kMaxSumParts + 1 : 0);
        constexpr int BARW = RS ? waitcnt_imm(63, 0) : waitcnt_imm(NPF, 0);
        fetch(0, 0, loader);
#pragma unroll
        for (int d = 1; d < kPrefetchAhead; ++d)
            if constexpr (LD) prefetch(d * BK);
        if constexpr (RING && PHASE >= 3) {
            // slab 0 (and the LDS writes of own_lds before the loop) complete; the ring's
            // loads stay in flight
            __builtin_amdgcn_s_waitcnt(LD ? waitcnt_imm(NPFT * (kPrefetchAhead - 1), 0)
                                          : waitcnt_imm(63, 0));
            __builtin_amdgcn_s_barrier();
        } else {
            __syncthreads();
        }
        read_frags(0, 0, fa[0], fb[0]);
        auto slab = [&](int kt, auto u_c) __attribute__((always_inline)) {
            const int cur = kt & 1;
            __builtin_amdgcn_sched_barrier(0);
            fetch((kt + 1) * BK, cur ^ 1, loader);
            if constexpr (LD) prefetch((kt + kPrefetchAhead) * BK);
            read_frags(cur, 1, fa[1], fb[1]);
            mma(fa[0], fb[0]);
            InterleaveGroups<0, NM, NR, NVW + (LD ? NPF : 0)>::emit();
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (PHASE == 2 && !LD) {
                stream_step(kt);
                __builtin_amdgcn_sched_barrier(0);
            } else if constexpr (RS) {
                ring_step(u_c, kt);
                __builtin_amdgcn_sched_barrier(0);
            }
            read_frags(cur, 2, fa[0], fb[0]);
            mma(fa[1], fb[1]);
            InterleaveGroups<0, NM, NR, 0>::emit();
            __builtin_amdgcn_sched_barrier(0);
            read_frags(cur, 3, fa[1], fb[1]);
            mma(fa[0], fb[0]);
            InterleaveGroups<0, NM, NR, 0>::emit();
            __builtin_amdgcn_sched_barrier(0);
            // this wave's slab loads have landed (only its NPF newer prefetches may still be
            // in flight) and its fragment reads are done; then the workgroup barrier
            __builtin_amdgcn_s_waitcnt(BARW);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            read_frags(cur ^ 1, 0, fa[0], fb[0]);   // after the last slab: reads zeros, unused
            mma(fa[1], fb[1]);
            InterleaveGroups<0, NM, NR, 0>::emit();
            __builtin_amdgcn_sched_barrier(0);
        };
        if constexpr (RS) {
            // the ring's slot is a compile-time index: RD slabs per trip (KT is a multiple of RD)
            for (int kt = 0; kt < KT; kt += RD)
                unroll_c<RD>([&](auto u) __attribute__((always_inline)) {
                    slab(kt + decltype(u)::value, u);
                });
        } else {
            for (int kt = 0; kt < KT; ++kt) slab(kt, std::integral_constant<int, 0>{});
        }
    };
    // Four waves (one per SIMD, each a 128 x 128 block of the tile): a third fewer fragment
    // reads per MFMA than the eight-wave layout, but no second wave on the SIMD to cover a
    // stall. Per-phase cycle counts show that fragment reads and slab loads cost almost
    // nothing when each MFMA is followed by one or two of them, and stall the wave when they
    // come in bursts (the LDS or the address queue fills). So the fragments go through four
    // register sets, each read at least a phase before its MFMAs, and the phase's reads and
    // loads are issued alternately, in program order, one or two after each MFMA; the slab
    // loads are spread over three of the four phases, most of them in the two after the
    // barrier (7/16 each), which leaves the loads issued before it the longest time to land.
    // Iteration kt (slab kt in buffer
    // kt & 1, its K-steps 0 and 1 in sets 0 and 1):
    //   phase 0: MFMAs set 0 | read step 2 into set 2 and half of step 3 into set 3 + load
    //            part 2 of slab kt+1 (into buffer kt+1 & 1), then the prefetch |
    //   phase 1: MFMAs set 1 | early in the phase, the rest of step 3 |
    //   wait for slab kt+1, barrier (every wave is done with slab kt) |
    //   phase 2: MFMAs set 2 | read slab kt+1 step 0 into set 0 + load part 0 of slab kt+2
    //            into buffer kt & 1 |
    //   phase 3: MFMAs set 3 | read slab kt+1 step 1 into set 1 + load part 1 of slab kt+2.
    // The wait before the barrier lets only the prefetch, issued after part 2, stay in flight.
    constexpr int LW4 = ACH + BCH;                       // slab loads per wave
    constexpr int LP0 = (7 * LW4 + 8) / 16, LP1 = (7 * LW4 + 8) / 16, LP2 = LW4 - LP0 - LP1;
    auto load_one = [&](int j, int k0, int buf) {   // j is a constant once unrolled
        const uint32_t oob = (uint32_t)(k0 + lchunk * 8 >= p.K) << 31;
        const uint32_t kb = (uint32_t)k0 * 2u;
        bf16* sbuf = smem + buf * (BM + BN) * BK;
        if (j < ACH) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rA, (lds_ptr)(sbuf + wave_u * 8 * BK + j * 8 * NW * BK), 16,
                (offA + j * stepA + kb) | oob, 0, 0, 0);
        } else {
            const int i = j - ACH;
            bf16* sB = sbuf + BM * BK + wave_u * 8 * BK + i * 8 * NW * BK;
            if constexpr (GLU) {
                const int gi = wave_u + i * NW;
                const int blk = gi >> 2;
                const uint32_t off = (uint32_t)(
                    (((blk >> 1) * 32 + (gi & 3) * 8 + grp_row) * p.ldb + lchunk * 8) * 2);
                __builtin_amdgcn_raw_ptr_buffer_load_lds((blk & 1) ? rB2 : rB, (lds_ptr)sB, 16,
                                                         (off + kb) | oob, 0, 0, 0);
            } else {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rB, (lds_ptr)sB, 16, (offB + i * stepB + kb) | oob, 0, 0, 0);
            }
        }
    };
    // fragment idx of K-step ks: A fragments 0 .. FM-1, then B fragments
    auto read_one = [&](int buf, int ks, int idx, bf16x8* fa, bf16x8* fb) {
        const bf16* sA = smem + buf * (BM + BN) * BK;
        const bf16* sB = sA + BM * BK;
        const int ch = ks * 2 + fg;
        if (idx < FM) {
            const int r = wm * WTM + idx * 32 + fr;
            fa[idx] = *reinterpret_cast<const bf16x8*>(sA + r * BK + ((ch ^ ((r >> 1) & 7)) << 3));
        } else {
            const int r = wn * WTN + (idx - FM) * 32 + fr;
            fb[idx - FM] = *reinterpret_cast<const bf16x8*>(sB + r * BK + ((ch ^ ((r >> 1) & 7)) << 3));
        }
    };
    auto k_loop_deep = [&]() {
        bf16x8 ga[4][FM], gb[4][FN];
        fetch_vw(wave_u, 0, 0);
        __syncthreads();
        read_frags(0, 0, ga[0], gb[0]);
        read_frags(0, 1, ga[1], gb[1]);
#pragma unroll
        for (int j = 0; j < LP0 + LP1; ++j) load_one(j, BK, 1);
        for (int kt = 0; kt < KT; ++kt) {
            const int cur = kt & 1;
            __builtin_amdgcn_sched_barrier(0);
            mma(ga[0], gb[0]);
#pragma unroll
            for (int t = 0; t < NR + NR / 2; ++t) {
                const int set = 2 + t / NR;
                read_one(cur, set, t % NR, ga[set], gb[set]);
                if (t < LP2) load_one(LP0 + LP1 + t, (kt + 1) * BK, cur ^ 1);
            }
            prefetch((kt + kPrefetchAhead) * BK);
            MixedOps<0, NM, NR + NR / 2 + LP2 + NPFT>::emit();
            __builtin_amdgcn_sched_barrier(0);
            mma(ga[1], gb[1]);
#pragma unroll
            for (int t = NR / 2; t < NR; ++t) read_one(cur, 3, t, ga[3], gb[3]);
            MixedOps<0, NM / 2, NR - NR / 2>::emit();
            __builtin_amdgcn_sched_barrier(0);
            // this wave's loads of slab kt+1 have landed (its NPFT newer prefetches may still
            // be in flight) and its reads of slab kt are done; then the workgroup barrier
            __builtin_amdgcn_s_waitcnt(0x0070 | NPFT);   // vmcnt(NPFT) expcnt(7) lgkmcnt(0)
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            mma(ga[2], gb[2]);
#pragma unroll
            for (int t = 0; t < NR || t < LP0; ++t) {
                if (t < NR) read_one(cur ^ 1, 0, t, ga[0], gb[0]);   // after the last slab: zeros
                if (t < LP0) load_one(t, (kt + 2) * BK, cur);
            }
            MixedOps<0, NM, NR + LP0>::emit();
            __builtin_amdgcn_sched_barrier(0);
            mma(ga[3], gb[3]);
#pragma unroll
            for (int t = 0; t < NR || t < LP1; ++t) {
                if (t < NR) read_one(cur ^ 1, 1, t, ga[1], gb[1]);
                if (t < LP1) load_one(LP0 + t, (kt + 2) * BK, cur);
            }
            MixedOps<0, NM, NR + LP1>::emit();
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if constexpr (NW == 4) {
        k_loop_deep();
    } else if (ROLE == 1 || (ROLE == 0 && (!SPLIT_LOADS || wave_u < NW / 2))) {
        if constexpr (ROLE != 2) k_loop(std::true_type{});
    } else {
        k_loop(std::false_type{});
        if constexpr (PHASE == 2) {   // the vector loaded at the last slab
            __builtin_amdgcn_s_waitcnt(0x0F70);
            stream_finish();
        }
        if constexpr (RING && PHASE == 4) {   // the ring's last RD vectors, oldest first
            unroll_c<RD>([&](auto u) __attribute__((always_inline)) {
                __builtin_amdgcn_s_waitcnt(
                    waitcnt_imm((kMaxSumParts - 1) * (RD - 1 - decltype(u)::value), 15));
                ring_finish(u);
            });
        }
    }

    if constexpr (GLU) {
        f32x16 gacc[FN / 2][FM];
        swiglu_combine<FN, FM>(acc, gacc);
        store_tile<Epi::Bias, WTM, WTN / 2, NW, (int)sizeof(smem)>(
            p, gacc, reinterpret_cast<char*>(smem), m0 + wm * WTM, f0 + wn * (WTN / 2), wave, lane);
    } else if constexpr (PHASE == 3) {
        // Ring: the product goes to own_lds once every wave is done with its LDS reads (the
        // slabs, and own_lds for the previous tile's stream). The loading waves also wait for
        // their last (out-of-range) loads, so that no LDS-DMA write is pending past this point.
        __builtin_amdgcn_s_waitcnt(ROLE == 1 ? waitcnt_imm(0, 0) : waitcnt_imm(63, 0));
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<f32x4*>(own_lds + (wm * WTM + j * 32 + fr) * OWN_PITCH +
                                              wn * WTN + i * 32 + 8 * q + 4 * fg) =
                        f32x4{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                              acc[i][j][4 * q + 3]};
        sm0 = m0;
        sn0 = n0;
    } else if constexpr (PHASE == 1) {
        // the own product of the first tile goes to C; its sum is streamed during the next
        // tile's K loop, once every wave's stores have completed
        store_tile<Epi::F32, WTM, WTN, NW, (int)sizeof(smem)>(p, acc, reinterpret_cast<char*>(smem),
                                                            m0 + wm * WTM, n0 + wn * WTN, wave, lane);
        __builtin_amdgcn_s_waitcnt(0);
        dm0 = m0;
        dn0 = n0;
    } else {
        store_tile<EPI, WTM, WTN, NW, (int)sizeof(smem)>(p, acc, reinterpret_cast<char*>(smem),
                                                       m0 + wm * WTM, n0 + wn * WTN, wave, lane);
    }
    };
    if constexpr (RING) {
        if (p.defer == 2) {
#pragma unroll
            for (int u = 0; u < RD; ++u) {
                ro[u] = f32x4{0.f, 0.f, 0.f, 0.f};
                roff[u] = 0;
                rok[u] = false;
#pragma unroll
                for (int j = 0; j < kMaxSumParts - 1; ++j) rv[u][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            // a slot past the partials re-reads the first peer's vector (its sum drops it)
#pragma unroll
            for (int j = 0; j < kMaxSumParts - 1; ++j) {
                const int q = j + (j >= p.part_rank ? 1 : 0);
                rP[j] = q < p.n_parts ? p.part[q] : p.part[p.part_rank == 0 ? 1 : 0];
            }
            const int G = (int)gridDim.x;
            auto ring = [&](auto role) __attribute__((always_inline)) {
                for (int j = 0; j + 1 < p.ring_tiles; ++j)
                    tile(std::integral_constant<int, 3>{}, (int)blockIdx.x + j * G, role);
                tile(std::integral_constant<int, 4>{}, (int)blockIdx.x + (p.ring_tiles - 1) * G,
                     role);
            };
            if (__builtin_amdgcn_readfirstlane(wave) < NW / 2)
                ring(std::integral_constant<int, 1>{});
            else
                ring(std::integral_constant<int, 2>{});
            return;
        }
    }
    if constexpr (DEFER) {
        if (p.defer == 1) {
            tile(std::integral_constant<int, 1>{}, (int)blockIdx.x, std::integral_constant<int, 0>{});
            __syncthreads();   // every wave's stores of the first tile have completed
            tile(std::integral_constant<int, 2>{}, (int)blockIdx.x + (int)gridDim.x,
                 std::integral_constant<int, 0>{});
            return;
        }
    }
    tile(std::integral_constant<int, 0>{}, (int)blockIdx.x, std::integral_constant<int, 0>{});
}

// ---- fp32 GEMM (true fp32 products, v_mfma_f32_16x16x4_f32) -------------------------------
// Same structure; a 16-byte chunk holds 4 fp32 K values, BK = 32 (128-byte rows again). Lane
// l reads chunk 4*ks + (l >> 4) and feeds its 4 values to 4 consecutive MFMAs, so MFMA t of
// step ks consumes K = 4*(4*ks + g) + t on lane group g, identically for both operands.
template <int BM, int BN, Epi EPI>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmProblem p)
{
    constexpr int BK = 32;
    constexpr int WTM = BM / 2, WTN = BN / 2;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int ACH = BM * 8 / kThreads;
    constexpr int BCH = BN * 8 / kThreads;
    static_assert(FM >= 1 && FN >= 1 && ACH >= 1 && BCH >= 1, "tile");

    __shared__ __attribute__((aligned(16))) float smem[2 * (BM + BN) * BK];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles_m = (p.M + BM - 1) / BM;
    const int tiles_n = (p.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(tiles_m, tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const float* __restrict__ gA = reinterpret_cast<const float*>(p.A);
    const float* __restrict__ gB = reinterpret_cast<const float*>(p.B);

    const int lc = tid & 7;
    const int lr = tid >> 3;
    u32x4 ra[ACH], rb[BCH];
    auto fetch = [&](int k0) {
        const int kk = k0 + lc * 4;
        const bool kin = kk < p.K;   // K is a multiple of 8, so a chunk is all in or all out
#pragma unroll
        for (int i = 0; i < ACH; ++i) {
            const int gm = m0 + lr + 32 * i;
            ra[i] = (kin && gm < p.M) ? ld16(gA + (int64_t)gm * p.lda + kk) : zero16();
        }
#pragma unroll
        for (int i = 0; i < BCH; ++i) {
            const int gn = n0 + lr + 32 * i;
            rb[i] = (kin && gn < p.N) ? ld16(gB + (int64_t)gn * p.ldb + kk) : zero16();
        }
    };
    auto stash = [&](int buf) {
        float* sA = smem + buf * (BM + BN) * BK;
        float* sB = sA + BM * BK;
#pragma unroll
        for (int i = 0; i < ACH; ++i) {
            const int r = lr + 32 * i;
            st16(sA + r * BK + ((lc ^ (r & 7)) << 2), ra[i]);
        }
#pragma unroll
        for (int i = 0; i < BCH; ++i) {
            const int r = lr + 32 * i;
            st16(sB + r * BK + ((lc ^ (r & 7)) << 2), rb[i]);
        }
    };

    f32x4 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int KT = (p.K + BK - 1) / BK;
    fetch(0);
    stash(0);
    __syncthreads();
    const int fr = lane & 15;
    const int fg = lane >> 4;
    for (int kt = 0; kt < KT; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < KT) fetch((kt + 1) * BK);
        const float* sA = smem + cur * (BM + BN) * BK;
        const float* sB = sA + BM * BK;
#pragma unroll
        for (int ks = 0; ks < BK / 16; ++ks) {
            const int ch = ks * 4 + fg;
            f32x4 fa[FM], fb[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int r = wm * WTM + i * 16 + fr;
                fa[i] = *reinterpret_cast<const f32x4*>(sA + r * BK + ((ch ^ (r & 7)) << 2));
            }
#pragma unroll
            for (int i = 0; i < FN; ++i) {
                const int r = wn * WTN + i * 16 + fr;
                fb[i] = *reinterpret_cast<const f32x4*>(sB + r * BK + ((ch ^ (r & 7)) << 2));
            }
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int i = 0; i < FN; ++i)
#pragma unroll
                    for (int j = 0; j < FM; ++j)
                        acc[i][j] = mfma16x16x4f32(fb[i][t], fa[j][t], acc[i][j]);
        }
        if (kt + 1 < KT) stash(cur ^ 1);
        __syncthreads();
    }
#pragma unroll
    for (int j = 0; j < FM; ++j) {
        const int m = m0 + wm * WTM + j * 16 + fr;
        if (m >= p.M) continue;
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            const int n = n0 + wn * WTN + i * 16 + 4 * fg;
            if (n < p.N) store_out<EPI, float>(p, m, n, acc[i][j]);
        }
    }
}

// ---- fp32 GEMM for few rows (M <= 64) ------------------------------------------------------
// With a handful of token rows (32 in the fp32 worked example) the product streams its weight
// once and does little arithmetic per byte; a grid of 32 x 64 tiles leaves most compute units
// idle and each workgroup walks the whole K range alone. Here a workgroup owns 16 output
// columns (one MFMA block-column) for all M rows and its sixteen waves split K: each wave loads
// the 16-byte chunks of its K range straight into MFMA operands (lane l: weight row (l & 15)
// or activation row (l & 15), the 4 consecutive K values at 4 (l >> 4) of a 16-wide chunk,
// fed to 4 consecutive MFMAs as in gemm_f32_kernel), the waves' partial accumulators are
// added through LDS in the fixed order 0 .. 15, and the epilogue runs once per output vector.
// Sixteen waves put a wave's whole K range (128 values at K = 2048) in flight at once. When
// the column blocks alone leave compute units idle, the rows are split too: workgroup
// (x, y) takes the MB 16-row blocks from y MB on (the same per-element arithmetic).
template <int MB, Epi EPI>
__global__ __launch_bounds__(1024) void gemm_f32_skinny_kernel(GemmProblem p)
{
    constexpr int NWV = 16;                     // waves
    constexpr int UNR = MB <= 2 ? 8 : 4;        // 16-wide K chunks in flight per wave
    __shared__ f32x4 part[NWV][MB][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n0 = blockIdx.x * 16;
    const int mrow0 = blockIdx.y * MB * 16;     // first row of this workgroup's blocks
    const int fr = lane & 15, fg = lane >> 4;
    const float* __restrict__ gA = reinterpret_cast<const float*>(p.A);
    const float* __restrict__ gB = reinterpret_cast<const float*>(p.B);
    const int nrow = n0 + fr;                   // the weight row (output column) this lane loads
    const bool nin = nrow < p.N;
    const int chunks = (p.K + 15) / 16;
    const int c_lo = wave * chunks / NWV, c_hi = (wave + 1) * chunks / NWV;
    f32x4 acc[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c0 = c_lo; c0 < c_hi; c0 += UNR) {
        u32x4 rb[UNR], ra[UNR][MB];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int k = (c0 + u) * 16 + 4 * fg;
            const bool kin = c0 + u < c_hi && k < p.K;   // K % 4 == 0: a chunk is in or out
            rb[u] = kin && nin ? ld16(gB + (int64_t)nrow * p.ldb + k) : zero16();
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const int m = mrow0 + mb * 16 + fr;
                ra[u][mb] = kin && m < p.M ? ld16(gA + (int64_t)m * p.lda + k) : zero16();
            }
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const f32x4 fb = __builtin_bit_cast(f32x4, rb[u]);
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int mb = 0; mb < MB; ++mb)
                    acc[mb] = mfma16x16x4f32(fb[t], __builtin_bit_cast(f32x4, ra[u][mb])[t], acc[mb]);
        }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) part[wave][mb][lane] = acc[mb];
    __syncthreads();
    if (wave != 0) return;
    // lane holds C[m][n0 + 4 fg + i], i = 0..3, m = 16 mb + fr
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        f32x4 v = part[0][mb][lane];
#pragma unroll
        for (int w = 1; w < NWV; ++w) v += part[w][mb][lane];
        const int m = mrow0 + mb * 16 + fr, n = n0 + 4 * fg;
        if (m < p.M && n < p.N) store_out<EPI, float>(p, m, n, v);
    }
}

// Ring form of the fused partial sum (128 x 128 tiles, eight waves; see the kernel), for a
// short K loop, where streaming the peers' partials outweighs the product: the tiles divide
// into rounds of 256 workgroups (each workgroup then takes tiles / 256 of them, all on its
// XCD), the K loop is the 16 slabs over which the next tile streams the 4096 vectors of one
// tile (K in (960, 1024]), the partials' byte offsets fit 31 bits, and there are partials to
// add. The output projection (4096 x 8192 x 1024 with 8 partials, bf16 H): 246 -> 230 us.
// With a longer K loop the 128 x 128 product costs more than the stream saves (the MLP row
// GEMM with its sum, K = 4096, keeps 256 x 256 tiles and the two-tile deferred form). The
// test override "sum_ring=1" turns it off.
static bool ring_feasible(const GemmProblem& p, Epi epi)
{
    if ((epi != Epi::SumF32 && epi != Epi::SumBf16) || tuning().sum_ring == 1) return false;
    const long tiles = (long)((p.M + 127) / 128) * ((p.N + 127) / 128);
    const int kt = (p.K + 63) / 64;
    static_assert(16 % kRingDepth == 0, "ring slots per K loop");
    return p.n_parts >= 2 && tiles % 256 == 0 && tiles / 256 >= 2 && kt == 16 &&
           (int64_t)p.M * p.ldc * 4 <= INT32_MAX;
}

// Form of a fused-sum launch with this tile: 2 ring, 1 deferred (two tiles per workgroup,
// when half the tiles still give every CU a workgroup and each XCD keeps its own tiles, the
// grid a multiple of 8, and the second tile's K loop has a slab per 256-lane pass over the
// first tile's vectors), 0 the sum in each tile's own epilogue.
static int fused_form(const GemmProblem& p, Epi epi, int bm, int bn, int nw)
{
    if (epi != Epi::SumF32 && epi != Epi::SumBf16) return 0;
    if (bm == 128 && bn == 128 && nw == 8 && ring_feasible(p, epi)) return 2;
    const long tiles = (long)((p.M + bm - 1) / bm) * ((p.N + bn - 1) / bn);
    if (epi == Epi::SumF32 && nw == 8 && tiles % 16 == 0 && tiles / 2 >= 256 &&
        (p.K + 63) / 64 >= bm * bn / 4 / 256 && (int64_t)p.M * p.ldc * 4 <= INT32_MAX &&
        !tuning().sum_nodefer)
        return 1;
    return 0;
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_bf16(const GemmProblem& p, Epi epi, hipStream_t s)
{
    const int ncols = epi == Epi::SwiGlu ? 2 * p.N : p.N;   // gate and up columns
    const int tiles = ((p.M + BM - 1) / BM) * ((ncols + BN - 1) / BN);
    const int splits = epi == Epi::F32 && p.k_splits > 1 ? p.k_splits : 1;
    GemmProblem q = p;
    q.defer = fused_form(p, epi, BM, BN, WM * WN);
    q.ring_tiles = q.defer == 2 ? tiles / 256 : 0;
    dim3 grid(q.defer == 2 ? 256 : q.defer == 1 ? tiles / 2 : tiles * splits),
        block(64 * WM * WN);
    // the ring's product buffer (dynamic LDS): BM rows of BN + 4 floats
    const size_t dyn = q.defer == 2 ? (size_t)BM * (BN + 4) * 4 : 0;
#define TPS_LAUNCH(E) \
    hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WM, WN, E>), grid, block, dyn, s, q);
    switch (epi) {
        case Epi::BiasGelu: TPS_LAUNCH(Epi::BiasGelu) break;
        case Epi::F32: TPS_LAUNCH(Epi::F32) break;
        case Epi::Qkv: TPS_LAUNCH(Epi::Qkv) break;
        case Epi::Bias: TPS_LAUNCH(Epi::Bias) break;
        case Epi::GeluGrad: TPS_LAUNCH(Epi::GeluGrad) break;
        case Epi::SumF32: TPS_LAUNCH(Epi::SumF32) break;
        case Epi::SumBf16: TPS_LAUNCH(Epi::SumBf16) break;
        case Epi::SwiGlu:
            if constexpr ((BN / WN / 32) % 2 == 0) {
                TPS_LAUNCH(Epi::SwiGlu)
            } else {
                return hipErrorInvalidValue;   // the wave's column blocks do not pair up
            }
            break;
    }
#undef TPS_LAUNCH
    return hipGetLastError();
}

}  // namespace

// Choose the tile that minimises (waves of 256 workgroups) x (tile area) x (per-flop cost of
// the tile shape); larger tiles re-read less operand data per MFMA.
GemmTile gemm_bf16_pick_tile(int M, int N, int K)
{
    (void)K;
    struct Cand { int bm, bn; double cost; };
    const Cand cands[] = {{256, 256, 1.00}, {256, 192, 1.04}, {256, 128, 1.12}, {128, 128, 1.35}};
    GemmTile best{128, 128};
    double best_t = 1e300;
    for (const Cand& c : cands) {
        const long tiles = (long)((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
        const long waves = (tiles + 255) / 256;
        const double t = (double)waves * c.bm * c.bn * c.cost;
        if (t < best_t - 1e-9) { best_t = t; best = GemmTile{c.bm, c.bn}; }
    }
    // Two 128 x 128 workgroups fit on one CU (64 KB of LDS each), which the model above does
    // not count. When the chosen 256-row tiles would leave more than 30 % of the CUs idle and
    // 128 x 128 tiles fill at most one round of 512 resident workgroups, the smaller tiles
    // win: 4096 x 1280 x 8192 (a grouped-query QKV shard) runs 160 tiles of 256 x 128 in
    // 144.5 us and 320 of 128 x 128 in 136.9 us.
    if (best.bm == 256) {
        const long tiles = (long)((M + best.bm - 1) / best.bm) * ((N + best.bn - 1) / best.bn);
        const long small = (long)((M + 127) / 128) * ((N + 127) / 128);
        if (tiles * 10 < 256 * 7 && small > 256 && small <= 512) best = GemmTile{128, 128};
    }
    return best;
}

// The test override (tp_set_test_overrides "gemm_tile=<bm>x<bn>[w4]") replaces the choice
// with one of the compiled shapes; "w4" selects the 4-wave layout instead of the default
// 8-wave one. Tests use it to run every tile layout.
static bool tile_override(GemmTile& t, bool& w4)
{
    const Tuning tu = tuning();
    if (tu.gemm_bm == 0) return false;
    t = GemmTile{tu.gemm_bm, tu.gemm_bn};
    w4 = tu.gemm_w4 != 0;
    return true;
}

// Four waves per workgroup (one per SIMD, 128 x 128 each) instead of eight for 256 x 256
// tiles when the launch has at least two of them per CU and K spans at least 32 slabs: a
// third fewer fragment reads per MFMA; the longer prologue and epilogue of a 4-wave
// workgroup need the second tile and the long K loop to pay off. Hot operands, one MI355X:
// 4096 x 8192 x 4096 (512 tiles) 1300 against 1267 TFLOP/s, 8192^3 1343 against 1314; one
// tile per CU (4096 x 4096 x 8192) 1226 against 1260. In the layer step: the MLP row GEMM
// 233 against 239 us, but the output projection (K = 1024) 3 us slower. The Qkv scatter
// keeps eight waves: its 4-wave build measured slower at 768 tiles (16384 x 3072 x 8192: 799
// against 691 us) as at one tile per CU (4096 x 3072 x 8192, 256 x 192: 219 against 195 us).
// 256 x 192 tiles follow the same rule: on the MLP block's row GEMMs (512 tiles) 2381 against
// 2500 us at 2048 x 12288 x 49152 and 1068 against 1175 us at K = 24576.
static bool prefer_four_waves(int M, int N, int K, GemmTile t, Epi epi)
{
    // The fused partial sum streams N - 1 partials in its epilogue, which one wave per SIMD
    // leaves latency-bound (4096 x 8192 x 4096 with 8 partials: 606 us against 405 us for the
    // product and a separate sum): it keeps eight waves.
    if (epi == Epi::SumF32 || epi == Epi::SumBf16) return false;
    if (t.bm != 256 || (t.bn != 256 && t.bn != 192) || epi == Epi::Qkv || K < 2048) return false;
    const long tiles = (long)((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
    return tiles >= 512;
}

GemmTile gemm_bf16_launch_tile(int M, int N, int K, int* waves)
{
    GemmTile t = gemm_bf16_pick_tile(M, N, K);
    bool w4 = prefer_four_waves(M, N, K, t, Epi::F32);
    tile_override(t, w4);
    if (waves) *waves = w4 ? 4 : 8;
    return t;
}

hipError_t gemm_bf16_tile(const GemmProblem& p, Epi epi, hipStream_t s, GemmTile t, bool w4)
{
    if (t.bm == 256 && t.bn == 256)
        return w4 ? launch_bf16<256, 256, 2, 2>(p, epi, s) : launch_bf16<256, 256, 2, 4>(p, epi, s);
    if (t.bm == 256 && t.bn == 192)
        return w4 ? launch_bf16<256, 192, 2, 2>(p, epi, s) : launch_bf16<256, 192, 4, 2>(p, epi, s);
    if (t.bm == 256 && t.bn == 128)
        return w4 ? launch_bf16<256, 128, 2, 2>(p, epi, s) : launch_bf16<256, 128, 4, 2>(p, epi, s);
    return w4 ? launch_bf16<128, 128, 2, 2>(p, epi, s) : launch_bf16<128, 128, 2, 4>(p, epi, s);
}

// Eight waves (two per SIMD) per workgroup by default: while one wave of a SIMD waits on
// LDS or the slab barrier, the other keeps the matrix core busy.
// SwiGlu needs an even number of 32-column blocks per wave (gate / up pairs): the 8-wave
// 256 x 256 (64 columns per wave) and 256 x 128 (64) layouts and the 4-wave ones except
// 256 x 192.
static bool glu_ok(GemmTile t, bool w4)
{
    if (w4) return t.bn != 192;
    return (t.bm == 256 && t.bn == 256) || (t.bm == 256 && t.bn == 128);
}

static GemmTile glu_pick_tile(int M, int N, int K, bool* w4)
{
    // same cost model as gemm_bf16_pick_tile over the 2 N gate and up columns
    struct Cand { int bm, bn; bool w4; double cost; };
    const Cand cands[] = {{256, 256, false, 1.00}, {256, 128, false, 1.12}, {128, 128, true, 1.45}};
    GemmTile best{256, 256};
    bool bw4 = false;
    double best_t = 1e300;
    for (const Cand& c : cands) {
        const long tiles = (long)((M + c.bm - 1) / c.bm) * ((2L * N + c.bn - 1) / c.bn);
        const double t = (double)((tiles + 255) / 256) * c.bm * c.bn * c.cost;
        if (t < best_t - 1e-9) { best_t = t; best = GemmTile{c.bm, c.bn}; bw4 = c.w4; }
    }
    // 256 x 256 with more than one tile per CU and a long K loop: four waves (the gated MLP
    // shard 4096 x 8192 x 28672, 448 gate/up tiles: 656 against 671 us for the whole shard)
    if (best.bm == 256 && best.bn == 256 && K >= 2048 &&
        (long)((M + 255) / 256) * ((2L * N + 255) / 256) > 256)
        bw4 = true;
    *w4 = bw4;
    return best;
}

// The tile and layout gemm_bf16 launches for this problem and epilogue.
static GemmTile choose_tile(const GemmProblem& p, Epi epi, bool& w4)
{
    w4 = false;
    GemmTile t;
    if (epi == Epi::SwiGlu) {
        t = glu_pick_tile(p.M, p.N, p.K, &w4);
        GemmTile o = t;
        bool ow4 = false;
        if (tile_override(o, ow4) && glu_ok(o, ow4)) { t = o; w4 = ow4; }
    } else if (epi == Epi::F32 && p.k_splits > 1) {
        // a K-split launch exists to fill the compute units with the largest tile
        t = GemmTile{256, 256};
        tile_override(t, w4);
    } else {
        t = gemm_bf16_pick_tile(p.M, p.N, p.K);
        w4 = prefer_four_waves(p.M, p.N, p.K, t, epi);
        if (ring_feasible(p, epi)) {
            t = GemmTile{128, 128};
            w4 = false;
        }
        tile_override(t, w4);
    }
    return t;
}

hipError_t gemm_bf16(const GemmProblem& p, Epi epi, hipStream_t s)
{
    bool w4 = false;
    const GemmTile t = choose_tile(p, epi, w4);
    return gemm_bf16_tile(p, epi, s, t, w4);
}

GemmTile gemm_bf16_sum_launch_tile(int M, int N, int K, int n_parts, bool bf16_out, int* waves,
                                   int* form)
{
    GemmProblem p{};
    p.M = M;
    p.N = N;
    p.K = K;
    p.lda = K;
    p.ldb = K;
    p.ldc = N;
    p.n_parts = n_parts;
    const Epi epi = bf16_out ? Epi::SumBf16 : Epi::SumF32;
    bool w4 = false;
    const GemmTile t = choose_tile(p, epi, w4);
    *waves = w4 ? 4 : 8;
    *form = fused_form(p, epi, t.bm, t.bn, *waves);
    return t;
}

// A Q/K/V projection with few output columns (grouped-query attention: 4096 x 1280 x 8192
// on a rank with 8 query and one key/value head) gives 80 tiles of 256 x 256 for 256 CUs,
// and smaller tiles run at a much lower rate. Cutting K into S parts gives S times the
// blocks; the parts' fp32 sums go through qkv_reduce_scatter. S = min(4, 256 / tiles) when
// the tiles fill at most half of the CUs and K is at least 4096. The test override
// "qkv_split=<1..8>" replaces the count (the workspace size follows it).
int qkv_k_splits(int M, int N, int K)
{
    const long tiles = (long)((M + 255) / 256) * ((N + 255) / 256);
    int s = 1;
    if (2 * tiles <= 256 && K >= 4096) s = (int)std::min<long>(4, 256 / std::max<long>(tiles, 1));
    if (const int v = tuning().qkv_split) s = v;
    return s;
}

namespace {

// One block per 32 x 64 tile of the [M, N] projection. Each thread first sums 8 consecutive
// columns of one row over the parts (in the fixed order 0, 1, ..., so the result does not
// depend on timing), adds the bias, scales the query columns and stages them in LDS; then
// query and key tiles leave as 8-column row chunks (one 16-byte store into a head's [seq, d]
// row) and value tiles as 8-token column chunks of V^T when the sequence length is a
// multiple of 8, else token by token. The query, key and value widths are multiples of 64,
// so a tile never straddles two of them or two heads.
constexpr int kRsRows = 32, kRsCols = 64;
__global__ __launch_bounds__(256) void qkv_reduce_scatter_kernel(GemmProblem p, const float* parts)
{
    __shared__ float tile[kRsRows][kRsCols + 4];
    const int tiles_n = p.N / kRsCols;
    const int tr = (int)blockIdx.x / tiles_n, tc = (int)blockIdx.x - tr * tiles_n;
    const int m0 = tr * kRsRows, n0 = tc * kRsCols;
    const int t = threadIdx.x;
    const int d = p.head_dim;
    const int wq = p.heads_local * d, wkv = p.kv_heads_local * d;
    {
        const int r = t >> 3, c8 = (t & 7) * 8;
        const int m = m0 + r, n = n0 + c8;
        if (m < p.M) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f}, b = {0.f, 0.f, 0.f, 0.f};
            for (int sp = 0; sp < p.k_splits; ++sp) {
                const float* src = parts + sp * p.split_stride + (int64_t)m * p.N + n;
                a += *reinterpret_cast<const f32x4*>(src);
                b += *reinterpret_cast<const f32x4*>(src + 4);
            }
            if (p.bias) {
                const bf16* bias = reinterpret_cast<const bf16*>(p.bias) + n;
                a += bf16x4_to_f32(*reinterpret_cast<const bf16x4*>(bias));
                b += bf16x4_to_f32(*reinterpret_cast<const bf16x4*>(bias + 4));
            }
            if (n < wq) {
                a *= p.q_scale;
                b *= p.q_scale;
            }
            *reinterpret_cast<f32x4*>(&tile[r][c8]) = a;
            *reinterpret_cast<f32x4*>(&tile[r][c8 + 4]) = b;
        }
    }
    __syncthreads();
    if (n0 < wq + wkv) {   // query or key columns
        const int r = t >> 3, c8 = (t & 7) * 8;
        const int m = m0 + r;
        if (m >= p.M) return;
        const int n = n0 + c8;
        const int b = m / p.seq, sq = m - b * p.seq;
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = bf16(tile[r][c8 + e]);
        bf16* dst;
        if (n < wq) {
            const int head = n / d, dd = n - head * d;
            dst = reinterpret_cast<bf16*>(p.q) +
                  (((int64_t)b * p.heads_local + head) * p.seq + sq) * d + dd;
        } else {
            const int nk = n - wq, head = nk / d, dd = nk - head * d;
            dst = reinterpret_cast<bf16*>(p.k) +
                  (((int64_t)b * p.kv_heads_local + head) * p.seq + sq) * d + dd;
        }
        *reinterpret_cast<bf16x8*>(dst) = v;
    } else {               // value columns, transposed
        const int c = t & 63, rc = (t >> 6) * 8;   // column, first of the chunk's 8 rows
        const int nv = n0 + c - wq - wkv, head = nv / d, dd = nv - head * d;
        bf16* vt = reinterpret_cast<bf16*>(p.vt);
        const int m = m0 + rc;
        if (p.seq % 8 == 0) {
            if (m >= p.M) return;   // M is a multiple of seq, so the whole chunk is valid
            const int b = m / p.seq, sq = m - b * p.seq;
            bf16x8 v;
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = bf16(tile[rc + e][c]);
            *reinterpret_cast<bf16x8*>(
                vt + (((int64_t)b * p.kv_heads_local + head) * d + dd) * p.ld_vt + sq) = v;
        } else {
            for (int e = 0; e < 8 && m + e < p.M; ++e) {
                const int b = (m + e) / p.seq, sq = m + e - b * p.seq;
                vt[(((int64_t)b * p.kv_heads_local + head) * d + dd) * p.ld_vt + sq] =
                    bf16(tile[rc + e][c]);
            }
        }
    }
}

}  // namespace

hipError_t qkv_reduce_scatter(const GemmProblem& p, const float* parts, hipStream_t s)
{
    if (p.N % kRsCols != 0 || p.k_splits < 1) return hipErrorInvalidValue;
    const int64_t blocks = (int64_t)((p.M + kRsRows - 1) / kRsRows) * (p.N / kRsCols);
    hipLaunchKernelGGL(qkv_reduce_scatter_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, parts);
    return hipGetLastError();
}

template <int MB>
hipError_t launch_f32_skinny(const GemmProblem& p, Epi epi, hipStream_t s)
{
    const int row_groups = (p.M + 16 * MB - 1) / (16 * MB);
    dim3 grid((unsigned)((p.N + 15) / 16), (unsigned)row_groups), block(1024);
    switch (epi) {
        case Epi::BiasGelu:
            hipLaunchKernelGGL((gemm_f32_skinny_kernel<MB, Epi::BiasGelu>), grid, block, 0, s, p);
            break;
        case Epi::F32:
            hipLaunchKernelGGL((gemm_f32_skinny_kernel<MB, Epi::F32>), grid, block, 0, s, p);
            break;
        case Epi::Bias:
            hipLaunchKernelGGL((gemm_f32_skinny_kernel<MB, Epi::Bias>), grid, block, 0, s, p);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// Up to 64 rows: the skinny kernel (16 columns and up to all rows per workgroup, K split over
// its waves); beyond, 32 x 64 tiles. The fp32 worked example (32 x 1024 x 2048 and 32 x 2048 x 1024): 20 and 34 us
// per product on the tiles, against the skinny kernel's times in the benchmark's configs.
hipError_t gemm_f32(const GemmProblem& p, Epi epi, hipStream_t s)
{
    if (p.M <= 64) {
        // 16-row blocks per workgroup: all of them, unless fewer per workgroup let the grid
        // cover more of the 256 compute units (the 32-token worked example: 128 and 64
        // column blocks, two row blocks each)
        const int cols = (p.N + 15) / 16, rblocks = (p.M + 15) / 16;
        const int groups = std::max(1, std::min(rblocks, 256 / cols));
        const int mb = (rblocks + groups - 1) / groups;
        if (mb <= 1) return launch_f32_skinny<1>(p, epi, s);
        if (mb <= 2) return launch_f32_skinny<2>(p, epi, s);
        return launch_f32_skinny<4>(p, epi, s);
    }
    constexpr int BM = 32, BN = 64;
    const int tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
    dim3 grid(tiles), block(kThreads);
    switch (epi) {
        case Epi::BiasGelu:
            hipLaunchKernelGGL((gemm_f32_kernel<BM, BN, Epi::BiasGelu>), grid, block, 0, s, p);
            break;
        case Epi::F32:
            hipLaunchKernelGGL((gemm_f32_kernel<BM, BN, Epi::F32>), grid, block, 0, s, p);
            break;
        case Epi::Bias:
            hipLaunchKernelGGL((gemm_f32_kernel<BM, BN, Epi::Bias>), grid, block, 0, s, p);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace tps
