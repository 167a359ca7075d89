// kernels.hpp -- internal launch interface between the C ABI (tp_shard_abi.hip) and the
// gfx950 kernels. Shapes reaching these functions have been validated by the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tps {

// Launch choices a test may force (tp_set_test_overrides); zero everywhere means "the
// library's own choice". The library reads no environment variable.
struct Tuning {
    int gemm_bm, gemm_bn, gemm_w4;   // GEMM tile (0: chosen per shape) and 4-wave layout
    int qkv_split;                   // K-split count of the Q/K/V projection (0: chosen)
    int attn_sets;                   // attention waves sets per workgroup, 1 or 2 (0: chosen)
    int attn_split;                  // key-range split: 1 off, 2 forced (0: chosen)
    int attn_pair;                   // paired causal layout: 1 off, 2 on (0: chosen)
    int sum_grid;                    // partial-sum workgroups (0: one lane per vector)
    int sum_unroll;                  // partial-sum vectors per lane, 1, 2 or 4 (0: 4)
    int sum_nodefer;                 // 1: the fused-sum GEMM never defers a tile's sum
    int sum_ring;                    // fused-sum GEMM in ring form: 1 off, 2 wherever feasible
};
// A copy of the current overrides (defined with the C ABI).
Tuning tuning();

// Output stage of the tensor-core GEMM C[m, n] = sum_k A[m, k] * B[n, k].
enum class Epi : int {
    BiasGelu = 0,   // C = GeLU(acc + bias[n])  stored in the GEMM's element type (Y_i)
    F32 = 1,        // C = acc                   stored as fp32 (row-parallel partial Z_i)
    Qkv = 2,        // acc + bias[n] scattered to Q / K / V^T per head, bf16
    Bias = 3,       // C = acc + bias[n]         stored in the GEMM's element type
    SwiGlu = 4,     // C = SiLU(X B^T) * (X B2^T), N output features, bf16 (gated MLP)
    GeluGrad = 5,   // C = acc * GeLU'(aux[m, n]), bf16 (backward through the activation)
    SumF32 = 6,     // C = sum_q P_q, P_rank = acc, P_q = part[q] otherwise: fp32 (the partial sum
    SumBf16 = 7,    //     of the row-parallel layer fused into its epilogue), or bf16
};

// Partials a Sum epilogue adds: at most this many shards.
constexpr int kMaxSumParts = 8;

struct GemmProblem {
    const void* A;        // [M, K] row-major, leading dimension lda (elements)
    const void* B;        // [N, K] row-major (weight in [out, in] layout), ldb
    const void* B2;       // SwiGlu: the up projection [N, K] (B is the gate), ldb
    const void* bias;     // [N] or nullptr
    const void* aux;      // GeluGrad: the pre-activation P [M, N] bf16, leading dim ldaux
    int64_t ldaux;
    void* C;              // [M, N] row-major, ldc (BiasGelu / F32)
    void* pre;            // BiasGelu, bf16 only, optional: the pre-activation acc + bias[n] is
                          // also stored here, bf16 [M, N] with leading dimension ldc (the
                          // MLP backward's P, kept from the forward)
    int64_t lda, ldb, ldc;
    int M, N, K;
    // Qkv scatter, row m = b * seq + s: columns [0, Hl d) are the local query heads, then
    // KVl d key columns and KVl d value columns (head-major, d per head; KVl = Hl for
    // multi-head attention, fewer for grouped-query attention).
    void* q;              // [batch, Hl, seq, d]
    void* k;              // [batch, KVl, seq, d]
    void* vt;             // [batch, KVl, d, ld_vt]
    int seq, heads_local, head_dim;
    int kv_heads_local;   // KVl
    int64_t ld_vt;
    float q_scale;        // factor on the query columns before rounding (the softmax's scale)
    // F32 only: with k_splits > 1 the K range is cut into k_splits slab-aligned parts and the
    // grid into as many groups of blocks; group s writes the partial product over its part to
    // C + s * split_stride (elements). Zero or one: no split.
    int k_splits;
    int64_t split_stride;
    // SumF32 / SumBf16: n_parts partials [M, N] fp32 with leading dimension ldc; part[part_rank]
    // is this product (never read), the others are added in the fixed order 0 .. n_parts-1.
    const float* part[kMaxSumParts];
    int n_parts, part_rank;
    // Set by the launcher. 1 (SumF32): each workgroup takes two tiles and streams the first
    // one's sum during the second one's K loop (C holds the first tile's own partial
    // meanwhile). 2 (ring, 128 x 128 tiles): each workgroup takes ring_tiles tiles, keeps
    // each one's product in LDS and streams its sum during the next tile's K loop.
    int defer;
    int ring_tiles;
};

// Tile shape chosen for a problem (exposed for the benchmark's bookkeeping).
struct GemmTile { int bm, bn; };

GemmTile gemm_bf16_pick_tile(int M, int N, int K);
// Tile and wave count gemm_bf16 launches for this shape (after the environment override).
GemmTile gemm_bf16_launch_tile(int M, int N, int K, int* waves);
// Tile, waves and form (0 in-epilogue, 1 deferred, 2 ring) of the fused-sum launch for an
// M x N x K row-parallel product over n_parts partials.
GemmTile gemm_bf16_sum_launch_tile(int M, int N, int K, int n_parts, bool bf16_out, int* waves,
                                   int* form);
hipError_t gemm_bf16(const GemmProblem& p, Epi epi, hipStream_t stream);
// K-split count for the Q/K/V projection of an M x N x K shape (1: no split): > 1 when 256 x
// 256 tiles would occupy at most half of the compute units.
int qkv_k_splits(int M, int N, int K);
// The split Q/K/V projection's second half: the sum of the k_splits fp32 partials at
// parts + s * split_stride ([M, N], leading dimension N), plus the bias, the query columns
// times q_scale, scattered per head like the Qkv epilogue (p supplies the layout).
hipError_t qkv_reduce_scatter(const GemmProblem& p, const float* parts, hipStream_t stream);
hipError_t gemm_f32(const GemmProblem& p, Epi epi, hipStream_t stream);

struct AttnProblem {
    const void* q;        // [batch, Hl, seq, d] bf16, Q times log2(e) / sqrt(d)
    const void* k;        // [batch, KVl, seq, d] bf16
    const void* vt;       // [batch, KVl, d, ld_vt] bf16
    void* o;              // [batch * seq, Hl * d] bf16
    int batch, heads_local, seq, head_dim;
    int kv_heads_local;   // KVl; local query head j reads key/value head j / (Hl / KVl)
    int64_t ld_vt;
    int causal;
    // Key-range split: with kv_split = 2 each query tile's key tiles are halved between two
    // workgroups, which write unnormalised partials (part_o [items][128][d] fp32 and the
    // running max and denominator part_ml [items][128][2]) merged by a second kernel.
    int kv_split;         // 1 or 2
    float* part_o;
    float* part_ml;
};
// Bytes of the key-range-split partials for a problem (0 when no split is used).
size_t attention_partial_bytes(int batch, int heads_local, int seq, int head_dim, bool causal,
                               int* kv_split);

hipError_t attention_fwd(const AttnProblem& p, hipStream_t stream);

// Sequence-parallel block boundary of rank `rank`: rows of its s/N slice of every sequence
// (slice row i = b * seq/N + s' is token b * seq + rank * seq/N + s').
//   hout[i] = sum_q parts[q][token(i)] (+ resid[i]);  yout[i] = LayerNorm(hout[i]) if gamma
struct SpProblem {
    const float* const* parts;   // n_parts device pointers, each [batch * seq, hidden] fp32
    int n_parts;                 // N (the slice count)
    const void* resid;           // [batch * seq/N, hidden] or nullptr
    const float* gamma;          // [hidden] fp32, nullptr: no LayerNorm (plain reduce-scatter)
    const float* beta;           // [hidden] fp32
    float eps;
    void* hout;                  // [batch * seq/N, hidden]
    void* yout;                  // [batch * seq/N, hidden] (with gamma)
    int batch, seq, rank, hidden;
    bool bf16;                   // resid, hout, yout element type: bf16 or fp32
};
hipError_t sp_boundary(const SpProblem& p, hipStream_t stream);
// Full-sequence rows from the N slices: out[b * seq + r * seq/N + s'] = slices[r][b * seq/N + s'].
hipError_t all_gather_rows(const void* const* slices, int n, int batch, int seq, int64_t row_bytes,
                           void* out, hipStream_t stream);

// out[c][r] = f(in[r][c]) for a bf16 [rows, cols] array (f = GeLU when gelu); out has leading
// dimension ld_out >= rows (a multiple of 8) and its columns [rows, ld_out) are zeroed.
hipError_t transpose_bf16(const void* in, int rows, int cols, int64_t ld_in, void* out,
                          int64_t ld_out, bool gelu, hipStream_t stream);
// out[r] = sum_c in[r][c] (fp32) of a bf16 [rows, cols] array with leading dimension ld.
hipError_t row_sum_bf16(const void* in, int rows, int cols, int64_t ld, float* out,
                        hipStream_t stream);

hipError_t sum_partials(const float* const* parts, int n_parts, int64_t numel, void* out,
                        bool out_bf16, hipStream_t stream);

}  // namespace tps
