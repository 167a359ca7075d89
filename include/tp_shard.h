/*
 * tp_shard.h -- C ABI of libtpshard: one tensor-parallel rank's share of a Transformer block
 * (the column-parallel / row-parallel MLP pair and the head-partitioned attention block),
 * computed by hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * The split follows the pages' statement of tensor parallelism:
 *   - Column-parallel linear (llms.blog, "The Core Primitives", 1. Column-Parallel Linear
 *     Layer): W = [W_1 ... W_N] split on its output dimension, each rank computes X W_i from
 *     the replicated X, no communication; an element-wise activation applies to the local
 *     slice (same section, last paragraph).
 *   - Row-parallel linear (same page, 2. Row-Parallel Linear Layer): W split on its input
 *     dimension, each rank computes the partial X_i W_i; the true output is the sum of the
 *     N partials, which the all-reduce forms.
 *   - MLP block (ai360xpert.com, "How It Works"; llms.blog, "Partitioning the Multi-Layer
 *     Perceptron (MLP) Block"): Y = GeLU(X A) B; rank i holds A_i (columns) and B_i (rows)
 *     and produces the partial Z_i = GeLU(X A_i + a_i) B_i.
 *   - Attention block (llms.blog, "Partitioning Multi-Head and Grouped-Query Attention",
 *     steps 1-3): h_heads / N heads per rank; Q, K, V projections column-parallel on the
 *     rank's heads; softmax(Q K^T / sqrt(d_k)) V per head with no cross-head exchange;
 *     head outputs concatenated locally and multiplied by the rank's row slice of W_O.
 *
 * Conventions shared by every call
 *   - Every tensor pointer is a DEVICE pointer, row-major, allocated and owned by the
 *     caller. The library allocates no device memory and keeps no state between calls
 *     (apart from the thread-local error string and a per-device capability check).
 *   - Weights are stored the way a linear layer stores its weight: [out_features,
 *     in_features] row-major, i.e. the transpose of the pages' W in R^{H_in x H_out}.
 *     Rank r's shards are passed as the rank's own contiguous arrays.
 *   - Token rows are t = b * seq + s (each sequence is a contiguous block of rows).
 *   - hidden, ffn and n_heads are the FULL (unsharded) sizes; the shard widths ffn / N
 *     and hidden / N are derived. N (n_shards) and rank follow the pages' split; a size
 *     that does not divide evenly is an error, never an uneven shard.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL is the
 *     default stream) and return after the kernels are enqueued. Results are bitwise
 *     reproducible for a given shape, dtype and device (no atomics, fixed reduction order).
 *   - Errors: validation runs on the host before any HIP call and returns a tp_status;
 *     nothing aborts and no exception crosses the ABI. tp_last_error() describes the last
 *     non-OK status on the calling thread. Pointers must be 16-byte aligned; hidden,
 *     ffn / N and the head width must be multiples of 8 (16-byte rows); tokens and seq may
 *     be any value >= 1. A GEMM's reduced dimension (hidden, ffn / N; the tokens in the MLP
 *     backward) must be below 2^22 and the attention's sequence length at most 2^22
 *     (TP_ERR_SHAPE): a tile's operand rows, and a head's keys and values, are addressed with
 *     32-bit offsets below 2^31.
 *   - Precision: TP_BF16 inputs, weights and intermediates (Y_i, Q/K/V, head outputs) are
 *     bfloat16 rounded to nearest even, with fp32 accumulation; TP_F32 is fp32 throughout.
 *     Partials Z_i are always fp32.
 */
#ifndef TP_SHARD_H
#define TP_SHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TP_F32 = 0,   /* IEEE binary32 */
    TP_BF16 = 1   /* bfloat16 (1-8-7), round to nearest even */
} tp_dtype;

typedef enum {
    TP_OK = 0,
    TP_ERR_NULL = 1,           /* a required pointer is NULL (or a partial is missing)   */
    TP_ERR_SHAPE = 2,          /* a size is out of range                                  */
    TP_ERR_NOT_DIVISIBLE = 3,  /* ffn % N, n_heads % N or hidden % n_heads is not zero     */
    TP_ERR_RANK = 4,           /* rank outside [0, N)                                     */
    TP_ERR_DTYPE = 5,          /* dtype not supported by this call                        */
    TP_ERR_ALIGN = 6,          /* pointer not 16-byte aligned or row width not 8-multiple */
    TP_ERR_WORKSPACE = 7,      /* workspace NULL or smaller than *_workspace_bytes()       */
    TP_ERR_HIP = 8,            /* a HIP runtime call or kernel launch failed               */
    TP_ERR_DEVICE = 9,         /* the current device is not gfx950                         */
    TP_ERR_ALIAS = 10          /* an output shares memory with an input it may not alias  */
} tp_status;

typedef enum {
    TP_ACT_NONE = 0,   /* identity                                     */
    TP_ACT_GELU = 1    /* exact GeLU, x * Phi(x) = x/2 (1 + erf(x/sqrt 2)) */
} tp_activation;

/* ------------------------------------------------------------------------------------------
 * Column-parallel linear layer of rank r (llms.blog, "The Core Primitives", 1. Column-Parallel
 * Linear Layer): W = [W_1 ... W_N] split on its output dimension, the replicated X times the
 * rank's slice, no communication; an element-wise activation applies to the local slice.
 *   Y_i = act(X W_i + b_i)
 *
 *   X    [rows, in_features]          dt   replicated input
 *   W_i  [out_features/N, in_features] dt   W_i[j][k] = W[k][rank*out_features/N + j]
 *   b_i  [out_features/N]             dt   or NULL for no bias
 *   Y_i  [rows, out_features/N]       dt
 * dt: TP_F32 or TP_BF16. in_features and out_features/N must be multiples of 8.
 * ---------------------------------------------------------------------------------------- */
tp_status tp_column_parallel_fwd(const void* X, const void* W_i, const void* b_i, void* Y_i,
                                 int64_t rows, int64_t in_features, int64_t out_features,
                                 int n_shards, int rank, tp_activation act, tp_dtype dt,
                                 void* stream);

/* ------------------------------------------------------------------------------------------
 * Row-parallel linear layer of rank r (same page, 2. Row-Parallel Linear Layer): W split on
 * its input dimension, the rank's channel slice X_i of the input times W_i gives a partial
 * that must be summed over the N ranks (tp_sum_partials).
 *   Z_i = X_i W_i
 *
 *   X_i  [rows, in_features/N]        dt   the rank's channel slice (a column-parallel output)
 *   W_i  [out_features, in_features/N] dt   W_i[o][j] = W[rank*in_features/N + j][o]
 *   Z_i  [rows, out_features]         fp32 partial
 * dt: TP_F32 or TP_BF16. in_features/N and out_features must be multiples of 8.
 * ---------------------------------------------------------------------------------------- */
tp_status tp_row_parallel_fwd(const void* X_i, const void* W_i, float* Z_i, int64_t rows,
                              int64_t in_features, int64_t out_features, int n_shards, int rank,
                              tp_dtype dt, void* stream);

/* ------------------------------------------------------------------------------------------
 * Row-parallel linear layer with the all-reduce's sum fused into it (same page, 2. Row-
 * Parallel Linear Layer: the output is the sum of the N partials X_q W_q). Rank r computes
 * its product X_i W_i and, in the same kernel, adds the other ranks' partials to it:
 *   Z = Z_0 + Z_1 + ... + Z_{N-1},   Z_r = X_i W_i (this rank's product, never stored)
 * in fp32, in the fixed order 0, 1, ..., N-1 with Z_r in its place, stored as out_dt: the same
 * bits as tp_row_parallel_fwd into Z_r followed by tp_sum_partials. The rank's own partial
 * neither goes to memory nor comes back (on one device the other partials are resident
 * inputs; across devices they are what the exchange delivers).
 *
 *   X_i      [rows, in_features/N]          bf16
 *   W_i      [out_features, in_features/N]  bf16
 *   Z_parts  HOST array of n_shards DEVICE pointers, each [rows, out_features] fp32 (16-byte
 *            aligned); entry rank is not read (may be NULL), a NULL elsewhere is a missing
 *            rank (TP_ERR_NULL)
 *   Z        [rows, out_features] out_dt (fp32, or bf16 rounded to nearest even); must not
 *            overlap any input (TP_ERR_ALIAS)
 * dt: TP_BF16 only; n_shards at most 8 (TP_ERR_SHAPE). Other rules as for
 * tp_row_parallel_fwd.
 * ---------------------------------------------------------------------------------------- */
tp_status tp_row_parallel_sum_fwd(const void* X_i, const void* W_i, const float* const* Z_parts,
                                  void* Z, tp_dtype out_dt, int64_t rows, int64_t in_features,
                                  int64_t out_features, int n_shards, int rank, tp_dtype dt,
                                  void* stream);

/* ------------------------------------------------------------------------------------------
 * MLP shard: Z_i = GeLU(X A_i + a_i) B_i          (ai360xpert.com "How It Works", steps 1-2;
 *                                                  llms.blog MLP block, steps 1-3)
 * GeLU is the exact form x * Phi(x) = x/2 (1 + erf(x / sqrt 2)).
 *
 *   X    [tokens, hidden]       dt   replicated input
 *   A_i  [ffn/N, hidden]        dt   rank's column shard of A, stored transposed:
 *                                    A_i[j][k] = A[k][rank*ffn/N + j]
 *   a_i  [ffn/N]                dt   rank's slice of the column bias a, or NULL for none
 *   B_i  [hidden, ffn/N]        dt   rank's row shard of B, stored transposed:
 *                                    B_i[o][j] = B[rank*ffn/N + j][o]
 *   Z_i  [tokens, hidden]       fp32 rank's partial (to be summed over ranks)
 *   workspace: Y_i = GeLU(X A_i + a_i) [tokens, ffn/N] in dt at byte offset 0.
 * A row-parallel output bias, if a model has one, is added once after the sum, not here.
 * dt: TP_F32 or TP_BF16. Equivalent to tp_column_parallel_fwd(TP_ACT_GELU) into the
 * workspace followed by tp_row_parallel_fwd (the same two kernels).
 * ---------------------------------------------------------------------------------------- */
size_t tp_mlp_workspace_bytes(int64_t tokens, int64_t hidden, int64_t ffn, int n_shards,
                              tp_dtype dt);

tp_status tp_mlp_shard_fwd(const void* X, const void* A_i, const void* a_i, const void* B_i,
                           float* Z_i, int64_t tokens, int64_t hidden, int64_t ffn,
                           int n_shards, int rank, tp_dtype dt,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * Allocation-free MLP shard, for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): tp_mlp_shard_fwd with Y_i = GeLU(X A_i + a_i) kept in a device scratch array
 * of the library instead of a workspace. Same arguments (without the workspace), same two
 * kernels, same bits, same errors; additionally TP_ERR_WORKSPACE when Y_i
 * (tokens * ffn/N * element size, rounded up to 256 bytes) exceeds TP_NOALLOC_SCRATCH_BYTES.
 * The call allocates nothing: the scratch is a static device array, one per device that runs
 * the library, held until the process ends (its address is looked up once per device).
 * Every call on a device shares that device's scratch, so calls that may overlap in time on
 * one device (different streams, different threads) race: serialize them.
 * ---------------------------------------------------------------------------------------- */
#define TP_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

tp_status tp_mlp_shard_fwd_noalloc(const void* X, const void* A_i, const void* a_i,
                                   const void* B_i, float* Z_i, int64_t tokens, int64_t hidden,
                                   int64_t ffn, int n_shards, int rank, tp_dtype dt, void* stream);

/* ------------------------------------------------------------------------------------------
 * MLP shard forward that also keeps the pre-activation for the backward pass:
 *   P_i = X A_r + a_r,   Z_i = GeLU(P_i) B_r     (llms.blog, "Partitioning the MLP Block",
 *                                                 steps 2-3, as tp_mlp_shard_fwd)
 * The same two launches and the same bits of Z_i as tp_mlp_shard_fwd; the column GEMM's
 * epilogue stores P_i (rounded once to bf16, before the GeLU) beside Y_i. P_i is what
 * tp_mlp_shard_bwd would otherwise recompute: tp_mlp_shard_bwd_saved takes it instead.
 *
 *   X, A_i, a_i, B_i, Z_i, workspace   as for tp_mlp_shard_fwd
 *   P_i     [tokens, ffn/N]   bf16  output, the caller's buffer; must not overlap the
 *                                   workspace, Z_i or an input (TP_ERR_ALIAS)
 * dt: TP_BF16 only (TP_ERR_DTYPE otherwise). Errors as tp_mlp_shard_fwd.
 * ---------------------------------------------------------------------------------------- */
tp_status tp_mlp_shard_fwd_save(const void* X, const void* A_i, const void* a_i, const void* B_i,
                                float* Z_i, void* P_i, int64_t tokens, int64_t hidden, int64_t ffn,
                                int n_shards, int rank, tp_dtype dt, void* workspace,
                                size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * Backward pass of the MLP shard (llms.blog, "Partitioning the MLP Block": one all-reduce in
 * the backward pass, over the input gradients of the column-parallel layer). For the
 * forward Z_i = GeLU(P) B_r, P = X A_r + a_r, and the upstream gradient dZ of the block
 * output (every rank receives the same dZ, since Z is the sum of the partials):
 *   dY = dZ B_r^T,   dP = dY * GeLU'(P),   GeLU'(x) = Phi(x) + x phi(x)
 *   dA_r = X^T dP,   da_r = sum over tokens of dP,   dB_r = GeLU(P)^T dZ
 *   dX_i = dP A_r^T  (rank i's input-gradient partial; the all-reduce sums them)
 * P is recomputed from X, A_i, a_i (tp_mlp_shard_bwd_saved takes the forward's P instead).
 *
 *   X, A_i, a_i, B_i   as for tp_mlp_shard_fwd (bf16; a_i may be NULL)
 *   dZ     [tokens, hidden]   bf16  upstream gradient
 *   dX_i   [tokens, hidden]   fp32  input-gradient partial
 *   dA_i   [ffn/N, hidden]    fp32  gradient of A_i in A_i's stored layout (dA_r transposed)
 *   da_i   [ffn/N]            fp32  gradient of a_i, or NULL to skip it
 *   dB_i   [hidden, ffn/N]    fp32  gradient of B_i in B_i's stored layout (dB_r transposed)
 * The products run on the bf16 MFMA GEMM (fp32 accumulation); P, dP and GeLU(P) are kept
 * in bf16 in the workspace, and the operands whose reduced dimension is not contiguous are
 * transposed into the workspace first (tokens padded to a multiple of 8 with zeros there).
 * dt: TP_BF16 only. hidden and ffn/N multiples of 8; tokens any value >= 1.
 * ---------------------------------------------------------------------------------------- */
size_t tp_mlp_bwd_workspace_bytes(int64_t tokens, int64_t hidden, int64_t ffn, int n_shards,
                                  tp_dtype dt);

tp_status tp_mlp_shard_bwd(const void* X, const void* A_i, const void* a_i, const void* B_i,
                           const void* dZ, float* dX_i, float* dA_i, float* da_i, float* dB_i,
                           int64_t tokens, int64_t hidden, int64_t ffn, int n_shards, int rank,
                           tp_dtype dt, void* workspace, size_t workspace_bytes, void* stream);

/* The same backward with P_i = X A_r + a_r taken from the forward (tp_mlp_shard_fwd_save)
 * instead of recomputed: one GEMM fewer. Outputs, workspace (tp_mlp_bwd_workspace_bytes) and
 * errors as tp_mlp_shard_bwd; with the P_i that tp_mlp_shard_fwd_save wrote for the same X,
 * A_i, a_i, the same bits as tp_mlp_shard_bwd. The bias a_i is not needed (P_i includes it).
 *   P_i     [tokens, ffn/N]   bf16  input; must not overlap the workspace or a gradient
 *                                   output (TP_ERR_ALIAS)
 */
tp_status tp_mlp_shard_bwd_saved(const void* X, const void* A_i, const void* B_i, const void* P_i,
                                 const void* dZ, float* dX_i, float* dA_i, float* da_i,
                                 float* dB_i, int64_t tokens, int64_t hidden, int64_t ffn,
                                 int n_shards, int rank, tp_dtype dt, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * Gated (SwiGLU) MLP shard:
 *   Z_i = (SiLU(X W_gate,i) * (X W_up,i)) W_down,i     (llms.blog, "Partitioning the MLP
 *                                                      Block", steps 2-3: gate and up
 *                                                      projections split by columns, the
 *                                                      element-wise product local, the
 *                                                      down projection split by rows)
 * SiLU(x) = x sigmoid(x) = x / (1 + exp(-x)); the gated product * is element-wise.
 *
 *   X        [tokens, hidden]   bf16  replicated input
 *   Wgate_i  [ffn/N, hidden]    bf16  rank's column shard of W_gate, stored transposed:
 *                                     Wgate_i[j][k] = W_gate[k][rank*ffn/N + j]
 *   Wup_i    [ffn/N, hidden]    bf16  the same for W_up
 *   Wdown_i  [hidden, ffn/N]    bf16  rank's row shard of W_down, stored transposed:
 *                                     Wdown_i[o][j] = W_down[rank*ffn/N + j][o]
 *   Z_i      [tokens, hidden]   fp32  rank's partial (to be summed over ranks)
 *   workspace: A_i = SiLU(X W_gate,i) * (X W_up,i) [tokens, ffn/N] bf16 at byte offset 0.
 * dt: TP_BF16 only (TP_ERR_DTYPE otherwise). No biases (the gated layers of the models the
 * page names have none). hidden and ffn/N must be multiples of 8.
 * ---------------------------------------------------------------------------------------- */
size_t tp_swiglu_workspace_bytes(int64_t tokens, int64_t hidden, int64_t ffn, int n_shards,
                                 tp_dtype dt);

tp_status tp_swiglu_shard_fwd(const void* X, const void* Wgate_i, const void* Wup_i,
                              const void* Wdown_i, float* Z_i, int64_t tokens, int64_t hidden,
                              int64_t ffn, int n_shards, int rank, tp_dtype dt,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * Attention shard: Z_i = concat_j(Head_j) W_O,i over the rank's heads j, with
 *   Head_j = softmax(Q_j K_j^T / sqrt(d) + M) V_j      (llms.blog attention, steps 1-3)
 * d = hidden / n_heads; Hl = n_heads / N local heads, rank r owning heads r*Hl ... r*Hl+Hl-1.
 * M is the causal mask (key k visible to query s iff k <= s within a sequence) when
 * causal != 0, else zero.
 *
 *   X       [batch*seq, hidden]   bf16
 *   Wqkv_i  [3*Hl*d, hidden]      bf16  rows 0..Hl*d-1 = W_Q[:, C_r]^T, then W_K[:, C_r]^T,
 *                                       then W_V[:, C_r]^T, C_r = columns r*Hl*d ... of the
 *                                       rank's heads (head-major, d columns per head)
 *   bqkv_i  [3*Hl*d]              bf16  matching bias slices, or NULL for none
 *   Wo_i    [hidden, Hl*d]        bf16  rank's row shard of W_O, stored transposed:
 *                                       Wo_i[o][j] = W_O[r*Hl*d + j][o]
 *   Z_i     [batch*seq, hidden]   fp32  rank's partial
 * Workspace layout (byte offsets from tp_attn_workspace_layout, each 256-byte aligned):
 *   Q   [batch, Hl, seq, d]  bf16     projected queries of the local heads, multiplied by
 *                                     log2(e)/sqrt(d) (the softmax's scale, folded in before
 *                                     the one rounding to bf16)
 *   K   [batch, Hl, seq, d]  bf16     projected keys
 *   Vt  [batch, Hl, d, seq]  bf16     projected values, transposed per head
 *   O   [batch*seq, Hl*d]    bf16     head outputs, concatenated locally
 *   then, when the shard has under 512 query tiles of 128 tokens (batch*Hl*ceil(seq/128)),
 *   the fp32 partial results of the two key-range halves of every query tile
 *   ([tiles][2][128][d] outputs, then [tiles][2][128][2] maxima and denominators), used for
 *   causal attention over sequences of 2048 tokens or more.
 *   When the projection's 256 x 256 output tiles (batch*seq by the local Q/K/V width) would
 *   occupy at most 128 compute units and hidden >= 4096, it runs split along hidden into S
 *   parts (S = min(4, 256 / tiles)); their fp32 partials [S][batch*seq][Q/K/V width] start
 *   at O's offset (the size covers whichever of the two regions reaches further).
 * dt: TP_BF16 only. d must be 64 or 128.
 * ---------------------------------------------------------------------------------------- */
size_t tp_attn_workspace_bytes(int64_t batch, int64_t seq, int64_t hidden, int n_heads,
                               int n_shards, tp_dtype dt);

tp_status tp_attn_workspace_layout(int64_t batch, int64_t seq, int64_t hidden, int n_heads,
                                   int n_shards, tp_dtype dt, size_t* q_off, size_t* k_off,
                                   size_t* vt_off, size_t* o_off);

tp_status tp_attn_shard_fwd(const void* X, const void* Wqkv_i, const void* bqkv_i,
                            const void* Wo_i, float* Z_i, int64_t batch, int64_t seq,
                            int64_t hidden, int n_heads, int causal, int n_shards, int rank,
                            tp_dtype dt, void* workspace, size_t workspace_bytes,
                            void* stream);

/* ------------------------------------------------------------------------------------------
 * Grouped-query attention shard (llms.blog, "Grouped-Query Attention (GQA) Constraints"):
 * the attention shard above with n_kv_heads key/value heads, each read by
 * n_heads / n_kv_heads query heads (query head j reads key/value head j / (n_heads /
 * n_kv_heads)); n_kv_heads = n_heads is the multi-head case (tp_attn_shard_fwd is exactly
 * that call), n_kv_heads = 1 multi-query attention.
 * The page's constraint: n_kv_heads must be divisible by N, and then rank r holds key/value
 * heads r*KVl ... r*KVl + KVl - 1 (KVl = n_kv_heads / N); when N exceeds n_kv_heads, N must
 * be a multiple of it and every key/value head is duplicated on N / n_kv_heads ranks: rank r
 * holds the single head its query heads r*Hl ... read (KVl = 1). Anything else, or n_heads
 * not a multiple of n_kv_heads, is TP_ERR_NOT_DIVISIBLE.
 *
 *   Wqkv_i  [(Hl + 2*KVl)*d, hidden] bf16  rows 0..Hl*d-1 = W_Q[:, C_r]^T (the rank's query
 *                                          heads), then W_K[:, K_r]^T and W_V[:, K_r]^T (the
 *                                          rank's key/value heads, head-major)
 *   bqkv_i  [(Hl + 2*KVl)*d]         bf16  matching bias slices, or NULL
 *   Wo_i    [hidden, Hl*d]           bf16  as for tp_attn_shard_fwd
 * Workspace: Q [batch, Hl, seq, d], K [batch, KVl, seq, d], Vt [batch, KVl, d, round8(seq)],
 * O [batch*seq, Hl*d], at the offsets tp_gqa_attn_workspace_layout returns. Other arguments,
 * dtype and head-width rules as for tp_attn_shard_fwd.
 * ---------------------------------------------------------------------------------------- */
size_t tp_gqa_attn_workspace_bytes(int64_t batch, int64_t seq, int64_t hidden, int n_heads,
                                   int n_kv_heads, int n_shards, tp_dtype dt);

tp_status tp_gqa_attn_workspace_layout(int64_t batch, int64_t seq, int64_t hidden, int n_heads,
                                       int n_kv_heads, int n_shards, tp_dtype dt, size_t* q_off,
                                       size_t* k_off, size_t* vt_off, size_t* o_off);

tp_status tp_gqa_attn_shard_fwd(const void* X, const void* Wqkv_i, const void* bqkv_i,
                                const void* Wo_i, float* Z_i, int64_t batch, int64_t seq,
                                int64_t hidden, int n_heads, int n_kv_heads, int causal,
                                int n_shards, int rank, tp_dtype dt, void* workspace,
                                size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * The attention shard's first two steps as separate calls (llms.blog, "Partitioning
 * Multi-Head and Grouped-Query Attention", steps 1 and 2); the third, Z_i = O_i W_O,i, is
 * tp_row_parallel_fwd on the workspace's O. tp_gqa_attn_shard_fwd is exactly these three
 * launches in order, so running them one by one gives its bits (and lets a caller time each).
 *
 * tp_qkv_projection_fwd: step 1, the column-parallel Q, K, V projections of the rank's heads
 *   into the workspace's Q, K and Vt regions (layout and scaling as for tp_gqa_attn_shard_fwd;
 *   n_kv_heads = n_heads for multi-head attention).
 * tp_head_attention_fwd: step 2, softmax(Q K^T / sqrt(d) + M) V of every local head from the
 *   workspace's Q, K and Vt into its O (heads concatenated locally), with no cross-head
 *   exchange. The workspace must hold step 1's results for the same sizes.
 * Arguments, workspace size (tp_gqa_attn_workspace_bytes) and errors as for
 * tp_gqa_attn_shard_fwd.
 * ---------------------------------------------------------------------------------------- */
tp_status tp_qkv_projection_fwd(const void* X, const void* Wqkv_i, const void* bqkv_i,
                                int64_t batch, int64_t seq, int64_t hidden, int n_heads,
                                int n_kv_heads, int n_shards, int rank, tp_dtype dt,
                                void* workspace, size_t workspace_bytes, void* stream);

tp_status tp_head_attention_fwd(int64_t batch, int64_t seq, int64_t hidden, int n_heads,
                                int n_kv_heads, int causal, int n_shards, int rank, tp_dtype dt,
                                void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------------------------
 * Partial sum, the single-device stand-in for the tensor-parallel all-reduce:
 *   Z = Z_0 + Z_1 + ... + Z_{n_parts-1}       (llms.blog, Row-Parallel Linear Layer: the
 *                                              output and communication bullets)
 * summed in fp32 in the fixed order 0, 1, ..., n_parts-1, then stored as out_dt (fp32, or
 * bf16 rounded to nearest even when the next block consumes bf16).
 *
 *   Z_parts  HOST array of n_parts DEVICE pointers, each [numel] fp32, 16-byte aligned;
 *            a NULL entry is a missing rank (TP_ERR_NULL).
 *   n_parts  1 ... 64
 *   Z        [numel] out_dt. An fp32 Z may be one of the partials itself (the same
 *            pointer: each element is read from every partial before it is written); any
 *            other overlap with a partial, and every overlap of a bf16 Z, is TP_ERR_ALIAS.
 * ---------------------------------------------------------------------------------------- */
tp_status tp_sum_partials(const float* const* Z_parts, int n_parts, int64_t numel,
                          void* Z, tp_dtype out_dt, void* stream);

/* ------------------------------------------------------------------------------------------
 * Sequence-parallel block boundary (llms.blog, "Sequence Parallelism"): the all-reduce after
 * a row-parallel layer becomes a reduce-scatter that sums the N partials but leaves rank r
 * only its slice of every sequence, positions r*seq/N ... (r+1)*seq/N - 1; the residual
 * addition and LayerNorm, which act on each token separately, run on that slice; an
 * all-gather restores the full sequence before the next column-parallel layer (a
 * reduce-scatter followed by an all-gather is the all-reduce, same page).
 *
 * Slice layout: slice row i = b*(seq/N) + s' holds token t = b*seq + r*(seq/N) + s'
 * (token rows of the full tensors are t = b*seq + s). N = n_parts must divide seq.
 *
 * tp_reduce_scatter_partials:  H_r[i] = sum_q Z_parts[q][t(i)]
 *   Z_parts  HOST array of n_parts DEVICE pointers, each [batch*seq, hidden] fp32
 *   H_r      [batch*seq/N, hidden] out_dt (fp32, or bf16 rounded to nearest even)
 * The sum runs in fp32 in the order q = 0, 1, ..., N-1 (the same bits as tp_sum_partials on
 * those rows).
 *
 * tp_sp_residual_layernorm_fwd:  H_r[i] = sum_q Z_parts[q][t(i)] + residual_r[i],
 *                                Y_r[i] = (H_r[i] - mean) / sqrt(var + eps) * gamma + beta
 * with mean and the biased variance var taken over the hidden values of the row (fp32).
 *   residual_r [batch*seq/N, hidden] dt, or NULL for none
 *   gamma, beta [hidden] fp32;  eps >= 0
 *   H_r, Y_r   [batch*seq/N, hidden] dt (H_r is the new residual stream, Y_r the normalised
 *              input of the next block)
 * dt: TP_F32 or TP_BF16. hidden must be a multiple of 8 and at most 16384 (the row is held
 * in LDS).
 *
 * tp_all_gather_rows:  X[t] = slices[r(t)][i(t)]
 *   slices  HOST array of n_parts DEVICE pointers, each [batch*seq/N, hidden] dt
 *   X       [batch*seq, hidden] dt
 * No output may share memory with an input or with the other output (TP_ERR_ALIAS; H_r
 * may be residual_r itself). Errors as for the other calls; seq % N != 0 is
 * TP_ERR_NOT_DIVISIBLE (the pages only use exact slices).
 * ---------------------------------------------------------------------------------------- */
tp_status tp_reduce_scatter_partials(const float* const* Z_parts, int n_parts, int64_t batch,
                                     int64_t seq, int64_t hidden, int rank, void* H_r,
                                     tp_dtype out_dt, void* stream);

tp_status tp_sp_residual_layernorm_fwd(const float* const* Z_parts, int n_parts,
                                       const void* residual_r, const float* gamma,
                                       const float* beta, float eps, void* H_r, void* Y_r,
                                       int64_t batch, int64_t seq, int64_t hidden, int rank,
                                       tp_dtype dt, void* stream);

tp_status tp_all_gather_rows(const void* const* slices, int n_parts, int64_t batch,
                             int64_t seq, int64_t hidden, void* X, tp_dtype dt, void* stream);

/* ------------------------------------------------------------------------------------------
 * Which bf16 GEMM tile the library launches for C[M, N] = A[M, K] B[N, K]^T: block tile
 * rows x columns and waves per workgroup (honours the gemm_tile test override). The
 * answer holds for every epilogue except the per-head Q/K/V scatter, which always runs eight
 * waves per workgroup, and the gated (SwiGLU) product, which picks its own tile. A query
 * for profiling and tuning; it launches nothing. Returns TP_ERR_NULL / TP_ERR_SHAPE on bad
 * arguments.
 * ---------------------------------------------------------------------------------------- */
tp_status tp_gemm_tile_info(int64_t M, int64_t N, int64_t K, int* tile_m, int* tile_n,
                            int* waves);

/* ------------------------------------------------------------------------------------------
 * Which launch tp_row_parallel_sum_fwd makes for a row-parallel product of rows x k_local by
 * out_features x k_local summed over n_parts partials into out_dt: block tile, waves per
 * workgroup, and form, 0 = each tile's sum in its own epilogue, 1 = deferred (two tiles per
 * workgroup, the first one's sum streamed during the second one's K loop; fp32 output only),
 * 2 = ring (each workgroup's tiles in turn, every tile's product kept in LDS and its sum
 * streamed during the next tile's K loop). Honours the test overrides; launches nothing.
 * Returns TP_ERR_NULL / TP_ERR_SHAPE / TP_ERR_DTYPE on bad arguments.
 * ---------------------------------------------------------------------------------------- */
tp_status tp_row_parallel_sum_tile_info(int64_t rows, int64_t out_features, int64_t k_local,
                                         int n_parts, tp_dtype out_dt, int* tile_m, int* tile_n,
                                         int* waves, int* form);

/* ------------------------------------------------------------------------------------------
 * Test and tuning hook, for callers that need every launch variant exercised (the library's
 * tests): forces launch choices that are otherwise made per shape. Not part of any passage of
 * the method; results stay within the documented precision whatever is forced.
 *   spec  NULL or "" restores the library's own choices; otherwise a comma-separated list of
 *         key=value items, each replacing one choice (the list replaces every earlier one):
 *           gemm_tile=<bm>x<bn>[w4]   bf16 GEMM tile 256x256, 256x192, 256x128 or 128x128,
 *                                     "w4": four waves per workgroup instead of eight
 *           qkv_split=1..8            K-split count of the Q/K/V projection
 *           attn_sets=1|2             attention wave sets per workgroup
 *           attn_split=1|2            key-range split of the attention off (1) or forced (2)
 *           attn_pair=1|2             paired causal layout (one workgroup per two 64-query
 *                                     tiles of equal total causal work) off (1) or on (2, the
 *                                     default wherever the split and one-set are not forced)
 *           sum_grid=<n>              partial-sum workgroups (0: one lane per vector)
 *           sum_unroll=1|2|4          partial-sum vectors per lane
 *           sum_defer=0|1             fused partial sum: 0 keeps every tile's sum in its own
 *                                     epilogue (1, the default, lets the launcher defer it)
 *           sum_ring=1|2              fused partial sum in ring form (128x128 tiles, each
 *                                     tile's sum streamed during the next tile's K loop) off
 *                                     (1) or wherever its shape conditions hold (2)
 * The setting is process-wide and applies to launches (and workspace sizes) from then on;
 * set it while no other thread is calling the library. TP_ERR_SHAPE (nothing changed) on an
 * unknown key or a bad value. The library reads no environment variable.
 * ---------------------------------------------------------------------------------------- */
tp_status tp_set_test_overrides(const char* spec);

/* Description of the last non-OK status returned on the calling thread ("" if none).
   The string is owned by the library and valid until the next call on that thread. */
const char* tp_last_error(void);

/* ABI version of this header (incremented on any signature or layout change). */
int tp_abi_version(void);

#define TP_SHARD_ABI_VERSION 12

#ifdef __cplusplus
}
#endif

#endif /* TP_SHARD_H */
