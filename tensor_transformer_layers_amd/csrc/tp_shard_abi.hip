// tp_shard_abi.hip -- the extern "C" boundary of libtpshard (declared in include/tp_shard.h).
//
// Every entry point validates its arguments on the host before any HIP call, returns a
// tp_status and records a message for tp_last_error(); no exception crosses the boundary.
// Valid calls enqueue the kernels on the caller's stream and return without synchronising.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/tp_shard.h"
#include "kernels.hpp"

namespace {

thread_local char g_err[512] = "";

tp_status fail(tp_status st, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return st;
}

tp_status ok()
{
    g_err[0] = '\0';
    return TP_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A GEMM tile addresses its 256 operand rows through one buffer descriptor (32-bit byte
// offsets, range below 2 GiB): 256 bf16 rows of K elements span 2^31 bytes at K = 2^22, so a
// reduced (K) dimension must stay below 2^22 (it is a multiple of 8: at most 2^22 - 8).
constexpr int64_t kMaxReduced = (int64_t(1) << 22) - 8;
// A head's keys and values are addressed the same way with 256-byte rows (d = 128).
constexpr int64_t kMaxSeq = int64_t(1) << 22;

// Whether two byte ranges [a, a + na) and [b, b + nb) share a byte.
bool overlap(const void* a, size_t na, const void* b, size_t nb)
{
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// ---- test overrides -------------------------------------------------------------------------
std::mutex g_tuning_mu;
tps::Tuning g_tuning{};

// Parse "key=value[,key=value...]" into t; false on an unknown key or a bad value.
bool parse_tuning(const char* spec, tps::Tuning& t)
{
    t = tps::Tuning{};
    const char* c = spec;
    while (*c) {
        const char* end = std::strchr(c, ',');
        const size_t len = end ? (size_t)(end - c) : std::strlen(c);
        char item[64];
        if (len == 0 || len >= sizeof(item)) return false;
        std::memcpy(item, c, len);
        item[len] = '\0';
        char* eq = std::strchr(item, '=');
        if (!eq) return false;
        *eq = '\0';
        const char* key = item;
        const char* val = eq + 1;
        char* stop = nullptr;
        if (std::strcmp(key, "gemm_tile") == 0) {
            int bm = 0, bn = 0, n = 0;
            if (std::sscanf(val, "%dx%d%n", &bm, &bn, &n) != 2) return false;
            const bool known = (bm == 256 && (bn == 256 || bn == 192 || bn == 128)) ||
                               (bm == 128 && bn == 128);
            const char* rest = val + n;
            if (!known || (*rest && std::strcmp(rest, "w4") != 0)) return false;
            t.gemm_bm = bm;
            t.gemm_bn = bn;
            t.gemm_w4 = *rest ? 1 : 0;
        } else {
            const long v = std::strtol(val, &stop, 10);
            if (stop == val || *stop) return false;
            if (std::strcmp(key, "qkv_split") == 0 && v >= 1 && v <= 8) t.qkv_split = (int)v;
            else if (std::strcmp(key, "attn_sets") == 0 && (v == 1 || v == 2)) t.attn_sets = (int)v;
            else if (std::strcmp(key, "attn_split") == 0 && (v == 1 || v == 2)) t.attn_split = (int)v;
            else if (std::strcmp(key, "attn_pair") == 0 && (v == 1 || v == 2)) t.attn_pair = (int)v;
            else if (std::strcmp(key, "sum_grid") == 0 && v >= 0 && v <= INT32_MAX) t.sum_grid = (int)v;
            else if (std::strcmp(key, "sum_unroll") == 0 && (v == 1 || v == 2 || v == 4)) t.sum_unroll = (int)v;
            else if (std::strcmp(key, "sum_defer") == 0 && (v == 0 || v == 1)) t.sum_nodefer = 1 - (int)v;
            else if (std::strcmp(key, "sum_ring") == 0 && (v == 1 || v == 2)) t.sum_ring = (int)v;
            else return false;
        }
        if (end && !end[1]) return false;   // a trailing comma
        c = end ? end + 1 : c + len;
    }
    return true;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t dt_size(tp_dtype dt) { return dt == TP_F32 ? 4 : 2; }

// The kernels are built for gfx950 only; check the current device once per device ordinal.
tp_status check_device()
{
    static std::mutex mu;
    static int checked[64] = {0};   // 0 unknown, 1 ok, 2 wrong arch
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(TP_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(TP_ERR_DEVICE, "device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lock(mu);
    if (checked[dev] == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess)
            return fail(TP_ERR_HIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
        checked[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        if (checked[dev] == 2)
            return fail(TP_ERR_DEVICE, "device %d is %s; libtpshard is built for gfx950 only", dev,
                        prop.gcnArchName);
    }
    if (checked[dev] == 2) return fail(TP_ERR_DEVICE, "device %d is not gfx950", dev);
    return TP_OK;
}

tp_status hip_status(hipError_t e, const char* what)
{
    if (e != hipSuccess) return fail(TP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// ---- MLP --------------------------------------------------------------------------------
tp_status validate_mlp_sizes(int64_t tokens, int64_t hidden, int64_t ffn, int n, tp_dtype dt)
{
    if (dt != TP_F32 && dt != TP_BF16) return fail(TP_ERR_DTYPE, "MLP dtype %d not supported", (int)dt);
    if (n < 1) return fail(TP_ERR_SHAPE, "n_shards %d < 1", n);
    if (tokens < 1 || hidden < 1 || ffn < 1)
        return fail(TP_ERR_SHAPE, "tokens=%lld hidden=%lld ffn=%lld must be >= 1", (long long)tokens,
                    (long long)hidden, (long long)ffn);
    if (ffn % n != 0)
        return fail(TP_ERR_NOT_DIVISIBLE, "ffn=%lld not divisible by n_shards=%d", (long long)ffn, n);
    if (tokens > INT32_MAX || hidden > INT32_MAX || ffn > INT32_MAX)
        return fail(TP_ERR_SHAPE, "sizes above 2^31-1 are not supported");
    if (hidden % 8 != 0 || (ffn / n) % 8 != 0)
        return fail(TP_ERR_ALIGN, "hidden=%lld and ffn/N=%lld must be multiples of 8",
                    (long long)hidden, (long long)(ffn / n));
    if (hidden > kMaxReduced || ffn / n > kMaxReduced)
        return fail(TP_ERR_SHAPE, "hidden=%lld and ffn/N=%lld must be below 2^22", (long long)hidden,
                    (long long)(ffn / n));
    return TP_OK;
}

// Backward workspace: P and dP [T, F/N]; B_i^T [F/N, h]; A_i^T [h, F/N]; dP^T and GeLU(P)^T
// [F/N, T8]; X^T and dZ^T [h, T8] (T8 = tokens rounded up to 8), all bf16, 256-byte aligned.
struct BwdLayout {
    int64_t t8;
    size_t p, dp, bt, at, dpt, yt, xt, dzt, total;
};

BwdLayout bwd_layout(int64_t T, int64_t h, int64_t fl)
{
    BwdLayout L;
    L.t8 = (T + 7) / 8 * 8;
    size_t o = 0;
    auto take = [&](size_t elems) { const size_t at = o; o = round_up(o + elems * 2, 256); return at; };
    L.p = take((size_t)T * fl);
    L.dp = take((size_t)T * fl);
    L.bt = take((size_t)fl * h);
    L.at = take((size_t)h * fl);
    L.dpt = take((size_t)fl * L.t8);
    L.yt = take((size_t)fl * L.t8);
    L.xt = take((size_t)h * L.t8);
    L.dzt = take((size_t)h * L.t8);
    L.total = o;
    return L;
}

// ---- column / row-parallel linear layers ---------------------------------------------------
// column: split dimension is out_features; row: split dimension is in_features.
tp_status validate_linear(int64_t rows, int64_t in_f, int64_t out_f, int n, int rank, tp_dtype dt,
                          bool column)
{
    if (dt != TP_F32 && dt != TP_BF16) return fail(TP_ERR_DTYPE, "dtype %d not supported", (int)dt);
    if (n < 1) return fail(TP_ERR_SHAPE, "n_shards %d < 1", n);
    if (rows < 1 || in_f < 1 || out_f < 1)
        return fail(TP_ERR_SHAPE, "rows=%lld in=%lld out=%lld must be >= 1", (long long)rows,
                    (long long)in_f, (long long)out_f);
    if (rows > INT32_MAX || in_f > INT32_MAX || out_f > INT32_MAX)
        return fail(TP_ERR_SHAPE, "sizes above 2^31-1 are not supported");
    const int64_t split = column ? out_f : in_f;
    if (split % n != 0)
        return fail(TP_ERR_NOT_DIVISIBLE, "%s_features=%lld not divisible by n_shards=%d",
                    column ? "out" : "in", (long long)split, n);
    if (rank < 0 || rank >= n) return fail(TP_ERR_RANK, "rank %d outside [0, %d)", rank, n);
    const int64_t k = column ? in_f : in_f / n;     // reduced dimension
    const int64_t w = column ? out_f / n : out_f;   // output width
    if (k % 8 != 0 || w % 8 != 0)
        return fail(TP_ERR_ALIGN, "reduced dimension %lld and output width %lld must be multiples of 8",
                    (long long)k, (long long)w);
    if (k > kMaxReduced)
        return fail(TP_ERR_SHAPE, "reduced dimension %lld must be below 2^22", (long long)k);
    return TP_OK;
}

// Y[rows, width] = act(X[rows, k] W[width, k]^T + b)
// With pre (bf16 GeLU only), the pre-activation X W^T + b is stored there as well.
hipError_t launch_column(const void* X, const void* W, const void* b, void* Y, int64_t rows,
                         int64_t k, int64_t width, tp_activation act, tp_dtype dt, hipStream_t s,
                         void* pre = nullptr)
{
    tps::GemmProblem g{};
    g.A = X; g.lda = k;
    g.B = W; g.ldb = k;
    g.bias = b;
    g.C = Y; g.ldc = width;
    g.pre = pre;
    g.M = (int)rows; g.N = (int)width; g.K = (int)k;
    const tps::Epi epi = act == TP_ACT_GELU ? tps::Epi::BiasGelu : tps::Epi::Bias;
    return dt == TP_BF16 ? tps::gemm_bf16(g, epi, s) : tps::gemm_f32(g, epi, s);
}

// Z[rows, width] (fp32) = X[rows, k] W[width, k]^T
hipError_t launch_row(const void* X, const void* W, float* Z, int64_t rows, int64_t k,
                      int64_t width, tp_dtype dt, hipStream_t s)
{
    tps::GemmProblem g{};
    g.A = X; g.lda = k;
    g.B = W; g.ldb = k;
    g.C = Z; g.ldc = width;
    g.M = (int)rows; g.N = (int)width; g.K = (int)k;
    return dt == TP_BF16 ? tps::gemm_bf16(g, tps::Epi::F32, s) : tps::gemm_f32(g, tps::Epi::F32, s);
}

// ---- attention ---------------------------------------------------------------------------
struct AttnLayout {
    int hl, kvl, d;
    int64_t ld_vt;
    size_t q, k, vt, o, part_o, part_ml, total;   // part_*: key-range-split partials (or none)
    int qkv_splits;                               // K-split count of the Q/K/V projection
    size_t qkv_part;                              // its fp32 partials (when qkv_splits > 1)
};

// n_kv_heads key/value heads (= n_heads for multi-head attention). A rank holds
// n_kv_heads / N of them when N divides n_kv_heads, else (N a multiple of n_kv_heads) one
// head duplicated on N / n_kv_heads ranks (llms.blog, "Grouped-Query Attention (GQA)
// Constraints").
tp_status validate_attn_sizes(int64_t batch, int64_t seq, int64_t hidden, int n_heads,
                              int n_kv_heads, int n, tp_dtype dt, AttnLayout* L)
{
    if (dt != TP_BF16) return fail(TP_ERR_DTYPE, "attention supports TP_BF16 only (got %d)", (int)dt);
    if (n < 1) return fail(TP_ERR_SHAPE, "n_shards %d < 1", n);
    if (batch < 1 || seq < 1 || hidden < 1 || n_heads < 1)
        return fail(TP_ERR_SHAPE, "batch, seq, hidden and n_heads must be >= 1");
    if (batch * seq > INT32_MAX || hidden > INT32_MAX)
        return fail(TP_ERR_SHAPE, "sizes above 2^31-1 are not supported");
    if (hidden > kMaxReduced || seq > kMaxSeq)
        return fail(TP_ERR_SHAPE, "hidden=%lld must be below 2^22 and seq=%lld at most 2^22",
                    (long long)hidden, (long long)seq);
    if (hidden % n_heads != 0)
        return fail(TP_ERR_NOT_DIVISIBLE, "hidden=%lld not divisible by n_heads=%d", (long long)hidden,
                    n_heads);
    if (n_heads % n != 0)
        return fail(TP_ERR_NOT_DIVISIBLE, "n_heads=%d not divisible by n_shards=%d", n_heads, n);
    if (n_kv_heads < 1 || n_heads % n_kv_heads != 0)
        return fail(TP_ERR_NOT_DIVISIBLE, "n_heads=%d is not a multiple of n_kv_heads=%d", n_heads,
                    n_kv_heads);
    if (n_kv_heads % n != 0 && n % n_kv_heads != 0)
        return fail(TP_ERR_NOT_DIVISIBLE,
                    "n_kv_heads=%d neither divisible by n_shards=%d nor dividing it", n_kv_heads, n);
    const int64_t d = hidden / n_heads;
    if (d != 64 && d != 128) return fail(TP_ERR_SHAPE, "head dim %lld not supported (64 or 128)", (long long)d);
    if (hidden % 8 != 0) return fail(TP_ERR_ALIGN, "hidden=%lld must be a multiple of 8", (long long)hidden);
    L->hl = n_heads / n;
    L->kvl = n_kv_heads % n == 0 ? n_kv_heads / n : 1;
    L->d = (int)d;
    L->ld_vt = (int64_t)round_up((size_t)seq, 8);
    const size_t q_elems = (size_t)batch * L->hl * seq * d;
    const size_t kv_elems = (size_t)batch * L->kvl * seq * d;
    L->q = 0;
    L->k = round_up(L->q + q_elems * 2, 256);
    L->vt = round_up(L->k + kv_elems * 2, 256);
    L->o = round_up(L->vt + (size_t)batch * L->kvl * d * L->ld_vt * 2, 256);
    const size_t o_end = round_up(L->o + (size_t)batch * seq * L->hl * d * 2, 256);
    const size_t part = tps::attention_partial_bytes((int)batch, L->hl, (int)seq, (int)d, true, nullptr);
    // split partials: outputs [items][128][d] then (max, denominator) [items][128][2]
    const size_t part_o_bytes = part / (size_t)(d + 2) * (size_t)d;
    L->part_o = o_end;
    L->part_ml = round_up(L->part_o + part_o_bytes, 256);
    L->total = part ? round_up(L->part_ml + (part - part_o_bytes), 256) : o_end;
    // The split Q/K/V projection's partials [splits][T][N] fp32 share the space from O on:
    // they are consumed by the scatter before the attention writes O or its own partials.
    const int64_t T = batch * seq, ncol = (int64_t)(L->hl + 2 * L->kvl) * d;
    L->qkv_splits = tps::qkv_k_splits((int)T, (int)ncol, (int)hidden);
    L->qkv_part = L->o;
    if (L->qkv_splits > 1)
        L->total = std::max(L->total, round_up(L->o + (size_t)L->qkv_splits * T * ncol * 4, 256));
    return TP_OK;
}

// ---- sequence-parallel boundary -------------------------------------------------------------
tp_status validate_sp(int n_parts, int64_t batch, int64_t seq, int64_t hidden, int rank,
                      tp_dtype dt, int64_t max_hidden)
{
    if (dt != TP_F32 && dt != TP_BF16) return fail(TP_ERR_DTYPE, "dtype %d not supported", (int)dt);
    if (n_parts < 1 || n_parts > 64) return fail(TP_ERR_SHAPE, "n_parts=%d outside [1, 64]", n_parts);
    if (batch < 1 || seq < 1 || hidden < 1)
        return fail(TP_ERR_SHAPE, "batch, seq and hidden must be >= 1");
    if (batch * seq > INT32_MAX || hidden > max_hidden)
        return fail(TP_ERR_SHAPE, "batch*seq must be < 2^31 and hidden <= %lld", (long long)max_hidden);
    if (seq % n_parts != 0)
        return fail(TP_ERR_NOT_DIVISIBLE, "seq=%lld not divisible into %d slices", (long long)seq, n_parts);
    if (rank < 0 || rank >= n_parts) return fail(TP_ERR_RANK, "rank %d outside [0, %d)", rank, n_parts);
    if (hidden % 8 != 0) return fail(TP_ERR_ALIGN, "hidden=%lld must be a multiple of 8", (long long)hidden);
    return TP_OK;
}

tp_status check_parts(const void* const* parts, int n_parts, const char* what)
{
    if (!parts) return fail(TP_ERR_NULL, "%s array is NULL", what);
    for (int q = 0; q < n_parts; ++q) {
        if (!parts[q]) return fail(TP_ERR_NULL, "%s %d is NULL (missing rank)", what, q);
        if (!aligned16(parts[q])) return fail(TP_ERR_ALIGN, "%s %d is not 16-byte aligned", what, q);
    }
    return TP_OK;
}

// Shape, rank and workspace checks shared by the attention calls.
tp_status validate_attn_call(int64_t batch, int64_t seq, int64_t hidden, int n_heads, int n_kv_heads,
                             int n_shards, int rank, tp_dtype dt, void* workspace,
                             size_t workspace_bytes, AttnLayout* L)
{
    tp_status st = validate_attn_sizes(batch, seq, hidden, n_heads, n_kv_heads, n_shards, dt, L);
    if (st != TP_OK) return st;
    if (rank < 0 || rank >= n_shards)
        return fail(TP_ERR_RANK, "rank %d outside [0, %d)", rank, n_shards);
    if (workspace && !aligned16(workspace))
        return fail(TP_ERR_ALIGN, "every pointer must be 16-byte aligned");
    if (!workspace || workspace_bytes < L->total)
        return fail(TP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L->total,
                    workspace ? workspace_bytes : (size_t)0);
    return TP_OK;
}

// Step 1 of the attention block: the column-parallel Q/K/V projection of the local heads into
// the workspace (Q scaled, per head; V transposed).
tp_status launch_qkv(const void* X, const void* Wqkv_i, const void* bqkv_i, int64_t batch,
                     int64_t seq, int64_t hidden, const AttnLayout& L, char* ws, hipStream_t s)
{
    const int T = (int)(batch * seq);
    const int w = L.hl * L.d;       // local query width
    const int wkv = L.kvl * L.d;    // local key (and value) width
    tps::GemmProblem g{};
    g.A = X; g.lda = hidden;
    g.B = Wqkv_i; g.ldb = hidden;
    g.bias = bqkv_i;
    g.M = T; g.N = w + 2 * wkv; g.K = (int)hidden;
    g.q = ws + L.q; g.k = ws + L.k; g.vt = ws + L.vt;
    g.seq = (int)seq; g.heads_local = L.hl; g.kv_heads_local = L.kvl; g.head_dim = L.d;
    g.ld_vt = L.ld_vt;
    // The softmax's scale 1/sqrt(d), with log2(e) for its base-2 exponentials, is folded into
    // the stored queries (one rounding of the fp32 result either way).
    g.q_scale = (float)(1.4426950408889634 / __builtin_sqrt((double)L.d));
    if (L.qkv_splits > 1) {
        // few output columns: the projection runs as K-split fp32 partials, then one pass
        // sums them and applies the bias, the scale and the scatter
        float* parts = reinterpret_cast<float*>(ws + L.qkv_part);
        g.k_splits = L.qkv_splits;
        g.split_stride = (int64_t)g.M * g.N;
        tps::GemmProblem gp = g;
        gp.bias = nullptr;
        gp.C = parts; gp.ldc = g.N;
        hipError_t e = tps::gemm_bf16(gp, tps::Epi::F32, s);
        if (e != hipSuccess) return hip_status(e, "QKV projection launch");
        return hip_status(tps::qkv_reduce_scatter(g, parts, s), "QKV scatter launch");
    }
    return hip_status(tps::gemm_bf16(g, tps::Epi::Qkv, s), "QKV projection launch");
}

// Step 2: head-local attention from the workspace's Q, K, V^T into its O (heads concatenated).
tp_status launch_heads(int64_t batch, int64_t seq, int causal, const AttnLayout& L, char* ws,
                       hipStream_t s)
{
    tps::AttnProblem a{};
    a.q = ws + L.q; a.k = ws + L.k; a.vt = ws + L.vt; a.o = ws + L.o;
    a.batch = (int)batch; a.heads_local = L.hl; a.kv_heads_local = L.kvl; a.seq = (int)seq;
    a.head_dim = L.d; a.ld_vt = L.ld_vt; a.causal = causal ? 1 : 0;
    const size_t part = tps::attention_partial_bytes((int)batch, L.hl, (int)seq, L.d, causal, &a.kv_split);
    if (part) {
        a.part_o = reinterpret_cast<float*>(ws + L.part_o);
        a.part_ml = reinterpret_cast<float*>(ws + L.part_ml);
    } else {
        a.kv_split = 1;
    }
    return hip_status(tps::attention_fwd(a, s), "attention launch");
}

// ---- allocation-free MLP shard -------------------------------------------------------------
// Scratch of tp_mlp_shard_fwd_noalloc: the hidden activation Y_i [tokens, ffn/N] that
// tp_mlp_shard_fwd keeps in the caller's workspace. Each device holds its own copy of this
// array (from the library's load until the process ends). In host code the name is only a
// stand-in: kernels receive the device address from hipGetSymbolAddress, kept per device.
constexpr size_t kScratchBytes = TP_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

// This device's address of the scratch array (looked up once per device, that device current).
tp_status device_scratch(void** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(TP_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= 64) return fail(TP_ERR_DEVICE, "device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(TP_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return TP_OK;
}

// The exchange kernels read every input range while other lanes write the output: an output
// that shares a byte with an input is rejected.
tp_status check_no_overlap(const void* const* parts, int n_parts, size_t part_bytes, const void* out,
                           size_t out_bytes, const char* what)
{
    for (int q = 0; q < n_parts; ++q)
        if (overlap(out, out_bytes, parts[q], part_bytes))
            return fail(TP_ERR_ALIAS, "%s overlaps input %d", what, q);
    return TP_OK;
}

}  // namespace

tps::Tuning tps::tuning()
{
    std::lock_guard<std::mutex> lock(g_tuning_mu);
    return g_tuning;
}

extern "C" {

int tp_abi_version(void) { return TP_SHARD_ABI_VERSION; }

tp_status tp_set_test_overrides(const char* spec)
{
    tps::Tuning t{};
    if (spec && !parse_tuning(spec, t))
        return fail(TP_ERR_SHAPE, "unknown override or bad value in \"%s\"", spec);
    std::lock_guard<std::mutex> lock(g_tuning_mu);
    g_tuning = t;
    return ok();
}

const char* tp_last_error(void) { return g_err; }

size_t tp_mlp_workspace_bytes(int64_t tokens, int64_t hidden, int64_t ffn, int n_shards, tp_dtype dt)
{
    if (validate_mlp_sizes(tokens, hidden, ffn, n_shards, dt) != TP_OK) return 0;
    return round_up((size_t)tokens * (size_t)(ffn / n_shards) * dt_size(dt), 256);
}

tp_status tp_mlp_shard_fwd(const void* X, const void* A_i, const void* a_i, const void* B_i,
                           float* Z_i, int64_t tokens, int64_t hidden, int64_t ffn, int n_shards,
                           int rank, tp_dtype dt, void* workspace, size_t workspace_bytes,
                           void* stream)
{
    if (!X || !A_i || !B_i || !Z_i) return fail(TP_ERR_NULL, "X, A_i, B_i and Z_i must be non-NULL");
    tp_status st = validate_mlp_sizes(tokens, hidden, ffn, n_shards, dt);
    if (st != TP_OK) return st;
    if (rank < 0 || rank >= n_shards)
        return fail(TP_ERR_RANK, "rank %d outside [0, %d)", rank, n_shards);
    if (!aligned16(X) || !aligned16(A_i) || !aligned16(B_i) || !aligned16(Z_i) ||
        (a_i && !aligned16(a_i)) || (workspace && !aligned16(workspace)))
        return fail(TP_ERR_ALIGN, "every pointer must be 16-byte aligned");
    const size_t need = tp_mlp_workspace_bytes(tokens, hidden, ffn, n_shards, dt);
    if (!workspace || workspace_bytes < need)
        return fail(TP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    st = check_device();
    if (st != TP_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // Column-parallel: Y_i = GeLU(X A_i + a_i), [tokens, F/N] (no communication).
    hipError_t e = launch_column(X, A_i, a_i, workspace, tokens, hidden, ffn / n_shards,
                                 TP_ACT_GELU, dt, s);
    if (e != hipSuccess) return hip_status(e, "column-parallel kernel launch");
    // Row-parallel: Z_i = Y_i B_i, [tokens, hidden] fp32 partial.
    e = launch_row(workspace, B_i, Z_i, tokens, ffn / n_shards, hidden, dt, s);
    return hip_status(e, "row-parallel kernel launch");
}

tp_status tp_mlp_shard_fwd_save(const void* X, const void* A_i, const void* a_i, const void* B_i,
                                float* Z_i, void* P_i, int64_t tokens, int64_t hidden, int64_t ffn,
                                int n_shards, int rank, tp_dtype dt, void* workspace,
                                size_t workspace_bytes, void* stream)
{
    if (!X || !A_i || !B_i || !Z_i || !P_i)
        return fail(TP_ERR_NULL, "X, A_i, B_i, Z_i and P_i must be non-NULL");
    if (dt != TP_BF16)
        return fail(TP_ERR_DTYPE, "the forward that keeps P supports TP_BF16 only (got %d)", (int)dt);
    tp_status st = validate_mlp_sizes(tokens, hidden, ffn, n_shards, dt);
    if (st != TP_OK) return st;
    if (rank < 0 || rank >= n_shards)
        return fail(TP_ERR_RANK, "rank %d outside [0, %d)", rank, n_shards);
    if (!aligned16(X) || !aligned16(A_i) || !aligned16(B_i) || !aligned16(Z_i) ||
        !aligned16(P_i) || (a_i && !aligned16(a_i)) || (workspace && !aligned16(workspace)))
        return fail(TP_ERR_ALIGN, "every pointer must be 16-byte aligned");
    const size_t need = tp_mlp_workspace_bytes(tokens, hidden, ffn, n_shards, dt);
    if (!workspace || workspace_bytes < need)
        return fail(TP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    // P_i is written by the same kernel as Y_i (the workspace), while X, A_i and a_i are read
    const size_t fl = (size_t)(ffn / n_shards), pbytes = (size_t)tokens * fl * 2;
    if (overlap(P_i, pbytes, workspace, need) ||
        overlap(P_i, pbytes, Z_i, (size_t)tokens * (size_t)hidden * 4) ||
        overlap(P_i, pbytes, X, (size_t)tokens * (size_t)hidden * 2) ||
        overlap(P_i, pbytes, A_i, fl * (size_t)hidden * 2) ||
        overlap(P_i, pbytes, B_i, (size_t)hidden * fl * 2) || (a_i && overlap(P_i, pbytes, a_i, fl * 2)))
        return fail(TP_ERR_ALIAS, "P_i overlaps the workspace, Z_i or an input");
    st = check_device();
    if (st != TP_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // the launches of tp_mlp_shard_fwd; the column GEMM's epilogue also stores P
    hipError_t e = launch_column(X, A_i, a_i, workspace, tokens, hidden, ffn / n_shards,
                                 TP_ACT_GELU, dt, s, P_i);
    if (e != hipSuccess) return hip_status(e, "column-parallel kernel launch");
    e = launch_row(workspace, B_i, Z_i, tokens, ffn / n_shards, hidden, dt, s);
    return hip_status(e, "row-parallel kernel launch");
}

tp_status tp_mlp_shard_fwd_noalloc(const void* X, const void* A_i, const void* a_i,
                                   const void* B_i, float* Z_i, int64_t tokens, int64_t hidden,
                                   int64_t ffn, int n_shards, int rank, tp_dtype dt, void* stream)
{
    if (!X || !A_i || !B_i || !Z_i) return fail(TP_ERR_NULL, "X, A_i, B_i and Z_i must be non-NULL");
    tp_status st = validate_mlp_sizes(tokens, hidden, ffn, n_shards, dt);
    if (st != TP_OK) return st;
    if (rank < 0 || rank >= n_shards)
        return fail(TP_ERR_RANK, "rank %d outside [0, %d)", rank, n_shards);
    if (!aligned16(X) || !aligned16(A_i) || !aligned16(B_i) || !aligned16(Z_i) ||
        (a_i && !aligned16(a_i)))
        return fail(TP_ERR_ALIGN, "every pointer must be 16-byte aligned");
    const size_t need = tp_mlp_workspace_bytes(tokens, hidden, ffn, n_shards, dt);
    if (need > kScratchBytes)
        return fail(TP_ERR_WORKSPACE,
                    "Y_i of %zu bytes exceeds the %zu-byte device scratch of the allocation-free "
                    "call; use tp_mlp_shard_fwd with a workspace", need, kScratchBytes);
    st = check_device();
    if (st != TP_OK) return st;
    void* ws = nullptr;
    st = device_scratch(&ws);
    if (st != TP_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    // the same two launches as tp_mlp_shard_fwd, with Y_i in the device scratch
    hipError_t e = launch_column(X, A_i, a_i, ws, tokens, hidden, ffn / n_shards, TP_ACT_GELU, dt, s);
    if (e != hipSuccess) return hip_status(e, "column-parallel kernel launch");
    e = launch_row(ws, B_i, Z_i, tokens, ffn / n_shards, hidden, dt, s);
    return hip_status(e, "row-parallel kernel launch");
}

size_t tp_mlp_bwd_workspace_bytes(int64_t tokens, int64_t hidden, int64_t ffn, int n_shards,
                                  tp_dtype dt)
{
    if (dt != TP_BF16 || tokens > kMaxReduced) return 0;
    if (validate_mlp_sizes(tokens, hidden, ffn, n_shards, dt) != TP_OK) return 0;
    return bwd_layout(tokens, hidden, ffn / n_shards).total;
}

namespace {

// The MLP shard's backward. P_saved: the forward's pre-activation P [T, F/N] bf16
// (tp_mlp_shard_fwd_save), or nullptr to recompute it into the workspace from X, A_i, a_i.
tp_status mlp_shard_bwd(const void* X, const void* A_i, const void* a_i, const void* B_i,
                        const void* P_saved, const void* dZ, float* dX_i, float* dA_i,
                        float* da_i, float* dB_i, int64_t tokens, int64_t hidden, int64_t ffn,
                        int n_shards, int rank, tp_dtype dt, void* workspace,
                        size_t workspace_bytes, void* stream)
{
    if (!X || !A_i || !B_i || !dZ || !dX_i || !dA_i || !dB_i)
        return fail(TP_ERR_NULL, "X, A_i, B_i, dZ, dX_i, dA_i and dB_i must be non-NULL");
    if (dt != TP_BF16) return fail(TP_ERR_DTYPE, "the MLP backward supports TP_BF16 only (got %d)", (int)dt);
    tp_status st = validate_mlp_sizes(tokens, hidden, ffn, n_shards, dt);
    if (st != TP_OK) return st;
    if (tokens > kMaxReduced)   // dA and dB reduce over the tokens
        return fail(TP_ERR_SHAPE, "tokens=%lld must be below 2^22 in the backward", (long long)tokens);
    if (rank < 0 || rank >= n_shards)
        return fail(TP_ERR_RANK, "rank %d outside [0, %d)", rank, n_shards);
    if (!aligned16(X) || !aligned16(A_i) || !aligned16(B_i) || !aligned16(dZ) ||
        !aligned16(dX_i) || !aligned16(dA_i) || !aligned16(dB_i) || (a_i && !aligned16(a_i)) ||
        (da_i && !aligned16(da_i)) || (workspace && !aligned16(workspace)) ||
        (P_saved && !aligned16(P_saved)))
        return fail(TP_ERR_ALIGN, "every pointer must be 16-byte aligned");
    const int64_t T = tokens, h = hidden, fl = ffn / n_shards;
    const BwdLayout L = bwd_layout(T, h, fl);
    if (!workspace || workspace_bytes < L.total)
        return fail(TP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", L.total,
                    workspace ? workspace_bytes : (size_t)0);
    // the workspace and the gradients are written while P is still to be read (the GeLU'
    // epilogue, then the GeLU(P) transpose after dX and dA are written)
    if (P_saved) {
        const size_t pb = (size_t)T * (size_t)fl * 2;
        if (overlap(P_saved, pb, workspace, L.total) ||
            overlap(P_saved, pb, dX_i, (size_t)T * (size_t)h * 4) ||
            overlap(P_saved, pb, dA_i, (size_t)fl * (size_t)h * 4) ||
            overlap(P_saved, pb, dB_i, (size_t)h * (size_t)fl * 4) ||
            (da_i && overlap(P_saved, pb, da_i, (size_t)fl * 4)))
            return fail(TP_ERR_ALIAS, "P_i overlaps the workspace or a gradient");
    }
    st = check_device();
    if (st != TP_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* ws = reinterpret_cast<char*>(workspace);
    hipError_t e;
#define TPS_TRY(call, what) \
    do { e = (call); if (e != hipSuccess) return hip_status(e, what); } while (0)
    // 1. P = X A_r + a_r [T, F/N] bf16: the forward's, or recomputed
    const char* P = P_saved ? reinterpret_cast<const char*>(P_saved) : ws + L.p;
    if (!P_saved)
        TPS_TRY(launch_column(X, A_i, a_i, ws + L.p, T, h, fl, TP_ACT_NONE, dt, s), "P = X A + a");
    // 2. dP = (dZ B_r^T) * GeLU'(P): B_r = B_i^T is [F/N, h], contiguous along h
    TPS_TRY(tps::transpose_bf16(B_i, (int)h, (int)fl, fl, ws + L.bt, h, false, s), "B transpose");
    {
        tps::GemmProblem g{};
        g.A = dZ; g.lda = h;
        g.B = ws + L.bt; g.ldb = h;
        g.aux = P; g.ldaux = fl;
        g.C = ws + L.dp; g.ldc = fl;
        g.M = (int)T; g.N = (int)fl; g.K = (int)h;
        TPS_TRY(tps::gemm_bf16(g, tps::Epi::GeluGrad, s), "dP = dZ B^T * GeLU'(P)");
    }
    // 3. dX_i = dP A_r^T: A_r = A_i^T is [h, F/N], contiguous along F/N
    TPS_TRY(tps::transpose_bf16(A_i, (int)fl, (int)h, h, ws + L.at, fl, false, s), "A transpose");
    TPS_TRY(launch_row(ws + L.dp, ws + L.at, dX_i, T, fl, h, dt, s), "dX = dP A^T");
    // 4. dP^T [F/N, T8]; da_r = its row sums; dA_i = dP^T X, reduced over tokens
    TPS_TRY(tps::transpose_bf16(ws + L.dp, (int)T, (int)fl, fl, ws + L.dpt, L.t8, false, s),
            "dP transpose");
    if (da_i) TPS_TRY(tps::row_sum_bf16(ws + L.dpt, (int)fl, (int)T, L.t8, da_i, s), "da = sum dP");
    TPS_TRY(tps::transpose_bf16(X, (int)T, (int)h, h, ws + L.xt, L.t8, false, s), "X transpose");
    TPS_TRY(launch_row(ws + L.dpt, ws + L.xt, dA_i, fl, L.t8, h, dt, s), "dA = dP^T X");
    // 5. dB_i = dZ^T GeLU(P), reduced over tokens: GeLU(P)^T [F/N, T8], dZ^T [h, T8]
    TPS_TRY(tps::transpose_bf16(P, (int)T, (int)fl, fl, ws + L.yt, L.t8, true, s),
            "GeLU(P) transpose");
    TPS_TRY(tps::transpose_bf16(dZ, (int)T, (int)h, h, ws + L.dzt, L.t8, false, s), "dZ transpose");
    TPS_TRY(launch_row(ws + L.dzt, ws + L.yt, dB_i, h, L.t8, fl, dt, s), "dB = dZ^T Y");
#undef TPS_TRY
    return ok();
}

}  // namespace

tp_status tp_mlp_shard_bwd(const void* X, const void* A_i, const void* a_i, const void* B_i,
                           const void* dZ, float* dX_i, float* dA_i, float* da_i, float* dB_i,
                           int64_t tokens, int64_t hidden, int64_t ffn, int n_shards, int rank,
                           tp_dtype dt, void* workspace, size_t workspace_bytes, void* stream)
{
    return mlp_shard_bwd(X, A_i, a_i, B_i, nullptr, dZ, dX_i, dA_i, da_i, dB_i, tokens, hidden,
                         ffn, n_shards, rank, dt, workspace, workspace_bytes, stream);
}

tp_status tp_mlp_shard_bwd_saved(const void* X, const void* A_i, const void* B_i, const void* P_i,
                                 const void* dZ, float* dX_i, float* dA_i, float* da_i,
                                 float* dB_i, int64_t tokens, int64_t hidden, int64_t ffn,
                                 int n_shards, int rank, tp_dtype dt, void* workspace,
                                 size_t workspace_bytes, void* stream)
{
    if (!P_i) return fail(TP_ERR_NULL, "P_i must be non-NULL");
    return mlp_shard_bwd(X, A_i, nullptr, B_i, P_i, dZ, dX_i, dA_i, da_i, dB_i, tokens, hidden,
                         ffn, n_shards, rank, dt, workspace, workspace_bytes, stream);
}

size_t tp_swiglu_workspace_bytes(int64_t tokens, int64_t hidden, int64_t ffn, int n_shards,
                                 tp_dtype dt)
{
    if (dt != TP_BF16) return 0;
    if (validate_mlp_sizes(tokens, hidden, ffn, n_shards, dt) != TP_OK) return 0;
    return round_up((size_t)tokens * (size_t)(ffn / n_shards) * 2, 256);
}

tp_status tp_swiglu_shard_fwd(const void* X, const void* Wgate_i, const void* Wup_i,
                              const void* Wdown_i, float* Z_i, int64_t tokens, int64_t hidden,
                              int64_t ffn, int n_shards, int rank, tp_dtype dt, void* workspace,
                              size_t workspace_bytes, void* stream)
{
    if (!X || !Wgate_i || !Wup_i || !Wdown_i || !Z_i)
        return fail(TP_ERR_NULL, "X, Wgate_i, Wup_i, Wdown_i and Z_i must be non-NULL");
    if (dt != TP_BF16) return fail(TP_ERR_DTYPE, "the SwiGLU shard supports TP_BF16 only (got %d)", (int)dt);
    tp_status st = validate_mlp_sizes(tokens, hidden, ffn, n_shards, dt);
    if (st != TP_OK) return st;
    if (rank < 0 || rank >= n_shards)
        return fail(TP_ERR_RANK, "rank %d outside [0, %d)", rank, n_shards);
    if (!aligned16(X) || !aligned16(Wgate_i) || !aligned16(Wup_i) || !aligned16(Wdown_i) ||
        !aligned16(Z_i) || (workspace && !aligned16(workspace)))
        return fail(TP_ERR_ALIGN, "every pointer must be 16-byte aligned");
    const size_t need = tp_swiglu_workspace_bytes(tokens, hidden, ffn, n_shards, dt);
    if (!workspace || workspace_bytes < need)
        return fail(TP_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    workspace ? workspace_bytes : (size_t)0);
    st = check_device();
    if (st != TP_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    const int64_t fl = ffn / n_shards;
    // Column-parallel gate and up projections with the gate applied locally:
    // A_i = SiLU(X W_gate,i) * (X W_up,i), [tokens, F/N] (no communication).
    tps::GemmProblem g{};
    g.A = X; g.lda = hidden;
    g.B = Wgate_i; g.B2 = Wup_i; g.ldb = hidden;
    g.C = workspace; g.ldc = fl;
    g.M = (int)tokens; g.N = (int)fl; g.K = (int)hidden;
    hipError_t e = tps::gemm_bf16(g, tps::Epi::SwiGlu, s);
    if (e != hipSuccess) return hip_status(e, "gated column-parallel kernel launch");
    // Row-parallel down projection: Z_i = A_i W_down,i, [tokens, hidden] fp32 partial.
    e = launch_row(workspace, Wdown_i, Z_i, tokens, fl, hidden, dt, s);
    return hip_status(e, "row-parallel kernel launch");
}

tp_status tp_column_parallel_fwd(const void* X, const void* W_i, const void* b_i, void* Y_i,
                                 int64_t rows, int64_t in_features, int64_t out_features,
                                 int n_shards, int rank, tp_activation act, tp_dtype dt,
                                 void* stream)
{
    if (!X || !W_i || !Y_i) return fail(TP_ERR_NULL, "X, W_i and Y_i must be non-NULL");
    tp_status st = validate_linear(rows, in_features, out_features, n_shards, rank, dt, true);
    if (st != TP_OK) return st;
    if (act != TP_ACT_NONE && act != TP_ACT_GELU)
        return fail(TP_ERR_SHAPE, "activation %d not supported", (int)act);
    if (!aligned16(X) || !aligned16(W_i) || !aligned16(Y_i) || (b_i && !aligned16(b_i)))
        return fail(TP_ERR_ALIGN, "every pointer must be 16-byte aligned");
    st = check_device();
    if (st != TP_OK) return st;
    hipError_t e = launch_column(X, W_i, b_i, Y_i, rows, in_features, out_features / n_shards,
                                 act, dt, reinterpret_cast<hipStream_t>(stream));
    return hip_status(e, "column-parallel kernel launch");
}

tp_status tp_row_parallel_fwd(const void* X_i, const void* W_i, float* Z_i, int64_t rows,
                              int64_t in_features, int64_t out_features, int n_shards, int rank,
                              tp_dtype dt, void* stream)
{
    if (!X_i || !W_i || !Z_i) return fail(TP_ERR_NULL, "X_i, W_i and Z_i must be non-NULL");
    tp_status st = validate_linear(rows, in_features, out_features, n_shards, rank, dt, false);
    if (st != TP_OK) return st;
    if (!aligned16(X_i) || !aligned16(W_i) || !aligned16(Z_i))
        return fail(TP_ERR_ALIGN, "every pointer must be 16-byte aligned");
    st = check_device();
    if (st != TP_OK) return st;
    hipError_t e = launch_row(X_i, W_i, Z_i, rows, in_features / n_shards, out_features, dt,
                              reinterpret_cast<hipStream_t>(stream));
    return hip_status(e, "row-parallel kernel launch");
}

tp_status tp_row_parallel_sum_fwd(const void* X_i, const void* W_i, const float* const* Z_parts,
                                  void* Z, tp_dtype out_dt, int64_t rows, int64_t in_features,
                                  int64_t out_features, int n_shards, int rank, tp_dtype dt,
                                  void* stream)
{
    if (!X_i || !W_i || !Z || !Z_parts) return fail(TP_ERR_NULL, "X_i, W_i, Z_parts and Z must be non-NULL");
    if (dt != TP_BF16) return fail(TP_ERR_DTYPE, "the fused row-parallel sum supports TP_BF16 inputs only");
    if (out_dt != TP_F32 && out_dt != TP_BF16) return fail(TP_ERR_DTYPE, "out_dt %d not supported", (int)out_dt);
    tp_status st = validate_linear(rows, in_features, out_features, n_shards, rank, dt, false);
    if (st != TP_OK) return st;
    if (n_shards > tps::kMaxSumParts)
        return fail(TP_ERR_SHAPE, "n_shards=%d above %d for the fused sum", n_shards, tps::kMaxSumParts);
    if (!aligned16(X_i) || !aligned16(W_i) || !aligned16(Z))
        return fail(TP_ERR_ALIGN, "every pointer must be 16-byte aligned");
    const size_t pbytes = (size_t)(rows * out_features) * 4;
    const size_t zbytes = (size_t)(rows * out_features) * dt_size(out_dt);
    for (int q = 0; q < n_shards; ++q) {
        if (q == rank) continue;
        if (!Z_parts[q]) return fail(TP_ERR_NULL, "partial %d is NULL (missing rank)", q);
        if (!aligned16(Z_parts[q])) return fail(TP_ERR_ALIGN, "partial %d is not 16-byte aligned", q);
        if (overlap(Z, zbytes, Z_parts[q], pbytes))
            return fail(TP_ERR_ALIAS, "Z overlaps partial %d", q);
    }
    const int64_t k = in_features / n_shards;
    if (overlap(Z, zbytes, X_i, (size_t)(rows * k) * 2) ||
        overlap(Z, zbytes, W_i, (size_t)(out_features * k) * 2))
        return fail(TP_ERR_ALIAS, "Z overlaps X_i or W_i");
    st = check_device();
    if (st != TP_OK) return st;
    tps::GemmProblem g{};
    g.A = X_i; g.lda = k;
    g.B = W_i; g.ldb = k;
    g.C = Z; g.ldc = out_features;
    g.M = (int)rows; g.N = (int)out_features; g.K = (int)k;
    g.n_parts = n_shards;
    g.part_rank = rank;
    for (int q = 0; q < n_shards; ++q) g.part[q] = q == rank ? nullptr : Z_parts[q];
    return hip_status(tps::gemm_bf16(g, out_dt == TP_BF16 ? tps::Epi::SumBf16 : tps::Epi::SumF32,
                                     reinterpret_cast<hipStream_t>(stream)),
                      "fused row-parallel sum kernel launch");
}

size_t tp_attn_workspace_bytes(int64_t batch, int64_t seq, int64_t hidden, int n_heads,
                               int n_shards, tp_dtype dt)
{
    return tp_gqa_attn_workspace_bytes(batch, seq, hidden, n_heads, n_heads, n_shards, dt);
}

tp_status tp_attn_workspace_layout(int64_t batch, int64_t seq, int64_t hidden, int n_heads,
                                   int n_shards, tp_dtype dt, size_t* q_off, size_t* k_off,
                                   size_t* vt_off, size_t* o_off)
{
    return tp_gqa_attn_workspace_layout(batch, seq, hidden, n_heads, n_heads, n_shards, dt, q_off,
                                        k_off, vt_off, o_off);
}

tp_status tp_attn_shard_fwd(const void* X, const void* Wqkv_i, const void* bqkv_i,
                            const void* Wo_i, float* Z_i, int64_t batch, int64_t seq,
                            int64_t hidden, int n_heads, int causal, int n_shards, int rank,
                            tp_dtype dt, void* workspace, size_t workspace_bytes, void* stream)
{
    return tp_gqa_attn_shard_fwd(X, Wqkv_i, bqkv_i, Wo_i, Z_i, batch, seq, hidden, n_heads,
                                 n_heads, causal, n_shards, rank, dt, workspace, workspace_bytes,
                                 stream);
}

size_t tp_gqa_attn_workspace_bytes(int64_t batch, int64_t seq, int64_t hidden, int n_heads,
                                   int n_kv_heads, int n_shards, tp_dtype dt)
{
    AttnLayout L;
    if (validate_attn_sizes(batch, seq, hidden, n_heads, n_kv_heads, n_shards, dt, &L) != TP_OK)
        return 0;
    return L.total;
}

tp_status tp_gqa_attn_workspace_layout(int64_t batch, int64_t seq, int64_t hidden, int n_heads,
                                       int n_kv_heads, int n_shards, tp_dtype dt, size_t* q_off,
                                       size_t* k_off, size_t* vt_off, size_t* o_off)
{
    AttnLayout L;
    tp_status st = validate_attn_sizes(batch, seq, hidden, n_heads, n_kv_heads, n_shards, dt, &L);
    if (st != TP_OK) return st;
    if (q_off) *q_off = L.q;
    if (k_off) *k_off = L.k;
    if (vt_off) *vt_off = L.vt;
    if (o_off) *o_off = L.o;
    return ok();
}

tp_status tp_qkv_projection_fwd(const void* X, const void* Wqkv_i, const void* bqkv_i,
                                int64_t batch, int64_t seq, int64_t hidden, int n_heads,
                                int n_kv_heads, int n_shards, int rank, tp_dtype dt,
                                void* workspace, size_t workspace_bytes, void* stream)
{
    if (!X || !Wqkv_i) return fail(TP_ERR_NULL, "X and Wqkv_i must be non-NULL");
    AttnLayout L;
    tp_status st = validate_attn_call(batch, seq, hidden, n_heads, n_kv_heads, n_shards, rank, dt,
                                      workspace, workspace_bytes, &L);
    if (st != TP_OK) return st;
    if (!aligned16(X) || !aligned16(Wqkv_i) || (bqkv_i && !aligned16(bqkv_i)))
        return fail(TP_ERR_ALIGN, "every pointer must be 16-byte aligned");
    st = check_device();
    if (st != TP_OK) return st;
    return launch_qkv(X, Wqkv_i, bqkv_i, batch, seq, hidden, L, reinterpret_cast<char*>(workspace),
                      reinterpret_cast<hipStream_t>(stream));
}

tp_status tp_head_attention_fwd(int64_t batch, int64_t seq, int64_t hidden, int n_heads,
                                int n_kv_heads, int causal, int n_shards, int rank, tp_dtype dt,
                                void* workspace, size_t workspace_bytes, void* stream)
{
    AttnLayout L;
    tp_status st = validate_attn_call(batch, seq, hidden, n_heads, n_kv_heads, n_shards, rank, dt,
                                      workspace, workspace_bytes, &L);
    if (st != TP_OK) return st;
    st = check_device();
    if (st != TP_OK) return st;
    return launch_heads(batch, seq, causal, L, reinterpret_cast<char*>(workspace),
                        reinterpret_cast<hipStream_t>(stream));
}

tp_status tp_gqa_attn_shard_fwd(const void* X, const void* Wqkv_i, const void* bqkv_i,
                                const void* Wo_i, float* Z_i, int64_t batch, int64_t seq,
                                int64_t hidden, int n_heads, int n_kv_heads, int causal,
                                int n_shards, int rank, tp_dtype dt, void* workspace,
                                size_t workspace_bytes, void* stream)
{
    if (!X || !Wqkv_i || !Wo_i || !Z_i)
        return fail(TP_ERR_NULL, "X, Wqkv_i, Wo_i and Z_i must be non-NULL");
    AttnLayout L;
    tp_status st = validate_attn_call(batch, seq, hidden, n_heads, n_kv_heads, n_shards, rank, dt,
                                      workspace, workspace_bytes, &L);
    if (st != TP_OK) return st;
    if (!aligned16(X) || !aligned16(Wqkv_i) || !aligned16(Wo_i) || !aligned16(Z_i) ||
        (bqkv_i && !aligned16(bqkv_i)))
        return fail(TP_ERR_ALIGN, "every pointer must be 16-byte aligned");
    st = check_device();
    if (st != TP_OK) return st;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* ws = reinterpret_cast<char*>(workspace);
    // 1. Column-parallel QKV projection of the local heads, scattered per head (V transposed).
    st = launch_qkv(X, Wqkv_i, bqkv_i, batch, seq, hidden, L, ws, s);
    if (st != TP_OK) return st;
    // 2. Head-local attention; heads concatenated locally into O_i.
    st = launch_heads(batch, seq, causal, L, ws, s);
    if (st != TP_OK) return st;
    // 3. Row-parallel output projection: Z_i = O_i W_O,i (fp32 partial).
    const int T = (int)(batch * seq);
    const int w = L.hl * L.d;
    tps::GemmProblem g3{};
    g3.A = ws + L.o; g3.lda = w;
    g3.B = Wo_i; g3.ldb = w;
    g3.C = Z_i; g3.ldc = hidden;
    g3.M = T; g3.N = (int)hidden; g3.K = w;
    return hip_status(tps::gemm_bf16(g3, tps::Epi::F32, s), "output projection launch");
}

tp_status tp_reduce_scatter_partials(const float* const* Z_parts, int n_parts, int64_t batch,
                                     int64_t seq, int64_t hidden, int rank, void* H_r,
                                     tp_dtype out_dt, void* stream)
{
    tp_status st = validate_sp(n_parts, batch, seq, hidden, rank, out_dt, INT32_MAX);
    if (st != TP_OK) return st;
    st = check_parts(reinterpret_cast<const void* const*>(Z_parts), n_parts, "partial");
    if (st != TP_OK) return st;
    if (!H_r) return fail(TP_ERR_NULL, "H_r must be non-NULL");
    if (!aligned16(H_r)) return fail(TP_ERR_ALIGN, "H_r is not 16-byte aligned");
    st = check_no_overlap(reinterpret_cast<const void* const*>(Z_parts), n_parts,
                          (size_t)(batch * seq * hidden) * 4, H_r,
                          (size_t)(batch * (seq / n_parts) * hidden) * dt_size(out_dt), "H_r");
    if (st != TP_OK) return st;
    st = check_device();
    if (st != TP_OK) return st;
    tps::SpProblem p{};
    p.parts = Z_parts; p.n_parts = n_parts;
    p.hout = H_r;
    p.batch = (int)batch; p.seq = (int)seq; p.rank = rank; p.hidden = (int)hidden;
    p.bf16 = out_dt == TP_BF16;
    return hip_status(tps::sp_boundary(p, reinterpret_cast<hipStream_t>(stream)),
                      "reduce-scatter kernel launch");
}

tp_status tp_sp_residual_layernorm_fwd(const float* const* Z_parts, int n_parts,
                                       const void* residual_r, const float* gamma,
                                       const float* beta, float eps, void* H_r, void* Y_r,
                                       int64_t batch, int64_t seq, int64_t hidden, int rank,
                                       tp_dtype dt, void* stream)
{
    tp_status st = validate_sp(n_parts, batch, seq, hidden, rank, dt, 16384);   // row in LDS
    if (st != TP_OK) return st;
    st = check_parts(reinterpret_cast<const void* const*>(Z_parts), n_parts, "partial");
    if (st != TP_OK) return st;
    if (!gamma || !beta || !H_r || !Y_r)
        return fail(TP_ERR_NULL, "gamma, beta, H_r and Y_r must be non-NULL");
    if (!aligned16(gamma) || !aligned16(beta) || !aligned16(H_r) || !aligned16(Y_r) ||
        (residual_r && !aligned16(residual_r)))
        return fail(TP_ERR_ALIGN, "every pointer must be 16-byte aligned");
    if (!(eps >= 0.0f) || eps > 1e30f) return fail(TP_ERR_SHAPE, "eps must be finite and >= 0");
    {
        const size_t pb = (size_t)(batch * seq * hidden) * 4;
        const size_t ob = (size_t)(batch * (seq / n_parts) * hidden) * dt_size(dt);
        st = check_no_overlap(reinterpret_cast<const void* const*>(Z_parts), n_parts, pb, H_r, ob, "H_r");
        if (st == TP_OK)
            st = check_no_overlap(reinterpret_cast<const void* const*>(Z_parts), n_parts, pb, Y_r, ob, "Y_r");
        if (st == TP_OK && overlap(H_r, ob, Y_r, ob))
            st = fail(TP_ERR_ALIAS, "H_r and Y_r overlap");
        if (st == TP_OK && residual_r && overlap(residual_r, ob, Y_r, ob))
            st = fail(TP_ERR_ALIAS, "residual_r and Y_r overlap");
        // each lane reads its residual vector before writing the same vector of H_r
        if (st == TP_OK && residual_r && residual_r != H_r && overlap(residual_r, ob, H_r, ob))
            st = fail(TP_ERR_ALIAS, "residual_r overlaps H_r without being H_r");
        if (st != TP_OK) return st;
    }
    st = check_device();
    if (st != TP_OK) return st;
    tps::SpProblem p{};
    p.parts = Z_parts; p.n_parts = n_parts;
    p.resid = residual_r; p.gamma = gamma; p.beta = beta; p.eps = eps;
    p.hout = H_r; p.yout = Y_r;
    p.batch = (int)batch; p.seq = (int)seq; p.rank = rank; p.hidden = (int)hidden;
    p.bf16 = dt == TP_BF16;
    return hip_status(tps::sp_boundary(p, reinterpret_cast<hipStream_t>(stream)),
                      "sequence-parallel boundary kernel launch");
}

tp_status tp_all_gather_rows(const void* const* slices, int n_parts, int64_t batch, int64_t seq,
                             int64_t hidden, void* X, tp_dtype dt, void* stream)
{
    tp_status st = validate_sp(n_parts, batch, seq, hidden, 0, dt, INT32_MAX);
    if (st != TP_OK) return st;
    st = check_parts(slices, n_parts, "slice");
    if (st != TP_OK) return st;
    if (!X) return fail(TP_ERR_NULL, "X must be non-NULL");
    if (!aligned16(X)) return fail(TP_ERR_ALIGN, "X is not 16-byte aligned");
    st = check_no_overlap(slices, n_parts, (size_t)(batch * (seq / n_parts) * hidden) * dt_size(dt),
                          X, (size_t)(batch * seq * hidden) * dt_size(dt), "X");
    if (st != TP_OK) return st;
    st = check_device();
    if (st != TP_OK) return st;
    return hip_status(tps::all_gather_rows(slices, n_parts, (int)batch, (int)seq,
                                           hidden * (int64_t)dt_size(dt), X,
                                           reinterpret_cast<hipStream_t>(stream)),
                      "all-gather kernel launch");
}

tp_status tp_gemm_tile_info(int64_t M, int64_t N, int64_t K, int* tile_m, int* tile_n, int* waves)
{
    if (!tile_m || !tile_n || !waves) return fail(TP_ERR_NULL, "output pointers must be non-NULL");
    if (M < 1 || N < 1 || K < 1 || M > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
        return fail(TP_ERR_SHAPE, "M, N, K must be in [1, 2^31-1]");
    const tps::GemmTile t = tps::gemm_bf16_launch_tile((int)M, (int)N, (int)K, waves);
    *tile_m = t.bm;
    *tile_n = t.bn;
    return ok();
}

tp_status tp_row_parallel_sum_tile_info(int64_t rows, int64_t out_features, int64_t k_local,
                                         int n_parts, tp_dtype out_dt, int* tile_m, int* tile_n,
                                         int* waves, int* form)
{
    if (!tile_m || !tile_n || !waves || !form)
        return fail(TP_ERR_NULL, "output pointers must be non-NULL");
    if (rows < 1 || out_features < 1 || k_local < 1 || rows > INT32_MAX ||
        out_features > INT32_MAX || k_local > INT32_MAX)
        return fail(TP_ERR_SHAPE, "rows, out_features, k_local must be in [1, 2^31-1]");
    if (n_parts < 1 || n_parts > tps::kMaxSumParts)
        return fail(TP_ERR_SHAPE, "n_parts=%d outside [1, %d]", n_parts, tps::kMaxSumParts);
    if (out_dt != TP_F32 && out_dt != TP_BF16)
        return fail(TP_ERR_DTYPE, "out_dt %d not supported", (int)out_dt);
    const tps::GemmTile t = tps::gemm_bf16_sum_launch_tile(
        (int)rows, (int)out_features, (int)k_local, n_parts, out_dt == TP_BF16, waves, form);
    *tile_m = t.bm;
    *tile_n = t.bn;
    return ok();
}

tp_status tp_sum_partials(const float* const* Z_parts, int n_parts, int64_t numel, void* Z,
                          tp_dtype out_dt, void* stream)
{
    if (!Z_parts || !Z) return fail(TP_ERR_NULL, "Z_parts and Z must be non-NULL");
    if (n_parts < 1 || n_parts > 64)
        return fail(TP_ERR_SHAPE, "n_parts=%d outside [1, 64]", n_parts);
    if (numel < 1) return fail(TP_ERR_SHAPE, "numel=%lld must be >= 1", (long long)numel);
    if (out_dt != TP_F32 && out_dt != TP_BF16)
        return fail(TP_ERR_DTYPE, "out_dt %d not supported", (int)out_dt);
    for (int r = 0; r < n_parts; ++r) {
        if (!Z_parts[r]) return fail(TP_ERR_NULL, "partial %d is NULL (missing rank)", r);
        if (!aligned16(Z_parts[r])) return fail(TP_ERR_ALIGN, "partial %d is not 16-byte aligned", r);
    }
    if (!aligned16(Z)) return fail(TP_ERR_ALIGN, "Z is not 16-byte aligned");
    // Each lane reads element vector i of every partial and then writes vector i of Z, so an
    // fp32 Z may be exactly one of the partials; a bf16 Z (half the row pitch) or any other
    // overlap would let one lane overwrite inputs another lane has not read yet.
    const size_t pbytes = (size_t)numel * 4, zbytes = (size_t)numel * dt_size(out_dt);
    for (int r = 0; r < n_parts; ++r) {
        const bool same = out_dt == TP_F32 && static_cast<const void*>(Z_parts[r]) == Z;
        if (!same && overlap(Z, zbytes, Z_parts[r], pbytes))
            return fail(TP_ERR_ALIAS, "Z overlaps partial %d (only an fp32 Z may be a partial itself)", r);
    }
    tp_status st = check_device();
    if (st != TP_OK) return st;
    hipError_t e = tps::sum_partials(Z_parts, n_parts, numel, Z, out_dt == TP_BF16,
                                     reinterpret_cast<hipStream_t>(stream));
    return hip_status(e, "sum kernel launch");
}

}  // extern "C"
