// C-ABI layer of libw8a8moe: argument checks, workspace layout and the launch
// sequence of the MoE layer.  No allocation, no host synchronisation; every
// kernel goes onto the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "internal.h"
#include "w8a8moe.h"

namespace {

thread_local std::string g_last_error;

w8a8_status fail(w8a8_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

w8a8_status check_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return W8A8_OK;
    return fail(W8A8_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// [p, p + np) and [q, q + nq) share a byte
bool overlap(const void* p, size_t np, const void* q, size_t nq) {
    const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
    return a < b + nq && b < a + np;
}

int64_t max_m_tiles(int64_t rows, int64_t groups, int64_t bm) {
    // sum over groups of ceil(count/bm) <= (rows + groups*(bm-1)) / bm, and <= rows
    const int64_t bound = (rows + groups * (bm - 1)) / bm;
    return bound < rows ? bound : rows;
}

// m-tile height of the grouped GEMMs: few rows per expert (decode) go to the
// register-fed skinny kernel, which streams the weights once (16-row blocks);
// otherwise the LDS-tiled MFMA kernel (256-row tiles)
int moe_bm(int64_t A, int64_t E) { return A <= 4 * E ? w8a8::SKINNY_BM : w8a8::GEMM_BM; }

struct MoePlan {
    w8a8_moe_workspace_layout lay;
    size_t partial, wplanes, rank, chunk_counts, chunk_base, mt_prefix, mt_info, tile_ctr, xcd_bounds;
    int splits, nchunks;
    bool has_planes;
};

w8a8_status check_moe_shape(const w8a8_moe_shape* sh) {
    if (!sh) return fail(W8A8_ERR_INVALID_ARGUMENT, "shape is NULL");
    if (sh->T < 0 || sh->H < 0 || sh->E < 0 || sh->top_k < 0 || sh->I < 0)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "negative size in shape");
    if (sh->H % 128 != 0 || sh->H < 128 || sh->H > 16384)
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "H=%lld: need H %% 128 == 0 and 128 <= H <= 16384",
                    (long long)sh->H);
    if (sh->I % 128 != 0 || sh->I < 128 || sh->I > 16384)
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "I=%lld: need I %% 128 == 0 and 128 <= I <= 16384",
                    (long long)sh->I);
    if (sh->E < 1 || sh->E > w8a8::MAX_EXPERTS)
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "E=%lld: need 1 <= E <= 256", (long long)sh->E);
    if (sh->top_k < 1 || sh->top_k > sh->E || sh->top_k > w8a8::MAX_TOPK)
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "top_k=%lld: need 1 <= top_k <= min(E, 8)",
                    (long long)sh->top_k);
    // T first: T * top_k of an unchecked T could overflow
    if (sh->T > (int64_t(1) << 24) || sh->T * sh->top_k > (int64_t(1) << 24))
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "T*top_k=%lld exceeds 2^24",
                    (long long)(sh->T * sh->top_k));
    return W8A8_OK;
}

MoePlan plan_moe(const w8a8_moe_shape* sh) {
    MoePlan p{};
    const int64_t T = sh->T, H = sh->H, E = sh->E, k = sh->top_k, I = sh->I, A = T * k;
    const w8a8::RouterPlan rp = T > 0 ? w8a8::router_plan((int)T, (int)E, (int)H) : w8a8::RouterPlan{1, 0};
    p.splits = rp.splits;
    p.nchunks = (int)((T + w8a8::ROUTE_CHUNK - 1) / w8a8::ROUTE_CHUNK);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    w8a8_moe_workspace_layout& L = p.lay;
    L.x_q = take(T * H);
    L.x_scale = take(T * 4);
    L.logits = take(T * E * 4);
    L.topk_ids = take(A * 4);
    L.topk_w = take(A * 4);
    L.expert_counts = take(E * 4);
    L.expert_offsets = take((E + 1) * 4);
    L.sorted_assign = take(A * 4);
    L.h = take(A * I * 4);
    L.h_q = take(A * I);
    L.h_scale = take(A * 4);
    L.o = take(A * H * 4);
    L.internal = off;
    p.partial = take((size_t)p.splits * T * E * 4);
    p.wplanes = rp.planes_bytes ? take(rp.planes_bytes) : 0;
    p.has_planes = rp.planes_bytes > 0;
    p.rank = take(A * 4);
    p.chunk_counts = take((size_t)E * p.nchunks * 4);
    p.chunk_base = take((size_t)E * p.nchunks * 4);
    p.mt_prefix = take((E + 1) * 4);
    p.mt_info = take((size_t)max_m_tiles(A, E, moe_bm(A, E)) * sizeof(w8a8::MtInfo));
    p.tile_ctr = take((size_t)w8a8::TILE_CTR_COUNT * w8a8::TILE_CTR_STRIDE * 4);
    p.xcd_bounds = take(2 * 9 * 4);
    L.total_bytes = off;
    return p;
}

}  // namespace

extern "C" {

const char* w8a8_status_string(int status) {
    switch (status) {
        case W8A8_OK: return "W8A8_OK";
        case W8A8_ERR_INVALID_ARGUMENT: return "W8A8_ERR_INVALID_ARGUMENT";
        case W8A8_ERR_UNSUPPORTED_SHAPE: return "W8A8_ERR_UNSUPPORTED_SHAPE";
        case W8A8_ERR_WORKSPACE_TOO_SMALL: return "W8A8_ERR_WORKSPACE_TOO_SMALL";
        case W8A8_ERR_MISALIGNED: return "W8A8_ERR_MISALIGNED";
        case W8A8_ERR_HIP: return "W8A8_ERR_HIP";
        default: return "W8A8_UNKNOWN_STATUS";
    }
}

const char* w8a8_last_error(void) { return g_last_error.c_str(); }

int w8a8_abi_version(void) { return 4; }

// The activation-scale options: mode and bound (clip > 0 and finite for the
// clipped and static modes; ignored for the dynamic one).
static w8a8_status check_scale_opts(int mode, float clip, const float* col_mul) {
    if (mode != W8A8_SCALE_DYNAMIC && mode != W8A8_SCALE_CLIPPED && mode != W8A8_SCALE_STATIC)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "unknown scale mode %d", mode);
    if (mode != W8A8_SCALE_DYNAMIC && !(clip > 0.0f && clip <= 3.4e38f))
        return fail(W8A8_ERR_INVALID_ARGUMENT, "clip must be positive and finite for scale mode %d", mode);
    if (col_mul && !aligned(col_mul, 4)) return fail(W8A8_ERR_MISALIGNED, "col_mul not 4-byte aligned");
    return W8A8_OK;
}

static w8a8_status quantize_rows_code(const float* x, int64_t rows, int64_t cols, int64_t ld, int8_t* q,
                                      float* scale, int code, w8a8_stream stream,
                                      const w8a8::QuantOpts& opt = w8a8::QuantOpts{}) {
    if (rows < 0 || cols < 0 || ld < 0) return fail(W8A8_ERR_INVALID_ARGUMENT, "negative size");
    if (cols < 1 || cols > (int64_t(1) << 24))
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "cols=%lld: need 1 <= cols <= 2^24", (long long)cols);
    if (ld < cols) return fail(W8A8_ERR_INVALID_ARGUMENT, "ld=%lld < cols=%lld", (long long)ld,
                               (long long)cols);
    // the long-row kernel runs one workgroup per row: 2^24 rows of 256 threads
    // is the 32-bit work-item count of a launch
    if (rows > (int64_t(1) << 24))
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "rows=%lld: need rows <= 2^24", (long long)rows);
    if (rows == 0) return W8A8_OK;
    if (!x || !q || !scale) return fail(W8A8_ERR_INVALID_ARGUMENT, "NULL pointer");
    if (!aligned(x, 4) || !aligned(scale, 4)) return fail(W8A8_ERR_MISALIGNED, "x/scale not 4-byte aligned");
    return check_hip(w8a8::launch_quantize_rows(x, rows, cols, ld, q, scale, code, (hipStream_t)stream, opt),
                     "quantize_rows launch");
}

w8a8_status w8a8_quantize_rows(const float* x, int64_t rows, int64_t cols, int64_t ld, int8_t* q,
                               float* scale, w8a8_stream stream) {
    return quantize_rows_code(x, rows, cols, ld, q, scale, w8a8::CODE_INT8, stream);
}

w8a8_status w8a8_quantize_rows_fp8(const float* x, int64_t rows, int64_t cols, int64_t ld, uint8_t* q,
                                   float* scale, w8a8_stream stream) {
    return quantize_rows_code(x, rows, cols, ld, (int8_t*)q, scale, w8a8::CODE_FP8, stream);
}

w8a8_status w8a8_quantize_rows_ex(const float* x, int64_t rows, int64_t cols, int64_t ld,
                                  const float* col_mul, int32_t scale_mode, float clip, int32_t code,
                                  void* q, float* scale, w8a8_stream stream) {
    const bool recip = (scale_mode & W8A8_SCALE_COL_RECIPROCAL) != 0;
    if (recip && !col_mul)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "W8A8_SCALE_COL_RECIPROCAL needs col_mul");
    scale_mode &= ~W8A8_SCALE_COL_RECIPROCAL;
    w8a8_status st = check_scale_opts(scale_mode, clip, col_mul);
    if (st != W8A8_OK) return st;
    if (code != W8A8_CODE_INT8 && code != W8A8_CODE_FP8_E4M3 && code != W8A8_CODE_FP8_E4M3_FAST)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "unknown code %d", (int)code);
    w8a8::QuantOpts opt;
    opt.col_mul = col_mul;
    opt.mode = scale_mode;
    opt.clip = clip;
    opt.col_recip = recip;
    // both FP8 codes store the same E4M3 values
    return quantize_rows_code(x, rows, cols, ld, (int8_t*)q, scale,
                              code == W8A8_CODE_INT8 ? w8a8::CODE_INT8 : w8a8::CODE_FP8, stream, opt);
}

w8a8_status w8a8_pack_weights_size(int64_t groups, int64_t n, int64_t k, int kind, size_t* bytes) {
    if (!bytes) return fail(W8A8_ERR_INVALID_ARGUMENT, "bytes is NULL");
    if (kind != W8A8_PACK_PLAIN && kind != W8A8_PACK_GATE_UP)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "unknown pack kind %d", kind);
    if (groups < 1 || n < 1 || k < 1) return fail(W8A8_ERR_INVALID_ARGUMENT, "sizes must be >= 1");
    if (k % 64 != 0) return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "k=%lld: need k %% 64 == 0", (long long)k);
    if (kind == W8A8_PACK_PLAIN && n % 16 != 0)
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "n=%lld: need n %% 16 == 0", (long long)n);
    if (kind == W8A8_PACK_GATE_UP && (n % 32 != 0))
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "gate-up n=%lld: need n %% 32 == 0", (long long)n);
    *bytes = (size_t)groups * (size_t)n * (size_t)k;
    return W8A8_OK;
}

w8a8_status w8a8_pack_weights(const int8_t* w, int64_t groups, int64_t n, int64_t k, int kind,
                              int8_t* packed, w8a8_stream stream) {
    size_t bytes;
    w8a8_status st = w8a8_pack_weights_size(groups, n, k, kind, &bytes);
    if (st != W8A8_OK) return st;
    if (!w || !packed) return fail(W8A8_ERR_INVALID_ARGUMENT, "NULL pointer");
    if (!aligned(w, 16) || !aligned(packed, 16))
        return fail(W8A8_ERR_MISALIGNED, "weights must be 16-byte aligned");
    if (w == packed) return fail(W8A8_ERR_INVALID_ARGUMENT, "packing cannot be in place");
    return check_hip(w8a8::launch_pack_weights(w, groups, n, k, kind, packed, (hipStream_t)stream),
                     "pack_weights launch");
}

static w8a8_status dense_gemm(int epi, int code, const int8_t* a_q, const float* s_a,
                              const int8_t* b_packed, const float* s_b, int64_t M, int64_t N,
                              int64_t K, float* out, int32_t* out_i32, w8a8_stream stream) {
    if (M < 0 || N < 0 || K < 0) return fail(W8A8_ERR_INVALID_ARGUMENT, "negative size");
    if (N % 128 != 0 || N < 128 || N > (int64_t(1) << 24))
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "N=%lld: need N %% 128 == 0, N >= 128", (long long)N);
    if (K % 128 != 0 || K < 128 || K > (int64_t(1) << 17))
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "K=%lld: need K %% 128 == 0, 128 <= K <= 2^17",
                    (long long)K);
    if (M > (int64_t(1) << 24)) return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "M too large");
    if (M == 0) return W8A8_OK;
    if (!a_q || !b_packed || (epi == w8a8::EPI_DENSE_F32 && (!s_a || !s_b || !out)) ||
        (epi == w8a8::EPI_DENSE_I32 && !out_i32))
        return fail(W8A8_ERR_INVALID_ARGUMENT, "NULL pointer");
    if (!aligned(a_q, 16) || !aligned(b_packed, 16))
        return fail(W8A8_ERR_MISALIGNED, "operands must be 16-byte aligned");
    w8a8::GemmParams p{};
    p.A = a_q;
    p.B = b_packed;
    p.b_group_bytes = N * K;
    p.M = M;
    p.N = (int)N;
    p.K = (int)K;
    p.G = 1;
    p.s_a = s_a;
    p.s_b = s_b;
    p.out_f32 = out;
    p.out_i32 = out_i32;
    p.a_rows = M;
    p.code = code;
    const int64_t mt = (M + w8a8::GEMM_BM - 1) / w8a8::GEMM_BM;
    return check_hip(w8a8::launch_gemm(epi, p, mt, (hipStream_t)stream), "gemm launch");
}

w8a8_status w8a8_gemm(const int8_t* a_q, const float* s_a, const int8_t* b_packed, const float* s_b,
                      int64_t M, int64_t N, int64_t K, float* out, w8a8_stream stream) {
    return dense_gemm(w8a8::EPI_DENSE_F32, w8a8::CODE_INT8, a_q, s_a, b_packed, s_b, M, N, K, out,
                      nullptr, stream);
}

w8a8_status w8a8_gemm_fp8(const uint8_t* a_q, const float* s_a, const uint8_t* b_packed, const float* s_b,
                          int64_t M, int64_t N, int64_t K, float* out, w8a8_stream stream) {
    return dense_gemm(w8a8::EPI_DENSE_F32, w8a8::CODE_FP8, (const int8_t*)a_q, s_a, (const int8_t*)b_packed,
                      s_b, M, N, K, out, nullptr, stream);
}

w8a8_status w8a8_gemm_fp8_fast(const uint8_t* a_q, const float* s_a, const uint8_t* b_packed,
                               const float* s_b, int64_t M, int64_t N, int64_t K, float* out,
                               w8a8_stream stream) {
    return dense_gemm(w8a8::EPI_DENSE_F32, w8a8::CODE_FP8_FAST, (const int8_t*)a_q, s_a,
                      (const int8_t*)b_packed, s_b, M, N, K, out, nullptr, stream);
}

w8a8_status w8a8_gemm_i32(const int8_t* a_q, const int8_t* b_packed, int64_t M, int64_t N,
                          int64_t K, int32_t* acc, w8a8_stream stream) {
    return dense_gemm(w8a8::EPI_DENSE_I32, w8a8::CODE_INT8, a_q, nullptr, b_packed, nullptr, M, N, K,
                      nullptr, acc, stream);
}

// The argument checks of the layer entry points (after the shape check, for
// T > 0): pointers, alignment, weight code and scale options, workspace size,
// and that x, y and the workspace do not overlap.  On success *plan, *code and
// *x_opt describe the call.
static w8a8_status check_forward(const w8a8_moe_shape* shape, const w8a8_moe_weights* wts, const float* x,
                                 const float* y, const void* workspace, size_t workspace_bytes,
                                 MoePlan* plan_out, int* code_out, w8a8::QuantOpts* x_opt_out) {
    w8a8_status st;
    if (!wts || !x || !y || !workspace || !wts->router_w || !wts->w_gate_up || !wts->s_gate_up ||
        !wts->w_down || !wts->s_down)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "NULL pointer");
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(wts->router_w, 16) ||
        !aligned(wts->w_gate_up, 16) || !aligned(wts->w_down, 16) || !aligned(wts->s_gate_up, 4) ||
        !aligned(wts->s_down, 4) || (wts->router_b && !aligned(wts->router_b, 4)))
        return fail(W8A8_ERR_MISALIGNED, "x, y, router_w and weights must be 16-byte aligned");
    if (!aligned(workspace, 256)) return fail(W8A8_ERR_MISALIGNED, "workspace must be 256-byte aligned");
    if (wts->code != W8A8_CODE_INT8 && wts->code != W8A8_CODE_FP8_E4M3 &&
        wts->code != W8A8_CODE_FP8_E4M3_FAST)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "unknown weight code %d", (int)wts->code);
    const int code = wts->code == W8A8_CODE_FP8_E4M3       ? w8a8::CODE_FP8
                     : wts->code == W8A8_CODE_FP8_E4M3_FAST ? w8a8::CODE_FP8_FAST
                                                            : w8a8::CODE_INT8;
    if ((st = check_scale_opts(wts->x_scale_mode, wts->x_clip, wts->x_smooth)) != W8A8_OK) return st;
    if (wts->x_smooth && !aligned(wts->x_smooth, 16))
        return fail(W8A8_ERR_MISALIGNED, "x_smooth must be 16-byte aligned");
    w8a8::QuantOpts x_opt;
    x_opt.col_mul = wts->x_smooth;
    x_opt.mode = wts->x_scale_mode;
    x_opt.clip = wts->x_clip;
    const MoePlan plan = plan_moe(shape);
    if (workspace_bytes < plan.lay.total_bytes)
        return fail(W8A8_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < required %zu", workspace_bytes,
                    plan.lay.total_bytes);
    // x is read while the workspace is written, and y is written while o (in
    // the workspace) is read: none of the three may share memory
    const size_t xy_bytes = (size_t)shape->T * (size_t)shape->H * 4;
    if (overlap(x, xy_bytes, y, xy_bytes)) return fail(W8A8_ERR_INVALID_ARGUMENT, "y must not overlap x");
    if (overlap(x, xy_bytes, workspace, plan.lay.total_bytes) ||
        overlap(y, xy_bytes, workspace, plan.lay.total_bytes))
        return fail(W8A8_ERR_INVALID_ARGUMENT, "x and y must not overlap the workspace");
    *plan_out = plan;
    *code_out = code;
    *x_opt_out = x_opt;
    return W8A8_OK;
}

w8a8_status w8a8_moe_workspace_query(const w8a8_moe_shape* shape, w8a8_moe_workspace_layout* layout) {
    if (!layout) return fail(W8A8_ERR_INVALID_ARGUMENT, "layout is NULL");
    w8a8_status st = check_moe_shape(shape);
    if (st != W8A8_OK) return st;
    *layout = plan_moe(shape).lay;
    return W8A8_OK;
}

w8a8_status w8a8_moe_forward(const w8a8_moe_shape* shape, const w8a8_moe_weights* wts,
                             const float* x, float* y, void* workspace, size_t workspace_bytes,
                             w8a8_stream stream) {
    return w8a8_moe_forward_events(shape, wts, x, y, workspace, workspace_bytes, nullptr, stream);
}

w8a8_status w8a8_moe_forward_events(const w8a8_moe_shape* shape, const w8a8_moe_weights* wts,
                                    const float* x, float* y, void* workspace,
                                    size_t workspace_bytes, void* const* events,
                                    w8a8_stream stream) {
    w8a8_status st = check_moe_shape(shape);
    if (st != W8A8_OK) return st;
    if (shape->T == 0) return W8A8_OK;
    MoePlan plan;
    int code;
    w8a8::QuantOpts x_opt;
    if ((st = check_forward(shape, wts, x, y, workspace, workspace_bytes, &plan, &code, &x_opt)) != W8A8_OK)
        return st;

    const int T = (int)shape->T, H = (int)shape->H, E = (int)shape->E, k = (int)shape->top_k,
              I = (int)shape->I;
    const int64_t A = (int64_t)T * k;
    const int bm = moe_bm(A, E);
    const bool skinny = bm == w8a8::SKINNY_BM;
    hipStream_t s = (hipStream_t)stream;
    char* ws = (char*)workspace;
    const w8a8_moe_workspace_layout& L = plan.lay;
    int8_t* x_q = (int8_t*)(ws + L.x_q);
    float* x_scale = (float*)(ws + L.x_scale);
    float* topk_w = (float*)(ws + L.topk_w);
    int32_t* offsets = (int32_t*)(ws + L.expert_offsets);
    int32_t* sorted = (int32_t*)(ws + L.sorted_assign);
    float* h = (float*)(ws + L.h);
    int8_t* h_q = (int8_t*)(ws + L.h_q);
    float* h_scale = (float*)(ws + L.h_scale);
    float* o = (float*)(ws + L.o);
    int32_t* mt_prefix = (int32_t*)(ws + plan.mt_prefix);
    int32_t* mt_info = (int32_t*)(ws + plan.mt_info);
    int32_t* tile_ctr = (int32_t*)(ws + plan.tile_ctr);

    auto mark = [&](int i) -> w8a8_status {
        if (!events || !events[i]) return W8A8_OK;
        return check_hip(hipEventRecord((hipEvent_t)events[i], s), "hipEventRecord");
    };

    // 1. per-token quantisation: its own launch, or (few tokens, router
    //    without weight planes) extra workgroups of the router's launch, which
    //    reads the same x; the "quant" stage is then empty
    const bool xq_in_route = !plan.has_planes && T <= w8a8::ROUTER_XQUANT_MAX_T;
    if ((st = mark(0)) != W8A8_OK) return st;
    if (!xq_in_route) {
        st = check_hip(w8a8::launch_quantize_rows(x, T, H, H, x_q, x_scale, code, s, x_opt), "quantize x");
        if (st != W8A8_OK) return st;
    }

    // 2-4. router, top-k, permutation
    const int ntv_gu = (int)(2 * I / w8a8::gemm_tile_n(2 * I, code));
    const int ntv_dn = (int)(H / w8a8::gemm_tile_n(H, code));
    w8a8::RouteInputs ri{x, wts->router_w, wts->router_b, T, H, E, k, plan.splits, bm, ntv_gu, ntv_dn, {}};
    if (xq_in_route) {
        ri.xq.q = x_q;
        ri.xq.scale = x_scale;
        ri.xq.opt = x_opt;
        ri.xq.code = code;
    }
    w8a8::RouteBuffers rb{};
    rb.partial = (float*)(ws + plan.partial);
    rb.wplanes = plan.has_planes ? (void*)(ws + plan.wplanes) : nullptr;
    rb.logits = (float*)(ws + L.logits);
    rb.topk_ids = (int32_t*)(ws + L.topk_ids);
    rb.topk_w = topk_w;
    rb.chunk_counts = (int32_t*)(ws + plan.chunk_counts);
    rb.chunk_base = (int32_t*)(ws + plan.chunk_base);
    rb.rank = (int32_t*)(ws + plan.rank);
    rb.expert_counts = (int32_t*)(ws + L.expert_counts);
    rb.expert_offsets = offsets;
    rb.mt_prefix = mt_prefix;
    rb.mt_info = mt_info;
    rb.tile_ctr = tile_ctr;
    rb.sorted_assign = sorted;
    rb.xcd_bounds = (int32_t*)(ws + plan.xcd_bounds);
    if ((st = mark(1)) != W8A8_OK) return st;
    st = check_hip(w8a8::launch_route(ri, rb, s), "route");
    if (st != W8A8_OK) return st;

    // 5. grouped gate-up GEMM, epilogue dequant + SiLU*up -> h (fp32)
    w8a8::GemmParams gu{};
    gu.A = x_q;
    gu.B = wts->w_gate_up;
    gu.b_group_bytes = (int64_t)2 * I * H;
    gu.M = A;
    gu.N = 2 * I;
    gu.K = H;
    gu.seg_offsets = offsets;
    gu.mt_prefix = mt_prefix;
    gu.mt_info = mt_info;
    gu.tile_ctr = skinny ? nullptr : tile_ctr;
    gu.xcd_bounds = rb.xcd_bounds;
    gu.G = E;
    gu.sorted_assign = sorted;
    gu.topk = k;
    gu.s_a = x_scale;
    gu.s_b = wts->s_gate_up;
    gu.out_f32 = h;
    gu.I = I;
    gu.a_rows = T;
    gu.code = code;
    if ((st = mark(2)) != W8A8_OK) return st;
    st = check_hip(skinny ? w8a8::launch_gemm_skinny(w8a8::EPI_GATE_UP, gu, max_m_tiles(A, E, bm), s)
                          : w8a8::launch_gemm(w8a8::EPI_GATE_UP, gu, max_m_tiles(A, E, bm), s),
                   "gate-up gemm");
    if (st != W8A8_OK) return st;

    // requantise h per assignment row
    if ((st = mark(3)) != W8A8_OK) return st;
    st = check_hip(w8a8::launch_quantize_rows(h, A, I, I, h_q, h_scale, code, s), "requantize h");
    if (st != W8A8_OK) return st;

    // 6. grouped down GEMM, epilogue dequant * routing weight -> o[t*k+j]
    w8a8::GemmParams dn{};
    dn.A = h_q;
    dn.B = wts->w_down;
    dn.b_group_bytes = (int64_t)H * I;
    dn.M = A;
    dn.N = H;
    dn.K = I;
    dn.seg_offsets = offsets;
    dn.mt_prefix = mt_prefix;
    dn.mt_info = mt_info;
    dn.tile_ctr = skinny ? nullptr : tile_ctr + 8 * w8a8::TILE_CTR_STRIDE;
    dn.xcd_bounds = rb.xcd_bounds + 9;
    dn.G = E;
    dn.sorted_assign = sorted;
    dn.topk = k;
    dn.s_a = h_scale;
    dn.s_b = wts->s_down;
    dn.route_w = topk_w;
    dn.out_f32 = o;
    dn.a_rows = A;
    dn.code = code;
    if ((st = mark(4)) != W8A8_OK) return st;
    st = check_hip(skinny ? w8a8::launch_gemm_skinny(w8a8::EPI_DOWN, dn, max_m_tiles(A, E, bm), s)
                          : w8a8::launch_gemm(w8a8::EPI_DOWN, dn, max_m_tiles(A, E, bm), s),
                   "down gemm");
    if (st != W8A8_OK) return st;

    // 7. combine
    if ((st = mark(5)) != W8A8_OK) return st;
    st = check_hip(w8a8::launch_combine(o, T, k, H, y, s), "combine");
    if (st != W8A8_OK) return st;
    return mark(6);
}

}  // extern "C"

// ---- the layer without a caller workspace ----
// One scratch array per device, allocated with the code object when the
// library is loaded on that device and held until the process ends.  Host
// code never uses the array's name as an address: it looks the device
// address up once per device and passes that to the kernels.
namespace {

static __device__ __align__(256) unsigned char scratch[W8A8_STATIC_WORKSPACE_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[MAX_DEVICES];  // device address of each device's array, set once

w8a8_status scratch_address(void** out) {
    int dev = -1;
    w8a8_status st = check_hip(hipGetDevice(&dev), "hipGetDevice");
    if (st != W8A8_OK) return st;
    if (dev < 0 || dev >= MAX_DEVICES) return fail(W8A8_ERR_HIP, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        st = check_hip(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
        if (st != W8A8_OK) return st;
        if (!p) return fail(W8A8_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return W8A8_OK;
}

}  // namespace

extern "C" {

w8a8_status w8a8_moe_forward_static(const w8a8_moe_shape* shape, const w8a8_moe_weights* wts,
                                    const float* x, float* y, w8a8_stream stream) {
    w8a8_status st = check_moe_shape(shape);
    if (st != W8A8_OK) return st;
    if (shape->T == 0) return W8A8_OK;
    const size_t need = plan_moe(shape).lay.total_bytes;
    if (need > (size_t)W8A8_STATIC_WORKSPACE_BYTES)
        return fail(W8A8_ERR_WORKSPACE_TOO_SMALL,
                    "the layer needs %zu bytes of scratch; the static scratch holds %zu "
                    "(use w8a8_moe_forward with a workspace)",
                    need, (size_t)W8A8_STATIC_WORKSPACE_BYTES);
    void* ws = nullptr;
    if ((st = scratch_address(&ws)) != W8A8_OK) return st;
    return w8a8_moe_forward_events(shape, wts, x, y, ws, (size_t)W8A8_STATIC_WORKSPACE_BYTES, nullptr,
                                   stream);
}

w8a8_status w8a8_moe_gate_up_acc(const w8a8_moe_shape* shape, const w8a8_moe_weights* wts,
                                 const void* workspace, size_t workspace_bytes, int32_t* acc,
                                 w8a8_stream stream) {
    w8a8_status st = check_moe_shape(shape);
    if (st != W8A8_OK) return st;
    if (shape->T == 0) return W8A8_OK;
    if (!wts || !workspace || !acc || !wts->w_gate_up)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "NULL pointer");
    if (wts->code != W8A8_CODE_INT8)
        return fail(W8A8_ERR_INVALID_ARGUMENT, "raw accumulators are int32 for INT8 codes only");
    if (!aligned(wts->w_gate_up, 16) || !aligned(acc, 4))
        return fail(W8A8_ERR_MISALIGNED, "w_gate_up must be 16-byte and acc 4-byte aligned");
    if (!aligned(workspace, 256)) return fail(W8A8_ERR_MISALIGNED, "workspace must be 256-byte aligned");
    const MoePlan plan = plan_moe(shape);
    if (workspace_bytes < plan.lay.total_bytes)
        return fail(W8A8_ERR_WORKSPACE_TOO_SMALL, "workspace %zu < required %zu", workspace_bytes,
                    plan.lay.total_bytes);
    const int T = (int)shape->T, H = (int)shape->H, E = (int)shape->E, k = (int)shape->top_k,
              I = (int)shape->I;
    const int64_t A = (int64_t)T * k;
    if (overlap(acc, (size_t)A * 2 * I * 4, workspace, plan.lay.total_bytes))
        return fail(W8A8_ERR_INVALID_ARGUMENT, "acc must not overlap the workspace");
    const int bm = moe_bm(A, E);
    const char* ws = (const char*)workspace;
    const w8a8_moe_workspace_layout& L = plan.lay;
    w8a8::GemmParams gu{};
    gu.A = (const int8_t*)(ws + L.x_q);
    gu.B = wts->w_gate_up;
    gu.b_group_bytes = (int64_t)2 * I * H;
    gu.M = A;
    gu.N = 2 * I;
    gu.K = H;
    gu.seg_offsets = (const int32_t*)(ws + L.expert_offsets);
    gu.mt_prefix = (const int32_t*)(ws + plan.mt_prefix);
    gu.mt_info = (const int32_t*)(ws + plan.mt_info);
    gu.tile_ctr = nullptr;  // one tile per workgroup (the queues were used by the layer's launch)
    gu.G = E;
    gu.sorted_assign = (const int32_t*)(ws + L.sorted_assign);
    gu.topk = k;
    gu.out_i32 = acc;
    gu.I = I;
    gu.a_rows = T;
    gu.code = w8a8::CODE_INT8;
    hipStream_t s = (hipStream_t)stream;
    return check_hip(bm == w8a8::SKINNY_BM
                         ? w8a8::launch_gemm_skinny(w8a8::EPI_GU_I32, gu, max_m_tiles(A, E, bm), s)
                         : w8a8::launch_gemm(w8a8::EPI_GU_I32, gu, max_m_tiles(A, E, bm), s),
                     "gate-up accumulators");
}

w8a8_status w8a8_moe_forward_fused(const w8a8_moe_shape* shape, const w8a8_moe_weights* wts, const float* x,
                                   float* y, void* workspace, size_t workspace_bytes, w8a8_stream stream) {
    w8a8_status st = check_moe_shape(shape);
    if (st != W8A8_OK) return st;
    if (shape->T == 0) return W8A8_OK;
    if (shape->T > w8a8::FUSED_MAX_T)
        return fail(W8A8_ERR_UNSUPPORTED_SHAPE, "T=%lld: the single-launch layer takes at most %d tokens",
                    (long long)shape->T, w8a8::FUSED_MAX_T);
    MoePlan plan;
    int code;
    w8a8::QuantOpts x_opt;
    if ((st = check_forward(shape, wts, x, y, workspace, workspace_bytes, &plan, &code, &x_opt)) != W8A8_OK)
        return st;
    char* ws = (char*)workspace;
    const w8a8_moe_workspace_layout& L = plan.lay;
    w8a8::FusedParams fp{};
    fp.x = x;
    fp.router_w = wts->router_w;
    fp.router_b = wts->router_b;
    fp.w_gu = wts->w_gate_up;
    fp.s_gu = wts->s_gate_up;
    fp.w_d = wts->w_down;
    fp.s_d = wts->s_down;
    fp.y = y;
    fp.T = (int)shape->T;
    fp.H = (int)shape->H;
    fp.E = (int)shape->E;
    fp.k = (int)shape->top_k;
    fp.I = (int)shape->I;
    fp.x_opt = x_opt;
    fp.x_q = (int8_t*)(ws + L.x_q);
    fp.x_scale = (float*)(ws + L.x_scale);
    fp.logits = (float*)(ws + L.logits);
    fp.topk_ids = (int32_t*)(ws + L.topk_ids);
    fp.topk_w = (float*)(ws + L.topk_w);
    fp.expert_counts = (int32_t*)(ws + L.expert_counts);
    fp.expert_offsets = (int32_t*)(ws + L.expert_offsets);
    fp.sorted_assign = (int32_t*)(ws + L.sorted_assign);
    fp.h = (float*)(ws + L.h);
    fp.h_q = (int8_t*)(ws + L.h_q);
    fp.h_scale = (float*)(ws + L.h_scale);
    fp.o = (float*)(ws + L.o);
    fp.sync = (int32_t*)(ws + plan.tile_ctr);  // the tile queues' words, unused by this launch
    return check_hip(w8a8::launch_moe_fused(fp, code, (hipStream_t)stream), "single-launch layer");
}

}  // extern "C"
