/*
 * w8a8moe -- a W8A8 Mixture-of-Experts expert layer for AMD MI355X (gfx950).
 *
 * C ABI.  Plain pointers and sizes only; every device pointer is memory the
 * caller owns (hipMalloc'd or a PyTorch tensor's storage).  The library never
 * allocates, frees or keeps a pointer after a call returns, and it never
 * synchronises the host: every entry point checks its arguments on the host,
 * enqueues its kernels on the caller's stream and returns.  Results are valid
 * once that stream has reached the point of the call.
 *
 * The computation follows these web pages (cited by title and section):
 *  [K100AI]  "W8A8 quantisation of MiniMax-M3 on K100AI: an MoE inference
 *            deployment guide", sec. 2.1 (q = clamp(round(x/s), -128, 127),
 *            per-token activation scales, per-channel weight scales, the
 *            [A,1] x [1,N] scale outer product applied inside the GEMM
 *            epilogue), sec. 2.2 (SmoothQuant factor, percentile-based
 *            activation bounds), sec. 3.1 (batch the small per-expert GEMMs),
 *            sec. 3.2 (pre-planned buffers for the routing reorder).
 *  [HUNYUAN] "Tencent Hunyuan AI Infra: inference optimisation of a
 *            100B-parameter model on Hopper GPUs", sec. 1.3 (FusedMoE:
 *            gate, top-k, index preparation into contiguous per-expert
 *            segments, gate-up GEMM reading the input through the routing
 *            index, expert GEMM, weighted combine).
 *  [DSV4]    "DeepSeek V4 '950' unified FP8 dataflow on H100", sec. 2.1
 *            (E4M3 codes), sec. 2.3
 *            (low-precision inputs, wide accumulator, requantised output),
 *            sec. 2.4 (weight scales per output channel), sec. 3.1 (static
 *            and dynamic parts of the activation scale), sec. 4.1 (router
 *            kept in fp32).
 *
 * Status codes: every entry point returns a w8a8_status.  On an error no
 * kernel has been enqueued (except W8A8_ERR_HIP, which reports a launch
 * failure after earlier kernels of the same call may have been enqueued).
 * w8a8_last_error() returns a thread-local message for the last failure.
 *
 * Thread safety: reentrant.  Calls that may run concurrently on the GPU need
 * distinct workspaces and outputs.
 */
#ifndef W8A8MOE_H
#define W8A8MOE_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define W8A8_API __attribute__((visibility("default")))
#else
#define W8A8_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    W8A8_OK = 0,
    W8A8_ERR_INVALID_ARGUMENT = 1,  /* NULL pointer, negative size, bad enum */
    W8A8_ERR_UNSUPPORTED_SHAPE = 2, /* a size outside the documented limits */
    W8A8_ERR_WORKSPACE_TOO_SMALL = 3,
    W8A8_ERR_MISALIGNED = 4,        /* a pointer or leading dimension not 16-byte aligned */
    W8A8_ERR_HIP = 5                /* the HIP runtime reported an error */
} w8a8_status;

/* A hipStream_t passed as an opaque pointer; NULL is the default stream. */
typedef void* w8a8_stream;

/* Name of a status code (static storage; never NULL). */
W8A8_API const char* w8a8_status_string(int status);

/* Thread-local detail of the last non-OK status returned on this thread. */
W8A8_API const char* w8a8_last_error(void);

/* ABI version of this header: 4. */
W8A8_API int w8a8_abi_version(void);

/* -------------------------------------------------------------------------
 * Per-row dynamic INT8 quantisation.  [K100AI] sec. 2.1.
 *   s[r] = max_c |x[r][c]| / 127          (fp32, IEEE division)
 *   q[r][c] = clamp(rne(x[r][c] / s[r]), -128, 127)   (fp32 quotient,
 *                                                      round half to even)
 * An all-zero row gives s = 0 and q = 0.  Used per token for activations
 * and, offline, per output channel for weights ([DSV4] sec. 2.4).
 *
 * x      device, fp32, rows x cols with leading dimension ld (elements)
 * q      device, int8, rows x cols, dense (leading dimension cols)
 * scale  device, fp32, rows
 * 0 <= rows <= 2^24 (0 is a no-op), 1 <= cols <= 2^24, ld >= cols.
 * Inputs must be finite (NaN/Inf give unspecified codes).
 * ------------------------------------------------------------------------- */
W8A8_API w8a8_status w8a8_quantize_rows(const float* x, int64_t rows, int64_t cols, int64_t ld, int8_t* q,
                               float* scale, w8a8_stream stream);

/* -------------------------------------------------------------------------
 * Codes of the quantised operands.  [DSV4] sec. 2.1 uses FP8 E4M3 (4
 * exponent bits, 3 mantissa bits, range +-448) for the forward weights and
 * activations; sec. 2.3 accumulates fp8 products in fp32.  E4M3 here is the
 * OCP E4M3FN format: sign | exponent (bias 7) | mantissa, exponent 0 for
 * subnormals m * 2^-9, no infinities, S.1111.111 = NaN, largest value 448.
 * ------------------------------------------------------------------------- */
/* W8A8_CODE_FP8_E4M3: E4M3 codes, every product of two codes exact and the
 * products summed in fp32 -- the fp32 accumulator of [DSV4] sec. 2.3 (E4M3
 * values are bf16 values, so the bf16 matrix cores multiply them exactly).
 * W8A8_CODE_FP8_E4M3_FAST: the same codes on the FP8 matrix cores, at twice
 * that rate, but below that contract: inside one instruction the hardware
 * aligns each group of 8 consecutive products to the largest of the group
 * and drops bits below about 2^-13 of it.  Both store identical codes. */
enum { W8A8_CODE_INT8 = 0, W8A8_CODE_FP8_E4M3 = 1, W8A8_CODE_FP8_E4M3_FAST = 2 };

/* Per-row dynamic FP8 quantisation: the scheme of w8a8_quantize_rows with the
 * E4M3 range ([DSV4] sec. 2.1):
 *   s[r] = max_c |x[r][c]| / 448          (fp32, IEEE division)
 *   q[r][c] = E4M3(x[r][c] / s[r])        (fp32 quotient, rounded to the
 *                                          nearest E4M3 value, ties to the
 *                                          even mantissa)
 * An all-zero row gives s = 0 and codes 0x00.  Arguments, limits and errors
 * as for w8a8_quantize_rows; q holds uint8 E4M3 codes. */
W8A8_API w8a8_status w8a8_quantize_rows_fp8(const float* x, int64_t rows, int64_t cols, int64_t ld,
                                            uint8_t* q, float* scale, w8a8_stream stream);

/* Activation-scale options ([K100AI] sec. 2.2: SmoothQuant's per-channel
 * factor, and a high percentile times a safety factor in place of absmax;
 * [DSV4] sec. 3.1: an activation scale with a static part and a dynamic
 * per-token part).  With x'[r][c] = x[r][c] * col_mul[c] (one fp32 product;
 * x' = x when col_mul is NULL) and Q = 127 (INT8) or 448 (E4M3):
 *   W8A8_SCALE_DYNAMIC  s[r] = max_c |x'[r][c]| / Q       (w8a8_quantize_rows)
 *   W8A8_SCALE_CLIPPED  s[r] = min(max_c |x'[r][c]|, clip) / Q
 *   W8A8_SCALE_STATIC   s[r] = clip / Q
 * and the codes of x'/s as in w8a8_quantize_rows / _fp8, saturating where
 * |x'/s| exceeds the range (INT8: clamp to [-128, 127]; E4M3: +-448).  The
 * factor and the bound come from calibration (not done here).  The weights
 * of a smoothed layer take the inverse factor on each input channel, which
 * leaves the product unchanged: quantise their rows with col_mul = the factor
 * and W8A8_SCALE_COL_RECIPROCAL or'ed into scale_mode, so that
 * x'[r][c] = x[r][c] * (1 / col_mul[c]), the reciprocal one IEEE fp32
 * division (round to nearest even) and the product one fp32 multiply. */
enum { W8A8_SCALE_DYNAMIC = 0, W8A8_SCALE_CLIPPED = 1, W8A8_SCALE_STATIC = 2,
       W8A8_SCALE_COL_RECIPROCAL = 0x10 };

/* Per-row quantisation with the options above.  col_mul: NULL or [cols]
 * fp32 device array (4-byte aligned; 16-byte alignment takes the vector
 * path); scale_mode: a W8A8_SCALE_* mode, optionally or'ed with
 * W8A8_SCALE_COL_RECIPROCAL (needs col_mul); clip: positive and finite for the
 * clipped and static modes, ignored for the dynamic one; code:
 * W8A8_CODE_INT8 (q is int8) or either FP8 code (q is uint8 E4M3).  Other
 * arguments, limits and errors as for w8a8_quantize_rows;
 * W8A8_ERR_INVALID_ARGUMENT for an unknown mode or code or a bad clip. */
W8A8_API w8a8_status w8a8_quantize_rows_ex(const float* x, int64_t rows, int64_t cols, int64_t ld,
                                           const float* col_mul, int32_t scale_mode, float clip,
                                           int32_t code, void* q, float* scale, w8a8_stream stream);

/* -------------------------------------------------------------------------
 * Weight packing.  The GEMM kernels read the int8 weight operand in a
 * tiled order: for each group g, each block of 16 output channels nb and
 * each block of 64 reduction elements kb, one contiguous 1 KiB tile.
 *
 * kind W8A8_PACK_PLAIN   : output channels kept in order (dense GEMM and the
 *                          MoE down projection, w[g] = [N][K]).
 * kind W8A8_PACK_GATE_UP : w[g] = [2I][K] with rows 0..I-1 the gate and rows
 *                          I..2I-1 the up projection; packed so each 16-row
 *                          gate block is followed by the up block of the same
 *                          16 channels (the SwiGLU epilogue then holds gate
 *                          and up of one channel side by side).
 *
 * w       device, int8 [groups][n][k], dense
 * packed  device, int8, w8a8_pack_weights_size() bytes (= groups*n*k)
 * Limits: groups, n, k >= 1; k % 64 == 0; PLAIN n % 16 == 0; GATE_UP n % 32
 * (so each half holds whole 16-channel blocks).  An unknown kind is
 * W8A8_ERR_INVALID_ARGUMENT; w and packed must not overlap.
 * ------------------------------------------------------------------------- */
enum { W8A8_PACK_PLAIN = 0, W8A8_PACK_GATE_UP = 1 };

W8A8_API w8a8_status w8a8_pack_weights_size(int64_t groups, int64_t n, int64_t k, int kind, size_t* bytes);
W8A8_API w8a8_status w8a8_pack_weights(const int8_t* w, int64_t groups, int64_t n, int64_t k, int kind,
                              int8_t* packed, w8a8_stream stream);

/* -------------------------------------------------------------------------
 * Dense W8A8 GEMM with the scale outer product in the epilogue.
 * [K100AI] sec. 2.1:  out[m][n] = ((float)acc[m][n] * s_a[m]) * s_b[n],
 *                     acc[m][n] = sum_k a_q[m][k] * b[n][k]   (int32, exact)
 *
 * a_q       device, int8 [M][K] row-major
 * s_a       device, fp32 [M]   (per-token activation scale)
 * b_packed  device, int8, w8a8_pack_weights(b [N][K], groups=1, PLAIN)
 * s_b       device, fp32 [N]   (per-output-channel weight scale)
 * out       device, fp32 [M][N] row-major
 * Limits: M >= 0, N % 128 == 0, K % 128 == 0, 1 <= K <= 2^17 (so the int32
 * accumulator cannot overflow), N, K >= 128.
 * w8a8_gemm_i32 returns the raw int32 accumulators instead (for checking).
 * ------------------------------------------------------------------------- */
W8A8_API w8a8_status w8a8_gemm(const int8_t* a_q, const float* s_a, const int8_t* b_packed, const float* s_b,
                      int64_t M, int64_t N, int64_t K, float* out, w8a8_stream stream);
W8A8_API w8a8_status w8a8_gemm_i32(const int8_t* a_q, const int8_t* b_packed, int64_t M, int64_t N,
                          int64_t K, int32_t* acc, w8a8_stream stream);

/* The same GEMM with FP8 E4M3 codes ([DSV4] sec. 2.3: fp8 inputs, fp32
 * accumulator): acc[m][n] = sum_k E4M3(a_q[m][k]) * E4M3(b[n][k]),
 * out = ((float)acc * s_a[m]) * s_b[n].  Every product is exact; they are
 * summed in fp32 (16 or 32 products per matrix instruction, then the running
 * fp32 accumulator): a chain of at most K/16 + 5 fp32 additions per output, so
 * |acc - exact| <= (K/16 + 5) * 2^-24 * sum_k |a_k b_k| to first order.
 * b_packed is the uint8 codes packed like int8 weights (w8a8_pack_weights
 * moves bytes).  Limits and errors as for w8a8_gemm. */
W8A8_API w8a8_status w8a8_gemm_fp8(const uint8_t* a_q, const float* s_a, const uint8_t* b_packed,
                                   const float* s_b, int64_t M, int64_t N, int64_t K, float* out,
                                   w8a8_stream stream);

/* w8a8_gemm_fp8 on the FP8 matrix cores (W8A8_CODE_FP8_E4M3_FAST): twice the
 * matrix rate, not exact products: inside one instruction each group of 8
 * consecutive k is aligned to its largest product and bits below 2^-13 of
 * that product are dropped; the group sums and the accumulator are fp32.
 * Arguments, limits and errors as for w8a8_gemm_fp8. */
W8A8_API w8a8_status w8a8_gemm_fp8_fast(const uint8_t* a_q, const float* s_a, const uint8_t* b_packed,
                                        const float* s_b, int64_t M, int64_t N, int64_t K, float* out,
                                        w8a8_stream stream);

/* -------------------------------------------------------------------------
 * The MoE expert layer.
 *
 *   1. x_q, s_x   = per-token quantisation of x          ([K100AI] sec. 2.1)
 *   2. logits     = x . router_w^T + router_b, fp32 on the unquantised x
 *                                                         ([DSV4] sec. 4.1)
 *   3. top-k experts per token by logit (descending, ties to the lower
 *      index); weights w = softmax over the k picked logits, which equals
 *      softmax over all experts renormalised over the picked ones
 *                                                         ([HUNYUAN] 1.3)
 *   4. assignments a = t*k + j grouped into contiguous per-expert segments,
 *      ascending token order inside a segment              ([HUNYUAN] 1.3)
 *   5. gate-up: acc = x_q[t] . W_gu[e]^T (int32); g = ((float)acc_g * s_x[t])
 *      * s_gu[e][i], u likewise with s_gu[e][I+i]; h = SiLU(g) * u with
 *      SiLU(g) = g / (1 + exp(-g)), the exponential correctly rounded to
 *      fp32; h requantised per assignment row like step 1  ([DSV4] sec. 2.3)
 *   6. down: acc = h_q . W_d[e]^T (int32); o = w * (((float)acc * s_h) *
 *      s_d[e][n])                                          ([K100AI] 2.1)
 *   7. y[t] = sum over j = 0..k-1 (in order) of o[t*k+j]   ([HUNYUAN] 1.3)
 *
 * Layouts (all device memory, row-major, 16-byte aligned):
 *   x [T][H] fp32 in, y [T][H] fp32 out (x, y and the workspace must not
 *   overlap: W8A8_ERR_INVALID_ARGUMENT)
 *   router_w [E][H] fp32, router_b [E] fp32 or NULL (zero bias)
 *   w_gate_up: w8a8_pack_weights([E][2I][H], GATE_UP); s_gate_up [E][2I]
 *   w_down:    w8a8_pack_weights([E][H][I], PLAIN);    s_down    [E][H]
 * Limits: T >= 0 (0 is a no-op), T*k <= 2^24; H % 128 == 0, 128 <= H <= 16384;
 * I % 128 == 0, 128 <= I <= 16384; 1 <= E <= 256; 1 <= top_k <= min(E, 8).
 *
 * workspace: device memory of at least w8a8_moe_workspace_query().total_bytes,
 * 256-byte aligned.  After the call completes on the stream the workspace
 * holds the intermediates at the offsets the query reports (for checking).
 * ------------------------------------------------------------------------- */
typedef struct {
    int64_t T, H, E, top_k, I;
} w8a8_moe_shape;

typedef struct {
    const float* router_w;
    const float* router_b;
    const int8_t* w_gate_up;
    const float* s_gate_up;
    const int8_t* w_down;
    const float* s_down;
    int32_t code;  /* W8A8_CODE_INT8, W8A8_CODE_FP8_E4M3 or W8A8_CODE_FP8_E4M3_FAST:
                      the code of w_gate_up and w_down, the code the layer
                      quantises x and h to, and (FP8) the matrix cores that
                      multiply them */
    /* Options of the per-token quantisation of x (see w8a8_quantize_rows_ex;
     * zero-initialised: plain dynamic absmax).  x_smooth: NULL or [H] fp32,
     * 16-byte aligned; w_gate_up must then hold the codes of the weights with
     * 1/x_smooth on their input channels.  The router reads the unsmoothed x. */
    const float* x_smooth;
    int32_t x_scale_mode;
    float x_clip;
} w8a8_moe_weights;

/* Byte offsets of the intermediates inside the workspace. */
typedef struct {
    size_t total_bytes;
    size_t x_q;            /* int8  [T][H]          per-token codes              */
    size_t x_scale;        /* fp32  [T]                                          */
    size_t logits;         /* fp32  [T][E]          router logits                */
    size_t topk_ids;       /* int32 [T][k]                                       */
    size_t topk_w;         /* fp32  [T][k]                                       */
    size_t expert_counts;  /* int32 [E]                                          */
    size_t expert_offsets; /* int32 [E+1]           segment starts               */
    size_t sorted_assign;  /* int32 [T*k]           a = t*k+j per sorted row     */
    size_t h;              /* fp32  [T*k][I]        SiLU(g)*u, sorted row order  */
    size_t h_q;            /* int8  [T*k][I]        requantised h, sorted order  */
    size_t h_scale;        /* fp32  [T*k]           sorted order                 */
    size_t o;              /* fp32  [T*k][H]        weighted expert outputs, row
                                                    a = t*k+j                    */
    size_t internal;       /* scratch: router split sums, router weight planes
                              (from 2048 tokens), routing tables, tile queues   */
} w8a8_moe_workspace_layout;

W8A8_API w8a8_status w8a8_moe_workspace_query(const w8a8_moe_shape* shape, w8a8_moe_workspace_layout* layout);

W8A8_API w8a8_status w8a8_moe_forward(const w8a8_moe_shape* shape, const w8a8_moe_weights* weights,
                             const float* x, float* y, void* workspace, size_t workspace_bytes,
                             w8a8_stream stream);

/* -------------------------------------------------------------------------
 * The same layer with stage-boundary timing events, for measurement.
 * events[i] (a hipEvent_t created by the caller, passed as void*) is recorded
 * on the stream right before stage i is enqueued, and events[W8A8_MOE_STAGES]
 * after the last one.  Stages: 0 per-token quantisation, 1 router + top-k +
 * permutation, 2 grouped gate-up GEMM (SwiGLU epilogue), 3 requantisation of
 * h, 4 grouped down GEMM (weighted scatter epilogue), 5 combine.
 * events == NULL behaves exactly like w8a8_moe_forward; a NULL entry skips
 * that boundary (each recorded event costs a few microseconds on the stream).
 * ------------------------------------------------------------------------- */
enum { W8A8_MOE_STAGES = 6 };

W8A8_API w8a8_status w8a8_moe_forward_events(const w8a8_moe_shape* shape,
                                             const w8a8_moe_weights* weights, const float* x,
                                             float* y, void* workspace, size_t workspace_bytes,
                                             void* const* events, w8a8_stream stream);

/* -------------------------------------------------------------------------
 * The layer for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same computation and kernels as w8a8_moe_forward, with the workspace in a
 * static device array of W8A8_STATIC_WORKSPACE_BYTES that the library holds
 * on each device it runs on until the process ends (its address is looked up
 * once per device, on the first call there).  The call allocates and frees
 * nothing.  Every call on one device shares that device's array and leaves
 * its intermediates there: calls that overlap on one device (other streams,
 * other host threads) race and must be serialised by the caller.  Shapes
 * whose workspace (w8a8_moe_workspace_query) exceeds the array return
 * W8A8_ERR_WORKSPACE_TOO_SMALL before any launch; otherwise arguments,
 * limits and errors as w8a8_moe_forward.
 * ------------------------------------------------------------------------- */
#define W8A8_STATIC_WORKSPACE_BYTES (64u << 20)

W8A8_API w8a8_status w8a8_moe_forward_static(const w8a8_moe_shape* shape, const w8a8_moe_weights* weights,
                                             const float* x, float* y, w8a8_stream stream);

/* -------------------------------------------------------------------------
 * The grouped gate-up GEMM's raw int32 accumulators, for checking ([K100AI]
 * sec. 2.1: int8 x int8 products summed in int32; [HUNYUAN] sec. 1.3: each
 * expert's rows read through the routing index).  Runs the layer's gate-up
 * GEMM again with an epilogue that stores the accumulators instead of
 * finishing them, over the routing tables a previous w8a8_moe_forward call
 * (same shape, weights and workspace, INT8 code) left in the workspace; the
 * workspace is only read.  Enqueue it after that call on the same stream.
 *   acc: device int32 [T*k][2I], 4-byte aligned, written in full; row r is
 *        the r-th row of the expert-sorted order (sorted_assign[r] names its
 *        assignment t*k+j); column c < I holds gate channel c, column I + c
 *        up channel c: acc[r][c] = sum_h x_q[t][h] * W_gate_up[e][c][h] with
 *        W_gate_up the unpacked [E][2I][H] codes.
 * Errors: as w8a8_moe_forward; W8A8_ERR_INVALID_ARGUMENT for E4M3 weights
 * (their accumulators are fp32), a NULL acc, and an acc that overlaps the
 * workspace.
 * ------------------------------------------------------------------------- */
W8A8_API w8a8_status w8a8_moe_gate_up_acc(const w8a8_moe_shape* shape, const w8a8_moe_weights* weights,
                                          const void* workspace, size_t workspace_bytes, int32_t* acc,
                                          w8a8_stream stream);

/* -------------------------------------------------------------------------
 * w8a8_moe_forward_fused: the same layer as w8a8_moe_forward for a
 * decode-sized batch (T <= 64), in one persistent launch ("Tencent Hunyuan AI
 * Infra ... Hopper", sec. 1.3: gate, top-k, the index preparation, the expert
 * GEMMs and the combine in a single FusedMoE kernel).  A cooperative launch
 * (all workgroups resident) whose phases -- quantisation and router; top-k and
 * the permutation; gate-up; requantisation of h; down; combine -- are
 * separated by grid barriers; every workgroup ranks the routing itself, in its
 * own LDS.  Preceded on the stream by a one-workgroup launch that clears the
 * barrier words.
 *   Arguments, layouts, ownership and the workspace as for w8a8_moe_forward
 *   (the workspace holds the same intermediates afterwards).  Results: x_q,
 *   h, h_q, o and y as w8a8_moe_forward computes them from the same routing;
 *   the logits are fp64 sums of the fp32 products rounded once to fp32 (the
 *   multi-launch router's bf16 three-term split agrees with them within the
 *   fp32 error bound), so top-k picks can differ only at near ties.
 *   Calls that share a workspace must not overlap.  The launch is
 *   cooperative, so it cannot be captured where cooperative launches are not.
 * Errors: as w8a8_moe_forward; W8A8_ERR_UNSUPPORTED_SHAPE for T > 64;
 * W8A8_ERR_HIP if the device cannot hold the cooperative grid.
 * ------------------------------------------------------------------------- */
W8A8_API w8a8_status w8a8_moe_forward_fused(const w8a8_moe_shape* shape, const w8a8_moe_weights* weights,
                                            const float* x, float* y, void* workspace, size_t workspace_bytes,
                                            w8a8_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* W8A8MOE_H */
