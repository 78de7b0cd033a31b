// Internal declarations shared by the HIP sources of libw8a8moe (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));

// Row-tile height of the int8 MFMA GEMM (the m-tile unit of the routing's
// per-expert tile prefix).
constexpr int GEMM_BM = 256;

// Routing works on chunks of 64 tokens (one bit per token in a 64-bit mask).
constexpr int ROUTE_CHUNK = 64;
constexpr int MAX_EXPERTS = 256;
constexpr int MAX_TOPK = 8;

// SiLU(g) = g / (1 + exp(-g)); the exponential is computed in double and
// rounded once to fp32 (correctly rounded fp32 exp but for vanishingly rare
// double-rounding cases); the add and the divide are IEEE fp32.  Every GEMM
// epilogue uses this one definition.
__device__ __forceinline__ float silu_f32(float g) {
    const float e = (float)exp(-(double)g);
    const float den = 1.0f + e;
    return g / den;
}

// ---- copy-pipeline helpers shared by the LDS-staged kernels ----
#define LDS_AS __attribute__((address_space(3)))


template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier without the implied memory fence of __syncthreads (which
// would wait for every load in flight, i.e. drain the copy pipeline); the
// "memory" clobber keeps the compiler from moving LDS accesses across it.
// Visibility of a copied stage is established by the vmcnt wait before it.
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

// One wave-wide 16-byte-per-lane global -> LDS copy (global_load_lds_dwordx4):
// lane l's 16 bytes land at lds_wave_base + 16*l; M0 carries the LDS base.
// Issued through inline asm so that the compiler does not model the LDS write:
// it would otherwise drain the whole copy pipeline (vmcnt(0)) before every
// LDS read it cannot prove disjoint.  The ring's hazards are handled by hand
// (explicit vmcnt waits before the workgroup barrier).  M0 is reserved by
// the compiler, so it is not named as clobbered (a reserved register in a
// clobber list is not preserved anyway); this is safe because nothing else in
// these kernels uses M0 (no LDS DMA builtins, no dynamic register indexing,
// no messages), which the generated code confirms: its only M0 writes are
// these.
__device__ __forceinline__ void dma16(const int8_t* gsrc, const LDS_AS int8_t* lds_wave_base) {
    const uint32_t lds = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off"
                 :
                 : "v"(gsrc), "s"(lds)
                 : "memory");
}
__device__ __forceinline__ void dma16(const int8_t* gsrc, const int8_t* lds_wave_base) {
    dma16(gsrc, (const LDS_AS int8_t*)lds_wave_base);
}

// Code type of the quantised operands.
enum Code : int {
    CODE_INT8 = 0,      // int8, int32 accumulation (exact)
    CODE_FP8 = 1,       // FP8 E4M3 (OCP E4M3FN): every product exact, summed in fp32
                        // (on the bf16 matrix cores)
    CODE_FP8_FAST = 2,  // FP8 E4M3 on the FP8 matrix cores (twice the rate; products
                        // aligned to the largest of each 8-k group inside an instruction)
};

// E4M3 values have at most 4 significant bits and exponents 2^-9 .. 2^8, so
// every one is a bf16 value and every product of two is exact in fp32.  Eight
// codes (two dwords, k in byte order) to eight bf16 values, exactly.
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
__device__ __forceinline__ v8bf e4m3x8_to_bf16(int lo, int hi) {
    const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    v8bf r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// One 16x16 output block += A fragment (16 rows x 64 k) . B fragment (16
// columns x 64 k), lane l holding row/column l%16 and the 16 k-bytes
// (l/16)*16 .. +15.  A and B lanes always pair the same byte positions, so an
// instruction may take any subset of a lane's bytes as its k, as long as both
// operands take the same one.
//  * INT8: v_mfma_i32_16x16x64_i8 (int32, exact).
//  * FP8: two v_mfma_f32_16x16x32_bf16, each on 8 of a lane's bytes decoded
//    to bf16 (lane l supplying k-slots (l/16)*8 .. +7 of the instruction's 32).
//  * FP8_FAST: two v_mfma_f32_16x16x32_fp8_fp8 on the same 8-byte groups.
//    (That FP8 MFMA issues at a quarter of the rate of the 32x32x64 one below:
//    the register-fed skinny kernel, which streams weights at HBM speed, uses
//    it; the LDS-tiled GEMM uses mma32.)
typedef long v2l __attribute__((ext_vector_type(2)));
template <int CODE>
struct AccOf {
    typedef v4f type;
};
template <>
struct AccOf<CODE_INT8> {
    typedef v4i type;
};
template <int CODE>
__device__ __forceinline__ typename AccOf<CODE>::type mma16(const v4i& a, const v4i& b,
                                                            const typename AccOf<CODE>::type& c) {
    if constexpr (CODE == CODE_INT8) {
        return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
    } else if constexpr (CODE == CODE_FP8) {
        const v4f c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(a[0], a[1]),
                                                               e4m3x8_to_bf16(b[0], b[1]), c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(a[2], a[3]), e4m3x8_to_bf16(b[2], b[3]),
                                                       c1, 0, 0, 0);
    } else {
        const v2l a2 = __builtin_bit_cast(v2l, a), b2 = __builtin_bit_cast(v2l, b);
        const v4f c1 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a2[0], b2[0], c, 0, 0, 0);
        return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a2[1], b2[1], c1, 0, 0, 0);
    }
}

// One 32x32 output block += 64 k of E4M3 codes, lane l supplying row (column)
// l%32 and 32 bytes of k; the 16 accumulator registers are held as 4 x v4f
// (register q in [q/4][q%4]), the layout of every 32x32 MFMA.
//  * FP8: four v_mfma_f32_32x32x16_bf16, each on 8 of a lane's bytes decoded
//    to bf16 (lane l supplying k-slots (l/32)*8 .. +7 of the instruction's 16).
//  * FP8_FAST: one v_mfma_scale_f32_32x32x64_f8f6f4 (block scales fixed at
//    2^0: E8M0 exponent 127).
typedef float v16f __attribute__((ext_vector_type(16)));
template <int CODE>
__device__ __forceinline__ void mma32(const v8i& a, const v8i& b, v4f (&c)[4]) {
    v16f t;
#pragma unroll
    for (int q = 0; q < 16; ++q) t[q] = c[q / 4][q % 4];
    if constexpr (CODE == CODE_FP8) {
#pragma unroll
        for (int g = 0; g < 4; ++g)
            t = __builtin_amdgcn_mfma_f32_32x32x16_bf16(e4m3x8_to_bf16(a[2 * g], a[2 * g + 1]),
                                                        e4m3x8_to_bf16(b[2 * g], b[2 * g + 1]), t, 0, 0, 0);
    } else {
        static_assert(CODE == CODE_FP8_FAST, "32x32 blocks are for E4M3 codes");
        t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, t, 0, 0, 0, 127, 0, 127);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) c[q / 4][q % 4] = t[q];
}

enum Epilogue : int {
    EPI_DENSE_F32 = 0,  // out[m][n] = ((float)acc * s_a[m]) * s_b[n]
    EPI_DENSE_I32 = 1,  // out[m][n] = acc
    EPI_GATE_UP = 2,    // h = SiLU(g) * u from interleaved gate/up columns
    EPI_DOWN = 3,       // o[slot][n] = w[slot] * (((float)acc * s_h[r]) * s_d[e][n])
    EPI_GU_I32 = 4,     // grouped gate-up, raw int32 accumulators: out[r][c] gate channel c,
                        // out[r][I + c] up channel c (r: sorted row)
};

struct GemmParams {
    const int8_t* A;          // activations, [rows][K] int8 row-major
    const int8_t* B;          // packed weights of group 0
    int64_t b_group_bytes;    // bytes per group of packed weights (N*K)
    int64_t M;                // dense: rows; grouped: total assignments
    int N, K;
    int VG, NTV;              // set by launch_gemm: column stripes and n-tiles per stripe
    const int32_t* seg_offsets;  // grouped: [G+1] segment starts, else nullptr
    const int32_t* mt_prefix;    // grouped: [G+1] prefix of m-tiles per group
    const int32_t* mt_info;      // grouped: per m-tile {group, first m-tile of the group,
                                 // segment start, segment end} (MtInfo)
    int G;
    const int32_t* sorted_assign;  // grouped: assignment a = t*k+j of each sorted row
    int topk;
    const float* s_a;    // dense: [M]; gate-up: s_x[T] by token; down: s_h[A] by sorted row
    const float* s_b;    // [G][N] per-output-channel scales (gate-up: [G][2I] unpermuted)
    const float* route_w;  // down: routing weight per assignment a
    float* out_f32;
    int32_t* out_i32;
    int I;               // gate-up: intermediate size (N = 2I)
    int64_t a_rows;      // rows of the A operand (gate-up: T); indices are clamped to it
    int code;            // CODE_INT8, CODE_FP8 or CODE_FP8_FAST (both operands)
    int32_t* tile_ctr;   // grouped: 8 zeroed tile counters (stride TILE_CTR_STRIDE), one
                         // queue per XCD, for a persistent launch; nullptr: one tile
                         // per workgroup
    const int32_t* xcd_bounds;  // grouped persistent: [9] tile ranges of the XCD queues (the
                                // routing balances them by work); nullptr: equal tile counts
};

// Column tile width of the tiled GEMM for N output columns.
int gemm_tile_n(int64_t N, int code);

// Tile-queue counters sit 128 bytes apart; the routing zeroes TILE_CTR_COUNT of them.
constexpr int TILE_CTR_STRIDE = 32;
constexpr int TILE_CTR_COUNT = 16;  // gate-up queues 0..7, down queues 8..15

// Compute units of the current device (queried once per device).
int device_cu_count();

// Activation-scale options of the per-row quantiser ("W8A8 quantisation of
// MiniMax-M3 on K100AI", sec. 2.2; "DeepSeek V4 '950'", sec. 3.1): a
// per-column factor applied before the scale is taken (SmoothQuant), and the
// scale's base: the row maximum (dynamic), the row maximum capped by a
// calibrated bound (clipped), or the bound alone (static).
enum ScaleMode : int { SCALE_DYNAMIC = 0, SCALE_CLIPPED = 1, SCALE_STATIC = 2 };
struct QuantOpts {
    const float* col_mul = nullptr;  // [cols] or nullptr
    int mode = SCALE_DYNAMIC;
    float clip = 0.0f;               // > 0 for the clipped and static modes
    bool col_recip = false;          // apply 1/col_mul[c] (an IEEE fp32 division) instead:
                                     // the inverse factor a smoothed layer's weights take
};

// ---- launchers (each returns the launch status) ----
hipError_t launch_quantize_rows(const float* x, int64_t rows, int64_t cols, int64_t ld, int8_t* q,
                                float* scale, int code, hipStream_t s, const QuantOpts& opt = QuantOpts{});

hipError_t launch_pack_weights(const int8_t* w, int64_t groups, int64_t n, int64_t k, int kind,
                               int8_t* packed, hipStream_t s);

// max_m_tiles: an upper bound of the number of BM-row tiles (grouped: over all
// experts); surplus workgroups exit on the device.
hipError_t launch_gemm(int epi, const GemmParams& p, int64_t max_m_tiles, hipStream_t s);

// Grouped GEMM for segments of a few rows (decode): 16-row blocks, no LDS,
// operands loaded straight into registers.  max_row_blocks bounds the number
// of 16-row blocks over all groups; the routing's m-tile prefix must use
// SKINNY_BM.  Gate-up and down epilogues only.
constexpr int SKINNY_BM = 16;
hipError_t launch_gemm_skinny(int epi, const GemmParams& p, int64_t max_row_blocks, hipStream_t s);

// How the router GEMM runs for a shape: the number of partial sums S it
// splits H into (so a small token count still yields enough workgroups; the
// workspace then holds S*T*E floats), and whether the router weights are
// first split into bf16 planes in the workspace (planes_bytes > 0, large
// token counts) or split inside the GEMM.
struct RouterPlan {
    int splits;
    size_t planes_bytes;
};
RouterPlan router_plan(int T, int E, int H);

// The per-token quantisation of x, run by extra workgroups of the router's
// launch when the tokens are few (one launch fewer on the layer's critical
// path; the two read the same x and are otherwise independent).
struct XQuantJob {
    int8_t* q = nullptr;     // [T][H] codes; nullptr: no job (x is quantised by its own launch)
    float* scale = nullptr;  // [T]
    QuantOpts opt;
    int code = CODE_INT8;
};
// Token counts up to which the router launch also quantises x (its
// workgroups hold the router's LDS, so many rows are better served by the
// quantisation kernel's own launch).
constexpr int ROUTER_XQUANT_MAX_T = 256;

struct RouteInputs {
    const float* x;         // [T][H]
    const float* router_w;  // [E][H]
    const float* router_b;  // [E] or nullptr
    int T, H, E, k;
    int splits;             // router_plan(T, E, H).splits
    int bm;                 // m-tile height of the grouped GEMMs (GEMM_BM or SKINNY_BM)
    int ntv_gu, ntv_dn;     // column tiles of the gate-up and down GEMMs (queue bounds)
    XQuantJob xq;           // x quantised in the same launch (no router planes, T <= ROUTER_XQUANT_MAX_T)
};

struct RouteBuffers {
    float* partial;           // [S][T][E]
    void* wplanes;            // router_plan(T, E, H).planes_bytes bytes, or nullptr
    float* logits;            // [T][E]
    int32_t* topk_ids;        // [T][k]
    float* topk_w;            // [T][k]
    int32_t* chunk_counts;    // [E][nchunks]
    int32_t* chunk_base;      // [E][nchunks]
    int32_t* rank;            // [T*k] rank of an assignment inside its chunk and expert
    int32_t* expert_counts;   // [E]
    int32_t* expert_offsets;  // [E+1]
    int32_t* mt_prefix;       // [E+1] prefix of m-tiles per expert
    int32_t* mt_info;         // [m-tiles][4] MtInfo of every m-tile
    int32_t* tile_ctr;        // [TILE_CTR_COUNT * TILE_CTR_STRIDE] zeroed here for the GEMMs' queues
    int32_t* sorted_assign;   // [T*k]
    int32_t* xcd_bounds;      // [2][9] XCD queue bounds of the gate-up and down GEMMs
};

hipError_t launch_route(const RouteInputs& in, const RouteBuffers& b, hipStream_t s);

// One entry of the per-m-tile table the routing writes for the grouped GEMMs,
// so that a workgroup finds its expert with one load instead of a search.  The
// table lists the experts' m-tiles largest segment first (ties to the lower
// expert index), so each of the GEMMs' XCD queues holds its longest tiles first
// (see write_ranked_tables).
struct MtInfo {
    int32_t group;       // expert
    int32_t first_tile;  // index of the expert's first m-tile
    int32_t seg_start;   // first row of the expert's segment
    int32_t seg_end;     // one past its last row
};
static_assert(sizeof(MtInfo) == 16, "one 16-byte load per m-tile");

hipError_t launch_combine(const float* o, int T, int k, int H, float* y, hipStream_t s);

// ---- the whole layer in one launch (decode-sized batches) ----
constexpr int FUSED_MAX_T = 64;     // tokens: one routing chunk, ranked in every workgroup's LDS
constexpr int FUSED_WG_PER_CU = 1;  // workgroups per compute unit, all resident (cooperative launch)

struct FusedParams {
    const float* x;         // [T][H]
    const float* router_w;  // [E][H]
    const float* router_b;  // [E] or nullptr
    const int8_t* w_gu;     // packed gate-up codes
    const float* s_gu;      // [E][2I]
    const int8_t* w_d;      // packed down codes
    const float* s_d;       // [E][H]
    float* y;               // [T][H]
    int T, H, E, k, I;
    QuantOpts x_opt;
    // the intermediates, at the workspace offsets of the multi-launch layer
    int8_t* x_q;
    float* x_scale;
    float* logits;
    int32_t* topk_ids;
    float* topk_w;
    int32_t* expert_counts;
    int32_t* expert_offsets;
    int32_t* sorted_assign;
    float* h;
    int8_t* h_q;
    float* h_scale;
    float* o;
    int32_t* sync;          // 2 words: barrier arrivals, timeout flag (zeroed by the launcher)
};
hipError_t launch_moe_fused(const FusedParams& p, int code, hipStream_t s);


}  // namespace w8a8
