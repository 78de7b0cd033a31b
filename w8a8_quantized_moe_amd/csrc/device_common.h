// Device building blocks of the routing and quantisation kernels: block
// scans, the per-m-tile table, wave top-k and routing weights, and the per-row
// quantisation arithmetic.
#pragma once

#include "internal.h"

namespace w8a8 {

// Block-wide exclusive scan of one int per thread (NW waves of 64).
// One step of a wave-wide maximum through a DPP lane permutation (a VALU
// operand modifier, no LDS traffic): lanes whose source lane is out of range,
// and rows outside ROW_MASK, keep their own value.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float max_dpp(float x) {
    const int y = __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, ROW_MASK, 0xF, false);
    return fmaxf(x, __int_as_float(y));
}

// The maximum over the 64 lanes of a wave, returned to every lane: the
// maximum of each quad (quad_perm), half row and row (mirrors), then rows 0-1
// into row 1 and rows 2-3 into row 3 (row_bcast:15), then row 1 into rows 2-3
// (row_bcast:31); lane 63 ends with the whole wave's maximum.
__device__ __forceinline__ float wave_max_dpp(float x) {
    x = max_dpp<0xB1, 0xF>(x);   // quad_perm [1,0,3,2]
    x = max_dpp<0x4E, 0xF>(x);   // quad_perm [2,3,0,1]
    x = max_dpp<0x141, 0xF>(x);  // row_half_mirror
    x = max_dpp<0x140, 0xF>(x);  // row_mirror
    x = max_dpp<0x142, 0xA>(x);  // row_bcast:15 into rows 1 and 3
    x = max_dpp<0x143, 0xC>(x);  // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// One step of a wave-wide inclusive sum through a DPP lane permutation:
// lanes outside ROW_MASK / BANK_MASK, and lanes whose source lane is out of
// range, add 0.
template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ int add_dpp(int acc, int src) {
    return acc + __builtin_amdgcn_update_dpp(0, src, CTRL, ROW_MASK, BANK_MASK, true);
}

// Inclusive prefix sum over the 64 lanes of a wave: sums of 4 within each row
// (row_shr 1..3 of the input), of 8 and 16 (row_shr 4 and 8 of the partial
// sums, upper banks only), then the totals of row 0 into row 1 and of row 2
// into row 3 (row_bcast:15) and of rows 0-1 into rows 2-3 (row_bcast:31).
__device__ __forceinline__ int wave_inclusive_scan_dpp(int x) {
    int s = add_dpp<0x111, 0xF, 0xF>(x, x);   // row_shr:1
    s = add_dpp<0x112, 0xF, 0xF>(s, x);       // row_shr:2
    s = add_dpp<0x113, 0xF, 0xF>(s, x);       // row_shr:3
    s = add_dpp<0x114, 0xF, 0xE>(s, s);       // row_shr:4, lanes 4-15 of each row
    s = add_dpp<0x118, 0xF, 0xC>(s, s);       // row_shr:8, lanes 8-15 of each row
    s = add_dpp<0x142, 0xA, 0xF>(s, s);       // row_bcast:15 into rows 1 and 3
    s = add_dpp<0x143, 0xC, 0xF>(s, s);       // row_bcast:31 into rows 2 and 3
    return s;
}

template <int NW>
__device__ __forceinline__ int block_exclusive_scan(int v, int* total, int* lds /* >= NW ints */) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int incl = wave_inclusive_scan_dpp(v);
    if (lane == 63) lds[w] = incl;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        if (i < w) base += lds[i];
        tot += lds[i];
    }
    __syncthreads();
    *total = tot;
    return base + incl - v;
}

// The m-tiles of expert e (first .. first + n - 1) all name e, its first
// m-tile and its segment [seg_start, seg_end).
__device__ __forceinline__ void write_mt_info(MtInfo* info, int e, int first, int n, int seg_start,
                                              int seg_end) {
    const MtInfo v{e, first, seg_start, seg_end};
    for (int q = 0; q < n; ++q) info[first + q] = v;
}

// Fixed cost of one GEMM tile in rows of work: a tile with r valid rows takes
// about as long as (TILE_FIXED_ROWS + r) rows' worth of a full tile's time
// (the whole weight tile streams through whatever the row count).
constexpr int TILE_FIXED_ROWS = 200;

// The per-m-tile table in longest-first order and the XCD queue bounds of the
// two grouped GEMMs.  Called by every thread of one workgroup of NT threads
// (NT >= MAX_EXPERTS); thread e < E holds expert e's row count cnt, segment
// start off and m-tile count mc.  Experts are ranked by row count, descending,
// ties to the lower index; their m-tiles are listed in rank order.  The tile
// order of a GEMM with ntv column tiles is (rank, column tile, m-tile), m-tile
// fastest; it is cut into 8 contiguous XCD queues of about equal work, each
// tile weighing TILE_FIXED_ROWS + its rows, at column-tile boundaries of an
// expert (the m-tiles sharing a weight tile stay on one XCD, and so do the
// column tiles of an expert, which share its activation rows, but for the
// experts a cut falls in).  xb[g*9 + x] (g = 0 gate-up, 1 down) is the first
// tile of queue x, xb[g*9 + 8] the tile count.
struct alignas(16) RankedLds {
    int cnt_e[MAX_EXPERTS];        // by expert
    int cnt_r[MAX_EXPERTS];        // by rank
    int mc_r[MAX_EXPERTS];         // by rank
    int first_r[MAX_EXPERTS];      // first m-tile, by rank
    long long work[MAX_EXPERTS];   // inclusive prefix of the ranks' work per column tile
    int scan[16];                  // one int per wave of the workgroup (at most 1024 threads)
};

template <int NT>
__device__ __forceinline__ void write_ranked_tables(int cnt, int off, int mc, int E, MtInfo* mt_info,
                                                    int32_t* xb, int ntv0, int ntv1, RankedLds& l) {
    static_assert(NT >= MAX_EXPERTS && NT % 64 == 0 && NT <= 1024, "one thread per expert");
    const int e = threadIdx.x;
    if (e < MAX_EXPERTS) l.cnt_e[e] = e < E ? cnt : -1;
    __syncthreads();
    int rank = 0;
    if (e < E) {
        const int4* c4 = reinterpret_cast<const int4*>(l.cnt_e);
        for (int i4 = 0; i4 < (E + 3) / 4; ++i4) {
            const int4 c = c4[i4];
            const int i = 4 * i4;
            rank += (c.x > cnt) || (c.x == cnt && i < e);
            rank += (c.y > cnt) || (c.y == cnt && i + 1 < e);
            rank += (c.z > cnt) || (c.z == cnt && i + 2 < e);
            rank += (c.w > cnt) || (c.w == cnt && i + 3 < e);
        }
        l.cnt_r[rank] = cnt;
        l.mc_r[rank] = mc;
    }
    __syncthreads();
    int total;
    const int r_mc = e < E ? l.mc_r[e] : 0;
    const int fr = block_exclusive_scan<NT / 64>(r_mc, &total, l.scan);
    long long w = e < E ? (long long)r_mc * TILE_FIXED_ROWS + l.cnt_r[e] : 0;
    if (e < MAX_EXPERTS) {
        l.first_r[e] = fr;
        l.work[e] = w;
    }
    __syncthreads();
    for (int o = 1; o < MAX_EXPERTS; o <<= 1) {  // inclusive prefix of the work
        const long long u = (e < MAX_EXPERTS && e >= o) ? l.work[e - o] : 0;
        __syncthreads();
        if (e < MAX_EXPERTS) l.work[e] = (w += u);
        __syncthreads();
    }
    if (e < E) write_mt_info(mt_info, e, l.first_r[rank], mc, off, off + cnt);
    if (e < 18) {
        const int g = e / 9, x = e % 9;
        const int64_t ntv = g ? ntv1 : ntv0;
        int64_t bound = (x == 8) ? (int64_t)total * ntv : 0;
        if (x > 0 && x < 8) {
            // the first rank whose work ends past x/8 of the total; the cut
            // falls at the column tile where x/8 of the work is reached
            const long long S = l.work[E - 1];
            const long long target = (long long)x * S;  // against 8 x cumulative work
            int lo = 0, hi = E;  // smallest r with 8 * work[r] > target
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (8 * l.work[mid] > target) hi = mid;
                else lo = mid + 1;
            }
            if (lo == E) {
                bound = (int64_t)total * ntv;
            } else {
                const long long gw = (long long)l.mc_r[lo] * TILE_FIXED_ROWS + l.cnt_r[lo];
                const long long cum = l.work[lo] - gw;
                long long cols = ntv * (target - 8 * cum) / (8 * gw);
                cols = cols < 0 ? 0 : (cols > ntv ? ntv : cols);
                bound = (int64_t)l.first_r[lo] * ntv + cols * l.mc_r[lo];
            }
        }
        xb[e] = (int32_t)bound;
    }
}

// k rounds of a wave-wide arg-max over the logits of N tokens of one wave
// (token u's lane l holds experts l, l+64, l+128, l+192 in v[u][0..3], -inf
// past E); ties go to the lower expert index.  Lane 0 writes the picks in
// descending order to ids/vals.  The rounds of the N tokens run in lockstep.
// A round takes the wave maximum m of the lanes' best values (DPP, no LDS
// traffic), then the lowest expert index holding m: the lowest lane among
// those whose best is m in slot 0, else in slot 1, ... (an index in slot s
// is below every index in slot s+1), from one ballot per slot.  Token u
// writes to ids/vals + u * ustride, and only if u < n_valid.
template <int N>
__device__ __forceinline__ void wave_topk_n(float (&v)[N][4], int lane, int E, int k, int n_valid,
                                            int* ids, float* vals, int ustride) {
#pragma unroll 1
    for (int j = 0; j < k; ++j) {
        float bv[N], m[N];
        int bs[N];
#pragma unroll
        for (int u = 0; u < N; ++u) {
            // the lane's best slot, the lower slot on ties
            bv[u] = v[u][0];
            bs[u] = 0;
            if (v[u][1] > bv[u]) { bv[u] = v[u][1]; bs[u] = 1; }
            if (v[u][2] > bv[u]) { bv[u] = v[u][2]; bs[u] = 2; }
            if (v[u][3] > bv[u]) { bv[u] = v[u][3]; bs[u] = 3; }
        }
#pragma unroll
        for (int u = 0; u < N; ++u) m[u] = wave_max_dpp(bv[u]);
#pragma unroll
        for (int u = 0; u < N; ++u) {
            // lowest (slot, lane) holding the maximum; padding (index >= E)
            // never counts.  Lane 0, slot 0 if none does (non-finite logits).
            int wl = 0, ws = 0;
#pragma unroll
            for (int s = 3; s >= 0; --s) {
                const unsigned long long msk = __ballot(bv[u] == m[u] && bs[u] == s && lane + 64 * s < E);
                if (msk) {
                    wl = __ffsll((long long)msk) - 1;
                    ws = s;
                }
            }
            const float val = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv[u]), wl));
            if (lane == 0 && u < n_valid) {
                ids[u * ustride + j] = wl + 64 * ws;
                vals[u * ustride + j] = val;
            }
            if (lane == wl) {
                if (ws == 0) v[u][0] = -INFINITY;
                else if (ws == 1) v[u][1] = -INFINITY;
                else if (ws == 2) v[u][2] = -INFINITY;
                else v[u][3] = -INFINITY;
            }
        }
    }
}

// Routing weights of one token from its k picked logits (descending): the
// softmax over the picks, which equals the full softmax renormalised over
// them; terms summed in pick order, fp32.
__device__ __forceinline__ void topk_weights(const float* vals, int k, float* w) {
    const float mx = vals[0];
    float z = 0.0f;
    for (int j = 0; j < k; ++j) z += expf(vals[j] - mx);
    for (int j = 0; j < k; ++j) w[j] = expf(vals[j] - mx) / z;
}

__device__ __forceinline__ float wave_max(float v) { return wave_max_dpp(v); }

__device__ __forceinline__ int quant_one(float v, float s) {
    if (s == 0.0f) return 0;
    float r = __builtin_rintf(v / s);
    r = fminf(fmaxf(r, -128.0f), 127.0f);
    return (int)r;
}

// Same result as quant_one, cheaper: y = v * (1/s) differs from the IEEE
// quotient fl(v/s) by less than 2.5 ulp, i.e. by less than 2^-15 for
// |v/s| <= 127.  Rounding y and fl(v/s) to the nearest integer can then only
// disagree if y lies within 2^-15 of a half-integer; those (rare) elements
// take the exact division.
__device__ __forceinline__ int quant_fast(float v, float s, float rs) {
    if (s == 0.0f) return 0;
    const float y = v * rs;
    const float fy = fabsf(y);
    const float frac = fy - __builtin_floorf(fy);
    float r;
    // the comparisons are written so that a non-finite y (1/s overflowing for
    // a subnormal scale) also takes the exact path
    if (fy <= 128.0f && fabsf(frac - 0.5f) >= 0x1p-15f) r = __builtin_rintf(y);
    else r = __builtin_rintf(v / s);
    r = fminf(fmaxf(r, -128.0f), 127.0f);
    return (int)r;
}

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
           ((uint32_t)(d & 0xff) << 24);
}

__device__ __forceinline__ float4 mul4(float4 v, float4 m) {
    return make_float4(v.x * m.x, v.y * m.y, v.z * m.z, v.w * m.w);
}

__device__ __forceinline__ float amax4(float4 v) {
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// ---- code types of the quantised operands ----
// INT8: s = max|x| / 127, q = clamp(rne(x / s), -128, 127)  ([K100AI] 2.1).
// FP8 E4M3 ([DSV4] 2.1: 4 exponent and 3 mantissa bits, range +-448): s =
// max|x| / 448, q = E4M3(x / s), the quotient an IEEE fp32 division and the
// conversion gfx950's v_cvt_pk_fp8_f32 (OCP E4M3FN, round to nearest even).
// An all-zero row gives s = 0 and code 0 in both.
template <int CODE>
__device__ __forceinline__ float code_range() {
    return CODE == CODE_FP8 ? 448.0f : 127.0f;
}

// The E4M3 conversion's input: the IEEE quotient v / s, saturated at +-448
// (a capped or static scale lets |v / s| exceed the range; below it the
// clamp changes nothing, since values up to 464 round to 448 anyway).
__device__ __forceinline__ float fp8_quotient(float v, float s) {
    if (s == 0.0f) return 0.0f;
    return fminf(fmaxf(v / s, -448.0f), 448.0f);
}

// The scale's base for a row whose (smoothed) maximum is amax.
__device__ __forceinline__ float scale_base(float amax, const QuantOpts& opt) {
    if (opt.mode == SCALE_STATIC) return opt.clip;
    if (opt.mode == SCALE_CLIPPED && opt.clip < amax) return opt.clip;
    return amax;
}

// Four codes of one row packed into a 32-bit word (element 0 in the low byte).
template <int CODE>
__device__ __forceinline__ uint32_t encode4(const float4& v, float s, float rs) {
    if (CODE == CODE_INT8)
        return pack4(quant_fast(v.x, s, rs), quant_fast(v.y, s, rs), quant_fast(v.z, s, rs),
                     quant_fast(v.w, s, rs));
    const float a = fp8_quotient(v.x, s), b = fp8_quotient(v.y, s);
    const float c = fp8_quotient(v.z, s), d = fp8_quotient(v.w, s);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// A row's float4 slots i*STRIDE + idx (i < N), times the per-column factor
// when there is one.  Every load is issued before any value is used: slots
// past the row's end re-read its last float4 instead of branching around the
// load (a branch per slot made the compiler wait for each load in turn), and
// the callers ignore them.  The row is read once, so the loads are
// non-temporal (streamed past the caches: 27% faster on the large layer's x).
template <int N, int STRIDE>
__device__ __forceinline__ void load_row(const float4* __restrict__ xr, const float* col_mul, bool recip,
                                         int nv, int idx, float4 (&v)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const v4f t = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(xr) + min(i * STRIDE + idx, nv - 1));
        v[i] = make_float4(t.x, t.y, t.z, t.w);
    }
    if (col_mul) {
        const float4* m = reinterpret_cast<const float4*>(col_mul);
        float4 f[N];
#pragma unroll
        for (int i = 0; i < N; ++i) f[i] = m[min(i * STRIDE + idx, nv - 1)];
        if (recip) {
#pragma unroll
            for (int i = 0; i < N; ++i) f[i] = make_float4(1.0f / f[i].x, 1.0f / f[i].y, 1.0f / f[i].z, 1.0f / f[i].w);
        }
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = mul4(v[i], f[i]);
    }
}

// One row quantised by a whole workgroup of NT threads, VPT float4 per thread
// held in registers (cols % 4 == 0, cols <= 4 * NT * VPT; the row and the
// factor 16-byte aligned): the row maximum through a wave reduction and NT/64
// LDS slots (wmax), then the codes as 4-byte stores.  Called by every thread
// of the workgroup.
template <int CODE, int NT, int VPT>
__device__ __forceinline__ void quant_row_wg(const float* __restrict__ xrow, int cols, const QuantOpts& opt,
                                             int8_t* __restrict__ qrow, float* __restrict__ scale_out,
                                             float* wmax) {
    constexpr int NW = NT / 64;
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const float4* xr = reinterpret_cast<const float4*>(xrow);
    const int nv = cols >> 2;
    float4 v[VPT];
    load_row<VPT, NT>(xr, opt.col_mul, opt.col_recip, nv, tid, v);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < VPT; ++i)
        if (i * NT + tid < nv) amax = fmaxf(amax, amax4(v[i]));
    amax = wave_max(amax);
    if (lane == 0) wmax[wv] = amax;
    __syncthreads();
    amax = wmax[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) amax = fmaxf(amax, wmax[i]);
    const float s = scale_base(amax, opt) / code_range<CODE>();
    const float rs = 1.0f / s;
    if (tid == 0) *scale_out = s;
    uint32_t* qr = reinterpret_cast<uint32_t*>(qrow);
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int c = i * NT + tid;
        if (c < nv) qr[c] = encode4<CODE>(v[i], s, rs);
    }
}

template <int CODE>
__device__ __forceinline__ uint8_t encode1(float v, float s) {
    if (CODE == CODE_INT8) return (uint8_t)(int8_t)quant_one(v, s);
    return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(fp8_quotient(v, s), 0.0f, 0, false) & 0xff);
}

}  // namespace w8a8
