// Router, top-k and permutation into contiguous per-expert segments.
//
// Sources: "DeepSeek V4 '950' unified FP8 dataflow on H100", sec. 4.1 (the
// router GEMM stays in fp32 on the unquantised activations);
// "Tencent Hunyuan AI Infra ... Hopper", sec. 1.3 (gate, top-k, then index
// preparation that reserves a contiguous output region per expert, so the
// expert GEMM reads its input rows through the index with no gather pass);
// "W8A8 quantisation of MiniMax-M3 on K100AI", sec. 3.2 (a pre-planned buffer
// for the routing reorder).
//
// Kernels, all on the caller's stream, no host synchronisation:
//   router_bf16x3   the fp32 router GEMM on the bf16 matrix cores at fp32
//                   accuracy (each operand split exactly into three bf16
//                   terms), 64-token x all-expert tiles (activations read
//                   once), optionally split along H into S partial sums so
//                   small token counts still fill the GPU;
//   router_w_planes (many tokens) splits the router weights into three bf16
//                   planes in MFMA fragment order, once per call;
//   router_planes   the same GEMM reading those planes, 128-token x
//                   32*EB-expert tiles (only the activations are split in
//                   the main loop);
//   router_reduce   (split only) sums the S partials in split order (a fixed,
//                   deterministic order) and adds the bias;
//   topk_count      per 64-token chunk: picks the top-k by wave arg-max rounds
//                   (ties to the lower index), computes the renormalised
//                   softmax weights, and ranks each assignment among the
//                   chunk's tokens routed to the same expert with a 64-bit
//                   token mask per expert (a single chunk also finishes the
//                   permutation below in the same workgroup);
//   chunk_scan      per expert: exclusive scan of its per-chunk counts;
//   finalize        exclusive scan over experts -> segment offsets, the
//                   prefix of m-tiles per expert and the per-m-tile table
//                   (expert, first m-tile, segment) of the grouped GEMMs;
//   scatter         sorted_assign[offset[e] + chunk_base + rank] = t*k + j.
// The resulting order inside a segment is ascending token order.
#include <type_traits>

#include "device_common.h"

namespace w8a8 {
namespace {

constexpr int RBM = 64, RBK = 32;
constexpr int TOPK_THREADS = 1024;  // 16 waves: 4 tokens of a 64-token chunk each

// partial[s][t][e] = sum over h in split s of x[t][h] * wr[e][h] on the bf16
// matrix cores at fp32 accuracy; with a single split the output is the logits
// themselves, bias included.
//
// "Tencent Hunyuan AI Infra ... Hopper", sec. 1.2, runs the router on tensor
// cores by splitting each operand into a high bf16 part and a residual.  Here
// both fp32 operands are split exactly into three bf16 terms,
//   v = v0 + v1 + v2,  v0 = bf16(v), v1 = bf16(v - v0), v2 = bf16(v - v0 - v1)
// (each difference is exact in fp32, and the three terms carry all 24 bits of
// the significand), and x.w is the sum of the six products whose terms have
// index sum <= 2:
//   x0*w0 + x0*w1 + x1*w0 + x0*w2 + x1*w1 + x2*w0.
// The three dropped products are each below 2^-25 |x*w|, bf16 x bf16 products
// are exact, and the matrix cores accumulate in fp32, so the logits keep fp32
// accuracy while the arithmetic runs at the bf16 rate (16x the fp32 rate, for
// 6x the products).
//
// Workgroup: 64 tokens x 64*EB experts, 8 waves = 2 token halves x 4 expert
// quarters; a wave owns 32 tokens x 16*EB experts (2 x EB blocks of
// v_mfma_f32_16x16x32_bf16).  K advances 32 per stage.  Both fp32 tiles move
// global -> LDS by direct copies (one wave instruction: 8 rows x 128 bytes),
// NS stages deep; chunk c of a row r lands in slot c ^ (r % 8), so the
// fragment reads (16 rows, one 16-byte chunk each per instruction) are
// conflict-free.  The split into bf16 terms happens in registers right before
// the MFMAs.  MFMA operand layout: lane l holds row (A) or column (B) l%16
// and k elements (l/16)*8 .. +7.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void split3(const float4& a, const float4& b, bf16x8 (&pl)[3]) {
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        float r = v[q];
#pragma unroll
        for (int t = 0; t < 3; ++t) {
            const __bf16 h = (__bf16)r;
            pl[t][q] = h;
            r -= (float)h;
        }
    }
}

template <int EB>
struct RouterBf16Cfg {
    static constexpr int XBLK = RBM / 8;                    // 1 KiB copy blocks of x per stage
    static constexpr int BBLK = 64 * EB / 8;                // ... of router rows
    static constexpr int DPW = (XBLK + BBLK) / 8;           // copies per wave per stage
    static constexpr int STAGE = (XBLK + BBLK) * 1024;      // bytes per stage
    static constexpr int NS = (163840 / STAGE) < 6 ? (163840 / STAGE) : 6;
};

// The x-quantisation workgroups of a router launch (blockIdx.y >= S): rows
// r = q, q + nq, ... with q the workgroup's index among the nq of them, each
// row by the whole workgroup (quant_row_wg, 512 threads).
template <int CODE>
__device__ __forceinline__ void router_xquant_rows(const float* __restrict__ x, int T, int H, int S,
                                                   const XQuantJob& xq, float* wmax) {
    const int nq = (gridDim.y - S) * gridDim.x;
    const int nv = H / 4;
    for (int r = (blockIdx.y - S) * gridDim.x + blockIdx.x; r < T; r += nq) {
        const float* xr = x + (int64_t)r * H;
        int8_t* qr = xq.q + (int64_t)r * H;
        if (nv <= 512) quant_row_wg<CODE, 512, 1>(xr, H, xq.opt, qr, xq.scale + r, wmax);
        else if (nv <= 1024) quant_row_wg<CODE, 512, 2>(xr, H, xq.opt, qr, xq.scale + r, wmax);
        else if (nv <= 2048) quant_row_wg<CODE, 512, 4>(xr, H, xq.opt, qr, xq.scale + r, wmax);
        else quant_row_wg<CODE, 512, 8>(xr, H, xq.opt, qr, xq.scale + r, wmax);
        __syncthreads();  // every wave has read wmax before the next row writes it
    }
}

template <int EB>
__global__ __launch_bounds__(512) void router_bf16x3(const float* __restrict__ x,
                                                     const float* __restrict__ wr,
                                                     const float* __restrict__ bias, int T, int H,
                                                     int E, int ksplit_len, int S, XQuantJob xq,
                                                     float* __restrict__ partial) {
    using C = RouterBf16Cfg<EB>;
    constexpr int NS = C::NS, DPW = C::DPW, STAGE = C::STAGE, XBLK = C::XBLK;
    static_assert(NS >= 3, "at least one stage in flight beyond the pair being read");
    __shared__ __attribute__((aligned(1024))) int8_t smem[NS * STAGE];
    if ((int)blockIdx.y >= S) {  // an x-quantisation workgroup (H <= 16384: 8 float4 per thread)
        float* wmax = reinterpret_cast<float*>(smem);
        if (xq.code == CODE_INT8) router_xquant_rows<CODE_INT8>(x, T, H, S, xq, wmax);
        else router_xquant_rows<CODE_FP8>(x, T, H, S, xq, wmax);
        return;
    }
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wt = w >> 2, we = w & 3;
    const int m0 = blockIdx.x * RBM;
    const int kbeg = blockIdx.y * ksplit_len;
    const int nk = ksplit_len / RBK;

    // copy sources: wave w moves blocks w, w+8, ... of every stage; block b < XBLK
    // holds x rows 8b..8b+7, the rest router rows; lane l fetches chunk
    // (l%8) ^ (l/8) of row l/8 of its block.  Rows past T or E repeat the last
    // row (their sums are dropped).
    const int8_t* src[DPW];
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
        const int b = w + 8 * i;
        const int chunk = (lane & 7) ^ (lane >> 3);
        if (b < XBLK) {
            const int t = min(m0 + b * 8 + (lane >> 3), T - 1);
            src[i] = reinterpret_cast<const int8_t*>(x + (int64_t)t * H + kbeg + chunk * 4);
        } else {
            const int e = min((b - XBLK) * 8 + (lane >> 3), E - 1);
            src[i] = reinterpret_cast<const int8_t*>(wr + (int64_t)e * H + kbeg + chunk * 4);
        }
    }
    auto issue = [&](int ks) {
        const int8_t* stage = smem + (ks % NS) * STAGE;
#pragma unroll
        for (int i = 0; i < DPW; ++i) dma16(src[i] + (int64_t)ks * RBK * 4, stage + (w + 8 * i) * 1024);
    };
    // Fragments: NF = 2 + EB per stage (A rows of this wave's two 16-token
    // blocks, then B rows of its EB 16-expert blocks).  Fragment f reads row
    // r's chunks 2*(l/16) and 2*(l/16)+1, at slots chunk ^ (r % 8).
    constexpr int NF = 2 + EB;
    const int frow = lane & 15, fc = (lane >> 4) * 2;
    auto read_raw = [&](int ks, float4 (&raw)[NF][2]) {
        const int8_t* stage = smem + (ks % NS) * STAGE;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const int row = f < 2 ? wt * 32 + f * 16 + frow : (we * EB + (f - 2)) * 16 + frow;
            const int8_t* rp = stage + (f < 2 ? 0 : XBLK * 1024) + row * 128;
            raw[f][0] = *reinterpret_cast<const float4*>(rp + ((fc ^ (row & 7)) * 16));
            raw[f][1] = *reinterpret_cast<const float4*>(rp + (((fc + 1) ^ (row & 7)) * 16));
        }
    };

    v4f acc[2][EB];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < EB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // planes of the stage whose MFMAs run next: pa[i][term], pb[j][term]
    bf16x8 pa[2][3], pb[EB][3];
    // term order: the small products first, x0*w0 last
    constexpr int TA[6] = {1, 0, 2, 0, 1, 0};
    constexpr int TB[6] = {1, 2, 0, 1, 0, 0};
    // Stage ks's MFMAs (six terms) run from pa/pb while stage ks+1's fragments
    // (NEXT) come in from LDS and are split, one fragment after each term.
    auto step = [&](int ks_next, auto next_tag) {
        constexpr bool NEXT = decltype(next_tag)::value;
        float4 raw[NF][2];
        bf16x8 na[2][3], nb[EB][3];
        if (NEXT) read_raw(ks_next, raw);
#pragma unroll
        for (int tm = 0; tm < 6; ++tm) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < EB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[i][TA[tm]], pb[j][TB[tm]],
                                                                        acc[i][j], 0, 0, 0);
            if (NEXT && tm < NF) {
                if (tm < 2) split3(raw[tm][0], raw[tm][1], na[tm]);
                else split3(raw[tm][0], raw[tm][1], nb[tm < 2 ? 0 : tm - 2]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (NEXT) {
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                pa[0][t] = na[0][t];
                pa[1][t] = na[1][t];
#pragma unroll
                for (int j = 0; j < EB; ++j) pb[j][t] = nb[j][t];
            }
        }
    };

    // prologue: NS-1 stages in flight, stage 0 split into pa/pb
    int issued = 0;
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (s < nk) {
            issue(s);
            ++issued;
        }
    if (issued == NS - 1) wait_vmcnt<(NS - 2) * DPW>();
    else wait_vmcnt<0>();
    barrier_nofence();
    {
        float4 raw[NF][2];
        read_raw(0, raw);
        split3(raw[0][0], raw[0][1], pa[0]);
        split3(raw[1][0], raw[1][1], pa[1]);
#pragma unroll
        for (int j = 0; j < EB; ++j) split3(raw[2 + j][0], raw[2 + j][1], pb[j]);
    }
    int ks = 0;
    // steady state: stage ks+1 landed (NS-3 newer stages may still fly); the
    // barrier also retires every wave's reads of the slot refilled next
    for (; ks + NS - 1 < nk; ++ks) {
        wait_vmcnt<(NS - 3) * DPW>();
        barrier_nofence();
        issue(ks + NS - 1);
        step(ks + 1, std::true_type{});
    }
    // drain: every stage is issued
    wait_vmcnt<0>();
    barrier_nofence();
    for (; ks + 1 < nk; ++ks) step(ks + 1, std::true_type{});
    step(0, std::false_type{});

    float* out = partial + (int64_t)blockIdx.y * T * E;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < EB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = m0 + wt * 32 + i * 16 + (lane >> 4) * 4 + r;
                const int e = (we * EB + j) * 16 + (lane & 15);
                // a single split writes the finished logits (bias added once)
                if (t < T && e < E)
                    out[(int64_t)t * E + e] = (bias && S == 1) ? acc[i][j][r] + bias[e] : acc[i][j][r];
            }
}

// The same product with the router weights split ahead of the GEMM.  In the
// kernel above each wave splits the router rows it multiplies, and the two
// token halves split the same rows: two thirds of its vector work.  For many
// tokens the weights are split once per call by router_w_planes into three
// bf16 planes laid out in MFMA fragment order, and router_planes copies those
// straight into LDS, so the GEMM splits only its activations.
//
// Plane layout: fragment (ks, b, p) = 1 KiB at ((ks * NEB + b) * 3 + p) * 1024
// for k-stage ks (32 of H), 16-expert block b (NEB blocks, padded with zero
// rows to a whole expert tile) and term p; lane l's 16 bytes are the eight
// bf16 terms of expert 16b + l%16, k = 32ks + (l/16)*8 .. +7.
__global__ __launch_bounds__(256) void router_w_planes(const float* __restrict__ wr, int E, int H, int NEB,
                                                       int8_t* __restrict__ planes) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one lane of one (ks, b)
    const int64_t n = (int64_t)(H / RBK) * NEB * 64;
    if (i >= n) return;
    const int lane = (int)(i & 63);
    const int64_t kb = i >> 6;  // ks * NEB + b
    const int b = (int)(kb % NEB), ks = (int)(kb / NEB);
    const int e = b * 16 + (lane & 15);
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), c = a;
    if (e < E) {
        const float* src = wr + (int64_t)e * H + ks * RBK + (lane >> 4) * 8;
        a = *reinterpret_cast<const float4*>(src);
        c = *reinterpret_cast<const float4*>(src + 4);
    }
    bf16x8 pl[3];
    split3(a, c, pl);
#pragma unroll
    for (int q = 0; q < 3; ++q)
        *reinterpret_cast<bf16x8*>(planes + (kb * 3 + q) * 1024 + lane * 16) = pl[q];
}

// Workgroup: 128 tokens x 32*EB experts, 8 waves = 4 token quarters x 2
// expert halves; a wave owns 32 tokens x 16*EB experts (2 x EB blocks of
// v_mfma_f32_16x16x32_bf16), as above.  blockIdx.x names the (token tile,
// expert tile) pair, the expert tiles of a token tile on one XCD (one grid
// dimension, as the token tiles can exceed the 65535 limit of the others),
// blockIdx.y the split of H.  A stage holds the
// activation tile (16 copy blocks of 8 rows, swizzled as above) and the
// expert tile's 6*EB plane fragments, padded with repeat copies to a whole
// number of blocks per wave (the repeats land in slots nobody reads).
template <int EB>
struct RouterPlanesCfg {
    static constexpr int XBLK = 16;
    static constexpr int WBLK = 6 * EB;
    static constexpr int NBLK = (XBLK + WBLK + 7) / 8 * 8;
    static constexpr int DPW = NBLK / 8;
    static constexpr int STAGE = NBLK * 1024;
    static constexpr int NS = (163840 / STAGE) < 6 ? (163840 / STAGE) : 6;
};

template <int EB>
__global__ __launch_bounds__(512) void router_planes(const float* __restrict__ x,
                                                     const int8_t* __restrict__ planes,
                                                     const float* __restrict__ bias, int T, int H,
                                                     int E, int NEB, int ksplit_len,
                                                     float* __restrict__ partial) {
    using C = RouterPlanesCfg<EB>;
    constexpr int NS = C::NS, DPW = C::DPW, STAGE = C::STAGE, XBLK = C::XBLK, WBLK = C::WBLK;
    static_assert(NS >= 3, "at least one stage in flight beyond the pair being read");
    __shared__ __attribute__((aligned(1024))) int8_t smem[NS * STAGE];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wt = w >> 1, we = w & 1;
    const int etiles = NEB / (2 * EB);
    // With several expert tiles, the tiles of one token tile (which read the
    // same activation rows) go to one XCD, so the rows come from HBM once and
    // from that XCD's L2 after: workgroup b runs on XCD b % 8, and slot b / 8
    // of XCD x takes token tile (slot / etiles) * 8 + x, expert tile
    // slot % etiles (token tiles past the end exit).
    int tt = (int)blockIdx.x, e_tile = 0;
    if (etiles > 1) {
        const int slot = (int)(blockIdx.x >> 3);
        tt = (slot / etiles) * 8 + (int)(blockIdx.x & 7);
        e_tile = slot % etiles;
        if (tt * 128 >= T) return;
    }
    const int m0 = tt * 128;
    const int kbeg = blockIdx.y * ksplit_len;
    const int nk = ksplit_len / RBK, ks0 = kbeg / RBK;

    // copy sources and their per-stage strides
    const int8_t* src[DPW];
    int64_t stride[DPW];
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
        const int b = w + 8 * i;
        if (b < XBLK) {
            const int chunk = (lane & 7) ^ (lane >> 3);
            const int t = min(m0 + b * 8 + (lane >> 3), T - 1);
            src[i] = reinterpret_cast<const int8_t*>(x + (int64_t)t * H + kbeg + chunk * 4);
            stride[i] = RBK * 4;
        } else {
            const int j = (b < XBLK + WBLK ? b : XBLK) - XBLK;  // padding repeats fragment 0
            const int64_t frag = ((int64_t)ks0 * NEB + e_tile * 2 * EB + j / 3) * 3 + j % 3;
            src[i] = planes + frag * 1024 + lane * 16;
            stride[i] = (int64_t)NEB * 3 * 1024;
        }
    }
    auto issue = [&](int ks) {
        const int8_t* stage = smem + (ks % NS) * STAGE;
#pragma unroll
        for (int i = 0; i < DPW; ++i) dma16(src[i] + (int64_t)ks * stride[i], stage + (w + 8 * i) * 1024);
    };
    const int frow = lane & 15, fc = (lane >> 4) * 2;
    auto read_x = [&](int ks, float4 (&raw)[2][2]) {
        const int8_t* stage = smem + (ks % NS) * STAGE;
#pragma unroll
        for (int f = 0; f < 2; ++f) {
            const int row = wt * 32 + f * 16 + frow;
            const int8_t* rp = stage + row * 128;
            raw[f][0] = *reinterpret_cast<const float4*>(rp + ((fc ^ (row & 7)) * 16));
            raw[f][1] = *reinterpret_cast<const float4*>(rp + (((fc + 1) ^ (row & 7)) * 16));
        }
    };
    auto read_w = [&](int ks, bf16x8 (&pb)[EB][3]) {
        const int8_t* stage = smem + (ks % NS) * STAGE + XBLK * 1024;
#pragma unroll
        for (int j = 0; j < EB; ++j)
#pragma unroll
            for (int q = 0; q < 3; ++q)
                pb[j][q] = *reinterpret_cast<const bf16x8*>(stage + ((we * EB + j) * 3 + q) * 1024 + lane * 16);
    };

    v4f acc[2][EB];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < EB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    bf16x8 pa[2][3], pb[EB][3];
    constexpr int TA[6] = {1, 0, 2, 0, 1, 0};
    constexpr int TB[6] = {1, 2, 0, 1, 0, 0};
    auto step = [&](int ks_next, auto next_tag) {
        constexpr bool NEXT = decltype(next_tag)::value;
        float4 raw[2][2];
        bf16x8 na[2][3], nb[EB][3];
        if (NEXT) {
            read_x(ks_next, raw);
            read_w(ks_next, nb);
        }
#pragma unroll
        for (int tm = 0; tm < 6; ++tm) {
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < EB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pa[i][TA[tm]], pb[j][TB[tm]],
                                                                        acc[i][j], 0, 0, 0);
            if (NEXT && tm < 2) split3(raw[tm][0], raw[tm][1], na[tm]);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (NEXT) {
#pragma unroll
            for (int t = 0; t < 3; ++t) {
                pa[0][t] = na[0][t];
                pa[1][t] = na[1][t];
#pragma unroll
                for (int j = 0; j < EB; ++j) pb[j][t] = nb[j][t];
            }
        }
    };

    int issued = 0;
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
        if (s < nk) {
            issue(s);
            ++issued;
        }
    if (issued == NS - 1) wait_vmcnt<(NS - 2) * DPW>();
    else wait_vmcnt<0>();
    barrier_nofence();
    {
        float4 raw[2][2];
        read_x(0, raw);
        read_w(0, pb);
        split3(raw[0][0], raw[0][1], pa[0]);
        split3(raw[1][0], raw[1][1], pa[1]);
    }
    int ks = 0;
    for (; ks + NS - 1 < nk; ++ks) {
        wait_vmcnt<(NS - 3) * DPW>();
        barrier_nofence();
        issue(ks + NS - 1);
        step(ks + 1, std::true_type{});
    }
    wait_vmcnt<0>();
    barrier_nofence();
    for (; ks + 1 < nk; ++ks) step(ks + 1, std::true_type{});
    step(0, std::false_type{});

    float* out = partial + (int64_t)blockIdx.y * T * E;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < EB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = m0 + wt * 32 + i * 16 + (lane >> 4) * 4 + r;
                const int e = (e_tile * 2 * EB + we * EB + j) * 16 + (lane & 15);
                if (t < T && e < E)
                    out[(int64_t)t * E + e] = (bias && gridDim.y == 1) ? acc[i][j][r] + bias[e] : acc[i][j][r];
            }
}

// logits[t][e] = (sum of the S split partials, in split order) + bias[e]
__global__ __launch_bounds__(256) void router_reduce(const float* __restrict__ partial, int S,
                                                     const float* __restrict__ bias, int T, int E,
                                                     float* __restrict__ logits) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n = (int64_t)T * E;
    if (i >= n) return;
    // loads are issued sixteen at a time so their latencies overlap; the sum
    // itself still runs in split order
    float v = 0.0f;
    int sp = 0;
    for (; sp + 16 <= S; sp += 16) {
        float u[16];
#pragma unroll
        for (int q = 0; q < 16; ++q) u[q] = partial[(int64_t)(sp + q) * n + i];
#pragma unroll
        for (int q = 0; q < 16; ++q) v += u[q];
    }
    for (; sp < S; ++sp) v += partial[(int64_t)sp * n + i];
    if (bias) v += bias[i % E];
    logits[i] = v;
}

// Per 64-token chunk: top-k per token by wave arg-max rounds (ties to the
// lower index), the renormalised softmax weights, and the rank of each
// assignment among the chunk's tokens routed to the same expert (a 64-bit
// token mask per expert in LDS).  With a single chunk (FUSED) the same
// workgroup also produces the expert counts, segment offsets, m-tile
// prefixes and the sorted assignment list, saving three launches.
template <bool FUSED>
__global__ __launch_bounds__(TOPK_THREADS) void topk_count(
    const float* __restrict__ logits, int T, int E, int k, int nchunks, int32_t* __restrict__ ids,
    float* __restrict__ wts, int32_t* __restrict__ rank, int32_t* __restrict__ chunk_counts,
    int32_t* __restrict__ expert_counts, int32_t* __restrict__ offsets, int bm,
    int32_t* __restrict__ mt_prefix, MtInfo* __restrict__ mt_info, int32_t* __restrict__ tile_ctr,
    int32_t* __restrict__ sorted_assign, int32_t* __restrict__ xcd_bounds, int ntv_gu, int ntv_dn) {
    constexpr int NWAVE = TOPK_THREADS / 64;
    constexpr int TPW = ROUTE_CHUNK / NWAVE;  // tokens per wave
    __shared__ int ids_s[ROUTE_CHUNK * MAX_TOPK];
    __shared__ float val_s[ROUTE_CHUNK * MAX_TOPK];
    __shared__ unsigned long long mask[MAX_EXPERTS];
    __shared__ int off_s[MAX_EXPERTS];
    __shared__ int scan_lds[NWAVE];
    __shared__ RankedLds ranked_lds[1];  // used by the single-chunk launch
    const int c = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int t0 = c * ROUTE_CHUNK;
    const int nt = min(ROUTE_CHUNK, T - t0);
    for (int e = tid; e < E; e += TOPK_THREADS) mask[e] = 0ull;

    // the wave's tokens w, w+NWAVE, ...: their logit rows are loaded together
    // (lane l holds experts l, l+64, l+128, l+192)
    float vall[TPW][4];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int t = t0 + min(w + NWAVE * u, nt - 1);
        const float* lrow = logits + (int64_t)t * E;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane + 64 * i;
            vall[u][i] = (e < E) ? lrow[min(e, E - 1)] : -INFINITY;
        }
    }
    // the wave's tokens are w + NWAVE*u: u < n_valid of them exist
    const int n_valid = w < nt ? (nt - 1 - w) / NWAVE + 1 : 0;
    wave_topk_n<TPW>(vall, lane, E, k, n_valid, ids_s + w * k, val_s + w * k, NWAVE * k);
    __syncthreads();
    for (int tl = tid; tl < nt; tl += TOPK_THREADS) {
        const int t = t0 + tl;
        float wj[MAX_TOPK];
        topk_weights(val_s + tl * k, k, wj);
        for (int j = 0; j < k; ++j) {
            ids[(int64_t)t * k + j] = ids_s[tl * k + j];
            wts[(int64_t)t * k + j] = wj[j];
        }
    }
    for (int al = tid; al < nt * k; al += TOPK_THREADS) atomicOr(&mask[ids_s[al]], 1ull << (al / k));
    __syncthreads();
    if (!FUSED) {
        for (int al = tid; al < nt * k; al += TOPK_THREADS) {
            const int tl = al / k;
            rank[(int64_t)t0 * k + al] = __popcll(mask[ids_s[al]] & ((1ull << tl) - 1ull));
        }
        for (int e = tid; e < E; e += TOPK_THREADS) chunk_counts[(int64_t)e * nchunks + c] = __popcll(mask[e]);
    } else {
        // single chunk: counts -> offsets -> m-tile prefixes -> sorted list
        const int cnt = tid < E ? __popcll(mask[tid]) : 0;
        // one scan for both prefixes: rows in the low 16 bits, m-tiles in the
        // high 16 (a single chunk holds at most 64*8 rows)
        int tot;
        const int both = block_exclusive_scan<NWAVE>(cnt | (((cnt + bm - 1) / bm) << 16), &tot, scan_lds);
        const int off = both & 0xffff, m1 = both >> 16;
        const int tot0 = tot & 0xffff, tot1 = tot >> 16;
        if (tid < E) {
            expert_counts[tid] = cnt;
            offsets[tid] = off;
            mt_prefix[tid] = m1;
            off_s[tid] = off;
        }
        if (tid == 0) {
            offsets[E] = tot0;
            mt_prefix[E] = tot1;
        }
        if (bm == SKINNY_BM) {  // the skinny GEMMs take the m-tiles in expert order
            if (tid < E) write_mt_info(mt_info, tid, m1, (cnt + bm - 1) / bm, off, off + cnt);
        } else {
            write_ranked_tables<TOPK_THREADS>(cnt, off, (cnt + bm - 1) / bm, E, mt_info, xcd_bounds, ntv_gu,
                                              ntv_dn, ranked_lds[0]);
        }
        if (tid < TILE_CTR_COUNT) tile_ctr[tid * TILE_CTR_STRIDE] = 0;
        __syncthreads();
        for (int al = tid; al < nt * k; al += TOPK_THREADS) {
            const int tl = al / k;
            const int e = ids_s[al];
            const int pos = off_s[e] + __popcll(mask[e] & ((1ull << tl) - 1ull));
            sorted_assign[pos] = (int32_t)al;  // t0 == 0
        }
    }
}

__global__ __launch_bounds__(256) void chunk_scan(const int32_t* __restrict__ chunk_counts,
                                                  int nchunks, int32_t* __restrict__ chunk_base,
                                                  int32_t* __restrict__ expert_counts) {
    __shared__ int lds[4];
    const int e = blockIdx.x, tid = threadIdx.x;
    const int32_t* cc = chunk_counts + (int64_t)e * nchunks;
    int32_t* cb = chunk_base + (int64_t)e * nchunks;
    const int per = (nchunks + 255) / 256;
    const int beg = min(tid * per, nchunks), end = min(beg + per, nchunks);
    int local = 0;
    for (int c = beg; c < end; ++c) local += cc[c];
    int total;
    int run = block_exclusive_scan<4>(local, &total, lds);
    for (int c = beg; c < end; ++c) {
        cb[c] = run;
        run += cc[c];
    }
    if (tid == 0) expert_counts[e] = total;
}

__global__ __launch_bounds__(256) void finalize(const int32_t* __restrict__ expert_counts, int E,
                                                int bm, int32_t* __restrict__ offsets,
                                                int32_t* __restrict__ mt_prefix,
                                                MtInfo* __restrict__ mt_info,
                                                int32_t* __restrict__ tile_ctr,
                                                int32_t* __restrict__ xcd_bounds, int ntv_gu,
                                                int ntv_dn) {
    __shared__ int lds[4];
    __shared__ RankedLds ranked_lds;
    const int e = threadIdx.x;
    const int cnt = e < E ? expert_counts[e] : 0;
    int tot0, tot1;
    const int off = block_exclusive_scan<4>(cnt, &tot0, lds);
    const int m1 = block_exclusive_scan<4>((cnt + bm - 1) / bm, &tot1, lds);
    if (e < E) {
        offsets[e] = off;
        mt_prefix[e] = m1;
    }
    if (bm == SKINNY_BM) {  // the skinny GEMMs take the m-tiles in expert order
        if (e < E) write_mt_info(mt_info, e, m1, (cnt + bm - 1) / bm, off, off + cnt);
    } else {
        write_ranked_tables<256>(cnt, off, (cnt + bm - 1) / bm, E, mt_info, xcd_bounds, ntv_gu, ntv_dn,
                                 ranked_lds);
    }
    if (e == 0) {
        offsets[E] = tot0;
        mt_prefix[E] = tot1;
    }
    if (e < TILE_CTR_COUNT) tile_ctr[e * TILE_CTR_STRIDE] = 0;
}

__global__ __launch_bounds__(256) void scatter(const int32_t* __restrict__ ids, int T, int k,
                                               int nchunks, const int32_t* __restrict__ offsets,
                                               const int32_t* __restrict__ chunk_base,
                                               const int32_t* __restrict__ rank,
                                               int32_t* __restrict__ sorted_assign) {
    const int c = blockIdx.x;
    for (int al = threadIdx.x; al < ROUTE_CHUNK * k; al += 256) {
        const int tl = al / k, j = al - tl * k;
        const int t = c * ROUTE_CHUNK + tl;
        if (t >= T) continue;
        const int64_t a = (int64_t)t * k + j;
        const int e = ids[a];
        const int pos = offsets[e] + chunk_base[(int64_t)e * nchunks + c] + rank[a];
        sorted_assign[pos] = (int32_t)a;
    }
}

}  // namespace

// Token counts from which the router weights are split ahead of the GEMM (the
// extra launch pays once the GEMM runs many token tiles).
constexpr int ROUTER_PLANES_MIN_T = 2048;

static int router_planes_eb(int E) { return E > 64 ? 4 : (E > 32 ? 2 : 1); }

RouterPlan router_plan(int T, int E, int H) {
    const bool planes = T >= ROUTER_PLANES_MIN_T;
    // enough workgroups to fill the GPU, at least 8 stages (256 of H) per split
    // (4 when there are few token tiles: each stage of a split costs about one
    // memory round trip); the split count divides the stage count H/32
    int tiles = (T + RBM - 1) / RBM;
    size_t bytes = 0;
    if (planes) {
        const int eb = router_planes_eb(E), etiles = (E + 32 * eb - 1) / (32 * eb);
        tiles = (T + 127) / 128 * etiles;
        bytes = (size_t)H * etiles * 32 * eb * 6;
    }
    const int stages = H / RBK;
    int s = 1;
    const int min_stages = tiles >= 16 ? 8 : 4;
    while (tiles * s < 256 && stages % (2 * s) == 0 && stages / (2 * s) >= min_stages) s *= 2;
    return RouterPlan{s, bytes};
}

hipError_t launch_route(const RouteInputs& in, const RouteBuffers& b, hipStream_t s) {
    const int T = in.T, E = in.E, k = in.k, H = in.H, S = in.splits;
    const int nchunks = (T + ROUTE_CHUNK - 1) / ROUTE_CHUNK;
    MtInfo* mt_info = reinterpret_cast<MtInfo*>(b.mt_info);
    float* out = (S == 1) ? b.logits : b.partial;
    const float *xx = in.x, *wr = in.router_w, *rb = in.router_b;
    const bool xquant = in.xq.q != nullptr;
    if (xquant && (b.wplanes || T > ROUTER_XQUANT_MAX_T || H % 4 != 0 || H > 16384))
        return hipErrorInvalidValue;
    if (b.wplanes) {
        const int eb = router_planes_eb(E), etiles = (E + 32 * eb - 1) / (32 * eb), neb = etiles * 2 * eb;
        int8_t* planes = static_cast<int8_t*>(b.wplanes);
        const int64_t n = (int64_t)(H / RBK) * neb * 64;
        router_w_planes<<<dim3((unsigned)((n + 255) / 256)), 256, 0, s>>>(wr, E, H, neb, planes);
        const int ttiles = (T + 127) / 128;
        const dim3 grid((unsigned)(etiles > 1 ? etiles * ((ttiles + 7) / 8 * 8) : ttiles), S);
        if (eb == 1) router_planes<1><<<grid, 512, 0, s>>>(xx, planes, rb, T, H, E, neb, H / S, out);
        else if (eb == 2) router_planes<2><<<grid, 512, 0, s>>>(xx, planes, rb, T, H, E, neb, H / S, out);
        else router_planes<4><<<grid, 512, 0, s>>>(xx, planes, rb, T, H, E, neb, H / S, out);
    } else {
        // S router splits per token tile, then (with the x job) enough rows of
        // quantisation workgroups for one x row each
        const int tiles = (T + RBM - 1) / RBM;
        const dim3 grid(tiles, S + (xquant ? (T + tiles - 1) / tiles : 0));
        const int eb = (E + 63) / 64;
        if (eb == 1) router_bf16x3<1><<<grid, 512, 0, s>>>(xx, wr, rb, T, H, E, H / S, S, in.xq, out);
        else if (eb == 2) router_bf16x3<2><<<grid, 512, 0, s>>>(xx, wr, rb, T, H, E, H / S, S, in.xq, out);
        else if (eb == 3) router_bf16x3<3><<<grid, 512, 0, s>>>(xx, wr, rb, T, H, E, H / S, S, in.xq, out);
        else router_bf16x3<4><<<grid, 512, 0, s>>>(xx, wr, rb, T, H, E, H / S, S, in.xq, out);
    }
    if (S > 1) {
        const int64_t n = (int64_t)T * E;
        router_reduce<<<dim3((unsigned)((n + 255) / 256)), 256, 0, s>>>(b.partial, S, in.router_b, T, E,
                                                                          b.logits);
    }
    if (nchunks == 1) {
        topk_count<true><<<1, TOPK_THREADS, 0, s>>>(b.logits, T, E, k, nchunks, b.topk_ids, b.topk_w, b.rank,
                                                    b.chunk_counts, b.expert_counts, b.expert_offsets, in.bm,
                                                    b.mt_prefix, mt_info, b.tile_ctr, b.sorted_assign,
                                                    b.xcd_bounds, in.ntv_gu, in.ntv_dn);
        return hipGetLastError();
    }
    topk_count<false><<<nchunks, TOPK_THREADS, 0, s>>>(b.logits, T, E, k, nchunks,
                                                       b.topk_ids, b.topk_w, b.rank, b.chunk_counts,
                                                       b.expert_counts, b.expert_offsets, in.bm, b.mt_prefix,
                                                       mt_info, b.tile_ctr, b.sorted_assign, b.xcd_bounds,
                                                       in.ntv_gu, in.ntv_dn);
    chunk_scan<<<E, 256, 0, s>>>(b.chunk_counts, nchunks, b.chunk_base, b.expert_counts);
    finalize<<<1, 256, 0, s>>>(b.expert_counts, E, in.bm, b.expert_offsets, b.mt_prefix, mt_info,
                               b.tile_ctr, b.xcd_bounds, in.ntv_gu, in.ntv_dn);
    scatter<<<nchunks, 256, 0, s>>>(b.topk_ids, T, k, nchunks, b.expert_offsets, b.chunk_base,
                                    b.rank, b.sorted_assign);
    return hipGetLastError();
}

}  // namespace w8a8
