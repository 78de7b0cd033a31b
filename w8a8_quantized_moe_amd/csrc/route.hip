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
//   router_partial  fp32 MFMA GEMM (v_mfma_f32_16x16x4_f32), 64-token x
//                   all-expert tiles (activations read once), optionally
//                   split along H into S partial sums so small token counts
//                   still fill the GPU;
//   router_reduce   (split only) sums the S partials in split order (a fixed,
//                   deterministic order) and adds the bias;
//   topk_count      per 64-token chunk: picks the top-k by wave arg-max rounds
//                   (ties to the lower index), computes the renormalised
//                   softmax weights, and ranks each assignment among the
//                   chunk's tokens routed to the same expert with a 64-bit
//                   token mask per expert (a single chunk also finishes the
//                   permutation below in the same workgroup);
//   chunk_scan      per expert: exclusive scan of its per-chunk counts;
//   finalize        exclusive scan over experts -> segment offsets, and the
//                   prefix of m-tiles per expert for the grouped GEMMs;
//   scatter         sorted_assign[offset[e] + chunk_base + rank] = t*k + j.
// The resulting order inside a segment is ascending token order.
#include "internal.h"

namespace w8a8 {
namespace {

constexpr int RBM = 64, RBK = 32, RPAD = 4;
constexpr int TOPK_THREADS = 1024;  // 16 waves: 4 tokens of a 64-token chunk each

// partial[s][t][e] = sum over h in split s of x[t][h] * wr[e][h]   (fp32 MFMA);
// with a single split the output is the logits themselves, bias included.
// One workgroup: 64 tokens x all experts (E padded to 64*EB), so the
// activations are read once; wave w owns experts [16*EB*w, 16*EB*(w+1)).
// K advances 32 per stage through a double-buffered, k-major LDS tile.
template <int EB>
__global__ __launch_bounds__(256) void router_partial(const float* __restrict__ x,
                                                      const float* __restrict__ wr,
                                                      const float* __restrict__ bias, int T, int H,
                                                      int E, int ksplit_len,
                                                      float* __restrict__ partial) {
    constexpr int EP = 64 * EB;  // padded expert count
    constexpr int AW = RBM + RPAD, BW = EP + RPAD;
    __shared__ float As[2][RBK][AW];
    __shared__ float Bs[2][RBK][BW];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int m0 = blockIdx.x * RBM;
    const int split = blockIdx.y;
    const int kbeg = split * ksplit_len;
    const int nstage = ksplit_len / RBK;

    // global tile loads: A 64x32 (2 float4 per thread), B EPx32 (2*EB float4 per thread)
    float4 ra0, ra1, rb[2 * EB];
    const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
#define ROUTER_GLOAD(k0)                                                                          \
    do {                                                                                          \
        {                                                                                         \
            const int t_ = m0 + (tid >> 3), t1_ = m0 + ((tid + 256) >> 3);                        \
            ra0 = *reinterpret_cast<const float4*>(x + (int64_t)min(t_, T - 1) * H + (k0) + (tid & 7) * 4); \
            ra1 = *reinterpret_cast<const float4*>(x + (int64_t)min(t1_, T - 1) * H + (k0) + (tid & 7) * 4); \
            if (t_ >= T) ra0 = zero4;                                                             \
            if (t1_ >= T) ra1 = zero4;                                                            \
        }                                                                                         \
        _Pragma("unroll") for (int i = 0; i < 2 * EB; ++i) {                                      \
            const int c_ = tid + i * 256;                                                         \
            const int e_ = c_ >> 3;                                                               \
            rb[i] = *reinterpret_cast<const float4*>(wr + (int64_t)min(e_, E - 1) * H + (k0) + (c_ & 7) * 4); \
            if (e_ >= E) rb[i] = zero4;                                                           \
        }                                                                                         \
    } while (0)
#define ROUTER_SSTORE(buf)                                                                        \
    do {                                                                                          \
        const int k4_ = (tid & 7) * 4, r0_ = tid >> 3, r1_ = (tid + 256) >> 3;                    \
        As[buf][k4_ + 0][r0_] = ra0.x; As[buf][k4_ + 1][r0_] = ra0.y;                             \
        As[buf][k4_ + 2][r0_] = ra0.z; As[buf][k4_ + 3][r0_] = ra0.w;                             \
        As[buf][k4_ + 0][r1_] = ra1.x; As[buf][k4_ + 1][r1_] = ra1.y;                             \
        As[buf][k4_ + 2][r1_] = ra1.z; As[buf][k4_ + 3][r1_] = ra1.w;                             \
        _Pragma("unroll") for (int i = 0; i < 2 * EB; ++i) {                                      \
            const int c_ = tid + i * 256;                                                         \
            const int e_ = c_ >> 3;                                                               \
            Bs[buf][k4_ + 0][e_] = rb[i].x; Bs[buf][k4_ + 1][e_] = rb[i].y;                       \
            Bs[buf][k4_ + 2][e_] = rb[i].z; Bs[buf][k4_ + 3][e_] = rb[i].w;                       \
        }                                                                                         \
    } while (0)

    v4f acc[4][EB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < EB; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    ROUTER_GLOAD(kbeg);
    ROUTER_SSTORE(0);
    __syncthreads();
    for (int st = 0; st < nstage; ++st) {
        const int buf = st & 1;
        if (st + 1 < nstage) ROUTER_GLOAD(kbeg + (st + 1) * RBK);
#pragma unroll
        for (int kk = 0; kk < RBK / 4; ++kk) {
            const int kr = kk * 4 + (lane >> 4);
            float a[4], bb[EB];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[buf][kr][i * 16 + (lane & 15)];
#pragma unroll
            for (int j = 0; j < EB; ++j) bb[j] = Bs[buf][kr][(w * EB + j) * 16 + (lane & 15)];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < EB; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], bb[j], acc[i][j], 0, 0, 0);
        }
        if (st + 1 < nstage) ROUTER_SSTORE(buf ^ 1);
        __syncthreads();
    }
#undef ROUTER_GLOAD
#undef ROUTER_SSTORE
    float* out = partial + (int64_t)split * T * E;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < EB; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = m0 + i * 16 + (lane >> 4) * 4 + r;
                const int e = (w * EB + j) * 16 + (lane & 15);
                // a single split writes the finished logits (bias added once)
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

// Block-wide exclusive scan of one int per thread (NW waves of 64).
template <int NW>
__device__ int block_exclusive_scan(int v, int* total, int* lds /* >= NW ints */) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
    }
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
    int32_t* __restrict__ expert_counts, int32_t* __restrict__ offsets, int bm_gu, int bm_dn,
    int32_t* __restrict__ mt_gu, int32_t* __restrict__ mt_dn, int32_t* __restrict__ sorted_assign) {
    constexpr int NWAVE = TOPK_THREADS / 64;
    constexpr int TPW = ROUTE_CHUNK / NWAVE;  // tokens per wave
    __shared__ int ids_s[ROUTE_CHUNK * MAX_TOPK];
    __shared__ float val_s[ROUTE_CHUNK * MAX_TOPK];
    __shared__ unsigned long long mask[MAX_EXPERTS];
    __shared__ int off_s[MAX_EXPERTS];
    __shared__ int scan_lds[NWAVE];
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
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int tl = w + NWAVE * u;
        if (tl >= nt) break;
        float v0 = vall[u][0], v1 = vall[u][1], v2 = vall[u][2], v3 = vall[u][3];
        // k rounds of a wave arg-max; ties go to the lower expert index
#pragma unroll 1
        for (int j = 0; j < k; ++j) {
            float bv = v0;
            int bi = lane;
            if (v1 > bv) { bv = v1; bi = lane + 64; }
            if (v2 > bv) { bv = v2; bi = lane + 128; }
            if (v3 > bv) { bv = v3; bi = lane + 192; }
            if (bi >= E) bi = 0x7fffffff;  // padding never wins a tie
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const float ov = __shfl_xor(bv, o, 64);
                const int oi = __shfl_xor(bi, o, 64);
                if (ov > bv || (ov == bv && oi < bi)) {
                    bv = ov;
                    bi = oi;
                }
            }
            if (lane == 0) {
                ids_s[tl * k + j] = bi;
                val_s[tl * k + j] = bv;
            }
            if (bi == lane) v0 = -INFINITY;
            if (bi == lane + 64) v1 = -INFINITY;
            if (bi == lane + 128) v2 = -INFINITY;
            if (bi == lane + 192) v3 = -INFINITY;
        }
    }
    __syncthreads();
    // softmax over the picked logits == full softmax renormalised over them;
    // one thread per token, terms summed in pick order
    for (int tl = tid; tl < nt; tl += TOPK_THREADS) {
        const int t = t0 + tl;
        const float mx = val_s[tl * k];
        float z = 0.0f;
        for (int j = 0; j < k; ++j) z += expf(val_s[tl * k + j] - mx);
        for (int j = 0; j < k; ++j) {
            ids[(int64_t)t * k + j] = ids_s[tl * k + j];
            wts[(int64_t)t * k + j] = expf(val_s[tl * k + j] - mx) / z;
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
        int tot0, tot1, tot2;
        const int off = block_exclusive_scan<NWAVE>(cnt, &tot0, scan_lds);
        const int m1 = block_exclusive_scan<NWAVE>((cnt + bm_gu - 1) / bm_gu, &tot1, scan_lds);
        const int m2 = block_exclusive_scan<NWAVE>((cnt + bm_dn - 1) / bm_dn, &tot2, scan_lds);
        if (tid < E) {
            expert_counts[tid] = cnt;
            offsets[tid] = off;
            mt_gu[tid] = m1;
            mt_dn[tid] = m2;
            off_s[tid] = off;
        }
        if (tid == 0) {
            offsets[E] = tot0;
            mt_gu[E] = tot1;
            mt_dn[E] = tot2;
        }
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
                                                int bm_gu, int bm_dn, int32_t* __restrict__ offsets,
                                                int32_t* __restrict__ mt_gu,
                                                int32_t* __restrict__ mt_dn) {
    __shared__ int lds[4];
    const int e = threadIdx.x;
    const int cnt = e < E ? expert_counts[e] : 0;
    int tot0, tot1, tot2;
    const int off = block_exclusive_scan<4>(cnt, &tot0, lds);
    const int m1 = block_exclusive_scan<4>((cnt + bm_gu - 1) / bm_gu, &tot1, lds);
    const int m2 = block_exclusive_scan<4>((cnt + bm_dn - 1) / bm_dn, &tot2, lds);
    if (e < E) {
        offsets[e] = off;
        mt_gu[e] = m1;
        mt_dn[e] = m2;
    }
    if (e == 0) {
        offsets[E] = tot0;
        mt_gu[E] = tot1;
        mt_dn[E] = tot2;
    }
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

int router_splits(int T, int E, int H) {
    (void)E;
    // enough workgroups to fill the GPU, at least 8 stages (256 of H) per split
    // (4 when there are few token tiles: each stage of a split costs about one
    // memory round trip); the split count divides the stage count H/32
    const int tiles = (T + RBM - 1) / RBM;
    const int stages = H / RBK;
    int s = 1;
    const int min_stages = tiles >= 16 ? 8 : 4;
    while (tiles * s < 256 && stages % (2 * s) == 0 && stages / (2 * s) >= min_stages) s *= 2;
    return s;
}

hipError_t launch_route(const RouteInputs& in, const RouteBuffers& b, hipStream_t s) {
    const int T = in.T, E = in.E, k = in.k, H = in.H, S = in.splits;
    const int nchunks = (T + ROUTE_CHUNK - 1) / ROUTE_CHUNK;
    {
        const dim3 grid((T + RBM - 1) / RBM, S);
        const int eb = (E + 63) / 64;
        float* out = (S == 1) ? b.logits : b.partial;
        if (eb == 1) router_partial<1><<<grid, 256, 0, s>>>(in.x, in.router_w, in.router_b, T, H, E, H / S, out);
        else if (eb == 2) router_partial<2><<<grid, 256, 0, s>>>(in.x, in.router_w, in.router_b, T, H, E, H / S, out);
        else if (eb == 3) router_partial<3><<<grid, 256, 0, s>>>(in.x, in.router_w, in.router_b, T, H, E, H / S, out);
        else router_partial<4><<<grid, 256, 0, s>>>(in.x, in.router_w, in.router_b, T, H, E, H / S, out);
    }
    if (S > 1) {
        const int64_t n = (int64_t)T * E;
        router_reduce<<<dim3((unsigned)((n + 255) / 256)), 256, 0, s>>>(b.partial, S, in.router_b, T, E,
                                                                          b.logits);
    }
    if (nchunks == 1) {
        topk_count<true><<<1, TOPK_THREADS, 0, s>>>(b.logits, T, E, k, nchunks, b.topk_ids, b.topk_w, b.rank,
                                           b.chunk_counts, b.expert_counts, b.expert_offsets, in.bm_gu,
                                           in.bm_dn, b.mt_prefix_gu, b.mt_prefix_dn, b.sorted_assign);
        return hipGetLastError();
    }
    topk_count<false><<<nchunks, TOPK_THREADS, 0, s>>>(b.logits, T, E, k, nchunks, b.topk_ids, b.topk_w, b.rank,
                                              b.chunk_counts, b.expert_counts, b.expert_offsets,
                                              in.bm_gu, in.bm_dn, b.mt_prefix_gu, b.mt_prefix_dn,
                                              b.sorted_assign);
    chunk_scan<<<E, 256, 0, s>>>(b.chunk_counts, nchunks, b.chunk_base, b.expert_counts);
    finalize<<<1, 256, 0, s>>>(b.expert_counts, E, in.bm_gu, in.bm_dn, b.expert_offsets,
                               b.mt_prefix_gu, b.mt_prefix_dn);
    scatter<<<nchunks, 256, 0, s>>>(b.topk_ids, T, k, nchunks, b.expert_offsets, b.chunk_base,
                                    b.rank, b.sorted_assign);
    return hipGetLastError();
}

}  // namespace w8a8
