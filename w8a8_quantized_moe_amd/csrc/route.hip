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
//   router_partial  fp32 MFMA GEMM (v_mfma_f32_16x16x4_f32), 64x64 tiles,
//                   optionally split along H into S partial sums so small
//                   token counts still fill the GPU;
//   topk_count      per 64-token chunk: sums the S partials in a fixed order
//                   (deterministic), adds the bias, picks the top-k by wave
//                   arg-max rounds (ties to the lower index), computes the
//                   renormalised softmax weights, and ranks each assignment
//                   among the chunk's tokens routed to the same expert with a
//                   64-bit token mask per expert in LDS;
//   chunk_scan      per expert: exclusive scan of its per-chunk counts;
//   finalize        exclusive scan over experts -> segment offsets, and the
//                   prefix of m-tiles per expert for the grouped GEMMs;
//   scatter         sorted_assign[offset[e] + chunk_base + rank] = t*k + j.
// The resulting order inside a segment is ascending token order.
#include "internal.h"

namespace w8a8 {
namespace {

constexpr int RBM = 64, RBN = 64, RBK = 32, RPAD = 16;

// partial[s][t][e] = sum over h in split s of x[t][h] * wr[e][h]
__global__ __launch_bounds__(256) void router_partial(const float* __restrict__ x,
                                                      const float* __restrict__ wr, int T, int H,
                                                      int E, int ksplit_len,
                                                      float* __restrict__ partial) {
    __shared__ float As[2][RBK][RBM + RPAD];
    __shared__ float Bs[2][RBK][RBN + RPAD];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w >> 1, wn = w & 1;
    const int m0 = blockIdx.x * RBM, n0 = blockIdx.y * RBN;
    const int split = blockIdx.z;
    const int kbeg = split * ksplit_len;
    const int nstage = ksplit_len / RBK;

    float4 ra[2], rb[2];
    const float4 zero4 = make_float4(0.f, 0.f, 0.f, 0.f);
    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + i * 256;
            const int row = c >> 3, k4 = c & 7;
            const int t = m0 + row, e = n0 + row;
            ra[i] = (t < T) ? *reinterpret_cast<const float4*>(x + (int64_t)t * H + k0 + k4 * 4) : zero4;
            rb[i] = (e < E) ? *reinterpret_cast<const float4*>(wr + (int64_t)e * H + k0 + k4 * 4) : zero4;
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int c = tid + i * 256;
            const int row = c >> 3, k4 = c & 7;
            As[buf][k4 * 4 + 0][row] = ra[i].x;
            As[buf][k4 * 4 + 1][row] = ra[i].y;
            As[buf][k4 * 4 + 2][row] = ra[i].z;
            As[buf][k4 * 4 + 3][row] = ra[i].w;
            Bs[buf][k4 * 4 + 0][row] = rb[i].x;
            Bs[buf][k4 * 4 + 1][row] = rb[i].y;
            Bs[buf][k4 * 4 + 2][row] = rb[i].z;
            Bs[buf][k4 * 4 + 3][row] = rb[i].w;
        }
    };

    v4f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    gload(kbeg);
    sstore(0);
    __syncthreads();
    for (int st = 0; st < nstage; ++st) {
        const int buf = st & 1;
        if (st + 1 < nstage) gload(kbeg + (st + 1) * RBK);
#pragma unroll
        for (int kk = 0; kk < RBK / 4; ++kk) {
            const int kr = kk * 4 + (lane >> 4);
            const float a0 = As[buf][kr][wm * 32 + (lane & 15)];
            const float a1 = As[buf][kr][wm * 32 + 16 + (lane & 15)];
            const float b0 = Bs[buf][kr][wn * 32 + (lane & 15)];
            const float b1 = Bs[buf][kr][wn * 32 + 16 + (lane & 15)];
            acc[0][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b0, acc[0][0], 0, 0, 0);
            acc[0][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a0, b1, acc[0][1], 0, 0, 0);
            acc[1][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b0, acc[1][0], 0, 0, 0);
            acc[1][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(a1, b1, acc[1][1], 0, 0, 0);
        }
        if (st + 1 < nstage) sstore(buf ^ 1);
        __syncthreads();
    }
    float* out = partial + (int64_t)split * T * E;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = m0 + wm * 32 + i * 16 + (lane >> 4) * 4 + r;
                const int e = n0 + wn * 32 + j * 16 + (lane & 15);
                if (t < T && e < E) out[(int64_t)t * E + e] = acc[i][j][r];
            }
}

__global__ __launch_bounds__(256) void topk_count(const float* __restrict__ partial, int S,
                                                  const float* __restrict__ bias, int T, int E, int k,
                                                  int nchunks, float* __restrict__ logits,
                                                  int32_t* __restrict__ ids, float* __restrict__ wts,
                                                  int32_t* __restrict__ rank,
                                                  int32_t* __restrict__ chunk_counts) {
    __shared__ int ids_s[ROUTE_CHUNK * MAX_TOPK];
    __shared__ unsigned long long mask[MAX_EXPERTS];
    const int c = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int e = tid; e < E; e += 256) mask[e] = 0ull;

    for (int tl = w; tl < ROUTE_CHUNK; tl += 4) {
        const int t = c * ROUTE_CHUNK + tl;
        if (t >= T) break;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane + 64 * i;
            if (e < E) {
                float s = 0.0f;
                for (int sp = 0; sp < S; ++sp) s += partial[((int64_t)sp * T + t) * E + e];
                if (bias) s += bias[e];
                v[i] = s;
                logits[(int64_t)t * E + e] = s;
            } else {
                v[i] = -INFINITY;
            }
        }
        float sel_v[MAX_TOPK];
        int sel_i[MAX_TOPK];
        for (int j = 0; j < k; ++j) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = lane + 64 * i;
                // lanes hold experts in ascending order: strict '>' keeps the lower index
                if (e < E && (v[i] > bv || bi == 0x7fffffff)) {
                    bv = v[i];
                    bi = e;
                }
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const float ov = __shfl_xor(bv, o, 64);
                const int oi = __shfl_xor(bi, o, 64);
                if (ov > bv || (ov == bv && oi < bi)) {
                    bv = ov;
                    bi = oi;
                }
            }
            sel_v[j] = bv;
            sel_i[j] = bi;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (lane + 64 * i == bi) v[i] = -INFINITY;
        }
        if (lane == 0) {
            // softmax over the picked logits == full softmax renormalised over them
            const float m = sel_v[0];
            float ex[MAX_TOPK];
            float sum = 0.0f;
            for (int j = 0; j < k; ++j) {
                ex[j] = expf(sel_v[j] - m);
                sum += ex[j];
            }
            for (int j = 0; j < k; ++j) {
                ids[(int64_t)t * k + j] = sel_i[j];
                wts[(int64_t)t * k + j] = ex[j] / sum;
                ids_s[tl * k + j] = sel_i[j];
            }
        }
    }
    __syncthreads();
    for (int al = tid; al < ROUTE_CHUNK * k; al += 256) {
        const int tl = al / k;
        if (c * ROUTE_CHUNK + tl < T) atomicOr(&mask[ids_s[al]], 1ull << tl);
    }
    __syncthreads();
    for (int al = tid; al < ROUTE_CHUNK * k; al += 256) {
        const int tl = al / k, j = al - tl * k;
        const int t = c * ROUTE_CHUNK + tl;
        if (t < T) {
            const int e = ids_s[al];
            rank[(int64_t)t * k + j] = __popcll(mask[e] & ((1ull << tl) - 1ull));
        }
    }
    for (int e = tid; e < E; e += 256) chunk_counts[(int64_t)e * nchunks + c] = __popcll(mask[e]);
}

// Block-wide exclusive scan of one int per thread (256 threads).
__device__ int block_exclusive_scan(int v, int* total, int* lds /* >= 4 ints */) {
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
    for (int i = 0; i < 4; ++i) {
        if (i < w) base += lds[i];
        tot += lds[i];
    }
    __syncthreads();
    *total = tot;
    return base + incl - v;
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
    int run = block_exclusive_scan(local, &total, lds);
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
    const int off = block_exclusive_scan(cnt, &tot0, lds);
    const int m1 = block_exclusive_scan((cnt + bm_gu - 1) / bm_gu, &tot1, lds);
    const int m2 = block_exclusive_scan((cnt + bm_dn - 1) / bm_dn, &tot2, lds);
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
    const int tiles = ((T + RBM - 1) / RBM) * ((E + RBN - 1) / RBN);
    const int stages = H / RBK;
    int s = 1;
    while (tiles * s < 512 && (stages % (2 * s)) == 0 && stages / (2 * s) >= 2) s *= 2;
    return s;
}

hipError_t launch_route(const RouteInputs& in, const RouteBuffers& b, hipStream_t s) {
    const int T = in.T, E = in.E, k = in.k, H = in.H, S = in.splits;
    const int nchunks = (T + ROUTE_CHUNK - 1) / ROUTE_CHUNK;
    {
        const dim3 grid((T + RBM - 1) / RBM, (E + RBN - 1) / RBN, S);
        router_partial<<<grid, 256, 0, s>>>(in.x, in.router_w, T, H, E, H / S, b.partial);
    }
    topk_count<<<nchunks, 256, 0, s>>>(b.partial, S, in.router_b, T, E, k, nchunks, b.logits,
                                       b.topk_ids, b.topk_w, b.rank, b.chunk_counts);
    chunk_scan<<<E, 256, 0, s>>>(b.chunk_counts, nchunks, b.chunk_base, b.expert_counts);
    finalize<<<1, 256, 0, s>>>(b.expert_counts, E, in.bm_gu, in.bm_dn, b.expert_offsets,
                               b.mt_prefix_gu, b.mt_prefix_dn);
    scatter<<<nchunks, 256, 0, s>>>(b.topk_ids, T, k, nchunks, b.expert_offsets, b.chunk_base,
                                    b.rank, b.sorted_assign);
    return hipGetLastError();
}

}  // namespace w8a8
