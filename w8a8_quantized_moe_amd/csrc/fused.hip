// The whole MoE layer of a decode-sized batch (T <= 64 tokens) in one
// persistent launch: quantisation and router, top-k and the permutation into
// per-expert segments, the gate-up GEMM, the requantisation of h, the down
// GEMM and the combine.
//
// "Tencent Hunyuan AI Infra ... Hopper", sec. 1.3: a single persistent
// FusedMoE kernel runs gate, top-k, gather, the expert GEMMs and the combine,
// with the index preparation on chip.  Here:
//  * one cooperative launch of one 1024-thread workgroup per CU (every
//    workgroup resident at once; 16 waves per CU stream the weights), phases
//    separated by grid barriers: an arrival counter behind agent-scope
//    release / acquire fences (the eight XCDs' L2 caches are not coherent
//    with each other), each wait bounded so that every wave exits;
//  * phase 1: x quantised per token (one row per workgroup) and the router
//    logits as fp64 dot products rounded once to fp32, one (token, expert)
//    pair per wave;
//  * phase 2: every workgroup ranks the logits of all tokens itself (top-k,
//    renormalised weights, counts, segment offsets, the per-row-block table
//    and the sorted assignment list, all in its own LDS), so no barrier is
//    needed between the routing and the gate-up GEMM; workgroup 0 also
//    writes them to the workspace;
//  * phases 3 and 5: the register-fed skinny GEMM's work items (16 rows x 32
//    columns of one expert per wave) dealt round-robin over all waves,
//    workgroup index fastest, so that the items beyond one per wave land on
//    every CU rather than on the first few; the same epilogues as the
//    separate launches;
//  * phase 4: the requantisation of h (one row per workgroup); phase 6: the
//    combine, summing each token's k rows in j order from 0.
// Every value equals what the separate launches compute except the logits
// (fp64 sums here, the bf16 three-term split there), which agree within the
// fp32 router's error bound.
#include "skinny_item.h"
#include "device_common.h"

namespace w8a8 {
namespace {

constexpr int FZ_THREADS = 1024;  // sixteen waves: four per SIMD stream the weights
constexpr int FZ_WAVES = FZ_THREADS / 64;
constexpr int FZ_TPW = FUSED_MAX_T / FZ_WAVES;                         // tokens per wave in the top-k
constexpr int FZ_MAX_A = FUSED_MAX_T * MAX_TOPK;                       // assignments
constexpr int FZ_MAX_RB = FZ_MAX_A / SKINNY_BM + MAX_EXPERTS;          // 16-row blocks over all experts
constexpr long long FZ_SPIN_LIMIT = 1ll << 22;                         // barrier polls before giving up

// Grid barrier number `phase` (1, 2, ...): every workgroup's writes before it
// are visible to every workgroup after it.  sync[0] counts arrivals; a wait
// that exceeds the poll limit sets sync[1] and goes on (the results are then
// wrong, but every wave still exits).
__device__ __forceinline__ void grid_sync(int32_t* sync, int phase) {
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();  // release this workgroup's writes to the whole device
        __hip_atomic_fetch_add(sync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int target = phase * (int)gridDim.x;
        long long polls = 0;
        while (__hip_atomic_load(sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
            if (++polls > FZ_SPIN_LIMIT) {
                __hip_atomic_fetch_or(sync + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        __threadfence();  // acquire the other workgroups' writes
    }
    __syncthreads();
}

// One row quantised by the whole workgroup; VPT float4 per thread cover
// cols <= 4 * FZ_THREADS * VPT.
template <int CODE>
__device__ __forceinline__ void fused_quant_row(const float* row, int cols, const QuantOpts& opt, int8_t* q,
                                                float* scale, float* wmax) {
    const int nv = cols / 4;
    static_assert(4 * FZ_THREADS * 4 >= 16384, "four float4 per thread cover the longest row");
    if (nv <= FZ_THREADS) quant_row_wg<CODE, FZ_THREADS, 1>(row, cols, opt, q, scale, wmax);
    else if (nv <= 2 * FZ_THREADS) quant_row_wg<CODE, FZ_THREADS, 2>(row, cols, opt, q, scale, wmax);
    else quant_row_wg<CODE, FZ_THREADS, 4>(row, cols, opt, q, scale, wmax);
    __syncthreads();  // every wave has read wmax before the next row writes it
}

template <int CODE>
__global__ __launch_bounds__(FZ_THREADS) void moe_fused(FusedParams p) {
    __shared__ int ids_s[FZ_MAX_A];
    __shared__ float val_s[FZ_MAX_A];
    __shared__ unsigned long long mask[MAX_EXPERTS];
    __shared__ int off_s[MAX_EXPERTS];
    __shared__ __attribute__((aligned(16))) MtInfo mt_s[FZ_MAX_RB];
    __shared__ int32_t sorted_s[FZ_MAX_A];
    __shared__ int scan_lds[FZ_WAVES];
    __shared__ float wmax[FZ_WAVES];
    __shared__ int total_rb_s;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nwg = (int)gridDim.x;
    const int T = p.T, H = p.H, E = p.E, k = p.k, I = p.I;
    const int A = T * k;
    const bool lead = blockIdx.x == 0;  // writes the routing to the workspace
    // both E4M3 codes quantise to the same bytes
    constexpr int QCODE = CODE == CODE_INT8 ? CODE_INT8 : CODE_FP8;

    // ---- 1. x quantisation and the router logits ----
    for (int t = blockIdx.x; t < T; t += nwg)
        fused_quant_row<QCODE>(p.x + (int64_t)t * H, H, p.x_opt, p.x_q + (int64_t)t * H, p.x_scale + t, wmax);
    for (int pr = blockIdx.x * FZ_WAVES + w; pr < T * E; pr += nwg * FZ_WAVES) {
        const int t = pr / E, e = pr - t * E;
        const float4* xr = reinterpret_cast<const float4*>(p.x + (int64_t)t * H);
        const float4* wr = reinterpret_cast<const float4*>(p.router_w + (int64_t)e * H);
        // fp32 x fp32 products are exact in fp64; each lane sums a strided
        // quarter of H, then the lanes' sums meet in a fixed butterfly order
        double s = 0.0;
        for (int c = lane; c < H / 4; c += 64) {
            const float4 a = xr[c], b = wr[c];
            s = fma((double)a.x, (double)b.x, s);
            s = fma((double)a.y, (double)b.y, s);
            s = fma((double)a.z, (double)b.z, s);
            s = fma((double)a.w, (double)b.w, s);
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
        if (lane == 0) p.logits[(int64_t)t * E + e] = (float)(s + (p.router_b ? (double)p.router_b[e] : 0.0));
    }
    grid_sync(p.sync, 1);

    // ---- 2. routing, in every workgroup's LDS ----
    for (int e = tid; e < MAX_EXPERTS; e += FZ_THREADS) mask[e] = 0ull;
    {
        float vall[FZ_TPW][4];
#pragma unroll
        for (int u = 0; u < FZ_TPW; ++u) {
            const int t = min(w + FZ_WAVES * u, T - 1);
            const float* lrow = p.logits + (int64_t)t * E;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int e = lane + 64 * i;
                vall[u][i] = (e < E) ? lrow[min(e, E - 1)] : -INFINITY;
            }
        }
        const int n_valid = w < T ? (T - 1 - w) / FZ_WAVES + 1 : 0;
        wave_topk_n<FZ_TPW>(vall, lane, E, k, n_valid, ids_s + w * k, val_s + w * k, FZ_WAVES * k);
    }
    __syncthreads();
    for (int t = tid; t < T; t += FZ_THREADS) {
        float wj[MAX_TOPK];
        topk_weights(val_s + t * k, k, wj);
        if (lead) {
            for (int j = 0; j < k; ++j) {
                p.topk_ids[(int64_t)t * k + j] = ids_s[t * k + j];
                p.topk_w[(int64_t)t * k + j] = wj[j];
            }
        }
    }
    for (int a = tid; a < A; a += FZ_THREADS) atomicOr(&mask[ids_s[a]], 1ull << (a / k));
    __syncthreads();
    {
        // counts -> rows (low 16 bits) and 16-row blocks (high 16 bits) in one scan
        const int cnt = tid < E ? __popcll(mask[tid]) : 0;
        const int nrb = (cnt + SKINNY_BM - 1) / SKINNY_BM;
        int tot;
        const int both = block_exclusive_scan<FZ_WAVES>(cnt | (nrb << 16), &tot, scan_lds);
        const int off = both & 0xffff, rb0 = both >> 16;
        if (tid < E) {
            off_s[tid] = off;
            write_mt_info(mt_s, tid, rb0, nrb, off, off + cnt);
            if (lead) {
                p.expert_counts[tid] = cnt;
                p.expert_offsets[tid] = off;
            }
        }
        if (tid == 0) {
            total_rb_s = tot >> 16;
            if (lead) p.expert_offsets[E] = tot & 0xffff;
        }
    }
    __syncthreads();
    for (int a = tid; a < A; a += FZ_THREADS) {
        const int e = ids_s[a];
        const int pos = off_s[e] + __popcll(mask[e] & ((1ull << (a / k)) - 1ull));
        sorted_s[pos] = a;
        if (lead) p.sorted_assign[pos] = a;
    }
    __syncthreads();
    const int total_rb = total_rb_s;

    // ---- 3. gate-up: h = SiLU(g) * u per sorted row ----
    {
        GemmParams gu{};
        gu.A = p.x_q;
        gu.B = p.w_gu;
        gu.b_group_bytes = (int64_t)2 * I * H;
        gu.M = A;
        gu.N = 2 * I;
        gu.K = H;
        gu.mt_info = reinterpret_cast<const int32_t*>(mt_s);
        gu.G = E;
        gu.sorted_assign = sorted_s;
        gu.topk = k;
        gu.s_a = p.x_scale;
        gu.s_b = p.s_gu;
        gu.out_f32 = p.h;
        gu.I = I;
        gu.a_rows = T;
        gu.code = CODE;
        const int NC = 2 * I / 32;
        const int64_t total = (int64_t)total_rb * NC;
        for (int64_t item = (int64_t)w * nwg + blockIdx.x; item < total; item += (int64_t)nwg * FZ_WAVES)
            skinny_item<EPI_GATE_UP, 2, 4, CODE>(gu, item, NC, lane);
    }
    grid_sync(p.sync, 2);

    // ---- 4. h requantised per sorted row ----
    for (int r = blockIdx.x; r < A; r += nwg)
        fused_quant_row<QCODE>(p.h + (int64_t)r * I, I, QuantOpts{}, p.h_q + (int64_t)r * I, p.h_scale + r, wmax);
    grid_sync(p.sync, 3);

    // ---- 5. down: o[t*k+j] = w * dequant(h_q . W_d^T) ----
    {
        GemmParams dn{};
        dn.A = p.h_q;
        dn.B = p.w_d;
        dn.b_group_bytes = (int64_t)H * I;
        dn.M = A;
        dn.N = H;
        dn.K = I;
        dn.mt_info = reinterpret_cast<const int32_t*>(mt_s);
        dn.G = E;
        dn.sorted_assign = sorted_s;
        dn.topk = k;
        dn.s_a = p.h_scale;
        dn.s_b = p.s_d;
        dn.route_w = p.topk_w;
        dn.out_f32 = p.o;
        dn.a_rows = A;
        dn.code = CODE;
        const int NC = H / 32;
        const int64_t total = (int64_t)total_rb * NC;
        for (int64_t item = (int64_t)w * nwg + blockIdx.x; item < total; item += (int64_t)nwg * FZ_WAVES)
            skinny_item<EPI_DOWN, 2, 4, CODE>(dn, item, NC, lane);
    }
    grid_sync(p.sync, 4);

    // ---- 6. combine: y[t] = sum over j = 0..k-1, in order, of o[t*k+j] ----
    const int nv = H / 4;
    for (int t = blockIdx.x; t < T; t += nwg) {
        const float4* o4 = reinterpret_cast<const float4*>(p.o + (int64_t)t * k * H);
        float4* y4 = reinterpret_cast<float4*>(p.y + (int64_t)t * H);
        for (int c = tid; c < nv; c += FZ_THREADS) {
            float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            for (int j = 0; j < k; ++j) {
                const float4 v = o4[(int64_t)j * nv + c];
                acc.x += v.x;
                acc.y += v.y;
                acc.z += v.z;
                acc.w += v.w;
            }
            y4[c] = acc;
        }
    }
}

__global__ void moe_fused_reset(int32_t* sync) {
    if (threadIdx.x < 2) sync[threadIdx.x] = 0;
}

template <int CODE>
hipError_t launch_fused_code(const FusedParams& p, hipStream_t s) {
    const void* fn = reinterpret_cast<const void*>(&moe_fused<CODE>);
    int per_cu = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, FZ_THREADS, 0);
    if (e != hipSuccess) return e;
    if (per_cu < 1) return hipErrorInvalidConfiguration;
    const int nwg = device_cu_count() * (per_cu < FUSED_WG_PER_CU ? per_cu : FUSED_WG_PER_CU);
    moe_fused_reset<<<1, 64, 0, s>>>(p.sync);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    FusedParams arg = p;
    void* args[] = {&arg};
    return hipLaunchCooperativeKernel(fn, dim3((unsigned)nwg), dim3(FZ_THREADS), args, 0, s);
}

}  // namespace

hipError_t launch_moe_fused(const FusedParams& p, int code, hipStream_t s) {
    if (p.T < 1 || p.T > FUSED_MAX_T || p.k < 1 || p.k > MAX_TOPK || p.E < 1 || p.E > MAX_EXPERTS ||
        p.H % 128 != 0 || p.I % 128 != 0 || p.H > 16384 || p.I > 16384)
        return hipErrorInvalidValue;
    if (code == CODE_INT8) return launch_fused_code<CODE_INT8>(p, s);
    if (code == CODE_FP8) return launch_fused_code<CODE_FP8>(p, s);
    if (code == CODE_FP8_FAST) return launch_fused_code<CODE_FP8_FAST>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace w8a8
