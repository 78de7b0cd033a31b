// Weighted combine: y[t][n] = sum over j = 0..k-1, in that order, of o[t*k+j][n]
// ("Tencent Hunyuan AI Infra ... Hopper", sec. 1.3: weighted aggregation at the
// end of the MoE pipeline; the routing weight is already applied to o by the
// down GEMM's epilogue).  fp32, a fixed summation order, no atomics, so the
// result is bit-reproducible.  HBM-bound: k*H*4 bytes read and H*4 written per
// token, 16 bytes per lane per access.
#include "internal.h"

namespace w8a8 {
namespace {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ o, int64_t T, int k,
                                                      int H, float* __restrict__ y) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // float4 index into y
    const int hv = H / 4;
    if (i >= T * hv) return;
    const int64_t t = i / hv;
    const int c = (int)(i - t * hv);
    const v4f* src = reinterpret_cast<const v4f*>(o) + (t * k) * hv + c;
    // all k loads in flight before the sum (k <= MAX_TOPK)
    v4f v[MAX_TOPK];
#pragma unroll
    for (int j = 0; j < MAX_TOPK; ++j)
        if (j < k) v[j] = __builtin_nontemporal_load(src + (int64_t)j * hv);
    v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < MAX_TOPK; ++j) {
        if (j < k) {
            acc.x += v[j].x;
            acc.y += v[j].y;
            acc.z += v[j].z;
            acc.w += v[j].w;
        }
    }
    reinterpret_cast<v4f*>(y)[i] = acc;
}

}  // namespace

hipError_t launch_combine(const float* o, int T, int k, int H, float* y, hipStream_t s) {
    const int64_t n = (int64_t)T * (H / 4);
    if (n == 0) return hipSuccess;
    combine_kernel<<<dim3((unsigned)((n + 255) / 256)), 256, 0, s>>>(o, T, k, H, y);
    return hipGetLastError();
}

}  // namespace w8a8
