// Per-row dynamic INT8 quantisation (one wave64 per row).
//
// "W8A8 quantisation of MiniMax-M3 on K100AI", sec. 2.1: q = clamp(round(x/s),
// -128, 127) with a per-token scale computed at run time from one extra
// reduction over the row.  Here s = max|x| / 127 (IEEE fp32 division), the
// quotient x/s is an IEEE fp32 division and round() is round-half-to-even
// (v_rndne).  An all-zero row gives s = 0 and all-zero codes.
//
// HBM-bound: each row is read once (cached in VGPRs while the wave reduces its
// maximum), and its codes and scale written once.  Loads and stores are full
// 16-byte (read) / 4-byte (write) per lane and contiguous across the wave.
#include "internal.h"

namespace w8a8 {
namespace {

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ int quant_one(float v, float s) {
    if (s == 0.0f) return 0;
    float r = __builtin_rintf(v / s);
    r = fminf(fmaxf(r, -128.0f), 127.0f);
    return (int)r;
}

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
    return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
           ((uint32_t)(d & 0xff) << 24);
}

__device__ __forceinline__ float amax4(float4 v) {
    return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// Vector path: cols % 4 == 0, ld % 4 == 0, x 16-byte aligned.  VPL float4 per
// lane stay in registers (rows up to VPL*256 elements).
template <int VPL>
__global__ __launch_bounds__(256) void quant_rows_cached(const float* __restrict__ x, int64_t rows,
                                                         int cols, int64_t ld, int8_t* __restrict__ q,
                                                         float* __restrict__ scale) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const float4* xr = reinterpret_cast<const float4*>(x + row * ld);
    const int nv = cols >> 2;
    float4 v[VPL];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int c = i * 64 + lane;
        if (c < nv) {
            v[i] = xr[c];
            amax = fmaxf(amax, amax4(v[i]));
        } else {
            v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    amax = wave_max(amax);
    const float s = amax / 127.0f;
    if (lane == 0) scale[row] = s;
    uint32_t* qr = reinterpret_cast<uint32_t*>(q + row * (int64_t)cols);
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int c = i * 64 + lane;
        if (c < nv)
            qr[c] = pack4(quant_one(v[i].x, s), quant_one(v[i].y, s), quant_one(v[i].z, s),
                          quant_one(v[i].w, s));
    }
}

// General path: any cols / ld / alignment; the row is read twice (the second
// read normally hits L2).
__global__ __launch_bounds__(256) void quant_rows_twopass(const float* __restrict__ x, int64_t rows,
                                                          int64_t cols, int64_t ld,
                                                          int8_t* __restrict__ q,
                                                          float* __restrict__ scale) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const float* xr = x + row * ld;
    float amax = 0.0f;
    for (int64_t c = lane; c < cols; c += 64) amax = fmaxf(amax, fabsf(xr[c]));
    amax = wave_max(amax);
    const float s = amax / 127.0f;
    if (lane == 0) scale[row] = s;
    int8_t* qr = q + row * cols;
    for (int64_t c = lane; c < cols; c += 64) qr[c] = (int8_t)quant_one(xr[c], s);
}

}  // namespace

hipError_t launch_quantize_rows(const float* x, int64_t rows, int64_t cols, int64_t ld, int8_t* q,
                                float* scale, hipStream_t s) {
    if (rows == 0) return hipSuccess;
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    const bool vec = (cols % 4 == 0) && (ld % 4 == 0) && ((uintptr_t)x % 16 == 0) &&
                     ((uintptr_t)q % 4 == 0) && cols <= 32 * 256;
    if (vec) {
        const int nv = (int)(cols / 4);
        const int need = (nv + 63) / 64;
        if (need <= 1)
            quant_rows_cached<1><<<grid, block, 0, s>>>(x, rows, (int)cols, ld, q, scale);
        else if (need <= 2)
            quant_rows_cached<2><<<grid, block, 0, s>>>(x, rows, (int)cols, ld, q, scale);
        else if (need <= 4)
            quant_rows_cached<4><<<grid, block, 0, s>>>(x, rows, (int)cols, ld, q, scale);
        else if (need <= 8)
            quant_rows_cached<8><<<grid, block, 0, s>>>(x, rows, (int)cols, ld, q, scale);
        else if (need <= 16)
            quant_rows_cached<16><<<grid, block, 0, s>>>(x, rows, (int)cols, ld, q, scale);
        else
            quant_rows_cached<32><<<grid, block, 0, s>>>(x, rows, (int)cols, ld, q, scale);
    } else {
        quant_rows_twopass<<<grid, block, 0, s>>>(x, rows, cols, ld, q, scale);
    }
    return hipGetLastError();
}

}  // namespace w8a8
