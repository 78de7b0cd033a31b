// Per-row dynamic quantisation to INT8 or FP8 E4M3 codes.
//
// "W8A8 quantisation of MiniMax-M3 on K100AI", sec. 2.1: q = clamp(round(x/s),
// -128, 127) with a per-token scale computed at run time from one extra
// reduction over the row.  Here s = max|x| / 127 (IEEE fp32 division), the
// quotient x/s is an IEEE fp32 division and round() is round-half-to-even
// (v_rndne).  An all-zero row gives s = 0 and all-zero codes.  With FP8 codes
// ("DeepSeek V4 '950' unified FP8 dataflow", sec. 2.1: E4M3, range +-448)
// s = max|x| / 448 and the code is E4M3(x / s), rounded to nearest even.
//
// Options ("W8A8 quantisation of MiniMax-M3 on K100AI", sec. 2.2; "DeepSeek V4
// '950'", sec. 3.1): a per-column factor (SmoothQuant) multiplies each value
// in fp32 before the row maximum is taken (or its reciprocal, an IEEE fp32
// division, for the weights of a smoothed layer), and the scale's base is the row
// maximum (dynamic), the row maximum capped by a calibrated bound (clipped)
// or the bound alone (static); codes then saturate (INT8 clamp, E4M3 +-448).
//
// HBM-bound: each row is read once (cached in VGPRs while its maximum is
// reduced: one wave per row up to 2048 columns, one 256-thread workgroup per
// row above), and its codes and scale written once.  Loads and stores are
// 16-byte (read) / 4-byte (write) per lane and contiguous across the wave.
#include "device_common.h"

namespace w8a8 {
namespace {

// Vector path: cols % 4 == 0, ld % 4 == 0, x 16-byte aligned.  VPL float4 per
// lane stay in registers (rows up to VPL*256 elements).
template <int CODE, int VPL>
__global__ __launch_bounds__(256) void quant_rows_cached(const float* __restrict__ x, int64_t rows,
                                                         int cols, int64_t ld, int8_t* __restrict__ q,
                                                         float* __restrict__ scale, QuantOpts opt) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const float4* xr = reinterpret_cast<const float4*>(x + row * ld);
    const int nv = cols >> 2;
    float4 v[VPL];
    load_row<VPL, 64>(xr, opt.col_mul, opt.col_recip, nv, lane, v);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
        if (i * 64 + lane < nv) amax = fmaxf(amax, amax4(v[i]));
    amax = wave_max(amax);
    const float s = scale_base(amax, opt) / code_range<CODE>();
    const float rs = 1.0f / s;
    if (lane == 0) scale[row] = s;
    uint32_t* qr = reinterpret_cast<uint32_t*>(q + row * (int64_t)cols);
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int c = i * 64 + lane;
        if (c < nv)
            qr[c] = encode4<CODE>(v[i], s, rs);
    }
}

// Long rows (vector path): one 256-thread workgroup per row, VPT float4 per
// thread held in registers; the row maximum goes through a wave reduction and
// four LDS slots.
template <int CODE, int VPT>
__global__ __launch_bounds__(256) void quant_rows_block(const float* __restrict__ x, int64_t rows,
                                                        int cols, int64_t ld, int8_t* __restrict__ q,
                                                        float* __restrict__ scale, QuantOpts opt) {
    (void)rows;  // the grid holds exactly one workgroup per row
    __shared__ float wmax[4];
    const int64_t row = blockIdx.x;
    quant_row_wg<CODE, 256, VPT>(x + row * ld, cols, opt, q + row * (int64_t)cols, scale + row, wmax);
}

// General path: any cols / ld / alignment; the row is read twice (the second
// read normally hits L2).
template <int CODE>
__global__ __launch_bounds__(256) void quant_rows_twopass(const float* __restrict__ x, int64_t rows,
                                                          int64_t cols, int64_t ld,
                                                          int8_t* __restrict__ q,
                                                          float* __restrict__ scale, QuantOpts opt) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;
    const float* xr = x + row * ld;
    const float* m = opt.col_mul;
    const bool rc = opt.col_recip;
    auto xv = [&](int64_t c) { return m ? xr[c] * (rc ? 1.0f / m[c] : m[c]) : xr[c]; };
    float amax = 0.0f;
    for (int64_t c = lane; c < cols; c += 64) amax = fmaxf(amax, fabsf(xv(c)));
    amax = wave_max(amax);
    const float s = scale_base(amax, opt) / code_range<CODE>();
    if (lane == 0) scale[row] = s;
    int8_t* qr = q + row * cols;
    for (int64_t c = lane; c < cols; c += 64) qr[c] = (int8_t)encode1<CODE>(xv(c), s);
}

template <int CODE>
hipError_t launch_quant(const float* x, int64_t rows, int64_t cols, int64_t ld, int8_t* q,
                        float* scale, const QuantOpts& opt, hipStream_t s) {
    const dim3 grid((unsigned)((rows + 3) / 4)), block(256);
    const bool vec = (cols % 4 == 0) && (ld % 4 == 0) && ((uintptr_t)x % 16 == 0) &&
                     ((uintptr_t)q % 4 == 0) && ((uintptr_t)opt.col_mul % 16 == 0) &&
                     cols <= 8 * 1024;
    if (vec && cols > 2048) {
        const int nv = (int)(cols / 4);
        const int need = (nv + 255) / 256;
        const dim3 g1((unsigned)rows);
        if (need <= 2)
            quant_rows_block<CODE, 2><<<g1, block, 0, s>>>(x, rows, (int)cols, ld, q, scale, opt);
        else if (need <= 4)
            quant_rows_block<CODE, 4><<<g1, block, 0, s>>>(x, rows, (int)cols, ld, q, scale, opt);
        else
            quant_rows_block<CODE, 8><<<g1, block, 0, s>>>(x, rows, (int)cols, ld, q, scale, opt);
    } else if (vec) {
        const int nv = (int)(cols / 4);
        const int need = (nv + 63) / 64;
        if (need <= 1)
            quant_rows_cached<CODE, 1><<<grid, block, 0, s>>>(x, rows, (int)cols, ld, q, scale, opt);
        else if (need <= 2)
            quant_rows_cached<CODE, 2><<<grid, block, 0, s>>>(x, rows, (int)cols, ld, q, scale, opt);
        else if (need <= 4)
            quant_rows_cached<CODE, 4><<<grid, block, 0, s>>>(x, rows, (int)cols, ld, q, scale, opt);
        else
            quant_rows_cached<CODE, 8><<<grid, block, 0, s>>>(x, rows, (int)cols, ld, q, scale, opt);
    } else {
        quant_rows_twopass<CODE><<<grid, block, 0, s>>>(x, rows, cols, ld, q, scale, opt);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_rows(const float* x, int64_t rows, int64_t cols, int64_t ld, int8_t* q,
                                float* scale, int code, hipStream_t s, const QuantOpts& opt) {
    if (rows == 0) return hipSuccess;
    // both FP8 codes store the same E4M3 values
    if (code == CODE_FP8 || code == CODE_FP8_FAST) return launch_quant<CODE_FP8>(x, rows, cols, ld, q, scale, opt, s);
    if (code == CODE_INT8) return launch_quant<CODE_INT8>(x, rows, cols, ld, q, scale, opt, s);
    return hipErrorInvalidValue;
}

}  // namespace w8a8
