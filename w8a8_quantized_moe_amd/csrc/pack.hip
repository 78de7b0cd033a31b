// Weight re-layout into the GEMM's fragment order (offline, not on the hot path).
//
// For each group g, 16-channel block nb and 64-byte reduction block kb, one
// contiguous 1 KiB tile holds, at byte offset l*16 for lane l = r + 16*q,
// the 16 bytes w[g][nb*16 + r][kb*64 + q*16 .. +16].  That is the B operand
// of v_mfma_i32_16x16x64_i8 for lane l, so a wave reads a whole fragment with
// one contiguous 1 KiB load.  Tiles of one column block are consecutive along
// the reduction dimension.
//
// GATE_UP: the [2I][K] matrix (gate rows 0..I-1, up rows I..2I-1) is packed
// with column blocks alternating gate and up: block 2q holds gate channels
// 16q..16q+15 and block 2q+1 the up channels with the same indices, so the
// SwiGLU epilogue finds gate and up of one channel in the same lane.
#include "internal.h"

namespace w8a8 {
namespace {

__global__ __launch_bounds__(256) void pack_kernel(const int8_t* __restrict__ w, int64_t groups,
                                                   int64_t n, int64_t k, int gate_up,
                                                   int8_t* __restrict__ packed) {
    const int64_t chunk = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 16-byte unit of the output
    const int64_t NB = n / 16, KB = k / 64;
    const int64_t total = groups * NB * KB * 64;
    if (chunk >= total) return;
    const int ln = (int)(chunk & 63);
    int64_t t = chunk >> 6;
    const int64_t kb = t % KB;
    t /= KB;
    const int64_t nb = t % NB;
    const int64_t g = t / NB;
    const int r = ln & 15, q = ln >> 4;
    int64_t src_row;
    if (gate_up) {
        const int64_t half = n / 2;
        src_row = (nb & 1) * half + (nb >> 1) * 16 + r;
    } else {
        src_row = nb * 16 + r;
    }
    const int8_t* src = w + (g * n + src_row) * k + kb * 64 + q * 16;
    *reinterpret_cast<v4i*>(packed + chunk * 16) = *reinterpret_cast<const v4i*>(src);
}

}  // namespace

hipError_t launch_pack_weights(const int8_t* w, int64_t groups, int64_t n, int64_t k, int kind,
                               int8_t* packed, hipStream_t s) {
    const int64_t total = groups * (n / 16) * (k / 64) * 64;
    if (total == 0) return hipSuccess;
    const int64_t blocks = (total + 255) / 256;
    pack_kernel<<<dim3((unsigned)blocks), 256, 0, s>>>(w, groups, n, k, kind == 1 ? 1 : 0, packed);
    return hipGetLastError();
}

}  // namespace w8a8
