// Grouped INT8 (or FP8 E4M3) GEMM for expert segments of a few rows (the
// decode regime).  FP8 codes take two matrix instructions per 64-k fragment
// (mma16: the bf16 cores on decoded codes, or with the fast code the FP8
// cores' 16x16x32 instruction); the weight streaming never needs more rate.
//
// Same computation and epilogues as the tiled grouped GEMM (gemm.hip): the
// int32 accumulators of x_q . W^T per expert ("W8A8 quantisation of
// MiniMax-M3 on K100AI", sec. 2.1 and 3.1), with the per-token x per-channel
// scale product, SiLU(gate) * up ("DeepSeek V4 '950' unified FP8 dataflow",
// sec. 2.3), or the routing-weighted scatter ("Tencent Hunyuan AI Infra ...
// Hopper", sec. 1.3) fused into the epilogue.
//
// When a batch has only a handful of rows per expert the layer is bound by
// streaming the experts' weights from HBM, and the tiled kernel's 256-row LDS
// tiles mostly carry padding.  Here every wave works alone on a 16-row x
// (16*FN)-column block:
//  * no LDS and no barriers: the packed weight fragments (one contiguous
//    1 KiB per wave instruction, already in MFMA register order) and the
//    gathered activation fragment go straight from global memory into
//    registers;
//  * D stages of loads stay in flight per wave, and many waves per CU keep
//    enough bytes in flight to cover the memory latency;
//  * work items are (expert, 16-row block, column block) with the row blocks
//    of an expert fastest, so the blocks that share a weight slice run side by
//    side and share its reads in L2;
//  * narrow items (32 columns: one gate / up channel pair of 16) and one wave
//    per workgroup: the most items and the finest dispatch, so every CU keeps
//    its share of the stream to the end (decode layer: gate-up 0.113 ->
//    0.098 ms, 6.5 TB/s, and down 0.057 -> 0.052 ms against 64-column items
//    in four-wave workgroups).
#include "skinny_item.h"

namespace w8a8 {
namespace {

constexpr int SK_WAVES = 1;  // waves per workgroup (independent of each other)

template <int EPI, int FN, int D, int CODE>
__global__ __launch_bounds__(SK_WAVES * 64) void gemm_skinny(GemmParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * SK_WAVES + (threadIdx.x >> 6);
    const int NC = p.N / (16 * FN);  // column blocks
    const int64_t total = (int64_t)p.mt_prefix[p.G] * NC;
    if (item >= total) return;  // wave-uniform

    skinny_item<EPI, FN, D, CODE>(p, item, NC, lane);
}

}  // namespace

hipError_t launch_gemm_skinny(int epi, const GemmParams& p, int64_t max_row_blocks, hipStream_t s) {
    constexpr int FN = 2, D = 4;
    if (p.N % (16 * FN) != 0 || !p.seg_offsets) return hipErrorInvalidValue;
    const int64_t items = max_row_blocks * (p.N / (16 * FN));
    if (items == 0) return hipSuccess;
    const dim3 grid((unsigned)((items + SK_WAVES - 1) / SK_WAVES)), block(SK_WAVES * 64);
    if (p.code == CODE_FP8) {
        switch (epi) {
            case EPI_GATE_UP: gemm_skinny<EPI_GATE_UP, FN, D, CODE_FP8><<<grid, block, 0, s>>>(p); break;
            case EPI_DOWN: gemm_skinny<EPI_DOWN, FN, D, CODE_FP8><<<grid, block, 0, s>>>(p); break;
            default: return hipErrorInvalidValue;
        }
    } else if (p.code == CODE_FP8_FAST) {
        switch (epi) {
            case EPI_GATE_UP: gemm_skinny<EPI_GATE_UP, FN, D, CODE_FP8_FAST><<<grid, block, 0, s>>>(p); break;
            case EPI_DOWN: gemm_skinny<EPI_DOWN, FN, D, CODE_FP8_FAST><<<grid, block, 0, s>>>(p); break;
            default: return hipErrorInvalidValue;
        }
    } else if (p.code == CODE_INT8) {
        switch (epi) {
            case EPI_GATE_UP: gemm_skinny<EPI_GATE_UP, FN, D, CODE_INT8><<<grid, block, 0, s>>>(p); break;
            case EPI_DOWN: gemm_skinny<EPI_DOWN, FN, D, CODE_INT8><<<grid, block, 0, s>>>(p); break;
            case EPI_GU_I32: gemm_skinny<EPI_GU_I32, FN, D, CODE_INT8><<<grid, block, 0, s>>>(p); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace w8a8
