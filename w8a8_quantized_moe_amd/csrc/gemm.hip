// INT8 x INT8 -> INT32 GEMM on gfx950 matrix cores, dense or grouped by expert,
// with the scale handling fused into the epilogue.
//
// "W8A8 quantisation of MiniMax-M3 on K100AI", sec. 2.1: the per-token [A,1] x
// per-channel [1,N] scale outer product is applied inside the GEMM epilogue,
// with no extra memory pass; sec. 3.1: many small per-expert GEMMs are batched
// into one launch.  "125B MoE on one RTX 3090", sec. 3.3: tokens routed to the
// same expert form one group.  "Tencent Hunyuan AI Infra ... Hopper",
// sec. 1.3: the gate-up GEMM reads its input rows through the routing index
// (no gather pass) and each expert writes a contiguous region.  "DeepSeek V4
// '950' unified FP8 dataflow", sec. 2.3: low-precision inputs, a wide
// accumulator, the output requantised for the next GEMM.
//
// Kernel shape: 256 threads (4 wave64 in a 2x2 grid), a 128x128 output tile,
// K consumed 128 bytes per stage, two LDS stages (64 KiB) so the next stage's
// global loads overlap the current stage's MFMAs.  Each wave owns a 64x64
// sub-tile = 4x4 v_mfma_i32_16x16x64_i8 blocks (64 accumulator VGPRs).
// LDS holds both operands in MFMA fragment order: each 16-row x 64-byte block
// is 1 KiB with lane l's 16 bytes at l*16, so every fragment read is one
// conflict-free ds_read_b128.  The weight operand arrives pre-packed in that
// order (pack.hip), so its global->LDS copy is a straight 16-byte-per-lane copy.
//
// Workgroup -> tile: blockIdx = m_tile * NT + n_tile.  Consecutive m-tiles of
// one n-tile are NT workgroups apart; with NT a multiple of 8 they land on the
// same XCD (workgroups are dealt round-robin over the 8 XCDs), so the weight
// tile they share is fetched from HBM once into that XCD's L2.
// Grouped mode: m-tiles are numbered expert by expert (mt_prefix); a
// workgroup finds its expert by binary search and exits if it is past the
// last tile (the grid is sized for the worst case, so no host sync is needed).
#include "internal.h"

namespace w8a8 {
namespace {

constexpr int BM = GEMM_BM, BN = GEMM_BN, BK = GEMM_BK;
constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK;
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;

// SiLU(g) = g / (1 + exp(-g)); the exponential is computed in double and
// rounded once to fp32 (correctly rounded fp32 exp but for vanishingly rare
// double-rounding cases); the add and the divide are IEEE fp32.
__device__ __forceinline__ float silu_f32(float g) {
    const float e = (float)exp(-(double)g);
    const float den = 1.0f + e;
    return g / den;
}

template <int EPI>
__global__ __launch_bounds__(256) void gemm_i8(GemmParams p) {
    __shared__ __attribute__((aligned(16))) int8_t smem[2 * STAGE_BYTES];
    __shared__ float row_scale[BM];
    __shared__ int row_slot[BM];
    __shared__ float row_w[BM];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t bid = blockIdx.x;
    const int mt = (int)(bid / p.NT), nt = (int)(bid % p.NT);

    // ---- which rows does this tile cover ----
    int g = 0;
    int64_t row0, row_end;
    if (p.seg_offsets) {
        if (mt >= p.mt_prefix[p.G]) return;
        int lo = 0, hi = p.G;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (p.mt_prefix[mid] <= mt) lo = mid; else hi = mid;
        }
        g = lo;
        row0 = p.seg_offsets[g] + (int64_t)(mt - p.mt_prefix[g]) * BM;
        row_end = min(row0 + BM, (int64_t)p.seg_offsets[g + 1]);
    } else {
        row0 = (int64_t)mt * BM;
        row_end = min(row0 + BM, p.M);
    }

    // ---- per-row metadata for the epilogue ----
    if (tid < BM) {
        const int64_t r = min(row0 + tid, row_end - 1);
        // routing indices are clamped into range so that even a corrupted
        // index (non-finite inputs) cannot address memory outside the buffers
        if (EPI == EPI_DENSE_F32) {
            row_scale[tid] = p.s_a[r];
        } else if (EPI == EPI_GATE_UP) {
            const int64_t t = min(max((int64_t)(p.sorted_assign[r] / p.topk), (int64_t)0), p.a_rows - 1);
            row_scale[tid] = p.s_a[t];
        } else if (EPI == EPI_DOWN) {
            const int64_t a = min(max((int64_t)p.sorted_assign[r], (int64_t)0), p.M - 1);
            row_scale[tid] = p.s_a[r];
            row_slot[tid] = (int)a;
            row_w[tid] = p.route_w[a];
        }
    }

    // ---- global source pointers: 4 A chunks and 4 B chunks of 16 B per thread ----
    const int K = p.K;
    const int8_t* a_src[4];
    int a_lds[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + i * 256;
        const int row = c >> 3, kc = c & 7;
        int64_t r = row0 + row;
        if (r >= row_end) r = row0;  // rows past the segment read a valid row; results dropped
        int64_t src_row = r;
        if (EPI == EPI_GATE_UP)
            src_row = min(max((int64_t)(p.sorted_assign[r] / p.topk), (int64_t)0), p.a_rows - 1);
        a_src[i] = p.A + src_row * K + kc * 16;
        const int kb = kc >> 2, gq = kc & 3, mb = row >> 4;
        a_lds[i] = (kb * (BM / 16) + mb) * 1024 + ((row & 15) + 16 * gq) * 16;
    }
    const int KB = K / 64;  // 1 KiB blocks per 16-channel column block
    const int8_t* b_base = p.B + (int64_t)g * p.b_group_bytes + (int64_t)(nt * (BN / 16)) * KB * 1024;
    const int8_t* b_src[4];
    int b_lds[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int c = tid + i * 256;
        const int nbl = c >> 7, within = c & 127;
        const int kbl = within >> 6, ln = within & 63;
        b_src[i] = b_base + (int64_t)nbl * KB * 1024 + kbl * 1024 + ln * 16;
        b_lds[i] = A_BYTES + (kbl * (BN / 16) + nbl) * 1024 + ln * 16;
    }

    v4i ra[4], rb[4];
    auto gload = [&](int ks) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ra[i] = *reinterpret_cast<const v4i*>(a_src[i] + (int64_t)ks * BK);
            rb[i] = *reinterpret_cast<const v4i*>(b_src[i] + (int64_t)ks * 2 * 1024);
        }
    };
    auto sstore = [&](int buf) {
        int8_t* base = smem + buf * STAGE_BYTES;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            *reinterpret_cast<v4i*>(base + a_lds[i]) = ra[i];
            *reinterpret_cast<v4i*>(base + b_lds[i]) = rb[i];
        }
    };

    v4i acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    const int nk = K / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int ks = 0; ks < nk; ++ks) {
        const int buf = ks & 1;
        if (ks + 1 < nk) gload(ks + 1);
        const int8_t* base = smem + buf * STAGE_BYTES;
#pragma unroll
        for (int kb = 0; kb < BK / 64; ++kb) {
            v4i fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                fa[i] = *reinterpret_cast<const v4i*>(base + (kb * (BM / 16) + wm * 4 + i) * 1024 + lane * 16);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                fb[j] = *reinterpret_cast<const v4i*>(base + A_BYTES + (kb * (BN / 16) + wn * 4 + j) * 1024 + lane * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
        if (ks + 1 < nk) sstore(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane l, register r of block (i, j) holds
    //      row = (wm*4+i)*16 + (l/16)*4 + r, col = (wn*4+j)*16 + l%16 ----
    const int col_in_blk = lane & 15;
    if (EPI == EPI_GATE_UP) {
        // column blocks alternate gate / up for the same 16 channels
        const int I = p.I;
        const float* sg = p.s_b + (int64_t)g * 2 * I;
#pragma unroll
        for (int jp = 0; jp < 2; ++jp) {
            const int gblk = nt * (BN / 16) + wn * 4 + 2 * jp;  // even: gate block
            const int ch = (gblk >> 1) * 16 + col_in_blk;
            const float s_gate = sg[ch], s_up = sg[I + ch];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = (wm * 4 + i) * 16 + (lane >> 4) * 4 + r;
                    const int64_t grow = row0 + row;
                    if (grow < row_end) {
                        const float sx = row_scale[row];
                        const float gv = ((float)acc[i][2 * jp][r] * sx) * s_gate;
                        const float uv = ((float)acc[i][2 * jp + 1][r] * sx) * s_up;
                        p.out_f32[grow * I + ch] = silu_f32(gv) * uv;
                    }
                }
        }
    } else {
        const int N = p.N;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = nt * BN + (wn * 4 + j) * 16 + col_in_blk;
            float sb = 0.0f;
            if (EPI != EPI_DENSE_I32) sb = p.s_b[(int64_t)g * N + n];
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = (wm * 4 + i) * 16 + (lane >> 4) * 4 + r;
                    const int64_t grow = row0 + row;
                    if (grow >= row_end) continue;
                    if (EPI == EPI_DENSE_I32) {
                        p.out_i32[grow * N + n] = acc[i][j][r];
                    } else if (EPI == EPI_DENSE_F32) {
                        p.out_f32[grow * N + n] = ((float)acc[i][j][r] * row_scale[row]) * sb;
                    } else {  // EPI_DOWN
                        const float v = ((float)acc[i][j][r] * row_scale[row]) * sb;
                        p.out_f32[(int64_t)row_slot[row] * N + n] = row_w[row] * v;
                    }
                }
        }
    }
}

}  // namespace

hipError_t launch_gemm(int epi, const GemmParams& p, int64_t m_tiles, hipStream_t s) {
    const int64_t blocks = m_tiles * p.NT;
    if (blocks == 0) return hipSuccess;
    const dim3 grid((unsigned)blocks), block(256);
    switch (epi) {
        case EPI_DENSE_F32: gemm_i8<EPI_DENSE_F32><<<grid, block, 0, s>>>(p); break;
        case EPI_DENSE_I32: gemm_i8<EPI_DENSE_I32><<<grid, block, 0, s>>>(p); break;
        case EPI_GATE_UP: gemm_i8<EPI_GATE_UP><<<grid, block, 0, s>>>(p); break;
        case EPI_DOWN: gemm_i8<EPI_DOWN><<<grid, block, 0, s>>>(p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace w8a8
