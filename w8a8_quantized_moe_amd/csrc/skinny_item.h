// One work item of the register-fed grouped INT8 GEMM for expert segments of
// a few rows (decode): a 16-row x (16*FN)-column block of one expert, run by
// one wave on its own (no LDS, no barriers).
//
// Same computation and epilogues as the tiled grouped GEMM: the int32
// accumulators of x_q . W^T per expert ("W8A8 quantisation of MiniMax-M3 on
// K100AI", sec. 2.1 and 3.1), with the per-token x per-channel scale product,
// SiLU(gate) * up ("DeepSeek V4 '950' unified FP8 dataflow", sec. 2.3), or the
// routing-weighted scatter ("Tencent Hunyuan AI Infra ... Hopper", sec. 1.3)
// fused into the epilogue.
#pragma once

#include "internal.h"

namespace w8a8 {

// item: (row block, column block) index in the expert-major order of the
// routing's per-row-block table, row blocks of an expert fastest; NC: column
// blocks (N / (16 * FN)).  The caller guarantees item < row blocks * NC.
template <int EPI, int FN, int D, int CODE>
__device__ __forceinline__ void skinny_item(const GemmParams& p, const int64_t item, const int NC,
                                            const int lane) {
    // expert of this item: one load from the routing's per-row-block table
    const MtInfo info = reinterpret_cast<const MtInfo*>(p.mt_info)[item / NC];
    const int g = info.group;
    const int mcount = (info.seg_end - info.seg_start + SKINNY_BM - 1) / SKINNY_BM;
    const int64_t local = item - (int64_t)info.first_tile * NC;
    const int rb = (int)(local % mcount);
    const int cb = (int)(local / mcount);
    const int64_t row0 = info.seg_start + (int64_t)rb * SKINNY_BM;
    const int64_t row_end = min(row0 + SKINNY_BM, (int64_t)info.seg_end);

    // MFMA A operand: lane l holds row l%16 and the 16-byte k-chunk l/16 of
    // each 64-byte k step; rows past the segment read a valid row (dropped)
    const int K = p.K;
    const int64_t KB = K / 64;
    int64_t r = row0 + (lane & 15);
    if (r >= row_end) r = row0;
    int64_t src_row = r;
    if (EPI == EPI_GATE_UP || EPI == EPI_GU_I32)
        src_row = min(max((int64_t)(p.sorted_assign[r] / p.topk), (int64_t)0), p.a_rows - 1);
    const int8_t* a_ptr = p.A + src_row * K + (lane >> 4) * 16;
    // packed weights: fragment (channel block nb, k step kb) at
    // g*b_group_bytes + (nb*KB + kb)*1024, lane l's 16 bytes at l*16
    const int8_t* b_ptr = p.B + (int64_t)g * p.b_group_bytes + (int64_t)cb * FN * KB * 1024 + lane * 16;

    const int nk = (int)KB;
    v4i ra[D], rbf[D][FN];
    auto load = [&](int slot, int ks) {
        ra[slot] = *reinterpret_cast<const v4i*>(a_ptr + (int64_t)ks * 64);
#pragma unroll
        for (int j = 0; j < FN; ++j)
            rbf[slot][j] = __builtin_nontemporal_load(
                reinterpret_cast<const v4i*>(b_ptr + ((int64_t)j * KB + ks) * 1024));
    };
    // prologue without branches (a slot past the last stage reloads the last
    // stage and is never multiplied), slot by slot as in the loop, so the
    // compiler's wait counts stay exact at the loop entry
#pragma unroll
    for (int d = 0; d < D; ++d) {
        load(d, min(d, nk - 1));
        __builtin_amdgcn_sched_barrier(0);
    }

    typename AccOf<CODE>::type acc[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[j] = typename AccOf<CODE>::type{};
    auto mfma = [&](int slot) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[j] = mma16<CODE>(ra[slot], rbf[slot][j], acc[j]);
    };
    // steady state without branches, so the compiler waits only for the
    // oldest stage (D-1 stages of loads stay in flight)
    int ks = 0;
    for (; ks + 2 * D <= nk; ks += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            mfma(d);
            load(d, ks + d + D);
            // keep the loads in stage order (the scheduler would otherwise
            // bunch them, and the waits would drain the whole pipeline)
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // tail: the last D to 2D-1 stages
#pragma unroll
    for (int d = 0; d < D; ++d) {
        if (ks + d < nk) {
            mfma(d);
            if (ks + d + D < nk) load(d, ks + d + D);
        }
    }
    ks += D;
#pragma unroll
    for (int d = 0; d < D; ++d)
        if (ks + d < nk) mfma(d);

    // epilogue: lane l, register q of block j holds row (l/16)*4 + q and
    // channel-block column l%16
    const int col_in_blk = lane & 15;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int64_t grow = row0 + (lane >> 4) * 4 + q;
        if (grow >= row_end) continue;
        if (EPI == EPI_GU_I32) {
            // raw accumulators (a checking path): gate channel c at column c,
            // up channel c at column I + c
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int ch = (cb * FN / 2 + j / 2) * 16 + col_in_blk;
                p.out_i32[grow * 2 * p.I + ((j & 1) ? p.I : 0) + ch] = (int)acc[j][q];
            }
        } else if (EPI == EPI_GATE_UP) {
            // column blocks alternate gate / up for the same 16 channels
            const int64_t t = min(max((int64_t)(p.sorted_assign[grow] / p.topk), (int64_t)0), p.a_rows - 1);
            const float sx = p.s_a[t];
#pragma unroll
            for (int jp = 0; jp < FN / 2; ++jp) {
                const int ch = (cb * FN / 2 + jp) * 16 + col_in_blk;
                const float gv = ((float)acc[2 * jp][q] * sx) * p.s_b[(int64_t)g * 2 * p.I + ch];
                const float uv = ((float)acc[2 * jp + 1][q] * sx) * p.s_b[(int64_t)g * 2 * p.I + p.I + ch];
                p.out_f32[grow * p.I + ch] = silu_f32(gv) * uv;
            }
        } else {  // EPI_DOWN
            const int64_t a = min(max((int64_t)p.sorted_assign[grow], (int64_t)0), p.M - 1);
            const float sh = p.s_a[grow];
            const float w = p.route_w[a];
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int col = (cb * FN + j) * 16 + col_in_blk;
                const float dq = ((float)acc[j][q] * sh) * p.s_b[(int64_t)g * p.N + col];
                p.out_f32[a * p.N + col] = w * dq;
            }
        }
    }
}

}  // namespace w8a8
