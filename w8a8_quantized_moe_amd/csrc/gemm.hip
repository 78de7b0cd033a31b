// INT8 x INT8 -> INT32 (or FP8 E4M3 x E4M3 -> FP32) GEMM on gfx950 matrix
// cores, dense or grouped by expert, with the scale handling fused into the
// epilogue.
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
// Kernel shape (BM x BN output tile, WM x WN waves of 64 lanes):
//  * every wave owns a (BM/WM) x (BN/WN) sub-tile: INT8 as 16x16 blocks of
//    v_mfma_i32_16x16x64_i8, FP8 as 32x32 blocks of
//    v_mfma_scale_f32_32x32x64_f8f6f4 (unit block scales);
//  * K advances 64 bytes per pipeline stage; NS stages live in LDS at once;
//  * operands move global -> LDS with global_load_lds_dwordx4 (no VGPR
//    staging): one wave instruction moves one 16-row x 64-byte block (1 KiB),
//    lane l writing its 16 bytes at l*16, and every fragment read later is a
//    conflict-free ds_read_b128 (two per 32-byte FP8 operand).  The weight
//    operand arrives pre-packed in fragment order (pack.hip); for the
//    activation operand each 4-lane group fetches one (possibly gathered)
//    row's 64 bytes, stored at an XOR-swizzled slot;
//  * NS-1 stages of copies stay in flight: wait for stage s+1 (explicit
//    vmcnt), barrier, issue stage s+NS-1, then run stage s's MFMAs from
//    registers while stage s+1's fragments stream in from LDS;
//  * a segment's last m-tile with at most 128 rows copies only those rows
//    through a deeper ring and spreads them over all waves (INT8 and FP8;
//    for FP8 on 256-wide tiles).
//
// Workgroup -> tile order (XCD-aware).  Workgroups are dealt round-robin to the
// 8 XCDs, so blockIdx % 8 names the XCD; each XCD owns one contiguous range
// of the logical tile order (expert, n-tile, m-tile; m-tile fastest), so each
// XCD works on whole experts and the m-tiles that share a weight tile start
// side by side.  Grouped GEMMs run persistent: one workgroup per CU drains
// its XCD's range as a queue (a counter the routing zeroed) and then helps
// the other XCDs.  The routing lists the experts largest first and cuts the
// order into eight ranges of about equal work, so every queue runs its
// longest tiles first ("Tencent Hunyuan AI Infra ... Hopper", sec. 1.1: tiles
// dealt to thread blocks by a greedy, load-even assignment, here longest
// first; "125B MoE on one RTX 3090", sec. 2.1: the hot and cold experts of a
// skewed routing).  The dense GEMM is split into 8 column
// stripes ("virtual groups" sharing the same rows), one per XCD, one tile per
// workgroup.
#include <atomic>
#include <type_traits>

#include "internal.h"

namespace w8a8 {
namespace {

template <int BM, int BN, int WM, int WN, int NS, int EPI, int CODE>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_i8(GemmParams p) {
    typedef typename AccOf<CODE>::type AccT;
    // the gate-up GEMMs read their activation rows through the routing index
    constexpr bool GATHER = (EPI == EPI_GATE_UP || EPI == EPI_GU_I32);
    constexpr int NW = WM * WN;                  // waves per workgroup
    constexpr int FM = BM / WM / 16;             // fragment rows per wave
    constexpr int FN = BN / WN / 16;             // fragment cols per wave
    constexpr int NBA = BM / 16, NBB = BN / 16;  // 1 KiB blocks per stage
    constexpr int NBLK = NBA + NBB;
    static_assert(NBLK % NW == 0, "blocks must split evenly over the waves");
    constexpr int DPW = NBLK / NW;               // copies per wave per stage
    constexpr int STAGE = NBLK * 1024;
    static_assert(NS >= 3, "the fragment prefetch needs at least three LDS stages");
    static_assert(FM % 2 == 0, "half-tile variant");
    // One LDS object only: the pipeline stages, then the per-row metadata.
    // (With several __shared__ objects the compiler can no longer tell the
    // copy target from other LDS data and drains the pipeline before every
    // LDS read.)
    __shared__ __attribute__((aligned(1024))) int8_t smem[NS * STAGE + 3 * BM * 4 + 16];
    // the ring through an LDS-typed pointer: copies and fragment reads address
    // LDS directly, also where the compiler cannot infer the address space
    // through the stage select
    const LDS_AS int8_t* lds = (const LDS_AS int8_t*)smem;
    float* row_scale = reinterpret_cast<float*>(smem + NS * STAGE);
    int* row_slot = reinterpret_cast<int*>(smem + NS * STAGE + BM * 4);
    float* row_w = reinterpret_cast<float*>(smem + NS * STAGE + 2 * BM * 4);
    int* next_tile = reinterpret_cast<int*>(smem + NS * STAGE + 3 * BM * 4);

    const int tid0 = threadIdx.x;

    // ---- logical tiles: XCD x owns the contiguous range [x*per_xcd, (x+1)*per_xcd) ----
    const int64_t n_mt_dense = (p.M + BM - 1) / BM;
    const int64_t total = (p.seg_offsets ? (int64_t)p.mt_prefix[p.G] : n_mt_dense * p.VG) * p.NTV;
    const int64_t per_xcd = (total + 7) / 8;

    // The claim of the workgroup's next tile (persistent launch): issued by
    // thread 0 when the current tile's epilogue starts, read after it.
    // Claiming at the epilogue rather than when a tile starts keeps the
    // claims in the order the tiles end, which is the order the claimed tiles
    // start: consecutive tiles (the m-tiles sharing a weight tile, the column
    // tiles sharing activation rows) then run side by side, whatever the
    // lengths of the tiles before them.  The epilogue hides the atomic's
    // latency.
    int claim_got = 0;
    auto claim_next = [&]() {
        if (p.tile_ctr && tid0 == 0) claim_got = atomicAdd(p.tile_ctr + TILE_CTR_STRIDE * (blockIdx.x & 7), 1);
    };

    // One output tile: L -> (group, m-tile, n-tile), K loop, epilogue.
    auto process = [&](const int64_t L) {
    // Thread indices pass through an opaque zero, so that the lane-dependent
    // addresses below are recomputed per tile instead of being hoisted out of
    // the tile loop (where they would stay live across the K loop and push
    // the register count past the limit).
    int opaque = 0;
    asm volatile("" : "+v"(opaque));
    const int tid = tid0 + opaque, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);
    const int wm = wave / WN, wn = wave % WN;
    int g = 0, nt;
    int64_t row0, row_end;
    if (p.seg_offsets) {
        // the m-tile table (largest expert first): one table load names the
        // expert (the routing built the table for this BM)
        const MtInfo info = reinterpret_cast<const MtInfo*>(p.mt_info)[L / p.NTV];
        g = info.group;
        const int64_t local = L - (int64_t)info.first_tile * p.NTV;
        // inside an expert, m-tiles vary fastest: the m-tiles that share one
        // weight tile run side by side and share its reads in L2
        const int mcount = (info.seg_end - info.seg_start + BM - 1) / BM;
        const int mtl = (int)(local % mcount);
        nt = (int)(local / mcount);
        row0 = info.seg_start + (int64_t)mtl * BM;
        row_end = min(row0 + BM, (int64_t)info.seg_end);
    } else {
        const int64_t per_vg = n_mt_dense * p.NTV;
        const int vg = (int)(L / per_vg);
        const int64_t local = L - vg * per_vg;
        const int64_t mt = local / p.NTV;
        nt = vg * p.NTV + (int)(local % p.NTV);
        row0 = mt * BM;
        row_end = min(row0 + BM, p.M);
    }
    // A segment's last tile with at most FM*16 valid rows (a "half tile" for
    // WM = 2) runs its own schedule (run_half below): only the first FM*16
    // rows are copied, so a stage is smaller and the ring deeper, and all
    // waves share those rows and split the columns, FN/WM fragment columns
    // each.  (For the gate-up epilogue and for FP8 codes, whose 32x32 MFMA
    // blocks span two fragment columns, only where each wave keeps an even
    // number of fragment columns.)
    constexpr bool HALF_OK = FN % WM == 0 &&
                             ((!GATHER && CODE == CODE_INT8) || (FN / WM) % 2 == 0);
    const int rows_valid = (int)(row_end - row0);
    const bool half = HALF_OK && rows_valid <= FM * 16;
    // first fragment row / column of this wave
    const int a_base = half ? 0 : wm * FM;
    const int b_base = half ? wn * FN + wm * (FN / WM) : wn * FN;
    // fragment rows of this wave holding at least one valid row (the rest of a
    // segment's last, partial tile is neither read nor multiplied)
    const int fm_active = __builtin_amdgcn_readfirstlane(
        half ? min(FM, (rows_valid + 15) / 16) : min(FM, max(0, (rows_valid - wm * FM * 16 + 15) / 16)));

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

    // ---- copy sources: this wave moves blocks wave, wave+NW, ... of each stage ----
    const int K = p.K;
    const int64_t KB = K / 64;
    const int8_t* src[DPW];
    int stride[DPW];
#pragma unroll
    for (int i = 0; i < DPW; ++i) {
        const int b = wave + NW * i;
        if (b < NBA) {
            // activation rows: each 4-lane group fetches one row's 64 bytes (one
            // contiguous request); chunk c of row r goes to LDS slot
            // 4r + (c ^ (r/4)), which keeps the fragment reads conflict-free
            int64_t r = row0 + b * 16 + (lane >> 2);
            if (r >= row_end) r = row0;  // rows past the segment read a valid row; results dropped
            int64_t src_row = r;
            if (GATHER)
                src_row = min(max((int64_t)(p.sorted_assign[r] / p.topk), (int64_t)0), p.a_rows - 1);
            src[i] = p.A + src_row * K + (((lane & 3) ^ ((lane >> 4) & 3)) * 16);
            stride[i] = 64;
        } else {        // packed weights: 1 KiB contiguous per (16 channels, 64 k)
            const int nb = nt * NBB + (b - NBA);
            src[i] = p.B + (int64_t)g * p.b_group_bytes + (int64_t)nb * KB * 1024 + lane * 16;
            stride[i] = 1024;
        }
    }
    auto issue = [&](int ks) {
        const LDS_AS int8_t* stage = lds + (ks % NS) * STAGE;
#pragma unroll
        for (int i = 0; i < DPW; ++i)
            dma16(src[i] + (int64_t)ks * stride[i], stage + (wave + NW * i) * 1024);
    };
    // MFMA A operand: lane l holds row l%16, 16-byte k-chunk l/16 of the block
    const int a_slot = 4 * (lane & 15) + ((lane >> 4) ^ ((lane >> 2) & 3));
    auto frag_a = [&](int ks, int i) {
        return *reinterpret_cast<const LDS_AS v4i*>(lds + (ks % NS) * STAGE + (a_base + i) * 1024 + a_slot * 16);
    };
    auto frag_b = [&](int ks, int j) {
        return *reinterpret_cast<const LDS_AS v4i*>(lds + (ks % NS) * STAGE + (NBA + b_base + j) * 1024 +
                                             lane * 16);
    };

    const int nk = K / 64;
    // FP8 codes run on the 32x32x64 FP8 MFMA (v_mfma_scale_f32_32x32x64_f8f6f4
    // with unit block scales): one 64-k stage feeds it directly, lane l
    // supplying row (column) l%32 and the stage's k bytes (l/32)*32 .. +31, read
    // as two 16-byte chunks from the same LDS blocks the INT8 fragments use.
    // A wave's 128x64 outputs are 4x2 blocks of 32x32.  (The 16x16x32 FP8 MFMA
    // issues at a quarter of the rate.)
    constexpr bool M32 = (CODE != CODE_INT8);
    constexpr int FM32 = FM / 2, FN32 = FN / 2;  // 32x32 blocks per wave
    static_assert(!M32 || (FM % 2 == 0 && FN % 2 == 0), "whole 32x32 blocks per wave");
    v4i fa[M32 ? 1 : FM], fb[M32 ? 1 : FN];
    v8i fa32[M32 ? FM32 : 1], fb32[M32 ? FN32 : 1];
    // rows (a_base + 2i + (l/16)%2)*16 + l%16, k chunks 2h and 2h+1 (h = l/32)
    auto frag_a32 = [&](int ks, int i) {
        const int blk = a_base + 2 * i + ((lane >> 4) & 1);
        const int rr = lane & 15, h = lane >> 5;
        const LDS_AS int8_t* base = lds + (ks % NS) * STAGE + blk * 1024;
        v8i t;
        t.lo = *reinterpret_cast<const LDS_AS v4i*>(base + (4 * rr + ((2 * h) ^ (rr >> 2))) * 16);
        t.hi = *reinterpret_cast<const LDS_AS v4i*>(base + (4 * rr + ((2 * h + 1) ^ (rr >> 2))) * 16);
        return t;
    };
    // columns (b_base + 2j + (l/16)%2)*16 + l%16 (packed lane slot c + 16*chunk)
    auto frag_b32 = [&](int ks, int j) {
        const int blk = NBA + b_base + 2 * j + ((lane >> 4) & 1);
        const int cc = lane & 15, h = lane >> 5;
        const LDS_AS int8_t* base = lds + (ks % NS) * STAGE + blk * 1024;
        v8i t;
        t.lo = *reinterpret_cast<const LDS_AS v4i*>(base + (cc + 32 * h) * 16);
        t.hi = *reinterpret_cast<const LDS_AS v4i*>(base + (cc + 32 * h + 16) * 16);
        return t;
    };
    if (half) {
        // (a half tile fills its own ring: run_half)
    } else if constexpr (M32) {
        // prologue: NS-1 stages in flight, stage 0's fragments in registers
#pragma unroll
        for (int s = 0; s < NS - 1; ++s)
            if (s < nk) issue(s);
        if (nk - 1 >= NS - 2) wait_vmcnt<(NS - 2) * DPW>();
        else wait_vmcnt<0>();
        barrier_nofence();
#pragma unroll
        for (int i = 0; i < FM32; ++i)
            if (2 * i < fm_active) fa32[i] = frag_a32(0, i);
#pragma unroll
        for (int j = 0; j < FN32; ++j) fb32[j] = frag_b32(0, j);
    } else {
        // prologue: NS-1 stages in flight, stage 0's fragments in registers
#pragma unroll
        for (int s = 0; s < NS - 1; ++s)
            if (s < nk) issue(s);
        if (nk - 1 >= NS - 2) wait_vmcnt<(NS - 2) * DPW>();
        else wait_vmcnt<0>();
        barrier_nofence();
#pragma unroll
        for (int i = 0; i < FM; ++i)
            if (i < fm_active) fa[i] = frag_a(0, i);
#pragma unroll
        for (int j = 0; j < FN; ++j) fb[j] = frag_b(0, j);
    }

    // ---- epilogue.  Lane l, register r of accumulator block (i, j) holds
    //      row (a_base+i)*16 + (l/16)*4 + r, column (b_base+j)*16 + l%16 (j < NF,
    //      the wave's fragment columns).  The
    //      values are finished in registers, staged through the (now idle) LDS
    //      ring 32 rows at a time, and leave as 16-byte stores that cover whole
    //      256-byte (128-byte for h) row segments.  It runs inside each compute
    //      variant below, so the accumulators never have to be merged across
    //      the variants' register assignments. ----
    static_assert(NW * 32 * (((EPI == EPI_GATE_UP) ? FN * 8 : FN * 16) + 4) * 4 <= NS * STAGE,
                  "epilogue staging fits in the LDS ring");
    // one staged pass of 32 rows (from tile row rbase) leaves as 16-byte stores
    auto write_pass = [&](auto n_tag, const uint32_t* stg, int rbase, int64_t col0) {
        constexpr int NF = decltype(n_tag)::value;
        constexpr int OCOLS = (EPI == EPI_GATE_UP) ? NF * 8 : NF * 16;
        constexpr int SROW = OCOLS + 4;
        const int I = p.I, N = p.N;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's staging complete
        // each lane moves 16 bytes; a wave covers 64*4/OCOLS rows per instruction
        constexpr int LPR = OCOLS / 4;   // lanes per row
        constexpr int RPI = 64 / LPR;    // rows per instruction
#pragma unroll
        for (int q = 0; q < 32 / RPI; ++q) {
            const int lr = q * RPI + lane / LPR;
            const int c4 = (lane % LPR) * 4;
            const int row = rbase + lr;
            const int64_t grow = row0 + row;
            if (grow < row_end) {
                const v4i v = *reinterpret_cast<const v4i*>(stg + lr * SROW + c4);
                int64_t dst;
                if (EPI == EPI_GATE_UP) dst = grow * I + col0 + c4;
                else if (EPI == EPI_DOWN) dst = (int64_t)row_slot[row] * N + col0 + c4;
                else dst = grow * N + col0 + c4;
                if (EPI == EPI_DENSE_I32) *reinterpret_cast<v4i*>(p.out_i32 + dst) = v;
                // h and o are read back once, by the next pass, from HBM (they
                // exceed the caches): stream them past the caches instead of
                // evicting the tiles' operands
                else if (EPI == EPI_DOWN || EPI == EPI_GATE_UP)
                    __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(p.out_f32 + dst));
                else *reinterpret_cast<v4i*>(p.out_f32 + dst) = v;
            }
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads done before the next pass
    };
    auto epilogue = [&](AccT (&acc)[FM][FN], auto n_tag) {
        constexpr int NF = decltype(n_tag)::value;
        claim_next();
        if constexpr (EPI == EPI_GU_I32) {
            // raw accumulators straight from registers (a checking path): the
            // column blocks alternate gate / up for the same 16 channels, as in
            // the gate-up epilogue
            const int64_t ch0 = (int64_t)(nt * NBB + b_base) / 2 * 16 + (lane & 15);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                if (i >= fm_active) break;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t grow = row0 + (a_base + i) * 16 + (lane >> 4) * 4 + r;
                    if (grow >= row_end) continue;
#pragma unroll
                    for (int j = 0; j < NF; ++j)
                        p.out_i32[grow * 2 * p.I + ((j & 1) ? p.I : 0) + ch0 + (j >> 1) * 16] = (int)acc[i][j][r];
                }
            }
            return;
        }
        constexpr int OCOLS = (EPI == EPI_GATE_UP) ? NF * 8 : NF * 16;  // output columns per wave
        constexpr int SROW = OCOLS + 4;                                 // padded staging stride (words)
        __syncthreads();  // the ring is idle; row metadata written before the loop is visible
        uint32_t* stg = reinterpret_cast<uint32_t*>(smem) + wave * (32 * SROW);
        const int col_in_blk = lane & 15;
        const int I = p.I, N = p.N;
        // first output column of this wave
        const int64_t col0 = (EPI == EPI_GATE_UP) ? (int64_t)(nt * NBB + b_base) / 2 * 16
                                                  : (int64_t)nt * BN + b_base * 16;
        float s_col[NF];
#pragma unroll
        for (int j = 0; j < NF; ++j) {
            if (EPI == EPI_GATE_UP) {
                const int jp = j >> 1;
                const int ch = (int)col0 + jp * 16 + col_in_blk;
                s_col[j] = p.s_b[(int64_t)g * 2 * I + ((j & 1) ? I : 0) + ch];
            } else if (EPI != EPI_DENSE_I32) {
                s_col[j] = p.s_b[(int64_t)g * N + col0 + j * 16 + col_in_blk];
            } else {
                s_col[j] = 0.0f;
            }
        }
#pragma unroll
        for (int i0 = 0; i0 < FM; i0 += 2) {
            if (i0 >= fm_active) break;
            // finish 2 fragment rows (32 rows) in registers, stage them
#pragma unroll
            for (int di = 0; di < 2; ++di) {
                const int i = i0 + di;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int lr = di * 16 + (lane >> 4) * 4 + r;            // staged row
                    const int row = (a_base + i) * 16 + (lane >> 4) * 4 + r;  // tile row
                    if (EPI == EPI_GATE_UP) {
                        // column blocks alternate gate / up for the same 16 channels
                        const float sx = row_scale[row];
#pragma unroll
                        for (int jp = 0; jp < NF / 2; ++jp) {
                            const float gv = ((float)acc[i][2 * jp][r] * sx) * s_col[2 * jp];
                            const float uv = ((float)acc[i][2 * jp + 1][r] * sx) * s_col[2 * jp + 1];
                            stg[lr * SROW + jp * 16 + col_in_blk] = __float_as_uint(silu_f32(gv) * uv);
                        }
                    } else {
#pragma unroll
                        for (int j = 0; j < NF; ++j) {
                            uint32_t v;
                            if (EPI == EPI_DENSE_I32) {
                                v = (uint32_t)(int)acc[i][j][r];
                            } else if (EPI == EPI_DENSE_F32) {
                                v = __float_as_uint(((float)acc[i][j][r] * row_scale[row]) * s_col[j]);
                            } else {  // EPI_DOWN
                                const float dq = ((float)acc[i][j][r] * row_scale[row]) * s_col[j];
                                v = __float_as_uint(row_w[row] * dq);
                            }
                            stg[lr * SROW + j * 16 + col_in_blk] = v;
                        }
                    }
                }
            }
            write_pass(n_tag, stg, (a_base + i0) * 16, col0);
        }
    };

    // ---- the FP8 epilogue: register q of 32x32 block (i, j) in lane l holds
    //      row (a_base + 2i)*16 + (q/4)*8 + (l/32)*4 + q%4, column
    //      (b_base + 2j)*16 + l%32; the gate and up values of one channel sit
    //      16 lanes apart. ----
    auto epilogue32 = [&](auto& acc, auto nj_tag) {
        constexpr int NJ = decltype(nj_tag)::value;  // 32-column blocks of this wave
        claim_next();
        constexpr int NF = 2 * NJ;
        constexpr int OCOLS = (EPI == EPI_GATE_UP) ? NF * 8 : NF * 16;
        constexpr int SROW = OCOLS + 4;
        __syncthreads();  // the ring is idle; row metadata written before the loop is visible
        uint32_t* stg = reinterpret_cast<uint32_t*>(smem) + wave * (32 * SROW);
        const int I = p.I, N = p.N;
        const int h = lane >> 5, c32 = lane & 31, up = (lane >> 4) & 1;
        const int64_t col0 = (EPI == EPI_GATE_UP) ? (int64_t)(nt * NBB + b_base) / 2 * 16
                                                  : (int64_t)nt * BN + b_base * 16;
        float s_col[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if (EPI == EPI_GATE_UP)
                s_col[j] = p.s_b[(int64_t)g * 2 * I + (up ? I : 0) + col0 + j * 16 + (lane & 15)];
            else
                s_col[j] = p.s_b[(int64_t)g * N + col0 + j * 32 + c32];
        }
#pragma unroll
        for (int i = 0; i < FM32; ++i) {
            if (2 * i >= fm_active) break;
            if (EPI == EPI_GATE_UP) {
                // registers q and q+1 are rows lr0 and lr0+1: a gate lane keeps
                // row lr0 and hands its row-(lr0+1) gate value to its up partner
                // (16 lanes away), which keeps row lr0+1 and hands back its row-lr0
                // up value, so every lane finishes one h value per register pair
#pragma unroll
                for (int q = 0; q < 16; q += 2) {
                    const int lr0 = (q / 4) * 8 + h * 4 + (q % 4);
                    const int row = (a_base + 2 * i) * 16 + lr0;
                    const float sx0 = row_scale[row], sx1 = row_scale[row + 1];
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        const float v0 = (acc[i][j][q / 4][q % 4] * sx0) * s_col[j];
                        const float v1 = (acc[i][j][q / 4][q % 4 + 1] * sx1) * s_col[j];
                        const float got = __shfl_xor(up ? v0 : v1, 16, 64);
                        const float gv = up ? got : v0, uv = up ? v1 : got;
                        stg[(lr0 + up) * SROW + j * 16 + (lane & 15)] = __float_as_uint(silu_f32(gv) * uv);
                    }
                }
            }
            if (EPI != EPI_GATE_UP) {
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int lr = (q / 4) * 8 + h * 4 + (q % 4);    // staged row
                    const int row = (a_base + 2 * i) * 16 + lr;      // tile row
#pragma unroll
                    for (int j = 0; j < NJ; ++j) {
                        const float dq = (acc[i][j][q / 4][q % 4] * row_scale[row]) * s_col[j];
                        const float v = (EPI == EPI_DOWN) ? row_w[row] * dq : dq;
                        stg[lr * SROW + j * 32 + c32] = __float_as_uint(v);
                    }
                }
            }
            write_pass(std::integral_constant<int, NF>{}, stg, (a_base + 2 * i) * 16, col0);
        }
    };

    // Stage ks's MFMAs run from registers while stage ks+1's fragments stream
    // in from LDS: each A fragment right after its last use, the B fragments
    // once the stage's MFMAs are issued.  F = fragment rows this wave computes: FM for a full
    // tile; in a segment's last, partial tile FM/2 or 0.
    auto mfma_and_refill = [&](auto f_tag, AccT (&acc)[FM][FN], int next_ks, bool refill) {
        constexpr int F = decltype(f_tag)::value;
#pragma unroll
        for (int i = 0; i < F; ++i) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = mma16<CODE>(fa[i], fb[j], acc[i][j]);
            if (refill) fa[i] = frag_a(next_ks, i);
            // keep each refill next to the MFMAs it follows (hoisting them all
            // would need a second set of A registers)
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    auto run = [&](auto f_tag) {
        constexpr int F = decltype(f_tag)::value;
        AccT acc[FM][FN];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = AccT{};
        int ks = 0;
        // steady state: stage ks+1 landed (NS-3 newer stages may still fly),
        // refill the ring with stage ks+NS-1
        for (; ks + NS - 1 < nk; ++ks) {
            wait_vmcnt<(NS - 3) * DPW>();
            barrier_nofence();
            issue(ks + NS - 1);
            mfma_and_refill(f_tag, acc, ks + 1, true);
            if (F > 0) {
#pragma unroll
                for (int j = 0; j < FN; ++j) fb[j] = frag_b(ks + 1, j);
            }
        }
        // drain: nothing left to issue
        for (; ks + 1 < nk; ++ks) {
            wait_vmcnt<0>();
            barrier_nofence();
            mfma_and_refill(f_tag, acc, ks + 1, true);
            if (F > 0) {
#pragma unroll
                for (int j = 0; j < FN; ++j) fb[j] = frag_b(ks + 1, j);
            }
        }
        mfma_and_refill(f_tag, acc, 0, false);
        epilogue(acc, std::integral_constant<int, FN>{});
    };
    // A half tile: only its first FM*16 rows are copied, so a stage holds
    // FM A blocks instead of BM/16 and the same LDS ring takes more stages
    // (5 instead of 4 for 256x256 tiles: four in flight instead of three).
    // A segment's last tile streams the whole weight tile for few rows,
    // which makes it bound by the copy pipeline's latency; the deeper
    // ring and all eight waves at work (each on FN/WM fragment columns of
    // those rows) shorten it.
    auto run_half = [&](auto f_tag) {
        constexpr int F = decltype(f_tag)::value;
        constexpr int NF = FN / WM;
        constexpr int NBLK_H = FM + NBB;
        static_assert(NBLK_H % NW == 0, "half-tile blocks must split evenly over the waves");
        constexpr int DPW_H = NBLK_H / NW;
        constexpr int STAGE_H = NBLK_H * 1024;
        constexpr int NS_H = (NS * STAGE) / STAGE_H < 8 ? (NS * STAGE) / STAGE_H : 8;
        static_assert(NS_H >= NS && NS_H * STAGE_H <= NS * STAGE, "the half-tile ring fits the ring");
        const int8_t* hsrc[DPW_H];
        int hstride[DPW_H];
#pragma unroll
        for (int i = 0; i < DPW_H; ++i) {
            const int b = wave + NW * i;
            if (b < FM) {  // activation rows b*16 .. b*16+15, swizzled as in the full tile
                int64_t r = row0 + b * 16 + (lane >> 2);
                if (r >= row_end) r = row0;
                int64_t src_row = r;
                if (GATHER)
                    src_row = min(max((int64_t)(p.sorted_assign[r] / p.topk), (int64_t)0), p.a_rows - 1);
                hsrc[i] = p.A + src_row * K + (((lane & 3) ^ ((lane >> 4) & 3)) * 16);
                hstride[i] = 64;
            } else {
                const int nb = nt * NBB + (b - FM);
                hsrc[i] = p.B + (int64_t)g * p.b_group_bytes + (int64_t)nb * KB * 1024 + lane * 16;
                hstride[i] = 1024;
            }
        }
        auto issue_h = [&](int ks) {
            const LDS_AS int8_t* stage = lds + (ks % NS_H) * STAGE_H;
#pragma unroll
            for (int i = 0; i < DPW_H; ++i)
                dma16(hsrc[i] + (int64_t)ks * hstride[i], stage + (wave + NW * i) * 1024);
        };
        if constexpr (!M32) {
            auto frag_a_h = [&](int ks, int i) {
                return *reinterpret_cast<const LDS_AS v4i*>(lds + (ks % NS_H) * STAGE_H + i * 1024 + a_slot * 16);
            };
            auto frag_b_h = [&](int ks, int j) {
                return *reinterpret_cast<const LDS_AS v4i*>(lds + (ks % NS_H) * STAGE_H +
                                                            (FM + b_base + j) * 1024 + lane * 16);
            };
            // prologue: NS_H-1 stages in flight, stage 0's fragments in registers
#pragma unroll
            for (int s = 0; s < NS_H - 1; ++s)
                if (s < nk) issue_h(s);
            if (nk - 1 >= NS_H - 2) wait_vmcnt<(NS_H - 2) * DPW_H>();
            else wait_vmcnt<0>();
            barrier_nofence();
#pragma unroll
            for (int i = 0; i < F; ++i) fa[i] = frag_a_h(0, i);
#pragma unroll
            for (int j = 0; j < NF; ++j) fb[j] = frag_b_h(0, j);
            AccT acc[FM][FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j) acc[i][j] = AccT{};
            auto mma_refill = [&](int next_ks, bool refill) {
#pragma unroll
                for (int i = 0; i < F; ++i) {
#pragma unroll
                    for (int j = 0; j < NF; ++j) acc[i][j] = mma16<CODE>(fa[i], fb[j], acc[i][j]);
                    if (refill) fa[i] = frag_a_h(next_ks, i);
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            int ks = 0;
            // steady state: stage ks+1 landed (NS_H-3 newer stages may still fly)
            for (; ks + NS_H - 1 < nk; ++ks) {
                wait_vmcnt<(NS_H - 3) * DPW_H>();
                barrier_nofence();
                issue_h(ks + NS_H - 1);
                mma_refill(ks + 1, true);
#pragma unroll
                for (int j = 0; j < NF; ++j) fb[j] = frag_b_h(ks + 1, j);
            }
            // drain: nothing left to issue
            for (; ks + 1 < nk; ++ks) {
                wait_vmcnt<0>();
                barrier_nofence();
                mma_refill(ks + 1, true);
#pragma unroll
                for (int j = 0; j < NF; ++j) fb[j] = frag_b_h(ks + 1, j);
            }
            mma_refill(0, false);
            epilogue(acc, std::integral_constant<int, NF>{});
        } else {
            // FP8: 32x32x64 blocks, each wave on all FM*16 rows (F blocks of 32)
            // and NF/2 blocks of 32 columns, fragments read as in the full tile
            constexpr int NJ = NF / 2 > 0 ? NF / 2 : 1;  // (NF is even wherever this runs)
            auto frag_a32_h = [&](int ks, int i) {
                const int blk = 2 * i + ((lane >> 4) & 1);
                const int rr = lane & 15, hh = lane >> 5;
                const LDS_AS int8_t* base = lds + (ks % NS_H) * STAGE_H + blk * 1024;
                v8i t;
                t.lo = *reinterpret_cast<const LDS_AS v4i*>(base + (4 * rr + ((2 * hh) ^ (rr >> 2))) * 16);
                t.hi = *reinterpret_cast<const LDS_AS v4i*>(base + (4 * rr + ((2 * hh + 1) ^ (rr >> 2))) * 16);
                return t;
            };
            auto frag_b32_h = [&](int ks, int j) {
                const int blk = FM + b_base + 2 * j + ((lane >> 4) & 1);
                const int cc = lane & 15, hh = lane >> 5;
                const LDS_AS int8_t* base = lds + (ks % NS_H) * STAGE_H + blk * 1024;
                v8i t;
                t.lo = *reinterpret_cast<const LDS_AS v4i*>(base + (cc + 32 * hh) * 16);
                t.hi = *reinterpret_cast<const LDS_AS v4i*>(base + (cc + 32 * hh + 16) * 16);
                return t;
            };
#pragma unroll
            for (int s = 0; s < NS_H - 1; ++s)
                if (s < nk) issue_h(s);
            if (nk - 1 >= NS_H - 2) wait_vmcnt<(NS_H - 2) * DPW_H>();
            else wait_vmcnt<0>();
            barrier_nofence();
#pragma unroll
            for (int i = 0; i < F; ++i) fa32[i] = frag_a32_h(0, i);
#pragma unroll
            for (int j = 0; j < NJ; ++j) fb32[j] = frag_b32_h(0, j);
            v4f acc[M32 ? FM32 : 1][NJ][4];
#pragma unroll
            for (int i = 0; i < FM32; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[i][j][c] = v4f{0.f, 0.f, 0.f, 0.f};
            auto mma_refill = [&](int next_ks, bool refill) {
#pragma unroll
                for (int i = 0; i < F; ++i) {
#pragma unroll
                    for (int j = 0; j < NJ; ++j) mma32<CODE>(fa32[i], fb32[j], acc[i][j]);
                    if (refill) fa32[i] = frag_a32_h(next_ks, i);
                    __builtin_amdgcn_sched_barrier(0);
                }
            };
            int ks = 0;
            for (; ks + NS_H - 1 < nk; ++ks) {
                wait_vmcnt<(NS_H - 3) * DPW_H>();
                barrier_nofence();
                issue_h(ks + NS_H - 1);
                mma_refill(ks + 1, true);
#pragma unroll
                for (int j = 0; j < NJ; ++j) fb32[j] = frag_b32_h(ks + 1, j);
            }
            for (; ks + 1 < nk; ++ks) {
                wait_vmcnt<0>();
                barrier_nofence();
                mma_refill(ks + 1, true);
#pragma unroll
                for (int j = 0; j < NJ; ++j) fb32[j] = frag_b32_h(ks + 1, j);
            }
            mma_refill(0, false);
            epilogue32(acc, std::integral_constant<int, NJ>{});
        }
    };
    bool done = false;
    if constexpr (HALF_OK) {
        if (half) {
            if (fm_active > FM / 2) run_half(std::integral_constant<int, M32 ? FM32 : FM>{});
            else run_half(std::integral_constant<int, M32 ? FM32 / 2 : FM / 2>{});
            done = true;
        }
    }
    if (!done) {
        if constexpr (M32) {
            // FP8: stage ks's MFMAs run from registers while stage ks+1's fragments
            // come in (each A fragment row right after its MFMAs, B after the
            // stage's MFMAs), as in the INT8 loop.  F = 32-row fragment rows computed.
            auto run32 = [&](auto f_tag) {
                constexpr int F = decltype(f_tag)::value;
                v4f acc[M32 ? FM32 : 1][M32 ? FN32 : 1][4];
#pragma unroll
                for (int i = 0; i < FM32; ++i)
#pragma unroll
                    for (int j = 0; j < FN32; ++j)
#pragma unroll
                        for (int c = 0; c < 4; ++c) acc[i][j][c] = v4f{0.f, 0.f, 0.f, 0.f};
                auto mma_refill = [&](int next_ks, bool refill) {
#pragma unroll
                    for (int i = 0; i < F; ++i) {
#pragma unroll
                        for (int j = 0; j < FN32; ++j) mma32<CODE>(fa32[i], fb32[j], acc[i][j]);
                        if (refill) fa32[i] = frag_a32(next_ks, i);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                };
                int ks = 0;
                for (; ks + NS - 1 < nk; ++ks) {
                    wait_vmcnt<(NS - 3) * DPW>();
                    barrier_nofence();
                    issue(ks + NS - 1);
                    mma_refill(ks + 1, true);
                    if (F > 0) {
#pragma unroll
                        for (int j = 0; j < FN32; ++j) fb32[j] = frag_b32(ks + 1, j);
                    }
                }
                for (; ks + 1 < nk; ++ks) {
                    wait_vmcnt<0>();
                    barrier_nofence();
                    mma_refill(ks + 1, true);
                    if (F > 0) {
#pragma unroll
                        for (int j = 0; j < FN32; ++j) fb32[j] = frag_b32(ks + 1, j);
                    }
                }
                mma_refill(0, false);
                epilogue32(acc, std::integral_constant<int, FN32>{});
            };
            if (fm_active > FM / 2) run32(std::integral_constant<int, FM32>{});
            else if (fm_active > 0) run32(std::integral_constant<int, FM32 / 2>{});
            else run32(std::integral_constant<int, 0>{});
        } else {
            if (fm_active > FM / 2) run(std::integral_constant<int, FM>{});
            else if (fm_active > 0) run(std::integral_constant<int, FM / 2>{});
            else run(std::integral_constant<int, 0>{});
        }
    }
    };

    // Tile schedule.  Static (no counters): slot s of XCD x takes tiles s,
    // s + slots, ... of the XCD's range (one tile per workgroup when the grid
    // covers every tile).  Persistent (tile_ctr): each XCD's range is a queue
    // (a counter the routing zeroed); a workgroup takes the next tile of its
    // own XCD's queue and, once that is empty, helps drain the others, so
    // every tile is taken exactly once whatever the number of workgroups per
    // XCD.  The claim of the next tile is issued when a tile's epilogue
    // starts and read when the tile ends (claim_next above).
    const int xcd = blockIdx.x & 7;
    const int64_t slots = gridDim.x >> 3;
    // queue xq: tiles [queue_beg(xq), queue_beg(xq) + queue_len(xq)) -- equal
    // tile counts, or the routing's work-balanced bounds (persistent grouped)
    const bool balanced = p.tile_ctr && p.xcd_bounds;
    auto queue_beg = [&](int xq) -> int64_t {
        return balanced ? (int64_t)p.xcd_bounds[xq] : min(total, (int64_t)xq * per_xcd);
    };
    auto queue_len = [&](int xq) -> int64_t {
        return balanced ? (int64_t)(p.xcd_bounds[xq + 1] - p.xcd_bounds[xq])
                        : min(per_xcd, max((int64_t)0, total - (int64_t)xq * per_xcd));
    };
    auto next_after = [&](int got_own) -> int {
        if (got_own < queue_len(xcd)) return (int)(queue_beg(xcd) + got_own);
        for (int q = 1; q < 8; ++q) {
            const int xq = (xcd + q) & 7;
            if (queue_len(xq) == 0) continue;
            const int got = atomicAdd(p.tile_ctr + TILE_CTR_STRIDE * xq, 1);
            if (got < queue_len(xq)) return (int)(queue_beg(xq) + got);
        }
        return -1;
    };
    int64_t sl = blockIdx.x >> 3;  // static slot
    int64_t L;
    if (!p.tile_ctr) {
        L = (sl < queue_len(xcd)) ? queue_beg(xcd) + sl : -1;
    } else {
        if (tid0 == 0) next_tile[0] = next_after(atomicAdd(p.tile_ctr + TILE_CTR_STRIDE * xcd, 1));
        __syncthreads();
        // uniform: keeps every per-tile value in scalar registers
        L = __builtin_amdgcn_readfirstlane(next_tile[0]);
    }
    while (L >= 0) {
        process(L);  // claims the next tile at its epilogue (claim_got)
        __syncthreads();  // every wave is done with the ring, the row metadata and next_tile
        if (!p.tile_ctr) {
            sl += slots;
            L = (sl < queue_len(xcd)) ? queue_beg(xcd) + sl : -1;
        } else {
            if (tid0 == 0) next_tile[0] = next_after(claim_got);
            __syncthreads();
            L = __builtin_amdgcn_readfirstlane(next_tile[0]);
        }
    }
}

template <int BM, int BN, int WM, int WN, int NS>
hipError_t launch_tile(int epi, const GemmParams& p, int64_t blocks, hipStream_t s) {
    const dim3 grid((unsigned)blocks), block(WM * WN * 64);
    if (p.code == CODE_FP8) {
        switch (epi) {
            case EPI_DENSE_F32: gemm_i8<BM, BN, WM, WN, NS, EPI_DENSE_F32, CODE_FP8><<<grid, block, 0, s>>>(p); break;
            case EPI_GATE_UP: gemm_i8<BM, BN, WM, WN, NS, EPI_GATE_UP, CODE_FP8><<<grid, block, 0, s>>>(p); break;
            case EPI_DOWN: gemm_i8<BM, BN, WM, WN, NS, EPI_DOWN, CODE_FP8><<<grid, block, 0, s>>>(p); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    if (p.code == CODE_FP8_FAST) {
        switch (epi) {
            case EPI_DENSE_F32: gemm_i8<BM, BN, WM, WN, NS, EPI_DENSE_F32, CODE_FP8_FAST><<<grid, block, 0, s>>>(p); break;
            case EPI_GATE_UP: gemm_i8<BM, BN, WM, WN, NS, EPI_GATE_UP, CODE_FP8_FAST><<<grid, block, 0, s>>>(p); break;
            case EPI_DOWN: gemm_i8<BM, BN, WM, WN, NS, EPI_DOWN, CODE_FP8_FAST><<<grid, block, 0, s>>>(p); break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    if (p.code != CODE_INT8) return hipErrorInvalidValue;
    switch (epi) {
        case EPI_DENSE_F32: gemm_i8<BM, BN, WM, WN, NS, EPI_DENSE_F32, CODE_INT8><<<grid, block, 0, s>>>(p); break;
        case EPI_DENSE_I32: gemm_i8<BM, BN, WM, WN, NS, EPI_DENSE_I32, CODE_INT8><<<grid, block, 0, s>>>(p); break;
        case EPI_GATE_UP: gemm_i8<BM, BN, WM, WN, NS, EPI_GATE_UP, CODE_INT8><<<grid, block, 0, s>>>(p); break;
        case EPI_DOWN: gemm_i8<BM, BN, WM, WN, NS, EPI_DOWN, CODE_INT8><<<grid, block, 0, s>>>(p); break;
        case EPI_GU_I32: gemm_i8<BM, BN, WM, WN, NS, EPI_GU_I32, CODE_INT8><<<grid, block, 0, s>>>(p); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

int gemm_tile_n(int64_t N, int /*code*/) { return (N % 256 == 0) ? 256 : 128; }

int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

hipError_t launch_gemm(int epi, const GemmParams& p_in, int64_t max_m_tiles, hipStream_t s) {
    GemmParams p = p_in;
    const int bn = gemm_tile_n(p.N, p.code);
    const int nt_all = (int)(p.N / bn);
    if (p.seg_offsets) {
        p.VG = 1;
        p.NTV = nt_all;
    } else {
        // dense: 8 column stripes (one per XCD) when the n-tiles divide evenly
        p.VG = (nt_all % 8 == 0) ? 8 : 1;
        p.NTV = nt_all / p.VG;
    }
    const int64_t max_tiles = max_m_tiles * nt_all;
    if (max_tiles == 0) return hipSuccess;
    // grouped: persistent, one workgroup per CU (the LDS ring allows one);
    // dense: one workgroup per tile
    int64_t blocks = 8 * ((max_tiles + 7) / 8);
    if (p.tile_ctr) {
        const int64_t cus = 8 * ((device_cu_count() + 7) / 8);
        if (cus < blocks) blocks = cus;
    }
    if (bn == 256) return launch_tile<GEMM_BM, 256, 2, 4, 4>(epi, p, blocks, s);
    return launch_tile<GEMM_BM, 128, 2, 4, 4>(epi, p, blocks, s);
}

}  // namespace w8a8
