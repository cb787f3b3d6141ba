// Large-M grouped expert GEMMs on CDNA4 MFMA (bf16 in, fp32 accumulate).
//
// The experts backend that sorts tokens by expert and runs one grouped GEMM
// over packed expert weights ("Transformer中的混合专家架构详解" page, experts
// backends section, grouped_mm) is re-designed here for gfx950:
//   * one persistent launch covers every expert; a device-side list of
//     M-tiles (rows of one expert, built by the routing kernels) replaces any
//     host read-back, and an expert with many rows simply owns many tiles,
//     so load imbalance is absorbed without padding experts or dropping
//     tokens (PhiMoE page, section 2, item 4);
//   * gate_up: a tile loads matching gate rows [n0, n0+BN/2) and up rows
//     [I+n0, I+n0+BN/2) of gate_up_proj, so silu(gate)*up is formed in
//     registers and only h is written (PhiMoE page, section 2, item 3);
//   * down: the epilogue multiplies each row by its routing weight and
//     writes it to that assignment's slot in token order (the weighted
//     un-permute); a later pass sums the k slots of each token in order.
//   * tiles are visited expert-major, then N-block, then M-tile, and each
//     XCD takes a contiguous run of tile ids per round, so the M-tiles that
//     share an expert's weight block run together on one XCD's L2.
#include "moe_internal.h"

#include <type_traits>

namespace moe {

namespace {

#ifndef MOE_TILED_BK
#define MOE_TILED_BK 32
#endif
#ifndef MOE_TILED_INTERLEAVE
#define MOE_TILED_INTERLEAVE 1
#endif
#ifndef MOE_TILED_STAGES
#define MOE_TILED_STAGES 4
#endif
constexpr int BK = MOE_TILED_BK;          // bf16 elements per k-stage (2*BK bytes per row)
constexpr int STAGES = MOE_TILED_STAGES;  // LDS ring depth
constexpr int CH = BK / 8;                // 16-byte chunks per row of a stage
constexpr int RPI = 64 / CH;              // rows filled by one 64-lane copy instruction
static_assert(CH == 4 || CH == 8, "stage rows of 64 or 128 bytes");

struct TiledParams {
    const __bf16 *A;
    const int32_t *a_rows;
    const __bf16 *W;
    int64_t w_expert_stride;
    int K;
    int N;
    void *C;
    const int32_t *c_rows;
    const float *c_scale;
    const MTile *tiles;
    const int32_t *tile_start;
    int E;
    int dense_rows;
    int NB;  // N-blocks
};

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void global_void_t;

// LDS stage layout: rows of CH chunks of 16 bytes; chunk c of row r sits at
// slot c ^ swz(r) with swz(r) = (r >> 2) & 3 for 64-byte rows and (r >> 1) & 7
// for 128-byte rows, so the 16 lanes a ds_read_b128 serves per cycle (16
// consecutive rows, one chunk column) hit 16 distinct 16-byte bank groups of
// the 64-bank LDS.
__device__ __forceinline__ int lds_swz(int r) { return CH == 4 ? ((r >> 2) & 3) : ((r >> 1) & 7); }
__device__ __forceinline__ int lds_slot(int r, int c) { return r * CH + (c ^ lds_swz(r)); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Wait until at most N vector-memory operations of this wave are outstanding
// (global_load_lds stages are counted there), then barrier. The memory clobber
// keeps the compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void wait_vm_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Direct-to-LDS copy of 16 bytes per lane: lane i writes LDS bytes
// [lds + 16 i, lds + 16 i + 16). Issued from inline assembly so that the
// compiler does not treat every later LDS read as possibly aliasing the copy
// (it would wait for all copies in flight before each read and serialize the
// ring); completion is tracked by wait_vm_barrier's explicit vmcnt instead.
// The copy has no register result; it only reads the address operands.
__device__ __forceinline__ void dma16(const void *gptr, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds)
                 : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) { return (uint32_t)(uintptr_t)p; }

template <int BM, int BN, int WM, int WN, int OCC, bool GATEUP>
__global__ __launch_bounds__(WM *WN * 64, OCC) void tiled_gemm_kernel(TiledParams p)
{
    constexpr int NT = WM * WN * 64;
    constexpr int NWAVE = WM * WN;
    constexpr int RM = BM / WM / 32;
    constexpr int RN = BN / WN / 32;
    constexpr int A_INS = BM / RPI / NWAVE;  // copy instructions per wave per stage
    constexpr int B_INS = BN / RPI / NWAVE;
    constexpr int LOADS = A_INS + B_INS;    // vector-memory ops per wave per stage
    static_assert(A_INS >= 1 && B_INS >= 1 && RM >= 1 && RN >= 1, "tile shape");
    static_assert(!GATEUP || (RN % 2 == 0), "gate/up pairing needs an even RN");

    __shared__ u32x4 sA[STAGES][BM * CH];
    __shared__ u32x4 sB[STAGES][BN * CH];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int wm = wave / WN;
    const int wn = wave - wm * WN;

    // first M-tile of each expert (read through the scalar cache, so the
    // whole LDS is left to the stage ring)
    const int32_t *s_ts = p.tile_start;
    int n_mtiles;
    if (p.tiles) {
        n_mtiles = s_ts[p.E];
    } else {
        n_mtiles = (p.dense_rows + BM - 1) / BM;
    }
    const int total = n_mtiles * p.NB;
    const int G = gridDim.x;
    const int nx = G >> 3;
    const int xcd = blockIdx.x & 7;
    const int li = blockIdx.x >> 3;
    const int nk = (p.K + BK - 1) / BK;

    // copy geometry: instruction i of this wave fills LDS rows
    // RPI*(wave*INS + i) + lane/CH, chunk slot lane%CH (logical chunk lc below)
    const int drow = lane / CH;

    for (int r = 0;; r++) {
        const int id = r * G + xcd * nx + li;
        if (id >= total) break;

        // ---- decode tile id -> (expert, M-tile, N-block)
        int e, nb, row0, rows;
        if (p.tiles) {
            int lo = 0, hi = p.E;  // find e: s_ts[e]*NB <= id < s_ts[e+1]*NB
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (s_ts[mid] * p.NB <= id) lo = mid; else hi = mid;
            }
            e = lo;
            const int nte = s_ts[e + 1] - s_ts[e];
            const int local = id - s_ts[e] * p.NB;
            nb = local / nte;
            const MTile t = p.tiles[s_ts[e] + (local - nb * nte)];
            row0 = t.row0;
            rows = t.rows;
        } else {
            e = 0;
            nb = id / n_mtiles;
            const int mt = id - nb * n_mtiles;
            row0 = mt * BM;
            rows = min(BM, p.dense_rows - row0);
        }

        // ---- per-lane DMA source rows (rows past the tile repeat row 0; dropped later)
        const __bf16 *asrc[A_INS];
        int alc[A_INS];
#pragma unroll
        for (int i = 0; i < A_INS; i++) {
            const int rr = RPI * (wave * A_INS + i) + drow;
            const int rc = rr < rows ? rr : 0;
            const int64_t src = p.a_rows ? (int64_t)p.a_rows[row0 + rc] : (int64_t)(row0 + rc);
            alc[i] = (lane % CH) ^ lds_swz(rr);
            asrc[i] = p.A + src * p.K + alc[i] * 8;
        }
        const __bf16 *wbase = p.W + (int64_t)e * p.w_expert_stride;
        const __bf16 *bsrc[B_INS];
        int blc[B_INS];
#pragma unroll
        for (int i = 0; i < B_INS; i++) {
            const int rr = RPI * (wave * B_INS + i) + drow;
            int wrow;
            if (GATEUP) {
                const int half = BN / 2;
                const int n = nb * half + (rr < half ? rr : rr - half);
                const int nc = n < p.N ? n : 0;
                wrow = rr < half ? nc : p.N + nc;
            } else {
                const int n = nb * BN + rr;
                wrow = n < p.N ? n : 0;
            }
            blc[i] = (lane % CH) ^ lds_swz(rr);
            bsrc[i] = wbase + (int64_t)wrow * p.K + blc[i] * 8;
        }

        // stage kt -> LDS buffer b: every lane copies 16 bytes. Only a final
        // partial stage (K not a multiple of BK) masks lanes; they zero-fill.
        auto issue = [&](int kt, int b) {
            const int k0 = kt * BK;
#pragma unroll
            for (int i = 0; i < A_INS; i++)
                dma16(asrc[i] + k0, lds_addr(&sA[b][(wave * A_INS + i) * 64]));
#pragma unroll
            for (int i = 0; i < B_INS; i++)
                dma16(bsrc[i] + k0, lds_addr(&sB[b][(wave * B_INS + i) * 64]));
        };
        auto issue_tail = [&](int kt, int b) {
            const int k0 = kt * BK;
#pragma unroll
            for (int i = 0; i < A_INS; i++) {
                u32x4 *dst = &sA[b][(wave * A_INS + i) * 64];
                if (k0 + alc[i] * 8 < p.K)
                    dma16(asrc[i] + k0, lds_addr(dst));
                else
                    dst[lane] = u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int i = 0; i < B_INS; i++) {
                u32x4 *dst = &sB[b][(wave * B_INS + i) * 64];
                if (k0 + blc[i] * 8 < p.K)
                    dma16(bsrc[i] + k0, lds_addr(dst));
                else
                    dst[lane] = u32x4{0u, 0u, 0u, 0u};
            }
        };
        const bool ragged = (p.K % BK) != 0;
        auto issue_any = [&](int kt, int b) {
            if (ragged && kt == nk - 1) issue_tail(kt, b);
            else issue(kt, b);
        };

        f32x16_t acc[RM][RN];
#pragma unroll
        for (int i = 0; i < RM; i++)
#pragma unroll
            for (int j = 0; j < RN; j++)
#pragma unroll
                for (int q = 0; q < 16; q++) acc[i][j][q] = 0.0f;

        // copy instruction q (A rows first, then B rows) of stage kt into buffer b
        auto issue_one = [&](int kt, int b, int q) {
            const int k0 = kt * BK;
            if (q < A_INS) dma16(asrc[q] + k0, lds_addr(&sA[b][(wave * A_INS + q) * 64]));
            else dma16(bsrc[q - A_INS] + k0, lds_addr(&sB[b][(wave * B_INS + q - A_INS) * 64]));
        };
        // Consume stage buffer b. When nkt >= 0, the copies of stage nkt into
        // buffer nb are spread between the MFMAs, one copy per MFMA_PER_COPY
        // MFMAs, so the copy engine never holds up the fragment reads.
        // NB (compile time): how many of this wave's RM 32-row blocks hold
        // rows of the tile; the rest skip their fragment reads and MFMAs, so
        // the short last tile of an expert costs less than a full one. The
        // copies keep their slots either way.
        auto compute_with = [&](auto nbc, int b, int nkt, int nb) {
            constexpr int NB = decltype(nbc)::value;
            constexpr int NMMA = (BK / 16) * RM * RN;
            constexpr int PER = NMMA / LOADS > 0 ? NMMA / LOADS : 1;
            static_assert(PER * LOADS <= NMMA, "every copy finds an MFMA slot");
#pragma unroll
            for (int kk = 0; kk < BK / 16; kk++) {
                bf16x8_t af[RM], bf[RN];
                const int c = kk * 2 + (lane >> 5);
#pragma unroll
                for (int i = 0; i < NB; i++) {
                    const int row = wm * (BM / WM) + i * 32 + (lane & 31);
                    af[i] = as_bf16x8(sA[b][lds_slot(row, c)]);
                }
#pragma unroll
                for (int j = 0; j < RN; j++) {
                    if (NB == 0) break;
                    int row;
                    if (GATEUP) {
                        constexpr int HW = BN / 2 / WN;
                        row = (j < RN / 2) ? wn * HW + j * 32 : BN / 2 + wn * HW + (j - RN / 2) * 32;
                    } else {
                        row = wn * (BN / WN) + j * 32;
                    }
                    row += lane & 31;
                    bf[j] = as_bf16x8(sB[b][lds_slot(row, c)]);
                }
#pragma unroll
                for (int i = 0; i < RM; i++)
#pragma unroll
                    for (int j = 0; j < RN; j++) {
                        if (i < NB)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
                        const int mi = (kk * RM + i) * RN + j;  // compile-time after unrolling
                        if ((mi + 1) % PER == 0 && (mi + 1) / PER - 1 < LOADS) issue_one(nkt, nb, (mi + 1) / PER - 1);
                    }
            }
        };
        // 32-row blocks of this wave that hold rows of the tile (wave-uniform)
        const int nvb = max(0, min(RM, (rows - wm * (BM / WM) + 31) / 32));
        auto compute = [&](int b) {
            if (nvb == 0) return;
#pragma unroll
            for (int kk = 0; kk < BK / 16; kk++) {
                bf16x8_t af[RM], bf[RN];
                const int c = kk * 2 + (lane >> 5);
#pragma unroll
                for (int i = 0; i < RM; i++) {
                    const int row = wm * (BM / WM) + i * 32 + (lane & 31);
                    if (i < nvb) af[i] = as_bf16x8(sA[b][lds_slot(row, c)]);
                }
#pragma unroll
                for (int j = 0; j < RN; j++) {
                    int row;
                    if (GATEUP) {
                        constexpr int HW = BN / 2 / WN;  // gate (or up) rows per wave
                        row = (j < RN / 2) ? wn * HW + j * 32 : BN / 2 + wn * HW + (j - RN / 2) * 32;
                    } else {
                        row = wn * (BN / WN) + j * 32;
                    }
                    row += lane & 31;
                    bf[j] = as_bf16x8(sB[b][lds_slot(row, c)]);
                }
#pragma unroll
                for (int i = 0; i < RM; i++)
#pragma unroll
                    for (int j = 0; j < RN; j++)
                        if (i < nvb) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
            }
        };

        // all waves are done with the previous tile's stages before refilling them
        wait_vm_barrier<0>();
#pragma unroll
        for (int s = 0; s < STAGES - 1; s++)
            if (s < nk) issue_any(s, s);

        // Steady state: stage kt is consumed while stages kt+1, kt+2 are in
        // flight and stage kt+3 is issued into the buffer stage kt-1 used.
        // Unrolled by STAGES so every buffer index is a compile-time constant.
        // (a ragged last stage is always left to the drain)
        int kt = 0;
        const int steady_last = nk - (ragged ? 1 : 0);
        auto steady = [&](auto nbc) {
            for (; kt + 2 * STAGES - 1 <= steady_last; kt += STAGES) {
#pragma unroll
                for (int b = 0; b < STAGES; b++) {
                    wait_vm_barrier<(STAGES - 2) * LOADS>();
                    const int nkt = kt + b + STAGES - 1, nb = (b + STAGES - 1) % STAGES;
#if MOE_TILED_INTERLEAVE
                    compute_with(nbc, b, nkt, nb);
#else
                    issue(nkt, nb);
                    compute(b);
#endif
                }
            }
        };
        // one copy of the loop per number of live 32-row blocks (RM is 1 or 2)
        static_assert(RM <= 2, "steady-state variants for up to two 32-row blocks per wave");
        if (nvb >= RM) steady(std::integral_constant<int, RM>{});
        else if (nvb == 1) steady(std::integral_constant<int, 1>{});
        else steady(std::integral_constant<int, 0>{});
        // Drain: fewer than 2*STAGES-1 stages remain (kt is a multiple of STAGES,
        // so stage kt + b lives in buffer b).
#pragma unroll
        for (int b = 0; b < 2 * STAGES - 1; b++) {
            if (kt + b >= nk) break;
            const int ahead = min(STAGES - 2, nk - 1 - (kt + b));
            if (ahead >= 2 && STAGES >= 4) wait_vm_barrier<(STAGES >= 4 ? 2 : 0) * LOADS>();
            else if (ahead == 1) wait_vm_barrier<LOADS>();
            else wait_vm_barrier<0>();
            if (kt + b + STAGES - 1 < nk) issue_any(kt + b + STAGES - 1, (b + STAGES - 1) % STAGES);
            compute(b % STAGES);
        }

        // ---- epilogue
        if (GATEUP) {
            constexpr int HW = BN / 2 / WN;
            __bf16 *H = reinterpret_cast<__bf16 *>(p.C);
#pragma unroll
            for (int i = 0; i < RM; i++)
#pragma unroll
                for (int j = 0; j < RN / 2; j++) {
                    const int c = nb * (BN / 2) + wn * HW + j * 32 + (lane & 31);
#pragma unroll
                    for (int q = 0; q < 16; q++) {
                        const int rr = wm * (BM / WM) + i * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                        if (rr < rows && c < p.N) {
                            const float g = acc[i][j][q];
                            const float u = acc[i][j + RN / 2][q];
                            const uint32_t hb = f32_to_bf16_bits(silu_f32(g) * u);
                            reinterpret_cast<uint16_t *>(H)[(int64_t)(row0 + rr) * p.N + c] = (uint16_t)hb;
                        }
                    }
                }
        } else {
            float *Y = reinterpret_cast<float *>(p.C);
#pragma unroll
            for (int i = 0; i < RM; i++)
#pragma unroll
                for (int q = 0; q < 16; q++) {
                    const int rr = wm * (BM / WM) + i * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                    if (rr < rows) {
                        const int pos = row0 + rr;
                        const int64_t orow = p.c_rows ? (int64_t)p.c_rows[pos] : (int64_t)pos;
                        const float sc = p.c_scale ? p.c_scale[pos] : 1.0f;
#pragma unroll
                        for (int j = 0; j < RN; j++) {
                            const int m = nb * BN + wn * (BN / WN) + j * 32 + (lane & 31);
                            if (m < p.N) Y[orow * p.N + m] = acc[i][j][q] * sc;
                        }
                    }
                }
        }
    }
}

// Software-pipelined variant: 4 waves (one per SIMD), 128 tokens x 128
// weight rows per wave (accumulators live in AGPRs), fragments
// double-buffered across the two 16-wide halves of a stage, with the barrier
// between the halves and each stage's copies split over both halves (the
// schedule is spelled out above the steady-state loop). Per stage it reads
// 64 KB of fragments from LDS against 96 KB for the 8-wave kernel; it is
// faster on the balanced prefill shapes and slower on the down GEMM of
// skewed routing, so it is off by default. The MFMA takes weight rows as its A operand and tokens as B, so a lane of
// the 32x32 result holds one token and 4 consecutive output columns per
// group of 4 registers: the epilogue writes packed 8-byte (h) or 16-byte
// (weighted fp32 slot) chunks and looks up each token's row once.
template <int BM, int BN, bool GATEUP>
__global__ __launch_bounds__(256) void tiled_pp_kernel(TiledParams p)
{
    constexpr int WM = 2, WN = 2, NT = 256, NWAVE = 4;
    constexpr int RT = BM / WM / 32;  // 32-token blocks per wave
    constexpr int RW = BN / WN / 32;  // 32-weight-row blocks per wave
    constexpr int A_INS = BM / RPI / NWAVE;
    constexpr int B_INS = BN / RPI / NWAVE;
    constexpr int LOADS = A_INS + B_INS;
    static_assert(!GATEUP || (RW % 2 == 0), "gate/up pairing needs an even RW");

    static_assert(BK == 32 && STAGES >= 3, "the pipelined schedule reads two 16-wide halves per stage");
    __shared__ u32x4 sA[STAGES][BM * CH];  // token rows
    __shared__ u32x4 sB[STAGES][BN * CH];  // weight rows

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int wm = wave / WN;
    const int wn = wave - wm * WN;

    // first M-tile of each expert (read through the scalar cache, so the
    // whole LDS is left to the stage ring)
    const int32_t *s_ts = p.tile_start;
    int n_mtiles;
    if (p.tiles) {
        n_mtiles = s_ts[p.E];
    } else {
        n_mtiles = (p.dense_rows + BM - 1) / BM;
    }
    const int total = n_mtiles * p.NB;
    const int G = gridDim.x;
    const int nx = G >> 3;
    const int xcd = blockIdx.x & 7;
    const int li = blockIdx.x >> 3;
    const int nk = (p.K + BK - 1) / BK;
    const bool ragged = (p.K % BK) != 0;
    const int drow = lane / CH;

    // Fragment addressing. Every fragment row is (multiple of 32) + lane%32, so
    // the swizzle term depends on the lane only and a fragment's LDS index is
    // (block row + lane row) * CH + (chunk ^ swizzle): the block part is a
    // compile-time constant per block.
    const int sw = lds_swz(lane & 31);
    const int lrow = (lane & 31) * CH;
    int xo[BK / 16];
#pragma unroll
    for (int h = 0; h < BK / 16; h++) xo[h] = lrow + ((2 * h + (lane >> 5)) ^ sw);
    auto t_blk = [&](int i) { return (wm * (BM / WM) + i * 32) * CH; };
    auto w_blk = [&](int j) {
        int row;
        if (GATEUP) {
            constexpr int HW = BN / 2 / WN;
            row = (j < RW / 2) ? wn * HW + j * 32 : BN / 2 + wn * HW + (j - RW / 2) * 32;
        } else {
            row = wn * (BN / WN) + j * 32;
        }
        return row * CH;
    };

    for (int r = 0;; r++) {
        const int id = r * G + xcd * nx + li;
        if (id >= total) break;

        int e, nb, row0, rows;
        if (p.tiles) {
            int lo = 0, hi = p.E;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (s_ts[mid] * p.NB <= id) lo = mid; else hi = mid;
            }
            e = lo;
            const int nte = s_ts[e + 1] - s_ts[e];
            const int local = id - s_ts[e] * p.NB;
            nb = local / nte;
            const MTile t = p.tiles[s_ts[e] + (local - nb * nte)];
            row0 = t.row0;
            rows = t.rows;
        } else {
            e = 0;
            nb = id / n_mtiles;
            const int mt = id - nb * n_mtiles;
            row0 = mt * BM;
            rows = min(BM, p.dense_rows - row0);
        }

        // element offsets of the lane's DMA rows: activations are < 2^31
        // elements and one expert's weights are < 2^31 elements (host checks)
        uint32_t aoff[A_INS];
        int alc[A_INS];
#pragma unroll
        for (int i = 0; i < A_INS; i++) {
            const int rr = RPI * (wave * A_INS + i) + drow;
            const int rc = rr < rows ? rr : 0;
            const uint32_t src = p.a_rows ? (uint32_t)p.a_rows[row0 + rc] : (uint32_t)(row0 + rc);
            alc[i] = (lane % CH) ^ lds_swz(rr);
            aoff[i] = src * (uint32_t)p.K + alc[i] * 8;
        }
        const __bf16 *wbase = p.W + (int64_t)e * p.w_expert_stride;
        uint32_t boff[B_INS];
        int blc[B_INS];
#pragma unroll
        for (int i = 0; i < B_INS; i++) {
            const int rr = RPI * (wave * B_INS + i) + drow;
            int wrow;
            if (GATEUP) {
                const int half = BN / 2;
                const int n = nb * half + (rr < half ? rr : rr - half);
                const int nc = n < p.N ? n : 0;
                wrow = rr < half ? nc : p.N + nc;
            } else {
                const int n = nb * BN + rr;
                wrow = n < p.N ? n : 0;
            }
            blc[i] = (lane % CH) ^ lds_swz(rr);
            boff[i] = (uint32_t)wrow * (uint32_t)p.K + blc[i] * 8;
        }

        // copy q (A rows first, then B rows; 64 chunks of 16 bytes each) of
        // stage kt into buffer b. Only a final partial stage masks lanes (they
        // zero-fill); every copy instruction still issues, since chunk 0 of
        // each of its rows is always in range, so each stage is exactly
        // LOADS vector-memory operations for the vmcnt waits below.
        auto copy_full = [&](int kt, int b, int q) {
            const int k0 = kt * BK;
            if (q < A_INS) dma16(p.A + aoff[q] + k0, lds_addr(&sA[b][(wave * A_INS + q) * 64]));
            else dma16(wbase + boff[q - A_INS] + k0, lds_addr(&sB[b][(wave * B_INS + q - A_INS) * 64]));
        };
        auto copy_any = [&](int kt, int b, int q) {
            if (ragged && kt == nk - 1) {
                const int k0 = kt * BK;
                u32x4 *dst = q < A_INS ? &sA[b][(wave * A_INS + q) * 64] : &sB[b][(wave * B_INS + q - A_INS) * 64];
                const int lc = q < A_INS ? alc[q] : blc[q - A_INS];
                if (k0 + lc * 8 < p.K)
                    dma16(q < A_INS ? (const void *)(p.A + aoff[q] + k0) : (const void *)(wbase + boff[q - A_INS] + k0),
                          lds_addr(dst));
                else
                    dst[lane] = u32x4{0u, 0u, 0u, 0u};
            } else {
                copy_full(kt, b, q);
            }
        };

        f32x16_t acc[RW][RT];
#pragma unroll
        for (int j = 0; j < RW; j++)
#pragma unroll
            for (int i = 0; i < RT; i++)
#pragma unroll
                for (int q = 0; q < 16; q++) acc[j][i][q] = 0.0f;

        bf16x8_t ft[2][RT], fw[2][RW];
        // fragments of half h (k16 step) of the stage in buffer b into set f
        auto frag = [&](int b, int h, int f) {
            const u32x4 *pa = &sA[b][xo[h]];
            const u32x4 *pb = &sB[b][xo[h]];
#pragma unroll
            for (int i = 0; i < RT; i++) ft[f][i] = as_bf16x8(pa[t_blk(i)]);
#pragma unroll
            for (int j = 0; j < RW; j++) fw[f][j] = as_bf16x8(pb[w_blk(j)]);
        };
        // MFMAs of fragment set f. With copies, copies q0 .. q0+HALF-1 of
        // stage nkt into buffer nbuf go out between them, one every PER MFMAs
        // (compile-time slots), so the vector-memory path is fed evenly.
        constexpr int HALF = LOADS / 2;
        static_assert(LOADS % 2 == 0, "copies split evenly over the two halves of a stage");
        auto mma = [&](int f, bool copies, int nkt, int nbuf, int q0) {
            constexpr int NM = RW * RT;
            constexpr int PER = NM / HALF > 0 ? NM / HALF : 1;
            constexpr int INL = NM / PER < HALF ? NM / PER : HALF;
#pragma unroll
            for (int j = 0; j < RW; j++)
#pragma unroll
                for (int i = 0; i < RT; i++) {
                    const int mi = j * RT + i;  // compile-time after unrolling
                    if (copies && mi % PER == 0 && mi / PER < INL) copy_full(nkt, nbuf, q0 + mi / PER);
                    acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[f][j], ft[f][i], acc[j][i], 0, 0, 0);
                }
#pragma unroll
            for (int q = INL; q < HALF; q++)
                if (copies) copy_full(nkt, nbuf, q0 + q);
        };

        // One 16-wide half in steady state, in a fixed instruction order: the
        // MFMAs of fragment set f, one fragment read (half rh of buffer rb into
        // set g) after each of the first RT+RW MFMAs, and the copies q0 ..
        // q0+HALF-1 of stage nkt into buffer nbuf after every second MFMA of
        // the rest. Scheduling fences pin the order: left to itself the
        // compiler bunches the reads and the copies, and a wave that queues
        // many LDS or memory instructions at once stops issuing MFMAs.
        auto half_step = [&](int f, int rb, int rh, int g, int nkt, int nbuf, int q0) {
            constexpr int NM = RW * RT;
            constexpr int NR = RT + RW;
            static_assert(NR + 2 * HALF <= NM + 1, "reads and copies fit between the MFMAs");
            const u32x4 *pa = &sA[rb][xo[rh]];
            const u32x4 *pb = &sB[rb][xo[rh]];
            // read r after MFMA r; copy c after MFMA NR + 2c (compile-time slots)
            auto read_at = [&](int mi) { return mi < NR ? mi : -1; };
            auto copy_at = [&](int mi) {
                return ((mi - NR) >= 0 && (mi - NR) % 2 == 0 && (mi - NR) / 2 < HALF) ? (mi - NR) / 2 : -1;
            };
#pragma unroll
            for (int mi = 0; mi < NM; mi++) {
                const int j = mi / RT, i = mi % RT;
                acc[j][i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[f][j], ft[f][i], acc[j][i], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                const int r = read_at(mi);
                if (r >= 0 && r < RT) {
                    ft[g][r] = as_bf16x8(pa[t_blk(r)]);
                    __builtin_amdgcn_sched_barrier(0);
                } else if (r >= RT) {
                    fw[g][r - RT] = as_bf16x8(pb[w_blk(r - RT)]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                const int c = copy_at(mi);
                if (c >= 0) {
                    copy_full(nkt, nbuf, q0 + c);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };

        // Schedule of stage s (buffer s % STAGES). The barrier sits between
        // the two 16-wide halves: before it, the second half of s is read and
        // the first half's MFMAs run; after it (stage s+1 has landed and
        // every wave is done with buffer s), the first half of s+1 is read
        // while the second half's MFMAs run. Copies of stage s+STAGES go
        // into buffer s in two parts: the first during the second half of s,
        // the rest during the first half of s+1, so copy traffic is spread
        // over the whole stage.
        wait_vm_barrier<0>();  // previous tile fully consumed
#pragma unroll
        for (int st = 0; st < STAGES - 1; st++)
            if (st < nk)
#pragma unroll
                for (int q = 0; q < LOADS; q++) copy_any(st, st, q);
        if (STAGES - 1 < nk)
#pragma unroll
            for (int q = 0; q < HALF; q++) copy_any(STAGES - 1, STAGES - 1, q);
        // stage 0 landed: what may stay in flight is everything issued for later stages
        if (nk >= STAGES) wait_vm_barrier<(STAGES - 2) * LOADS + HALF>();
        else if (nk == 3 && STAGES >= 4) wait_vm_barrier<2 * LOADS>();
        else if (nk == 2) wait_vm_barrier<LOADS>();
        else wait_vm_barrier<0>();
        frag(0, 0, 0);

        // Steady state, unrolled by STAGES so buffer indices are constants;
        // every stage it copies is a full one. Scheduling fences keep each
        // fragment read ahead of the MFMAs it overlaps (the compiler would
        // otherwise sink the reads below them).
        int kt = 0;
        const int steady_last = nk - (ragged ? 1 : 0);
        for (; kt + 2 * STAGES <= steady_last; kt += STAGES) {
#pragma unroll
            for (int b = 0; b < STAGES; b++) {
                __builtin_amdgcn_sched_barrier(0);
                half_step(0, b, 1, 1, kt + b + STAGES - 1, (b + STAGES - 1) % STAGES, HALF);
                __builtin_amdgcn_sched_barrier(0);
                wait_vm_barrier<(STAGES - 2) * LOADS>();
                __builtin_amdgcn_sched_barrier(0);
                half_step(1, (b + 1) % STAGES, 0, 0, kt + b + STAGES, b, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // Drain: same schedule with run-time buffers and exact waits.
#pragma unroll 1
        for (; kt < nk; kt++) {
            const int b = kt % STAGES;
            frag(b, 1, 1);
            if (kt + STAGES - 1 < nk)
#pragma unroll
                for (int q = HALF; q < LOADS; q++) copy_any(kt + STAGES - 1, (kt + STAGES - 1) % STAGES, q);
            mma(0, false, 0, 0, 0);
            if (kt + 1 < nk) {
                const int beyond = min(nk - 1, kt + STAGES - 1) - (kt + 1);  // later stages, all issued
                if (beyond >= 2 && STAGES >= 4) wait_vm_barrier<(STAGES >= 4 ? 2 : 0) * LOADS>();
                else if (beyond >= 1) wait_vm_barrier<LOADS>();
                else wait_vm_barrier<0>();
                frag((b + 1) % STAGES, 0, 0);
                if (kt + STAGES < nk)
#pragma unroll
                    for (int q = 0; q < HALF; q++) copy_any(kt + STAGES, b, q);
            }
            mma(1, false, 0, 0, 0);
        }

        // ---- epilogue: lane = one token of each 32-token block, 4 columns per group
#pragma unroll
        for (int i = 0; i < RT; i++) {
            const int t = wm * (BM / WM) + i * 32 + (lane & 31);
            if (t < rows) {
                const int pos = row0 + t;
                if (GATEUP) {
                    constexpr int HW = BN / 2 / WN;
                    uint16_t *Hh = reinterpret_cast<uint16_t *>(p.C) + (int64_t)pos * p.N;
#pragma unroll
                    for (int j = 0; j < RW / 2; j++)
#pragma unroll
                        for (int g4 = 0; g4 < 4; g4++) {
                            const int c = nb * (BN / 2) + wn * HW + j * 32 + 8 * g4 + 4 * (lane >> 5);
                            if (c < p.N) {
                                float hv[4];
#pragma unroll
                                for (int u = 0; u < 4; u++)
                                    hv[u] = silu_f32(acc[j][i][4 * g4 + u]) * acc[j + RW / 2][i][4 * g4 + u];
                                uint2 pk;
                                pk.x = pack_bf16x2(hv[0], hv[1]);
                                pk.y = pack_bf16x2(hv[2], hv[3]);
                                *reinterpret_cast<uint2 *>(Hh + c) = pk;
                            }
                        }
                } else {
                    const int64_t orow = p.c_rows ? (int64_t)p.c_rows[pos] : (int64_t)pos;
                    const float sc = p.c_scale ? p.c_scale[pos] : 1.0f;
                    float *Y = reinterpret_cast<float *>(p.C) + orow * p.N;
#pragma unroll
                    for (int j = 0; j < RW; j++)
#pragma unroll
                        for (int g4 = 0; g4 < 4; g4++) {
                            const int m = nb * BN + wn * (BN / WN) + j * 32 + 8 * g4 + 4 * (lane >> 5);
                            if (m < p.N) {
                                float4 y = make_float4(acc[j][i][4 * g4] * sc, acc[j][i][4 * g4 + 1] * sc,
                                                       acc[j][i][4 * g4 + 2] * sc, acc[j][i][4 * g4 + 3] * sc);
                                *reinterpret_cast<float4 *>(Y + m) = y;
                            }
                        }
                }
            }
        }
    }
}

// Persistent grid: OCC workgroups per CU, rounded to whole XCD rounds.
int persistent_grid(int occ)
{
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
    }
    return ((cus + 7) / 8) * 8 * occ;
}

TiledParams make_params(const GemmProblem &g, int NB)
{
    TiledParams t;
    t.A = (const __bf16 *)g.A;
    t.a_rows = g.a_rows;
    t.W = (const __bf16 *)g.W;
    t.w_expert_stride = g.w_expert_stride;
    t.K = (int)g.K;
    t.N = (int)g.N;
    t.C = g.C;
    t.c_rows = g.c_rows;
    t.c_scale = g.c_scale;
    t.tiles = g.dense_rows > 0 ? nullptr : g.tiles;
    t.tile_start = g.tile_start;
    t.E = (int)g.E;
    t.dense_rows = (int)g.dense_rows;
    t.NB = NB;
    return t;
}

template <int BM, int BN, int WM, int WN, int OCC, bool GATEUP>
hipError_t launch_cfg(const GemmProblem &g, hipStream_t st)
{
    const int cols = GATEUP ? BN / 2 : BN;  // output columns per N-block
    TiledParams t = make_params(g, (int)((g.N + cols - 1) / cols));
    hipLaunchKernelGGL((tiled_gemm_kernel<BM, BN, WM, WN, OCC, GATEUP>), dim3(persistent_grid(OCC)),
                       dim3(WM * WN * 64), 0, st, t);
    return hipGetLastError();
}

#ifndef MOE_TILED_PP
#define MOE_TILED_PP 0
#endif

#if MOE_TILED_PP
template <bool GATEUP>
hipError_t launch_pp(const GemmProblem &g, hipStream_t st)
{
    const int cols = GATEUP ? 128 : 256;
    TiledParams t = make_params(g, (int)((g.N + cols - 1) / cols));
    hipLaunchKernelGGL((tiled_pp_kernel<256, 256, GATEUP>), dim3(persistent_grid(1)), dim3(256), 0, st, t);
    return hipGetLastError();
}
#endif

}  // namespace

// Routed experts: 256x256 tiles, 8 waves, one workgroup per CU; the M-tile
// list is built for this height. Dense problems (the shared expert, all T
// rows) use smaller tiles so that a few thousand rows still fill the CUs:
// 128x256 (gate_up) and 128x128 with two workgroups per CU (down).
int tiled_block_m() { return 256; }

hipError_t launch_gate_up_tiled(const GemmProblem &g, hipStream_t st)
{
    if (g.dense_rows > 0) return launch_cfg<128, 256, 2, 2, 1, true>(g, st);
#if MOE_TILED_PP
    return launch_pp<true>(g, st);
#else
    return launch_cfg<256, 256, 4, 2, 1, true>(g, st);
#endif
}

hipError_t launch_down_tiled(const GemmProblem &g, hipStream_t st)
{
    if (g.dense_rows > 0) return launch_cfg<128, 128, 2, 2, 2, false>(g, st);
#if MOE_TILED_PP
    return launch_pp<false>(g, st);
#else
    return launch_cfg<256, 256, 4, 2, 1, false>(g, st);
#endif
}

}  // namespace moe
