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
//     share an expert's weight block run together on one XCD's L2;
//   * an expert's last few rows ride in its previous tile (XT below) and the
//     tiles of a short last round are split along K (SplitPlan below), so
//     neither a handful of rows nor a handful of tiles holds the launch.
#include "moe_internal.h"

#include <algorithm>
#include <type_traits>

namespace moe {

namespace {

#ifndef MOE_TILED_BK
#define MOE_TILED_BK 32
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
    int NB;     // N-blocks
    float *part;  // partial sums of split tiles (null: no splitting)
    int G;      // workgroups of the persistent launch
    int cap;    // pieces the partial-sum buffer holds for this tile shape
};

// The last, partial round of a persistent launch leaves most CUs idle when
// only a few tiles remain (total % G of them). Such tiles are split along K
// into up to kMaxSplit pieces, one workgroup each; every piece writes its
// fp32 partial sums (in accumulator layout) and a second kernel adds the
// pieces in piece order and runs the tile's epilogue, so the result does not
// depend on timing.
constexpr int kSplitPieces = 256;  // routed 256x256 tiles: pieces the buffer is sized for
constexpr int kMaxSplit = 8;

struct SplitPlan {
    int full;   // tiles [0, full) run whole
    int split;  // pieces per remaining tile (1: none)
    int nks;    // k-stages per piece
    int nwork;  // work items of the persistent loop
};

__device__ __forceinline__ SplitPlan split_plan(int total, int G, int cap, int nk, bool enabled)
{
    SplitPlan sp{total, 1, nk, total};
    cap = min(G, cap);
    const int rem = total % G;
    if (!enabled || rem == 0 || 2 * rem > cap || nk < 2) return sp;
    int split = min(min(cap / rem, kMaxSplit), nk);
    const int nks = (nk + split - 1) / split;
    split = (nk + nks - 1) / nks;  // every piece holds at least one stage
    if (split < 2) return sp;
    sp.full = total - rem;
    sp.split = split;
    sp.nks = nks;
    sp.nwork = sp.full + rem * split;
    return sp;
}

// tile id -> (expert, N-block, first row, rows); M-tiles of one expert are
// consecutive within each N-block
template <int BM>
__device__ __forceinline__ void decode_tile(const TiledParams &p, int id, int n_mtiles, int &e, int &nb, int &row0,
                                            int &rows)
{
    if (p.tiles) {
        const int32_t *s_ts = p.tile_start;
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
}

// Epilogue of one tile from the accumulators of wave (wm, wn): h = silu(gate)
// * up as bf16 (gate_up) or the weighted fp32 slot rows (down). xg: LDS for
// the gate halves of the extra rows (gate_up with XT > 0).
template <int BM, int BN, int WM, int WN, bool GATEUP, int XT>
__device__ __forceinline__ void tile_epilogue(const TiledParams &p, const f32x16_t (&acc)[BM / WM / 32][BN / WN / 32],
                                              const f32x16_t &accx, int wm, int wn, int lane, int row0, int rows,
                                              int nb, bool xtra, float *xgs)
{
    constexpr int RM = BM / WM / 32;
    constexpr int RN = BN / WN / 32;
    const int jx = GATEUP ? (wm >> 1) + (RN / 2) * (wm & 1) : wm;
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
        if (XT > 0 && xtra) {
            // gate blocks (even wm) to LDS; the up waves (odd wm) combine
            float *xg = xgs + (wn * 2 + (wm >> 1)) * (16 * 64);
            if ((wm & 1) == 0) {
#pragma unroll
                for (int q = 0; q < 16; q++) xg[q * 64 + lane] = accx[q];
            }
            __syncthreads();
            if (wm & 1) {
                const int c = nb * (BN / 2) + wn * HW + (wm >> 1) * 32 + (lane & 31);
#pragma unroll
                for (int q = 0; q < 16; q++) {
                    const int rr = BM + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                    if (rr < rows && c < p.N) {
                        const uint32_t hb = f32_to_bf16_bits(silu_f32(xg[q * 64 + lane]) * accx[q]);
                        reinterpret_cast<uint16_t *>(H)[(int64_t)(row0 + rr) * p.N + c] = (uint16_t)hb;
                    }
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
        if (XT > 0 && xtra) {
            const int m = nb * BN + wn * (BN / WN) + jx * 32 + (lane & 31);
#pragma unroll
            for (int q = 0; q < 16; q++) {
                const int rr = BM + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                if (rr < rows && m < p.N) {
                    const int pos = row0 + rr;
                    const int64_t orow = p.c_rows ? (int64_t)p.c_rows[pos] : (int64_t)pos;
                    const float sc = p.c_scale ? p.c_scale[pos] : 1.0f;
                    Y[orow * p.N + m] = accx[q] * sc;
                }
            }
        }
    }
}

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

// XT: token rows a tile may carry past BM (0, or 32 for the routed
// schedule). The routing kernels fold an expert's last rows, when at most XT
// of them lie past a multiple of BM, into its previous tile instead of
// opening a tile for them: the expert's weight block is then streamed once
// for BM + tail rows instead of a second time for a handful of rows. The
// extra 32-row block costs each wave one more 32x32 MFMA block per step:
// down: wave (wm, wn) takes output column block wm of its own columns;
// gate_up: the four waves of a column half take the gate and the up block of
// its two output column blocks, and the gate blocks reach the matching up
// waves through LDS in the epilogue.
template <int BM, int BN, int WM, int WN, int OCC, bool GATEUP, int XT = 0>
__global__ __launch_bounds__(WM *WN * 64, OCC) void tiled_gemm_kernel(TiledParams p)
{
    constexpr int NT = WM * WN * 64;
    constexpr int NWAVE = WM * WN;
    constexpr int RM = BM / WM / 32;
    constexpr int RN = BN / WN / 32;
    constexpr int A_INS = BM / RPI / NWAVE;  // copy instructions per wave per stage
    constexpr int B_INS = BN / RPI / NWAVE;
    constexpr int LOADS = A_INS + B_INS;    // vector-memory ops per wave per stage
    // extra rows: every wave copies XT / NWAVE of them with one instruction
    // of CH * XT / NWAVE lanes, so all waves issue the same number of copies
    constexpr int XR = XT / NWAVE;
    static_assert(A_INS >= 1 && B_INS >= 1 && RM >= 1 && RN >= 1, "tile shape");
    static_assert(!GATEUP || (RN % 2 == 0), "gate/up pairing needs an even RN");
    static_assert(XT == 0 || (XT == 32 && WM == 4 && RN == 4 && XR * CH <= 64), "extra-block layout");
    (void)NT;

    __shared__ u32x4 sA[STAGES][(BM + XT) * CH];
    __shared__ u32x4 sB[STAGES][BN * CH];
    constexpr bool XG = XT > 0 && GATEUP;
    __shared__ float s_xg[XG ? 2 * WN : 1][XG ? 16 * 64 : 1];  // gate halves of the extra block

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
    const int wm = wave / WN;
    const int wn = wave - wm * WN;
    // this wave's B block for the extra rows (see above) and its LDS row
    const int jx = GATEUP ? (wm >> 1) + (RN / 2) * (wm & 1) : wm;
    const int xrow = (GATEUP ? ((jx < RN / 2) ? wn * (BN / 2 / WN) + jx * 32
                                              : BN / 2 + wn * (BN / 2 / WN) + (jx - RN / 2) * 32)
                             : wn * (BN / WN) + jx * 32) +
                     (lane & 31);

    // number of M-tiles (read through the scalar cache, so the whole LDS is
    // left to the stage ring)
    int n_mtiles;
    if (p.tiles) {
        n_mtiles = p.tile_start[p.E];
    } else {
        n_mtiles = (p.dense_rows + BM - 1) / BM;
    }
    const int total = n_mtiles * p.NB;
    const int G = gridDim.x;
    const int nx = G >> 3;
    const int xcd = blockIdx.x & 7;
    const int li = blockIdx.x >> 3;
    const int nk_all = (p.K + BK - 1) / BK;

    // copy geometry: instruction i of this wave fills LDS rows
    // RPI*(wave*INS + i) + lane/CH, chunk slot lane%CH (logical chunk lc below)
    const int drow = lane / CH;

    const SplitPlan sp = split_plan(total, G, p.cap, nk_all, p.part != nullptr);

    for (int r = 0;; r++) {
        const int wid = r * G + xcd * nx + li;
        if (wid >= sp.nwork) break;
        // work item -> tile and its k-stages [ks, ke): whole tiles first, then
        // the pieces of the split ones (piece = wid - full)
        int id = wid, ks = 0, ke = nk_all;
        if (wid >= sp.full) {
            const int q = wid - sp.full;
            id = sp.full + q / sp.split;
            ks = (q % sp.split) * sp.nks;
            ke = min(nk_all, ks + sp.nks);
        }
        const int nk = ke - ks;                               // k-stages of this work item
        const int64_t kbase = (int64_t)ks * BK;               // its first k
        const int Kl = p.K - (int)kbase;                      // k bound relative to kbase
        const bool ragged = ke == nk_all && (p.K % BK) != 0;  // a partial last stage

        // ---- decode tile id -> (expert, M-tile, N-block)
        int e, nb, row0, rows;
        decode_tile<BM>(p, id, n_mtiles, e, nb, row0, rows);
        const bool xtra = XT > 0 && rows > BM;  // tile-uniform

        // ---- per-lane DMA source rows (rows past the tile repeat row 0; dropped later)
        // logical chunk (of 8 elements) a lane copies for LDS row rr
        auto chunk_of = [&](int rr) { return (lane % CH) ^ lds_swz(rr); };
        const __bf16 *asrc[A_INS];
#pragma unroll
        for (int i = 0; i < A_INS; i++) {
            const int rr = RPI * (wave * A_INS + i) + drow;
            const int rc = rr < rows ? rr : 0;
            const int64_t src = p.a_rows ? (int64_t)p.a_rows[row0 + rc] : (int64_t)(row0 + rc);
            asrc[i] = p.A + src * p.K + kbase + chunk_of(rr) * 8;
        }
        // extra rows BM + XR*wave + lane/CH, lanes below XR*CH (rows past the
        // tile repeat row BM)
        const __bf16 *xsrc = p.A;
        const bool xlane = lane < XR * CH;
        const int xrr = BM + XR * wave + (xlane ? drow : 0);
        if (XT > 0 && xtra) {
            const int rc = xrr < rows ? xrr : BM;
            const int64_t src = p.a_rows ? (int64_t)p.a_rows[row0 + rc] : (int64_t)(row0 + rc);
            xsrc = p.A + src * p.K + kbase + chunk_of(xrr) * 8;
        }
        const __bf16 *wbase = p.W + (int64_t)e * p.w_expert_stride;
        const __bf16 *bsrc[B_INS];
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
            bsrc[i] = wbase + (int64_t)wrow * p.K + kbase + chunk_of(rr) * 8;
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
            if (XT > 0 && xtra && xlane) dma16(xsrc + k0, lds_addr(&sA[b][(BM + XR * wave) * CH]));
        };
        auto issue_tail = [&](int kt, int b) {
            const int k0 = kt * BK;
#pragma unroll
            for (int i = 0; i < A_INS; i++) {
                u32x4 *dst = &sA[b][(wave * A_INS + i) * 64];
                if (k0 + chunk_of(RPI * (wave * A_INS + i) + drow) * 8 < Kl)
                    dma16(asrc[i] + k0, lds_addr(dst));
                else
                    dst[lane] = u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int i = 0; i < B_INS; i++) {
                u32x4 *dst = &sB[b][(wave * B_INS + i) * 64];
                if (k0 + chunk_of(RPI * (wave * B_INS + i) + drow) * 8 < Kl)
                    dma16(bsrc[i] + k0, lds_addr(dst));
                else
                    dst[lane] = u32x4{0u, 0u, 0u, 0u};
            }
            if (XT > 0 && xtra && xlane) {
                u32x4 *dst = &sA[b][(BM + XR * wave) * CH];
                if (k0 + chunk_of(xrr) * 8 < Kl)
                    dma16(xsrc + k0, lds_addr(dst));
                else
                    dst[lane] = u32x4{0u, 0u, 0u, 0u};
            }
        };
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
        f32x16_t accx;
#pragma unroll
        for (int q = 0; q < 16; q++) accx[q] = 0.0f;

        // copy instruction q (A rows, then B rows, then the extra rows) of stage kt into buffer b
        auto issue_one = [&](int kt, int b, int q) {
            const int k0 = kt * BK;
            if (q < A_INS) dma16(asrc[q] + k0, lds_addr(&sA[b][(wave * A_INS + q) * 64]));
            else if (q < LOADS) dma16(bsrc[q - A_INS] + k0, lds_addr(&sB[b][(wave * B_INS + q - A_INS) * 64]));
            else if (xlane) dma16(xsrc + k0, lds_addr(&sA[b][(BM + XR * wave) * CH]));
        };
        // Consume stage buffer b. When nkt >= 0, the LX copies of stage nkt
        // into buffer nbuf are spread between the MFMAs, one copy per PER
        // MFMA slots, so the copy engine never holds up the fragment reads.
        // NB (compile time): how many of this wave's RM 32-row blocks hold
        // rows of the tile; the rest skip their fragment reads and MFMAs, so
        // the short last tile of an expert costs less than a full one. The
        // copies keep their slots either way. EX: the tile has extra rows.
        auto compute_stage = [&](auto nbc, auto exc, auto cpc, int b, int nkt, int nbuf) {
            constexpr int NB = decltype(nbc)::value;
            constexpr bool EX = decltype(exc)::value;
            constexpr bool CP = decltype(cpc)::value;  // issue the copies of stage nkt
            constexpr int LX = LOADS + (EX ? 1 : 0);
            constexpr int NMMA = (BK / 16) * (RM * RN + (EX ? 1 : 0));
            constexpr int PER = NMMA / LX > 0 ? NMMA / LX : 1;
            static_assert(PER * LX <= NMMA, "every copy finds an MFMA slot");
#pragma unroll
            for (int kk = 0; kk < BK / 16; kk++) {
                bf16x8_t af[RM], bf[RN], ax, bx;
                const int c = kk * 2 + (lane >> 5);
#pragma unroll
                for (int i = 0; i < NB; i++) {
                    const int row = wm * (BM / WM) + i * 32 + (lane & 31);
                    af[i] = as_bf16x8(sA[b][lds_slot(row, c)]);
                }
                if (EX) {
                    // the extra rows and this wave's B block jx for them (read
                    // again rather than picked from bf[] with a runtime index)
                    ax = as_bf16x8(sA[b][lds_slot(BM + (lane & 31), c)]);
                    bx = as_bf16x8(sB[b][lds_slot(xrow, c)]);
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
                auto slot = [&](int mi) {  // compile-time after unrolling
                    if (CP && (mi + 1) % PER == 0 && (mi + 1) / PER - 1 < LX)
                        issue_one(nkt, nbuf, (mi + 1) / PER - 1);
                };
#pragma unroll
                for (int i = 0; i < RM; i++)
#pragma unroll
                    for (int j = 0; j < RN; j++) {
                        if (i < NB)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
                        slot((kk * (RM * RN + (EX ? 1 : 0)) + i * RN + j));
                    }
                if (EX) {
                    accx = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ax, bx, accx, 0, 0, 0);
                    slot(kk * (RM * RN + 1) + RM * RN);
                }
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
        // (a ragged last stage is always left to the drain). Then the drain:
        // fewer than 2*STAGES-1 stages remain (kt is a multiple of STAGES, so
        // stage kt + b lives in buffer b). LX: this wave's copies per stage.
        const int steady_last = nk - (ragged ? 1 : 0);
        auto kloop = [&](auto nbc, auto exc) {
            constexpr int LX = LOADS + (decltype(exc)::value ? 1 : 0);
            using CP = std::integral_constant<bool, true>;
            using NOCP = std::integral_constant<bool, false>;
            int kt = 0;
            for (; kt + 2 * STAGES - 1 <= steady_last; kt += STAGES) {
#pragma unroll
                for (int b = 0; b < STAGES; b++) {
                    wait_vm_barrier<(STAGES - 2) * LX>();
                    compute_stage(nbc, exc, CP{}, b, kt + b + STAGES - 1, (b + STAGES - 1) % STAGES);
                }
            }
#pragma unroll
            for (int b = 0; b < 2 * STAGES - 1; b++) {
                if (kt + b >= nk) break;
                const int ahead = min(STAGES - 2, nk - 1 - (kt + b));
                if (ahead >= 2 && STAGES >= 4) wait_vm_barrier<(STAGES >= 4 ? 2 : 0) * LX>();
                else if (ahead == 1) wait_vm_barrier<LX>();
                else wait_vm_barrier<0>();
                if (kt + b + STAGES - 1 < nk) issue_any(kt + b + STAGES - 1, (b + STAGES - 1) % STAGES);
                compute_stage(nbc, exc, NOCP{}, b % STAGES, 0, 0);
            }
        };
        // 32-row blocks of this wave that hold rows of the tile (wave-uniform);
        // one copy of the loop per case
        const int nvb = max(0, min(RM, (rows - wm * (BM / WM) + 31) / 32));
        static_assert(RM <= 2, "loop variants for up to two 32-row blocks per wave");
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using IRM = std::integral_constant<int, RM>;
        using F = std::integral_constant<bool, false>;
        using T = std::integral_constant<bool, true>;
        if (XT > 0 && xtra) kloop(IRM{}, std::integral_constant<bool, XT != 0>{});
        else if (nvb >= RM) kloop(IRM{}, F{});
        else if (nvb == 1) kloop(I1{}, F{});
        else kloop(I0{}, F{});
        (void)T{};

        // ---- epilogue, or the partial sums of a piece of a split tile
        if (wid >= sp.full) {
            constexpr int NBLK = RM * RN + (XT > 0 ? 1 : 0);
            float *pp = p.part + ((int64_t)(wid - sp.full) * NWAVE + wave) * NBLK * 1024 + lane;
#pragma unroll
            for (int i = 0; i < RM; i++)
#pragma unroll
                for (int j = 0; j < RN; j++)
#pragma unroll
                    for (int q = 0; q < 16; q++) pp[(i * RN + j) * 1024 + q * 64] = acc[i][j][q];
            if (XT > 0) {
#pragma unroll
                for (int q = 0; q < 16; q++) pp[(RM * RN) * 1024 + q * 64] = accx[q];
            }
        } else {
            tile_epilogue<BM, BN, WM, WN, GATEUP, XT>(p, acc, accx, wm, wn, lane, row0, rows, nb, xtra, &s_xg[0][0]);
        }
    }
}

// Second half of a split launch: one single-wave workgroup per (split tile,
// wave of the main kernel, 32-row block of that wave) adds the block's
// partial sums over the tile's pieces, in piece order, and writes its part of
// the tile as the main kernel's epilogue would (the extra rows go with row
// block 0; for gate_up an up wave sums its gate partner's partials as well). The split plan is recomputed from the
// same inputs as the main kernel's.
template <int BM, int BN, int WM, int WN, bool GATEUP, int XT>
__global__ __launch_bounds__(64) void tiled_split_finish_kernel(TiledParams p)
{
    constexpr int NWAVE = WM * WN;
    constexpr int RM = BM / WM / 32;
    constexpr int RN = BN / WN / 32;
    constexpr int NBLK = RM * RN + (XT > 0 ? 1 : 0);

    const int n_mtiles = p.tiles ? p.tile_start[p.E] : (p.dense_rows + BM - 1) / BM;
    const int total = n_mtiles * p.NB;
    const int nk_all = (p.K + BK - 1) / BK;
    const SplitPlan sp = split_plan(total, p.G, p.cap, nk_all, p.part != nullptr);
    const int t = blockIdx.x / (NWAVE * RM);
    const int wave = (blockIdx.x / RM) % NWAVE;
    const int i = blockIdx.x % RM;  // this workgroup's 32-row block
    if (sp.split < 2 || sp.full + t >= total) return;  // workgroup-uniform

    const int lane = threadIdx.x;
    const int wm = wave / WN;
    const int wn = wave - wm * WN;
    int e, nb, row0, rows;
    decode_tile<BM>(p, sp.full + t, n_mtiles, e, nb, row0, rows);
    (void)e;
    const bool xtra = XT > 0 && rows > BM;

    const int64_t pstride = (int64_t)NWAVE * NBLK * 1024;  // between pieces
    // block b of wave w summed over the pieces in piece order; all kMaxSplit
    // loads are issued unconditionally (pieces past the last re-read it and
    // count 0)
    auto sum_block = [&](int w, int b, f32x16_t &v) {
        const float *pp = p.part + ((int64_t)t * sp.split * NWAVE + w) * NBLK * 1024 + b * 1024 + lane;
        float x[kMaxSplit][16];
#pragma unroll
        for (int c = 0; c < kMaxSplit; c++)
#pragma unroll
            for (int q = 0; q < 16; q++) x[c][q] = pp[min(c, sp.split - 1) * pstride + q * 64];
#pragma unroll
        for (int q = 0; q < 16; q++) {
            float a = x[0][q];
#pragma unroll
            for (int c = 1; c < kMaxSplit; c++) a += c < sp.split ? x[c][q] : 0.0f;
            v[q] = a;
        }
    };

    if (GATEUP) {
        constexpr int HW = BN / 2 / WN;
        uint16_t *H = reinterpret_cast<uint16_t *>(p.C);
#pragma unroll
            for (int j = 0; j < RN / 2; j++) {
                f32x16_t g, u;
                sum_block(wave, i * RN + j, g);
                sum_block(wave, i * RN + j + RN / 2, u);
                const int c = nb * (BN / 2) + wn * HW + j * 32 + (lane & 31);
#pragma unroll
                for (int q = 0; q < 16; q++) {
                    const int rr = wm * (BM / WM) + i * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                    if (rr < rows && c < p.N)
                        H[(int64_t)(row0 + rr) * p.N + c] = (uint16_t)f32_to_bf16_bits(silu_f32(g[q]) * u[q]);
                }
            }
        if (XT > 0 && xtra && (wm & 1) && i == 0) {
            // up block of the extra rows; its gate block is in wave (wm - 1, wn)
            f32x16_t g, u;
            sum_block(wave - WN, RM * RN, g);
            sum_block(wave, RM * RN, u);
            const int c = nb * (BN / 2) + wn * HW + (wm >> 1) * 32 + (lane & 31);
#pragma unroll
            for (int q = 0; q < 16; q++) {
                const int rr = BM + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                if (rr < rows && c < p.N)
                    H[(int64_t)(row0 + rr) * p.N + c] = (uint16_t)f32_to_bf16_bits(silu_f32(g[q]) * u[q]);
            }
        }
    } else {
        float *Y = reinterpret_cast<float *>(p.C);
#pragma unroll
            for (int j = 0; j < RN; j++) {
                f32x16_t y;
                sum_block(wave, i * RN + j, y);
                const int m = nb * BN + wn * (BN / WN) + j * 32 + (lane & 31);
#pragma unroll
                for (int q = 0; q < 16; q++) {
                    const int rr = wm * (BM / WM) + i * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                    if (rr < rows && m < p.N) {
                        const int pos = row0 + rr;
                        const int64_t orow = p.c_rows ? (int64_t)p.c_rows[pos] : (int64_t)pos;
                        const float sc = p.c_scale ? p.c_scale[pos] : 1.0f;
                        Y[orow * p.N + m] = y[q] * sc;
                    }
                }
            }
        if (XT > 0 && xtra && i == 0) {
            f32x16_t y;
            sum_block(wave, RM * RN, y);
            const int jx = wm;
            const int m = nb * BN + wn * (BN / WN) + jx * 32 + (lane & 31);
#pragma unroll
            for (int q = 0; q < 16; q++) {
                const int rr = BM + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                if (rr < rows && m < p.N) {
                    const int pos = row0 + rr;
                    const int64_t orow = p.c_rows ? (int64_t)p.c_rows[pos] : (int64_t)pos;
                    const float sc = p.c_scale ? p.c_scale[pos] : 1.0f;
                    Y[orow * p.N + m] = y[q] * sc;
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
    t.part = nullptr;
    t.G = 0;
    t.cap = 0;
    return t;
}

template <int BM, int BN, int WM, int WN, int OCC, bool GATEUP, int XT = 0>
hipError_t launch_cfg(const GemmProblem &g, hipStream_t st)
{
    const int cols = GATEUP ? BN / 2 : BN;  // output columns per N-block
    TiledParams t = make_params(g, (int)((g.N + cols - 1) / cols));
    t.G = persistent_grid(OCC);
    // pieces of this tile shape that fit the buffer (sized for kSplitPieces
    // routed 256x256 pieces), at most one round of the launch
    constexpr int64_t piece_bytes = (int64_t)WM * WN * ((BM / WM / 32) * (BN / WN / 32) + (XT > 0 ? 1 : 0)) * 1024 * 4;
    t.cap = (int)std::min<int64_t>(t.G, tiled_split_bytes() / piece_bytes);
    t.part = g.part;
    hipLaunchKernelGGL((tiled_gemm_kernel<BM, BN, WM, WN, OCC, GATEUP, XT>), dim3(t.G), dim3(WM * WN * 64), 0, st, t);
    if (t.part) {
        // at most cap / 2 tiles are split (two pieces or more each)
        hipLaunchKernelGGL((tiled_split_finish_kernel<BM, BN, WM, WN, GATEUP, XT>),
                           dim3(t.cap / 2 * WM * WN * (BM / WM / 32)), dim3(64), 0, st, t);
    }
    return hipGetLastError();
}

#ifndef MOE_TILED_TAIL
#define MOE_TILED_TAIL 32
#endif

}  // namespace

// Routed experts: 256x256 tiles (up to 32 more token rows in an expert's
// last tile), 8 waves, one workgroup per CU; the M-tile list is built for
// these sizes. Dense problems (the shared expert, all T rows) use smaller
// tiles so that a few thousand rows still fill the CUs: 128x256 (gate_up)
// and 128x128 with two workgroups per CU (down).
int tiled_block_m() { return 256; }
// partial-sum buffer of split tiles for the routed launches (256x256 tiles,
// 8 waves, 9 accumulator blocks of 32x32 per wave)
int64_t tiled_split_bytes() { return (int64_t)kSplitPieces * 8 * (2 * 4 + 1) * 1024 * sizeof(float); }
int tiled_tail_m() { return MOE_TILED_TAIL; }

hipError_t launch_gate_up_tiled(const GemmProblem &g, hipStream_t st)
{
    if (g.dense_rows > 0) return launch_cfg<128, 256, 2, 2, 1, true>(g, st);
    return launch_cfg<256, 256, 4, 2, 1, true, MOE_TILED_TAIL>(g, st);
}

hipError_t launch_down_tiled(const GemmProblem &g, hipStream_t st)
{
    if (g.dense_rows > 0) return launch_cfg<128, 128, 2, 2, 2, false>(g, st);
    return launch_cfg<256, 256, 4, 2, 1, false, MOE_TILED_TAIL>(g, st);
}

}  // namespace moe
