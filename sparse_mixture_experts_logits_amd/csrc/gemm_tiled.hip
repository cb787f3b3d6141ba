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
//   * tiles are visited expert-major, then in bands of a few M-tiles that
//     run through every N-block, and each XCD takes a contiguous run of tile
//     ids per round, so the tiles running together on one XCD share both
//     their token rows and their weight blocks through its L2;
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
// Routed launches: BK bf16 elements per k-stage (2*BK bytes per row) and an
// LDS ring of STAGES stages. Every launch configuration takes its own pair.
constexpr int kRoutedBK = MOE_TILED_BK;
constexpr int kRoutedStages = MOE_TILED_STAGES;

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
    uint32_t a_bytes;  // bytes of A the rows may reach (buffer resource bound)
    int kgran;         // k-stages of a split piece are a multiple of this (2: A copied in pairs of stages)
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

__host__ __device__ __forceinline__ SplitPlan split_plan(int total, int G, int cap, int nk, bool enabled, int gran)
{
    SplitPlan sp{total, 1, nk, total};
    cap = std::min(G, cap);
    const int rem = total % G;
    if (!enabled || rem == 0 || 2 * rem > cap || nk < 2) return sp;
    int split = std::min(std::min(cap / rem, kMaxSplit), nk);
    const int nks = ((nk + split - 1) / split + gran - 1) / gran * gran;
    split = (nk + nks - 1) / nks;  // every piece holds at least one stage
    if (split < 2) return sp;
    sp.full = total - rem;
    sp.split = split;
    sp.nks = nks;
    sp.nwork = sp.full + rem * split;
    return sp;
}

#ifndef MOE_TILED_BAND
#define MOE_TILED_BAND 8
#endif
// Tile order inside an expert (or the dense problem): its M-tiles are taken
// in bands of BAND; a band runs through every N-block with its M-tiles
// innermost. Each XCD takes a contiguous run of tile ids per round (see the
// persistent loop), so the run covers a few M-tiles times several N-blocks
// and both the token rows and the weight blocks it streams are shared
// through that XCD's L2, instead of one operand being fetched anew by every
// tile. Returns the M-tile index and the N-block of local tile id `local`
// among nte M-tiles and NB N-blocks.
__device__ __forceinline__ void band_order(int local, int nte, int NB, int &mt, int &nb)
{
    constexpr int BAND = MOE_TILED_BAND;
    const int band = local / (BAND * NB);
    const int mbase = band * BAND;
    const int sm = min(BAND, nte - mbase);  // M-tiles in this band (the last may be short)
    const int within = local - band * BAND * NB;
    nb = within / sm;
    mt = mbase + (within - nb * sm);
}

// tile id -> (expert, N-block, first row, rows, index in the M-tile list)
template <int BM>
__device__ __forceinline__ void decode_tile(const TiledParams &p, int id, int n_mtiles, int &e, int &nb, int &row0,
                                            int &rows, int &tix)
{
    if (p.tiles) {
        const int32_t *s_ts = p.tile_start;
        int lo = 0, hi = p.E;  // find e: s_ts[e]*NB <= id < s_ts[e+1]*NB
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_ts[mid] * p.NB <= id) lo = mid; else hi = mid;
        }
        e = lo;
        int mt;
        band_order(id - s_ts[e] * p.NB, s_ts[e + 1] - s_ts[e], p.NB, mt, nb);
        tix = s_ts[e] + mt;
        const MTile t = p.tiles[tix];
        row0 = t.row0;
        rows = t.rows;
    } else {
        e = 0;
        int mt;
        band_order(id, n_mtiles, p.NB, mt, nb);
        tix = mt;
        row0 = mt * BM;
        rows = min(BM, p.dense_rows - row0);
    }
}

// Stores 16 bf16 values of h: column c0 + lane % 32 (c0 a wave-uniform
// multiple of 32), rows rbase + 8 (q / 4) + 4 (lane / 32) + q % 4 of M-tile
// tix (first row row0), skipping rows past the tile's and columns past N.
// Rows are row-major, or in the h row blocks of the tile list, where the
// block of the 32 columns is wave-uniform (one scalar base per block).
template <bool HB>
__device__ __forceinline__ void store_h16(const TiledParams &p, int tix, int row0, int rows, int c0, int rbase,
                                          int lane, const uint32_t (&v)[16])
{
    static_assert(kBlockCols == 32, "column block of 32");
    const int c = c0 + (lane & 31);
    uint16_t *h = reinterpret_cast<uint16_t *>(p.C);
    if (HB) {
        // the block through a buffer resource (scalar registers) and one
        // 32-bit offset a lane: no per-element 64-bit addresses
        const int nkb = (p.N + kBlockCols - 1) / kBlockCols;
        uint16_t *hb = h + ((int64_t)tix * nkb + (c0 >> 5)) * (kHBlockRows * kBlockCols);
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc(hb, 0, kHBlockRows * kBlockCols * 2, 0x00020000);
#pragma unroll
        for (int q = 0; q < 16; q++) {
            const int rr = rbase + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
            if (rr < rows && c < p.N)
                __builtin_amdgcn_raw_buffer_store_b16((uint16_t)v[q], r, (rr * kBlockCols + (lane & 31)) * 2, 0, 0);
        }
    } else {
#pragma unroll
        for (int q = 0; q < 16; q++) {
            const int rr = rbase + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
            if (rr < rows && c < p.N) h[(int64_t)(row0 + rr) * p.N + c] = (uint16_t)v[q];
        }
    }
}

// Epilogue of one tile from the accumulators of wave (wm, wn): h = silu(gate)
// * up as bf16 (gate_up) or the weighted fp32 slot rows (down). xg: LDS for
// the gate halves of the extra rows (gate_up with XT > 0).
template <int BM, int BN, int WM, int WN, bool GATEUP, int XT, bool HB>
__device__ __forceinline__ void tile_epilogue(const TiledParams &p, const f32x16_t (&acc)[BM / WM / 32][BN / WN / 32],
                                              const f32x16_t &accx, int wm, int wn, int lane, int row0, int rows,
                                              int nb, bool xtra, float *xgs, int tix, uint16_t *stage)
{
    constexpr int RM = BM / WM / 32;
    constexpr int RN = BN / WN / 32;
    const int jx = GATEUP ? (wm >> 1) + (RN / 2) * (wm & 1) : wm;
    if constexpr (GATEUP && HB) {
        // h row blocks: the tile's h goes through LDS (the idle stage ring) in
        // block order, then out in 16-byte pieces, each 32-column block of
        // the tile one contiguous run of its rows
        constexpr int HW = BN / 2 / WN;
        constexpr int NCB = BN / 2 / kBlockCols;  // column blocks of the tile
        constexpr int NT = WM * WN * 64;
        __syncthreads();  // every wave is done with the stage ring
#pragma unroll
        for (int i = 0; i < RM; i++)
#pragma unroll
            for (int j = 0; j < RN / 2; j++) {
                const int cb = (wn * HW + j * 32) / kBlockCols;  // wave-uniform
#pragma unroll
                for (int q = 0; q < 16; q++) {
                    const int rr = wm * (BM / WM) + i * 32 + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                    stage[(cb * kHBlockRows + rr) * kBlockCols + (lane & 31)] =
                        (uint16_t)f32_to_bf16_bits(silu_f32(acc[i][j][q]) * acc[i][j + RN / 2][q]);
                }
            }
        if (XT > 0 && xtra) {
            float *xg = xgs + (wn * 2 + (wm >> 1)) * (16 * 64);
            if ((wm & 1) == 0) {
#pragma unroll
                for (int q = 0; q < 16; q++) xg[q * 64 + lane] = accx[q];
            }
            __syncthreads();
            if (wm & 1) {
                const int cb = (wn * HW + (wm >> 1) * 32) / kBlockCols;
#pragma unroll
                for (int q = 0; q < 16; q++) {
                    const int rr = BM + 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
                    stage[(cb * kHBlockRows + rr) * kBlockCols + (lane & 31)] =
                        (uint16_t)f32_to_bf16_bits(silu_f32(xg[q * 64 + lane]) * accx[q]);
                }
            }
        }
        __syncthreads();
        const int nkb = (p.N + kBlockCols - 1) / kBlockCols;
        const u32x4 *src = reinterpret_cast<const u32x4 *>(stage);
        u32x4 *dst = reinterpret_cast<u32x4 *>(p.C);
        constexpr int PIECES = kBlockCols * 2 / 16;  // 16-byte pieces per block row
        for (int ch = threadIdx.x; ch < NCB * kHBlockRows * PIECES; ch += NT) {
            const int cb = ch / (kHBlockRows * PIECES);
            const int r = (ch / PIECES) % kHBlockRows;
            if (r < rows && (nb * NCB + cb) * kBlockCols < p.N)
                dst[(((int64_t)tix * nkb + nb * NCB + cb) * kHBlockRows + r) * PIECES + ch % PIECES] = src[ch];
        }
        return;
    }
    if (GATEUP) {
        constexpr int HW = BN / 2 / WN;
#pragma unroll
        for (int i = 0; i < RM; i++)
#pragma unroll
            for (int j = 0; j < RN / 2; j++) {
                uint32_t v[16];
#pragma unroll
                for (int q = 0; q < 16; q++) v[q] = f32_to_bf16_bits(silu_f32(acc[i][j][q]) * acc[i][j + RN / 2][q]);
                store_h16<HB>(p, tix, row0, rows, nb * (BN / 2) + wn * HW + j * 32, wm * (BM / WM) + i * 32, lane, v);
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
                uint32_t v[16];
#pragma unroll
                for (int q = 0; q < 16; q++) v[q] = f32_to_bf16_bits(silu_f32(xg[q * 64 + lane]) * accx[q]);
                store_h16<HB>(p, tix, row0, rows, nb * (BN / 2) + wn * HW + (wm >> 1) * 32, BM, lane, v);
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

// LDS stage layout: rows of CH = BK / 8 chunks of 16 bytes; chunk c of row r sits at
// slot c ^ swz(r) with swz(r) = (r >> 2) & 3 for 64-byte rows and (r >> 1) & 7
// for 128-byte rows, so the 16 lanes a ds_read_b128 serves per cycle (16
// consecutive rows, one chunk column) hit 16 distinct 16-byte bank groups of
// the 64-bank LDS.
template <int CH>
__device__ __forceinline__ int lds_swz(int r) { return CH == 4 ? ((r >> 2) & 3) : ((r >> 1) & 7); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Wait until at most N vector-memory operations of this wave are outstanding
// (global_load_lds stages are counted there), then barrier. The memory clobber
// keeps the compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void wait_vm_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer resource over n bytes at base (gfx9 layout: base, stride 0,
// num_records, untyped), wave-uniform: it lives in scalar registers.
__device__ __forceinline__ i32x4_t buf_rsrc(const void *base, uint32_t n)
{
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return i32x4_t{(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)n, 0x00020000};
}

// Direct-to-LDS copy of 16 bytes per lane: lane i reads the buffer at byte
// voff (its own) + soff (the stage's K offset, wave-uniform) and writes LDS
// bytes [lds + 16 i, lds + 16 i + 16). Issued from inline assembly so that
// the compiler does not treat every later LDS read as possibly aliasing the
// copy (it would wait for all copies in flight before each read and
// serialize the ring); completion is tracked by wait_vm_barrier's explicit
// vmcnt instead. The copy has no register result; it only reads its
// operands. A lane's address is one 32-bit offset, so a stage's copies cost
// no address arithmetic in vector registers.
__device__ __forceinline__ void dma16(i32x4_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, %3 offen lds" ::"v"(voff), "s"(rsrc),
                 "s"(lds), "s"(soff)
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
// AP (32-wide stages, 4-deep ring, K a multiple of 64): one operand is
// copied for two stages at once, 8 rows x 128 bytes per copy instruction
// instead of 16 rows x 64 bytes (half the copies, each at the address unit's
// full rate): gate_up's token rows, or down's row-layout weights. A pair
// buffer is two ring slots of that operand seen as rows of 8 chunks,
// swizzled like 128-byte stage rows; the other operand keeps its 32-wide
// 4-deep ring. Pair q + 1 is copied during stage 2q, into the pair buffer
// that stages 2q - 2 and 2q - 1 used.
template <int BM, int BN, int WM, int WN, int OCC, bool GATEUP, int XT, int BK, int STAGES, bool WPACK, bool HB,
          bool AP>
__global__ __launch_bounds__(WM *WN * 64, OCC) void tiled_gemm_kernel(TiledParams p)
{
    static_assert(!AP || (BK == 32 && STAGES == 4 && (GATEUP || !WPACK)), "pairs of 32-wide stages, 4-deep ring");
    // WPACK: the weights are in tile blocks (one stage of one N-block = 256
    // rows x 32 columns, contiguous; zero-filled past N and K)
    static_assert(!WPACK || (BN == kBlockRows && BK == kBlockCols), "tile blocks are 256 x 32");
    // a routed down launch may read h row blocks: one tile's rows, 32 columns a stage
    static_assert(GATEUP || XT == 0 || (BM + XT == kHBlockRows && BK == kBlockCols), "h row blocks are 288 x 32");
    constexpr int CH = BK / 8;    // 16-byte chunks per row of a stage
    constexpr int RPI = 64 / CH;  // rows filled by one 64-lane copy instruction
    static_assert(CH == 4 || CH == 8, "stage rows of 64 or 128 bytes");
    static_assert(STAGES >= 2, "at least a double buffer");
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

    const SplitPlan sp = split_plan(total, G, p.cap, nk_all, p.part != nullptr, p.kgran);

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
        int tix;
        decode_tile<BM>(p, id, n_mtiles, e, nb, row0, rows, tix);
        const bool xtra = XT > 0 && rows > BM;  // tile-uniform

        // ---- per-lane DMA sources (rows past the tile repeat row 0; dropped
        // later) as byte offsets into a buffer resource over A, or over the
        // expert's weights; a stage adds its K offset in a scalar register
        // logical chunk (of 8 elements) a lane copies for LDS row rr
        auto chunk_of = [&](int rr) { return (lane % CH) ^ lds_swz<CH>(rr); };
        const uint32_t krow = (uint32_t)p.K * 2u;  // bytes per row
        const i32x4_t ra = buf_rsrc(p.A, p.a_bytes);
        // A in h row blocks (down after a tiled gate_up): row rc of the tile's
        // block for stage kt at ((tix * nk_all + kt) * kHBlockRows + rc) * 64
        constexpr bool ablk = !GATEUP && HB;
        const uint32_t ablock0 = (uint32_t)(tix * nk_all + ks) * (uint32_t)kHBlockRows;
        uint32_t aoff[A_INS];
#pragma unroll
        for (int i = 0; i < A_INS; i++) {
            const int rr = RPI * (wave * A_INS + i) + drow;
            const int rc = rr < rows ? rr : 0;
            if (ablk) {
                aoff[i] = (ablock0 + (uint32_t)rc) * (BK * 2u) + (uint32_t)chunk_of(rr) * 16u;
            } else {
                const uint32_t src = p.a_rows ? (uint32_t)p.a_rows[row0 + rc] : (uint32_t)(row0 + rc);
                aoff[i] = src * krow + (uint32_t)kbase * 2u + (uint32_t)chunk_of(rr) * 16u;
            }
        }
        // extra rows BM + XR*wave + lane/CH, lanes below XR*CH (rows past the
        // tile repeat row BM)
        uint32_t xoff = 0;
        const bool xlane = lane < XR * CH;
        const int xrr = BM + XR * wave + (xlane ? drow : 0);
        if (XT > 0 && xtra) {
            const int rc = xrr < rows ? xrr : BM;
            if (ablk) {
                xoff = (ablock0 + (uint32_t)rc) * (BK * 2u) + (uint32_t)chunk_of(xrr) * 16u;
            } else {
                const uint32_t src = p.a_rows ? (uint32_t)p.a_rows[row0 + rc] : (uint32_t)(row0 + rc);
                xoff = src * krow + (uint32_t)kbase * 2u + (uint32_t)chunk_of(xrr) * 16u;
            }
        }
        // AP: the pair copies' sources (the same rows, 8 rows x 8 chunks a
        // copy): gate_up's token rows (and extra rows), or down's weight rows
        constexpr int CHA = 8;
        constexpr int RPIA = 64 / CHA;
        constexpr int P_INS = AP ? (GATEUP ? BM : BN) / RPIA / NWAVE : 1;
        static_assert(!AP || (P_INS * RPIA * NWAVE == (GATEUP ? BM : BN) && XR * CHA <= 64), "pair copy geometry");
        auto chunk_a = [&](int rr) { return (lane % CHA) ^ lds_swz<CHA>(rr); };
        uint32_t poff[P_INS];
        uint32_t xoffa = 0;
        const bool xlanea = lane < XR * CHA;
        if constexpr (AP && GATEUP) {
#pragma unroll
            for (int i = 0; i < P_INS; i++) {
                const int rr = RPIA * (wave * P_INS + i) + lane / CHA;
                const int rc = rr < rows ? rr : 0;
                const uint32_t src = p.a_rows ? (uint32_t)p.a_rows[row0 + rc] : (uint32_t)(row0 + rc);
                poff[i] = src * krow + (uint32_t)kbase * 2u + (uint32_t)chunk_a(rr) * 16u;
            }
            if (XT > 0 && xtra) {
                const int xr = BM + XR * wave + (xlanea ? lane / CHA : 0);
                const int rc = xr < rows ? xr : BM;
                const uint32_t src = p.a_rows ? (uint32_t)p.a_rows[row0 + rc] : (uint32_t)(row0 + rc);
                xoffa = src * krow + (uint32_t)kbase * 2u + (uint32_t)chunk_a(xr) * 16u;
            }
        }
        if constexpr (AP && !GATEUP) {
#pragma unroll
            for (int i = 0; i < P_INS; i++) {
                const int rr = RPIA * (wave * P_INS + i) + lane / CHA;
                const int n = nb * BN + rr;
                const uint32_t wrow = (uint32_t)(n < p.N ? n : 0);
                poff[i] = wrow * krow + (uint32_t)kbase * 2u + (uint32_t)chunk_a(rr) * 16u;
            }
        }
        const i32x4_t rb = buf_rsrc(p.W + (int64_t)e * p.w_expert_stride,
                                    WPACK ? (uint32_t)p.w_expert_stride * 2u : (uint32_t)(GATEUP ? 2 * p.N : p.N) * krow);
        uint32_t boff[B_INS];
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
            if (WPACK)  // block (nb, ks): rows rr in LDS order; a stage adds one block (BN * BK * 2 bytes)
                boff[i] = ((uint32_t)(nb * nk_all + ks) * BN + (uint32_t)rr) * (BK * 2u) + (uint32_t)chunk_of(rr) * 16u;
            else
                boff[i] = (uint32_t)wrow * krow + (uint32_t)kbase * 2u + (uint32_t)chunk_of(rr) * 16u;
        }

        // stage kt -> LDS buffer b: every lane copies 16 bytes. Only a final
        // partial stage (K not a multiple of BK) masks lanes; they zero-fill.
        // stage kt's offset into the weights: BK columns of a row, or one tile block
        auto wstage = [&](int kt) { return WPACK ? (uint32_t)kt * (BN * BK * 2u) : (uint32_t)(kt * BK) * 2u; };
        // and into A: BK columns of a row, or one block of the h row blocks
        auto astage = [&](int kt) { return ablk ? (uint32_t)kt * (kHBlockRows * BK * 2u) : (uint32_t)(kt * BK) * 2u; };
        auto issue = [&](int kt, int b) {
            const uint32_t k0 = astage(kt);
#pragma unroll
            for (int i = 0; i < A_INS; i++) dma16(ra, aoff[i], k0, lds_addr(&sA[b][(wave * A_INS + i) * 64]));
#pragma unroll
            for (int i = 0; i < B_INS; i++) dma16(rb, boff[i], wstage(kt), lds_addr(&sB[b][(wave * B_INS + i) * 64]));
            if (XT > 0 && xtra && xlane) dma16(ra, xoff, k0, lds_addr(&sA[b][(BM + XR * wave) * CH]));
        };
        auto issue_tail = [&](int kt, int b) {
            const int k0 = kt * BK;
            const uint32_t k0b = astage(kt);
#pragma unroll
            for (int i = 0; i < A_INS; i++) {
                u32x4 *dst = &sA[b][(wave * A_INS + i) * 64];
                if (k0 + chunk_of(RPI * (wave * A_INS + i) + drow) * 8 < Kl)
                    dma16(ra, aoff[i], k0b, lds_addr(dst));
                else
                    dst[lane] = u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int i = 0; i < B_INS; i++) {
                u32x4 *dst = &sB[b][(wave * B_INS + i) * 64];
                if (WPACK)  // the block's columns past K are zeros already
                    dma16(rb, boff[i], wstage(kt), lds_addr(dst));
                else if (k0 + chunk_of(RPI * (wave * B_INS + i) + drow) * 8 < Kl)
                    dma16(rb, boff[i], k0b, lds_addr(dst));
                else
                    dst[lane] = u32x4{0u, 0u, 0u, 0u};
            }
            if (XT > 0 && xtra && xlane) {
                u32x4 *dst = &sA[b][(BM + XR * wave) * CH];
                if (k0 + chunk_of(xrr) * 8 < Kl)
                    dma16(ra, xoff, k0b, lds_addr(dst));
                else
                    dst[lane] = u32x4{0u, 0u, 0u, 0u};
            }
        };
        auto issue_any = [&](int kt, int b) {
            if (ragged && kt == nk - 1) issue_tail(kt, b);
            else issue(kt, b);
        };
        // AP: copy q of pair pr (stages 2pr, 2pr + 1) into pair buffer pb
        // (q < P_INS: rows; q == P_INS: gate_up's extra rows for this wave),
        // and copy q of the other operand's stage kt alone (gate_up: weight
        // rows; down: h rows, then the extra rows)
        auto issue_pair = [&](int pr, int pb, int q) {
            u32x4 *base = GATEUP ? &sA[2 * pb][0] : &sB[2 * pb][0];
            const uint32_t k0 = (uint32_t)pr * (2u * BK * 2u);
            if (q < P_INS) dma16(GATEUP ? ra : rb, poff[q], k0, lds_addr(base + (wave * P_INS + q) * 64));
            else if (xlanea) dma16(ra, xoffa, k0, lds_addr(base + (BM + XR * wave) * CHA));
        };
        auto issue_single = [&](int kt, int b, int q) {
            if (GATEUP) {
                dma16(rb, boff[q], wstage(kt), lds_addr(&sB[b][(wave * B_INS + q) * 64]));
            } else {
                if (q < A_INS) dma16(ra, aoff[q], astage(kt), lds_addr(&sA[b][(wave * A_INS + q) * 64]));
                else if (xlane) dma16(ra, xoff, astage(kt), lds_addr(&sA[b][(BM + XR * wave) * CH]));
            }
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

        // Every fragment row is a multiple of 32 plus lane % 32, and the LDS
        // swizzle only looks at the row's low five bits, so a fragment's
        // address is a per-lane base (one per k-step and operand, wave part
        // included) plus a compile-time offset (buffer, row block).
        constexpr int KSTEPS = BK / 16;  // MFMA k-steps per stage
        const int l32 = lane & 31;
        auto laneoff = [&](int kk) { return l32 * CH + ((kk * 2 + (lane >> 5)) ^ lds_swz<CH>(l32)); };
        constexpr int HWB = GATEUP ? BN / 2 / WN : BN / WN;  // B rows per wave (per half for gate_up)
        int va[KSTEPS], vb[KSTEPS], vxa[KSTEPS], vxb[KSTEPS];
#pragma unroll
        for (int kk = 0; kk < KSTEPS; kk++) {
            va[kk] = wm * (BM / WM) * CH + laneoff(kk);
            vb[kk] = wn * HWB * CH + laneoff(kk);
            vxa[kk] = BM * CH + laneoff(kk);
            vxb[kk] = (xrow - l32) * CH + laneoff(kk);
        }

        // copy instruction q (A rows, then B rows, then the extra rows) of stage kt into buffer b
        auto issue_one = [&](int kt, int b, int q) {
            const uint32_t k0 = astage(kt);
            if (q < A_INS) dma16(ra, aoff[q], k0, lds_addr(&sA[b][(wave * A_INS + q) * 64]));
            else if (q < LOADS) dma16(rb, boff[q - A_INS], wstage(kt), lds_addr(&sB[b][(wave * B_INS + q - A_INS) * 64]));
            else if (xlane) dma16(ra, xoff, k0, lds_addr(&sA[b][(BM + XR * wave) * CH]));
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
            // with a double buffer the next stage has only this stage to land:
            // its copies go out together, before the first fragment read
            constexpr bool BURST = STAGES <= 2;
            if (CP && BURST) {
#pragma unroll
                for (int q = 0; q < LX; q++) issue_one(nkt, nbuf, q);
            }
            const u32x4 *A = &sA[b][0];
            const u32x4 *Bw = &sB[b][0];
#pragma unroll
            for (int kk = 0; kk < BK / 16; kk++) {
                bf16x8_t af[RM], bf[RN], ax, bx;
#pragma unroll
                for (int i = 0; i < NB; i++) af[i] = as_bf16x8(A[va[kk] + i * 32 * CH]);
                if (EX) {
                    // the extra rows and this wave's B block jx for them (read
                    // again rather than picked from bf[] with a runtime index)
                    ax = as_bf16x8(A[vxa[kk]]);
                    bx = as_bf16x8(Bw[vxb[kk]]);
                }
#pragma unroll
                for (int j = 0; j < RN; j++) {
                    if (NB == 0) break;
                    const int row = GATEUP ? ((j < RN / 2) ? j * 32 : BN / 2 + (j - RN / 2) * 32) : j * 32;
                    bf[j] = as_bf16x8(Bw[vb[kk] + row * CH]);
                }
                auto slot = [&](int mi) {  // compile-time after unrolling
                    if (CP && !BURST && (mi + 1) % PER == 0 && (mi + 1) / PER - 1 < LX)
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

        // AP: fragment offsets into a pair buffer, half h (stage 2q + h) and
        // k-step kk: row l32 of 8 chunks, logical chunk 4h + 2kk + lane / 32
        int vpa[2][KSTEPS], vpx[2][KSTEPS];
#pragma unroll
        for (int h = 0; h < 2; h++)
#pragma unroll
            for (int kk = 0; kk < KSTEPS; kk++) {
                const int lo = l32 * CHA + ((h * 4 + kk * 2 + (lane >> 5)) ^ lds_swz<CHA>(l32));
                vpa[h][kk] = (GATEUP ? wm * (BM / WM) : wn * HWB) * CHA + lo;
                vpx[h][kk] = (GATEUP ? BM : xrow - l32) * CHA + lo;
            }
        // AP: consume single-stage buffer b and half h of pair buffer pb; with
        // CP, spread between the MFMAs the copies of stage nkt into buffer
        // nbuf and (CA) before them those of pair npr into pair buffer npb
        auto compute_stage_ap = [&](auto nbc, auto exc, auto cpc, auto cac, auto hc, int b, int pb, int nkt, int nbuf,
                                    int npr, int npb) {
            constexpr int NB = decltype(nbc)::value;
            constexpr bool EX = decltype(exc)::value;
            constexpr bool CP = decltype(cpc)::value;
            constexpr bool CA = decltype(cac)::value;
            constexpr int H = decltype(hc)::value;
            constexpr int LA = CA ? P_INS + (GATEUP && EX ? 1 : 0) : 0;
            constexpr int LX = LA + (GATEUP ? B_INS : A_INS + (EX ? 1 : 0));
            constexpr int NMMA = (BK / 16) * (RM * RN + (EX ? 1 : 0));
            constexpr int PER = NMMA / LX > 0 ? NMMA / LX : 1;
            static_assert(PER * LX <= NMMA, "every copy finds an MFMA slot");
            auto copy = [&](int q) {
                if (q < LA) issue_pair(npr, npb, q);
                else issue_single(nkt, nbuf, q - LA);
            };
            const u32x4 *A = GATEUP ? &sA[2 * pb][0] : &sA[b][0];
            const u32x4 *Bw = GATEUP ? &sB[b][0] : &sB[2 * pb][0];
            constexpr int CHAv = GATEUP ? CHA : CH;  // chunks per row of A's buffer
            constexpr int CHBv = GATEUP ? CH : CHA;  // and of B's
#pragma unroll
            for (int kk = 0; kk < BK / 16; kk++) {
                const int oa = GATEUP ? vpa[H][kk] : va[kk];
                const int oxa = GATEUP ? vpx[H][kk] : vxa[kk];
                const int ob = GATEUP ? vb[kk] : vpa[H][kk];
                const int oxb = GATEUP ? vxb[kk] : vpx[H][kk];
                bf16x8_t af[RM], bf[RN], ax, bx;
#pragma unroll
                for (int i = 0; i < NB; i++) af[i] = as_bf16x8(A[oa + i * 32 * CHAv]);
                if (EX) {
                    ax = as_bf16x8(A[oxa]);
                    bx = as_bf16x8(Bw[oxb]);
                }
#pragma unroll
                for (int j = 0; j < RN; j++) {
                    if (NB == 0) break;
                    const int row = GATEUP ? ((j < RN / 2) ? j * 32 : BN / 2 + (j - RN / 2) * 32) : j * 32;
                    bf[j] = as_bf16x8(Bw[ob + row * CHBv]);
                }
                auto slot = [&](int mi) {
                    if (CP && (mi + 1) % PER == 0 && (mi + 1) / PER - 1 < LX) copy((mi + 1) / PER - 1);
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
        if constexpr (AP) {
            // single stages 0, 1, 2 and pair 0, in the order the waits count:
            // S0, P0, S1, S2 (nk is even)
            constexpr int LS0 = GATEUP ? B_INS : A_INS + (XT > 0 ? 1 : 0);
            constexpr int LP0 = P_INS + (GATEUP && XT > 0 ? 1 : 0);
#pragma unroll
            for (int q = 0; q < LS0; q++)
                if (GATEUP || q < A_INS || xtra) issue_single(0, 0, q);
#pragma unroll
            for (int q = 0; q < LP0; q++)
                if (!GATEUP || q < P_INS || xtra) issue_pair(0, 0, q);
#pragma unroll
            for (int q = 0; q < LS0; q++)
                if (GATEUP || q < A_INS || xtra) issue_single(1, 1, q);
            if (2 < nk) {
#pragma unroll
                for (int q = 0; q < LS0; q++)
                    if (GATEUP || q < A_INS || xtra) issue_single(2, 2, q);
            }
        } else {
#pragma unroll
            for (int s = 0; s < STAGES - 1; s++)
                if (s < nk) issue_any(s, s);
        }

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
        // AP: stage s needs single stage s and pair s / 2. Copies go out in
        // the order S(s + 3) at stage s, with pair s / 2 + 1 before it at even
        // s, so at even s the copies after pair s / 2 are S(s + 1) and
        // S(s + 2), and at odd s those after S(s) are S(s + 1), pair
        // (s + 1) / 2 and S(s + 2) (each only if it exists).
        auto kloop_ap = [&](auto nbc, auto exc) {
            constexpr bool EXv = decltype(exc)::value;
            constexpr int LW = GATEUP ? B_INS : A_INS + (EXv ? 1 : 0);  // single-stage copies
            constexpr int LA = P_INS + (GATEUP && EXv ? 1 : 0);         // pair copies
            using CP = std::integral_constant<bool, true>;
            using NOCP = std::integral_constant<bool, false>;
            using CA = std::integral_constant<bool, true>;
            using NOCA = std::integral_constant<bool, false>;
            using H0 = std::integral_constant<int, 0>;
            using H1 = std::integral_constant<int, 1>;
            int kt = 0;
            for (; kt + 2 * STAGES - 1 <= nk; kt += STAGES) {
                const int pr = kt / 2;  // even: the pair of stages kt, kt + 1 lives in pair buffer 0
                wait_vm_barrier<2 * LW>();
                compute_stage_ap(nbc, exc, CP{}, CA{}, H0{}, 0, 0, kt + 3, 3, pr + 1, 1);
                wait_vm_barrier<2 * LW + LA>();
                compute_stage_ap(nbc, exc, CP{}, NOCA{}, H1{}, 1, 0, kt + 4, 0, 0, 0);
                wait_vm_barrier<2 * LW>();
                compute_stage_ap(nbc, exc, CP{}, CA{}, H0{}, 2, 1, kt + 5, 1, pr + 2, 0);
                wait_vm_barrier<2 * LW + LA>();
                compute_stage_ap(nbc, exc, CP{}, NOCA{}, H1{}, 3, 1, kt + 6, 2, 0, 0);
            }
#pragma unroll
            for (int b = 0; b < 2 * STAGES - 1; b++) {
                const int st = kt + b;
                if (st >= nk) break;
                const bool a1 = st + 1 < nk, a2 = st + 2 < nk;
                if (b % 2 == 0) {
                    if (a2) wait_vm_barrier<2 * LW>();
                    else if (a1) wait_vm_barrier<LW>();
                    else wait_vm_barrier<0>();
                    if (st + 2 < nk) {
#pragma unroll
                        for (int q = 0; q < LA; q++) issue_pair(st / 2 + 1, (b / 2 + 1) % 2, q);
                    }
                } else {
                    if (a2) wait_vm_barrier<2 * LW + LA>();
                    else if (a1) wait_vm_barrier<LW + LA>();
                    else wait_vm_barrier<0>();
                }
                if (st + 3 < nk) {
#pragma unroll
                    for (int q = 0; q < LW; q++) issue_single(st + 3, (b + 3) % STAGES, q);
                }
                if (b % 2 == 0) compute_stage_ap(nbc, exc, NOCP{}, NOCA{}, H0{}, b % STAGES, (b / 2) % 2, 0, 0, 0, 0);
                else compute_stage_ap(nbc, exc, NOCP{}, NOCA{}, H1{}, b % STAGES, (b / 2) % 2, 0, 0, 0, 0);
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
        if constexpr (AP) {
            if (XT > 0 && xtra) kloop_ap(IRM{}, std::integral_constant<bool, XT != 0>{});
            else if (nvb >= RM) kloop_ap(IRM{}, F{});
            else if (nvb == 1) kloop_ap(I1{}, F{});
            else kloop_ap(I0{}, F{});
        } else {
            if (XT > 0 && xtra) kloop(IRM{}, std::integral_constant<bool, XT != 0>{});
            else if (nvb >= RM) kloop(IRM{}, F{});
            else if (nvb == 1) kloop(I1{}, F{});
            else kloop(I0{}, F{});
        }
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
            static_assert(!(GATEUP && HB) || (BN / 2 / kBlockCols) * kHBlockRows * kBlockCols * 2 <= (int)sizeof(sA),
                          "the tile's h row blocks fit the stage ring");
            tile_epilogue<BM, BN, WM, WN, GATEUP, XT, HB>(p, acc, accx, wm, wn, lane, row0, rows, nb, xtra, &s_xg[0][0],
                                                      tix, reinterpret_cast<uint16_t *>(&sA[0][0]));
        }
    }
}

// Second half of a split launch: one single-wave workgroup per (split tile,
// wave of the main kernel, 32-row block of that wave) adds the block's
// partial sums over the tile's pieces, in piece order, and writes its part of
// the tile as the main kernel's epilogue would (the extra rows go with row
// block 0; for gate_up an up wave sums its gate partner's partials as well). The split plan is recomputed from the
// same inputs as the main kernel's.
template <int BM, int BN, int WM, int WN, bool GATEUP, int XT, int BK, bool HB>
__global__ __launch_bounds__(64) void tiled_split_finish_kernel(TiledParams p)
{
    constexpr int NWAVE = WM * WN;
    constexpr int RM = BM / WM / 32;
    constexpr int RN = BN / WN / 32;
    constexpr int NBLK = RM * RN + (XT > 0 ? 1 : 0);

    const int n_mtiles = p.tiles ? p.tile_start[p.E] : (p.dense_rows + BM - 1) / BM;
    const int total = n_mtiles * p.NB;
    const int nk_all = (p.K + BK - 1) / BK;
    const SplitPlan sp = split_plan(total, p.G, p.cap, nk_all, p.part != nullptr, p.kgran);
    const int t = blockIdx.x / (NWAVE * RM);
    const int wave = (blockIdx.x / RM) % NWAVE;
    const int i = blockIdx.x % RM;  // this workgroup's 32-row block
    if (sp.split < 2 || sp.full + t >= total) return;  // workgroup-uniform

    const int lane = threadIdx.x;
    const int wm = wave / WN;
    const int wn = wave - wm * WN;
    int e, nb, row0, rows;
    int tix;
    decode_tile<BM>(p, sp.full + t, n_mtiles, e, nb, row0, rows, tix);
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
#pragma unroll
            for (int j = 0; j < RN / 2; j++) {
                f32x16_t g, u;
                sum_block(wave, i * RN + j, g);
                sum_block(wave, i * RN + j + RN / 2, u);
                uint32_t v[16];
#pragma unroll
                for (int q = 0; q < 16; q++) v[q] = f32_to_bf16_bits(silu_f32(g[q]) * u[q]);
                store_h16<HB>(p, tix, row0, rows, nb * (BN / 2) + wn * HW + j * 32, wm * (BM / WM) + i * 32, lane, v);
            }
        if (XT > 0 && xtra && (wm & 1) && i == 0) {
            // up block of the extra rows; its gate block is in wave (wm - 1, wn)
            f32x16_t g, u;
            sum_block(wave - WN, RM * RN, g);
            sum_block(wave, RM * RN, u);
            uint32_t v[16];
#pragma unroll
            for (int q = 0; q < 16; q++) v[q] = f32_to_bf16_bits(silu_f32(g[q]) * u[q]);
            store_h16<HB>(p, tix, row0, rows, nb * (BN / 2) + wn * HW + (wm >> 1) * 32, BM, lane, v);
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

// Persistent grid: OCC workgroups per CU, rounded to whole XCD rounds. The
// caller queries the CU count of the current device on every call, so the
// library keeps no cached device state.
int persistent_grid(int cus, int occ)
{
    if (cus <= 0) cus = 256;
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
    // down reads A from the h row blocks when they are in use
    const int64_t abytes = (g.h_blocks && g.dense_rows == 0 && g.a_rows == nullptr) ? g.h_bytes : g.a_rows_total * g.K * 2;
    t.a_bytes = (uint32_t)std::min<int64_t>(abytes, 0xFFFFFFFFll);
    t.kgran = 1;
    return t;
}

template <int BM, int BN, int WM, int WN, int OCC, bool GATEUP, int XT, int BK, int STAGES, bool WPACK = false,
          bool HB = false, bool AP = false>
hipError_t launch_cfg(const GemmProblem &g, hipStream_t st)
{
    const int cols = GATEUP ? BN / 2 : BN;  // output columns per N-block
    TiledParams t = make_params(g, (int)((g.N + cols - 1) / cols));
    t.G = persistent_grid(g.cus, OCC);
    // Split pieces hold whole 64-column pairs of 32-wide stages whenever K
    // has them, with or without paired copies (AP needs it), so the pieces,
    // and with them the rounding of the summed partials, are the same for
    // every kernel variant of a shape.
    t.kgran = (BK == 32 && g.K % 64 == 0) ? 2 : 1;
    // pieces of this tile shape that fit the buffer (sized for kSplitPieces
    // routed 256x256 pieces), at most one round of the launch
    constexpr int64_t piece_bytes = (int64_t)WM * WN * ((BM / WM / 32) * (BN / WN / 32) + (XT > 0 ? 1 : 0)) * 1024 * 4;
    t.cap = (int)std::min<int64_t>(t.G, tiled_split_bytes() / piece_bytes);
    t.part = g.part;
    // a dense problem's tile count is known here: no second launch when no tile is split
    if (t.part && g.dense_rows > 0) {
        const int total = (int)((g.dense_rows + BM - 1) / BM) * t.NB;
        if (split_plan(total, t.G, t.cap, (int)((g.K + BK - 1) / BK), true, t.kgran).split < 2) t.part = nullptr;
    }
    hipLaunchKernelGGL((tiled_gemm_kernel<BM, BN, WM, WN, OCC, GATEUP, XT, BK, STAGES, WPACK, HB, AP>), dim3(t.G),
                       dim3(WM * WN * 64), 0, st, t);
    if (t.part) {
        // at most cap / 2 tiles are split (two pieces or more each)
        hipLaunchKernelGGL((tiled_split_finish_kernel<BM, BN, WM, WN, GATEUP, XT, BK, HB>),
                           dim3(t.cap / 2 * WM * WN * (BM / WM / 32)), dim3(64), 0, st, t);
    }
    return hipGetLastError();
}

#ifndef MOE_TILED_TAIL
#define MOE_TILED_TAIL 32
#endif
// Copies in pairs of stages (AP) for the routed gate_up (token rows) and
// down (row-layout weights) on the tiled schedule: compile-time switches, on
// by default; off, every launch copies single stages (same results).
#ifndef MOE_TILED_APAIR
#define MOE_TILED_APAIR 1
#endif
#ifndef MOE_TILED_APAIR_DN
#define MOE_TILED_APAIR_DN MOE_TILED_APAIR
#endif
// Dense problems (the shared expert over all T rows): one tile per CU for a
// few thousand rows, so each tile takes 8 waves (two per SIMD) to keep the
// MFMA pipe fed while a wave waits: gate_up waves 2 x 4 (64 rows x 32 gate +
// 32 up columns each), down waves 4 x 2 (32 rows x 64 columns each).
#ifndef MOE_DENSE_GATE_UP_CFG
#define MOE_DENSE_GATE_UP_CFG launch_cfg<128, 256, 2, 4, 1, true, 0, 64, 3>
#endif
#ifndef MOE_DENSE_DOWN_CFG
#define MOE_DENSE_DOWN_CFG launch_cfg<128, 128, 4, 2, 1, false, 0, 64, 4>
#endif

// Tile blocks from the nn.Linear layout: one thread per 16 bytes (8 columns)
// of the output, zeros past the matrix. Columns come in whole 8-column
// chunks (K is a multiple of 8), so a chunk is all inside or all outside.
__global__ __launch_bounds__(256) void pack_tile_blocks_kernel(const u32x4 *__restrict__ w, int which, int64_t I,
                                                               int64_t H, int64_t nbk, int64_t nk,
                                                               u32x4 *__restrict__ out, int64_t nchunks)
{
    const int64_t K = which == 0 ? H : I;              // columns of a weight row
    const int64_t rows = which == 0 ? 2 * I : H;      // weight rows of one expert
    constexpr int CPR = kBlockCols / 8;                // 16-byte chunks per block row
    for (int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x; q < nchunks; q += (int64_t)gridDim.x * 256) {
        const int c8 = (int)(q % CPR);
        const int64_t rq = q / CPR;
        const int r = (int)(rq % kBlockRows);
        const int64_t blk = rq / kBlockRows;  // (e, nb, kt), kt innermost
        const int64_t kt = blk % nk;
        const int64_t nb = (blk / nk) % nbk;
        const int64_t e = blk / (nk * nbk);
        int64_t row;
        bool in;
        if (which == 0) {  // gate rows then the matching up rows
            const int64_t j = nb * (kBlockRows / 2) + (r % (kBlockRows / 2));
            in = j < I;
            row = r < kBlockRows / 2 ? j : I + j;
        } else {
            row = nb * kBlockRows + r;
            in = row < H;
        }
        const int64_t col = kt * kBlockCols + c8 * 8;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (in && col < K) v = w[((e * rows + row) * K + col) / 8];
        out[q] = v;
    }
}

}  // namespace

hipError_t launch_pack_tile_blocks(int which, const void *w, int64_t E, int64_t I, int64_t H, void *out,
                                   hipStream_t st)
{
    const int64_t nbk = which == 0 ? (I + kBlockRows / 2 - 1) / (kBlockRows / 2) : (H + kBlockRows - 1) / kBlockRows;
    const int64_t nk = which == 0 ? (H + kBlockCols - 1) / kBlockCols : (I + kBlockCols - 1) / kBlockCols;
    const int64_t nchunks = E * nbk * nk * kBlockRows * (kBlockCols / 8);
    const int64_t blocks = std::min<int64_t>((nchunks + 255) / 256, 16384);
    hipLaunchKernelGGL(pack_tile_blocks_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const u32x4 *)w, which, I,
                       H, nbk, nk, (u32x4 *)out, nchunks);
    return hipGetLastError();
}

// Routed experts: 256x256 tiles (up to 32 more token rows in an expert's
// last tile), 8 waves, one workgroup per CU, 64-byte row segments per stage
// in a 4-deep ring; the M-tile list is built for these sizes. Dense problems
// (the shared expert, all T rows) use smaller tiles so that a few thousand
// rows still fill the CUs, with 128-byte row segments (half the address work
// per byte copied): 128x256 in a 3-deep ring (gate_up) and 128x128 in a
// 4-deep ring (down).
int tiled_block_m() { return 256; }
// partial-sum buffer of split tiles for the routed launches (256x256 tiles,
// 8 waves, 9 accumulator blocks of 32x32 per wave)
int64_t tiled_split_bytes() { return (int64_t)kSplitPieces * 8 * (2 * 4 + 1) * 1024 * sizeof(float); }
int tiled_tail_m() { return MOE_TILED_TAIL; }

hipError_t launch_gate_up_tiled(const GemmProblem &g, hipStream_t st)
{
    if (g.dense_rows > 0) return MOE_DENSE_GATE_UP_CFG(g, st);
    // Token rows copied in pairs of stages when K holds whole pairs: on the
    // tiled schedule (h in row blocks) with row-layout weights, whose
    // 16-row weight copies keep the address unit busiest (prefill gate_up
    // 0.85 -> 0.82 ms); with tile-block weights it measured even to 1% slower
    // on prefill and skewed batches, so those keep single stages, and so do
    // the mixed schedule's few tiles.
    if (MOE_TILED_APAIR && kRoutedBK == 32 && kRoutedStages == 4 && g.K % 64 == 0 && g.h_blocks && !g.w_blocks)
        return launch_cfg<256, 256, 4, 2, 1, true, MOE_TILED_TAIL, 32, 4, false, true, true>(g, st);
    if (g.w_blocks) {
        if (g.h_blocks) return launch_cfg<256, 256, 4, 2, 1, true, MOE_TILED_TAIL, kBlockCols, kRoutedStages, true, true>(g, st);
        return launch_cfg<256, 256, 4, 2, 1, true, MOE_TILED_TAIL, kBlockCols, kRoutedStages, true>(g, st);
    }
    if (g.h_blocks) return launch_cfg<256, 256, 4, 2, 1, true, MOE_TILED_TAIL, kRoutedBK, kRoutedStages, false, true>(g, st);
    return launch_cfg<256, 256, 4, 2, 1, true, MOE_TILED_TAIL, kRoutedBK, kRoutedStages>(g, st);
}

hipError_t launch_down_tiled(const GemmProblem &g, hipStream_t st)
{
    if (g.dense_rows > 0) return MOE_DENSE_DOWN_CFG(g, st);
    // row-layout weights copied in pairs of stages (the h rows are 1 KB
    // runs already), on the tiled schedule when K holds whole pairs
    if (MOE_TILED_APAIR_DN && kRoutedBK == 32 && kRoutedStages == 4 && g.K % 64 == 0 && g.h_blocks && !g.w_blocks)
        return launch_cfg<256, 256, 4, 2, 1, false, MOE_TILED_TAIL, 32, 4, false, true, true>(g, st);
    if (g.w_blocks) {
        if (g.h_blocks) return launch_cfg<256, 256, 4, 2, 1, false, MOE_TILED_TAIL, kBlockCols, kRoutedStages, true, true>(g, st);
        return launch_cfg<256, 256, 4, 2, 1, false, MOE_TILED_TAIL, kBlockCols, kRoutedStages, true>(g, st);
    }
    if (g.h_blocks) return launch_cfg<256, 256, 4, 2, 1, false, MOE_TILED_TAIL, kRoutedBK, kRoutedStages, false, true>(g, st);
    return launch_cfg<256, 256, 4, 2, 1, false, MOE_TILED_TAIL, kRoutedBK, kRoutedStages>(g, st);
}

}  // namespace moe
