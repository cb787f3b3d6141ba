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

namespace moe {

namespace {

constexpr int BK = 32;     // bf16 elements per k-stage (64 bytes per row)
constexpr int STAGES = 4;  // LDS ring depth: three stages in flight while one is consumed

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

// LDS stage layout: rows of 64 bytes (4 chunks of 16 bytes); chunk c of row r
// sits at chunk slot c ^ ((r >> 2) & 3), so the 16 lanes a ds_read_b128 serves
// per cycle (16 consecutive rows, one chunk column) hit 16 distinct 16-byte
// bank groups of the 64-bank LDS.
__device__ __forceinline__ int lds_slot(int r, int c) { return r * 4 + (c ^ ((r >> 2) & 3)); }

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Wait until at most N vector-memory operations of this wave are outstanding
// (global_load_lds stages are counted there), then barrier. The memory clobber
// keeps the compiler from moving LDS accesses across it.
template <int N>
__device__ __forceinline__ void wait_vm_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int BM, int BN, int WM, int WN, bool GATEUP>
__global__ __launch_bounds__(WM *WN * 64) void tiled_gemm_kernel(TiledParams p)
{
    constexpr int NT = WM * WN * 64;
    constexpr int NWAVE = WM * WN;
    constexpr int RM = BM / WM / 32;
    constexpr int RN = BN / WN / 32;
    constexpr int A_INS = BM / 16 / NWAVE;  // 16-row DMA instructions per wave per stage
    constexpr int B_INS = BN / 16 / NWAVE;
    constexpr int LOADS = A_INS + B_INS;    // vector-memory ops per wave per stage
    static_assert(A_INS >= 1 && B_INS >= 1 && RM >= 1 && RN >= 1, "tile shape");
    static_assert(!GATEUP || (RN % 2 == 0), "gate/up pairing needs an even RN");

    __shared__ u32x4 sA[STAGES][BM * 4];
    __shared__ u32x4 sB[STAGES][BN * 4];
    __shared__ int s_ts[kMaxExperts + 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN;
    const int wn = wave - wm * WN;

    int n_mtiles;
    if (p.tiles) {
        for (int e = tid; e <= p.E; e += NT) s_ts[e] = p.tile_start[e];
        __syncthreads();
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

    // DMA lane geometry: instruction i of this wave fills LDS rows
    // 16*(wave*INS + i) + lane/4, chunk slot lane%4 (logical chunk lc below)
    const int drow = lane >> 2;

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
            const int rr = 16 * (wave * A_INS + i) + drow;
            const int rc = rr < rows ? rr : 0;
            const int64_t src = p.a_rows ? (int64_t)p.a_rows[row0 + rc] : (int64_t)(row0 + rc);
            alc[i] = (lane & 3) ^ ((rr >> 2) & 3);
            asrc[i] = p.A + src * p.K + alc[i] * 8;
        }
        const __bf16 *wbase = p.W + (int64_t)e * p.w_expert_stride;
        const __bf16 *bsrc[B_INS];
        int blc[B_INS];
#pragma unroll
        for (int i = 0; i < B_INS; i++) {
            const int rr = 16 * (wave * B_INS + i) + drow;
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
            blc[i] = (lane & 3) ^ ((rr >> 2) & 3);
            bsrc[i] = wbase + (int64_t)wrow * p.K + blc[i] * 8;
        }

        // stage kt -> LDS buffer b: every lane copies 16 bytes; chunks past K are zero-filled
        auto issue = [&](int kt, int b) {
            const int k0 = kt * BK;
#pragma unroll
            for (int i = 0; i < A_INS; i++) {
                u32x4 *dst = &sA[b][(wave * A_INS + i) * 64];
                if (k0 + alc[i] * 8 < p.K)
                    __builtin_amdgcn_global_load_lds((global_void_t *)(asrc[i] + k0), (lds_void_t *)dst, 16, 0, 0);
                else
                    dst[lane] = u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int i = 0; i < B_INS; i++) {
                u32x4 *dst = &sB[b][(wave * B_INS + i) * 64];
                if (k0 + blc[i] * 8 < p.K)
                    __builtin_amdgcn_global_load_lds((global_void_t *)(bsrc[i] + k0), (lds_void_t *)dst, 16, 0, 0);
                else
                    dst[lane] = u32x4{0u, 0u, 0u, 0u};
            }
        };

        f32x16_t acc[RM][RN];
#pragma unroll
        for (int i = 0; i < RM; i++)
#pragma unroll
            for (int j = 0; j < RN; j++)
#pragma unroll
                for (int q = 0; q < 16; q++) acc[i][j][q] = 0.0f;

        auto compute = [&](int b) {
#pragma unroll
            for (int kk = 0; kk < BK / 16; kk++) {
                bf16x8_t af[RM], bf[RN];
                const int c = kk * 2 + (lane >> 5);
#pragma unroll
                for (int i = 0; i < RM; i++) {
                    const int row = wm * (BM / WM) + i * 32 + (lane & 31);
                    af[i] = as_bf16x8(sA[b][lds_slot(row, c)]);
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
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
            }
        };

        // all waves are done with the previous tile's stages before refilling them
        wait_vm_barrier<0>();
#pragma unroll
        for (int s = 0; s < STAGES - 1; s++)
            if (s < nk) issue(s, s);

        // stage kt lives in buffer kt % STAGES; the loop is unrolled by STAGES so
        // buffer indices are compile-time constants
        auto step = [&](int kt, int b) {
            const int ahead = min(STAGES - 2, nk - 1 - kt);  // issued stages after kt
            if (ahead >= 2) wait_vm_barrier<2 * LOADS>();
            else if (ahead == 1) wait_vm_barrier<LOADS>();
            else wait_vm_barrier<0>();
            if (kt + STAGES - 1 < nk) issue(kt + STAGES - 1, (b + STAGES - 1) % STAGES);
            compute(b);
        };
        int kt = 0;
        for (; kt + STAGES <= nk; kt += STAGES) {
#pragma unroll
            for (int b = 0; b < STAGES; b++) step(kt + b, b);
        }
#pragma unroll
        for (int b = 0; b < STAGES - 1; b++)
            if (kt + b < nk) step(kt + b, b);

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

// Tile configuration of the large-M schedule.
constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kWM = 4;
constexpr int kWN = 2;

int persistent_grid()
{
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
    }
    return ((cus + 7) / 8) * 8;
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

}  // namespace

int tiled_block_m() { return kBM; }

hipError_t launch_gate_up_tiled(const GemmProblem &g, hipStream_t st)
{
    const int NB = (int)((g.N + kBN / 2 - 1) / (kBN / 2));
    TiledParams t = make_params(g, NB);
    hipLaunchKernelGGL((tiled_gemm_kernel<kBM, kBN, kWM, kWN, true>), dim3(persistent_grid()),
                       dim3(kWM * kWN * 64), 0, st, t);
    return hipGetLastError();
}

hipError_t launch_down_tiled(const GemmProblem &g, hipStream_t st)
{
    const int NB = (int)((g.N + kBN - 1) / kBN);
    TiledParams t = make_params(g, NB);
    hipLaunchKernelGGL((tiled_gemm_kernel<kBM, kBN, kWM, kWN, false>), dim3(persistent_grid()),
                       dim3(kWM * kWN * 64), 0, st, t);
    return hipGetLastError();
}

}  // namespace moe
