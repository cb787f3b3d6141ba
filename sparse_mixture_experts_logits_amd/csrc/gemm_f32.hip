// fp32 expert GEMMs (dtype MOE_F32) on the matrix cores: v_mfma_f32_32x32x2_f32
// tiles of 32 rows of one expert x 32 output columns, fp32 operands and
// accumulation. Same packed layouts and fused epilogues as the bf16 kernels:
// gate_up_proj rows [0, I) gate, [I, 2I) up, h = silu(g) * u ("深入解析
// Transformers 中的 PhiMoE" page, section 2, item 3); down output scaled by
// the routing weight and written to the assignment's slot. This path serves
// small fp32 layers; the bf16 paths carry the performance work.
#include "moe_internal.h"

#include <algorithm>

namespace moe {

namespace {

struct F32Params {
    const float *A;         // [rows of A, K]
    const int32_t *a_rows;  // sorted position -> row of A (null = identity)
    const float *W;         // packed weights
    int64_t w_expert_stride;
    int K;
    int N;                  // h columns (gate_up) or output columns (down)
    float *C;
    const int32_t *c_rows;  // sorted position -> output row (null = identity)
    const float *c_scale;   // sorted position -> routing weight (null = 1)
    const int32_t *counts;  // [E] rows per expert (null: one dense problem)
    const int32_t *offsets; // [E+1]
    int dense_rows;
};

constexpr int KC = 32;  // reduction elements staged per chunk

// One wave: output columns [n0, n0 + 32) of expert blockIdx.y (gate_up: the
// matching gate and up weight rows, two accumulators), for the expert's
// 32-row blocks blockIdx.z, blockIdx.z + gridDim.z, ... A chunk of K is
// loaded with row-contiguous loads (a lane reads 16 bytes; 8 rows of 128
// bytes per instruction), staged in LDS while the next chunk's loads are in
// flight, then KC / 2 MFMAs consume it: lane l supplies
// A[row l % 32][k + l / 32] and W[col l % 32][k + l / 32].
template <bool GATEUP>
__global__ __launch_bounds__(64) void f32_mfma_kernel(F32Params p)
{
    constexpr int NWR = GATEUP ? 64 : 32;  // weight rows staged per chunk
    __shared__ float sA[32][KC + 1];       // +1: consecutive rows land in other banks
    __shared__ float sW[NWR][KC + 1];
    const int lane = threadIdx.x;
    const int e = p.counts ? (int)blockIdx.y : 0;
    const int M = p.counts ? p.counts[e] : p.dense_rows;
    const int row0 = p.counts ? p.offsets[e] : 0;
    const int n0 = blockIdx.x * 32;
    if (M <= 0) return;  // workgroup-uniform
    const float *wbase = p.W + (int64_t)e * p.w_expert_stride;

    // staging geometry: lane -> (row lane / 8 + 8 i, elements 4 (lane % 8) .. + 3)
    const int sr = lane >> 3, sc = (lane & 7) * 4;
    for (int m0 = 32 * (int)blockIdx.z; m0 < M; m0 += 32 * (int)gridDim.z) {
        f32x16_t acc[GATEUP ? 2 : 1];
#pragma unroll
        for (int a = 0; a < (GATEUP ? 2 : 1); a++)
#pragma unroll
            for (int q = 0; q < 16; q++) acc[a][q] = 0.0f;
        // the chunk at k0 into registers (zeros past K or past the rows)
        float4 ra[4], rw[NWR / 8];
        auto load = [&](int k0) {
            const bool kin = k0 + sc < p.K;  // K is a multiple of 8: a float4 is all in or all out
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = sr + 8 * i;
                ra[i] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (m0 + r < M && kin) {
                    const int pos = row0 + m0 + r;
                    const int64_t src = p.a_rows ? (int64_t)p.a_rows[pos] : (int64_t)pos;
                    ra[i] = *reinterpret_cast<const float4 *>(p.A + src * p.K + k0 + sc);
                }
            }
#pragma unroll
            for (int i = 0; i < NWR / 8; i++) {
                const int r = sr + 8 * i;  // staged weight row: gate rows 0..31, then up rows 32..63
                const int n = n0 + (r & 31);
                rw[i] = make_float4(0.f, 0.f, 0.f, 0.f);
                if (n < p.N && kin) {
                    const int64_t wrow = (GATEUP && r >= 32) ? (int64_t)p.N + n : (int64_t)n;
                    rw[i] = *reinterpret_cast<const float4 *>(wbase + wrow * p.K + k0 + sc);
                }
            }
        };
        load(0);
        for (int k0 = 0; k0 < p.K; k0 += KC) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                float *d = &sA[sr + 8 * i][sc];
                d[0] = ra[i].x; d[1] = ra[i].y; d[2] = ra[i].z; d[3] = ra[i].w;
            }
#pragma unroll
            for (int i = 0; i < NWR / 8; i++) {
                float *d = &sW[sr + 8 * i][sc];
                d[0] = rw[i].x; d[1] = rw[i].y; d[2] = rw[i].z; d[3] = rw[i].w;
            }
            __syncthreads();
            if (k0 + KC < p.K) load(k0 + KC);  // the next chunk is in flight during this one's MFMAs
#pragma unroll
            for (int kk = 0; kk < KC; kk += 2) {
                const int k = kk + (lane >> 5);
                const float a = sA[lane & 31][k];
                acc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, sW[lane & 31][k], acc[0], 0, 0, 0);
                if (GATEUP) acc[GATEUP ? 1 : 0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, sW[32 + (lane & 31)][k],
                                                                                      acc[GATEUP ? 1 : 0], 0, 0, 0);
            }
            __syncthreads();
        }
        // accumulator element q of lane l: row 8 (q / 4) + 4 (l / 32) + q % 4, column l % 32
        const int c = n0 + (lane & 31);
#pragma unroll
        for (int q = 0; q < 16; q++) {
            const int rr = 8 * (q >> 2) + 4 * (lane >> 5) + (q & 3);
            if (m0 + rr >= M || c >= p.N) continue;
            const int pos = row0 + m0 + rr;
            if (GATEUP) {
                p.C[(int64_t)pos * p.N + c] = silu_f32(acc[0][q]) * acc[GATEUP ? 1 : 0][q];
            } else {
                const int64_t orow = p.c_rows ? (int64_t)p.c_rows[pos] : (int64_t)pos;
                const float s = p.c_scale ? p.c_scale[pos] : 1.0f;
                p.C[orow * p.N + c] = acc[0][q] * s;
            }
        }
    }
}

F32Params make_params(const GemmProblem &g)
{
    F32Params f;
    f.A = (const float *)g.A;
    f.a_rows = g.a_rows;
    f.W = (const float *)g.W;
    f.w_expert_stride = g.w_expert_stride;
    f.K = (int)g.K;
    f.N = (int)g.N;
    f.C = (float *)g.C;
    f.c_rows = g.c_rows;
    f.c_scale = g.c_scale;
    f.counts = g.dense_rows > 0 ? nullptr : g.counts;
    f.offsets = g.dense_rows > 0 ? nullptr : g.offsets;
    f.dense_rows = (int)g.dense_rows;
    return f;
}

template <bool GATEUP>
hipError_t launch_f32(const GemmProblem &g, hipStream_t st)
{
    const F32Params f = make_params(g);
    // row blocks of an expert are spread over grid z (a workgroup takes every
    // gridDim.z-th one), up to what the rows could need
    const int64_t rows = g.dense_rows > 0 ? g.dense_rows : g.total_rows;
    const unsigned zb = (unsigned)std::min<int64_t>((rows + 31) / 32, 16);
    const dim3 grid((unsigned)((g.N + 31) / 32), g.dense_rows > 0 ? 1u : (unsigned)g.E, zb > 0 ? zb : 1u);
    hipLaunchKernelGGL(f32_mfma_kernel<GATEUP>, grid, dim3(64), 0, st, f);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_f32(const GemmProblem &g, hipStream_t st) { return launch_f32<true>(g, st); }

hipError_t launch_down_f32(const GemmProblem &g, hipStream_t st) { return launch_f32<false>(g, st); }

}  // namespace moe
