// Weight-streaming grouped expert GEMMs for few rows per expert (decode).
//
// With a handful of tokens per expert the layer is bound by reading the
// selected experts' weights once from HBM (the bandwidth model of the
// "Transformer中的混合专家架构详解" page, section "from dense to sparse":
// decode speed ~ memory bandwidth / bytes of active weights). So the roles
// swap: weight rows are the MFMA M side (16 rows per v_mfma_f32_16x16x32_bf16)
// and the expert's tokens are the N side (16 per group, two groups per pass).
//   * Each lane streams 64 contiguous bytes of one weight row per step; the
//     reduction index is permuted identically for weights and tokens, which
//     leaves the dot products unchanged.
//   * A workgroup owns 16 output rows (gate_up: 16 gate + the matching 16 up
//     rows) and splits K over its 4 waves; partial sums meet in LDS in wave
//     order, so the result does not depend on timing.
//   * Experts with no tokens exit before reading anything, so only the
//     weights of experts that received tokens are read.
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int KB = 128;  // reduction elements per lane-group step (4 x 32)

struct SkinnyParams {
    const __bf16 *A;
    const int32_t *a_rows;
    const __bf16 *W;
    int64_t w_expert_stride;
    int K;
    int N;
    void *C;
    const int32_t *c_rows;
    const float *c_scale;
    const int32_t *counts;
    const int32_t *offsets;
    int dense_rows;
};

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

template <bool GATEUP>
__global__ __launch_bounds__(256) void skinny_gemm_kernel(SkinnyParams p)
{
    constexpr int NG = 2;  // token groups of 16 per pass
    constexpr int NW = GATEUP ? 2 : 1;
    __shared__ f32x4_t s_red[4][NG][NW][64];

    const int e = p.counts ? (int)blockIdx.y : 0;
    const int M = p.counts ? p.counts[e] : p.dense_rows;
    if (M <= 0) return;
    const int row0 = p.counts ? p.offsets[e] : 0;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n0 = blockIdx.x * 16;
    const int lgrp = lane >> 4;  // which 32-element quarter of a 128-element step

    const int nkb = (p.K + KB - 1) / KB;
    const int kb_lo = wave * nkb / 4;
    const int kb_hi = (wave + 1) * nkb / 4;

    const int wr = n0 + (lane & 15);
    const int wrc = wr < p.N ? wr : 0;
    const __bf16 *wbase = p.W + (int64_t)e * p.w_expert_stride;
    const __bf16 *wg = wbase + (int64_t)wrc * p.K + lgrp * 32;
    const __bf16 *wu = GATEUP ? wg + (int64_t)p.N * p.K : wg;
    const u32x4 zero = {0u, 0u, 0u, 0u};

    for (int pass = 0; pass < M; pass += 16 * NG) {
        const __bf16 *xp[NG];
        bool xv[NG];
#pragma unroll
        for (int g = 0; g < NG; g++) {
            const int q = pass + g * 16 + (lane & 15);
            xv[g] = q < M;
            const int qc = q < M ? q : M - 1;
            const int64_t src = p.a_rows ? (int64_t)p.a_rows[row0 + qc] : (int64_t)(row0 + qc);
            xp[g] = p.A + src * p.K + lgrp * 32;
        }
        const bool g1 = pass + 16 < M;  // second token group present (wave-uniform)

        f32x4_t acc[NG][NW];
#pragma unroll
        for (int g = 0; g < NG; g++)
#pragma unroll
            for (int w = 0; w < NW; w++) acc[g][w] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        for (int kb = kb_lo; kb < kb_hi; kb++) {
            const int k = kb * KB;
            u32x4 a[NW][4], b[NG][4];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const bool ok = k + lgrp * 32 + j * 8 < p.K;
                a[0][j] = ok ? *reinterpret_cast<const u32x4 *>(wg + k + j * 8) : zero;
                if (GATEUP) a[NW - 1][j] = ok ? *reinterpret_cast<const u32x4 *>(wu + k + j * 8) : zero;
                b[0][j] = (ok && xv[0]) ? *reinterpret_cast<const u32x4 *>(xp[0] + k + j * 8) : zero;
                if (g1) b[1][j] = (ok && xv[1]) ? *reinterpret_cast<const u32x4 *>(xp[1] + k + j * 8) : zero;
            }
#pragma unroll
            for (int j = 0; j < 4; j++) {
#pragma unroll
                for (int w = 0; w < NW; w++)
                    acc[0][w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[w][j]), as_bf16x8(b[0][j]),
                                                                        acc[0][w], 0, 0, 0);
                if (g1) {
#pragma unroll
                    for (int w = 0; w < NW; w++)
                        acc[1][w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            as_bf16x8(a[w][j]), as_bf16x8(b[1][j]), acc[1][w], 0, 0, 0);
                }
            }
        }

        // ---- split-K reduction across the 4 waves, in wave order
#pragma unroll
        for (int g = 0; g < NG; g++)
#pragma unroll
            for (int w = 0; w < NW; w++) s_red[wave][g][w][lane] = acc[g][w];
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int g = 0; g < NG; g++) {
                if (g == 1 && !g1) break;
                f32x4_t s[NW];
#pragma unroll
                for (int w = 0; w < NW; w++) {
                    s[w] = s_red[0][g][w][lane];
#pragma unroll
                    for (int v = 1; v < 4; v++) {
                        const f32x4_t o = s_red[v][g][w][lane];
                        s[w][0] += o[0]; s[w][1] += o[1]; s[w][2] += o[2]; s[w][3] += o[3];
                    }
                }
                const int q = pass + g * 16 + (lane & 15);
                const int c = n0 + 4 * lgrp;  // 4 consecutive output columns
                if (q < M && c < p.N) {
                    const int pos = row0 + q;
                    if (GATEUP) {
                        float hv[4];
#pragma unroll
                        for (int i = 0; i < 4; i++) hv[i] = silu_f32(s[0][i]) * s[NW - 1][i];
                        uint2 packed;
                        packed.x = pack_bf16x2(hv[0], hv[1]);
                        packed.y = pack_bf16x2(hv[2], hv[3]);
                        *reinterpret_cast<uint2 *>(reinterpret_cast<__bf16 *>(p.C) + (int64_t)pos * p.N + c) = packed;
                    } else {
                        const int64_t orow = p.c_rows ? (int64_t)p.c_rows[pos] : (int64_t)pos;
                        const float sc = p.c_scale ? p.c_scale[pos] : 1.0f;
                        float4 y = make_float4(s[0][0] * sc, s[0][1] * sc, s[0][2] * sc, s[0][3] * sc);
                        *reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.C) + orow * p.N + c) = y;
                    }
                }
            }
        }
        __syncthreads();
    }
}

SkinnyParams make_params(const GemmProblem &g)
{
    SkinnyParams s;
    s.A = (const __bf16 *)g.A;
    s.a_rows = g.a_rows;
    s.W = (const __bf16 *)g.W;
    s.w_expert_stride = g.w_expert_stride;
    s.K = (int)g.K;
    s.N = (int)g.N;
    s.C = g.C;
    s.c_rows = g.c_rows;
    s.c_scale = g.c_scale;
    s.counts = g.dense_rows > 0 ? nullptr : g.counts;
    s.offsets = g.dense_rows > 0 ? nullptr : g.offsets;
    s.dense_rows = (int)g.dense_rows;
    return s;
}

}  // namespace

hipError_t launch_gate_up_skinny(const GemmProblem &g, hipStream_t st)
{
    SkinnyParams s = make_params(g);
    dim3 grid((unsigned)((g.N + 15) / 16), g.dense_rows > 0 ? 1u : (unsigned)g.E);
    hipLaunchKernelGGL(skinny_gemm_kernel<true>, grid, dim3(256), 0, st, s);
    return hipGetLastError();
}

hipError_t launch_down_skinny(const GemmProblem &g, hipStream_t st)
{
    SkinnyParams s = make_params(g);
    dim3 grid((unsigned)((g.N + 15) / 16), g.dense_rows > 0 ? 1u : (unsigned)g.E);
    hipLaunchKernelGGL(skinny_gemm_kernel<false>, grid, dim3(256), 0, st, s);
    return hipGetLastError();
}

}  // namespace moe
