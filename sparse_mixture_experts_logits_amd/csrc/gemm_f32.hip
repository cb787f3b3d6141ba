// fp32 expert GEMMs (dtype MOE_F32): plain VALU dot products, one output
// element per thread. This path serves small fp32 layers; the bf16 paths
// carry the performance work. Same packed layouts and fused epilogues as the
// bf16 kernels: gate_up_proj rows [0, I) gate, [I, 2I) up, h = silu(g) * u
// ("深入解析 Transformers 中的 PhiMoE" page, section 2, item 3); down output
// scaled by the routing weight and written to the assignment's slot.
#include "moe_internal.h"

namespace moe {

namespace {

struct F32Params {
    const float *A;
    const int32_t *a_rows;
    const float *W;
    int64_t w_expert_stride;
    int K;
    int N;
    float *C;
    const int32_t *c_rows;
    const float *c_scale;
    const int32_t *row_expert;
    int rows;
};

__global__ __launch_bounds__(256) void f32_gate_up_kernel(F32Params p)
{
    const int nbk = (p.N + 255) / 256;
    const int r = blockIdx.x / nbk;
    const int n = (blockIdx.x - r * nbk) * 256 + threadIdx.x;
    if (r >= p.rows || n >= p.N) return;
    const int64_t src = p.a_rows ? (int64_t)p.a_rows[r] : (int64_t)r;
    const int e = p.row_expert ? p.row_expert[r] : 0;
    const float *x = p.A + src * p.K;
    const float *wg = p.W + (int64_t)e * p.w_expert_stride + (int64_t)n * p.K;
    const float *wu = wg + (int64_t)p.N * p.K;
    float g = 0.f, u = 0.f;
    for (int i = 0; i < p.K; i++) {
        g = __builtin_fmaf(wg[i], x[i], g);
        u = __builtin_fmaf(wu[i], x[i], u);
    }
    p.C[(int64_t)r * p.N + n] = silu_f32(g) * u;
}

__global__ __launch_bounds__(256) void f32_down_kernel(F32Params p)
{
    const int nbk = (p.N + 255) / 256;
    const int r = blockIdx.x / nbk;
    const int m = (blockIdx.x - r * nbk) * 256 + threadIdx.x;
    if (r >= p.rows || m >= p.N) return;
    const int e = p.row_expert ? p.row_expert[r] : 0;
    const float *h = p.A + (int64_t)r * p.K;
    const float *wd = p.W + (int64_t)e * p.w_expert_stride + (int64_t)m * p.K;
    float y = 0.f;
    for (int i = 0; i < p.K; i++) y = __builtin_fmaf(wd[i], h[i], y);
    const int64_t orow = p.c_rows ? (int64_t)p.c_rows[r] : (int64_t)r;
    const float sc = p.c_scale ? p.c_scale[r] : 1.0f;
    p.C[orow * p.N + m] = y * sc;
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
    f.row_expert = g.dense_rows > 0 ? nullptr : g.row_expert;
    f.rows = (int)g.total_rows;
    return f;
}

}  // namespace

hipError_t launch_gate_up_f32(const GemmProblem &g, hipStream_t st)
{
    F32Params f = make_params(g);
    dim3 grid((unsigned)(((g.N + 255) / 256) * g.total_rows));
    hipLaunchKernelGGL(f32_gate_up_kernel, grid, dim3(256), 0, st, f);
    return hipGetLastError();
}

hipError_t launch_down_f32(const GemmProblem &g, hipStream_t st)
{
    F32Params f = make_params(g);
    dim3 grid((unsigned)(((g.N + 255) / 256) * g.total_rows));
    hipLaunchKernelGGL(f32_down_kernel, grid, dim3(256), 0, st, f);
    return hipGetLastError();
}

}  // namespace moe
