// Weighted combine back to token order: out[t] = sum_j slot[t*k + j]
// (+ shared expert output), j ascending, fp32, one rounding to the output
// type. The slots already hold w[t,j] * expert output (written by the down
// GEMM epilogue), so this is the "apply routing weights, gather and reorder"
// step of the dispatch/combine flow ("Transformer中的混合专家架构详解" page,
// experts backends section) plus the shared-expert add (GraniteMoeSWA page,
// decoder-layer section; Instella page, FarSkipMoE: routed + shared).
#include "moe_internal.h"

namespace moe {

namespace {

// Slots and the shared output are read once: non-temporal loads keep them
// from displacing what the next launches reuse (skewed workload: 128 ->
// 108 us for 0.54 GB of slots; the Instella-style layer's next gate_up also
// ran 4% faster).
__device__ __forceinline__ float4 ld4(const float *p)
{
    typedef float f4v __attribute__((ext_vector_type(4)));
    const f4v v = __builtin_nontemporal_load(reinterpret_cast<const f4v *>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}

template <bool BF16OUT>
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ slot,
                                                      const float *__restrict__ sh_y, int64_t T,
                                                      int64_t H, int k, void *__restrict__ out)
{
    const int64_t n4 = T * (H / 4);
    for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < n4; idx += (int64_t)gridDim.x * 256) {
        const int64_t t = idx / (H / 4);
        const int64_t c = (idx - t * (H / 4)) * 4;
        const float *s = slot + (t * k) * H + c;
        float4 acc = ld4(s);
        for (int j = 1; j < k; j++) {
            const float4 v = ld4(s + (int64_t)j * H);
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        if (sh_y) {
            const float4 v = ld4(sh_y + t * H + c);
            acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
        }
        if (BF16OUT) {
            uint2 pk;
            pk.x = pack_bf16x2(acc.x, acc.y);
            pk.y = pack_bf16x2(acc.z, acc.w);
            *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(out) + t * H + c) = pk;
        } else {
            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(out) + t * H + c) = acc;
        }
    }
}

}  // namespace

hipError_t launch_combine(const Shape &s, const float *slot, const float *sh_y, void *out, hipStream_t st)
{
    const int64_t n4 = s.T * (s.H / 4);
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (s.dtype == 0)
        hipLaunchKernelGGL(combine_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, st, slot, sh_y,
                           s.T, s.H, s.k, out);
    else
        hipLaunchKernelGGL(combine_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, st, slot, sh_y,
                           s.T, s.H, s.k, out);
    return hipGetLastError();
}

}  // namespace moe
