// Per-row FP8 (OCP E4M3) quantisation of packed expert weights: the
// storage behind the FP8 decode path. The MoEs in Transformers page
// (section on why MoEs are fast) prices decode at memory bandwidth over the
// bytes of the active weights and notes that kernels for a native
// low-precision format are faster still; its weight-loading section adds
// that per-expert quantisation only makes sense once experts are packed in
// one tensor. Here each row of a packed tensor gets its own scale:
//   scale = max |w| / 448 (fp32 division), q = nearest E4M3 value to
//   w / scale (fp32 division), ties to the even code, saturating at 448.
// One workgroup per row; the row maximum is order-independent, and the
// code of each element is found from its fp32 bits, so the result is the
// same on every run.
#include "moe_internal.h"

namespace moe {

namespace {

// E4M3 byte of an fp32 value v with |v| <= 448 (plus rounding slack).
__device__ __forceinline__ uint32_t e4m3_code(float v)
{
    const uint32_t u = __float_as_uint(v);
    const uint32_t sign = (u >> 24) & 0x80u;
    const uint32_t a = u & 0x7fffffffu;
    uint32_t c;
    if (a >= 0x43e00000u) {
        c = 0x7eu;  // 448 and above: the largest finite code
    } else if (a < 0x3c800000u) {
        // below 2^-6: the subnormal grid m * 2^-9, m = 0..8 (8 is the first
        // normal code); the scaling by 512 is exact and rint rounds ties to even
        c = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
    } else {
        // normal: keep 3 mantissa bits, round to nearest even at bit 20,
        // re-bias the exponent from 127 to 7
        const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u);
        c = (r >> 20) - (120u << 3);
        c = c > 0x7eu ? 0x7eu : c;
    }
    return c ? (sign | c) : 0u;  // zero is stored as +0
}

// A row whose largest magnitude is below 448 * 2^-126 would need a
// subnormal scale; such rows are stored as zeros with scale 1.
constexpr float kMinRowMax = 0x1.cp-118f;  // 448 * 2^-126

__global__ __launch_bounds__(256) void quantize_e4m3_rows_kernel(const __bf16 *__restrict__ w, int64_t cols,
                                                                 uint8_t *__restrict__ q, float *__restrict__ scale)
{
    __shared__ float s_max[4];
    const int64_t r = blockIdx.x;
    const u32x4 *row = reinterpret_cast<const u32x4 *>(w + r * cols);
    const int nchunk = (int)(cols / 8);  // 8 bf16 per 16-byte chunk

    float m = 0.0f;
    for (int c = threadIdx.x; c < nchunk; c += 256) {
        const u32x4 v = row[c];
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 4; i++) m = fmaxf(m, fmaxf(fabsf(bf16_lo(wd[i])), fabsf(bf16_hi(wd[i]))));
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
    if ((threadIdx.x & 63) == 0) s_max[threadIdx.x >> 6] = m;
    __syncthreads();
    const float amax = fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
    const bool zero_row = !(amax >= kMinRowMax);
    const float s = zero_row ? 1.0f : amax / 448.0f;

    uint2 *qrow = reinterpret_cast<uint2 *>(q + r * cols);
    for (int c = threadIdx.x; c < nchunk; c += 256) {
        const u32x4 v = row[c];
        const uint32_t wd[4] = {v.x, v.y, v.z, v.w};
        uint32_t b[8];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            b[2 * i] = zero_row ? 0u : e4m3_code(bf16_lo(wd[i]) / s);
            b[2 * i + 1] = zero_row ? 0u : e4m3_code(bf16_hi(wd[i]) / s);
        }
        uint2 o;
        o.x = b[0] | (b[1] << 8) | (b[2] << 16) | (b[3] << 24);
        o.y = b[4] | (b[5] << 8) | (b[6] << 16) | (b[7] << 24);
        qrow[c] = o;
    }
    if (threadIdx.x == 0) scale[r] = s;
}

// MXFP4 (OCP Microscaling Formats v1.0): one thread per block of 32
// consecutive elements of a row. The block factor 2^x has x = floor(log2 a)
// - 2 for the block's largest magnitude a (read off a's fp32 exponent field;
// x = -127 below 2^-126), clamped to [-127, 127]; y = |w| * 2^-x is exact;
// its E2M1 code counts the rounding boundaries at or below it (ties go to
// the even code: 0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2, 2.5 -> 2,
// 3.5 -> 4, 5 -> 4, past 5 -> 6), and the sign bit is w's.
__device__ __forceinline__ uint32_t e2m1_code(float y)
{
    return (uint32_t)(y > 0.25f) + (uint32_t)(y >= 0.75f) + (uint32_t)(y > 1.25f) + (uint32_t)(y >= 1.75f) +
           (uint32_t)(y > 2.5f) + (uint32_t)(y >= 3.5f) + (uint32_t)(y > 5.0f);
}

__global__ __launch_bounds__(256) void quantize_mxfp4_rows_kernel(const __bf16 *__restrict__ w, int64_t nblocks,
                                                                  uint8_t *__restrict__ q, uint8_t *__restrict__ scale)
{
    const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;  // block of 32 elements
    if (b >= nblocks) return;
    const u32x4 *src = reinterpret_cast<const u32x4 *>(w + b * 32);
    uint32_t wd[16];
#pragma unroll
    for (int c = 0; c < 4; c++) {
        const u32x4 v = src[c];
        wd[4 * c] = v.x;
        wd[4 * c + 1] = v.y;
        wd[4 * c + 2] = v.z;
        wd[4 * c + 3] = v.w;
    }
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; i++) a = fmaxf(a, fmaxf(fabsf(bf16_lo(wd[i])), fabsf(bf16_hi(wd[i]))));
    const int ef = (int)((__float_as_uint(a) >> 23) & 0xffu);
    const int x = ef == 0 ? -127 : max(-127, min(127, ef - 129));
    uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; i++) {  // word i holds elements 2i (low half) and 2i+1
#pragma unroll
        for (int h = 0; h < 2; h++) {
            const float v = h ? bf16_hi(wd[i]) : bf16_lo(wd[i]);
            const uint32_t sign = h ? (wd[i] >> 31) : ((wd[i] >> 15) & 1u);
            const uint32_t code = e2m1_code(__builtin_ldexpf(fabsf(v), -x)) | (sign << 3);
            const int el = 2 * i + h;  // element: byte el / 2, nibble el % 2
            out[el / 8] |= code << (4 * (el % 8));
        }
    }
    reinterpret_cast<u32x4 *>(q)[b] = u32x4{out[0], out[1], out[2], out[3]};
    scale[b] = (uint8_t)(x + 127);
}

}  // namespace

hipError_t launch_quantize_mxfp4_rows(const void *w, int64_t rows, int64_t cols, void *q, void *scale, hipStream_t st)
{
    const int64_t nblocks = rows * (cols / 32);
    hipLaunchKernelGGL(quantize_mxfp4_rows_kernel, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, st,
                       (const __bf16 *)w, nblocks, (uint8_t *)q, (uint8_t *)scale);
    return hipGetLastError();
}

hipError_t launch_quantize_fp8_rows(const void *w, int64_t rows, int64_t cols, void *q, float *scale,
                                    hipStream_t st)
{
    hipLaunchKernelGGL(quantize_e4m3_rows_kernel, dim3((unsigned)rows), dim3(256), 0, st, (const __bf16 *)w, cols,
                       (uint8_t *)q, scale);
    return hipGetLastError();
}

}  // namespace moe
