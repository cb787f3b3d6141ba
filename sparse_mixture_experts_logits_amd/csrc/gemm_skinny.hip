// Weight-streaming grouped expert GEMMs for few rows per expert (decode).
//
// With a handful of tokens per expert the layer is bound by reading the
// selected experts' weights once from HBM (the bandwidth model of the
// "Transformer中的混合专家架构详解" page, section "from dense to sparse":
// decode speed ~ memory bandwidth / bytes of active weights). So the roles
// swap: weight rows are the MFMA M side (16 rows per v_mfma_f32_16x16x32_bf16)
// and the expert's tokens are the N side (groups of 16).
//   * Loads are shaped for HBM, not for the MFMA: one load instruction reads
//     4 whole 256-byte row segments (16 lanes per row, non-temporal) through
//     a buffer resource, the row group's offset in a scalar register. Each
//     wave writes them to its own LDS tile and reads MFMA fragments back with
//     an xor swizzle that keeps both directions free of bank conflicts.
//   * The weight loads of the next steps (two ahead for bf16, one for the
//     low-precision formats) are issued as soon as the current step's data
//     is in LDS, the token fragments after the MFMAs that use the current
//     ones, so the bytes in flight per wave stay constant.
//   * A workgroup owns 32 weight rows (gate_up: 16 gate + the matching 16 up
//     rows; down: 32 consecutive rows; MXFP4: 32 + 32 and 64) and splits K
//     over its waves; partial sums meet in LDS in wave order, so the result
//     does not depend on timing.
//   * Experts with no tokens exit before reading anything, so only the
//     weights of experts that received tokens are read.
//   * FP8 weights (one byte each, OCP E4M3, one fp32 scale per weight row):
//     the same 256-byte row segments now hold 256 weights; each 16-byte
//     chunk is widened to two bf16 MFMA fragments in registers (exact: every
//     E4M3 value is a bf16 value) and the row scale multiplies the
//     accumulated sum in the epilogue, so a decode step reads half the bytes.
//   * MXFP4 weights (OCP MX: FP4 E2M1, two per byte, one E8M0 scale per 32
//     weights of a row): a 16-byte chunk is one block of 32 weights; its
//     scale byte travels with it through LDS, and each 32-bit word becomes
//     one bf16 MFMA fragment through four gfx950 scaled conversions (exact:
//     an E2M1 value times a power of two is a bf16 value), a quarter of the
//     bf16 bytes per decode step.
#include "moe_internal.h"

#include <limits.h>

namespace moe {

namespace {

constexpr int KB = 128;  // reduction elements per step: 256 bytes of each row
// Compile-time shape knobs of the streaming kernels, per GEMM and weight
// storage (bf16 / E4M3 "W8" / MXFP4 "W4"); the defaults are the fastest
// measured on MI355X for the decode shapes:
//   MOE_SKINNY_WAVES*     waves per workgroup, each taking a contiguous K range
//   MOE_SKINNY_PD_*       weight steps in flight per wave (staging registers)
//   MOE_SKINNY_*BLOCKS*   16-row blocks per workgroup (gate_up: half gate, half up)
#ifndef MOE_SKINNY_WAVES
#define MOE_SKINNY_WAVES 4
#endif
#ifndef MOE_SKINNY_PD_GU
#define MOE_SKINNY_PD_GU 2
#endif
#ifndef MOE_SKINNY_PD_DN
#define MOE_SKINNY_PD_DN 2
#endif
#ifndef MOE_SKINNY_PD_W8
#define MOE_SKINNY_PD_W8 1
#endif
#ifndef MOE_SKINNY_PD_W4
#define MOE_SKINNY_PD_W4 1
#endif
#ifndef MOE_SKINNY_DOWN_BLOCKS
#define MOE_SKINNY_DOWN_BLOCKS 2
#endif
#ifndef MOE_SKINNY_WAVES_W8
#define MOE_SKINNY_WAVES_W8 4
#endif
#ifndef MOE_SKINNY_GU_BLOCKS_W8
#define MOE_SKINNY_GU_BLOCKS_W8 2
#endif
#ifndef MOE_SKINNY_GU_BLOCKS_W4
#define MOE_SKINNY_GU_BLOCKS_W4 4
#endif
#ifndef MOE_SKINNY_DN_BLOCKS_W8
#define MOE_SKINNY_DN_BLOCKS_W8 MOE_SKINNY_DOWN_BLOCKS
#endif
#ifndef MOE_SKINNY_DN_BLOCKS_W4
#define MOE_SKINNY_DN_BLOCKS_W4 4
#endif
#ifndef MOE_SKINNY_WAVES_W4
#define MOE_SKINNY_WAVES_W4 2
#endif
#ifndef MOE_SKINNY_WAVES_DN
#define MOE_SKINNY_WAVES_DN MOE_SKINNY_WAVES
#endif
#ifndef MOE_SKINNY_WAVES_W4_DN
#define MOE_SKINNY_WAVES_W4_DN MOE_SKINNY_WAVES_W4
#endif
// waves per workgroup, splitting K, per GEMM and weight storage (bf16, E4M3, MXFP4)
constexpr int skinny_waves(bool gateup, int fmt)
{
    return fmt >= 2 ? (gateup ? MOE_SKINNY_WAVES_W4 : MOE_SKINNY_WAVES_W4_DN)
                    : fmt == 1 ? MOE_SKINNY_WAVES_W8 : (gateup ? MOE_SKINNY_WAVES : MOE_SKINNY_WAVES_DN);
}

// 16-row MFMA blocks per workgroup. gate_up: half of them gate rows, half the
// matching up rows; down: consecutive rows. A wave's token fragments serve
// all of its blocks, so the formats with more weights per byte (and so more
// token fragments per byte streamed) take more rows.
constexpr int skinny_blocks(bool gateup, int fmt)
{
    return gateup ? (fmt >= 2 ? MOE_SKINNY_GU_BLOCKS_W4 : fmt == 1 ? MOE_SKINNY_GU_BLOCKS_W8 : 2)
                  : (fmt >= 2 ? MOE_SKINNY_DN_BLOCKS_W4 : fmt == 1 ? MOE_SKINNY_DN_BLOCKS_W8 : MOE_SKINNY_DOWN_BLOCKS);
}
// output columns of h (gate_up) or output rows (down) per workgroup
constexpr int skinny_cols(bool gateup, int fmt) { return (gateup ? 8 : 16) * skinny_blocks(gateup, fmt); }

struct SkinnyParams {
    const __bf16 *A;
    const int32_t *a_rows;
    const void *W;             // bf16, E4M3 bytes or packed E2M1 nibbles
    const float *w_scale;      // E4M3: [E, rows per expert] scales, else null
    const uint8_t *w_bscale;   // MXFP4: [E, rows per expert, K / 32] E8M0 bytes, else null
    int64_t w_expert_stride;
    int K;
    int N;
    void *C;
    const int32_t *c_rows;
    const float *c_scale;
    const int32_t *counts;
    const int32_t *offsets;
    int dense_rows;
    // direct routing (ids != null): the expert's rows, their order and its
    // first sorted position come straight from the top-k ids, with no sorted
    // tables: row q of expert e is the q-th assignment a (ascending) with
    // ids[a] == e, its first position is the number of assignments to lower
    // experts, token a / k and routing weight wts[a]; down writes slot a.
    const int32_t *ids;
    const float *wts;
    int k;
    int TK;
    int max_rows;  // > 0: experts with more rows are left to the tiled kernel
};

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8_t, v); }

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

// Eight E4M3 weights (two 32-bit words, byte 0 first) -> eight bf16, two per
// instruction (gfx950's scaled FP8 conversion with scale 1: exact, since
// every E4M3 value is a bf16 value).
__device__ __forceinline__ u32x4 e4m3x8_to_bf16(uint32_t w0, uint32_t w1)
{
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true))};
}

// Eight E2M1 weights (one 32-bit word, element 2i in the low nibble of byte
// i) times the block factor s -> eight bf16 (exact for these products).
__device__ __forceinline__ u32x4 e2m1x8_to_bf16(uint32_t w, float s)
{
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3))};
}

// Buffer resource over n bytes at base (raw, untyped: word 3 as for gfx9
// raw buffers); loads through it take a per-lane 32-bit offset and a
// wave-uniform offset in a scalar register, so a row group's base address
// never occupies vector registers.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t n)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n, 0x00020000);
}
// 16 bytes at base + soff + voff, non-temporal (cache policy bit nt)
__device__ __forceinline__ u32x4 buffer_load_nt16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff)
{
    const u32x4v_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 2);
    return u32x4{v.x, v.y, v.z, v.w};
}

// the factor 2^(b - 127) of an E8M0 byte b as fp32 (b = 0: the subnormal 2^-127)
__device__ __forceinline__ float e8m0_factor(uint32_t b) { return __uint_as_float(b ? b << 23 : 0x00400000u); }

// v, or zeros when c is false (a per-component select: selecting between two
// lvalues would take their addresses and keep the staging arrays in memory)
__device__ __forceinline__ u32x4 keep_if(bool c, const u32x4 v)
{
    return u32x4{c ? v.x : 0u, c ? v.y : 0u, c ? v.z : 0u, c ? v.w : 0u};
}

// 16-byte chunk c (0..15) of row r (0..31) in a wave's LDS tile of 256-byte rows
__device__ __forceinline__ int tswz(int r, int c) { return r * 16 + (c ^ (r & 15)); }

#ifndef MOE_SKINNY_W8_OCC
#define MOE_SKINNY_W8_OCC 3
#endif
#ifndef MOE_SKINNY_W4_OCC
#define MOE_SKINNY_W4_OCC 2
#endif
#ifndef MOE_SKINNY_BF_OCC
#define MOE_SKINNY_BF_OCC 1
#endif
// FMT: weight storage, 0 bf16, 1 E4M3 (row scales), 2 MXFP4 (block scales),
// 3 MXFP4 whose rows of block scales start 4-byte aligned (K % 128 == 0), so
// a lane reads one row's 16 scales of a step with one 16-byte load.
// DIRECT: route straight from the top-k ids (see SkinnyParams).
template <bool GATEUP, int FMT, bool DIRECT, int G>
__global__ __launch_bounds__(skinny_waves(GATEUP, FMT) * 64,
                             FMT >= 2 ? MOE_SKINNY_W4_OCC : FMT ? MOE_SKINNY_W8_OCC : MOE_SKINNY_BF_OCC) void skinny_gemm_kernel(SkinnyParams p)
{
    constexpr bool W8 = FMT == 1;
    constexpr bool W4 = FMT >= 2;
    constexpr bool SC4 = FMT == 3;
    constexpr int SW = skinny_waves(GATEUP, FMT);
    constexpr int PD = W4 ? MOE_SKINNY_PD_W4 : W8 ? MOE_SKINNY_PD_W8 : GATEUP ? MOE_SKINNY_PD_GU : MOE_SKINNY_PD_DN;  // steps in flight
    constexpr int KS = W4 ? 4 * KB : W8 ? 2 * KB : KB;  // reduction elements per step (256 bytes of each row)
    constexpr int EPC = W4 ? 32 : W8 ? 16 : 8;          // elements per 16-byte chunk
    constexpr int FPC = EPC / 8;                        // MFMA fragments per chunk
    constexpr int XF = 4 * FPC;                         // token fragments per step
    // bytes of x weights (compile-time shifts, no multiply-then-divide)
    auto wbytes = [](uint32_t x) -> uint32_t { return W4 ? x >> 1 : W8 ? x : x << 1; };
    constexpr int NW = skinny_blocks(GATEUP, FMT);
    constexpr int NR = 16 * NW;         // weight rows per step (gate_up: NR / 2 gate, then NR / 2 up rows)
    constexpr int NL = NR / 4;          // load instructions per step
    static_assert(!GATEUP || NW % 2 == 0, "gate_up pairs gate and up blocks");
    // each wave's weight tile; after the K loop it holds the wave's partial sums
    __shared__ u32x4 s_w[SW][NR * 16];
    // MXFP4: the block scale of each chunk, row r's 16 in bytes [16r, 16r + 16)
    __shared__ __attribute__((aligned(16))) uint32_t s_bs[W4 ? SW : 1][W4 ? NR * 4 : 1];
    // direct routing: per row of the expert, its token (gate_up) or its
    // assignment (down)
    __shared__ int s_rows[DIRECT ? kSkinnyDirectMax : 1];
    __shared__ int s_cnt[2];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int e = (DIRECT || p.counts) ? (int)blockIdx.y : 0;
    int M, row0;
    if (DIRECT) {
        // one wave scans the ids 64 at a time: a ballot of "== e" gives each
        // match its rank, a ballot of "< e" counts the lower experts' rows
        if (wave == 0) {
            int cnt = 0, lower = 0;
            for (int a0 = 0; a0 < p.TK; a0 += 64) {
                const int a = a0 + lane;
                const int id = a < p.TK ? p.ids[a] : INT_MAX;
                const uint64_t eq = __ballot(id == e);
                const uint64_t lt = __ballot(id < e);
                const int rank = __builtin_amdgcn_mbcnt_hi((uint32_t)(eq >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)eq, 0u));
                if (id == e) s_rows[cnt + rank] = GATEUP ? a / p.k : a;
                cnt += __popcll(eq);
                lower += __popcll(lt);
            }
            if (lane == 0) {
                s_cnt[0] = cnt;
                s_cnt[1] = lower;
            }
        }
        __syncthreads();
        M = s_cnt[0];
        row0 = s_cnt[1];
    } else {
        M = p.counts ? p.counts[e] : p.dense_rows;
        row0 = p.counts ? p.offsets[e] : 0;
    }
    // workgroup-uniform: no rows, or more than this launch serves (those
    // experts run on the large-M tiled kernel)
    if (M <= 0 || (p.max_rows > 0 && M > p.max_rows)) return;
    const int n0 = blockIdx.x * skinny_cols(GATEUP, FMT);
    const int lgrp = lane >> 4;
    const int l16 = lane & 15;

    const int nkb = (p.K + KS - 1) / KS;
    const int kb_lo = wave * nkb / SW;
    const int kb_hi = (wave + 1) * nkb / SW;

    // load instruction i covers tile rows 4i..4i+3; this lane: row 4i + lgrp, chunk l16
    // element offsets inside one expert fit in 32 bits (2*I*H < 2^31 is checked on the host)
    // the expert's weights; a lane's chunk adds l16 * EPC elements to its row
    const uint8_t *wbase = reinterpret_cast<const uint8_t *>(p.W) +
                           (W4 ? (int64_t)e * p.w_expert_stride / 2 : (int64_t)e * p.w_expert_stride * (W8 ? 1 : 2));
    // MXFP4: the expert's block scales, K / 32 per row; chunk l16 of a step is block kb * 16 + l16
    const uint8_t *sbase = W4 ? p.w_bscale + (int64_t)e * (GATEUP ? 2 * p.N : p.N) * (p.K / 32) : nullptr;
    // Weights are read through buffer resources: load i's group of 4 rows
    // starts at a wave-uniform row (a scalar offset) and a lane adds its row
    // in the group (lgrp) and its chunk (a 32-bit vector offset), so no
    // per-load address occupies vector registers. A group past N is moved
    // back to rows N-4..N-1 (N % 4 == 0); columns past N are never written.
    auto urow = [&](int i) -> uint32_t {
        constexpr int half = GATEUP ? NR / 2 : NR;
        const int tr = 4 * i;
        const int n = min(n0 + tr % half, p.N - 4);
        return (GATEUP && tr >= half) ? p.N + n : n;
    };
    const uint32_t wrows = GATEUP ? 2 * p.N : p.N;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(wbase, wbytes(wrows * (uint32_t)p.K));
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(sbase, W4 ? wrows * (uint32_t)(p.K / 32) : 0u);
    u32x4 *tile = s_w[wave];
    const u32x4 zero = {0u, 0u, 0u, 0u};

    // wave 0: sum the waves' partials of one token group (rows q, valid xv)
    // and write them out
    auto red = [&](int v) { return reinterpret_cast<f32x4_t *>(s_w[v]); };
    auto epilogue = [&](const int q, const bool xv) {
            f32x4_t sm[NW];
#pragma unroll
            for (int w = 0; w < NW; w++) {
                sm[w] = red(0)[w * 64 + lane];
#pragma unroll
                for (int v = 1; v < SW; v++) {
                    const f32x4_t o = red(v)[w * 64 + lane];
                    sm[w][0] += o[0]; sm[w][1] += o[1]; sm[w][2] += o[2]; sm[w][3] += o[3];
                }
            }
            // lane: token column l16, output rows 4*lgrp + 0..3 of each 16-row block
            if (W8) {  // weight-row scales (E4M3 storage)
                const float *sc = p.w_scale + (int64_t)e * (GATEUP ? 2 * p.N : p.N);
#pragma unroll
                for (int w = 0; w < NW; w++)
#pragma unroll
                    for (int i = 0; i < 4; i++) {
                        const int cn = n0 + 16 * (GATEUP ? w % (NW / 2) : w) + 4 * lgrp + i;
                        const int r = GATEUP && w >= NW / 2 ? cn + p.N : cn;
                        sm[w][i] *= cn < p.N ? sc[r] : 0.0f;
                    }
            }
            if (xv) {
                const int pos = row0 + q;
                if (GATEUP) {
#pragma unroll
                    for (int w = 0; w < NW / 2; w++) {  // gate block w, up block w + NW / 2
                        const int c = n0 + 16 * w + 4 * lgrp;
                        if (c < p.N) {
                            float hv[4];
#pragma unroll
                            for (int i = 0; i < 4; i++) hv[i] = silu_f32(sm[w][i]) * sm[w + NW / 2][i];
                            uint2 packed;
                            packed.x = pack_bf16x2(hv[0], hv[1]);
                            packed.y = pack_bf16x2(hv[2], hv[3]);
                            *reinterpret_cast<uint2 *>(reinterpret_cast<__bf16 *>(p.C) + (int64_t)pos * p.N + c) = packed;
                        }
                    }
                } else {
                    const int64_t orow = DIRECT ? (int64_t)s_rows[q] : p.c_rows ? (int64_t)p.c_rows[pos] : (int64_t)pos;
                    const float sc = DIRECT ? p.wts[s_rows[q]] : p.c_scale ? p.c_scale[pos] : 1.0f;
#pragma unroll
                    for (int w = 0; w < NW; w++) {
                        const int c = n0 + 16 * w + 4 * lgrp;
                        if (c < p.N) {
                            float4 y = make_float4(sm[w][0] * sc, sm[w][1] * sc, sm[w][2] * sc, sm[w][3] * sc);
                            *reinterpret_cast<float4 *>(reinterpret_cast<float *>(p.C) + orow * p.N + c) = y;
                        }
                    }
                }
            }
    };

    // G groups of 16 tokens per pass share every weight step, so an expert
    // with up to 16 * G rows streams its weights exactly once; a group with
    // no rows skips its loads and MFMAs (pass-uniform).
    for (int pass = 0; pass < M; pass += 16 * G) {
        bool gon[G];
        int q[G];
        bool xv[G];
        const __bf16 *xp[G];
#pragma unroll
        for (int g = 0; g < G; g++) {
            gon[g] = pass + 16 * g < M;
            q[g] = pass + 16 * g + l16;
            xv[g] = q[g] < M;
            const int qc = xv[g] ? q[g] : M - 1;
            const int64_t src = (GATEUP && DIRECT) ? (int64_t)s_rows[qc]
                                : p.a_rows ? (int64_t)p.a_rows[row0 + qc] : (int64_t)(row0 + qc);
            xp[g] = p.A + src * p.K;  // the token's row; lanes add their chunk offsets
        }

        f32x4_t acc[G][NW];
#pragma unroll
        for (int g = 0; g < G; g++)
#pragma unroll
            for (int w = 0; w < NW; w++) acc[g][w] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        u32x4 st[PD][NL];
        uint32_t bs[PD][FMT == 2 ? NL : 1];  // MXFP4 block scale bytes of the staged chunks
        u32x4 sc[PD];                        // MXFP4, aligned scale rows: this lane's row's 16 scales
        u32x4 xs[G][PD][XF];
        // weights of step kb and the token fragments it needs: MFMA j takes
        // chunk 4j + lgrp (bf16: 8 elements; E4M3: 16 elements, as two MFMAs
        // over its halves, fragment 2j + half; MXFP4: 32 elements, as four
        // MFMAs over its words, fragment 4j + word)
        // Loads are unconditional and whole 16-byte loads: a chunk past K (or
        // a token past the expert's rows) reads the row's first chunk instead,
        // and the consumer zeroes it. With no branches or selects between a
        // load and its use, the compiler's wait counts stay exact and every
        // load of a step is in flight together.
        // (plain '&' and masks below, not '&&' or '?:', so that no branch is formed)
        auto w_ok = [&](int kb) { return kb * KS + l16 * EPC < p.K; };
        auto x_ok = [&](int kb, int f, int g) { return xv[g] & (kb * KS + (4 * (f / FPC) + lgrp) * EPC < p.K); };
        // (a chunk that is not read falls back to the row's first chunk, so
        // every address stays inside a row that exists)
        auto gload_w = [&](int kb, int b) {
            const uint32_t okm = 0u - (uint32_t)w_ok(kb);
            const uint32_t kbytes = wbytes((uint32_t)(kb * KS + l16 * EPC)) & okm;
            const uint32_t lw = wbytes((uint32_t)lgrp * (uint32_t)p.K) + kbytes;
            const uint32_t ls = (uint32_t)lgrp * (uint32_t)(p.K / 32) + ((uint32_t)(kb * 16 + l16) & okm);
#pragma unroll
            for (int i = 0; i < NL; i++) {
                st[b][i] = buffer_load_nt16(rw, lw, wbytes(urow(i) * (uint32_t)p.K));
                if (FMT == 2) bs[b][i] = __builtin_amdgcn_raw_buffer_load_b8(rs, ls, urow(i) * (uint32_t)(p.K / 32), 0);
            }
            if (SC4) {
                // lane r (mod NR) reads tile row r's 16 scales of the step (a
                // row past N reads row N - 1; its columns are never written)
                constexpr int half = GATEUP ? NR / 2 : NR;
                const int r = lane % NR;
                const int n = min(n0 + r % half, p.N - 1);
                const uint32_t grow = (GATEUP && r >= half) ? p.N + n : n;
                const u32x4v_t v = __builtin_amdgcn_raw_buffer_load_b128(rs, grow * (uint32_t)(p.K / 32) + kb * 16, 0, 0);
                sc[b] = u32x4{v.x, v.y, v.z, v.w};
            }
        };
        auto gload_x = [&](int kb, int b) {
#pragma unroll
            for (int g = 0; g < G; g++) {
                if (g > 0 && !gon[g]) break;
#pragma unroll
                for (int f = 0; f < XF; f++) {
                    // fragment f: chunk 4 * (f / FPC) + lgrp, its 8 elements (f % FPC)
                    const int off = (f / FPC) * 4 * EPC + (f % FPC) * 8;
                    xs[g][b][f] = load16(xp[g] + ((kb * KS + lgrp * EPC + off) & (0 - (int)x_ok(kb, f, g))));
                }
            }
        };
        // One reduction step from staging buffer b (a compile-time index after
        // unrolling). The next weights (from HBM, the long wait) are requested
        // as soon as this step's are in LDS; the next token fragments (L2
        // hits) only after this step's MFMAs have consumed the current ones, so
        // they need no second register copy and more waves fit on a SIMD.
        auto step = [&](int kb, int b) {
            const bool okw = w_ok(kb);
#pragma unroll
            for (int i = 0; i < NL; i++) tile[tswz(4 * i + lgrp, l16)] = keep_if(okw, st[b][i]);
            if (FMT == 2) {
                uint8_t *sb = reinterpret_cast<uint8_t *>(s_bs[W4 ? wave : 0]);
#pragma unroll
                for (int i = 0; i < NL; i++) sb[(4 * i + lgrp) * 16 + l16] = (uint8_t)bs[b][i];
            }
            if (SC4) {
                // scales of blocks past K (a ragged last step) read the next
                // row's; they become 127 (factor 1) so that the zero weights
                // there stay zero whatever those bytes hold
                const int nb = p.K / 32 - kb * 16;  // blocks of this step inside K
                auto keep = [&](uint32_t v, int d) {
                    const int nv = nb - 4 * d;
                    const uint32_t m = nv >= 4 ? 0xFFFFFFFFu : nv <= 0 ? 0u : (1u << (8 * nv)) - 1u;
                    return (v & m) | (0x7F7F7F7Fu & ~m);
                };
                if (lane < NR)
                    reinterpret_cast<u32x4 *>(s_bs[W4 ? wave : 0])[lane] =
                        u32x4{keep(sc[b].x, 0), keep(sc[b].y, 1), keep(sc[b].z, 2), keep(sc[b].w, 3)};
            }
            const bool more = kb + PD < kb_hi;
            if (more) gload_w(kb + PD, b);
            u32x4 xb[G][XF];
#pragma unroll
            for (int g = 0; g < G; g++)
#pragma unroll
                for (int f = 0; f < XF; f++) xb[g][f] = W4 ? xs[g][b][f] : keep_if(x_ok(kb, f, g), xs[g][b][f]);
#pragma unroll
            for (int j = 0; j < 4; j++) {
#pragma unroll
                for (int w = 0; w < NW; w++) {
                    const u32x4 a = tile[tswz(16 * w + l16, 4 * j + lgrp)];
                    // this chunk's weights as bf16 MFMA fragments, shared by every token group
                    constexpr int NF = W4 ? 4 : W8 ? 2 : 1;
                    bf16x8_t wf[NF];
                    if (W4) {
                        const uint8_t *sb = reinterpret_cast<const uint8_t *>(s_bs[W4 ? wave : 0]);
                        const float sf = e8m0_factor(sb[(16 * w + l16) * 16 + 4 * j + lgrp]);
                        wf[0] = as_bf16x8(e2m1x8_to_bf16(a.x, sf));
                        wf[NF > 1 ? 1 : 0] = as_bf16x8(e2m1x8_to_bf16(a.y, sf));
                        wf[NF > 2 ? 2 : 0] = as_bf16x8(e2m1x8_to_bf16(a.z, sf));
                        wf[NF > 3 ? 3 : 0] = as_bf16x8(e2m1x8_to_bf16(a.w, sf));
                    } else if (W8) {
                        wf[0] = as_bf16x8(e4m3x8_to_bf16(a.x, a.y));
                        wf[NF > 1 ? 1 : 0] = as_bf16x8(e4m3x8_to_bf16(a.z, a.w));
                    } else {
                        wf[0] = as_bf16x8(a);
                    }
#pragma unroll
                    for (int g = 0; g < G; g++) {
                        if (g > 0 && !gon[g]) break;
#pragma unroll
                        for (int h = 0; h < NF; h++)
                            acc[g][w] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[h], as_bf16x8(xb[g][NF * j + h]),
                                                                                acc[g][w], 0, 0, 0);
                    }
                }
                // MXFP4: convert each chunk just before its MFMAs; hoisting
                // every conversion of a step would need 256 more registers
                if (W4) __builtin_amdgcn_sched_barrier(0);
            }
            if (more) gload_x(kb + PD, b);
        };
#pragma unroll
        for (int b = 0; b < PD; b++)
            if (kb_lo + b < kb_hi) {
                gload_w(kb_lo + b, b);
                gload_x(kb_lo + b, b);
            }
        int kb = kb_lo;
        for (; kb + PD <= kb_hi; kb += PD) {
#pragma unroll
            for (int b = 0; b < PD; b++) step(kb + b, b);
        }
#pragma unroll
        for (int b = 0; b < PD - 1; b++)
            if (kb + b < kb_hi) step(kb + b, b);

        // ---- split-K reduction across the waves, in wave order (each wave's
        // partial sums go to its own tile, which it no longer reads), one
        // token group at a time
        static_assert(NW * 64 * sizeof(f32x4_t) <= NR * 16 * sizeof(u32x4), "partials fit the tile");
#pragma unroll
        for (int g = 0; g < G; g++) {
            if (g > 0 && !gon[g]) break;
            if (g > 0) __syncthreads();  // wave 0 is done with the previous group's partials
#pragma unroll
            for (int w = 0; w < NW; w++) red(wave)[w * 64 + lane] = acc[g][w];
            __syncthreads();
            if (wave == 0) epilogue(q[g], xv[g]);
        }
        __syncthreads();
    }
}

SkinnyParams make_params(const GemmProblem &g)
{
    SkinnyParams s;
    s.A = (const __bf16 *)g.A;
    s.a_rows = g.a_rows;
    s.W = g.W;
    s.w_scale = g.w_scale;
    s.w_bscale = g.w_bscale;
    s.w_expert_stride = g.w_expert_stride;
    s.K = (int)g.K;
    s.N = (int)g.N;
    s.C = g.C;
    s.c_rows = g.c_rows;
    s.c_scale = g.c_scale;
    s.counts = g.dense_rows > 0 ? nullptr : g.counts;
    s.offsets = g.dense_rows > 0 ? nullptr : g.offsets;
    s.dense_rows = (int)g.dense_rows;
    const bool direct = g.ids && g.dense_rows <= 0;
    s.ids = direct ? g.ids : nullptr;
    s.wts = direct ? g.wts : nullptr;
    s.k = g.k;
    s.TK = (int)g.total_rows;
    s.max_rows = g.dense_rows > 0 ? 0 : g.skinny_max_rows;
    return s;
}

}  // namespace

namespace {

// Token groups per pass: one when no expert can have more than 16 rows
// (max_rows, the host's bound), else two, so that an expert with up to 32
// rows streams its weights once (bf16 weights; the FP8 and MXFP4 variants
// keep one group: a second would not fit their registers).
template <bool GATEUP, int FMT>
void launch_fmt(dim3 grid, const SkinnyParams &s, int max_rows, hipStream_t st)
{
    const dim3 block(skinny_waves(GATEUP, FMT) * 64);
    if (FMT != 0 || max_rows <= 16) {  // the low-precision formats keep one group (register budget)
        if (s.ids) hipLaunchKernelGGL((skinny_gemm_kernel<GATEUP, FMT, true, 1>), grid, block, 0, st, s);
        else hipLaunchKernelGGL((skinny_gemm_kernel<GATEUP, FMT, false, 1>), grid, block, 0, st, s);
    } else {
        if (s.ids) hipLaunchKernelGGL((skinny_gemm_kernel<GATEUP, FMT, true, 2>), grid, block, 0, st, s);
        else hipLaunchKernelGGL((skinny_gemm_kernel<GATEUP, FMT, false, 2>), grid, block, 0, st, s);
    }
}

template <bool GATEUP>
hipError_t launch_skinny(const GemmProblem &g, hipStream_t st)
{
    const SkinnyParams s = make_params(g);
    // MXFP4 with 16-byte scale loads when every row of scales starts 4-byte
    // aligned: K / 32 a multiple of 4 and an aligned scale array
    const bool sc4 = g.w_bscale && (g.K / 32) % 4 == 0 && (uintptr_t)g.w_bscale % 4 == 0;
    const int fmt = g.w_bscale ? (sc4 ? 3 : 2) : g.w_scale ? 1 : 0;
    const int cols = skinny_cols(GATEUP, fmt);
    const dim3 grid((unsigned)((g.N + cols - 1) / cols), g.dense_rows > 0 ? 1u : (unsigned)g.E);
    // most rows one expert can hold: every row of a dense problem, at most
    // one per token otherwise (a token's k experts are distinct), and no
    // more than the launch serves
    int64_t mr = g.dense_rows > 0 ? g.dense_rows : g.total_rows / (g.k > 0 ? g.k : 1);
    if (s.max_rows > 0 && mr > s.max_rows) mr = s.max_rows;
    const int max_rows = (int)(mr < (1 << 30) ? mr : (1 << 30));
    switch (fmt) {
    case 3: launch_fmt<GATEUP, 3>(grid, s, max_rows, st); break;
    case 2: launch_fmt<GATEUP, 2>(grid, s, max_rows, st); break;
    case 1: launch_fmt<GATEUP, 1>(grid, s, max_rows, st); break;
    default: launch_fmt<GATEUP, 0>(grid, s, max_rows, st); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gate_up_skinny(const GemmProblem &g, hipStream_t st) { return launch_skinny<true>(g, st); }

hipError_t launch_down_skinny(const GemmProblem &g, hipStream_t st) { return launch_skinny<false>(g, st); }

}  // namespace moe
