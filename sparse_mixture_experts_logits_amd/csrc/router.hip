// Router, top-k selection and the expert-major permutation.
//
// Router: a bias-free linear layer hidden -> experts, top-k by logit with
// the weights renormalised over the selected experts ("深入解析 Transformers
// 中的 PhiMoE" page, section 6: PhimoeTopKRouter and sparsemixer at
// inference). Permutation: assignments sorted by expert id and grouped, as
// the grouped_mm experts backend does ("Transformer中的混合专家架构详解" page,
// experts backends section), with no token dropped (PhiMoE page, section 2,
// item 4).
//
// Bit-exactness: the logit is the fp32 sum in the fixed order stated in
// moe_mi355x.h (lane L of a wave owns elements 512c + 8L + v, c then v
// ascending, then an xor butterfly 32..1). This translation unit is built
// with -ffp-contract=off and uses explicit fmaf, so the compiler cannot
// change that order. Counts come from integer atomics (order-independent)
// and the permutation from explicit stable ranks, so ids, counts, offsets
// and perm are identical on every run.
#include "moe_internal.h"

#include <float.h>
#include <limits.h>

namespace moe {

namespace {

// A slice of 8 consecutive row elements as loaded (bf16: one 16-byte load,
// widened to fp32 exactly only when used, so more slices fit in flight).
template <typename Tin>
struct Slice;

template <>
struct Slice<__bf16> {
    u32x4 q;
    __device__ __forceinline__ void load(const __bf16 *row, int64_t i) { q = *reinterpret_cast<const u32x4 *>(row + i); }
    __device__ __forceinline__ float at(int v) const
    {
        const uint32_t w = v < 2 ? q.x : v < 4 ? q.y : v < 6 ? q.z : q.w;
        return (v & 1) ? bf16_hi(w) : bf16_lo(w);
    }
};

template <>
struct Slice<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float *row, int64_t i)
    {
        a = *reinterpret_cast<const float4 *>(row + i);
        b = *reinterpret_cast<const float4 *>(row + i + 4);
    }
    __device__ __forceinline__ float at(int v) const
    {
        return v == 0 ? a.x : v == 1 ? a.y : v == 2 ? a.z : v == 3 ? a.w : v == 4 ? b.x : v == 5 ? b.y : v == 6 ? b.z : b.w;
    }
};

// e^x for x in [-80, 80] from IEEE operations only (so it is the same bit for
// bit wherever fma, rint, ldexp and the basic operations are correctly
// rounded): x = n ln2 + r with ln2 split in two for an exact-enough r,
// |r| <= ln2/2, e^r by its Taylor series to degree 8 (Horner, fused
// multiply-adds), then scaled by 2^n.
__device__ __forceinline__ float exp_ieee(float x)
{
    const float n = __builtin_rintf(x * 1.44269502f);
    float r = __builtin_fmaf(-n, 0.693145751953125f, x);  // ln2 high part (exact product)
    r = __builtin_fmaf(-n, 1.42860682e-06f, r);           // ln2 low part
    float p = 2.48015873e-05f;                             // 1/8!
    p = __builtin_fmaf(p, r, 1.98412698e-04f);             // 1/7!
    p = __builtin_fmaf(p, r, 1.38888889e-03f);             // 1/6!
    p = __builtin_fmaf(p, r, 8.33333333e-03f);             // 1/5!
    p = __builtin_fmaf(p, r, 4.16666667e-02f);             // 1/4!
    p = __builtin_fmaf(p, r, 1.66666667e-01f);             // 1/3!
    p = __builtin_fmaf(p, r, 0.5f);
    p = __builtin_fmaf(p, r, 1.0f);
    p = __builtin_fmaf(p, r, 1.0f);
    return __builtin_ldexpf(p, (int)n);
}

// sigmoid with the logit clamped to [-80, 80] (no subnormal results)
__device__ __forceinline__ float sigmoid_ieee(float l)
{
    const float c = fminf(fmaxf(l, -80.0f), 80.0f);
    return 1.0f / (1.0f + exp_ieee(-c));
}

// (va, ia) ranks before (vb, ib): larger logit first, then lower expert index.
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib)
{
    return va > vb || (va == vb && ia < ib);
}

// One workgroup routes RT tokens. The 4 waves split the experts; each wave
// takes TG tokens x 4 experts at a time so every loaded slice of hidden and
// router weights feeds several dot products, and all loads of a 512-element
// chunk are issued before its fmas.
template <typename Tin, int RT, int NW>
__global__ __launch_bounds__(NW * 64) void router_topk_kernel(
    const Tin *__restrict__ X, const Tin *__restrict__ Wr, const float *__restrict__ bias, int T,
    int H, int E, int k, float routed_scale, int32_t *__restrict__ ids, float *__restrict__ wts,
    int32_t *__restrict__ ids_out, float *__restrict__ wts_out, float *__restrict__ logits_out,
    int32_t *__restrict__ blk_counts, const int32_t *__restrict__ stats_mask, float *__restrict__ blk_prob,
    int32_t *__restrict__ blk_mcnt, int32_t *__restrict__ blk_ntok, int score_func,
    const float *__restrict__ sel_bias, int n_group, int topk_group, float jitter_eps)
{
    constexpr int TG = RT < 8 ? RT : 8;  // tokens per pass
    constexpr int EG = 4;                // experts per pass
    __shared__ float s_logit[RT][kMaxExperts];
    __shared__ float s_sel[4][kMaxExperts];
    __shared__ int s_hist[kMaxExperts];
    // router statistics (when blk_prob is set): softmax over all experts of
    // each counted token, and the assignments and number of counted tokens
    __shared__ float s_prob[RT][kMaxExperts];
    __shared__ int s_mhist[kMaxExperts];
    __shared__ int s_ntok;
    // group-limited selection: selection keys and kept groups of each wave's token
    __shared__ float s_key[4][kMaxExperts];
    __shared__ int s_gkeep[4][kMaxGroups];
    const bool sigm = score_func == 1;
    const bool smix = score_func == 2;
    const float thr = 2.0f * jitter_eps;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int tblk = blockIdx.x * RT;
    const bool stats = blk_prob != nullptr;

    for (int e = threadIdx.x; e < E; e += NW * 64) {
        s_hist[e] = 0;
        s_mhist[e] = 0;
    }
    if (threadIdx.x == 0) s_ntok = 0;

    // ---- logits
    const int epw = (E + NW - 1) / NW;
    const int e_lo = wave * epw;
    const int e_hi = min(E, e_lo + epw);
    const int nchunk = (H + 511) / 512;
    for (int tg = 0; tg < RT; tg += TG) {
        const Tin *xrow[TG];
#pragma unroll
        for (int j = 0; j < TG; j++) {
            int t = tblk + tg + j;
            t = t < T ? t : T - 1;  // rows past T repeat a valid row; results dropped
            xrow[j] = X + (int64_t)t * H;
        }
        for (int es = e_lo; es < e_hi; es += EG) {
            const Tin *wrow[EG];
#pragma unroll
            for (int q = 0; q < EG; q++) {
                const int e = min(es + q, E - 1);  // clamped rows are computed and dropped
                wrow[q] = Wr + (int64_t)e * H;
            }
            float acc[TG][EG];
#pragma unroll
            for (int j = 0; j < TG; j++)
#pragma unroll
                for (int q = 0; q < EG; q++) acc[j][q] = 0.0f;
            // CU chunks per step: every load of a step is issued before its
            // fmas, which still run in chunk order
            constexpr int CU = TG == 1 ? 8 : 2;
            for (int c0 = 0; c0 < nchunk; c0 += CU) {
                Slice<Tin> xv[CU][TG], wv[CU][EG];
#pragma unroll
                for (int u = 0; u < CU; u++) {
                    // H is a multiple of 8: a slice is all valid or all absent. An
                    // absent slice loads the row's first slice (and is not used), so
                    // the loads need no branch and all of them are in flight at once.
                    const int64_t i0 = (int64_t)(c0 + u) * 512 + lane * 8;
                    const int64_t ia = i0 & -(int64_t)(i0 < H);
#pragma unroll
                    for (int j = 0; j < TG; j++) xv[u][j].load(xrow[j], ia);
#pragma unroll
                    for (int q = 0; q < EG; q++) wv[u][q].load(wrow[q], ia);
                }
#pragma unroll
                for (int u = 0; u < CU; u++) {
                    const int64_t i0 = (int64_t)(c0 + u) * 512 + lane * 8;
                    if (i0 < H) {
#pragma unroll
                        for (int j = 0; j < TG; j++)
#pragma unroll
                            for (int q = 0; q < EG; q++)
#pragma unroll
                                for (int v = 0; v < 8; v++)
                                    acc[j][q] = __builtin_fmaf(xv[u][j].at(v), wv[u][q].at(v), acc[j][q]);
                    }
                }
            }
            // xor butterfly over the 64 lanes: P[L] <- P[L] + P[L ^ d], d = 32..1
#pragma unroll
            for (int j = 0; j < TG; j++)
#pragma unroll
                for (int q = 0; q < EG; q++) {
                    float v = acc[j][q];
#pragma unroll
                    for (int d = 32; d >= 1; d >>= 1) v = v + __shfl_xor(v, d, 64);
                    acc[j][q] = v;
                }
            if (lane == 0) {
#pragma unroll
                for (int j = 0; j < TG; j++)
#pragma unroll
                    for (int q = 0; q < EG; q++) {
                        const int e = es + q;
                        if (e < e_hi) {
                            float l = acc[j][q];
                            if (bias) l = l + bias[e];
                            s_logit[tg + j][e] = l;
                        }
                    }
            }
        }
    }
    __syncthreads();

    // ---- optional logits output
    if (logits_out) {
        for (int idx = threadIdx.x; idx < RT * E; idx += NW * 64) {
            const int j = idx / E, e = idx - j * E;
            const int t = tblk + j;
            if (t < T) logits_out[(int64_t)t * E + e] = s_logit[j][e];
        }
    }

    // ---- top-k per token: k rounds of a wave-wide arg-max under the ranking rule
    for (int j = wave; j < RT; j += NW) {  // RT <= 4 with NW = 8: waves 4..7 route no token
        const int t = tblk + j;
        if (t >= T) break;  // wave-uniform
        const float *lrow = s_logit[j];
        float v[4];
        bool taken[4];
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int e = lane + 64 * q;
            v[q] = e < E ? lrow[e] : -FLT_MAX;
            taken[q] = e >= E;
        }
        // scores (weights) and selection keys
        float sc[4], key[4];
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int e = lane + 64 * q;
            sc[q] = (e < E && sigm) ? sigmoid_ieee(v[q]) : v[q];
            key[q] = sc[q];
            if (e < E && sel_bias) key[q] = key[q] + sel_bias[e];
            if (key[q] != key[q]) key[q] = -INFINITY;  // a NaN key ranks below every number
        }
        const bool counted = stats && (!stats_mask || stats_mask[t] != 0);  // wave-uniform
        if (stats) {
            // probabilities over all E experts (zero rows for tokens not counted)
            float m = -FLT_MAX;
#pragma unroll
            for (int q = 0; q < 4; q++) m = fmaxf(m, v[q]);
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
            float ex[4], sum = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                ex[q] = taken[q] ? 0.0f : __expf(v[q] - m);  // taken[] marks e >= E here
                sum += ex[q];
            }
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) sum += __shfl_xor(sum, d, 64);
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int e = lane + 64 * q;
                if (e < E) s_prob[j][e] = counted ? ex[q] / sum : 0.0f;
            }
            if (counted && lane == 0) atomicAdd(&s_ntok, 1);
        }
        if (n_group > 1) {
            // group score: fp32 sum of the group's best two keys (one if the
            // group has one expert), best first
            float *kr = s_key[wave];
#pragma unroll
            for (int q = 0; q < 4; q++)
                if (lane + 64 * q < E) kr[lane + 64 * q] = key[q];
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
            const int gsz = E / n_group;
            const int gtop = min(2, gsz);
            float gsc = -INFINITY;
            if (lane < n_group) {
                float sum = 0.0f, pv = INFINITY;
                int pi = -1;
                for (int r = 0; r < gtop; r++) {
                    float bv = -INFINITY;
                    int bi = INT_MAX;
                    for (int x = 0; x < gsz; x++) {
                        const int e = lane * gsz + x;
                        const float kv = kr[e];
                        if (ranks_before(pv, pi, kv, e) && ranks_before(kv, e, bv, bi)) {
                            bv = kv;
                            bi = e;
                        }
                    }
                    sum += bv;
                    pv = bv;
                    pi = bi;
                }
                gsc = sum != sum ? -INFINITY : sum;  // (+inf) + (-inf)
            }
            // keep the topk_group best groups (ties to the lower group)
            bool kept = false;
            for (int r = 0; r < topk_group; r++) {
                float bv = (lane < n_group && !kept) ? gsc : -INFINITY;
                int bi = (lane < n_group && !kept) ? lane : INT_MAX;
#pragma unroll
                for (int d = 32; d >= 1; d >>= 1) {
                    const float ov = __shfl_xor(bv, d, 64);
                    const int oi = __shfl_xor(bi, d, 64);
                    if (ranks_before(ov, oi, bv, bi)) {
                        bv = ov;
                        bi = oi;
                    }
                }
                if (lane == bi) kept = true;
            }
            if (lane < n_group) s_gkeep[wave][lane] = kept ? 1 : 0;
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int e = lane + 64 * q;
                if (e < E && !s_gkeep[wave][e / gsz]) taken[q] = true;
            }
        }
        for (int s = 0; s < k; s++) {
            // -inf, so that an expert whose key is -inf can still be chosen:
            // every token gets k valid experts whatever its logits
            float bv = -INFINITY;
            int bi = INT_MAX;
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int e = lane + 64 * q;
                if (!taken[q] && ranks_before(key[q], e, bv, bi)) {
                    bv = key[q];
                    bi = e;
                }
            }
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) {
                const float ov = __shfl_xor(bv, d, 64);
                const int oi = __shfl_xor(bi, d, 64);
                if (ranks_before(ov, oi, bv, bi)) {
                    bv = ov;
                    bi = oi;
                }
            }
            // every lane now holds the winner (bv, bi)
            if (smix) {
                // sparsemixer round: a softmax, taken at the winner, over the
                // experts not chosen yet whose logit is within the relative
                // threshold of the winner's (bv is the winner's logit here)
                float z = 0.0f;
#pragma unroll
                for (int q = 0; q < 4; q++)
                    if (!taken[q]) {
                        const float f = fmaxf(fabsf(v[q]), bv);
                        if (!((bv - v[q]) / f > thr)) z += __expf(v[q] - bv);
                    }
#pragma unroll
                for (int d = 32; d >= 1; d >>= 1) z += __shfl_xor(z, d, 64);
                if (lane == 0) s_sel[wave][s] = 1.0f / z;
            }
            // the winner's owner marks it and records its unbiased score (the
            // logit for softmax)
#pragma unroll
            for (int q = 0; q < 4; q++)
                if (lane + 64 * q == bi) {
                    taken[q] = true;
                    if (!smix) s_sel[wave][s] = sc[q];
                }
            if (lane == 0) {
                ids[(int64_t)t * k + s] = bi;
                if (ids_out) ids_out[(int64_t)t * k + s] = bi;
                atomicAdd(&s_hist[bi], 1);
                if (counted) atomicAdd(&s_mhist[bi], 1);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
        // weights, times the routed scale: softmax over the selected logits
        // (relative to their largest), the selected sigmoid scores over
        // their sum, or each sparsemixer round's own softmax value
        if (smix) {
            for (int s = lane; s < k; s += 64) {
                const float w = routed_scale * s_sel[wave][s];
                wts[(int64_t)t * k + s] = w;
                if (wts_out) wts_out[(int64_t)t * k + s] = w;
            }
            __builtin_amdgcn_wave_barrier();
            continue;
        }
        float m = -FLT_MAX;
        for (int s = lane; s < k; s += 64) m = fmaxf(m, s_sel[wave][s]);
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
        float psum = 0.0f;
        for (int s = lane; s < k; s += 64) psum += sigm ? s_sel[wave][s] : __expf(s_sel[wave][s] - m);
#pragma unroll
        for (int d = 32; d >= 1; d >>= 1) psum += __shfl_xor(psum, d, 64);
        for (int s = lane; s < k; s += 64) {
            const float num = sigm ? s_sel[wave][s] : __expf(s_sel[wave][s] - m);
            const float w = routed_scale * (num / psum);
            wts[(int64_t)t * k + s] = w;
            if (wts_out) wts_out[(int64_t)t * k + s] = w;
        }
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += NW * 64) blk_counts[(int64_t)blockIdx.x * E + e] = s_hist[e];
    if (stats) {
        const int nt = min(RT, T - tblk);
        for (int e = threadIdx.x; e < E; e += NW * 64) {
            float ps = 0.0f;
            for (int j = 0; j < nt; j++) ps += s_prob[j][e];  // token order
            blk_prob[(int64_t)blockIdx.x * E + e] = ps;
            blk_mcnt[(int64_t)blockIdx.x * E + e] = s_mhist[e];
        }
        if (threadIdx.x == 0) blk_ntok[blockIdx.x] = s_ntok;
    }
}

// One workgroup: expert totals, exclusive offsets, per-block bases and the
// M-tile list of the large-M schedule.
__global__ __launch_bounds__(1024) void route_scan_kernel(
    const int32_t *__restrict__ blk_counts, int nblk, int E, int BM, int XT, int min_rows, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ blk_base, int32_t *__restrict__ tile_start,
    MTile *__restrict__ tiles, int32_t *__restrict__ counts_out, int32_t *__restrict__ offsets_out,
    const float *__restrict__ blk_prob, const int32_t *__restrict__ blk_mcnt, const int32_t *__restrict__ blk_ntok,
    float *__restrict__ prob_mean, float *__restrict__ load, float *__restrict__ aux)
{
    __shared__ int s_part[1024];
    __shared__ int s_cnt[kMaxExperts];
    __shared__ int s_off[kMaxExperts + 1];
    __shared__ int s_ts[kMaxExperts + 1];
    // M-tiles of an expert with c rows: as few as hold them at up to BM + XT
    // rows each. When c exceeds n * BM, the excess rides as extra rows in the
    // first tiles (XT each, the rest in the next), so no tile is left with a
    // handful of rows that would stream a whole weight block for them; else
    // the tiles hold BM rows and the last one the remainder.
    // Experts with fewer than min_rows rows get no tile: the weight-streaming
    // kernel serves them (mixed schedule).
    auto n_tiles = [&](int c) { return c < min_rows ? 0 : (c + BM + XT - 1) / (BM + XT); };
    // first row (relative to the expert's offset) and rows of its tile i of n
    auto tile_rows = [&](int c, int n, int i, int &r0, int &rows) {
        const int extra = max(c - n * BM, 0);
        r0 = i * BM + min(extra, i * XT);
        rows = extra > 0 ? BM + min(max(extra - i * XT, 0), XT) : (i == n - 1 ? c - i * BM : BM);
    };

    const int tid = threadIdx.x;
    // G groups of threads split the router blocks per expert; E <= 256 so
    // G >= 4, and at most 64 so that the serial pass over the groups below
    // stays short when there are few experts
    const int G = min(1024 / E, 64);
    const int g = tid / E, e = tid - (tid / E) * E;
    const int chunk = (nblk + G - 1) / G;
    const int b0 = g * chunk;
    const int b1 = min(nblk, b0 + chunk);
    if (g < G) {
        int s = 0;
        int b = b0;
        for (; b + 16 <= b1; b += 16) {  // sixteen independent loads per step
            int v[16];
#pragma unroll
            for (int u = 0; u < 16; u++) v[u] = blk_counts[(int64_t)(b + u) * E + e];
#pragma unroll
            for (int u = 0; u < 16; u++) s += v[u];
        }
        for (; b < b1; b++) s += blk_counts[(int64_t)b * E + e];
        s_part[g * E + e] = s;
    }
    __syncthreads();
    if (tid < E) {
        int run = 0;
        for (int gg = 0; gg < G; gg++) {
            const int c = s_part[gg * E + tid];
            s_part[gg * E + tid] = run;
            run += c;
        }
        s_cnt[tid] = run;
    }
    __syncthreads();
    // expert offsets and first tiles: inclusive prefix sums of the counts and
    // tile counts over the experts, log2(E) doubling steps (integer sums, so
    // the same values as a serial pass)
    __shared__ int s_scan[2][2][kMaxExperts];
    if (tid < E) {
        s_scan[0][0][tid] = s_cnt[tid];
        s_scan[0][1][tid] = n_tiles(s_cnt[tid]);
    }
    __syncthreads();
    int src = 0;
    for (int d = 1; d < E; d <<= 1) {
        if (tid < E) {
            int a = s_scan[src][0][tid], t = s_scan[src][1][tid];
            if (tid >= d) {
                a += s_scan[src][0][tid - d];
                t += s_scan[src][1][tid - d];
            }
            s_scan[src ^ 1][0][tid] = a;
            s_scan[src ^ 1][1][tid] = t;
        }
        src ^= 1;
        __syncthreads();
    }
    if (tid < E) {
        s_off[tid + 1] = s_scan[src][0][tid];
        s_ts[tid + 1] = s_scan[src][1][tid];
    }
    if (tid == 0) {
        s_off[0] = 0;
        s_ts[0] = 0;
    }
    __syncthreads();
    if (g < G) {
        int base = s_off[e] + s_part[g * E + e];
        int b = b0;
        for (; b + 16 <= b1; b += 16) {
            int v[16];
#pragma unroll
            for (int u = 0; u < 16; u++) v[u] = blk_counts[(int64_t)(b + u) * E + e];
#pragma unroll
            for (int u = 0; u < 16; u++) {
                blk_base[(int64_t)(b + u) * E + e] = base;
                base += v[u];
            }
        }
        for (; b < b1; b++) {
            blk_base[(int64_t)b * E + e] = base;
            base += blk_counts[(int64_t)b * E + e];
        }
    }
    if (tid < E) {
        counts[tid] = s_cnt[tid];
        if (counts_out) counts_out[tid] = s_cnt[tid];
    }
    // the tile list, one thread per tile: its expert is the last one whose
    // first tile is at or before it (binary search over the first tiles)
    for (int idx = tid; idx < s_ts[E]; idx += 1024) {
        int lo = 0, hi = E;  // s_ts[lo] <= idx < s_ts[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_ts[mid] <= idx) lo = mid;
            else hi = mid;
        }
        const int nt = s_ts[lo + 1] - s_ts[lo];
        MTile m;
        int r0, rows;
        tile_rows(s_cnt[lo], nt, idx - s_ts[lo], r0, rows);
        m.expert = lo;
        m.row0 = s_off[lo] + r0;
        m.rows = rows;
        m.pad = 0;
        tiles[idx] = m;
    }
    if (tid <= E) {
        offsets[tid] = s_off[tid];
        tile_start[tid] = s_ts[tid];
        if (offsets_out) offsets_out[tid] = s_off[tid];
    }
    if (!blk_prob) return;

    // ---- router statistics: the same fixed group order for the fp32 sums
    __shared__ float s_pp[1024];
    __shared__ int s_mp[1024];
    __shared__ int s_nt[1024];
    __shared__ float s_load[kMaxExperts];
    __shared__ float s_prob[kMaxExperts];
    if (g < G) {
        // sixteen blocks' loads in flight per step, summed in block order
        float ps = 0.0f;
        int ms = 0;
        int b = b0;
        for (; b + 16 <= b1; b += 16) {
            float pv[16];
            int mv[16];
#pragma unroll
            for (int u = 0; u < 16; u++) {
                pv[u] = blk_prob[(int64_t)(b + u) * E + e];
                mv[u] = blk_mcnt[(int64_t)(b + u) * E + e];
            }
#pragma unroll
            for (int u = 0; u < 16; u++) {
                ps += pv[u];
                ms += mv[u];
            }
        }
        for (; b < b1; b++) {
            ps += blk_prob[(int64_t)b * E + e];
            ms += blk_mcnt[(int64_t)b * E + e];
        }
        s_pp[g * E + e] = ps;
        s_mp[g * E + e] = ms;
    }
    int nt = 0;
    for (int b = tid; b < nblk; b += 1024) nt += blk_ntok[b];
    s_nt[tid] = nt;
    __syncthreads();
    for (int w = 512; w >= 1; w >>= 1) {  // integer tree sum (exact in any order)
        if (tid < w) s_nt[tid] += s_nt[tid + w];
        __syncthreads();
    }
    const int n = s_nt[0];
    if (tid < E) {
        float ps = 0.0f;
        int ms = 0;
        for (int gg = 0; gg < G; gg++) {
            ps += s_pp[gg * E + tid];
            ms += s_mp[gg * E + tid];
        }
        const float pm = n > 0 ? ps / (float)n : 0.0f;
        const float ld = n > 0 ? (float)ms / (float)n : 0.0f;
        s_prob[tid] = pm;
        s_load[tid] = ld;
        if (prob_mean) prob_mean[tid] = pm;
        if (load) load[tid] = ld;
    }
    __syncthreads();
    if (tid == 0 && aux) {
        float a = 0.0f;
        for (int x = 0; x < E; x++) a += s_load[x] * s_prob[x];
        aux[0] = (float)E * a;
    }
}

// Scatter: assignment a of router block b goes to sorted position
// blk_base[b][e] + (number of earlier assignments of block b with expert e).
__global__ __launch_bounds__(256) void route_permute_kernel(
    const int32_t *__restrict__ ids, const float *__restrict__ wts, const int32_t *__restrict__ blk_base,
    int T, int k, int E, int RT, int32_t *__restrict__ perm, int32_t *__restrict__ inv,
    int32_t *__restrict__ row_token, float *__restrict__ row_weight, int32_t *__restrict__ row_expert,
    int32_t *__restrict__ perm_out, int32_t *__restrict__ inv_out)
{
    __shared__ int s_ids[kRouterMaxTokensPerBlock * kMaxExperts];
    const int t0 = blockIdx.x * RT;
    const int nt = min(RT, T - t0);
    const int n = nt * k;
    const int64_t a0 = (int64_t)t0 * k;
    for (int i = threadIdx.x; i < n; i += 256) s_ids[i] = ids[a0 + i];
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += 256) {
        const int e = s_ids[i];
        int r = 0;
        for (int j = 0; j < i; j++) r += (s_ids[j] == e);
        const int p = blk_base[(int64_t)blockIdx.x * E + e] + r;
        const int a = (int)(a0 + i);
        perm[p] = a;
        inv[a] = p;
        row_token[p] = a / k;
        row_weight[p] = wts[a];
        row_expert[p] = e;
        if (perm_out) perm_out[p] = a;
        if (inv_out) inv_out[a] = p;
    }
}

}  // namespace

hipError_t launch_router_topk(const Shape &s, const void *X, const void *Wr, const float *bias,
                              float routed_scale, float *logits_out, int32_t *ids_out, float *wts_out,
                              const RouterStats &rs, const RouterCfg &rc, const Workspace &ws, hipStream_t st)
{
    dim3 grid(s.nblk);
    float *bp = rs.on() ? ws.blk_prob : nullptr;
#define MOE_ROUTER_LAUNCH(TIN, RT, NW)                                                                  \
    hipLaunchKernelGGL((router_topk_kernel<TIN, RT, NW>), grid, dim3(NW * 64), 0, st, (const TIN *)X, (const TIN *)Wr, \
                       bias, (int)s.T, (int)s.H, (int)s.E, s.k, routed_scale, ws.ids, ws.wts, ids_out,  \
                       wts_out, logits_out, ws.blk_counts, rs.mask, bp, ws.blk_mcnt, ws.blk_ntok,     \
                       rc.score_func, rc.sel_bias, rc.n_group, rc.topk_group, rc.jitter_eps)
    static_assert(kRouterMaxTokensPerBlock == 4, "router blocks of 1 or 4 tokens");
    // 32 experts or more: 8 waves share a block's experts (each wave's chain of
    // chunk loads half as long); fewer: 4 waves
    const bool wide = s.E >= 32;
    if (s.dtype == 0) {
        if (s.rtok == 1) {
            if (wide) MOE_ROUTER_LAUNCH(__bf16, 1, 8);
            else MOE_ROUTER_LAUNCH(__bf16, 1, 4);
        } else {
            if (wide) MOE_ROUTER_LAUNCH(__bf16, 4, 8);
            else MOE_ROUTER_LAUNCH(__bf16, 4, 4);
        }
    } else {
        if (s.rtok == 1) MOE_ROUTER_LAUNCH(float, 1, 4);
        else MOE_ROUTER_LAUNCH(float, 4, 4);
    }
#undef MOE_ROUTER_LAUNCH
    return hipGetLastError();
}

hipError_t launch_route_scan(const Shape &s, int32_t *counts_out, int32_t *offsets_out,
                             const RouterStats &rs, const Workspace &ws, hipStream_t st)
{
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(1024), 0, st, ws.blk_counts, s.nblk,
                       (int)s.E, s.tileBM, s.tileXT, s.tileMinRows, ws.counts, ws.offsets, ws.blk_base, ws.tile_start,
                       ws.tiles, counts_out, offsets_out, rs.on() ? ws.blk_prob : nullptr, ws.blk_mcnt,
                       ws.blk_ntok, rs.prob_mean, rs.load, rs.aux);
    return hipGetLastError();
}

hipError_t launch_route_permute(const Shape &s, int32_t *perm_out, int32_t *inv_out,
                                const Workspace &ws, hipStream_t st)
{
    hipLaunchKernelGGL(route_permute_kernel, dim3(s.nblk), dim3(256), 0, st, ws.ids, ws.wts,
                       ws.blk_base, (int)s.T, s.k, (int)s.E, s.rtok, ws.perm, ws.inv, ws.row_token,
                       ws.row_weight, ws.row_expert, perm_out, inv_out);
    return hipGetLastError();
}

}  // namespace moe
