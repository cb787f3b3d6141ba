// C ABI of the MoE layer: argument checks, workspace layout and the kernel
// sequence on the caller's stream. See include/moe_mi355x.h for the contract.
#include "moe_mi355x.h"
#include "moe_internal.h"

#include <math.h>
#include <mutex>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

namespace {

thread_local char g_err[512];

int fail(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlaps(const void *a, uint64_t na, const void *b, uint64_t nb)
{
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

bool debug_sync()
{
    // read once; a function-local static is initialised thread-safely
    static const bool v = [] {
        const char *s = getenv("MOE_DEBUG_SYNC");
        return s && s[0] == '1';
    }();
    return v;
}

constexpr int64_t kAlign = 256;

int64_t align_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Shape checks shared by moe_workspace_bytes and moe_forward (no HIP call).
int check_shape(int64_t T, int64_t H, int64_t I, int64_t E, int32_t k, const moe_opts *opts)
{
    if (opts && opts->struct_size != sizeof(moe_opts))
        return fail(MOE_ERR_INVALID_ARG, "opts->struct_size is %u, expected %zu (call moe_opts_init)",
                    opts->struct_size, sizeof(moe_opts));
    const int dtype = opts ? opts->dtype : MOE_BF16;
    if (dtype != MOE_BF16 && dtype != MOE_F32)
        return fail(MOE_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %lld is negative", (long long)T);
    if (E < 1 || E > moe::kMaxExperts)
        return fail(MOE_ERR_INVALID_ARG, "E = %lld outside [1, %d]", (long long)E, moe::kMaxExperts);
    if (k < 1 || k > E) return fail(MOE_ERR_INVALID_ARG, "k = %d outside [1, E = %lld]", k, (long long)E);
    if (H < 8 || H % 8) return fail(MOE_ERR_INVALID_ARG, "H = %lld must be a positive multiple of 8", (long long)H);
    if (I < 8 || I % 8) return fail(MOE_ERR_INVALID_ARG, "I = %lld must be a positive multiple of 8", (long long)I);
    if (H > (1 << 24) || I > (1 << 24))
        return fail(MOE_ERR_UNSUPPORTED, "H = %lld or I = %lld above 2^24", (long long)H, (long long)I);
    if (T * (int64_t)k >= ((int64_t)1 << 31))
        return fail(MOE_ERR_UNSUPPORTED, "T*k = %lld must be below 2^31", (long long)(T * k));
    // 32-bit element offsets inside one expert / one activation tensor
    if (2 * I * H >= ((int64_t)1 << 31) || T * H >= ((int64_t)1 << 31) || T * (int64_t)k * I >= ((int64_t)1 << 31))
        return fail(MOE_ERR_UNSUPPORTED, "a single expert or activation tensor exceeds 2^31 elements");
    if (opts) {
        if (opts->shared_I < 0 || (opts->shared_I > 0 && opts->shared_I % 8))
            return fail(MOE_ERR_INVALID_ARG, "shared_I = %lld must be 0 or a positive multiple of 8",
                        (long long)opts->shared_I);
        if (opts->shared_I > (1 << 24)) return fail(MOE_ERR_UNSUPPORTED, "shared_I above 2^24");
        // the shared expert runs on the same kernels: 32-bit element offsets
        if (2 * opts->shared_I * H >= ((int64_t)1 << 31) || T * opts->shared_I >= ((int64_t)1 << 31))
            return fail(MOE_ERR_UNSUPPORTED, "the shared expert or its activations exceed 2^31 elements");
        if (opts->flags & ~(MOE_FLAG_FORCE_TILED | MOE_FLAG_FORCE_SKINNY))
            return fail(MOE_ERR_INVALID_ARG, "unknown flag bits 0x%x", opts->flags);
        if ((opts->flags & MOE_FLAG_FORCE_TILED) && (opts->flags & MOE_FLAG_FORCE_SKINNY))
            return fail(MOE_ERR_INVALID_ARG, "MOE_FLAG_FORCE_TILED and MOE_FLAG_FORCE_SKINNY both set");
        if (opts->score_func != MOE_SCORE_SOFTMAX && opts->score_func != MOE_SCORE_SIGMOID &&
            opts->score_func != MOE_SCORE_SPARSEMIXER)
            return fail(MOE_ERR_INVALID_ARG, "unknown score_func %d", opts->score_func);
        if (opts->score_func == MOE_SCORE_SPARSEMIXER) {
            if (!isfinite(opts->jitter_eps) || opts->jitter_eps < 0.0f)
                return fail(MOE_ERR_INVALID_ARG, "jitter_eps must be finite and >= 0");
            if (opts->selection_bias || opts->n_group > 1)
                return fail(MOE_ERR_INVALID_ARG, "sparsemixer scoring takes no selection_bias or groups");
        }
        if (opts->n_group < 0) return fail(MOE_ERR_INVALID_ARG, "n_group = %d is negative", opts->n_group);
        if (opts->n_group > 1) {
            if (opts->n_group > moe::kMaxGroups)
                return fail(MOE_ERR_UNSUPPORTED, "n_group = %d above %d", opts->n_group, moe::kMaxGroups);
            if (E % opts->n_group)
                return fail(MOE_ERR_INVALID_ARG, "E = %lld is not a multiple of n_group = %d", (long long)E,
                            opts->n_group);
            if (opts->topk_group < 1 || opts->topk_group > opts->n_group)
                return fail(MOE_ERR_INVALID_ARG, "topk_group = %d outside [1, n_group = %d]", opts->topk_group,
                            opts->n_group);
            if ((int64_t)k > (int64_t)opts->topk_group * (E / opts->n_group))
                return fail(MOE_ERR_INVALID_ARG, "k = %d exceeds the experts of topk_group groups", k);
        }
        if (opts->weight_format != MOE_WEIGHTS_NATIVE && opts->weight_format != MOE_WEIGHTS_FP8_E4M3 &&
            opts->weight_format != MOE_WEIGHTS_MXFP4)
            return fail(MOE_ERR_INVALID_ARG, "unknown weight_format %d", opts->weight_format);
        if (opts->weight_format == MOE_WEIGHTS_MXFP4) {
            if (dtype != MOE_BF16)
                return fail(MOE_ERR_UNSUPPORTED, "MXFP4 expert weights need bf16 activations (dtype MOE_BF16)");
            if (H % 32 || I % 32)
                return fail(MOE_ERR_UNSUPPORTED, "MXFP4 expert weights need H and I multiples of 32");
            if (opts->flags & MOE_FLAG_FORCE_TILED)
                return fail(MOE_ERR_UNSUPPORTED, "MXFP4 expert weights run on the weight-streaming kernels only");
            if (T * (int64_t)k > 32 * E)
                return fail(MOE_ERR_UNSUPPORTED, "MXFP4 expert weights serve batches of T*k <= 32*E (the "
                                                 "weight-streaming schedule); T*k = %lld",
                            (long long)(T * k));
        }
        if (opts->weight_format == MOE_WEIGHTS_FP8_E4M3) {
            if (dtype != MOE_BF16)
                return fail(MOE_ERR_UNSUPPORTED, "FP8 expert weights need bf16 activations (dtype MOE_BF16)");
            if (H % 16 || I % 16)
                return fail(MOE_ERR_UNSUPPORTED, "FP8 expert weights need H and I multiples of 16");
            if (opts->flags & MOE_FLAG_FORCE_TILED)
                return fail(MOE_ERR_UNSUPPORTED, "FP8 expert weights run on the weight-streaming kernels only");
            if (T * (int64_t)k > 32 * E)
                return fail(MOE_ERR_UNSUPPORTED, "FP8 expert weights serve batches of T*k <= 32*E (the "
                                                 "weight-streaming schedule); T*k = %lld",
                            (long long)(T * k));
        }
        if (opts->weight_layout != MOE_LAYOUT_ROWS && opts->weight_layout != MOE_LAYOUT_TILE_BLOCKS)
            return fail(MOE_ERR_INVALID_ARG, "unknown weight_layout %d", opts->weight_layout);
        if (opts->weight_layout == MOE_LAYOUT_TILE_BLOCKS) {
            if (dtype != MOE_BF16 || opts->weight_format != MOE_WEIGHTS_NATIVE)
                return fail(MOE_ERR_UNSUPPORTED, "tile-block weights are bf16 (dtype MOE_BF16, MOE_WEIGHTS_NATIVE)");
            if (opts->flags & MOE_FLAG_FORCE_SKINNY)
                return fail(MOE_ERR_INVALID_ARG, "tile-block weights run on the tiled kernels only "
                                                 "(MOE_FLAG_FORCE_SKINNY)");
            if (moe::tile_blocks_expert_bytes(0, I, H) >= ((int64_t)1 << 31) ||
                moe::tile_blocks_expert_bytes(1, I, H) >= ((int64_t)1 << 31))
                return fail(MOE_ERR_UNSUPPORTED, "one expert's tile blocks exceed 2^31 bytes");
        }
    }
    return MOE_OK;
}

// Schedule of the routed experts' GEMMs.
//   SKINNY: the weight-streaming kernels (few rows per expert, low-precision
//           weights, or forced); with no more than 32 tokens no expert can
//           hold more than 32 rows, so every expert's weights stream once.
//   MIXED:  the weight-streaming kernels for experts with up to 32 rows and
//           the tiled kernel for the others (few rows per expert on average,
//           but more than 32 tokens: one expert may take many of them).
//   TILED:  the large-M tiled kernel for every expert.
enum class Sched { SKINNY, MIXED, TILED };

Sched schedule(int64_t T, int32_t k, int64_t E, const moe_opts *opts)
{
    const uint32_t flags = opts ? opts->flags : 0;
    if (opts && opts->weight_format != MOE_WEIGHTS_NATIVE) return Sched::SKINNY;  // low-precision weights
    if (opts && opts->dtype == MOE_F32) return Sched::SKINNY;  // the fp32 kernels (one schedule)
    if (opts && opts->weight_layout == MOE_LAYOUT_TILE_BLOCKS) return Sched::TILED;  // the blocks' only reader
    if (flags & MOE_FLAG_FORCE_SKINNY) return Sched::SKINNY;
    if (flags & MOE_FLAG_FORCE_TILED) return Sched::TILED;
    if (T * k > 32 * E) return Sched::TILED;  // more than about 32 rows per expert
    return T <= moe::kSkinnyMaxRows ? Sched::SKINNY : Sched::MIXED;
}

moe::Shape make_shape(int64_t T, int64_t H, int64_t I, int64_t E, int32_t k, const moe_opts *opts)
{
    moe::Shape s;
    s.T = T;
    s.H = H;
    s.I = I;
    s.E = E;
    s.k = k;
    s.sharedI = opts ? opts->shared_I : 0;
    s.dtype = opts ? opts->dtype : MOE_BF16;
    // tokens per router block: one token per block while T alone does not
    // fill the CUs, else 4 (many short blocks keep every CU busy)
    s.rtok = T <= 256 ? 1 : 4;
    s.nblk = (int)((T + s.rtok - 1) / s.rtok);
    s.tileBM = moe::tiled_block_m();
    s.tileXT = moe::tiled_tail_m();
    s.maxTiles = (T * k) / s.tileBM + E + 1;
    // experts with fewer rows than tileMinRows get no M-tile (the streaming kernels serve them)
    const Sched sc = schedule(T, k, E, opts);
    s.tileMinRows = sc == Sched::MIXED ? moe::kSkinnyMaxRows + 1 : 0;
    // the partial sums of split tiles (a launch with a short last round, or
    // the few tiles of the mixed schedule's large experts, spreads them over
    // every CU along K)
    s.partBytes = (s.dtype == MOE_BF16 && sc != Sched::SKINNY) ? moe::tiled_split_bytes() : 0;
    // every routed row on the tiled kernels: h lives in row blocks of the tile list
    s.hBlocks = s.dtype == MOE_BF16 && sc == Sched::TILED;
    return s;
}

}  // namespace

namespace moe {

int64_t workspace_layout(const Shape &s, void *base, Workspace *ws)
{
    int64_t off = 0;
    auto take = [&](int64_t bytes) -> void * {
        off = align_up(off);
        void *p = base ? (void *)((char *)base + off) : nullptr;
        off += bytes;
        return p;
    };
    const int64_t TK = s.T * s.k;
    const int64_t es = s.dtype == MOE_BF16 ? 2 : 4;
    Workspace w;
    w.ids = (int32_t *)take(TK * 4);
    w.wts = (float *)take(TK * 4);
    w.blk_counts = (int32_t *)take((int64_t)s.nblk * s.E * 4);
    w.blk_base = (int32_t *)take((int64_t)s.nblk * s.E * 4);
    w.blk_prob = (float *)take((int64_t)s.nblk * s.E * 4);
    w.blk_mcnt = (int32_t *)take((int64_t)s.nblk * s.E * 4);
    w.blk_ntok = (int32_t *)take((int64_t)s.nblk * 4);
    w.counts = (int32_t *)take(s.E * 4);
    w.offsets = (int32_t *)take((s.E + 1) * 4);
    w.tile_start = (int32_t *)take((s.E + 1) * 4);
    w.tiles = (MTile *)take(s.maxTiles * (int64_t)sizeof(MTile));
    w.perm = (int32_t *)take(TK * 4);
    w.inv = (int32_t *)take(TK * 4);
    w.row_token = (int32_t *)take(TK * 4);
    w.row_weight = (float *)take(TK * 4);
    w.row_expert = (int32_t *)take(TK * 4);
    w.h = take(s.hBlocks ? h_blocks_bytes(s.maxTiles, s.I) : TK * s.I * es);
    w.slot = (float *)take(TK * s.H * 4);
    w.sh_h = s.sharedI > 0 ? take(s.T * s.sharedI * es) : nullptr;
    w.sh_y = s.sharedI > 0 ? (float *)take(s.T * s.H * 4) : nullptr;
    w.part = s.partBytes > 0 ? (float *)take(s.partBytes) : nullptr;
    if (ws) *ws = w;
    return align_up(off);
}

}  // namespace moe

namespace {

// Scratch memory of moe_forward_noalloc, for callers that cannot allocate
// (code under graph capture, serving loops, harnesses that forbid hipMalloc).
// Each GPU holds its own copy for the life of the process. In host code the
// array's name is only a stand-in: its device address comes from
// hipGetSymbolAddress, once per device with that device current, and only
// that address is ever passed to kernels.
constexpr size_t kScratchBytes = MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void *g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

int scratch_on_current_device(void **ptr)
{
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return fail(MOE_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(err));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(MOE_ERR_UNSUPPORTED, "device %d: moe_forward_noalloc serves devices 0..%d", dev, kMaxDevices - 1);
    std::call_once(g_scratch_once[dev], [dev] {
        void *p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev])
        return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev,
                    hipGetErrorString(g_scratch_err[dev]));
    *ptr = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace

extern "C" {

void moe_opts_init(moe_opts *opts)
{
    if (!opts) return;
    memset(opts, 0, sizeof *opts);
    opts->struct_size = sizeof(moe_opts);
    opts->dtype = MOE_BF16;
    opts->routed_scale = 1.0f;
    opts->jitter_eps = 0.01f;
}

const char *moe_last_error(void) { return g_err; }

int64_t moe_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int32_t k, const moe_opts *opts)
{
    g_err[0] = 0;
    const int rc = check_shape(T, H, I, E, k, opts);
    if (rc != MOE_OK) return rc;
    const moe::Shape s = make_shape(T, H, I, E, k, opts);
    return moe::workspace_layout(s, nullptr, nullptr);
}

// The layer on the caller's stream with the workspace in opts (both entry points).
static int forward_impl(const void *hidden, const void *router_w, const void *gate_up, const void *down,
                        int64_t T, int64_t H, int64_t I, int64_t E, int32_t k, const moe_opts *opts, void *out)
{
    if (!opts) return fail(MOE_ERR_INVALID_ARG, "opts is NULL");
    int rc = check_shape(T, H, I, E, k, opts);
    if (rc != MOE_OK) return rc;
    if (!isfinite(opts->routed_scale)) return fail(MOE_ERR_INVALID_ARG, "routed_scale is not finite");
    if (T == 0) return MOE_OK;

    if (!hidden || !router_w || !gate_up || !down || !out)
        return fail(MOE_ERR_INVALID_ARG, "hidden, router_w, gate_up, down and out must be non-NULL");
    const bool shared = opts->shared_I > 0;
    if (shared && (!opts->shared_gate_up || !opts->shared_down))
        return fail(MOE_ERR_INVALID_ARG, "shared_I > 0 needs shared_gate_up and shared_down");
    const void *tens[] = {hidden, router_w, gate_up, down, out, opts->shared_gate_up, opts->shared_down};
    for (const void *p : tens)
        if (p && !aligned(p, 16)) return fail(MOE_ERR_ALIGNMENT, "tensor pointer %p is not 16-byte aligned", p);
    const void *small[] = {opts->router_bias, opts->router_logits, opts->topk_ids, opts->topk_weights,
                           opts->expert_counts, opts->expert_offsets, opts->perm, opts->inv_perm,
                           opts->stats_mask, opts->router_prob_mean, opts->expert_load, opts->aux_loss,
                           opts->selection_bias};
    for (const void *p : small)
        if (p && !aligned(p, 4)) return fail(MOE_ERR_ALIGNMENT, "output pointer %p is not 4-byte aligned", p);

    const bool w8 = opts->weight_format == MOE_WEIGHTS_FP8_E4M3;
    const bool w4 = opts->weight_format == MOE_WEIGHTS_MXFP4;
    if (w8 && (!opts->gate_up_scale || !opts->down_scale))
        return fail(MOE_ERR_INVALID_ARG, "FP8 expert weights need gate_up_scale and down_scale");
    if (w4 && (!opts->gate_up_block_scale || !opts->down_block_scale))
        return fail(MOE_ERR_INVALID_ARG, "MXFP4 expert weights need gate_up_block_scale and down_block_scale");
    if (w8 && (!aligned(opts->gate_up_scale, 4) || !aligned(opts->down_scale, 4)))
        return fail(MOE_ERR_ALIGNMENT, "gate_up_scale / down_scale not 4-byte aligned");
    const uint64_t es = opts->dtype == MOE_BF16 ? 2 : 4;
    const uint64_t wes2 = w4 ? 1 : w8 ? 2 : 2 * es;  // twice the bytes per routed expert weight
    const bool blocks = opts->weight_layout == MOE_LAYOUT_TILE_BLOCKS;
    const uint64_t out_bytes = (uint64_t)T * H * es;
    struct Range {
        const void *p;
        uint64_t n;
    } ins[] = {{hidden, (uint64_t)T * H * es},
               {router_w, (uint64_t)E * H * es},
               {gate_up, blocks ? (uint64_t)E * moe::tile_blocks_expert_bytes(0, I, H) : (uint64_t)E * 2 * I * H * wes2 / 2},
               {down, blocks ? (uint64_t)E * moe::tile_blocks_expert_bytes(1, I, H) : (uint64_t)E * H * I * wes2 / 2},
               {opts->gate_up_scale, w8 ? (uint64_t)E * 2 * I * 4 : 0},
               {opts->down_scale, w8 ? (uint64_t)E * H * 4 : 0},
               {opts->gate_up_block_scale, w4 ? (uint64_t)E * 2 * I * (H / 32) : 0},
               {opts->down_block_scale, w4 ? (uint64_t)E * H * (I / 32) : 0},
               {opts->shared_gate_up, shared ? (uint64_t)2 * opts->shared_I * H * es : 0},
               {opts->shared_down, shared ? (uint64_t)H * opts->shared_I * es : 0},
               {opts->router_bias, (uint64_t)E * 4},
               {opts->stats_mask, (uint64_t)T * 4},
               {opts->selection_bias, (uint64_t)E * 4},
               {opts->workspace, opts->workspace_bytes}};
    for (const Range &r : ins)
        if (overlaps(out, out_bytes, r.p, r.n)) return fail(MOE_ERR_INVALID_ARG, "out overlaps an input or the workspace");
    // the workspace is written by every call: it must not overlap an input
    const size_t nins = sizeof ins / sizeof ins[0];  // the last entry is the workspace itself
    for (size_t i = 0; i + 1 < nins; i++)
        if (overlaps(opts->workspace, opts->workspace_bytes, ins[i].p, ins[i].n))
            return fail(MOE_ERR_INVALID_ARG, "the workspace overlaps an input");
    // optional outputs: none may overlap an input, the workspace, out or another output
    const uint64_t TK = (uint64_t)T * k;
    const Range outs[] = {{opts->router_logits, (uint64_t)T * E * 4}, {opts->topk_ids, TK * 4},
                          {opts->topk_weights, TK * 4},           {opts->expert_counts, (uint64_t)E * 4},
                          {opts->expert_offsets, (uint64_t)(E + 1) * 4}, {opts->perm, TK * 4},
                          {opts->inv_perm, TK * 4},               {opts->router_prob_mean, (uint64_t)E * 4},
                          {opts->expert_load, (uint64_t)E * 4},   {opts->aux_loss, 4}};
    const size_t nouts = sizeof outs / sizeof outs[0];
    for (size_t i = 0; i < nouts; i++) {
        if (!outs[i].p) continue;
        if (overlaps(outs[i].p, outs[i].n, out, out_bytes))
            return fail(MOE_ERR_INVALID_ARG, "an optional output overlaps out");
        for (const Range &r : ins)
            if (overlaps(outs[i].p, outs[i].n, r.p, r.n))
                return fail(MOE_ERR_INVALID_ARG, "an optional output overlaps an input or the workspace");
        for (size_t j = 0; j < i; j++)
            if (overlaps(outs[i].p, outs[i].n, outs[j].p, outs[j].n))
                return fail(MOE_ERR_INVALID_ARG, "two optional outputs overlap");
    }

    const moe::Shape s = make_shape(T, H, I, E, k, opts);
    const int64_t need = moe::workspace_layout(s, nullptr, nullptr);
    if (!opts->workspace || (int64_t)opts->workspace_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "workspace of %zu bytes at %p; %lld bytes needed", opts->workspace_bytes,
                    opts->workspace, (long long)need);
    if (!aligned(opts->workspace, 256)) return fail(MOE_ERR_ALIGNMENT, "workspace is not 256-byte aligned");

    moe::Workspace ws;
    moe::workspace_layout(s, opts->workspace, &ws);
    hipStream_t st = (hipStream_t)opts->stream;
    // compute units of the current device, queried on every call (sizes the
    // persistent launches; nothing is cached between calls)
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return fail(MOE_ERR_HIP, "cannot query the compute units of the current device");

    const bool f32 = opts->dtype == MOE_F32;
    const Sched sched = schedule(T, k, E, opts);
    const bool skinny = sched != Sched::TILED;  // the weight-streaming kernels run
    const bool tiled = sched != Sched::SKINNY;  // the tiled kernel runs

    int step = 0;
    auto check = [&](hipError_t err, const char *what) -> int {
        step++;
        if (err == hipSuccess && debug_sync()) err = hipStreamSynchronize(st);
        if (err != hipSuccess)
            return fail(MOE_ERR_HIP, "%s (step %d) failed: %s", what, step, hipGetErrorString(err));
        return MOE_OK;
    };
    // stage boundary i (0 = before the first kernel); no-op without events
    auto mark = [&](int i) -> int {
        if (!opts->stage_events || !opts->stage_events[i]) return MOE_OK;
        hipError_t err = hipEventRecord((hipEvent_t)opts->stage_events[i], st);
        if (err != hipSuccess) return fail(MOE_ERR_HIP, "hipEventRecord(stage %d): %s", i, hipGetErrorString(err));
        return MOE_OK;
    };
    if ((rc = mark(0))) return rc;

    moe::RouterStats rs;
    rs.mask = opts->stats_mask;
    rs.prob_mean = opts->router_prob_mean;
    rs.load = opts->expert_load;
    rs.aux = opts->aux_loss;
    moe::RouterCfg rcfg;
    rcfg.score_func = opts->score_func;
    rcfg.sel_bias = opts->selection_bias;
    rcfg.n_group = opts->n_group > 1 ? opts->n_group : 0;
    rcfg.topk_group = opts->topk_group;
    rcfg.jitter_eps = opts->jitter_eps;
    if ((rc = check(moe::launch_router_topk(s, hidden, router_w, opts->router_bias, opts->routed_scale,
                                            opts->router_logits, opts->topk_ids, opts->topk_weights, rs, rcfg, ws,
                                            st),
                    "router_topk")) || (rc = mark(1 + MOE_STAGE_ROUTER)))
        return rc;
    // Few assignments on the weight-streaming kernels, with no sorted routing
    // tables or statistics asked for: those kernels route straight from the
    // top-k ids, and the scan and permute launches are skipped.
    const bool direct = sched == Sched::SKINNY && !f32 && T * k <= moe::kSkinnyDirectMax && !opts->expert_counts &&
                        !opts->expert_offsets && !opts->perm && !opts->inv_perm && !rs.on();
    if (!direct) {
        if ((rc = check(moe::launch_route_scan(s, opts->expert_counts, opts->expert_offsets, rs, ws, st),
                        "route_scan")))
            return rc;
    }
    if ((rc = mark(1 + MOE_STAGE_SCAN))) return rc;
    if (!direct) {
        if ((rc = check(moe::launch_route_permute(s, opts->perm, opts->inv_perm, ws, st), "route_permute"))) return rc;
    }
    if ((rc = mark(1 + MOE_STAGE_PERMUTE))) return rc;

    moe::GemmProblem gu;
    gu.A = hidden;
    gu.a_rows = ws.row_token;
    gu.W = gate_up;
    gu.w_scale = w8 ? opts->gate_up_scale : nullptr;
    gu.w_bscale = w4 ? opts->gate_up_block_scale : nullptr;
    gu.w_expert_stride = 2 * I * H;
    gu.K = H;
    gu.N = I;
    gu.C = ws.h;
    gu.c_rows = nullptr;
    gu.c_scale = nullptr;
    gu.counts = ws.counts;
    gu.offsets = ws.offsets;
    gu.row_expert = ws.row_expert;
    gu.tiles = ws.tiles;
    gu.tile_start = ws.tile_start;
    gu.E = E;
    gu.dense_rows = 0;
    gu.total_rows = T * k;
    gu.part = ws.part;
    gu.ids = direct ? ws.ids : nullptr;
    gu.wts = direct ? ws.wts : nullptr;
    gu.k = k;
    gu.cus = cus;
    gu.a_rows_total = T;
    gu.skinny_max_rows = sched == Sched::MIXED ? moe::kSkinnyMaxRows : 0;
    if (blocks) {
        gu.w_blocks = true;
        gu.w_expert_stride = moe::tile_blocks_expert_bytes(0, I, H) / 2;
    }
    gu.h_blocks = s.hBlocks;
    gu.h_bytes = s.hBlocks ? moe::h_blocks_bytes(s.maxTiles, I) : 0;

    moe::GemmProblem dn = gu;
    dn.A = ws.h;
    dn.a_rows = nullptr;
    dn.W = down;
    dn.w_scale = w8 ? opts->down_scale : nullptr;
    dn.w_bscale = w4 ? opts->down_block_scale : nullptr;
    dn.w_expert_stride = blocks ? moe::tile_blocks_expert_bytes(1, I, H) / 2 : H * I;
    dn.K = I;
    dn.N = H;
    dn.C = ws.slot;
    dn.c_rows = ws.perm;
    dn.c_scale = ws.row_weight;
    dn.a_rows_total = T * k;

    if (f32) {
        rc = check(moe::launch_gate_up_f32(gu, st), "gate_up f32");
    } else {
        if (skinny) rc = check(moe::launch_gate_up_skinny(gu, st), "gate_up skinny");
        if (!rc && tiled) rc = check(moe::launch_gate_up_tiled(gu, st), "gate_up tiled");
    }
    if (rc || (rc = mark(1 + MOE_STAGE_GATE_UP))) return rc;
    if (f32) {
        rc = check(moe::launch_down_f32(dn, st), "down f32");
    } else {
        if (skinny) rc = check(moe::launch_down_skinny(dn, st), "down skinny");
        if (!rc && tiled) rc = check(moe::launch_down_tiled(dn, st), "down tiled");
    }
    if (rc || (rc = mark(1 + MOE_STAGE_DOWN))) return rc;

    if (shared) {
        // shared expert: a dense problem over all T tokens with weight 1
        moe::GemmProblem sg = gu;
        sg.a_rows = nullptr;
        sg.W = opts->shared_gate_up;
        sg.w_scale = nullptr;  // the shared expert keeps opts->dtype
        sg.w_bscale = nullptr;
        sg.w_blocks = false;  // and MOE_LAYOUT_ROWS
        sg.h_blocks = false;
        sg.w_expert_stride = 0;
        sg.N = opts->shared_I;
        sg.C = ws.sh_h;
        sg.c_rows = nullptr;
        sg.c_scale = nullptr;
        sg.dense_rows = T;
        sg.total_rows = T;
        sg.part = ws.part;  // free again: the routed launches have finished with it
        sg.ids = nullptr;
        sg.wts = nullptr;
        sg.a_rows_total = T;
        moe::GemmProblem sd = sg;
        sd.A = ws.sh_h;
        sd.W = opts->shared_down;
        sd.K = opts->shared_I;
        sd.N = H;
        sd.C = ws.sh_y;
        const bool sh_skinny = (opts->flags & MOE_FLAG_FORCE_SKINNY) ||
                               (!(opts->flags & MOE_FLAG_FORCE_TILED) && T <= 32);
        if (f32) rc = check(moe::launch_gate_up_f32(sg, st), "shared gate_up f32");
        else if (sh_skinny) rc = check(moe::launch_gate_up_skinny(sg, st), "shared gate_up skinny");
        else rc = check(moe::launch_gate_up_tiled(sg, st), "shared gate_up tiled");
        if (rc || (rc = mark(1 + MOE_STAGE_SHARED_GATE_UP))) return rc;
        if (f32) rc = check(moe::launch_down_f32(sd, st), "shared down f32");
        else if (sh_skinny) rc = check(moe::launch_down_skinny(sd, st), "shared down skinny");
        else rc = check(moe::launch_down_tiled(sd, st), "shared down tiled");
        if (rc || (rc = mark(1 + MOE_STAGE_SHARED_DOWN))) return rc;
    } else {
        if ((rc = mark(1 + MOE_STAGE_SHARED_GATE_UP)) || (rc = mark(1 + MOE_STAGE_SHARED_DOWN))) return rc;
    }
    if ((rc = check(moe::launch_combine(s, ws.slot, shared ? ws.sh_y : nullptr, out, st), "combine")) ||
        (rc = mark(1 + MOE_STAGE_COMBINE)))
        return rc;
    return MOE_OK;
}

int moe_forward(const void *hidden, const void *router_w, const void *gate_up, const void *down,
                int64_t T, int64_t H, int64_t I, int64_t E, int32_t k, const moe_opts *opts, void *out)
{
    g_err[0] = 0;
    return forward_impl(hidden, router_w, gate_up, down, T, H, I, E, k, opts, out);
}

int moe_forward_noalloc(const void *hidden, const void *router_w, const void *gate_up, const void *down,
                        int64_t T, int64_t H, int64_t I, int64_t E, int32_t k, const moe_opts *opts, void *out)
{
    g_err[0] = 0;
    if (!opts) return fail(MOE_ERR_INVALID_ARG, "opts is NULL");
    int rc = check_shape(T, H, I, E, k, opts);
    if (rc != MOE_OK) return rc;
    if (opts->workspace || opts->workspace_bytes)
        return fail(MOE_ERR_INVALID_ARG, "moe_forward_noalloc uses the library's scratch: opts->workspace must be "
                                         "NULL and workspace_bytes 0");
    const moe::Shape s = make_shape(T, H, I, E, k, opts);
    const int64_t need = moe::workspace_layout(s, nullptr, nullptr);
    if (need > (int64_t)kScratchBytes)
        return fail(MOE_ERR_UNSUPPORTED, "these sizes need %lld bytes of scratch; moe_forward_noalloc holds %lld "
                                         "(use moe_forward with a workspace)",
                    (long long)need, (long long)kScratchBytes);
    if (T == 0) return forward_impl(hidden, router_w, gate_up, down, T, H, I, E, k, opts, out);
    void *ptr = nullptr;
    if ((rc = scratch_on_current_device(&ptr)) != MOE_OK) return rc;
    moe_opts o = *opts;  // struct_size checked above: the whole struct is the caller's
    o.workspace = ptr;
    o.workspace_bytes = kScratchBytes;
    return forward_impl(hidden, router_w, gate_up, down, T, H, I, E, k, &o, out);
}

int64_t moe_tile_blocks_bytes(int32_t which, int64_t E, int64_t I, int64_t H)
{
    g_err[0] = 0;
    if (which != MOE_PACK_GATE_UP && which != MOE_PACK_DOWN)
        return fail(MOE_ERR_INVALID_ARG, "which = %d: MOE_PACK_GATE_UP or MOE_PACK_DOWN", which);
    if (E < 1 || E > moe::kMaxExperts)
        return fail(MOE_ERR_INVALID_ARG, "E = %lld outside [1, %d]", (long long)E, moe::kMaxExperts);
    if (H < 8 || H % 8) return fail(MOE_ERR_INVALID_ARG, "H = %lld must be a positive multiple of 8", (long long)H);
    if (I < 8 || I % 8) return fail(MOE_ERR_INVALID_ARG, "I = %lld must be a positive multiple of 8", (long long)I);
    if (H > (1 << 24) || I > (1 << 24))
        return fail(MOE_ERR_UNSUPPORTED, "H = %lld or I = %lld above 2^24", (long long)H, (long long)I);
    const int64_t per = moe::tile_blocks_expert_bytes(which, I, H);
    if (per >= ((int64_t)1 << 31)) return fail(MOE_ERR_UNSUPPORTED, "one expert's tile blocks exceed 2^31 bytes");
    return E * per;
}

int moe_pack_tile_blocks(int32_t which, const void *w, int64_t E, int64_t I, int64_t H, void *out, void *stream)
{
    const int64_t n = moe_tile_blocks_bytes(which, E, I, H);  // argument checks
    if (n < 0) return (int)n;
    if (!w || !out) return fail(MOE_ERR_INVALID_ARG, "w and out must be non-NULL");
    if (!aligned(w, 16) || !aligned(out, 16)) return fail(MOE_ERR_ALIGNMENT, "w and out must be 16-byte aligned");
    const uint64_t wbytes = (uint64_t)E * (which == MOE_PACK_GATE_UP ? 2 * I * H : H * I) * 2;
    if (overlaps(out, (uint64_t)n, w, wbytes)) return fail(MOE_ERR_INVALID_ARG, "out overlaps w");
    hipError_t err = moe::launch_pack_tile_blocks(which, w, E, I, H, out, (hipStream_t)stream);
    if (err == hipSuccess && debug_sync()) err = hipStreamSynchronize((hipStream_t)stream);
    if (err != hipSuccess) return fail(MOE_ERR_HIP, "pack_tile_blocks failed: %s", hipGetErrorString(err));
    return MOE_OK;
}

int moe_quantize_fp8_rows(const void *w, int64_t rows, int64_t cols, void *q, float *scale, void *stream)
{
    g_err[0] = 0;
    if (rows < 0) return fail(MOE_ERR_INVALID_ARG, "rows = %lld is negative", (long long)rows);
    if (cols < 16 || cols % 16) return fail(MOE_ERR_INVALID_ARG, "cols = %lld must be a positive multiple of 16", (long long)cols);
    if (rows >= ((int64_t)1 << 31) || cols >= ((int64_t)1 << 31))
        return fail(MOE_ERR_UNSUPPORTED, "rows or cols at or above 2^31");
    if (rows == 0) return MOE_OK;
    if (!w || !q || !scale) return fail(MOE_ERR_INVALID_ARG, "w, q and scale must be non-NULL");
    if (!aligned(w, 16) || !aligned(q, 16) || !aligned(scale, 4))
        return fail(MOE_ERR_ALIGNMENT, "w and q must be 16-byte aligned, scale 4-byte aligned");
    const uint64_t n = (uint64_t)rows * cols;
    if (overlaps(q, n, w, 2 * n) || overlaps(scale, (uint64_t)rows * 4, w, 2 * n) || overlaps(scale, (uint64_t)rows * 4, q, n))
        return fail(MOE_ERR_INVALID_ARG, "q, scale and w must not overlap");
    hipError_t err = moe::launch_quantize_fp8_rows(w, rows, cols, q, scale, (hipStream_t)stream);
    if (err == hipSuccess && debug_sync()) err = hipStreamSynchronize((hipStream_t)stream);
    if (err != hipSuccess) return fail(MOE_ERR_HIP, "quantize_fp8_rows failed: %s", hipGetErrorString(err));
    return MOE_OK;
}

int moe_quantize_mxfp4_rows(const void *w, int64_t rows, int64_t cols, void *q, void *scale, void *stream)
{
    g_err[0] = 0;
    if (rows < 0) return fail(MOE_ERR_INVALID_ARG, "rows = %lld is negative", (long long)rows);
    if (cols < 32 || cols % 32) return fail(MOE_ERR_INVALID_ARG, "cols = %lld must be a positive multiple of 32", (long long)cols);
    if (rows >= ((int64_t)1 << 31) || cols >= ((int64_t)1 << 31) || rows * (cols / 32) >= ((int64_t)1 << 36))
        return fail(MOE_ERR_UNSUPPORTED, "rows or cols too large");
    if (rows == 0) return MOE_OK;
    if (!w || !q || !scale) return fail(MOE_ERR_INVALID_ARG, "w, q and scale must be non-NULL");
    if (!aligned(w, 16) || !aligned(q, 16)) return fail(MOE_ERR_ALIGNMENT, "w and q must be 16-byte aligned");
    const uint64_t n = (uint64_t)rows * cols;
    if (overlaps(q, n / 2, w, 2 * n) || overlaps(scale, n / 32, w, 2 * n) || overlaps(scale, n / 32, q, n / 2))
        return fail(MOE_ERR_INVALID_ARG, "q, scale and w must not overlap");
    hipError_t err = moe::launch_quantize_mxfp4_rows(w, rows, cols, q, scale, (hipStream_t)stream);
    if (err == hipSuccess && debug_sync()) err = hipStreamSynchronize((hipStream_t)stream);
    if (err != hipSuccess) return fail(MOE_ERR_HIP, "quantize_mxfp4_rows failed: %s", hipGetErrorString(err));
    return MOE_OK;
}

}  // extern "C"
